"""Pins of the oracle's 1-bit sign error-feedback step (CPU only).

Checked against a hand-worked case, an independent numpy float32 evaluation,
numpy's sign and packbits, the 32-to-1-bit ratio the page states, and closed
forms of the recurrences (page "1-bit Adam gradient compression", sections
2.1 and 2.2).
"""
import json
import os
import pathlib

import numpy as np
import pytest

import gen
import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def numpy_sign_step(g, e, m, beta1, clip):
    """Same recurrences, evaluated array-wise by numpy in float32 (each op rounded once)."""
    f = np.float32
    g = np.asarray(g, f)
    gc = np.where(g > f(clip), f(clip), np.where(g < f(-clip), f(-clip), g)).astype(f)
    x = (gc + e).astype(f)
    s = np.sign(x)
    s = np.where(np.isnan(s), f(0), s).astype(f)
    d = (x - s).astype(f)
    c = f(f(1.0) - f(beta1))
    e2 = ((f(beta1) * e).astype(f) + (c * d).astype(f)).astype(f)
    m2 = ((f(beta1) * m).astype(f) + (c * s).astype(f)).astype(f)
    return e2, m2, s.astype(np.int8)


def bits_of(a):
    return np.asarray(a, np.float32).view(np.uint32)


def test_hand_worked():
    d = json.loads(pathlib.Path(os.path.join(GOLD, "sign_worked.json")).read_text())
    e2, m2, s, bits, bad = oracle.sign(d["g"], d["e"], d["m"], d["beta1"], d["clip"])
    assert s.tolist() == d["sign"]
    assert bits.tolist() == d["bits"]
    assert np.array_equal(bits_of(e2), bits_of(d["e_new"]))
    assert np.array_equal(bits_of(m2), bits_of(d["m_new"]))
    assert bad == 0


@pytest.mark.parametrize("n", [1, 7, 8, 9, 63, 1000, 65_537])
@pytest.mark.parametrize("beta1", [0.9, 0.8, 0.0, 1.0])
def test_matches_numpy_evaluation(n, beta1):
    g = gen.normal_small(n, 1, n, scale=3.0)
    e = gen.normal_small(n, 2, n, scale=0.5)
    m = gen.normal_small(n, 3, n, scale=0.5)
    e2, m2, s, bits, bad = oracle.sign(g, e, m, beta1, 5.0)
    ne, nm, ns = numpy_sign_step(g, e, m, beta1, 5.0)
    assert np.array_equal(bits_of(e2), bits_of(ne))
    assert np.array_equal(bits_of(m2), bits_of(nm))
    assert np.array_equal(s, ns)
    assert np.array_equal(bits, np.packbits(s == 1, bitorder="little"))
    assert bits.size == (n + 7) // 8


def test_specials():
    n = 4096
    g = gen.specials(n, 7)
    e = gen.specials(n, 8)
    m = gen.normal_small(n, 9)
    e2, m2, s, bits, bad = oracle.sign(g, e, m, 0.9, 5.0)
    ne, nm, ns = numpy_sign_step(g, e, m, 0.9, 5.0)
    both_nan = np.isnan(e2) & np.isnan(ne)
    assert np.array_equal(bits_of(e2)[~both_nan], bits_of(ne)[~both_nan])
    assert np.array_equal(np.isnan(e2), np.isnan(ne))
    assert np.array_equal(bits_of(m2), bits_of(nm))
    assert np.array_equal(s, ns)
    assert bad == int((~np.isfinite(e2)).sum() + (~np.isfinite(m2)).sum())
    # subnormal x still has a sign; +-0 has sign 0
    e0, m0, s0, _, _ = oracle.sign(np.array([1e-45, -1e-45, 0.0, -0.0], np.float32),
                                   np.zeros(4, np.float32), np.zeros(4, np.float32), 0.9, 5.0)
    assert s0.tolist() == [1, -1, 0, 0]


def test_one_bit_ratio():
    ratio = json.loads(pathlib.Path(os.path.join(GOLD, "ratios.json")).read_text())["one_bit_reduction"]["value"]
    n = 8 * 12345
    _, _, _, bits, _ = oracle.sign(np.ones(n, np.float32), np.zeros(n, np.float32),
                                   np.zeros(n, np.float32), 0.9, 5.0)
    assert 1.0 - bits.nbytes / (4.0 * n) == ratio


def test_clip():
    g = np.array([7.0, -7.0, 5.0, -5.0, 4.0, np.inf, -np.inf], np.float32)
    z = np.zeros(g.size, np.float32)
    e2, _, s, _, _ = oracle.sign(g, z, z, 0.0, 5.0)  # beta1 = 0: e' = x - s exactly
    assert e2.tolist() == [4.0, -4.0, 4.0, -4.0, 3.0, 4.0, -4.0]
    e2, _, _, _, bad = oracle.sign(g, z, z, 0.0, np.inf)  # clip disabled
    assert e2[:5].tolist() == [6.0, -6.0, 4.0, -4.0, 3.0] and bad == 2


def test_beta_zero_is_plain_sign_residual():
    n = 10_000
    g = gen.normal_small(n, 11)
    e = gen.normal_small(n, 12, scale=0.3)
    m = gen.normal_small(n, 13)
    e2, m2, s, _, _ = oracle.sign(g, e, m, 0.0, np.inf)
    x = (g + e).astype(np.float32)
    assert np.array_equal(bits_of(e2), bits_of((x - s.astype(np.float32)).astype(np.float32)))
    assert np.array_equal(m2, s.astype(np.float32))


def test_zero_gradient_stays_zero():
    n = 1000
    z = np.zeros(n, np.float32)
    e2, m2, s, bits, _ = oracle.sign(z, z, z, 0.9, 5.0)
    assert not s.any() and not bits.any() and not e2.any() and not m2.any()


def test_constant_gradient_closed_form():
    """g = c > 1 every step from zero state: q = +1 always, e_t = t (1-b)(c-1),
    m_t = 1 - b^t (exact arithmetic; float32 chain within a few ulp per step)."""
    c, b, T = 1.5, 0.9, 30
    n = 4
    e = np.zeros(n, np.float32)
    m = np.zeros(n, np.float32)
    for t in range(1, T + 1):
        e, m, s, _, _ = oracle.sign(np.full(n, c, np.float32), e, m, b, 5.0)
        assert np.all(s == 1)
        assert abs(float(e[0]) - t * (1 - b) * (c - 1)) <= 4 * t * np.spacing(np.float32(t * 0.05))
        assert abs(float(m[0]) - (1 - b ** t)) <= 4 * t * 2.0 ** -24


def test_chain_telescopes():
    """e_T - e_0 = (1-b) sum_t (g_t - q_t) and m_T = b^T m_0 + (1-b) sum_t b^(T-t) q_t."""
    n, T, b = 20_000, 50, 0.9
    e = np.zeros(n, np.float32)
    m = np.zeros(n, np.float32)
    c = float(np.float32(1.0) - np.float32(b))
    acc = np.zeros(n)
    mom = np.zeros(n)
    scale = np.zeros(n)
    for t in range(T):
        g = gen.sign_gradient(t, n=n)
        e, m, s, _, _ = oracle.sign(g, e, m, b, 5.0)
        acc += g.astype(np.float64) - s
        mom = float(np.float32(b)) * mom + c * s
        scale += np.abs(g) + 1.0
    assert np.max(np.abs(e - c * acc)) <= 1e-5 * np.max(scale)
    assert np.max(np.abs(m - mom)) <= 1e-5
