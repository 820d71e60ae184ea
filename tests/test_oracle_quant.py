"""Pins of the oracle's 8-bit quantisation of a sent packet (CPU only)."""
import json
import os
import pathlib

import numpy as np
import pytest

import gen
import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def numpy_quant(vals, idx, e):
    """The same reading evaluated by numpy, float32 elementwise."""
    f = np.float32
    v = np.asarray(vals, f)
    fin = np.isfinite(v)
    amax = f(np.max(np.abs(v[fin]))) if fin.any() else f(0)
    e2 = np.asarray(e, f).copy()
    if amax > 0:
        inv = f(f(127) / amax)
        scale = f(amax / f(127))
        q = np.where(fin, np.clip(np.rint((v * inv).astype(f)), -127, 127), 0).astype(np.int8)
    else:
        scale = f(0)
        q = np.zeros(v.size, np.int8)
    with np.errstate(over="ignore"):  # q * scale may round past the float32 maximum next to it
        e2[idx] = (v - (q.astype(f) * scale).astype(f)).astype(f)
    return q, float(scale), e2


def test_hand_worked():
    d = json.loads(pathlib.Path(os.path.join(GOLD, "quant_worked.json")).read_text())
    e = np.full(d["n"], 7.0, np.float32)
    q, scale, e2 = oracle.quantize_int8(d["vals"], d["idx"], e)
    assert q.tolist() == d["q"] and scale == d["scale"]
    assert e2.tolist() == d["e_new"]


@pytest.mark.parametrize("kind", ["normal", "lognormal", "ties", "specials"])
def test_matches_numpy_and_reconstructs_exactly(kind):
    n, k = 50_000, 1234
    idx = gen.sorted_unique_indices(n, k, 60, 1)
    if kind == "normal":
        v = gen.normal_small(k, 61)
    elif kind == "lognormal":
        v = gen.large_gradient(3, n=k)
    elif kind == "ties":
        v = gen.uniform_ties(k, 9, 62)
    else:
        v = gen.specials(k, 63)
    e = gen.normal_small(n, 64)
    q, scale, e2 = oracle.quantize_int8(v, idx, e)
    nq, nscale, ne2 = numpy_quant(v, idx, e)
    assert np.array_equal(q, nq) and scale == nscale
    both_nan = np.isnan(e2) & np.isnan(ne2)
    assert np.array_equal(e2.view(np.uint32)[~both_nan], ne2.view(np.uint32)[~both_nan])
    mask = np.ones(n, bool)
    mask[idx] = False
    assert np.array_equal(e2[mask].view(np.uint32), e[mask].view(np.uint32))  # untouched elsewhere
    fin = np.isfinite(v)
    assert np.all(np.abs(q.astype(int)) <= 127)
    # exact reconstruction: q*scale + e' == v (Sterbenz: v and q*scale are within a factor 2),
    # wherever q*scale itself does not overflow (only for values next to the float32 maximum)
    with np.errstate(over="ignore"):
        deq32 = (q.astype(np.float32) * np.float32(scale)).astype(np.float64)
    ok = fin & np.isfinite(deq32)
    assert np.array_equal(deq32[ok] + e2[idx][ok].astype(np.float64), v[ok].astype(np.float64))
    # the largest finite magnitude maps to +-127 and every error is at most half a step
    if fin.any() and scale > 0:
        j = np.argmax(np.where(fin, np.abs(v), -1))
        assert abs(int(q[j])) == 127
        assert np.all(np.abs(e2[idx][ok]) <= 0.5 * scale * (1 + 1e-6))
    # non-finite kept values stay whole in the residual
    assert np.all(q[~fin] == 0)
    assert np.array_equal(np.isnan(e2[idx][~fin]), np.isnan(v[~fin]))


def test_zero_and_empty():
    idx = np.array([0, 2], np.int32)
    e = np.ones(3, np.float32)
    q, scale, e2 = oracle.quantize_int8(np.array([0.0, -0.0], np.float32), idx, e)
    assert q.tolist() == [0, 0] and scale == 0.0 and e2.tolist() == [0.0, 1.0, 0.0]
    q, scale, e2 = oracle.quantize_int8(np.zeros(0, np.float32), np.zeros(0, np.int32), e)
    assert q.size == 0 and scale == 0.0 and e2.tolist() == [1.0, 1.0, 1.0]


def test_single_value_round_trip():
    v = np.array([-0.3], np.float32)
    q, scale, e2 = oracle.quantize_int8(v, np.array([0], np.int32), np.zeros(1, np.float32))
    assert q.tolist() == [-127] and e2[0] + np.float32(-127) * np.float32(scale) == v[0]


def _straddling_case():
    """A packet whose rounding depends on computing 127/amax (not 1/(amax/127)):
    an amax where the two reciprocals differ, and a value whose product with
    them falls on opposite sides of a half-integer."""
    f = np.float32
    r = np.random.default_rng(7)
    for _ in range(100_000):
        amax = f(r.uniform(0.5, 2.0))
        inv = f(f(127) / amax)
        alt = f(f(1) / f(amax / f(127)))
        if inv == alt:
            continue
        for qh in range(1, 126):
            v = f((qh + 0.5) / float(inv))
            for cand in (v, np.nextafter(v, f(0)), np.nextafter(v, f(1e9))):
                cand = f(cand)
                if cand >= amax:
                    continue
                if np.rint(f(cand * inv)) != np.rint(f(cand * alt)):
                    return amax, cand
    raise AssertionError("no straddling case found")


def test_reciprocal_is_127_over_amax():
    amax, v = _straddling_case()
    vals = np.array([amax, v], np.float32)
    idx = np.array([0, 1], np.int32)
    q, scale, e2 = oracle.quantize_int8(vals, idx, np.zeros(2, np.float32))
    nq, nscale, ne2 = numpy_quant(vals, idx, np.zeros(2, np.float32))
    assert q.tolist() == nq.tolist() and scale == nscale
