"""Pins of the oracle's Adam warm-up step and 1-bit Adam compression-phase
update (CPU only).

Independent references: torch.optim.Adam (textbook Adam with bias
correction, CPU float32), closed forms for constant and zero gradients, and
the already pinned sign compression (orc_sign) for the momentum on the
exchanged signs.
"""
import math

import numpy as np
import pytest
import torch

import gen
import oracle

B1, B2, EPS, LR = 0.9, 0.999, 1e-8, 2e-5


def run_adam(g_steps, w0, lr=LR, beta1=B1, beta2=B2, eps=EPS):
    m = np.zeros_like(w0)
    v = np.zeros_like(w0)
    w = w0.copy()
    for t, g in enumerate(g_steps, start=1):
        ss, sb = oracle.adam_scalars(lr, beta1, beta2, t)
        m, v, w, _ = oracle.adam_step(g, m, v, w, beta1, beta2, ss, sb, eps)
    return m, v, w


def test_matches_torch_adam():
    n, T = 20_000, 12
    r = np.random.default_rng(3)
    w0 = r.standard_normal(n).astype(np.float32)
    gs = [(r.standard_normal(n) * np.exp(r.uniform(-6, 2, n))).astype(np.float32) for _ in range(T)]
    m, v, w = run_adam(gs, w0, lr=1e-3)
    p = torch.nn.Parameter(torch.from_numpy(w0.copy()))
    # the betas as the float32 values the library receives, so that 1 - beta is
    # the same (exactly representable) weight on both sides
    b1, b2 = float(np.float32(B1)), float(np.float32(B2))
    opt = torch.optim.Adam([p], lr=1e-3, betas=(b1, b2), eps=EPS, foreach=False)
    for g in gs:
        p.grad = torch.from_numpy(g.copy())
        opt.step()
    st = opt.state[p]
    # torch forms m by lerp, so the two differ by a few roundings of the summands:
    # bound each element by the largest gradient it has seen (and its square for v)
    gmax = np.max(np.abs(np.stack(gs)), axis=0).astype(np.float64)
    assert np.all(np.abs(m - st["exp_avg"].numpy()) <= 1e-6 * gmax + 2e-6 * np.abs(m))
    assert np.all(np.abs(v - st["exp_avg_sq"].numpy()) <= 1e-6 * gmax ** 2 * (1 - B2) + 2e-6 * np.abs(v))
    # each of the T steps rounds w once on each side: allow T ulps of w plus a
    # relative 1e-4 of the total movement
    wt = p.detach().numpy()
    assert np.all(np.abs(w - wt) <= T * np.spacing(np.abs(wt)) + 1e-4 * np.abs(wt - w0))


def test_constant_gradient_closed_form():
    """g constant: m_t = (1-b1^t) g, v_t = (1-b2^t) g^2, so with eps = 0 every
    bias-corrected step moves w by exactly lr * sign(g) (up to rounding)."""
    g = np.array([3.0, -0.25, 1e-3, -7.5, 1e15, -1e-15], np.float32)
    w0 = np.linspace(-1, 1, g.size).astype(np.float32)
    T = 30
    m, v, w = run_adam([g] * T, w0, lr=1e-2, eps=0.0)
    g64 = g.astype(np.float64)
    b1, b2 = float(np.float32(B1)), float(np.float32(B2))  # the float32 betas the step uses
    np.testing.assert_allclose(m, (1 - b1 ** T) * g64, rtol=1e-5)
    np.testing.assert_allclose(v, (1 - b2 ** T) * g64 ** 2, rtol=1e-5)
    np.testing.assert_allclose(w, w0 - T * 1e-2 * np.sign(g64), rtol=0, atol=T * 4e-8)


def test_zero_gradient_leaves_state():
    w0 = gen.normal_small(1000, 5)
    m, v, w = run_adam([np.zeros(1000, np.float32)] * 3, w0)
    assert np.all(m == 0) and np.all(v == 0)
    assert np.array_equal(w.view(np.uint32), w0.view(np.uint32))


def test_eps_dominates_tiny_variance():
    """|g| << eps: the step is lr * g / eps in the limit (float64 closed form)."""
    g = np.full(8, 1e-12, np.float32)
    w0 = np.zeros(8, np.float32)
    _, _, w = run_adam([g], w0, lr=1.0, eps=1e-6)
    # mhat = g, sqrt(vhat) = g: step = g / (g + eps)
    np.testing.assert_allclose(w, -1e-12 / (1e-12 + 1e-6), rtol=1e-5)


def test_onebit_update_single_worker_equals_fused_sign_momentum():
    n = 50_003
    g = gen.sign_gradient(0, n=n)
    e = gen.normal_small(n, 6, scale=1e-3)
    m = gen.normal_small(n, 7, scale=1e-2)
    v = np.abs(gen.normal_small(n, 8, scale=1e-4))
    w = gen.normal_small(n, 9)
    e_f, m_f, q_f, _, _ = oracle.sign(g, e, m, B1, 5.0)
    e_c, m_c, q_c, _, _ = oracle.sign(g, e, None, B1, 5.0)
    assert m_c is None
    assert np.array_equal(e_c.view(np.uint32), e_f.view(np.uint32)) and np.array_equal(q_c, q_f)
    ss, sb = oracle.adam_scalars(LR, B1, B2, 20, 10)
    m2, w2, _ = oracle.onebit_adam_update(q_c, 1, m, v, w, B1, ss, sb, EPS)
    assert np.array_equal(m2.view(np.uint32), m_f.view(np.uint32))


@pytest.mark.parametrize("nworkers", [1, 2, 3, 7, 127])
def test_onebit_update_is_adam_on_the_averaged_signs_with_frozen_variance(nworkers):
    """The update equals a full Adam step fed ghat = qsum / nworkers with
    beta2 = 1 (v' = 1*v + 0*g^2 = v): the variance is frozen."""
    n = 20_000
    r = np.random.default_rng(nworkers)
    qsum = np.zeros(n, np.int64)
    for _ in range(nworkers):
        qsum += r.integers(-1, 2, n)
    qsum = qsum.astype(np.int8)
    m = gen.normal_small(n, 10, scale=0.1)
    v = np.abs(gen.normal_small(n, 11, scale=1e-3))
    w = gen.normal_small(n, 12)
    ss, sb = oracle.adam_scalars(1e-3, B1, B2, 50, 20)
    m2, w2, bad = oracle.onebit_adam_update(qsum, nworkers, m, v, w, B1, ss, sb, EPS)
    ghat = (qsum.astype(np.float32) / np.float32(nworkers)).astype(np.float32)
    m3, v3, w3, _ = oracle.adam_step(ghat, m, v, w, B1, 1.0, ss, sb, EPS)
    assert np.array_equal(v3.view(np.uint32), v.view(np.uint32))
    assert np.array_equal(m2.view(np.uint32), m3.view(np.uint32))
    assert np.array_equal(w2.view(np.uint32), w3.view(np.uint32))
    # and the momentum is the EMA of the worker mean (float64 closed form)
    b1 = float(np.float32(B1))
    a, b = b1 * m.astype(np.float64), (1 - b1) * qsum.astype(np.float64) / nworkers
    assert np.all(np.abs(m2 - (a + b)) <= 2.5 * 2.0 ** -24 * (np.abs(a) + np.abs(b)) * 2)
    assert bad == 0


def test_non_finite_counts():
    g = np.array([np.inf, 1.0, np.nan, 0.0], np.float32)
    z = np.zeros(4, np.float32)
    ss, sb = oracle.adam_scalars(LR, B1, B2, 1)
    m, v, w, bad = oracle.adam_step(g, z, z, z, B1, B2, ss, sb, EPS)
    # inf: m inf, v inf, w nan (inf/inf);  nan: all three nan
    assert bad == 6


def test_scalars():
    b1, b2 = float(np.float32(0.9)), float(np.float32(0.999))
    ss, sb = oracle.adam_scalars(2e-5, 0.9, 0.999, 1)
    assert ss == float(np.float32(2e-5 / (1 - b1))) and sb == float(np.float32(math.sqrt(1 - b2)))
    ss, sb = oracle.adam_scalars(2e-5, 0.9, 0.999, 100, 10)
    assert sb == float(np.float32(math.sqrt(1 - b2 ** 10)))


@pytest.mark.parametrize("nworkers", [1, 3, 8])
def test_onebit_update_var_is_torch_adam_fed_the_averaged_signs(nworkers):
    """The 1-bit step that keeps updating the variance is textbook Adam (here
    torch.optim.Adam) fed ghat = qsum / nworkers, ghat formed by torch."""
    n, T = 20_000, 10
    r = np.random.default_rng(40 + nworkers)
    w0 = r.standard_normal(n).astype(np.float32)
    qs = []
    for _ in range(T):
        q = np.zeros(n, np.int64)
        for _ in range(nworkers):
            q += r.integers(-1, 2, n)
        qs.append(q.astype(np.int8))
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    w = w0.copy()
    for t, q in enumerate(qs, start=1):
        ss, sb = oracle.adam_scalars(1e-3, B1, B2, t)
        m, v, w, _ = oracle.onebit_adam_update_var(q, nworkers, m, v, w, B1, B2, ss, sb, EPS)
    p = torch.nn.Parameter(torch.from_numpy(w0.copy()))
    b1, b2 = float(np.float32(B1)), float(np.float32(B2))
    opt = torch.optim.Adam([p], lr=1e-3, betas=(b1, b2), eps=EPS, foreach=False)
    for q in qs:
        p.grad = torch.from_numpy(q).to(torch.float32) / nworkers
        opt.step()
    st = opt.state[p]
    assert np.all(np.abs(m - st["exp_avg"].numpy()) <= 1e-6 + 2e-6 * np.abs(m))
    assert np.all(np.abs(v - st["exp_avg_sq"].numpy()) <= 1e-6 * (1 - B2) + 2e-6 * np.abs(v))
    wt = p.detach().numpy()
    assert np.all(np.abs(w - wt) <= T * np.spacing(np.abs(wt)) + 1e-4 * np.abs(wt - w0))
