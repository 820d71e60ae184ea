"""GPU parity of the Adam warm-up step, the compress-only sign step and the
1-bit Adam update against the CPU oracle: bit for bit on m, v, w, e, the
signs and the non-finite counts at sizes across region boundaries with ragged
tails, and through a full run of the adam workload (N = 340M: 3 warm-up steps,
then 1-bit steps) on 200,000 sampled positions that the oracle follows through
every step (all updates are elementwise, so the sampled chain is exact)."""
import numpy as np
import pytest
import torch

import error_feedback_gradient_amd as efg
import gen
import oracle
from gpu_util import assert_bits_equal, device, host, say, to_dev

pytestmark = pytest.mark.gpu

B1, B2, EPS = gen.ADAM_BETA1, gen.ADAM_BETA2, gen.ADAM_EPS
SIZES = [1, 3, 4, 5, 255, 4095, 4096, 4097, 3 * 4096 + 7, 100_003, (1 << 20) + 1]


def state(n, key, kind="normal"):
    if kind == "normal":
        g = gen.normal_small(n, 800, key)
    elif kind == "lognormal":
        g = gen.large_gradient(key, n=n)
    else:
        g = gen.specials(n, 801, key)
    m = gen.normal_small(n, 802, key, scale=0.05)
    v = np.abs(gen.normal_small(n, 803, key, scale=1e-3)) ** 2
    w = gen.normal_small(n, 804, key, scale=0.02)
    return g, m, v, w


def bits_or_nan_equal(got, want, what):
    nan = np.isnan(got) & np.isnan(want)
    assert np.array_equal(np.isnan(got), np.isnan(want)), what
    assert_bits_equal(got[~nan], want[~nan], what)


@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("kind", ["normal", "lognormal", "specials"])
def test_adam_step(n, kind):
    dev = device()
    g, m, v, w = state(n, n % 997, kind)
    for t, tv in [(1, 1), (7, 7)]:
        ss, sb = efg.adam_scalars(1e-3, B1, B2, t, tv)
        md, vd, wd = to_dev(m, dev), to_dev(v, dev), to_dev(w, dev)
        nf = torch.zeros(1, dtype=torch.int32, device=dev)
        efg.ef_adam_step(to_dev(g, dev), md, vd, wd, B1, B2, ss, sb, EPS, nonfinite=nf)
        om, ov, ow, onf = oracle.adam_step(g, m, v, w, B1, B2, ss, sb, EPS)
        bits_or_nan_equal(host(md), om, f"m {kind} n={n} t={t}")
        bits_or_nan_equal(host(vd), ov, f"v {kind} n={n} t={t}")
        bits_or_nan_equal(host(wd), ow, f"w {kind} n={n} t={t}")
        assert int(host(nf)[0]) == onf


@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("nworkers", [1, 2, 3, 64, 127])
def test_onebit_update(n, nworkers):
    dev = device()
    _, m, v, w = state(n, n % 991)
    r = np.random.default_rng(n + nworkers)
    qsum = np.zeros(n, np.int64)
    for _ in range(nworkers):
        qsum += r.integers(-1, 2, n)
    qsum = qsum.astype(np.int8)
    ss, sb = efg.adam_scalars(2e-5, B1, B2, 40, 3)
    md, vd, wd = to_dev(m, dev), to_dev(v, dev), to_dev(w, dev)
    nf = torch.zeros(1, dtype=torch.int32, device=dev)
    efg.ef_onebit_adam_update(to_dev(qsum, dev), nworkers, md, vd, wd, B1, ss, sb, EPS, nonfinite=nf)
    om, ow, onf = oracle.onebit_adam_update(qsum, nworkers, m, v, w, B1, ss, sb, EPS)
    assert_bits_equal(host(md), om, f"m n={n} N={nworkers}")
    assert_bits_equal(host(wd), ow, f"w n={n} N={nworkers}")
    assert_bits_equal(host(vd), v, "v untouched")
    assert int(host(nf)[0]) == onf


@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("nworkers", [1, 3, 64, 127])
def test_onebit_update_var(n, nworkers):
    """The 1-bit step with the variance updated from ghat, against the oracle."""
    dev = device()
    _, m, v, w = state(n, n % 983)
    r = np.random.default_rng(n + 7 * nworkers)
    qsum = np.zeros(n, np.int64)
    for _ in range(nworkers):
        qsum += r.integers(-1, 2, n)
    qsum = qsum.astype(np.int8)
    ss, sb = efg.adam_scalars(2e-5, B1, B2, 40)
    md, vd, wd = to_dev(m, dev), to_dev(v, dev), to_dev(w, dev)
    nf = torch.zeros(1, dtype=torch.int32, device=dev)
    efg.ef_onebit_adam_update_var(to_dev(qsum, dev), nworkers, md, vd, wd, B1, B2, ss, sb, EPS, nonfinite=nf)
    om, ov, ow, onf = oracle.onebit_adam_update_var(qsum, nworkers, m, v, w, B1, B2, ss, sb, EPS)
    assert_bits_equal(host(md), om, f"m n={n} N={nworkers}")
    assert_bits_equal(host(vd), ov, f"v n={n} N={nworkers}")
    assert_bits_equal(host(wd), ow, f"w n={n} N={nworkers}")
    assert int(host(nf)[0]) == onf


@pytest.mark.parametrize("n", [1, 7, 8, 9, 8191, 8192, 8193, 100_003])
def test_compress_only_sign(n):
    dev = device()
    g = gen.sign_gradient(1, n=n)
    e = gen.normal_small(n, 805, scale=1e-3)
    ed = to_dev(e, dev)
    s, b = efg.ef_sign_compress(to_dev(g, dev), ed, None, B1, 5.0)
    oe, om, osg, ob, _ = oracle.sign(g, e, None, B1, 5.0)
    assert om is None
    assert_bits_equal(host(ed), oe, f"e n={n}")
    assert_bits_equal(host(s), osg, f"sign n={n}")
    assert_bits_equal(host(b), ob, f"bits n={n}")


def test_single_worker_split_equals_fused_momentum():
    """compress-only + update(nworkers = 1) gives the fused sign step's m."""
    dev = device()
    n = 300_007
    g = gen.sign_gradient(2, n=n)
    e = gen.normal_small(n, 806, scale=1e-3)
    m = gen.normal_small(n, 807, scale=1e-2)
    v = np.abs(gen.normal_small(n, 808, scale=1e-4))
    w = gen.normal_small(n, 809)
    e1, m1 = to_dev(e, dev), to_dev(m, dev)
    efg.ef_sign_compress(to_dev(g, dev), e1, m1, B1, 5.0)
    e2, m2, w2 = to_dev(e, dev), to_dev(m, dev), to_dev(w, dev)
    q, _ = efg.ef_sign_compress(to_dev(g, dev), e2, None, B1, 5.0)
    ss, sb = efg.adam_scalars(2e-5, B1, B2, 10, 3)
    efg.ef_onebit_adam_update(q, 1, m2, to_dev(v, dev), w2, B1, ss, sb, EPS)
    assert_bits_equal(host(e2), host(e1), "e")
    assert_bits_equal(host(m2), host(m1), "m")


def test_adam_workload_full_run():
    """N = 340M: 3 full-precision warm-up steps, then 5 one-bit steps
    (compress only, signs summed over one worker, update with frozen v), on
    device-drawn inputs; the oracle follows 200,000 sampled positions."""
    dev = device()
    n = gen.ADAM_N
    pos = np.sort(gen.rng(210).choice(n, size=200_000, replace=False))
    pos_d = torch.from_numpy(pos).to(dev)
    w = gen.adam_weights_device(n, dev)
    m = torch.zeros(n, device=dev)
    v = torch.zeros(n, device=dev)
    e = torch.zeros(n, device=dev)
    q = torch.empty(n, dtype=torch.int8, device=dev)
    w_r = host(w[pos_d])
    m_r = np.zeros(pos.size, np.float32)
    v_r = np.zeros(pos.size, np.float32)
    e_r = np.zeros(pos.size, np.float32)
    for t in range(1, gen.ADAM_STEPS + 1):
        g = gen.sign_gradient_device(t, n, dev)
        g_s = host(g[pos_d])
        if t <= gen.ADAM_WARMUP:
            ss, sb = efg.adam_scalars(gen.ADAM_LR, B1, B2, t)
            efg.ef_adam_step(g, m, v, w, B1, B2, ss, sb, EPS)
            m_r, v_r, w_r, _ = oracle.adam_step(g_s, m_r, v_r, w_r, B1, B2, ss, sb, EPS)
        else:
            ss, sb = efg.adam_scalars(gen.ADAM_LR, B1, B2, t, gen.ADAM_WARMUP)
            efg.ef_sign_compress(g, e, None, B1, gen.SIGN_CLIP, sign_out=q, want_bits=False)
            efg.ef_onebit_adam_update(q, 1, m, v, w, B1, ss, sb, EPS)
            e_r, _, q_r, _, _ = oracle.sign(g_s, e_r, None, B1, gen.SIGN_CLIP)
            m_r, w_r, _ = oracle.onebit_adam_update(q_r, 1, m_r, v_r, w_r, B1, ss, sb, EPS)
            assert_bits_equal(host(q[pos_d]), q_r, f"q step {t}")
            assert_bits_equal(host(e[pos_d]), e_r, f"e step {t}")
        assert_bits_equal(host(m[pos_d]), m_r, f"m step {t}")
        assert_bits_equal(host(v[pos_d]), v_r, f"v step {t}")
        assert_bits_equal(host(w[pos_d]), w_r, f"w step {t}")
        say(f"adam run step {t} ({'warm-up' if t <= gen.ADAM_WARMUP else '1-bit'}): sampled state bit-exact")
        del g
