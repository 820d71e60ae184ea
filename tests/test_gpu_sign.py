"""GPU parity of the 1-bit sign error-feedback path against the CPU oracle.

Signs, packed bits and the non-finite count must match bit for bit; the
residual and momentum are held to 2 ulp per step and 1e-5 relative over 50
chained steps, and are expected (and reported) to match exactly."""
import numpy as np
import pytest
import torch

import error_feedback_gradient_amd as efg
import gen
import oracle
from gpu_util import assert_bits_equal, bits, device, host, say, to_dev

pytestmark = pytest.mark.gpu


def ulp_diff(a, b):
    a = bits(a).astype(np.int64)
    b = bits(b).astype(np.int64)
    # map to a monotone integer line so that ulp distance is a difference
    a = np.where(a & 0x80000000, 0x80000000 - a, a)
    b = np.where(b & 0x80000000, 0x80000000 - b, b)
    return np.abs(a - b)


def run_gpu(g, e, m, beta1, clip):
    dev = device()
    ed, md = to_dev(e, dev), to_dev(m, dev)
    nf = torch.zeros(1, dtype=torch.int32, device=dev)
    s, b = efg.ef_sign_compress(to_dev(g, dev), ed, md, beta1, clip, nonfinite=nf)
    return host(ed), host(md), host(s), host(b), int(host(nf)[0])


SIZES = [1, 7, 8, 9, 63, 64, 65, 1000, 4097, 100_003, 1_000_005]


@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("beta1,clip", [(0.9, 5.0), (0.5, 5.0), (0.0, np.inf), (1.0, 5.0), (0.8, 0.25)])
def test_small(n, beta1, clip):
    g = gen.normal_small(n, 200, n, scale=3.0)
    e = gen.normal_small(n, 201, n)
    m = gen.normal_small(n, 202, n)
    got = run_gpu(g, e, m, beta1, clip)
    want = oracle.sign(g, e, m, beta1, clip)
    for a, b, what in zip(got[:4], want[:4], ("e", "m", "sign", "bits")):
        assert_bits_equal(a, b, f"{what} n={n} b={beta1}")
    assert got[4] == want[4]


@pytest.mark.parametrize("n", [9, 1000, 65_537])
def test_specials(n):
    g = gen.specials(n, 203, n)
    e = gen.specials(n, 204, n)
    m = gen.normal_small(n, 205, n)
    got = run_gpu(g, e, m, 0.9, 5.0)
    want = oracle.sign(g, e, m, 0.9, 5.0)
    assert_bits_equal(got[2], want[2], "sign")
    assert_bits_equal(got[3], want[3], "bits")
    for a, b, what in ((got[0], want[0], "e"), (got[1], want[1], "m")):
        nan = np.isnan(a) & np.isnan(b)
        assert np.array_equal(np.isnan(a), np.isnan(b)), what
        assert_bits_equal(a[~nan], b[~nan], what)
    assert got[4] == want[4]


def test_optional_outputs():
    dev = device()
    n = 10_001
    g = gen.normal_small(n, 206)
    e = gen.normal_small(n, 207)
    m = gen.normal_small(n, 208)
    ed, md = to_dev(e, dev), to_dev(m, dev)
    s, b = efg.ef_sign_compress(to_dev(g, dev), ed, md, 0.9, 5.0, want_sign=False, want_bits=False)
    assert s is None and b is None
    oe, om, _, _, _ = oracle.sign(g, e, m, 0.9, 5.0)
    assert_bits_equal(host(ed), oe, "e without optional outputs")
    assert_bits_equal(host(md), om, "m without optional outputs")


def test_full_size_fifty_steps():
    """N = 340M, 50 chained steps from zero state, beta1 = 0.9, clip 5.  Inputs
    are drawn on the device (torch's seeded generator, same law as the numpy
    stream) and the oracle follows a random sample of 200,000 positions through
    all 50 steps on host copies of those inputs (the update is elementwise, so
    its chain is exact there).  Signs and bits are compared at every step, e
    and m within 2 ulp at every step and within 1e-5 relative to max |ref|
    after 50 steps."""
    dev = device()
    n = gen.SIGN_N
    pos = np.sort(gen.rng(209).choice(n, size=200_000, replace=False))
    ed = torch.zeros(n, dtype=torch.float32, device=dev)
    md = torch.zeros(n, dtype=torch.float32, device=dev)
    sd = torch.empty(n, dtype=torch.int8, device=dev)
    bd = torch.empty((n + 7) // 8, dtype=torch.uint8, device=dev)
    pos_d = torch.from_numpy(pos).to(dev)
    e_ref = np.zeros(pos.size, np.float32)
    m_ref = np.zeros(pos.size, np.float32)
    worst = 0
    for t in range(gen.SIGN_STEPS):
        gd = gen.sign_gradient_device(t, n, dev)
        g_s = host(gd[pos_d])
        efg.ef_sign_compress(gd, ed, md, gen.SIGN_BETA1, gen.SIGN_CLIP, sign_out=sd, bits=bd)
        e_ref, m_ref, s_ref, _, _ = oracle.sign(g_s, e_ref, m_ref, gen.SIGN_BETA1, gen.SIGN_CLIP)
        eg, mg, sg = host(ed[pos_d]), host(md[pos_d]), host(sd[pos_d])
        assert_bits_equal(sg, s_ref, f"sign step {t}")
        bit = (host(bd[pos_d >> 3]) >> (pos & 7)) & 1
        assert np.array_equal(bit, (s_ref == 1).astype(np.uint8)), f"bits step {t}"
        worst = max(worst, int(ulp_diff(eg, e_ref).max()), int(ulp_diff(mg, m_ref).max()))
        assert worst <= 2, (t, worst)
        if t % 10 == 9:
            say(f"sign chain step {t + 1}: max ulp difference so far {worst}")
    say(f"sign chain: max ulp difference over 50 steps = {worst}")
    for a, b in ((eg, e_ref), (mg, m_ref)):
        assert np.max(np.abs(a.astype(np.float64) - b)) <= 1e-5 * max(1e-30, np.max(np.abs(b)))
