"""GPU parity of the fused monitoring statistics.

The oracle's float64 sums run in index order, the kernels' in a fixed tree
order; both add n exact squares, so each is within (n-1) * 2^-53 of the true
sum relative to it, and the test allows twice that.  The main outputs must be
bit-identical with and without statistics, and the statistics must repeat bit
for bit from run to run."""
import numpy as np
import pytest
import torch

import error_feedback_gradient_amd as efg
import gen
import oracle
from gpu_util import assert_bits_equal, device, host, to_dev

pytestmark = pytest.mark.gpu


def close(got, want, nterms):
    tol = 2.0 * max(nterms, 1) * 2.0 ** -53 * abs(want)
    return abs(got - want) <= tol


def topk_with_stats(g, e, k, flags=0):
    dev = device()
    ed = to_dev(e, dev)
    st = torch.full((2,), -1.0, dtype=torch.float64, device=dev)
    v, i = efg.ef_topk_compress(to_dev(g, dev), ed, k, stats=st, flags=flags)
    return host(v), host(i), host(ed), host(st)


@pytest.mark.parametrize("n,k", [(1, 1), (1000, 0), (1000, 1000), (1000, 10), (100_003, 997), (2_000_017, 2000)])
@pytest.mark.parametrize("kind", ["normal", "lognormal", "specials"])
@pytest.mark.parametrize("flags", [0, efg.EF_FLAG_FORCE_FALLBACK])
def test_topk_stats(n, k, kind, flags):
    g = {"normal": lambda: gen.normal_small(n, 500, n), "lognormal": lambda: gen.large_gradient(5, n=n),
         "specials": lambda: gen.specials(n, 501, n)}[kind]()
    e = gen.normal_small(n, 502, n, scale=0.1)
    v, i, en, st = topk_with_stats(g, e, k, flags)
    ov, oi, oe, _ = oracle.topk(g, e, k)
    assert_bits_equal(i, oi, "idx")
    assert_bits_equal(v, ov, "vals")
    assert close(st[0], oracle.sumsq(ov), k), (st[0], oracle.sumsq(ov))
    assert close(st[1], oracle.sumsq(oe), n), (st[1], oracle.sumsq(oe))


def test_stats_do_not_change_outputs_and_repeat():
    dev = device()
    n, k = 3_000_017, 3001
    g = gen.large_gradient(8, n=n)
    e0 = gen.normal_small(n, 503, scale=1e-3)
    outs = []
    for with_stats in (False, True, True):
        ed = to_dev(e0, dev)
        st = torch.zeros(2, dtype=torch.float64, device=dev) if with_stats else None
        v, i = efg.ef_topk_compress(to_dev(g, dev), ed, k, stats=st)
        outs.append((host(v), host(i), host(ed), None if st is None else host(st)))
    for a, b in zip(outs[0][:3], outs[1][:3]):
        assert np.array_equal(np.asarray(a).view(np.uint8), np.asarray(b).view(np.uint8))
    assert np.array_equal(outs[1][3].view(np.uint64), outs[2][3].view(np.uint64))


@pytest.mark.parametrize("flags", [0, efg.EF_FLAG_FORCE_FALLBACK])
def test_segmented_stats_per_tensor(flags):
    dev = device()
    sizes = [7, 0, 1, 300, 64, 1001, 5, 16385, 40_000, 70_001, 2]
    ks = [3, 0, 1, 0, 64, 17, 5, 160, 400, 701, 2]
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    n = int(off[-1])
    g = gen.normal_small(n, 504)
    e = gen.normal_small(n, 505, scale=0.2)
    ed = to_dev(e, dev)
    st = torch.full((2 * len(ks),), -1.0, dtype=torch.float64, device=dev)
    v, i = efg.ef_topk_compress_segmented(to_dev(g, dev), ed, off, ks, stats=st, flags=flags)
    st = host(st)
    ov, oi, oe, _ = oracle.topk_segmented(g, e, off, ks)
    assert_bits_equal(host(i), oi, "idx")
    assert_bits_equal(host(ed), oe, "e")
    o = 0
    for s in range(len(ks)):
        a, b = off[s], off[s + 1]
        assert close(st[2 * s], oracle.sumsq(ov[o:o + ks[s]]), ks[s]), s
        assert close(st[2 * s + 1], oracle.sumsq(oe[a:b]), b - a), s
        o += ks[s]


@pytest.mark.parametrize("n", [1, 9, 1000, 100_003, 3_000_001])
def test_sign_stats(n):
    dev = device()
    g = gen.normal_small(n, 506, n, scale=2.0)
    e = gen.specials(n, 507, n) if n > 100 else gen.normal_small(n, 507, n)
    m = gen.normal_small(n, 508, n)
    ed, md = to_dev(e, dev), to_dev(m, dev)
    st = torch.full((4,), -1.0, dtype=torch.float64, device=dev)
    s, b = efg.ef_sign_compress(to_dev(g, dev), ed, md, 0.9, 5.0, stats=st)
    st = host(st)
    oe, om, os_, ob, _ = oracle.sign(g, e, m, 0.9, 5.0)
    assert_bits_equal(host(s), os_, "sign")
    assert close(st[0], oracle.sumsq(oe), n) and close(st[1], oracle.sumsq(om), n), st
    assert st[2] == np.count_nonzero(os_ == 1) and st[3] == np.count_nonzero(os_ == -1)
