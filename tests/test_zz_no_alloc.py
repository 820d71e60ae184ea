"""The allocation-free top-k entry point against ef_topk_compress.

ef_topk_compress_noalloc takes its scratch from the library's static device
array instead of a caller workspace.  Through the C ABI it must give the same
bits as ef_topk_compress on the same inputs: packet (vals, idx), residual e,
non-finite count and statistics.  Two calls in a row share the array, the
second on a smaller input (it must not see the first call's leftovers); a
chain of steps carries the residual.  Collected last (its name), so that a
failure here hides no other test."""
import numpy as np
import pytest
import torch

import error_feedback_gradient_amd as efg
import gen
import oracle
from gpu_util import assert_bits_equal, device, host, say, to_dev

pytestmark = pytest.mark.gpu


def both(g, e, k, flags=0):
    """(vals, idx, e, nonfinite, stats) from each entry point on copies of e."""
    dev = device()
    gd = to_dev(g, dev)
    out = []
    for fn in ("ws", "noalloc"):
        ed = to_dev(e, dev)
        nf = torch.full((1,), 12345, dtype=torch.int32, device=dev)
        st = torch.full((2,), -1.0, dtype=torch.float64, device=dev)
        if fn == "ws":
            v, i = efg.ef_topk_compress(gd, ed, k, nonfinite=nf, stats=st, flags=flags)
        else:
            v, i = efg.ef_topk_compress_noalloc(gd, ed, k, nonfinite=nf, stats=st, flags=flags)
        out.append((host(v), host(i), host(ed), host(nf), host(st)))
    return out


def same(a, b, what):
    for x, y, name in zip(a, b, ("vals", "idx", "e", "nonfinite", "stats")):
        if x.dtype == np.float64:
            assert np.array_equal(x.view(np.uint64), y.view(np.uint64)), f"{what}: {name}"
        else:
            assert_bits_equal(x, y, f"{what}: {name}")


def test_noalloc_two_calls_second_smaller():
    n1, k1 = 3_000_017, 30_000
    n2, k2 = 200_003, 701
    g1, e1 = gen.large_gradient(3, n=n1), gen.normal_small(n1, 140, scale=1e-3)
    g2, e2 = gen.specials(n2, 141), gen.normal_small(n2, 142)
    say(f"noalloc: n={n1} k={k1}, then n={n2} k={k2}")
    a, b = both(g1, e1, k1)
    same(a, b, "first call")
    a, b = both(g2, e2, k2)
    same(a, b, "second, smaller call")
    # the static scratch's status word: no stray index in either call
    assert int(host(efg.ef_topk_workspace_status(None, device=device()))[0]) == 0
    # and the oracle agrees with the second call
    ov, oi, oe, onf = oracle.topk(g2, e2, k2)
    assert_bits_equal(b[1], oi, "idx vs oracle")
    assert_bits_equal(b[0], ov, "vals vs oracle")
    assert_bits_equal(b[2], oe, "e vs oracle")
    assert int(b[3][0]) == onf


@pytest.mark.parametrize("n,k", [(1, 1), (1000, 0), (4099, 4099), (65_536, 3000), (1_000_000, 10_000)])
def test_noalloc_sizes(n, k):
    g, e = gen.normal_small(n, 143, n), gen.normal_small(n, 144, n, scale=0.3)
    a, b = both(g, e, k)
    same(a, b, f"n={n} k={k}")


def test_noalloc_forced_fallback_then_fast_path():
    n = 2_000_003
    g, e = gen.large_gradient(4, n=n), np.zeros(n, np.float32)
    a, b = both(g, e, 2000, flags=efg.EF_FLAG_FORCE_FALLBACK)
    same(a, b, "forced fallback")
    a, b = both(g[:500_001], e[:500_001], 500)
    same(a, b, "fast path after the fallback")


def test_noalloc_flat_chain():
    """The flat workload's chain (N = 1e6, k = 1e4), 10 steps, residual carried
    through the allocation-free call, against the workspace call's chain."""
    dev = device()
    n, k = gen.FLAT_N, gen.FLAT_K
    ea = torch.zeros(n, device=dev)
    eb = torch.zeros(n, device=dev)
    ws = efg.workspace(efg.ef_topk_workspace_bytes(n, k), dev)
    for t in range(gen.FLAT_STEPS):
        gd = to_dev(gen.flat_gradient(t), dev)
        va, ia = efg.ef_topk_compress(gd, ea, k, ws=ws)
        vb, ib = efg.ef_topk_compress_noalloc(gd, eb, k)
        assert_bits_equal(host(ib), host(ia), f"idx step {t}")
        assert_bits_equal(host(vb), host(va), f"vals step {t}")
        assert_bits_equal(host(eb), host(ea), f"e step {t}")


def test_noalloc_rejects_beyond_scratch():
    dev = device()
    n = 1 << 24
    k = n // 10
    assert efg.ef_topk_workspace_bytes(n, k) > efg.EF_TOPK_NOALLOC_SCRATCH_BYTES
    g = torch.zeros(n, device=dev)
    e = torch.zeros(n, device=dev)
    with pytest.raises(efg.EfError) as ei:
        efg.ef_topk_compress_noalloc(g, e, k)
    assert ei.value.code == efg.EF_EWS
