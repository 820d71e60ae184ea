"""GPU parity of the top-k error-feedback path against the CPU oracle.

Outputs (vals, idx, updated e, non-finite count) must match bit for bit."""
import numpy as np
import pytest
import torch

import error_feedback_gradient_amd as efg
import gen
import oracle
from gpu_util import assert_bits_equal, check_topk_invariants_device, device, host, say, to_dev

pytestmark = pytest.mark.gpu


def run_gpu(g, e, k, flags=0):
    dev = device()
    gd, ed = to_dev(g, dev), to_dev(e, dev)
    nf = torch.zeros(1, dtype=torch.int32, device=dev)
    vals, idx = efg.ef_topk_compress(gd, ed, k, nonfinite=nf, flags=flags)
    return host(vals), host(idx), host(ed), int(host(nf)[0])


def check(g, e, k, flags=0, what=""):
    v, i, en, nf = run_gpu(g, e, k, flags)
    ov, oi, oe, onf = oracle.topk(g, e, k)
    assert_bits_equal(i, oi, f"idx {what}")
    assert_bits_equal(v, ov, f"vals {what}")
    assert_bits_equal(en, oe, f"e {what}")
    assert nf == onf, (what, nf, onf)


SIZES = [1, 2, 3, 5, 63, 64, 65, 255, 257, 1000, 4099, 16383, 16384, 16385, 50_001, 100_003, 300_007]


def inputs(n, kind, seed):
    if kind == "normal":
        return gen.normal_small(n, 100, seed, n), gen.normal_small(n, 101, seed, n, scale=0.3)
    if kind == "ties":
        return gen.uniform_ties(n, 5, 102, seed, n), gen.uniform_ties(n, 2, 103, seed, n)
    if kind == "specials":
        return gen.specials(n, 104, seed, n), gen.normal_small(n, 105, seed, n)
    if kind == "allsame":
        return np.full(n, 1.5, np.float32), np.zeros(n, np.float32)
    if kind == "lognormal":
        return gen.large_gradient(seed, n=n), np.zeros(n, np.float32)
    raise ValueError(kind)


@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("kind", ["normal", "ties", "specials", "allsame", "lognormal"])
def test_small_sizes(n, kind):
    g, e = inputs(n, kind, 1)
    for k in sorted({0, 1, max(0, n - 1), n, n // 3, max(1, n // 1000), max(1, n // 100)}):
        check(g, e, k, what=f"n={n} {kind} k={k}")


@pytest.mark.parametrize("n,k", [(1000, 10), (100_003, 997), (300_007, 300), (65_536, 3000)])
@pytest.mark.parametrize("kind", ["normal", "ties", "allsame"])
def test_forced_fallback(n, k, kind):
    g, e = inputs(n, kind, 2)
    check(g, e, k, flags=efg.EF_FLAG_FORCE_FALLBACK, what=f"fallback n={n} k={k} {kind}")


def test_forced_fallback_many_units():
    """The exact path over 20,000,003 elements: 1,221 units of 16,384 shared
    out among the write blocks in contiguous ranges (each block's place in
    the output is the totals of the blocks before it), the last unit ragged."""
    n, k = 20_000_003, 20_000
    g, e = inputs(n, "lognormal", 7)
    say(f"forced fallback n={n} k={k}")
    check(g, e, k, flags=efg.EF_FLAG_FORCE_FALLBACK, what=f"fallback n={n} k={k}")


def test_forced_fallback_mixed_segments():
    """The exact path's last select pass collects each block's possible
    survivors (keys with T's top 21 bits or above) into the block's segment;
    a block whose segment overflows places by reading x again.  Here a
    stretch of 300,000 copies of T itself overflows the segments of the
    blocks that cover it while every other block places from its segment,
    and the r ties kept are the lowest-indexed ones."""
    n = 2_000_003
    g = gen.normal_small(n, 211)
    e = np.zeros(n, np.float32)
    v = np.float32(3.0)
    g[700_001:1_000_001] = v
    k = int((np.abs(g) > v).sum()) + 1000
    say(f"forced fallback, mixed segments n={n} k={k}")
    check(g, e, k, flags=efg.EF_FLAG_FORCE_FALLBACK, what="fallback mixed segments")
    check(g, e, k, what="fast path, same input")


def test_clustered_magnitudes_overflow():
    # all large values sit in a few regions: their candidate slots overflow and
    # the rest of their candidates are read again from e
    n, k = 2_000_000, 20_000
    g = gen.normal_small(n, 110, 0, scale=1e-3)
    g[500_000:540_000] = gen.normal_small(40_000, 111, 0, scale=10.0)
    e = np.zeros(n, np.float32)
    check(g, e, k, what="clustered")


@pytest.mark.parametrize("where", ["start", "end", "two", "ties", "residual"])
def test_clustered_regions_recollected(where):
    """Crowded regions at the tensor's start, at its ragged end, in two places,
    full of equal keys, or carried in the residual; several k."""
    n = 3_000_017
    g = gen.normal_small(n, 112, 1, scale=1e-3)
    e = np.zeros(n, np.float32)
    if where == "start":
        g[:30_000] = gen.normal_small(30_000, 113, 1, scale=5.0)
    elif where == "end":
        g[-30_001:] = gen.normal_small(30_001, 114, 1, scale=5.0)
    elif where == "two":
        g[100_003:112_003] = gen.normal_small(12_000, 115, 1, scale=5.0)
        g[2_000_000:2_020_000] = gen.normal_small(20_000, 116, 1, scale=3.0)
    elif where == "ties":
        g[700_000:740_000] = np.float32(2.5)
    else:
        e[1_234_567:1_264_567] = gen.normal_small(30_000, 117, 1, scale=5.0)
    for k in (3000, 10_000, 25_000):
        check(g, e, k, what=f"clustered {where} k={k}")


def test_clustered_flat_layers():
    """A flat call over tensors of very different scales (the usual way a whole
    model's gradient is compressed at once): the top entries crowd into the
    large-scale tensors."""
    r = gen.rng(118)
    sizes = [768] * 20 + [3072] * 4 + [589_824] * 4 + [393_216]
    parts = [gen.normal_small(m, 119, i, scale=float(10.0 ** r.uniform(-4, -1))) for i, m in enumerate(sizes)]
    g = np.concatenate(parts).astype(np.float32)
    e = gen.normal_small(g.size, 120, scale=1e-5)
    for k in (g.size // 1000, g.size // 300):
        check(g, e, k, what=f"flat layers k={k}")


def sampled_chunk_mask(n):
    """Elements the top-k sample reads for a tensor of n elements (chunks of 256
    starting at c * (n - 256) / (S - 1), S = max(256, min(4096, chunks / 16)))."""
    chunks = -(-n // 256)
    S = min(chunks, max(256, min(4096, chunks // 16)))
    m = np.zeros(n, bool)
    for c in range(S):
        st = c * (n - 256) // (S - 1)
        m[st:st + 256] = True
    return m


def test_upper_edge_below_threshold_gives_x_back():
    """The sample sees N(0,1) values only, while k large values sit in chunks it
    does not read: its upper edge T_hi lies below the true threshold, so the
    stream clears e for N(0,1) tail values that are not kept, and the emit must
    give each of them x back (the fast path, not the fallback: the candidates
    fit their slots).  Spread so that no region holds more than a few."""
    n, k = 1_000_000, 1000
    m = sampled_chunk_mask(n)
    g = gen.normal_small(n, 122)
    free = np.flatnonzero(~m)
    big = free[np.linspace(0, free.size - 1, k).astype(np.int64)]
    g[big] = gen.normal_small(k, 123, scale=1.0) + np.float32(20.0)
    check(g, gen.normal_small(n, 124, scale=1e-3), k, what="T_hi below T")
    check(g, gen.normal_small(n, 124, scale=1e-3), k + 300, what="T_hi below T, k beyond the planted values")


def test_candidates_beyond_capacity_fall_back():
    """The sample sees only small values, so the threshold it gives lets most
    of the tensor through: more candidates than the slots hold in total, and
    the exact fallback decides."""
    n, k = 2_000_000, 2000
    m = sampled_chunk_mask(n)
    g = np.where(m, gen.normal_small(n, 121, scale=1e-3), np.float32(1.0)).astype(np.float32)
    g[::7] = np.float32(0.5)
    check(g, np.zeros(n, np.float32), k, what="beyond capacity")


def test_flat_chain_ten_steps():
    """N = 1,000,000 N(0,1), k = 10,000, residual carried over 10 steps."""
    dev = device()
    n, k = gen.FLAT_N, gen.FLAT_K
    e_ref = np.zeros(n, np.float32)
    ed = torch.zeros(n, dtype=torch.float32, device=dev)
    ws = efg.workspace(efg.ef_topk_workspace_bytes(n, k), dev)
    for t in range(gen.FLAT_STEPS):
        g = gen.flat_gradient(t)
        vals, idx = efg.ef_topk_compress(to_dev(g, dev), ed, k, ws=ws)
        ov, oi, e_ref, _ = oracle.topk(g, e_ref, k)
        assert_bits_equal(host(idx), oi, f"idx step {t}")
        assert_bits_equal(host(vals), ov, f"vals step {t}")
        assert_bits_equal(host(ed), e_ref, f"e step {t}")


def test_repeatable_bitwise():
    dev = device()
    n, k = 3_000_017, 3001
    g = gen.large_gradient(7, n=n)
    e0 = gen.normal_small(n, 120, scale=1e-3)
    outs = []
    for _ in range(2):
        ed = to_dev(e0, dev)
        v, i = efg.ef_topk_compress(to_dev(g, dev), ed, k)
        outs.append((host(v), host(i), host(ed)))
    for a, b in zip(outs[0], outs[1]):
        assert np.array_equal(np.asarray(a).view(np.uint32 if a.dtype == np.float32 else a.dtype),
                              np.asarray(b).view(np.uint32 if b.dtype == np.float32 else b.dtype))


def test_guard_zones_untouched():
    dev = device()
    n, k = 100_003, 1000
    g, e = inputs(n, "normal", 9)
    pad = 4096
    gd = torch.full((n + 2 * pad,), 7.0, device=dev)
    ed = torch.full((n + 2 * pad,), 7.0, device=dev)
    gd[pad:pad + n] = to_dev(g, dev)
    ed[pad:pad + n] = to_dev(e, dev)
    vbuf = torch.full((k + 2 * pad,), 7.0, device=dev)
    ibuf = torch.full((k + 2 * pad,), 7, dtype=torch.int32, device=dev)
    efg.ef_topk_compress(gd[pad:pad + n], ed[pad:pad + n], k, vals=vbuf[pad:pad + k], idx=ibuf[pad:pad + k])
    for buf in (gd, ed, vbuf):
        h = host(buf)
        assert np.all(h[:pad] == 7.0) and np.all(h[-pad:] == 7.0)
    hi = host(ibuf)
    assert np.all(hi[:pad] == 7) and np.all(hi[-pad:] == 7)
    ov, oi, oe, _ = oracle.topk(g, e, k)
    assert_bits_equal(host(vbuf)[pad:pad + k], ov, "vals in guarded buffer")


# ------------------------------------------------------------- segmented
def seg_check(sizes, ks, seed, kind="normal", flags=0):
    dev = device()
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    n = int(off[-1])
    g, e = inputs(n, kind, seed) if n > 0 else (np.zeros(0, np.float32), np.zeros(0, np.float32))
    ed = to_dev(e, dev)
    nf = torch.zeros(1, dtype=torch.int32, device=dev)
    v, i = efg.ef_topk_compress_segmented(to_dev(g, dev), ed, off, ks, nonfinite=nf, flags=flags)
    ov, oi, oe, onf = oracle.topk_segmented(g, e, off, ks)
    assert_bits_equal(host(i), oi, "seg idx")
    assert_bits_equal(host(v), ov, "seg vals")
    assert_bits_equal(host(ed), oe, "seg e")
    assert int(host(nf)[0]) == onf


@pytest.mark.parametrize("kind", ["normal", "ties", "specials"])
def test_segmented_ragged(kind):
    # unaligned offsets, empty tensors, k = 0 and k = n tensors, sizes across region boundaries
    sizes = [7, 0, 1, 300, 64, 1001, 5, 16385, 3, 40_000, 0, 70_001, 2]
    ks = [3, 0, 1, 0, 64, 17, 5, 160, 2, 400, 0, 701, 2]
    seg_check(sizes, ks, 3, kind)
    seg_check(sizes, ks, 4, kind, flags=efg.EF_FLAG_FORCE_FALLBACK)


def seg_check_arrays(g, e, sizes, ks, what):
    dev = device()
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    ed = to_dev(e, dev)
    v, i = efg.ef_topk_compress_segmented(to_dev(g, dev), ed, off, ks)
    ov, oi, oe, _ = oracle.topk_segmented(g, e, off, ks)
    assert_bits_equal(host(i), oi, f"seg idx {what}")
    assert_bits_equal(host(v), ov, f"seg vals {what}")
    assert_bits_equal(host(ed), oe, f"seg e {what}")


def test_segmented_crowded_regions():
    """Several tensors, some with crowded regions (their slots overflow and are
    read again), one whose sample sees only small values (more candidates than
    its slots: the exact fallback), and plain ones, in one call: each tensor's
    dense list sits at its own base."""
    sizes = [100_003, 2_000_000, 50_000, 3_000_017, 2_000_000, 700_001]
    parts, es = [], []
    for t, m in enumerate(sizes):
        x = gen.normal_small(m, 130, t, scale=1e-3)
        if t == 1:
            x[400_000:440_000] = gen.normal_small(40_000, 131, t, scale=5.0)
        if t == 3:
            x[5:20_005] = gen.normal_small(20_000, 132, t, scale=5.0)
            x[-30_000:] = np.float32(3.0)
        if t == 4:
            x = np.where(sampled_chunk_mask(m), x, np.float32(1.0)).astype(np.float32)
        parts.append(x)
        es.append(gen.normal_small(m, 133, t, scale=1e-4))
    g, e = np.concatenate(parts), np.concatenate(es)
    for ks in ([1000, 20_000, 500, 30_000, 2000, 7000], [100, 5000, 1, 25_000, 20_000, 70_000]):
        seg_check_arrays(g, e, sizes, np.array(ks, np.int64), f"ks={ks}")


def test_segmented_many_small():
    r = gen.rng(130)
    sizes = r.integers(1, 3000, size=700).tolist()
    ks = [int(r.integers(0, s + 1)) for s in sizes]
    seg_check(sizes, ks, 5)


def test_segmented_five_thousand_tensors():
    """5,000 tensors of 1 to 400 elements (plus two long ones): the kernels'
    64-way search for a block's tensor takes three rounds over these tables,
    and the plan (about 560 KB) goes through the staging ring."""
    r = gen.rng(131)
    sizes = r.integers(1, 400, size=5000).tolist()
    sizes[1234] = 300_007
    sizes[4321] = 150_001
    ks = [int(r.integers(0, s + 1)) if s < 1000 else s // 100 for s in sizes]
    seg_check(sizes, ks, 6)
    seg_check(sizes, ks, 7, "ties")


def test_segmented_bert_two_steps():
    """The BERT-base layout (194 tensors, 108,888,576 elements), two chained steps."""
    dev = device()
    off, ks = gen.bert_segments()
    n = int(off[-1])
    ed = torch.zeros(n, dtype=torch.float32, device=dev)
    e_ref = np.zeros(n, np.float32)
    ws = efg.workspace(efg.ef_topk_segmented_workspace_bytes(off, ks), dev)
    for t in range(2):
        g = gen.bert_gradient(t)
        v, i = efg.ef_topk_compress_segmented(to_dev(g, dev), ed, off, ks, ws=ws)
        say(f"bert step {t}: oracle ...")
        ov, oi, e_ref, _ = oracle.topk_segmented(g, e_ref, off, ks)
        assert_bits_equal(host(i), oi, f"bert idx step {t}")
        assert_bits_equal(host(v), ov, f"bert vals step {t}")
        assert_bits_equal(host(ed), e_ref, f"bert e step {t}")


# ------------------------------------------------------------- full size
def test_large_invariants_two_steps():
    """N = 1.3e9, k = 1.3e6: the result is pinned by the invariants that make the
    kept set unique (exactly k; every kept key >= every dropped key; ties by
    lower index; vals are x bit for bit; e is x where dropped and +0 where kept),
    with x = g + e evaluated on the host by numpy.  Gradients are drawn on the
    device (torch's seeded generator, same law as the numpy stream) and copied
    to the host before the call."""
    dev = device()
    n, k = gen.LARGE_N, gen.LARGE_K
    free, _ = torch.cuda.mem_get_info(dev)
    if free < 4 * 4 * n + (1 << 30):
        pytest.skip("not enough device memory")
    ed = torch.zeros(n, dtype=torch.float32, device=dev)
    e_prev = np.zeros(n, np.float32)
    ws = efg.workspace(efg.ef_topk_workspace_bytes(n, k), dev)
    st = torch.zeros(2, dtype=torch.float64, device=dev)
    for t in range(2):
        gd = gen.large_gradient_device(t, n, dev)
        g = host(gd)
        v, i = efg.ef_topk_compress(gd, ed, k, ws=ws, stats=st if t == 1 else None)
        vh, ih, eh = host(v), host(i), host(ed)
        del gd
        say(f"large step {t}: checking invariants")
        x = g + e_prev
        del g
        key = x.view(np.uint32) & np.uint32(0x7FFFFFFF)
        assert ih.size == k and np.all(np.diff(ih) > 0) and ih[0] >= 0 and ih[-1] < n
        assert_bits_equal(vh, x[ih], f"large vals step {t}")
        kept = np.zeros(n, bool)
        kept[ih] = True
        T = key[ih].min()
        drop_max = np.max(key[~kept])
        assert T >= drop_max
        if T == drop_max:
            assert ih[key[ih] == T].max() < np.nonzero((key == T) & ~kept)[0].min()
        del key, kept
        x[ih] = 0.0
        assert_bits_equal(eh, x, f"large e step {t}")
        e_prev = x  # host-computed state, equal to the GPU's bit for bit
        del eh
        if t == 1:
            # monitoring statistics against float64 sums of the host copies
            sh = host(st)
            v64 = vh.astype(np.float64)
            sent = float(np.dot(v64, v64))
            resid = 0.0
            for lo in range(0, n, 1 << 26):
                c = x[lo:lo + (1 << 26)].astype(np.float64)
                resid += float(np.dot(c, c))
            assert abs(sh[0] - sent) <= 2 * k * 2.0 ** -53 * sent
            assert abs(sh[1] - resid) <= 2 * n * 2.0 ** -53 * resid
        say(f"large step {t}: ok")


def test_large_forced_fallback_two_steps():
    """The exact fallback at the headline size, N = 1.3e9, k = 1.3e6, two
    chained steps (the second on a residual the fallback wrote): its raw units
    address e past 4 GiB and its per-tensor unit scan covers about 635,000
    units.  Checked on the device by the invariants that fix the result."""
    dev = device()
    n, k = gen.LARGE_N, gen.LARGE_K
    free, _ = torch.cuda.mem_get_info(dev)
    if free < 24 * n + (1 << 30):
        pytest.skip("not enough device memory")
    e = torch.zeros(n, dtype=torch.float32, device=dev)
    ws = efg.workspace(efg.ef_topk_workspace_bytes(n, k), dev)
    nf = torch.zeros(1, dtype=torch.int32, device=dev)
    for t in range(2):
        say(f"large forced fallback step {t}")
        g = gen.large_gradient_device(t, n, dev)
        x = g + e  # float32 elementwise on the device, as the kernel adds
        v, i = efg.ef_topk_compress(g, e, k, ws=ws, nonfinite=nf, flags=efg.EF_FLAG_FORCE_FALLBACK)
        torch.cuda.synchronize()
        del g
        assert int(nf.item()) == 0
        check_topk_invariants_device(x, v, i, e, k)
        del x
        say(f"large forced fallback step {t}: ok")
    del e, ws
    torch.cuda.empty_cache()


def test_segmented_bert_forced_fallback():
    """The BERT-base layout (194 tensors) with every tensor on the exact
    fallback, bit for bit against the oracle, on a residual carried from a
    fast-path step."""
    dev = device()
    off, ks = gen.bert_segments()
    n = int(off[-1])
    ed = torch.zeros(n, dtype=torch.float32, device=dev)
    e_ref = np.zeros(n, np.float32)
    ws = efg.workspace(efg.ef_topk_segmented_workspace_bytes(off, ks), dev)
    for t, flags in ((0, 0), (1, efg.EF_FLAG_FORCE_FALLBACK)):
        g = gen.bert_gradient(t)
        v, i = efg.ef_topk_compress_segmented(to_dev(g, dev), ed, off, ks, ws=ws, flags=flags)
        say(f"bert forced fallback step {t} (flags {flags}): oracle ...")
        ov, oi, e_ref, _ = oracle.topk_segmented(g, e_ref, off, ks)
        assert_bits_equal(host(i), oi, f"bert idx step {t}")
        assert_bits_equal(host(v), ov, f"bert vals step {t}")
        assert_bits_equal(host(ed), e_ref, f"bert e step {t}")


def test_segmented_plan_cache_rotation():
    """More distinct layouts than the plan cache holds (16), each of more than
    11 tensors (so their tables go through the cache's pinned copy), called in
    rotation twice with one workspace, interleaved with a flat call on the
    same workspace: every call equals the oracle, and the workspace status
    word stays 0."""
    dev = device()
    r = gen.rng(150)
    layouts = []
    for j in range(20):
        sizes = r.integers(1, 5000, size=int(r.integers(12, 40))).tolist()
        ks = [int(r.integers(0, s_ + 1)) for s_ in sizes]
        layouts.append((sizes, ks))
    big = max(efg.ef_topk_segmented_workspace_bytes(np.concatenate([[0], np.cumsum(sz)]), ks)
              for sz, ks in layouts)
    ws = efg.workspace(max(big, efg.ef_topk_workspace_bytes(100_000, 1000)), dev)
    for rnd in range(2):
        for j, (sizes, ks) in enumerate(layouts):
            off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
            n = int(off[-1])
            g, e = gen.normal_small(n, 151, rnd, j), gen.normal_small(n, 152, rnd, j, scale=0.1)
            ed = to_dev(e, dev)
            v, i = efg.ef_topk_compress_segmented(to_dev(g, dev), ed, off, ks, ws=ws)
            ov, oi, oe, _ = oracle.topk_segmented(g, e, off, np.array(ks, np.int64))
            assert_bits_equal(host(i), oi, f"idx round {rnd} layout {j}")
            assert_bits_equal(host(v), ov, f"vals round {rnd} layout {j}")
            assert_bits_equal(host(ed), oe, f"e round {rnd} layout {j}")
            assert int(host(efg.ef_topk_workspace_status(ws))[0]) == 0
            if j % 7 == 3:
                gf = gen.normal_small(100_000, 153, rnd, j)
                check(gf, np.zeros(100_000, np.float32), 1000, what="flat between layouts")


def test_workspace_status_zero_after_calls():
    dev = device()
    n, k = 300_007, 3000
    g, e = inputs(n, "normal", 11)
    ws = efg.workspace(efg.ef_topk_workspace_bytes(n, k), dev)
    for flags in (0, efg.EF_FLAG_FORCE_FALLBACK):
        efg.ef_topk_compress(to_dev(g, dev), to_dev(e, dev), k, ws=ws, flags=flags)
        assert int(host(efg.ef_topk_workspace_status(ws))[0]) == 0


def drift_chain(g, n, k, steps, with_stats, dev):
    """`steps` error-feedback steps with the same gradient every step (the
    residual of the slow coordinates grows until it is kept, so values crowd
    just below the threshold); per step the path and candidates of the call
    (ef_topk_workspace_paths).  Returns them, e before the last step and the
    last step's outputs."""
    e = torch.zeros(n, dtype=torch.float32, device=dev)
    ws = efg.workspace(efg.ef_topk_workspace_bytes(n, k), dev)
    vals = torch.empty(k, dtype=torch.float32, device=dev)
    idx = torch.empty(k, dtype=torch.int32, device=dev)
    st = torch.zeros(2, dtype=torch.float64, device=dev) if with_stats else None
    paths = torch.empty((steps, 2), dtype=torch.int32, device=dev)
    e_before = None
    for t in range(steps):
        if t == steps - 1:
            e_before = host(e).copy()
        efg.ef_topk_compress(g, e, k, vals=vals, idx=idx, ws=ws, stats=st)
        efg.ef_topk_workspace_paths(ws, 1, out=paths[t])
    return host(paths), e_before, host(vals), host(idx), host(e)


@pytest.mark.parametrize("n", [4_000_000, 20_000_000])  # split stream / one wave per region
def test_drift_chain_keeps_candidates_few(n):
    """Under a gradient with a drift the residual crowds just below the
    threshold.  The call samples the magnitudes around its previous
    threshold at 1/1024 octave, so the candidates stay near k and no step
    takes the exact fallback; a call that asks for statistics samples the
    12-bit bins only and, as the control, collects many times k.  Both
    chains keep identical results at every step (the path never changes
    them), and the last step matches the oracle."""
    dev = device()
    k = n // 200
    steps = 500
    g_np = gen.large_gradient(3, n=n)
    g = to_dev(g_np, dev)
    p_fine, e_prev, v, i, e_last = drift_chain(g, n, k, steps, False, dev)
    p_ctrl, _, v2, i2, e2 = drift_chain(g, n, k, steps, True, dev)
    tail = p_fine[-100:]
    say(f"n={n} k={k}: fine max {p_fine[:, 1].max() / k:.2f} k, control max {p_ctrl[:, 1].max() / k:.2f} k, "
        f"control fallbacks {int(p_ctrl[:, 0].sum())}")
    assert int(p_fine[:, 0].sum()) == 0, "a step took the exact fallback with the fine window"
    assert tail[:, 1].max() <= 2.5 * k, tail[:, 1].max() / k
    assert p_ctrl[:, 1].max() >= 3 * k or int(p_ctrl[:, 0].sum()) > 0, "the control chain did not crowd"
    assert_bits_equal(i2, i, "idx fine vs control")
    assert_bits_equal(v2, v, "vals fine vs control")
    assert_bits_equal(e2, e_last, "e fine vs control")
    ov, oi, oe, _ = oracle.topk(g_np, e_prev, k)
    assert_bits_equal(i, oi, "idx last step")
    assert_bits_equal(v, ov, "vals last step")
    assert_bits_equal(e_last, oe, "e last step")


def test_workspace_garbage_changes_nothing():
    """Workspace bytes left by anything (the hint of the last threshold
    included) only change the path: random bytes in the workspace, then the
    same call on a cleared workspace, both equal to the oracle."""
    dev = device()
    n, k = 6_000_011, 6000
    g, e = inputs(n, "lognormal", 12)
    ov, oi, oe, _ = oracle.topk(g, e, k)
    nb = efg.ef_topk_workspace_bytes(n, k)
    gz = torch.Generator(device=dev)
    gz.manual_seed(77)
    for fill in ("random", "zero", "ones"):
        ws = efg.workspace(nb, dev)
        if fill == "random":
            ws.copy_(torch.randint(0, 256, (ws.numel(),), generator=gz, device=dev, dtype=torch.int32).to(torch.uint8))
        elif fill == "zero":
            ws.zero_()
        else:
            ws.fill_(255)
        ed = to_dev(e, dev)
        v, i = efg.ef_topk_compress(to_dev(g, dev), ed, k, ws=ws)
        assert_bits_equal(host(i), oi, f"idx {fill}")
        assert_bits_equal(host(v), ov, f"vals {fill}")
        assert_bits_equal(host(ed), oe, f"e {fill}")


def test_workspace_paths_segmented():
    """ef_topk_workspace_paths over a layer-wise call: 1 for every selecting
    tensor after a forced fallback, 0 on the sampled path; 0 and no
    candidates for tensors with k = 0 or k = n; candidates >= k otherwise."""
    dev = device()
    sizes = [70_000, 5, 300_000, 1000, 2_000_000]
    ks = [700, 0, 3000, 1000, 20_000]
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    kk = np.array(ks, np.int64)
    n = int(off[-1])
    g, e = inputs(n, "normal", 21)
    ws = efg.workspace(efg.ef_topk_segmented_workspace_bytes(off, kk), dev)
    for flags, want in ((efg.EF_FLAG_FORCE_FALLBACK, 1), (0, 0)):
        efg.ef_topk_compress_segmented(to_dev(g, dev), to_dev(e, dev), off, kk, ws=ws, flags=flags)
        p = host(efg.ef_topk_workspace_paths(ws, len(ks)))
        for s_, (sz, kv) in enumerate(zip(sizes, ks)):
            if kv in (0, sz):
                assert p[s_, 0] == 0 and p[s_, 1] == 0, (flags, s_, p[s_])
            else:
                assert p[s_, 0] == want, (flags, s_, p[s_])
                assert p[s_, 1] >= kv, (flags, s_, p[s_])


def test_drift_chain_segmented_keeps_candidates_few():
    """The same drift chain over a layer-wise call of 24 tensors of mixed
    sizes and scales (both stream shapes' sizes: the call has more than 4096
    regions): each tensor keeps its own hint, so every tensor's candidates
    stay near its k and none falls back; the chain's results equal those of
    the statistics control (12-bit bins only) at the end, and the last step
    matches the oracle."""
    dev = device()
    rs = np.random.default_rng(2026)
    sizes = [int(x) for x in rs.choice([3000, 50_000, 300_007, 1_000_000, 2_400_000], size=24)]
    ks = [max(1, s_ // 200) for s_ in sizes]
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    kk = np.array(ks, np.int64)
    n, K = int(off[-1]), int(kk.sum())
    g_np = gen.large_gradient(5, n=n)
    for t in range(len(sizes)):
        g_np[off[t]:off[t + 1]] *= np.float32(10.0 ** rs.uniform(-3, 1))
    g = to_dev(g_np, dev)
    steps = 400
    res = []
    for with_stats in (False, True):
        e = torch.zeros(n, dtype=torch.float32, device=dev)
        ws = efg.workspace(efg.ef_topk_segmented_workspace_bytes(off, kk), dev)
        vals = torch.empty(K, dtype=torch.float32, device=dev)
        idx = torch.empty(K, dtype=torch.int32, device=dev)
        st = torch.zeros(2 * len(ks), dtype=torch.float64, device=dev) if with_stats else None
        paths = torch.empty((steps, len(ks), 2), dtype=torch.int32, device=dev)
        e_prev = None
        for t in range(steps):
            if t == steps - 1:
                e_prev = host(e).copy()
            efg.ef_topk_compress_segmented(g, e, off, kk, vals=vals, idx=idx, ws=ws, stats=st)
            efg.ef_topk_workspace_paths(ws, len(ks), out=paths[t])
        res.append((host(paths), e_prev, host(vals), host(idx), host(e)))
    (pf, e_prev, v, i, e_last), (pc, _, v2, i2, e2) = res
    ratio_f = (pf[-100:, :, 1] / kk[None, :]).max()
    ratio_c = (pc[:, :, 1] / kk[None, :]).max()
    say(f"segmented drift: fine max {ratio_f:.2f} k, control max {ratio_c:.2f} k, "
        f"control fallbacks {int(pc[:, :, 0].sum())}")
    assert int(pf[:, :, 0].sum()) == 0, "a tensor took the exact fallback with the fine window"
    assert ratio_f <= 2.5, ratio_f
    assert ratio_c >= 3.0 or int(pc[:, :, 0].sum()) > 0, "the control chain did not crowd"
    assert_bits_equal(i2, i, "idx fine vs control")
    assert_bits_equal(v2, v, "vals fine vs control")
    assert_bits_equal(e2, e_last, "e fine vs control")
    ov, oi, oe, _ = oracle.topk_segmented(g_np, e_prev, off, kk)
    assert_bits_equal(i, oi, "idx last step")
    assert_bits_equal(v, ov, "vals last step")
    assert_bits_equal(e_last, oe, "e last step")
