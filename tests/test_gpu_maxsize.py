"""The largest tensor the library accepts, n = 2^31 - 1: an odd length, so
every pass ends on a ragged tail, and kept indices reach 2^31 - 2.  Top-k
(with the block encoding round trip of its packet), random sparsification on
both of its decision paths, sign compression, the two Adam updates and the
decode (onto a zero G, and in one pass with the SGD update), each
checked by the properties that pin its result at any size and, for the
elementwise and random paths, against the oracle at sampled positions that
include the first and last elements."""
import numpy as np
import pytest
import torch

import error_feedback_gradient_amd as efg
import gen
import oracle
from gpu_util import assert_bits_equal, device, host, say, to_dev

pytestmark = pytest.mark.gpu

NMAX = 2**31 - 1


def need(dev, nbytes):
    free, _ = torch.cuda.mem_get_info(dev)
    if free < nbytes:
        pytest.skip(f"needs {nbytes / 2**30:.0f} GiB of free device memory")


def positions(seed, m=200_000):
    """Sorted sample of positions: random ones plus the first and last 4096."""
    r = np.random.default_rng(seed)
    pos = np.concatenate([r.integers(0, NMAX, m), np.arange(4096), np.arange(NMAX - 4096, NMAX)])
    return np.unique(pos).astype(np.int64)


def f32_bits(t):
    return t.view(torch.int32)


def test_topk_max_size_two_steps():
    dev = device()
    n, k = NMAX, NMAX // 1000
    need(dev, 26 * n)
    e = torch.zeros(n, device=dev)
    ws = efg.workspace(efg.ef_topk_workspace_bytes(n, k), dev)
    for t in range(2):
        say(f"top-k n=2^31-1 step {t}: compress")
        g = gen.large_gradient_device(t, n, dev)
        x = g + e  # float32 elementwise on the device, as the kernel adds
        v, i = efg.ef_topk_compress(g, e, k, ws=ws)
        torch.cuda.synchronize()
        del g
        say(f"top-k n=2^31-1 step {t}: invariants")
        ik = i.long()
        assert i.numel() == k
        assert bool((ik[1:] > ik[:-1]).all()) and int(ik[0]) >= 0 and int(ik[-1]) < n
        assert torch.equal(f32_bits(v), f32_bits(x[ik]))
        key = f32_bits(x) & 0x7FFFFFFF
        kept = torch.zeros(n, dtype=torch.bool, device=dev)
        kept[ik] = True
        T = int(key[ik].min())
        drop_max = int(key.masked_fill(kept, -1).max())
        assert T >= drop_max
        if T == drop_max:  # ties at the threshold: the lower indices are kept
            last_kept = int(ik[key[ik] == T].max())
            first_dropped = int(torch.nonzero((key == T) & ~kept)[0, 0])
            assert last_kept < first_dropped
        del key, kept
        x[ik] = 0.0
        assert torch.equal(f32_bits(e), f32_bits(x))
        del x
    say("top-k n=2^31-1: block encoding round trip")
    mask, cm1, offs, nblk = efg.encode_blocks(i, n)
    back = efg.decode_blocks(mask, cm1, offs, n, k)
    assert torch.equal(back, i)
    del e, ws, v, i, mask, cm1, offs, back
    torch.cuda.empty_cache()


def test_topk_max_size_forced_fallback():
    """The exact fallback at n = 2^31 - 1 (raw units up to the last index,
    kept indices up to 2^31 - 2), on a residual carried from a fast-path step."""
    dev = device()
    n, k = NMAX, NMAX // 1000
    need(dev, 26 * n)
    from gpu_util import check_topk_invariants_device
    e = torch.zeros(n, device=dev)
    ws = efg.workspace(efg.ef_topk_workspace_bytes(n, k), dev)
    for t, flags in ((0, 0), (1, efg.EF_FLAG_FORCE_FALLBACK)):
        say(f"top-k n=2^31-1 step {t} flags {flags}")
        g = gen.large_gradient_device(10 + t, n, dev)
        x = g + e
        v, i = efg.ef_topk_compress(g, e, k, ws=ws, flags=flags)
        torch.cuda.synchronize()
        del g
        check_topk_invariants_device(x, v, i, e, k)
        del x
    del e, ws, v, i
    torch.cuda.empty_cache()


def call_path(ws):
    """'slots' or 'two-pass', from the call state at the start of the workspace
    (float32 S32 at byte 8, float32 S_lo at byte 24, uint32 overflow flag at 28)."""
    b = host(ws[:64]).tobytes()
    s32, slo = np.frombuffer(b, np.float32, 1, 8)[0], np.frombuffer(b, np.float32, 1, 24)[0]
    return "slots" if slo > 0 and np.frombuffer(b, np.uint32, 1, 28)[0] == 0 and s32 >= slo else "two-pass"


@pytest.mark.parametrize("flags", [0, 1])
def test_random_max_size(flags):
    dev = device()
    n, k, seed, step = NMAX, NMAX // 1000, gen.RANDOM_SEED, 3
    need(dev, 22 * n)
    cap = 2 * k + 64
    e = torch.from_numpy(gen.normal_small(1 << 20, 901, scale=1e-3)).to(dev).repeat(2048)[:n].contiguous()
    g = gen.large_gradient_device(7, n, dev)
    x = g + e
    s32 = torch.empty(1, dtype=torch.float32, device=dev)
    ws = efg.workspace(efg.lib().ef_random_sparsify_workspace_bytes(n), dev)
    say(f"random n=2^31-1 flags={flags}: sparsify")
    vals, idx, cnt = efg.ef_random_sparsify(g, e, k, seed, step, cap=cap, sum_out=s32, ws=ws, flags=flags)
    torch.cuda.synchronize()
    del g
    assert call_path(ws) == ("two-pass" if flags else "slots")
    c = int(host(cnt)[0])
    S = np.float32(host(s32)[0])
    assert 0 < c <= cap
    ik = idx[:c].long()
    assert bool((ik[1:] > ik[:-1]).all()) and int(ik[0]) >= 0 and int(ik[-1]) < n
    assert torch.equal(f32_bits(vals[:c]), f32_bits(x[ik]))
    want = x.clone()
    want[ik] = 0.0
    assert torch.equal(f32_bits(e), f32_bits(want))
    del want, e
    say(f"random n=2^31-1 flags={flags}: S and decisions")
    xh = host(x)
    del x
    assert np.float32(oracle.sum_abs_exact(xh)).view(np.uint32) == S.view(np.uint32)
    kept = host(ik)
    pos = np.unique(np.concatenate([positions(31), kept]))
    keep = oracle.random_keep_at(xh[pos], pos, k, S, seed, step)
    member = np.isin(pos, kept, assume_unique=True)
    bad = np.nonzero(keep != member)[0]
    assert bad.size == 0, (bad.size, pos[bad[:5]])
    del xh, vals, idx, ws
    torch.cuda.empty_cache()


def test_sign_max_size():
    dev = device()
    n = NMAX
    need(dev, 15 * n)
    pos = positions(41)
    pd = torch.from_numpy(pos).to(dev)
    g = gen.sign_gradient_device(5, n, dev)
    e = torch.from_numpy(gen.normal_small(1 << 20, 902, scale=1e-3)).to(dev).repeat(2048)[:n].contiguous()
    m = torch.from_numpy(gen.normal_small(1 << 20, 903, scale=1e-2)).to(dev).repeat(2048)[:n].contiguous()
    gs, es, ms = host(g[pd]), host(e[pd]), host(m[pd])
    tail = [host(a[n - 7:]) for a in (g, e, m)]
    say("sign n=2^31-1: compress")
    s, b = efg.ef_sign_compress(g, e, m, gen.SIGN_BETA1, gen.SIGN_CLIP)
    torch.cuda.synchronize()
    oe, om, osg, _, _ = oracle.sign(gs, es, ms, gen.SIGN_BETA1, gen.SIGN_CLIP)
    assert_bits_equal(host(e[pd]), oe, "e")
    assert_bits_equal(host(m[pd]), om, "m")
    assert_bits_equal(host(s[pd]), osg, "sign")
    bh = host(b[pd >> 3])
    assert np.array_equal((bh >> (pos & 7)) & 1, (osg == 1).astype(np.uint8))
    # the last byte holds the final 7 elements (n - 7 is a multiple of 8)
    _, _, _, ob, _ = oracle.sign(*tail, gen.SIGN_BETA1, gen.SIGN_CLIP)
    assert_bits_equal(host(b[-1:]), ob, "last bits byte")
    del g, e, m, s, b
    torch.cuda.empty_cache()


def test_adam_max_size():
    dev = device()
    n = NMAX
    need(dev, 26 * n)
    B1, B2, EPS = gen.ADAM_BETA1, gen.ADAM_BETA2, gen.ADAM_EPS
    pos = positions(51)
    pd = torch.from_numpy(pos).to(dev)
    w = gen.adam_weights_device(n, dev)
    m = torch.zeros(n, device=dev)
    v = torch.zeros(n, device=dev)
    g = gen.sign_gradient_device(1, n, dev)
    gs, ws_ = host(g[pd]), host(w[pd])
    z = np.zeros(pos.size, np.float32)
    say("adam n=2^31-1: warm-up step")
    ss, sb = efg.adam_scalars(gen.ADAM_LR, B1, B2, 1)
    efg.ef_adam_step(g, m, v, w, B1, B2, ss, sb, EPS)
    om, ov, ow, _ = oracle.adam_step(gs, z, z, ws_, B1, B2, ss, sb, EPS)
    assert_bits_equal(host(m[pd]), om, "m warm-up")
    assert_bits_equal(host(v[pd]), ov, "v warm-up")
    assert_bits_equal(host(w[pd]), ow, "w warm-up")
    say("adam n=2^31-1: 1-bit step")
    del g
    g = gen.sign_gradient_device(2, n, dev)
    gs = host(g[pd])
    e = torch.zeros(n, device=dev)
    q, _ = efg.ef_sign_compress(g, e, None, B1, gen.SIGN_CLIP, want_bits=False)
    ss, sb = efg.adam_scalars(gen.ADAM_LR, B1, B2, 2, 1)
    efg.ef_onebit_adam_update(q, 1, m, v, w, B1, ss, sb, EPS)
    oe, _, oq, _, _ = oracle.sign(gs, z, None, B1, gen.SIGN_CLIP)
    om2, ow2, _ = oracle.onebit_adam_update(oq, 1, om, ov, ow, B1, ss, sb, EPS)
    assert_bits_equal(host(q[pd]), oq, "q")
    assert_bits_equal(host(e[pd]), oe, "e")
    assert_bits_equal(host(m[pd]), om2, "m 1-bit")
    assert_bits_equal(host(w[pd]), ow2, "w 1-bit")
    assert_bits_equal(host(v[pd]), ov, "v frozen")
    del g, e, q, m, v, w
    torch.cuda.empty_cache()


def test_decode_and_sgd_max_size():
    """Four packets over n = 2^31 - 1 (entries at 0 and n - 1, a crowd in the
    last, ragged tile), added onto a zero G and, in one pass, applied to w:
    G and w at every packet position and at sampled others against the oracle
    (run on the positions the packets name, which is where G can be nonzero)."""
    dev = device()
    n, P, kp = NMAX, 4, 20_000
    need(dev, 10 * n)
    r = np.random.default_rng(61)
    idx_l = []
    for p in range(P):
        core = r.choice(n - 3000, size=kp - 1002, replace=False)
        tail = np.arange(n - 1000, n) if p % 2 == 0 else r.choice(np.arange(n - 3000, n), size=1000, replace=False)
        idx_l.append(np.unique(np.concatenate([core, tail, [0, n - 1]]))[:kp].astype(np.int64))
    idx = np.concatenate(idx_l)
    off = np.concatenate([[0], np.cumsum([a.size for a in idx_l])]).astype(np.int64)
    vals = gen.normal_small(idx.size, 62)
    # the oracle on the union of the named positions (G is zero everywhere else)
    uni = np.unique(idx)
    G_u = oracle.decode(np.zeros(uni.size, np.float32), vals, np.searchsorted(uni, idx).astype(np.int32), off)
    pos = np.unique(np.concatenate([positions(63, 50_000), uni]))
    G_exp = np.zeros(pos.size, np.float32)
    G_exp[np.searchsorted(pos, uni)] = G_u
    pd = torch.from_numpy(pos).to(dev)
    vd, idd, offd = to_dev(vals, dev), torch.from_numpy(idx.astype(np.int32)).to(dev), torch.from_numpy(off).to(dev)
    say("decode n=2^31-1: accumulate onto zero")
    G = torch.zeros(n, device=dev)
    inv = torch.zeros(1, dtype=torch.int32, device=dev)
    efg.sparse_decode_accumulate(G, vd, idd, offd, invalid=inv)
    torch.cuda.synchronize()
    assert int(host(inv)[0]) == 0
    assert_bits_equal(host(G[pd]), G_exp, "G accumulate")
    say("decode n=2^31-1: one pass with the SGD update")
    w = torch.full((n,), 0.5, dtype=torch.float32, device=dev)
    G.fill_(7.0)
    efg.sparse_decode_sgd(w, vd, idd, offd, 0.1, G=G)
    torch.cuda.synchronize()
    assert_bits_equal(host(G[pd]), G_exp, "G one pass")
    assert_bits_equal(host(w[pd]), oracle.sgd(np.full(pos.size, 0.5, np.float32), G_exp, 0.1), "w one pass")
    del G, w
    torch.cuda.empty_cache()
