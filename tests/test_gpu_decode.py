"""GPU parity of decode (packet-ordered scatter-add), SGD and the index
encodings against the CPU oracle; everything bit for bit."""
import numpy as np
import pytest
import torch

import error_feedback_gradient_amd as efg
import gen
import oracle
from gpu_util import assert_bits_equal, device, host, say, to_dev

pytestmark = pytest.mark.gpu


def packets_from(n, P, k, seed, sizes=None):
    """P packets of sorted unique indices (seeded) with N(0,1) values."""
    idx, vals = [], []
    for p in range(P):
        kp = k if sizes is None else sizes[p]
        idx.append(gen.sorted_unique_indices(n, kp, seed, p))
        vals.append(gen.normal_small(kp, seed + 1, p))
    off = np.concatenate([[0], np.cumsum([a.size for a in idx])]).astype(np.int64)
    return np.concatenate(vals).astype(np.float32), np.concatenate(idx).astype(np.int32), off


def gpu_decode(G0, vals, idx, off):
    dev = device()
    Gd = to_dev(G0, dev)
    inv = torch.zeros(1, dtype=torch.int32, device=dev)
    efg.sparse_decode_accumulate(Gd, to_dev(vals, dev), to_dev(idx, dev), to_dev(off, dev), invalid=inv)
    return host(Gd), int(host(inv)[0])


@pytest.mark.parametrize("n,P,k", [(1, 1, 1), (5000, 16, 100), (100_003, 16, 5000), (4096, 3, 4096),
                                   (4097, 2, 4097), (1_000_000, 1, 3), (777, 40, 700), (300_000, 300, 2000)])
def test_decode_small(n, P, k):
    vals, idx, off = packets_from(n, P, min(k, n), 300)
    G0 = gen.normal_small(n, 301)
    got, inv = gpu_decode(G0, vals, idx, off)
    assert_bits_equal(got, oracle.decode(G0, vals, idx, off), f"decode n={n} P={P} k={k}")
    assert inv == 0


def test_decode_dense_tile_overflow_path():
    # many packets all dense in the same tiles: more staged entries than fit in LDS
    n, P = 20_000, 8
    vals, idx, off = packets_from(n, P, n, 302)
    G0 = np.zeros(n, np.float32)
    got, _ = gpu_decode(G0, vals, idx, off)
    assert_bits_equal(got, oracle.decode(G0, vals, idx, off), "dense decode")


def test_decode_empty_packets_and_invalid_entries():
    n = 10_000
    sizes = [0, 50, 0, 0, 70, 0]
    vals, idx, off = packets_from(n, len(sizes), 0, 303, sizes=sizes)
    G0 = gen.normal_small(n, 304)
    got, inv = gpu_decode(G0, vals, idx, off)
    assert_bits_equal(got, oracle.decode(G0, vals, idx, off), "empty packets")
    assert inv == 0
    # an out-of-range index and an order violation are skipped and counted
    bad_idx = idx.copy()
    bad_idx[off[1]] = n + 5  # first entry of packet 1 (its range is [off[1], off[2]))
    bad_idx[off[4] + 3] = bad_idx[off[4] + 2]  # duplicate inside packet 4
    got, inv = gpu_decode(G0, vals, bad_idx, off)
    assert inv >= 2
    assert np.all(np.isfinite(got))


def test_decode_full_size_sixteen_packets_then_sgd():
    """N = 25.6M, 16 packets of the top 0.1 % (25,600 entries) of independent
    N(0,1) gradients, G = 0, then w -= 0.1 G from N(0,1) weights."""
    dev = device()
    n, P, k = gen.DECODE_N, gen.DECODE_PACKETS, gen.DECODE_K
    vals, idx = [], []
    for p in range(P):
        g = gen.decode_packet_gradient(p)
        # the packet is an input here: a top-0.1 % selection made by numpy
        sel = np.sort(np.argpartition(-np.abs(g), k - 1)[:k]).astype(np.int32)
        idx.append(sel)
        vals.append(g[sel])
    off = np.concatenate([[0], np.cumsum([k] * P)]).astype(np.int64)
    vals = np.concatenate(vals)
    idx = np.concatenate(idx)
    Gd = torch.zeros(n, dtype=torch.float32, device=dev)
    efg.sparse_decode_accumulate(Gd, to_dev(vals, dev), to_dev(idx, dev), to_dev(off, dev))
    G_ref = oracle.decode(np.zeros(n, np.float32), vals, idx, off)
    assert_bits_equal(host(Gd), G_ref, "decode full size")
    w0 = gen.decode_weights()
    wd = to_dev(w0, dev)
    efg.sgd_apply(wd, Gd, gen.DECODE_LR)
    assert_bits_equal(host(wd), oracle.sgd(w0, G_ref, gen.DECODE_LR), "sgd full size")
    # per-packet encodings round trip on the GPU and equal the oracle's bytes
    for p in (0, P - 1):
        ip = idx[off[p]:off[p + 1]]
        ipd = to_dev(ip, dev)
        bits = efg.encode_bitmap(ipd, n)
        assert_bits_equal(host(bits), oracle.bitmap_encode(ip, n), f"bitmap packet {p}")
        back, kk = efg.decode_bitmap(bits, n, k)
        assert int(host(kk)[0]) == k
        assert_bits_equal(host(back)[:k], ip, f"bitmap round trip packet {p}")
        st, nb = efg.encode_delta(ipd)
        want = oracle.delta_encode(ip)
        nbytes = int(host(nb)[0])
        assert nbytes == want.size
        assert_bits_equal(host(st)[:nbytes], want, f"delta packet {p}")
        back, status = efg.decode_delta(st, nbytes, k)
        assert int(host(status)[0]) == 0
        assert_bits_equal(host(back), ip, f"delta round trip packet {p}")


def fused(w0, vals, idx, off, lr, with_G=True):
    """sparse_decode_sgd on the GPU: (w, G or None, invalid count)."""
    dev = device()
    wd = to_dev(w0, dev)
    Gd = torch.full((w0.size,), 7.0, dtype=torch.float32, device=dev) if with_G else None
    inv = torch.zeros(1, dtype=torch.int32, device=dev)
    efg.sparse_decode_sgd(wd, to_dev(vals, dev), to_dev(idx, dev), to_dev(off, dev), lr, G=Gd, invalid=inv)
    return host(wd), (host(Gd) if with_G else None), int(host(inv)[0])


def fused_ref(w0, vals, idx, off, lr):
    """The oracle's two steps: decode onto a zero G, then the SGD update."""
    G = oracle.decode(np.zeros(w0.size, np.float32), vals, idx, off)
    return oracle.sgd(w0, G, lr), G


@pytest.mark.parametrize("n,P,k", [(1, 1, 1), (5, 2, 3), (5000, 16, 100), (100_003, 16, 5000), (4096, 3, 4096),
                                   (4097, 2, 4097), (1_000_000, 1, 3), (777, 40, 700), (300_000, 300, 2000)])
@pytest.mark.parametrize("lr", [0.1, 1.0])
def test_decode_sgd_fused(n, P, k, lr):
    """The one-pass receiver step equals zeroing G, the decode and the SGD
    update, bit for bit, for w and G (ragged last tiles, empty tiles, tiles
    fuller than the staging area)."""
    vals, idx, off = packets_from(n, P, min(k, n), 310)
    w0 = gen.normal_small(n, 311)
    w, G, inv = fused(w0, vals, idx, off, lr)
    w_ref, G_ref = fused_ref(w0, vals, idx, off, lr)
    assert_bits_equal(G, G_ref, f"fused G n={n} P={P} k={k}")
    assert_bits_equal(w, w_ref, f"fused w n={n} P={P} k={k}")
    assert inv == 0


def test_decode_sgd_fused_edges():
    dev = device()
    n = 10_001
    w0 = gen.normal_small(n, 312)
    w0[:6] = np.array([0.0, -0.0, np.inf, -np.inf, 1e-45, -3.4e38], np.float32)
    # no packets: G = +0 everywhere and w unchanged (w - 0.1 * +0 keeps -0)
    empty = np.zeros(1, np.int64)
    w, G, _ = fused(w0, np.zeros(0, np.float32), np.zeros(0, np.int32), empty, 0.1)
    assert_bits_equal(w, w0, "no packets: w")
    assert_bits_equal(G, np.zeros(n, np.float32), "no packets: G")
    # without G, and with out-of-range / out-of-order entries (skipped and counted)
    vals, idx, off = packets_from(n, 6, 0, 313, sizes=[0, 50, 0, 3000, 70, 1])
    w, _, inv = fused(w0, vals, idx, off, 0.5, with_G=False)
    assert_bits_equal(w, fused_ref(w0, vals, idx, off, 0.5)[0], "no G output")
    assert inv == 0
    bad = idx.copy()
    bad[off[1]] = n + 5
    bad[off[3] + 3] = bad[off[3] + 2]
    w, G, inv = fused(w0, vals, bad, off, 0.5)
    assert inv >= 2
    assert np.all(np.isfinite(G))


def test_decode_sgd_fused_full_size():
    """The decode workload's 16 packets at N = 25.6M in one pass: w and G equal
    the oracle's decode onto zero followed by its SGD update."""
    n, P, k = gen.DECODE_N, gen.DECODE_PACKETS, gen.DECODE_K
    vals, idx = [], []
    for p in range(P):
        g = gen.decode_packet_gradient(p)
        sel = np.sort(np.argpartition(-np.abs(g), k - 1)[:k]).astype(np.int32)
        idx.append(sel)
        vals.append(g[sel])
    off = np.concatenate([[0], np.cumsum([k] * P)]).astype(np.int64)
    vals, idx = np.concatenate(vals), np.concatenate(idx)
    w0 = gen.decode_weights()
    w, G, _ = fused(w0, vals, idx, off, gen.DECODE_LR)
    w_ref, G_ref = fused_ref(w0, vals, idx, off, gen.DECODE_LR)
    assert_bits_equal(G, G_ref, "fused G full size")
    assert_bits_equal(w, w_ref, "fused w full size")


@pytest.mark.parametrize("n", [1, 3, 4, 5, 1000, 4099, 1_000_003])
@pytest.mark.parametrize("lr", [0.1, 1.0, 0.0])
def test_sgd_small(n, lr):
    dev = device()
    w = gen.normal_small(n, 310, n)
    G = gen.normal_small(n, 311, n)
    G[::5] = 0.0
    wd = to_dev(w, dev)
    efg.sgd_apply(wd, to_dev(G, dev), lr)
    assert_bits_equal(host(wd), oracle.sgd(w, G, lr), f"sgd n={n} lr={lr}")


# ------------------------------------------------------------- encodings
IDX_CASES = [(1, 0), (1, 1), (8, 8), (9, 3), (1000, 1), (100_000, 100), (25_600, 25_600), (1_000_003, 4000),
             (513, 300), (70_000, 70_000), (5_000_000, 200_000), (3_000_000, 2_999_000)]


@pytest.mark.parametrize("n,k", IDX_CASES)
def test_bitmap(n, k):
    dev = device()
    idx = gen.sorted_unique_indices(n, k, 320, n)
    bits = efg.encode_bitmap(to_dev(idx, dev), n)
    assert_bits_equal(host(bits), oracle.bitmap_encode(idx, n), "bitmap")
    back, kk = efg.decode_bitmap(bits, n, k)
    assert int(host(kk)[0]) == k
    assert_bits_equal(host(back)[:k], idx, "bitmap decode")
    # a capacity below the count keeps the first entries and still reports the count
    if k > 2:
        back, kk = efg.decode_bitmap(bits, n, k // 2)
        assert int(host(kk)[0]) == k
        assert_bits_equal(host(back)[:k // 2], idx[:k // 2], "bitmap decode capped")


@pytest.mark.parametrize("n,k", IDX_CASES)
def test_delta(n, k):
    dev = device()
    idx = gen.sorted_unique_indices(n, k, 321, n)
    st, nb = efg.encode_delta(to_dev(idx, dev))
    want = oracle.delta_encode(idx)
    nbytes = int(host(nb)[0])
    assert nbytes == want.size
    assert_bits_equal(host(st)[:nbytes], want, "delta bytes")
    back, status = efg.decode_delta(to_dev(want, dev) if want.size else st, nbytes, k)
    assert int(host(status)[0]) == 0
    assert_bits_equal(host(back), idx, "delta decode")


def test_delta_extreme_gaps_and_malformed():
    dev = device()
    idx = np.array([0, 1, 127, 128, 16_511, 2**31 - 2, 2**31 - 1], np.int32)
    st, nb = efg.encode_delta(to_dev(idx, dev))
    want = oracle.delta_encode(idx)
    assert_bits_equal(host(st)[:int(host(nb)[0])], want, "delta extreme")
    back, status = efg.decode_delta(to_dev(want, dev), want.size, idx.size)
    assert int(host(status)[0]) == 0
    assert_bits_equal(host(back), idx, "delta extreme decode")
    # truncated stream: fewer varints than k -> status 1
    _, status = efg.decode_delta(to_dev(want[:-1], dev), want.size - 1, idx.size)
    assert int(host(status)[0]) == 1
    # six-byte varint -> status 1
    bad = np.array([0x80, 0x80, 0x80, 0x80, 0x80, 0x01], np.uint8)
    _, status = efg.decode_delta(to_dev(bad, dev), bad.size, 1)
    assert int(host(status)[0]) == 1


@pytest.mark.parametrize("n,k", IDX_CASES + [(256, 256), (257, 2), (300_000, 30_000)])
def test_blocks(n, k):
    dev = device()
    idx = gen.sorted_unique_indices(n, k, 322, n)
    mask, counts, offs, nblk = efg.encode_blocks(to_dev(idx, dev), n)
    wm, wc, wo = oracle.blocks_encode(idx, n)
    nb = int(host(nblk)[0])
    assert nb == wc.size
    assert_bits_equal(host(mask)[:wm.size], wm, "blocks mask")
    assert_bits_equal(host(counts)[:nb], wc, "blocks counts")
    assert_bits_equal(host(offs)[:k], wo, "blocks offs")
    back = efg.decode_blocks(to_dev(wm, dev), to_dev(wc if wc.size else np.zeros(1, np.uint8), dev),
                             to_dev(wo if wo.size else np.zeros(1, np.uint8), dev), n, k)
    assert_bits_equal(host(back), idx, "blocks decode")


def test_blocks_large_workload():
    """The 1.3e9-element index space with 1.3e6 kept positions (block-sparse output)."""
    dev = device()
    n, k = gen.LARGE_N, gen.LARGE_K
    idx = gen.sorted_unique_indices(n, k, 323)
    mask, counts, offs, nblk = efg.encode_blocks(to_dev(idx, dev), n)
    wm, wc, wo = oracle.blocks_encode(idx, n)
    nb = int(host(nblk)[0])
    assert nb == wc.size
    assert_bits_equal(host(mask), wm, "large mask")
    assert_bits_equal(host(counts)[:nb], wc, "large counts")
    assert_bits_equal(host(offs)[:k], wo, "large offs")
    back = efg.decode_blocks(mask, counts, offs, n, k)
    assert_bits_equal(host(back), idx, "large blocks decode")
    say(f"blocks: {nb} non-empty of {(n + 255) // 256}")
