"""Pins of the oracle's decode (scatter-add), SGD and index encodings (CPU only)."""
import json
import os
import pathlib

import numpy as np
import pytest

import gen
import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_decode_hand_worked():
    d = json.loads(pathlib.Path(os.path.join(GOLD, "decode_worked.json")).read_text())
    G = oracle.decode(np.zeros(d["n"], np.float32), d["vals"], d["idx"], d["pk_off"])
    assert G.tolist() == d["G"]
    w = oracle.sgd(d["w"], G, d["lr"])
    assert w.tolist() == d["w_new"]


def _packets(n, P, k, seed):
    idx = [gen.sorted_unique_indices(n, k, seed, p) for p in range(P)]
    vals = [gen.normal_small(k, seed + 1, p) for p in range(P)]
    off = np.concatenate([[0], np.cumsum([k] * P)]).astype(np.int64)
    return np.concatenate(vals), np.concatenate(idx), off


@pytest.mark.parametrize("n,P,k", [(1000, 16, 100), (100_000, 16, 5000), (37, 3, 37)])
def test_decode_matches_add_at(n, P, k):
    vals, idx, off = _packets(n, P, k, 7)
    G0 = gen.normal_small(n, 99)
    G = oracle.decode(G0, vals, idx, off)
    ref = G0.copy()
    np.add.at(ref, idx, vals)  # unbuffered, applied in array order (= packet order)
    assert np.array_equal(G.view(np.uint32), ref.view(np.uint32))


def test_decode_integer_values_exact():
    n, P, k = 5000, 16, 700
    _, idx, off = _packets(n, P, k, 8)
    vals = gen.rng(9, 1).integers(-1000, 1000, size=idx.size).astype(np.float32)
    G = oracle.decode(np.zeros(n, np.float32), vals, idx, off)
    ref = np.zeros(n, np.int64)
    np.add.at(ref, idx, vals.astype(np.int64))
    assert np.array_equal(G.astype(np.int64), ref)


def test_decode_rejects_out_of_range():
    with pytest.raises(ValueError):
        oracle.decode(np.zeros(4, np.float32), [1.0], [4], [0, 1])


@pytest.mark.parametrize("lr", [0.1, 1.0, 0.0, 3.5])
def test_sgd_matches_numpy(lr):
    n = 70_001
    w = gen.normal_small(n, 1)
    G = gen.normal_small(n, 2)
    G[::7] = 0.0
    w[::11] = -0.0
    got = oracle.sgd(w, G, lr)
    want = (w - (np.float32(lr) * G).astype(np.float32)).astype(np.float32)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_sgd_zero_gradient_is_identity():
    w = np.array([-0.0, 0.0, 1.0, -2.5], np.float32)
    got = oracle.sgd(w, np.zeros(4, np.float32), 0.1)
    assert np.array_equal(got.view(np.uint32), w.view(np.uint32))


# ------------------------------------------------------------- encodings
IDX_CASES = [(1, 0), (1, 1), (8, 8), (9, 3), (1000, 1), (100_000, 100), (25_600, 25_600),
             (1_000_003, 4000), (513, 300)]


@pytest.mark.parametrize("n,k", IDX_CASES)
def test_bitmap(n, k):
    idx = gen.sorted_unique_indices(n, k, 3, n)
    bits = oracle.bitmap_encode(idx, n)
    mask = np.zeros(n, bool)
    mask[idx] = True
    assert np.array_equal(bits, np.packbits(mask, bitorder="little"))
    assert bits.size == (n + 7) // 8
    back, kk = oracle.bitmap_decode(bits, n)
    assert kk == k and back.tolist() == idx.tolist()


def leb128_len(d):
    return max(1, (int(d).bit_length() + 6) // 7)


def test_delta_textbook_values():
    # unsigned LEB128 of 300 is AC 02; of 624485 is E5 8E 26; 0 and 127 take one byte
    s = oracle.delta_encode(np.array([0, 127, 427, 427 + 624485], np.int32))
    assert s.tolist() == [0x00, 0x7F, 0xAC, 0x02, 0xE5, 0x8E, 0x26]


@pytest.mark.parametrize("n,k", IDX_CASES)
def test_delta(n, k):
    idx = gen.sorted_unique_indices(n, k, 4, n)
    s = oracle.delta_encode(idx)
    d = np.diff(np.concatenate([[0], idx.astype(np.int64)]))
    assert s.size == sum(leb128_len(v) for v in d)
    assert int((s & 0x80 == 0).sum()) == k  # one terminating byte per index
    assert oracle.delta_decode(s, k).tolist() == idx.tolist()


def test_delta_max_index():
    idx = np.array([0, 2**31 - 2, 2**31 - 1], np.int32)
    s = oracle.delta_encode(idx)
    assert s.size == 1 + 5 + 1
    assert oracle.delta_decode(s, 3).tolist() == idx.tolist()


@pytest.mark.parametrize("n,k", IDX_CASES + [(256, 256), (257, 2), (300_000, 300_000 // 10)])
def test_blocks(n, k):
    idx = gen.sorted_unique_indices(n, k, 5, n)
    mask, counts, offs = oracle.blocks_encode(idx, n)
    nb = (n + 255) // 256
    assert mask.size == (nb + 7) // 8
    nonempty = np.unique(idx // 256)
    flags = np.zeros(nb, bool)
    flags[nonempty] = True
    assert np.array_equal(mask, np.packbits(flags, bitorder="little"))
    assert counts.size == nonempty.size
    assert int((counts.astype(np.int64) + 1).sum()) == k
    assert np.array_equal(counts.astype(np.int64) + 1, np.bincount(idx // 256)[nonempty])
    assert np.array_equal(offs, (idx % 256).astype(np.uint8))
    back, kk = oracle.blocks_decode(mask, counts, offs, n)
    assert kk == k and back.tolist() == idx.tolist()


def test_blocks_full_block_count():
    idx = np.arange(512, dtype=np.int32)  # two full blocks: count-1 = 255 each
    mask, counts, offs = oracle.blocks_encode(idx, 512)
    assert counts.tolist() == [255, 255] and mask.tolist() == [3]
