"""Pins of the oracle's top-k error-feedback step (CPU only).

The oracle is checked against things other than itself: hand-worked cases,
pure-Python full-sort brute force, numpy/torch selection on tie-free inputs,
the invariants that make the kept set unique, and the residual identities of
error feedback (page "Gradient sparsification", sections on error
compensation and the step-by-step algorithm).
"""
import json
import os
import pathlib
import struct

import numpy as np
import pytest

import gen
import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def f32bits(v):
    return struct.unpack("<I", struct.pack("<f", float(v)))[0]


def brute_topk(g, e, k):
    """Pure-Python full sort of every position by (larger |x| first, lower index first)."""
    n = len(g)
    x = [np.float32(g[i]) + np.float32(e[i]) for i in range(n)]
    key = [f32bits(v) & 0x7FFFFFFF for v in x]
    order = sorted(range(n), key=lambda i: (-key[i], i))
    kept = sorted(order[:k])
    e_new = [np.float32(0.0) if i in set(kept) else x[i] for i in range(n)]
    return (np.array([x[i] for i in kept], np.float32), np.array(kept, np.int32),
            np.array(e_new, np.float32))


def same_bits(a, b):
    a = np.asarray(a, np.float32)
    b = np.asarray(b, np.float32)
    return a.shape == b.shape and np.array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.parametrize("name", ["topk_worked.json", "topk_ties_worked.json"])
def test_hand_worked(name):
    d = json.loads(pathlib.Path(os.path.join(GOLD, name)).read_text())
    vals, idx, e_new, bad = oracle.topk(d["g"], d["e"], d["k"])
    assert same_bits(vals, d["vals"])
    assert idx.tolist() == d["idx"]
    assert same_bits(e_new, d["e_new"])
    assert bad == 0


def _cases():
    out = []
    for n in (1, 2, 3, 7, 64, 257, 1000):
        for kind in ("normal", "ties", "specials", "allsame"):
            out.append((n, kind))
    return out


@pytest.mark.parametrize("n,kind", _cases())
def test_brute_force(n, kind):
    if kind == "normal":
        g = gen.normal_small(n, 1, n)
        e = gen.normal_small(n, 2, n, scale=0.5)
    elif kind == "ties":
        g = gen.uniform_ties(n, 4, 3, n)
        e = gen.uniform_ties(n, 2, 4, n)
    elif kind == "specials":
        g = gen.specials(n, 5, n)
        e = gen.normal_small(n, 6, n)
    else:
        g = np.full(n, -0.75, np.float32)
        e = np.zeros(n, np.float32)
    ks = sorted({0, 1, max(0, n - 1), n, n // 3, n // 2})
    for k in ks:
        vals, idx, e_new, bad = oracle.topk(g, e, k)
        bv, bi, be = brute_topk(g, e, k)
        assert idx.tolist() == bi.tolist(), (n, kind, k)
        assert same_bits(vals, bv), (n, kind, k)
        assert same_bits(e_new, be), (n, kind, k)
        x = (g + e).astype(np.float32)
        assert bad == int((~np.isfinite(x)).sum())


def test_signed_zero_and_negative_ties():
    # -0 and +0 are the same magnitude; +-v are ties; lower index wins.
    g = np.array([-0.0, 0.0, -3.0, 3.0, -0.0, 3.0], np.float32)
    e = np.full(6, -0.0, np.float32)  # -0 + -0 = -0, +0 + -0 = +0
    vals, idx, e_new, _ = oracle.topk(g, e, 2)
    assert idx.tolist() == [2, 3]
    vals, idx, e_new, _ = oracle.topk(g, e, 4)
    assert idx.tolist() == [0, 2, 3, 5]
    assert f32bits(vals[0]) == 0x80000000  # the sent value is x itself, -0.0


def test_tie_free_matches_library_selection():
    n, k = 200_000, 1234
    r = gen.rng(10, 1)
    # distinct magnitudes by construction (integers), random signs, plus a residual
    # of multiples of 1/4 that cannot create ties between distinct integers
    g = ((r.permutation(n) + 1) * np.where(r.random(n) < 0.5, -1, 1)).astype(np.float32)
    e = np.full(n, 0.25, np.float32)
    x = (g + e).astype(np.float32)
    assert np.unique(np.abs(x)).size == n  # no ties: the library answer is unique
    vals, idx, e_new, _ = oracle.topk(g, e, k)
    want = np.sort(np.argpartition(-np.abs(x), k - 1)[:k])
    assert idx.tolist() == want.tolist()
    torch = pytest.importorskip("torch")
    t = torch.topk(torch.from_numpy(np.abs(x)), k).indices.sort().values.numpy()
    assert idx.tolist() == t.tolist()


@pytest.mark.parametrize("kind", ["normal", "ties", "lognormal"])
def test_invariants(kind):
    n, k = 100_003, 997
    if kind == "normal":
        g = gen.normal_small(n, 20)
    elif kind == "ties":
        g = gen.uniform_ties(n, 6, 21)
    else:
        g = gen.large_gradient(0, n=n)
    e = gen.normal_small(n, 22, scale=0.01) if kind != "ties" else gen.uniform_ties(n, 3, 23)
    vals, idx, e_new, _ = oracle.topk(g, e, k)
    x = (g + e).astype(np.float32)
    key = x.view(np.uint32) & 0x7FFFFFFF
    assert idx.size == k and np.all(np.diff(idx) > 0)
    kept = np.zeros(n, bool)
    kept[idx] = True
    assert key[kept].min() >= key[~kept].max()
    T = key[kept].min()
    tie_kept = np.nonzero(kept & (key == T))[0]
    tie_drop = np.nonzero(~kept & (key == T))[0]
    if tie_drop.size:
        assert tie_kept.max() < tie_drop.min()
    assert same_bits(vals, x[idx])
    # the residual identity x~ + e' == g + e: exact as numbers (bitwise up to the
    # sign of a zero sum), and e' is x bit for bit wherever x was not sent
    dense = np.zeros(n, np.float32)
    dense[idx] = vals
    assert np.array_equal(dense + e_new, x)
    assert same_bits(e_new[~kept], x[~kept])
    assert np.all(e_new[idx].view(np.uint32) == 0)  # exactly +0.0 where kept


def test_special_k():
    n = 5000
    g = gen.normal_small(n, 30)
    e = gen.normal_small(n, 31)
    x = (g + e).astype(np.float32)
    vals, idx, e_new, _ = oracle.topk(g, e, 0)
    assert vals.size == 0 and same_bits(e_new, x)
    vals, idx, e_new, _ = oracle.topk(g, e, n)
    assert idx.tolist() == list(range(n)) and same_bits(vals, x)
    assert np.all(e_new.view(np.uint32) == 0)


def test_chain_conserves_gradient():
    """Summed over steps, what is sent plus what is still held equals everything
    that came in: sum_t x~_t + e_T = sum_t g_t + e_0 (exact arithmetic; fp64 check
    with a bound of one rounding of |x| per step)."""
    n, k, T = 50_000, 500, 10
    e = np.zeros(n, np.float32)
    sent = np.zeros(n, np.float64)
    total = np.zeros(n, np.float64)
    bound = np.zeros(n, np.float64)
    for t in range(T):
        g = gen.flat_gradient(t, n=n)
        x = (g + e).astype(np.float32)
        bound += np.abs(x.astype(np.float64)) * 2.0 ** -24
        vals, idx, e, _ = oracle.topk(g, e, k)
        np.add.at(sent, idx, vals.astype(np.float64))
        total += g
    err = np.abs(sent + e - total)
    assert np.all(err <= bound + 1e-30)


def test_nonfinite_count():
    n = 4096
    g = gen.specials(n, 40)
    e = gen.specials(n, 41)
    with np.errstate(invalid="ignore"):  # inf + -inf is meant to give NaN here
        x = (g + e).astype(np.float32)
    _, _, _, bad = oracle.topk(g, e, 100)
    assert bad == int((~np.isfinite(x)).sum()) and bad > 0


def test_segmented_is_per_tensor():
    sizes = [7, 1, 300, 64, 1000, 5]
    ks = [3, 1, 0, 64, 17, 2]
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    n = int(off[-1])
    g = gen.uniform_ties(n, 5, 50)
    e = gen.normal_small(n, 51, scale=0.2)
    vals, idx, e_new, _ = oracle.topk_segmented(g, e, off, ks)
    o = 0
    for s in range(len(sizes)):
        a, b = off[s], off[s + 1]
        v, i, en, _ = oracle.topk(g[a:b], e[a:b], ks[s])
        assert same_bits(vals[o:o + ks[s]], v)
        assert idx[o:o + ks[s]].tolist() == (i + a).tolist()
        assert same_bits(e_new[a:b], en)
        o += ks[s]
    assert np.all(np.diff(idx) > 0)


def test_bert_layerwise_k_total():
    off, ks = gen.bert_segments()
    assert len(ks) == 194
    assert int(off[-1]) == 108_888_576
    assert int(ks.sum()) == 368_208
    ratios = json.loads(pathlib.Path(os.path.join(GOLD, "ratios.json")).read_text())["layerwise_ratios"]
    sizes = np.diff(off)
    assert np.all(ks[sizes > 1_000_000] == sizes[sizes > 1_000_000] * ratios["large_layer"] // 1)


def test_oracle_chain_split_and_resumed(tmp_path):
    """The residual is the whole state of the top-k chain: the oracle's chain
    split at step 5, e written with np.save and read back, gives the same
    packets and final e as the unsplit chain."""
    n, k, T, split = 20_000, 200, 10, 5
    grads = [gen.normal_small(n, 160, t) for t in range(T)]
    e_full = np.zeros(n, np.float32)
    full = []
    for g in grads:
        v, i, e_full, _ = oracle.topk(g, e_full, k)
        full.append((v, i))
    e = np.zeros(n, np.float32)
    for g in grads[:split]:
        _, _, e, _ = oracle.topk(g, e, k)
    np.save(tmp_path / "e.npy", e)
    e = np.load(tmp_path / "e.npy")
    for t in range(split, T):
        v, i, e, _ = oracle.topk(grads[t], e, k)
        assert np.array_equal(i, full[t][1]) and np.array_equal(v.view(np.uint32), full[t][0].view(np.uint32))
    assert np.array_equal(e.view(np.uint32), e_full.view(np.uint32))
