"""Property tests of the oracle (Hypothesis): random sizes and k, values drawn
from every float32 (subnormals, ±0, Inf, NaN included) or from a small
tie-heavy pool, each result checked against what the pages fix, computed
here independently of the oracle's code: a brute-force selection in Python,
numpy's float32 arithmetic, np.add.at, np.packbits, np.bincount and the
identities the methods guarantee.  CPU only."""
import numpy as np
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle

SETTINGS = settings(max_examples=250, deadline=None, suppress_health_check=[HealthCheck.too_slow])

ANY32 = st.floats(width=32, allow_nan=True, allow_infinity=True, allow_subnormal=True)
POOL = st.sampled_from([0.0, -0.0, 1.0, -1.0, 1.5, -1.5, 2.0, 1e-40, -1e-40, np.inf, -np.inf, np.nan])


def u32(a):
    return np.asarray(a, np.float32).view(np.uint32)


def same(a, b):
    """Bitwise equal, except that any NaN matches any NaN."""
    a, b = np.asarray(a, np.float32), np.asarray(b, np.float32)
    return a.shape == b.shape and bool(np.all((u32(a) == u32(b)) | (np.isnan(a) & np.isnan(b))))


@st.composite
def vectors(draw, n, count):
    elems = draw(st.sampled_from([ANY32, POOL]))
    return [np.array(draw(st.lists(elems, min_size=n, max_size=n)), np.float32) for _ in range(count)]


@st.composite
def topk_case(draw):
    n = draw(st.integers(0, 300))
    g, e = draw(vectors(n, 2))
    return g, e, draw(st.integers(0, n))


@SETTINGS
@given(topk_case())
def test_topk_is_the_brute_force_selection(case):
    """Kept: the k largest |x| (x = g + e, compared by the bit pattern without
    the sign, so +0 = -0, Inf above every finite value and NaN above Inf),
    equal keys by lower index; sent in index order; residual +0 where kept
    and x elsewhere ('Gradient sparsification' page, top-k and error
    compensation sections)."""
    g, e, k = case
    with np.errstate(all="ignore"):
        x = (g + e).astype(np.float32)
    keys = (u32(x) & 0x7FFFFFFF).astype(np.int64)
    order = sorted(range(x.size), key=lambda i: (-keys[i], i))
    sel = sorted(order[:k])
    vals, idx, e2, nf = oracle.topk(g, e, k)
    assert idx.tolist() == sel
    assert same(vals, x[sel])
    want = x.copy()
    want[sel] = np.float32(0.0)
    assert np.array_equal(u32(e2), u32(want)) or same(e2, want)
    assert np.array_equal(u32(e2)[sel], np.zeros(len(sel), np.uint32))  # +0, never -0
    assert nf == int(np.count_nonzero(~np.isfinite(x)))


@st.composite
def sign_case(draw):
    n = draw(st.integers(0, 200))
    g, e, m = draw(vectors(n, 3))
    beta1 = float(np.float32(draw(st.floats(0.0, 1.0, width=32))))
    clip = draw(st.sampled_from([np.inf, 5.0, float(np.float32(draw(st.floats(0.0009765625, 1024.0, width=32))))]))
    return g, e, m, beta1, clip


@SETTINGS
@given(sign_case())
def test_sign_step_is_its_formulas(case):
    """The 1-bit step ('1bit Adam' page, sections 2.1, 2.2 and 3.2) in numpy
    float32, one rounding per operation: clip g, x = g + e, s = sign(x) with
    sign(±0) = sign(NaN) = 0, e' = b1 e + (1 - b1)(x - s), m' = b1 m + (1 - b1) s,
    bits LSB-first with bit = (s == +1)."""
    g, e, m, b1, clip = case
    f = np.float32
    with np.errstate(all="ignore"):
        gc = np.where(g > f(clip), f(clip), np.where(g < f(-clip), f(-clip), g)).astype(np.float32)
        x = (gc + e).astype(np.float32)
        s = ((x > 0).astype(np.int8) - (x < 0).astype(np.int8)).astype(np.int8)
        sf = s.astype(np.float32)
        c = f(f(1.0) - f(b1))
        d = (x - sf).astype(np.float32)
        e_w = ((f(b1) * e).astype(np.float32) + (c * d).astype(np.float32)).astype(np.float32)
        m_w = ((f(b1) * m).astype(np.float32) + (c * sf).astype(np.float32)).astype(np.float32)
    e2, m2, q, bits, nf = oracle.sign(g, e, m, b1, clip)
    assert np.array_equal(q, s)
    assert np.array_equal(bits, np.packbits(s == 1, bitorder="little"))
    assert same(e2, e_w) and same(m2, m_w)
    assert nf == int(np.count_nonzero(~np.isfinite(e_w)) + np.count_nonzero(~np.isfinite(m_w)))


@st.composite
def packets(draw):
    n = draw(st.integers(1, 2000))
    npk = draw(st.integers(0, 6))
    idx, vals = [], []
    for _ in range(npk):
        k = draw(st.integers(0, min(n, 60)))
        ix = np.array(sorted(draw(st.sets(st.integers(0, n - 1), min_size=k, max_size=k))), np.int32)
        idx.append(ix)
        vals.append(np.array(draw(st.lists(st.floats(-65536.0, 65536.0, width=32), min_size=k, max_size=k)),
                             np.float32))
    G = np.array(draw(st.lists(st.floats(-1024.0, 1024.0, width=32), min_size=n, max_size=n)), np.float32)
    return n, G, idx, vals


@SETTINGS
@given(packets())
def test_decode_is_the_packet_ordered_sum(case):
    """The receiver adds every packet into G in packet order, one rounding per
    addition ('Gradient sparsification' page, basic principle): np.add.at
    over the packets one after another."""
    n, G, idx, vals = case
    off = np.concatenate([[0], np.cumsum([len(i) for i in idx])]).astype(np.int64)
    cat_i = np.concatenate(idx) if idx else np.zeros(0, np.int32)
    cat_v = np.concatenate(vals) if vals else np.zeros(0, np.float32)
    want = G.copy()
    for ix, v in zip(idx, vals):
        np.add.at(want, ix, v)
    assert np.array_equal(u32(oracle.decode(G, cat_v, cat_i, off)), u32(want))


@st.composite
def index_sets(draw):
    n = draw(st.integers(1, 5000))
    k = draw(st.integers(0, min(n, 400)))
    return n, np.array(sorted(draw(st.sets(st.integers(0, n - 1), min_size=k, max_size=k))), np.int32)


@SETTINGS
@given(index_sets())
def test_index_encodings_round_trip(case):
    """Bitmap (LSB-first), delta LEB128 and 256-element block encodings of an
    ascending index list decode back to it; the bitmap is np.packbits of the
    membership mask, and the block form holds one count - 1 per non-empty
    block (np.bincount) and each index's offset in its block ('Gradient
    sparsification' page, index encoding section)."""
    n, idx = case
    bits = oracle.bitmap_encode(idx, n)
    member = np.zeros(n, bool)
    member[idx] = True
    assert np.array_equal(bits, np.packbits(member, bitorder="little"))
    back, k = oracle.bitmap_decode(bits, n)
    assert k == idx.size and np.array_equal(back, idx)
    assert np.array_equal(oracle.delta_decode(oracle.delta_encode(idx), idx.size), idx)
    mask, counts, offs = oracle.blocks_encode(idx, n)
    per_block = np.bincount(idx >> 8, minlength=(n + 255) // 256)
    assert np.array_equal(mask, np.packbits(per_block > 0, bitorder="little"))
    assert np.array_equal(counts.astype(np.int64), per_block[per_block > 0] - 1)
    assert np.array_equal(offs, (idx & 255).astype(np.uint8))
    back, k = oracle.blocks_decode(mask, counts, offs, n)
    assert k == idx.size and np.array_equal(back, idx)


@st.composite
def quant_case(draw):
    n = draw(st.integers(1, 300))
    k = draw(st.integers(0, n))
    idx = np.array(sorted(draw(st.sets(st.integers(0, n - 1), min_size=k, max_size=k))), np.int32)
    vals = draw(vectors(k, 1))[0]
    e = np.zeros(n, np.float32)
    return vals, idx, e


@SETTINGS
@given(quant_case())
def test_quantisation_keeps_the_error_in_the_residual(case):
    """8-bit values with one scale ('Gradient sparsification' page,
    comparison with other compression techniques): codes within ±127, the
    scale from the largest finite magnitude, and for every finite value the
    dequantised code plus the new residual gives the value back exactly,
    as long as the dequantised code is finite: 127 * fl(amax / 127) can round
    up past FLT_MAX only when amax lies within 2^-24 of it (relative)."""
    vals, idx, e = case
    q, scale, e2 = oracle.quantize_int8(vals, idx, e)
    assert np.all(np.abs(q.astype(np.int32)) <= 127)
    fin = np.isfinite(vals)
    amax = float(np.max(np.abs(vals[fin]))) if fin.any() else 0.0
    assert scale == (float(np.float32(np.float32(amax) / np.float32(127.0))) if amax > 0 else 0.0)
    assert np.all(q[~fin] == 0)
    with np.errstate(all="ignore"):
        deq = (q.astype(np.float32) * np.float32(scale)).astype(np.float32)
        back = (e2[idx] + deq).astype(np.float32)
    ok = fin & np.isfinite(deq)
    assert np.all(back[ok] == vals[ok])
    if not np.all(np.isfinite(deq[fin])):
        assert amax >= float(np.finfo(np.float32).max) * (1.0 - 2.0 ** -24)
