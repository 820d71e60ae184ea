"""Pins of the oracle's random magnitude-proportional sparsification (CPU only).

What fixes each piece, other than the oracle itself:
  * Philox4x32-10: the known-answer vectors published with the generator
    (Salmon et al., SC 2011, and the Random123 distribution's kat_vectors);
  * the exact sum: Python's math.fsum (correctly rounded float64 sum) and
    fractions.Fraction (exact rational arithmetic);
  * the sampling law: keep frequencies over many independent steps against
    p_i = min(1, k|x_i| / S), the expected count against k, neighbouring
    elements uncorrelated, and the special cases p = 0, p = 1, u = 0;
  * the error-feedback bookkeeping: sent + residual == x, index order, cap.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import gen
import oracle

M32 = np.uint64(0xFFFFFFFF)


def philox_np(c0, c1, c2, c3, k0, k1):
    """Philox4x32-10 on uint64 arrays that hold 32-bit words (numpy, vectorised)."""
    c0, c1, c2, c3 = (np.asarray(c, np.uint64) for c in (c0, c1, c2, c3))
    k0, k1 = np.uint64(k0), np.uint64(k1)
    for r in range(10):
        if r:
            k0 = (k0 + np.uint64(0x9E3779B9)) & M32
            k1 = (k1 + np.uint64(0xBB67AE85)) & M32
        p0 = c0 * np.uint64(0xD2511F53)
        p1 = c2 * np.uint64(0xCD9E8D57)
        c0, c1, c2, c3 = ((p1 >> np.uint64(32)) ^ c1 ^ k0) & M32, p1 & M32, ((p0 >> np.uint64(32)) ^ c3 ^ k1) & M32, p0 & M32
    return c0, c1, c2, c3


KAT = [  # (counter, key, output) from the generator's published known-answer tests
    ([0, 0, 0, 0], [0, 0], [0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8]),
    ([0xFFFFFFFF] * 4, [0xFFFFFFFF] * 2, [0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD]),
    ([0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344], [0xA4093822, 0x299F31D0],
     [0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1]),
]


@pytest.mark.parametrize("ctr,key,out", KAT)
def test_philox_known_answers(ctr, key, out):
    assert oracle.philox4x32_10(ctr, key) == out
    got = philox_np(*(np.array([c], np.uint64) for c in ctr), *key)
    assert [int(w[0]) for w in got] == out


def uniforms_np(seed, step, n):
    """u_i for i < n, by the stated counter layout, from the numpy generator."""
    q = np.arange((n + 3) // 4, dtype=np.uint64)
    z = np.zeros_like(q)
    words = philox_np(q, z, z + np.uint64(step & 0xFFFFFFFF), z + np.uint64(step >> 32),
                      seed & 0xFFFFFFFF, seed >> 32)
    w = np.stack(words, axis=1).reshape(-1)[:n]
    return (w >> np.uint64(8)).astype(np.float32) * np.float32(2.0 ** -24)


def test_uniform_counter_layout():
    seed, step = 0x0123456789ABCDEF, (7 << 32) + 5
    u = uniforms_np(seed, step, 41)
    for i in range(41):
        assert oracle.uniform(seed, step, i) == u[i]
    assert np.all(u >= 0) and np.all(u < 1)


# ---------------------------------------------------------------- exact sum

def fsum_abs(x):
    x = np.asarray(x, np.float32)
    return math.fsum(np.abs(x[np.isfinite(x)]).astype(np.float64).tolist())


def exact_abs(x):
    x = np.asarray(x, np.float32)
    return float(sum((Fraction(float(abs(v))) for v in x[np.isfinite(x)]), Fraction(0)))


@pytest.mark.parametrize("case", range(6))
def test_sum_abs_exact_matches_fsum(case):
    r = np.random.default_rng(100 + case)
    n = 20_000
    if case == 0:
        x = r.standard_normal(n)
    elif case == 1:  # the whole float32 exponent range, subnormals included
        x = r.uniform(-1.99, 1.99, n) * np.exp2(r.integers(-149, 127, n).astype(np.float64))
    elif case == 2:  # many values near the float32 maximum: the sum leaves float32's range
        x = np.full(n, np.finfo(np.float32).max) * r.uniform(0.5, 1, n)
    elif case == 3:
        x = gen.large_gradient(1, n=n)
    elif case == 4:
        x = gen.specials(n, 5)
    else:  # only subnormals
        x = r.integers(-2**23 + 1, 2**23, n).astype(np.float64) * 2.0 ** -149
    x = np.asarray(x, np.float32)
    assert oracle.sum_abs_exact(x) == fsum_abs(x)


def test_sum_abs_exact_rounding_cases():
    f = np.float32
    cases = [
        [],
        [0.0, -0.0],
        [np.inf, np.nan, -np.inf],
        [1.0, 2.0 ** -53],                 # exact tie, rounds to even (1.0)
        [1.0 + 2.0 ** -23, 2.0 ** -53],    # tie from an odd last bit ... 1+2^-23 is even at 2^-52
        [1.0, 2.0 ** -53, 2.0 ** -149],    # just above the tie
        [1.0, 2.0 ** -52, 2.0 ** -53],     # odd last bit plus half: rounds up
        [2.0 ** 127, 2.0 ** -149],         # far apart: the small one is sticky only
        [2.0 ** -149] * 3,
        [3.0 * 2.0 ** 100, -2.0 ** 47, 2.0 ** 46],
    ]
    for c in cases:
        x = np.array(c, dtype=np.float64).astype(f)
        assert oracle.sum_abs_exact(x) == exact_abs(x) == (fsum_abs(x) if len(x) else 0.0), c


def test_sum_abs_exact_long_carry_chains():
    # 2^24 - 1 in every position of a long sum: carries ripple through several limbs
    x = np.full(300_000, np.float32(16777215.0) * np.float32(2.0 ** 104))
    x = np.concatenate([x, np.full(1000, np.float32(2.0 ** -149))])
    assert oracle.sum_abs_exact(x) == fsum_abs(x)


# ------------------------------------------------------------ sparsification

def draw(n, seed):
    r = np.random.default_rng(seed)
    g = (r.standard_normal(n) * np.exp(r.uniform(-3, 3, n))).astype(np.float32)
    e = (0.1 * r.standard_normal(n)).astype(np.float32)
    return g, e


def check_bookkeeping(g, e, k, seed, step, cap=None):
    x = (g + e).astype(np.float32)
    vals, idx, e2, count, s32, bad = oracle.random_sparsify(g, e, k, seed, step, cap)
    w = len(idx)
    assert w == min(count, x.size if cap is None else cap)
    assert np.all(np.diff(idx) > 0)
    assert np.array_equal(vals.view(np.uint32), x[idx].view(np.uint32))  # sent unscaled
    assert np.all(e2[idx].view(np.uint32) == 0)                          # +0 where sent
    rest = np.ones(x.size, bool)
    rest[idx] = False
    assert np.array_equal(e2[rest].view(np.uint32), x[rest].view(np.uint32))
    assert s32 == np.float32(fsum_abs(x))
    assert bad == int((~np.isfinite(x)).sum())
    return vals, idx, e2, count, s32


def test_brute_force_small():
    """Every decision on small inputs against u < p evaluated with numpy and the
    numpy generator."""
    for n, k, seed, step in [(1, 1, 0, 0), (7, 3, 1, 2), (64, 10, 3, 4), (1001, 100, 2**40 + 9, 2**33 + 1)]:
        g, e = draw(n, n)
        x = (g + e).astype(np.float32)
        s32 = np.float32(fsum_abs(x))
        p = np.float32(k) * np.abs(x) / s32
        p = np.where(p > 1, np.float32(1), p)
        keep = uniforms_np(seed, step, n) < p
        vals, idx, e2, count, _ = check_bookkeeping(g, e, k, seed, step)
        assert idx.tolist() == np.nonzero(keep)[0].tolist()
        assert count == int(keep.sum())


def test_keep_frequencies_follow_magnitude():
    """Over many steps each element is kept with frequency p_i = k|x_i|/S:
    magnitudes 1, 2, 4 and 8 are kept 1:2:4:8 as often, and the mean count is k."""
    mags = np.repeat(np.array([1, 2, 4, 8], np.float32), 16)
    sgn = np.where(np.arange(64) % 3 == 0, -1, 1).astype(np.float32)
    g = mags * sgn
    e = np.zeros_like(g)
    k = 20
    S = float(mags.sum())
    p = np.minimum(1.0, k * mags / S)
    T = 6000
    hits = np.zeros(64)
    counts = []
    for step in range(T):
        _, idx, _, c, _, _ = oracle.random_sparsify(g, e, k, 11, step)
        hits[idx] += 1
        counts.append(c)
    f = hits / T
    sigma = np.sqrt(p * (1 - p) / T)
    assert np.all(np.abs(f - p) < 5 * sigma + 1e-3), np.max(np.abs(f - p) / (sigma + 1e-12))
    assert abs(np.mean(counts) - k) < 5 * np.sqrt(np.sum(p * (1 - p)) / T)


def test_clipped_probabilities_always_kept():
    g = np.array([1000.0] + [1.0] * 99, np.float32)  # k|x0|/S = 10*1000/1099 > 1
    for step in range(200):
        _, idx, _, c, _, _ = oracle.random_sparsify(g, np.zeros(100, np.float32), 10, 3, step)
        assert idx[0] == 0


def test_neighbours_independent():
    """p = 1/2 everywhere: the four elements that share one generator call
    agree about half the time, as independent draws do."""
    n = 40_000
    g = np.ones(n, np.float32)
    _, idx, _, c, _, _ = oracle.random_sparsify(g, np.zeros(n, np.float32), n // 2, 5, 9)
    keep = np.zeros(n, bool)
    keep[idx] = True
    q = keep.reshape(-1, 4)
    for a, b in [(0, 1), (1, 2), (2, 3), (0, 3)]:
        agree = np.mean(q[:, a] == q[:, b])
        assert abs(agree - 0.5) < 5 * 0.5 / np.sqrt(n / 4)
    assert abs(c - n / 2) < 5 * np.sqrt(n / 4)


def test_steps_and_seeds_draw_afresh():
    g, e = draw(5000, 1)
    a = oracle.random_sparsify(g, e, 300, 1, 1)[1]
    assert np.array_equal(a, oracle.random_sparsify(g, e, 300, 1, 1)[1])
    for seed, step in [(1, 2), (2, 1), (1, 1 + 2**32), (1 + 2**32, 1)]:
        b = oracle.random_sparsify(g, e, 300, seed, step)[1]
        assert not np.array_equal(a, b)


def test_zero_probability_with_zero_draw():
    """An element whose draw is exactly 0 (found once by scanning the numpy
    generator over seed 70, step 0): a zero there is not kept (0 < 0 is false)
    while any non-zero value there is (p > 0)."""
    seed, step, i = 70, 0, 5026263
    q = np.array([i // 4], np.uint64)
    z = np.zeros_like(q)
    assert int(philox_np(q, z, z, z, seed, 0)[i % 4][0]) >> 8 == 0
    assert oracle.uniform(seed, step, i) == 0.0
    g = np.ones(i + 1, np.float32)
    g[i] = 0.0
    _, idx, _, _, _, _ = oracle.random_sparsify(g, np.zeros_like(g), 1, seed, step)
    assert i not in set(idx.tolist())
    g[i] = 1e-30
    _, idx, _, _, _, _ = oracle.random_sparsify(g, np.zeros_like(g), 1, seed, step)
    assert i in set(idx.tolist())


def test_k_zero_cap_and_degenerate():
    g, e = draw(3000, 2)
    x = (g + e).astype(np.float32)
    vals, idx, e2, c, _, _ = oracle.random_sparsify(g, e, 0, 1, 1)
    assert c == 0 and idx.size == 0 and np.array_equal(e2.view(np.uint32), x.view(np.uint32))
    # cap below the count: the first cap in index order are sent, the rest stay in e
    full = oracle.random_sparsify(g, e, 500, 4, 4)
    assert full[3] > 100
    vals, idx, e2, c, _ = check_bookkeeping(g, e, 500, 4, 4, cap=100)
    assert c == full[3] and idx.tolist() == full[1][:100].tolist()
    late = full[1][100:]
    assert np.array_equal(e2[late].view(np.uint32), x[late].view(np.uint32))
    # all zero: S = 0 and nothing is kept; empty input
    z = np.zeros(100, np.float32)
    assert oracle.random_sparsify(z, z, 10, 1, 1)[3] == 0
    assert oracle.random_sparsify(np.zeros(0, np.float32), np.zeros(0, np.float32), 10, 1, 1)[3] == 0
    # k larger than n: every p is clipped to 1 for magnitudes above the mean
    g2 = np.array([1, 1, 1, 5], np.float32)
    _, idx, _, _, _, _ = oracle.random_sparsify(g2, np.zeros(4, np.float32), 100, 1, 1)
    assert idx.tolist() == [0, 1, 2, 3]


def test_non_finite_never_kept():
    g, e = draw(4000, 3)
    g[::97] = np.inf
    g[5::101] = np.nan
    vals, idx, e2, c, s32 = check_bookkeeping(g, e, 3999, 6, 6)
    x = g + e
    assert np.all(np.isfinite(x[idx]))
    assert s32 == np.float32(fsum_abs(x))


def test_lognormal_workload_expected_count():
    """The large workload's gradient law at a reduced size: the count stays
    within a few standard deviations of sum(p) <= k."""
    n, k = 2_000_000, 2000
    g = gen.large_gradient(0, n=n)
    x = g.astype(np.float32)
    s32 = np.float32(fsum_abs(x))
    p = np.minimum(np.float32(1), np.float32(k) * np.abs(x) / s32).astype(np.float64)
    _, idx, _, c, _, _ = oracle.random_sparsify(g, np.zeros(n, np.float32), k, 123, 0)
    mu, sd = p.sum(), math.sqrt(np.sum(p * (1 - p)))
    assert mu <= k and abs(c - mu) < 6 * sd


def test_keep_at_matches_full_run():
    g, e = draw(20_000, 8)
    x = (g + e).astype(np.float32)
    _, idx, _, c, s32, _ = oracle.random_sparsify(g, e, 700, 9, 3)
    pos = np.arange(x.size)
    keep = oracle.random_keep_at(x, pos, 700, np.float32(s32), 9, 3)
    assert np.nonzero(keep)[0].tolist() == idx.tolist()
    sub = np.array([19_999, 0, 5, 4, 12_345], np.int64)
    assert oracle.random_keep_at(x[sub], sub, 700, np.float32(s32), 9, 3).tolist() == keep[sub].tolist()
