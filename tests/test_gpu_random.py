"""GPU parity of random magnitude-proportional sparsification against the CPU
oracle: bit for bit on vals, idx, the count, S32, the non-finite count and the
whole residual, at sizes that span many regions and ragged tails; at the large
workload's full size, S32 against a certified float64 sum, every decision in
sampled windows and at every kept position, and the bookkeeping everywhere."""
import math

import numpy as np
import pytest
import torch

import error_feedback_gradient_amd as efg
import gen
import oracle
from gpu_util import assert_bits_equal, device, host, say, to_dev

pytestmark = pytest.mark.gpu

REGION = 8192


def inputs(kind, n, key):
    if kind == "normal":
        g = gen.normal_small(n, 700, key)
    elif kind == "lognormal":
        g = gen.large_gradient(key, n=n)
    elif kind == "ties":
        g = gen.uniform_ties(n, 5, 701, key)
    elif kind == "specials":
        g = gen.specials(n, 702, key)
    elif kind == "zeros":
        g = np.zeros(n, np.float32)
    else:
        raise ValueError(kind)
    e = gen.normal_small(n, 703, key, scale=0.01)
    return g, e


def run_gpu(g, e, k, seed, step, cap, flags=0):
    dev = device()
    gd, ed = to_dev(g, dev), to_dev(e, dev)
    s32 = torch.empty(1, dtype=torch.float32, device=dev)
    nf = torch.zeros(1, dtype=torch.int32, device=dev)
    vals, idx, cnt = efg.ef_random_sparsify(gd, ed, k, seed, step, cap=cap, sum_out=s32, nonfinite=nf, flags=flags)
    c = int(host(cnt)[0])
    w = min(c, cap)
    return host(vals)[:w], host(idx)[:w], host(ed), c, np.float32(host(s32)[0]), int(host(nf)[0])


def check(g, e, k, seed, step, cap=None, flags=0, what=""):
    n = g.size
    if cap is None:
        cap = max(1, 2 * k + 64)
    v, i, e2, c, s32, nf = run_gpu(g, e, k, seed, step, cap, flags)
    ov, oi, oe, oc, os32, onf = oracle.random_sparsify(g, e, k, seed, step, cap)
    assert c == oc, (what, c, oc)
    assert np.float32(s32).view(np.uint32) == np.float32(os32).view(np.uint32), (what, s32, os32)
    assert nf == onf, (what, nf, onf)
    assert_bits_equal(i, oi, f"idx {what}")
    assert_bits_equal(v, ov, f"vals {what}")
    assert_bits_equal(e2, oe, f"e {what}")
    return c


SIZES = [1, 3, 4, 5, 63, 1000, REGION - 1, REGION, REGION + 1, 3 * REGION + 7, 100_003, (1 << 20) + 3]


@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("kind", ["normal", "lognormal", "ties", "specials"])
def test_sizes_and_kinds(n, kind):
    g, e = inputs(kind, n, n % 1000)
    for k in sorted({0, 1, max(1, n // 100), n}):
        check(g, e, k, 12345, 7, what=f"{kind} n={n} k={k}")


@pytest.mark.parametrize("n", [5, REGION + 1, 100_003, (1 << 20) + 3])
def test_forced_exact_sum(n):
    g, e = inputs("lognormal", n, 3)
    check(g, e, max(1, n // 50), 1, 2, flags=efg.EF_FLAG_FORCE_FALLBACK, what=f"exact n={n}")
    g, e = inputs("specials", n, 4)
    check(g, e, max(1, n // 50), 1, 2, flags=efg.EF_FLAG_FORCE_FALLBACK, what=f"exact specials n={n}")


def test_wide_exponent_range_and_subnormals():
    r = np.random.default_rng(5)
    n = 3 * REGION + 5
    g = (r.uniform(-1.99, 1.99, n) * np.exp2(r.integers(-149, 127, n).astype(np.float64))).astype(np.float32)
    e = np.zeros(n, np.float32)
    for flags in (0, efg.EF_FLAG_FORCE_FALLBACK):
        check(g, e, 500, 2, 2, flags=flags, what=f"wide flags={flags}")
    sub = (r.integers(-2**23 + 1, 2**23, n).astype(np.float64) * 2.0 ** -149).astype(np.float32)
    for flags in (0, efg.EF_FLAG_FORCE_FALLBACK):
        check(sub, e, 500, 2, 2, flags=flags, what=f"subnormal flags={flags}")
    big = np.full(n, np.finfo(np.float32).max, np.float32) * np.float32(0.75)  # S32 = inf: nothing kept
    assert check(big, e, 500, 2, 2, what="S overflow") == 0


def test_degenerate_inputs():
    z = np.zeros(REGION + 3, np.float32)
    assert check(z, z, 100, 1, 1, what="all zero") == 0
    one = np.zeros(1000, np.float32)
    one[777] = -3.0
    assert check(one, np.zeros_like(one), 1, 1, 1, what="single non-zero") == 1  # p = 1
    nan = np.full(1000, np.nan, np.float32)
    assert check(nan, np.zeros_like(nan), 10, 1, 1, what="all NaN") == 0


def test_cap_below_count():
    g, e = inputs("normal", 200_003, 8)
    full = check(g, e, 5000, 3, 3, what="uncapped")
    for cap in (0, 1, 4999, full - 1, full):
        check(g, e, 5000, 3, 3, cap=cap, what=f"cap={cap}")


def test_seed_and_step_words():
    g, e = inputs("lognormal", 50_000, 9)
    for seed, step in [(0, 0), (2**64 - 1, 2**64 - 1), (0x0123456789ABCDEF, 2**32 + 3), (7, 2**40)]:
        check(g, e, 1000, seed, step, what=f"seed={seed} step={step}")


def test_chained_steps():
    """Ten steps with a fresh gradient each: the residual carries between calls."""
    n, k = 1_000_003, 10_000
    dev = device()
    e_o = np.zeros(n, np.float32)
    ed = torch.zeros(n, dtype=torch.float32, device=dev)
    for step in range(10):
        g = gen.flat_gradient(step, n=n)
        vals, idx, cnt = efg.ef_random_sparsify(to_dev(g, dev), ed, k, 99, step)
        c = int(host(cnt)[0])
        ov, oi, e_o, oc, _, _ = oracle.random_sparsify(g, e_o, k, 99, step)
        assert c == oc, (step, c, oc)
        assert_bits_equal(host(idx)[:c], oi, f"idx step {step}")
        assert_bits_equal(host(vals)[:c], ov, f"vals step {step}")
        assert_bits_equal(host(ed), e_o, f"e step {step}")


def test_empty():
    dev = device()
    g = torch.zeros(0, dtype=torch.float32, device=dev)
    cnt = torch.full((1,), 5, dtype=torch.int64, device=dev)
    s32 = torch.full((1,), 5.0, dtype=torch.float32, device=dev)
    efg.ef_random_sparsify(g, g.clone(), 10, 1, 1, count=cnt, sum_out=s32)
    assert int(host(cnt)[0]) == 0 and float(host(s32)[0]) == 0.0


def certified_s32(x_host):
    """float32(S) from a float64 sum with an error bound (None if the bound
    straddles a float32 rounding boundary)."""
    t = 0.0
    terms = 0
    for lo in range(0, x_host.size, 1 << 26):
        a = np.abs(x_host[lo:lo + (1 << 26)]).astype(np.float64)
        a[~np.isfinite(a)] = 0.0
        t = t + float(np.sum(a))  # numpy: pairwise summation, error <= ~27 u per chunk
        terms += 1
    rel = (64 + terms) * 2.0 ** -53
    lo, hi = np.float32(t * (1 - 4 * rel)), np.float32(t * (1 + 4 * rel))
    return lo if lo == hi else None


@pytest.mark.parametrize("flags", [0, 1])
def test_large_workload_full_size(flags):
    """N = 1.3e9, k = 1.3e6, two chained steps of the large workload's gradient
    law (drawn on the device), in the configuration the benchmark times."""
    dev = device()
    n, k, seed = gen.LARGE_N, gen.LARGE_K, gen.RANDOM_SEED
    cap = 2 * k + 64
    e = torch.zeros(n, dtype=torch.float32, device=dev)
    ws = efg.workspace(efg.lib().ef_random_sparsify_workspace_bytes(n), dev)
    r = np.random.default_rng(17)
    for step in range(2):
        say(f"random full size flags={flags} step={step}: drawing")
        g = gen.large_gradient_device(step, n, dev)
        x = g + e  # float32 elementwise, as the kernel does
        s32 = torch.empty(1, dtype=torch.float32, device=dev)
        nf = torch.zeros(1, dtype=torch.int32, device=dev)
        say(f"random full size flags={flags} step={step}: compress")
        vals, idx, cnt = efg.ef_random_sparsify(g, e, k, seed, step, cap=cap, sum_out=s32, nonfinite=nf, ws=ws,
                                                flags=flags)
        torch.cuda.synchronize()
        c = int(host(cnt)[0])
        S = np.float32(host(s32)[0])
        assert 0 < c <= cap and int(host(nf)[0]) == 0
        ik = idx[:c].long()
        # bookkeeping on the device: vals = x[idx], idx increasing, e = x except +0 at idx
        assert bool((ik[1:] > ik[:-1]).all()) and int(ik[0]) >= 0 and int(ik[-1]) < n
        assert torch.equal(vals[:c].view(torch.int32), x[ik].view(torch.int32))
        want = x.clone()
        want[ik] = 0.0
        assert torch.equal(e.view(torch.int32), want.view(torch.int32))
        del want
        # S32 against an independent float64 sum
        say(f"random full size flags={flags} step={step}: checking S and decisions")
        xh = host(x)
        cs = certified_s32(xh)
        if cs is None:
            cs = np.float32(oracle.sum_abs_exact(xh))
        assert cs.view(np.uint32) == S.view(np.uint32), (cs, S)
        # every decision in 48 random windows (and the final one) and at every kept position
        kept = host(ik)
        starts = np.concatenate([r.integers(0, n - 65536, 48), [n - 65536]])
        pos = np.unique(np.concatenate([np.arange(s, s + 65536) for s in starts] + [kept]))
        keep = oracle.random_keep_at(xh[pos], pos, k, S, seed, step)
        member = np.isin(pos, kept, assume_unique=True)
        bad = np.nonzero(keep != member)[0]
        assert bad.size == 0, (bad.size, pos[bad[:5]])
        # count against its law: mean sum(p) <= k
        p = torch.clamp(float(k) * x.abs() / float(S), max=1.0).double()
        mu, sd = float(p.sum()), math.sqrt(float((p * (1 - p)).sum()))
        assert abs(c - mu) < 6 * sd and mu <= k * (1 + 1e-6), (c, mu, sd)
        say(f"random full size flags={flags} step={step}: ok (kept {c}, S={S})")
        del g, x, p, xh


def boundary_case(k, delta_ulps, seed=31, step=4, n=4096):
    """Probabilities that sit on top of their draws: x_j = u_j for j >= 1 and
    x_0 chosen so that S32 = k (+- a few ulps); every p_j is then u_j up to
    the last bits, so each decision is settled by rounding alone."""
    u = np.array([oracle.uniform(seed, step, j) for j in range(n)], np.float32)
    g = u.copy()
    rest = float(np.sum(u[1:].astype(np.float64)))
    ulp = float(np.spacing(np.float32(k)))
    g[0] = np.float32(k + delta_ulps * ulp - rest)
    return g, np.zeros(n, np.float32), seed, step


@pytest.mark.parametrize("k,d", [(8192, -3), (8192, -1), (8192, 0), (8192, 1), (8191, -1), (8191, 0), (8191, 1),
                                 (6000, 0), (6001, 2)])
def test_probabilities_on_their_draws(k, d):
    g, e, seed, step = boundary_case(k, d)
    for flags in (0, efg.EF_FLAG_FORCE_FALLBACK):
        check(g, e, k, seed, step, flags=flags, what=f"boundary k={k} d={d} flags={flags}")


def test_sum_above_reciprocal_range():
    """S between 2^126 and the float32 maximum: 1/S is subnormal, every
    decision takes the division."""
    n = 1000
    g = np.full(n, np.float32(2.0 ** 117), np.float32) * gen.normal_small(n, 710).astype(np.float32)
    e = np.zeros(n, np.float32)
    S = oracle.sum_abs_exact(g)
    assert 2.0 ** 126 < S < float(np.finfo(np.float32).max)
    check(g, e, 100, 5, 5, what="S > 2^126")
