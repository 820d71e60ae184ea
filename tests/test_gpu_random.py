"""GPU parity of random magnitude-proportional sparsification against the CPU
oracle: bit for bit on vals, idx, the count, S32, the non-finite count and the
whole residual, at sizes that span many regions and ragged tails; at the large
workload's full size, S32 against a certified float64 sum, every decision in
sampled windows and at every kept position, and the bookkeeping everywhere.

Both ways a call can decide are covered: the candidate slots filled by the
accumulation pass (calls with n >= 65536 and k <= n / 512, when the sampled
guess S_lo is at most S32 and no slot overflows) and the second marking pass;
call_path reads which one a call took from the library's call state."""
import math

import numpy as np
import pytest
import torch

import error_feedback_gradient_amd as efg
import gen
import oracle
from gpu_util import assert_bits_equal, device, host, say, to_dev

pytestmark = pytest.mark.gpu

REGION = 4096


def call_path(ws):
    """'slots' or 'two-pass', from the call state the library keeps at the
    start of its workspace (float32 S32 at byte 8, float32 S_lo at byte 24,
    uint32 slot-overflow flag at byte 28)."""
    b = host(ws[:64]).tobytes()
    s32 = np.frombuffer(b, np.float32, 1, 8)[0]
    slo = np.frombuffer(b, np.float32, 1, 24)[0]
    ovf = np.frombuffer(b, np.uint32, 1, 28)[0]
    return "slots" if slo > 0 and ovf == 0 and s32 >= slo else "two-pass"


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
    ws = efg.workspace(efg.lib().ef_random_sparsify_workspace_bytes(g.size), dev)
    vals, idx, cnt = efg.ef_random_sparsify(gd, ed, k, seed, step, cap=cap, sum_out=s32, nonfinite=nf, ws=ws,
                                            flags=flags)
    c = int(host(cnt)[0])
    w = min(c, cap)
    return host(vals)[:w], host(idx)[:w], host(ed), c, np.float32(host(s32)[0]), int(host(nf)[0]), call_path(ws)


def check(g, e, k, seed, step, cap=None, flags=0, what="", path=None):
    n = g.size
    if cap is None:
        cap = max(1, 2 * k + 64)
    v, i, e2, c, s32, nf, took = run_gpu(g, e, k, seed, step, cap, flags)
    if path is not None:
        assert took == path, (what, took, path)
    ov, oi, oe, oc, os32, onf = oracle.random_sparsify(g, e, k, seed, step, cap)
    assert c == oc, (what, c, oc)
    assert np.float32(s32).view(np.uint32) == np.float32(os32).view(np.uint32), (what, s32, os32)
    assert nf == onf, (what, nf, onf)
    assert_bits_equal(i, oi, f"idx {what}")
    assert_bits_equal(v, ov, f"vals {what}")
    assert_bits_equal(e2, oe, f"e {what}")
    return c


SIZES = [1, 3, 4, 5, 63, 1000, REGION - 1, REGION, REGION + 1, 2 * REGION + 1, 3 * REGION + 7, 100_003,
         (1 << 20) + 3]


@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("kind", ["normal", "lognormal", "ties", "specials"])
def test_sizes_and_kinds(n, kind):
    g, e = inputs(kind, n, n % 1000)
    for k in sorted({0, 1, max(1, n // 100), n}):
        check(g, e, k, 12345, 7, what=f"{kind} n={n} k={k}")


@pytest.mark.parametrize("n", [65536, 65536 + 5, 16 * REGION * 3 + 7, (1 << 20) + 3, 3_000_017])
@pytest.mark.parametrize("kind", ["normal", "lognormal", "ties"])
def test_candidate_slots(n, kind):
    """Few kept per region: the accumulation pass's candidates decide."""
    g, e = inputs(kind, n, n % 997)
    for k in sorted({1, n // 4096, n // 512}):
        check(g, e, k, 4242, 3, what=f"slots {kind} n={n} k={k}", path="slots")
        check(g, e, k, 4242, 3, flags=efg.EF_FLAG_FORCE_FALLBACK, what=f"forced {kind} n={n} k={k}",
              path="two-pass")


def test_slots_given_up_on_a_high_guess():
    """n = 2^22: the sample reads chunks 4j of 256 elements.  Mass only there
    makes the guess S_lo = 7/8 n * 1 three and a half times S: the second pass
    decides."""
    n = 1 << 22
    x = np.repeat((np.arange(n // 256) % 4 == 0).astype(np.float32), 256)
    check(x, np.zeros(n, np.float32), 4096, 5, 6, what="high guess", path="two-pass")


def test_slots_given_up_on_overflow():
    """One region holding most of S has far more than 64 candidates."""
    n = 1 << 20
    g, e = inputs("normal", n, 11)
    g[7 * REGION:8 * REGION] = np.float32(1000.0)
    dev = device()
    ws = efg.workspace(efg.lib().ef_random_sparsify_workspace_bytes(n), dev)
    efg.ef_random_sparsify(to_dev(g, dev), to_dev(e, dev), n // 512, 5, 6, ws=ws)
    assert np.frombuffer(host(ws[:64]).tobytes(), np.uint32, 1, 28)[0] == 1
    check(g, e, n // 512, 5, 6, what="overflow", path="two-pass")


def guess_equals_sum_case(delta, seed=77, step=5):
    """n = 2^22, k = 4096.  Ones fill the sampled chunks (chunks 4j of 256), so
    S_lo = 0.875 * 2^22 = 3670016 exactly; the other chunks hold 200 elements
    whose probabilities k v / S32 = v / 896 sit within two ulps of their draws,
    then ones and one fraction so that S32 = S_lo + delta ulps (ulp 0.25)."""
    n, k = 1 << 22, 4096
    smask = np.repeat(np.arange(n // 256) % 4 == 0, 256)
    x = smask.astype(np.float32)
    free = np.nonzero(~smask)[0]
    bpos = free[::15000][:200]
    u = np.array([oracle.uniform(seed, step, int(j)) for j in bpos], np.float32)
    v = (np.float32(896.0) * u).astype(np.float32)
    v = (v.view(np.int32) + (np.arange(bpos.size, dtype=np.int32) % 5 - 2)).view(np.float32)
    v[v <= 0] = np.float32(1.0)
    x[bpos] = v
    rest = 3670016.0 + 0.25 * delta - float(np.sum(x.astype(np.float64)))
    ones = int(math.floor(rest))
    fill = np.setdiff1d(free, bpos)[:ones + 1]
    x[fill[:ones]] = 1.0
    x[fill[ones]] = np.float32(rest - ones)
    assert np.float32(oracle.sum_abs_exact(x)) == np.float32(3670016.0 + 0.25 * delta)
    return x, k, seed, step


@pytest.mark.parametrize("delta,path", [(-1, "two-pass"), (0, "slots"), (1, "slots")])
def test_guess_at_the_sum(delta, path):
    """S_lo against S32 at equality and one ulp either side, with decisions
    settled by the last bits of the probability."""
    x, k, seed, step = guess_equals_sum_case(delta)
    check(x, np.zeros_like(x), k, seed, step, what=f"S32 = S_lo + {delta} ulp", path=path)


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


@pytest.mark.parametrize("k", [10_000, 1_000])
def test_chained_steps(k):
    """Ten steps with a fresh gradient each: the residual carries between calls
    (k = 1000 decides from the candidate slots, k = 10000 by the second pass)."""
    n = 1_000_003
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
        assert call_path(ws) == ("two-pass" if flags else "slots")
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
