"""Pins of the oracle's float32 recurrences against exact rational arithmetic.

Every operation of the 1-bit step (page "1bit Adam梯度压缩技术原理与分布式训练优化",
sections 2.1 and 2.2), of the Adam step around it (section 3.1's state, the
textbook Adam rules) and of the SGD update (page "梯度稀疏化：只传输重要的梯度元素",
step-by-step algorithm, step 7) is evaluated here on Python Fractions, and each
result is rounded to binary32 by `rnd32`, written from the IEEE 754 definition
(round to nearest, ties to even, gradual underflow, overflow to infinity).
Nothing here goes through numpy's or the C compiler's float32 arithmetic, so
these pins are independent of the oracle's own evaluation.

The readings they fix: one rounding per product, sum and difference (no fused
multiply-add), (1 - beta) as the float32 difference of 1 and the float32 beta,
and correctly rounded square roots and divisions.  Each test also shows, on
the same inputs, that the alternatives (a fused multiply-add, or (1 - beta)
taken as the float32 value of the decimal complement) give different bits, so
a mistake of that kind in the oracle would fail here.
"""
from __future__ import annotations

import math
import struct
from fractions import Fraction

import numpy as np
import pytest

import oracle


# ------------------------------------------------------------ exact binary32 model
def pow2(e: int) -> Fraction:
    return Fraction(1 << e) if e >= 0 else Fraction(1, 1 << -e)


def f32_bits(x: float) -> int:
    return struct.unpack("<I", struct.pack("<f", x))[0]


def neg_zero(x: float) -> bool:
    return x == 0.0 and math.copysign(1.0, x) < 0


def rnd32(q: Fraction, zero_sign: float = 1.0) -> float:
    """q rounded to binary32 (nearest, ties to even), as a Python float (which
    holds every binary32 value exactly).  A zero result takes zero_sign's sign
    when q is 0, else q's sign (underflow keeps the sign)."""
    if q == 0:
        return math.copysign(0.0, zero_sign)
    neg = q < 0
    a = -q if neg else q
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if a < pow2(e):
        e -= 1
    e = max(e, -126)                   # below 2^-126 the quantum stays 2^-149
    quantum = pow2(e - 23)
    m = a / quantum
    n = m.numerator // m.denominator
    rem = m - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    r = n * quantum
    if r >= pow2(128):
        return -math.inf if neg else math.inf
    v = float(r)                       # exact: r is a binary32 value
    return -v if neg else v


def F(x: float) -> Fraction:
    return Fraction(x)


def add32(x: float, y: float) -> float:
    s = F(x) + F(y)
    # an exact zero sum is +0, except (-0) + (-0)
    return rnd32(s, -1.0 if (s == 0 and neg_zero(x) and neg_zero(y)) else 1.0)


def sub32(x: float, y: float) -> float:
    return add32(x, -y)


def mul32(x: float, y: float) -> float:
    sgn = -1.0 if (math.copysign(1.0, x) * math.copysign(1.0, y)) < 0 else 1.0
    return rnd32(F(x) * F(y), sgn)


def div32(x: float, y: float) -> float:
    sgn = -1.0 if (math.copysign(1.0, x) * math.copysign(1.0, y)) < 0 else 1.0
    return rnd32(F(x) / F(y), sgn)


def next32(y: float) -> float:
    b = f32_bits(y)
    return struct.unpack("<f", struct.pack("<I", b + 1))[0]


def prev32(y: float) -> float:
    b = f32_bits(y)
    return struct.unpack("<f", struct.pack("<I", b - 1))[0]


def sqrt32(x: float) -> float:
    """Correctly rounded binary32 square root of a binary32 x >= 0: the
    neighbours around sqrt(x) are found by exact squares, and the midpoint
    between them decides (a binary32 square root is never exactly halfway)."""
    if x == 0.0:
        return x
    X = F(x)
    y = rnd32(Fraction(math.sqrt(x)))
    while F(y) * F(y) > X:
        y = prev32(y)
    while F(next32(y)) * F(next32(y)) <= X:
        y = next32(y)
    lo, hi = y, next32(y)
    if F(lo) * F(lo) == X:
        return lo
    mid = (F(lo) + F(hi)) / 2
    return hi if mid * mid < X else lo


def f32(x) -> float:
    return float(np.float32(x))


def bits(a) -> np.ndarray:
    return np.asarray(a, np.float32).view(np.uint32)


def rand_f32(rs: np.random.Generator, n: int, lo: int, hi: int) -> np.ndarray:
    """n float32 values with random signs, exponents in [lo, hi) and full
    random mantissas (so products and sums round, and some underflow)."""
    mant = rs.integers(1 << 23, 1 << 24, size=n).astype(np.float64)
    ex = rs.integers(lo, hi, size=n)
    sgn = np.where(rs.integers(0, 2, size=n) == 1, -1.0, 1.0)
    return (sgn * np.ldexp(mant, ex - 23)).astype(np.float32)


# ------------------------------------------------------------ checks of the model itself
def test_rnd32_agrees_with_the_hardware_rounding_of_doubles():
    """rnd32 of a double equals numpy's float32 conversion of it (both round
    to nearest, ties to even) on random doubles, halfway cases, subnormals and
    the overflow edge."""
    rs = np.random.default_rng(5)
    xs = list(rs.standard_normal(2000) * np.exp2(rs.integers(-160, 130, size=2000)))
    one = 1.0 + 2.0 ** -24          # halfway between 1 and the next float32: ties to even -> 1
    xs += [one, 1.0 + 3 * 2.0 ** -24, 2.0 ** -149, 2.0 ** -150, 3 * 2.0 ** -150, 2.0 ** -126 * (1 - 2.0 ** -25),
           float(np.finfo(np.float32).max), 2.0 ** 128 * (1 - 2.0 ** -25), -2.0 ** 128 * (1 - 2.0 ** -24)]
    with np.errstate(over="ignore"):
        for x in xs:
            assert f32_bits(rnd32(Fraction(x))) == f32_bits(float(np.float32(x))), x


# ------------------------------------------------------------ 1-bit step
def sign_model(g, e, m, beta1, clip):
    b = f32(beta1)
    c = sub32(1.0, b)
    out_e, out_m, out_s = [], [], []
    for gi, ei, mi in zip(g.tolist(), e.tolist(), m.tolist()):
        gc = clip if gi > clip else (-clip if gi < -clip else gi)
        x = add32(gc, ei)
        s = 1 if x > 0 else (-1 if x < 0 else 0)
        q = float(s)
        d = sub32(x, q)
        out_e.append(add32(mul32(b, ei), mul32(c, d)))
        out_m.append(add32(mul32(b, mi), mul32(c, q)))
        out_s.append(s)
    return np.array(out_e, np.float32), np.array(out_m, np.float32), np.array(out_s, np.int8)


@pytest.mark.parametrize("beta1", [0.9, 0.999, 0.37])
def test_sign_step_matches_exact_rounding_per_operation(beta1):
    rs = np.random.default_rng(int(beta1 * 1000))
    n = 600
    g = rand_f32(rs, n, -8, 4)
    e = rand_f32(rs, n, -140, 2)   # down to subnormals: beta1 * e underflows gradually
    m = rand_f32(rs, n, -20, 1)
    g[:4] = [7.0, -7.0, 5.0, -5.0]  # clipped, and at the clip bound
    e2, m2, s, _, _ = oracle.sign(g, e, m, beta1, 5.0)
    me, mm, ms = sign_model(g, e, m, beta1, 5.0)
    assert np.array_equal(s, ms)
    assert np.array_equal(bits(e2), bits(me))
    assert np.array_equal(bits(m2), bits(mm))


def test_sign_step_alternative_readings_differ():
    """On the same kind of inputs a fused multiply-add in e' (one rounding of
    beta1*e + fl(c*delta)), or c = fl32(0.1) instead of 1 - fl32(0.9), changes
    the bits of some e' or m': the exact per-operation model above is what
    tells the readings apart, and the oracle follows the plain one."""
    rs = np.random.default_rng(77)
    n = 600
    g = rand_f32(rs, n, -8, 4)
    e = rand_f32(rs, n, -12, 2)
    m = rand_f32(rs, n, -20, 1)
    beta1 = 0.9
    b = f32(beta1)
    c = sub32(1.0, b)
    c_dec = rnd32(Fraction(1, 10))
    assert c != c_dec, "1 - fl32(0.9) and fl32(0.1) are different float32 values"
    e2, m2, _, _, _ = oracle.sign(g, e, m, beta1, 5.0)
    fused = dec = 0
    for i, (gi, ei, mi) in enumerate(zip(g.tolist(), e.tolist(), m.tolist())):
        x = add32(gi, ei)
        q = float(1 if x > 0 else (-1 if x < 0 else 0))
        d = sub32(x, q)
        eb = mul32(c, d)
        fma = rnd32(F(b) * F(ei) + F(eb))
        fused += f32_bits(fma) != f32_bits(float(e2[i]))
        alt = add32(mul32(b, ei), mul32(c_dec, d))
        dec += f32_bits(alt) != f32_bits(float(e2[i]))
    assert fused > 0, "no input separates the fused from the plain evaluation"
    assert dec > n // 4, "c = fl32(0.1) should change most residuals"


# ------------------------------------------------------------ SGD update
def test_sgd_matches_exact_rounding_and_is_not_fused():
    rs = np.random.default_rng(3)
    n = 2000
    w = rand_f32(rs, n, -6, 3)
    G = rand_f32(rs, n, -10, 4)
    lr = 0.1
    out = oracle.sgd(w, G, lr)
    L = f32(lr)
    model = np.array([sub32(wi, mul32(L, gi)) for wi, gi in zip(w.tolist(), G.tolist())], np.float32)
    assert np.array_equal(bits(out), bits(model))
    fused = sum(f32_bits(rnd32(F(wi) - F(L) * F(gi))) != f32_bits(float(o))
                for wi, gi, o in zip(w.tolist(), G.tolist(), out.tolist()))
    assert fused > 0


# ------------------------------------------------------------ Adam step (warm-up) and 1-bit update
def adam_param_model(w, m, v, step_size, sqrt_bc2, eps):
    r = sqrt32(v)
    q = div32(r, sqrt_bc2)
    d = add32(q, eps)
    u = div32(m, d)
    s = mul32(step_size, u)
    return sub32(w, s)


def test_sqrt32_is_correctly_rounded():
    rs = np.random.default_rng(9)
    for v in rand_f32(rs, 500, -149, 100).tolist() + [2.0, 3.0, 0.5, 1e-45, 2.0 ** -148]:
        v = abs(v)
        y = sqrt32(v)
        # y is the float32 nearest to sqrt(v): both neighbours are farther away (compared exactly via squares)
        lo, hi = prev32(y), next32(y)
        assert (F(lo) + F(y)) ** 2 / 4 <= F(v) <= (F(y) + F(hi)) ** 2 / 4, v


@pytest.mark.parametrize("beta1,beta2", [(0.9, 0.999), (0.8, 0.99)])
def test_adam_step_matches_exact_rounding_per_operation(beta1, beta2):
    rs = np.random.default_rng(11)
    n = 400
    g = rand_f32(rs, n, -14, 2)
    m = rand_f32(rs, n, -16, -2)
    v = np.abs(rand_f32(rs, n, -30, -4))
    w = rand_f32(rs, n, -6, 2)
    step_size, sqrt_bc2 = oracle.adam_scalars(2e-5, beta1, beta2, 3)
    eps = 1e-8
    m2, v2, w2, _ = oracle.adam_step(g, m, v, w, beta1, beta2, step_size, sqrt_bc2, eps)
    b1, b2, E = f32(beta1), f32(beta2), f32(eps)
    c1, c2 = sub32(1.0, b1), sub32(1.0, b2)
    S, B = f32(step_size), f32(sqrt_bc2)
    for i in range(n):
        gi, mi, vi, wi = float(g[i]), float(m[i]), float(v[i]), float(w[i])
        mn = add32(mul32(b1, mi), mul32(c1, gi))
        vn = add32(mul32(b2, vi), mul32(c2, mul32(gi, gi)))
        wn = adam_param_model(wi, mn, vn, S, B, E)
        assert f32_bits(float(m2[i])) == f32_bits(mn), ("m", i)
        assert f32_bits(float(v2[i])) == f32_bits(vn), ("v", i)
        assert f32_bits(float(w2[i])) == f32_bits(wn), ("w", i)


@pytest.mark.parametrize("nworkers", [1, 3, 7])
def test_onebit_update_matches_exact_rounding_per_operation(nworkers):
    rs = np.random.default_rng(13 + nworkers)
    n = 400
    qsum = rs.integers(-nworkers, nworkers + 1, size=n).astype(np.int8)
    m = rand_f32(rs, n, -16, -2)
    v = np.abs(rand_f32(rs, n, -30, -4))
    w = rand_f32(rs, n, -6, 2)
    beta1, eps = 0.9, 1e-8
    step_size, sqrt_bc2 = oracle.adam_scalars(2e-5, beta1, 0.999, 9, 3)
    m2, w2, _ = oracle.onebit_adam_update(qsum, nworkers, m, v, w, beta1, step_size, sqrt_bc2, eps)
    b1, E = f32(beta1), f32(eps)
    c1 = sub32(1.0, b1)
    S, B = f32(step_size), f32(sqrt_bc2)
    for i in range(n):
        ghat = div32(float(qsum[i]), float(nworkers))
        mn = add32(mul32(b1, float(m[i])), mul32(c1, ghat))
        wn = adam_param_model(float(w[i]), mn, float(v[i]), S, B, E)
        assert f32_bits(float(m2[i])) == f32_bits(mn), ("m", i)
        assert f32_bits(float(w2[i])) == f32_bits(wn), ("w", i)
