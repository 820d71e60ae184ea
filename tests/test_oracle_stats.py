"""Pins of the oracle's monitoring statistic (CPU only)."""
import math

import numpy as np

import gen
import oracle


def test_closed_forms():
    assert oracle.sumsq(np.ones(1000, np.float32)) == 1000.0
    assert oracle.sumsq(np.arange(1, 101, dtype=np.float32)) == 100 * 101 * 201 / 6
    assert oracle.sumsq(np.zeros(0, np.float32)) == 0.0
    assert oracle.sumsq(np.array([np.nan, np.inf, -np.inf, 3.0, -4.0], np.float32)) == 25.0


def test_against_exact_summation():
    a = gen.large_gradient(2, n=200_000)
    exact = math.fsum(float(v) * float(v) for v in a)  # squares are exact; fsum is correctly rounded
    got = oracle.sumsq(a)
    assert abs(got - exact) <= a.size * 2.0 ** -53 * exact
    # in-order summation: bitwise equal to a plain Python loop in the same order
    s = 0.0
    for v in a[:5000]:
        s += float(v) * float(v)
    assert oracle.sumsq(a[:5000]) == s
