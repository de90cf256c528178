"""Pins for the oracle add: exact fp64 sum rounded once to fp32 (single
rounding equals the IEEE fp32 add whenever the fp64 sum is exact), plus
special cases."""
import numpy as np

from oracle.add import add_f32


def test_add_equals_exact_sum_rounded_once():
    r = np.random.default_rng(1)
    X = r.standard_normal(200_000).astype(np.float32)
    Y = r.standard_normal(200_000).astype(np.float32)
    ex = np.frexp(X)[1].astype(np.int64)
    ey = np.frexp(Y)[1].astype(np.int64)
    ok = np.abs(ex - ey) <= 28          # then x + y is exact in fp64
    ok &= (X != 0) & (Y != 0)
    assert ok.mean() > 0.99
    want = (X[ok].astype(np.float64) + Y[ok].astype(np.float64)).astype(np.float32)
    got = add_f32(X[ok], Y[ok])
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_add_special_cases():
    x = np.array([1.5, -2.0, 3.0e38, 1e-45, 0.0], np.float32)
    got = add_f32(x, -x)
    assert np.array_equal(got.view(np.uint32), np.zeros(5, np.uint32))  # +0.0
    assert np.array_equal(add_f32(x, np.zeros(5, np.float32)), x)
    big = np.array([3.0e38], np.float32)
    with np.errstate(over="ignore"):
        assert np.isinf(add_f32(big, big))[0]
    # ties round to even: 1 + 2**-24 -> 1 ; (1 + 2**-23) + 2**-24 -> 1 + 2**-22
    one = np.float32(1.0)
    assert add_f32(np.array([one]), np.array([np.float32(2.0 ** -24)]))[0] == one
    a = np.array([np.float32(1.0 + 2.0 ** -23)])
    assert add_f32(a, np.array([np.float32(2.0 ** -24)]))[0] == np.float32(1.0 + 2.0 ** -22)
