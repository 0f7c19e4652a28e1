"""Pins of the oracle's large reductions: batch-normalization statistics, the normalization
itself and the row softmax.

Source: "Mixed Precision Training", long-form analysis page, §3.4 "FP16 Arithmetic with FP32
Accumulation" (large reductions: batch-normalization mean and variance and the softmax
normalization constant are summed in FP32 from binary16 tensors, the arithmetic is FP32 and
binary16 results are written back), and the summary list of precision rules near the page's
top (large reductions in FP32, still reading and writing FP16 tensors).

The statistics and the softmax are pinned by closed forms and by exact rational arithmetic
(Python fractions) on small inputs; the normalization by dyadic cases whose FP32 result is
exact, and by its special cases. None of them re-evaluates the oracle's own formula.
"""
import math
from fractions import Fraction as Fr

import numpy as np
import pytest

import oracle


def f16(vals) -> np.ndarray:
    a = np.asarray(vals, np.float64).astype(np.float16)
    assert np.array_equal(a.astype(np.float64), np.asarray(vals, np.float64)), "must be exact in binary16"
    return a.view(np.uint16)


def as_f64(bits) -> np.ndarray:
    return bits.view(np.float16).astype(np.float64)


# ---------------------------------------------------------------- statistics
def test_bn_stats_constant_channels():
    x = np.tile(f16([1.5, -3.0, 0.0, 65504.0]), (1000, 1))
    mean, var = oracle.bn_stats(x)
    assert list(mean) == [1.5, -3.0, 0.0, 65504.0] and list(var) == [0.0] * 4


@pytest.mark.parametrize("n,a,d", [(7, 3, 2), (1000, -500, 1), (4096, -1024, 0.5), (3, 2048, -1024)])
def test_bn_stats_arithmetic_progression(n, a, d):
    """x_r = a + r d: mean a + d (n - 1) / 2, population variance d^2 (n^2 - 1) / 12."""
    col = [a + r * d for r in range(n)]
    x = np.stack([f16(col), f16([-v for v in col])], axis=1)
    mean, var = oracle.bn_stats(x)
    m, v = a + d * (n - 1) / 2, d * d * (n * n - 1) / 12
    assert math.isclose(mean[0], m, rel_tol=1e-13, abs_tol=1e-13) and math.isclose(mean[1], -m, rel_tol=1e-13, abs_tol=1e-13)
    assert math.isclose(var[0], v, rel_tol=1e-12) and math.isclose(var[1], v, rel_tol=1e-12)


def test_bn_stats_against_exact_rationals():
    """Brute force: mean and variance of binary16 values computed exactly with fractions."""
    rng = np.random.Generator(np.random.PCG64(41))
    x = (rng.standard_normal((37, 5)) * 2.0 ** rng.integers(-6, 6, (37, 5))).astype(np.float16).view(np.uint16)
    mean, var = oracle.bn_stats(x)
    vals = as_f64(x)
    for c in range(5):
        col = [Fr(float(v)) for v in vals[:, c]]
        m = sum(col) / len(col)
        v = sum((t - m) ** 2 for t in col) / len(col)
        assert abs(Fr(mean[c]) - m) <= abs(m) * Fr(2) ** -50 + Fr(2) ** -200
        assert abs(Fr(var[c]) - v) <= v * Fr(2) ** -48


def test_bn_stats_large_offset():
    """1024 + {0, 1, 2, 3} repeated: mean 1025.5 and variance 1.25 exactly (two passes keep
    the variance exact where E[x^2] - E[x]^2 would cancel 20 bits)."""
    x = np.tile(f16([1024, 1025, 1026, 1027]), 2500).reshape(-1, 1)
    mean, var = oracle.bn_stats(x)
    assert mean[0] == 1025.5 and var[0] == 1.25


def test_bn_stats_strided_rows_ignore_padding():
    wide = np.full((6, 5), 0x7E00, np.uint16)          # NaN in the padding
    wide[:, :3] = f16(np.arange(18).reshape(6, 3))
    mean, var = oracle.bn_stats(wide[:, :3])
    assert list(mean) == [7.5, 8.5, 9.5] and all(math.isclose(v, 9 * 35 / 12) for v in var)


# ---------------------------------------------------------------- normalization
def test_bn_apply_dyadic_closed_form():
    """var + eps = 4 exactly (eps = 2^-10), so 1 / sqrt = 0.5; dyadic x, mean, gamma, beta make
    every FP32 operation exact: y = (x - mean) / 2 * gamma + beta."""
    eps = 2.0 ** -10
    x = f16([[1.5, -2.0], [3.25, 0.5], [-7.0, 12.0]])
    mean, var = [0.25, 1.0], [4.0 - eps, 4.0 - eps]
    gamma, beta = [1.5, -0.75], [0.125, 2.0]
    y = oracle.bn_apply(x, mean, var, gamma, beta, eps)
    for i in range(3):
        for c in range(2):
            e = (Fr(float(as_f64(x)[i, c])) - Fr(mean[c])) / 2 * Fr(gamma[c]) + Fr(beta[c])
            assert Fr(float(as_f64(y)[i, c])) == e


def test_bn_apply_special_cases():
    x = f16([[2.0, 5.0, 1.0]])
    # x = mean gives beta; gamma = 0 gives beta; a product beyond 65504 overflows to +inf
    y = oracle.bn_apply(x, [2.0, 0.0, 0.0], [1.0, 1.0, 0.0], [3.0, 0.0, 70000.0], [0.5, -1.25, 0.0], 0.0)
    assert list(as_f64(y)[0][:2]) == [0.5, -1.25] and as_f64(y)[0][2] == np.inf


# ---------------------------------------------------------------- softmax
@pytest.mark.parametrize("V", [1, 3, 10, 1000, 65536])
@pytest.mark.parametrize("value", [0.75, 60000.0])
def test_softmax_constant_row(V, value):
    """Every entry 1 / V; at 60000 exp overflows unless the row maximum is subtracted first."""
    y = oracle.softmax(np.full((2, V), f16([value])[0], np.uint16))
    expect = np.float16(np.float32(1.0 / V)).view(np.uint16)
    assert (y == expect).all()


@pytest.mark.parametrize("V,k,t", [(2, 1, 1.0), (10, 3, 2.5), (1000, 1, -4.0), (793471, 17, 6.0)])
def test_softmax_two_valued_row(V, k, t):
    """k entries t, V - k entries 0: p_t = e^t / (k e^t + V - k), p_0 = 1 / (k e^t + V - k)."""
    row = np.zeros(V, np.uint16); row[:k] = f16([t])[0]
    y = oracle.softmax(row.reshape(1, -1))[0]
    den = k * math.exp(t) + (V - k)
    assert (y[:k] == np.float16(np.float32(math.exp(t) / den)).view(np.uint16)).all()
    assert (y[k:] == np.float16(np.float32(1.0 / den)).view(np.uint16)).all()


def test_softmax_shift_invariance_and_sum():
    rng = np.random.Generator(np.random.PCG64(5))
    x = rng.integers(-8, 9, (4, 300)).astype(np.float64)
    a, b = oracle.softmax(f16(x)), oracle.softmax(f16(x + 8))
    assert np.array_equal(a, b)
    s = as_f64(a).sum(axis=1)
    assert np.all(np.abs(s - 1.0) <= 300 * 2.0 ** -11)


def test_softmax_infinities_and_nan():
    ninf, pinf, nan = 0xFC00, 0x7C00, 0x7E00
    x = np.array([[ninf, 0, 0, ninf], [0, pinf, 0, 0], [nan, 0, 0, 0], [ninf] * 4], np.uint16)
    y = as_f64(oracle.softmax(x))
    assert list(y[0]) == [0.0, 0.5, 0.5, 0.0]
    assert np.isnan(y[1]).all() and np.isnan(y[2]).all() and np.isnan(y[3]).all()


def test_softmax_strided_rows():
    wide = np.full((3, 9), 0x7E00, np.uint16)
    wide[:, :4] = f16([[0, 0, 0, 0], [1, 1, 1, 1], [-2, -2, -2, -2]])
    y = as_f64(oracle.softmax(wide[:, :4]))
    assert (y == 0.25).all()
