"""Pins of the oracle's three dot-product layers (forward, dgrad, wgrad).

Source: "Mixed Precision Training", long-form analysis page, §3.4 "FP16
Arithmetic with FP32 Accumulation" and "The Integrated Training Procedure"
(Steps 2 and 4).
"""
import numpy as np
import pytest


def exact_grid(rng, shape, scale_log2=-8, lim=2.0):
    """binary16 values that are multiples of 2^scale_log2 with |x| <= lim, and their integers."""
    q = 2.0 ** scale_log2
    ints = rng.integers(-int(lim / q), int(lim / q) + 1, shape)
    vals = (ints * q).astype(np.float32)
    bits = vals.astype(np.float16).view(np.uint16)
    assert np.array_equal(bits.view(np.float16).astype(np.float64), ints * q)
    return bits, ints.astype(np.int64)


@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (3, 5, 7), (17, 9, 32), (64, 10, 32)])
def test_exact_integer_sums(orc, M, N, K):
    """Pin P8: inputs on a 2^-8 grid with |x| <= 2 and K <= 32 keep every partial sum exact in
    FP32, so each layer equals the integer result for any summation order."""
    rng = np.random.Generator(np.random.PCG64(M * 1000 + N * 10 + K))
    X, Xi = exact_grid(rng, (M, K))
    W, Wi = exact_grid(rng, (N, K))
    dY, dYi = exact_grid(rng, (M, N))
    q2 = 2.0 ** -16
    assert np.array_equal(orc.linear_fwd(X, W).astype(np.float64), (Xi @ Wi.T) * q2)
    assert np.array_equal(orc.linear_dgrad(dY, W).astype(np.float64), (dYi @ Wi) * q2)
    assert np.array_equal(orc.linear_wgrad(dY, X).astype(np.float64), (dYi.T @ Xi) * q2)


def test_exact_subnormal_inputs(orc):
    """Pin P8, subnormal variant: operands m * 2^-24 (binary16 subnormals) times small integers."""
    rng = np.random.Generator(np.random.PCG64(11))
    M, N, K = 8, 6, 16
    Xi = rng.integers(-1023, 1024, (M, K))
    X = (np.abs(Xi) | np.where(Xi < 0, 0x8000, 0)).astype(np.uint16)   # sign | mantissa, exponent 0
    Wi = rng.integers(-4, 5, (N, K))
    W = Wi.astype(np.float16).view(np.uint16)
    ref = (Xi @ Wi.T).astype(np.float64) * 2.0 ** -24
    got = orc.linear_fwd(X.astype(np.uint16), W).astype(np.float64)
    assert np.array_equal(got, ref)


def test_fp32_accumulation_of_4096_ones(orc):
    """Pin P9: X = W = 1 with K = 4096 gives exactly 4096; a binary16 running sum stalls at 2048."""
    K = 4096
    X = np.full((2, K), 0x3C00, np.uint16)
    W = np.full((3, K), 0x3C00, np.uint16)
    assert (orc.linear_fwd(X, W) == 4096.0).all()
    acc = np.zeros(1, np.float32)
    one = np.float32(1.0)
    for _ in range(K):
        acc = orc.f16_to_f32(orc.f32_to_f16((acc + one).astype(np.float32)))
    assert float(acc[0]) == 2048.0


@pytest.mark.parametrize("M,N,K", [(33, 47, 300), (64, 128, 1000)])
def test_fp64_error_bound(orc, M, N, K):
    """Random N(0,1) binary16 inputs: |oracle - exact| <= gamma_K * sum|a||b| with the FP32 unit
    roundoff u = 2^-24 (products are exact)."""
    rng = np.random.Generator(np.random.PCG64(K))
    X = rng.standard_normal((M, K)).astype(np.float16)
    W = rng.standard_normal((N, K)).astype(np.float16)
    dY = rng.standard_normal((M, N)).astype(np.float16)
    u = 2.0 ** -24
    for got, a, b in [
        (orc.linear_fwd(X.view(np.uint16), W.view(np.uint16)), X.astype(np.float64), W.astype(np.float64).T),
        (orc.linear_dgrad(dY.view(np.uint16), W.view(np.uint16)), dY.astype(np.float64), W.astype(np.float64)),
        (orc.linear_wgrad(dY.view(np.uint16), X.view(np.uint16)), dY.astype(np.float64).T, X.astype(np.float64)),
    ]:
        exact = a @ b
        red = a.shape[1]
        gamma = red * u / (1 - red * u)
        bound = gamma * (np.abs(a) @ np.abs(b))
        assert (np.abs(got.astype(np.float64) - exact) <= bound).all()


def test_sampled_points_equal_full_result(orc):
    rng = np.random.Generator(np.random.PCG64(2))
    M, N, K = 40, 24, 72
    X = rng.standard_normal((M, K)).astype(np.float16).view(np.uint16)
    W = rng.standard_normal((N, K)).astype(np.float16).view(np.uint16)
    dY = rng.standard_normal((M, N)).astype(np.float16).view(np.uint16)
    full = [orc.linear_fwd(X, W), orc.linear_dgrad(dY, W), orc.linear_wgrad(dY, X)]
    at = [orc.linear_fwd_at, orc.linear_dgrad_at, orc.linear_wgrad_at]
    args = [(X, W), (dY, W), (dY, X)]
    for F, fn, (a, b) in zip(full, at, args):
        r = rng.integers(0, F.shape[0], 50)
        c = rng.integers(0, F.shape[1], 50)
        assert np.array_equal(fn(a, b, r, c), F[r, c])


def test_f16_output_is_rounded_f32_result(orc):
    rng = np.random.Generator(np.random.PCG64(4))
    X = rng.standard_normal((16, 64)).astype(np.float16).view(np.uint16)
    W = (rng.standard_normal((8, 64)) * 8000).astype(np.float16).view(np.uint16)
    f32 = orc.linear_fwd(X, W)
    f16 = orc.linear_fwd(X, W, out_f16=True)
    assert np.array_equal(f16, orc.f32_to_f16(f32))
    assert ((f16 & 0x7C00) == 0x7C00).any()      # some outputs overflow to inf, none saturate
