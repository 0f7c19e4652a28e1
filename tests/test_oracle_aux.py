"""Pins of the oracle's point-wise ops and losses (used by the 2-layer and 12-layer MLP steps).

Source: "Mixed Precision Training", long-form analysis page, §3.4 "FP16
Arithmetic with FP32 Accumulation" (point-wise ops, large reductions) and
"The Integrated Training Procedure" (Step 3, loss scaling).
"""
import math

import numpy as np
import scipy.special
import scipy.stats


def h(x):
    return np.asarray(x, np.float32).astype(np.float16).view(np.uint16)


def v(b):
    return np.asarray(b, np.uint16).view(np.float16).astype(np.float64)


def test_relu(orc):
    x = h([-2.0, -0.0, 0.0, 1e-7, 3.0, -65504, 65504])
    y = orc.relu_fwd(x)
    assert list(v(y)) == [0.0, 0.0, 0.0, float(np.float16(1e-7)), 3.0, 0.0, 65504.0]
    dy = h([5.0] * 7)
    assert list(v(orc.relu_bwd(x, dy))) == [0, 0, 0, 5, 5, 0, 5]


def test_gelu_against_normal_cdf(orc):
    """GELU(x) = x * Phi(x) with Phi the standard normal CDF (scipy's)."""
    xs = np.linspace(-8, 8, 20001).astype(np.float16)
    xb = xs.view(np.uint16)
    got = v(orc.gelu_fwd(xb))
    x64 = xs.astype(np.float64)
    ref = x64 * scipy.stats.norm.cdf(x64)
    ulp = np.maximum(np.abs(ref), 2.0 ** -14) * 2.0 ** -10
    assert (np.abs(got - ref) <= ulp).all()


def test_gelu_backward_matches_finite_differences(orc):
    xs = np.linspace(-6, 6, 4001)
    xb = h(xs)
    x64 = v(xb)
    eps = 1e-6
    fd = ((x64 + eps) * scipy.stats.norm.cdf(x64 + eps) - (x64 - eps) * scipy.stats.norm.cdf(x64 - eps)) / (2 * eps)
    got = v(orc.gelu_bwd(xb, h(np.ones_like(xs))))
    assert np.abs(got - fd).max() <= 2.0 ** -9 * max(1.0, np.abs(fd).max())


def test_softmax_ce_against_scipy(orc):
    rng = np.random.Generator(np.random.PCG64(0))
    B, Cn = 64, 10
    z = h(rng.standard_normal((B, Cn)) * 3)
    y = rng.integers(0, Cn, B).astype(np.int32)
    S = 1024.0
    loss, d = orc.softmax_ce(z, y, S)
    z64 = v(z).reshape(B, Cn)
    ls = scipy.special.log_softmax(z64, axis=1)
    assert math.isclose(loss, -ls[np.arange(B), y].mean(), rel_tol=1e-12)
    onehot = np.eye(Cn)[y]
    ref = S * (np.exp(ls) - onehot) / B
    got = v(d).reshape(B, Cn)
    assert (np.abs(got - ref) <= np.maximum(np.abs(ref), 2.0 ** -14) * 2.0 ** -10).all()


def test_softmax_ce_uniform_logits(orc):
    B, Cn = 4, 10
    z = np.zeros((B, Cn), np.uint16)
    loss, d = orc.softmax_ce(z, np.arange(B, dtype=np.int32), 1.0)
    assert math.isclose(loss, math.log(Cn), rel_tol=1e-15)
    g = v(d).reshape(B, Cn)
    # (1/10 - [c == y]) / 4
    assert np.allclose(g, (0.1 - np.eye(Cn)[:B]) / B, rtol=2 ** -10, atol=0)


def test_mse_closed_form(orc):
    y = h(np.full((4, 8), 3.0))
    t = h(np.full((4, 8), 1.0))
    loss, d = orc.mse(y, t, 0.5, 8.0)
    assert loss == 0.5 * 4.0
    # dL/dy = c * 2 (y - t) / (M N) = 0.5 * 4 / 32 = 1/16; times S = 8 -> 0.5
    assert (v(d) == 0.5).all()


def test_mse_grad_finite_difference(orc):
    rng = np.random.Generator(np.random.PCG64(1))
    y = h(rng.standard_normal((8, 16)))
    t = h(rng.standard_normal((8, 16)))
    c = 1.7
    g = orc.mse_grad_f64(y, t, 8, c)
    y64, t64 = v(y).reshape(8, 16), v(t).reshape(8, 16)
    eps = 1e-6
    L = lambda Y: c * ((Y - t64) ** 2).mean()
    E = np.zeros_like(y64); E[3, 5] = eps
    fd = (L(y64 + E) - L(y64 - E)) / (2 * eps)
    assert math.isclose(g[3, 5], fd, rel_tol=1e-6)
