"""Pins of the oracle's optimizer variants and of loss-scale method 2.

Sources: "Mixed Precision Training", long-form analysis page, §3.1 "Empirical validation
(Figure 2a)" and §4.3 (Nesterov-momentum SGD), §4.5 (Figure 5) and §6.4 (Adagrad); §3.4
"Choosing the scaling factor — the direct statistical approach" (S = 65504 / max|g|, and
65504 / (2 max|g|) with one bit of headroom).

The pages print no Nesterov or Adagrad update rule; the oracle takes the textbook forms.
These pins fix them by closed forms computed here with exact rational arithmetic (every
value is a short dyadic fraction, so FP32 holds each intermediate exactly), by special
cases that reduce to plain SGD or to a sign step, and by fp64 bounds where a square root
enters. None of them re-evaluates the oracle's own formula in FP32.
"""
import math
from fractions import Fraction as Fr

import numpy as np
import pytest

import oracle

F16_ONE = 0x3C00


def f16_bits(x: float) -> int:
    return int(np.array([x], np.float16).view(np.uint16)[0])


def run(kind, w0, v0, g_true, steps, lr, mu=0.0, wd=0.0, eps=0.0, scale=1024.0):
    """`steps` updates of one element with the constant unscaled gradient g_true."""
    w = np.array([w0], np.float32); v = np.array([v0], np.float32)
    h = np.zeros(1, np.uint16)
    g16 = np.array([f16_bits(g_true * scale)], np.uint16)
    assert float(g16.view(np.float16)[0]) == g_true * scale, "test gradient must be exact in binary16"
    ws, vs = [], []
    for _ in range(steps):
        f = oracle.step_opt(kind, [w], [v], [g16], [h], lr, mu, wd, eps, 1.0 / scale)
        assert f == 0
        ws.append(float(w[0])); vs.append(float(v[0]))
    return ws, vs, h


def test_nesterov_closed_form_exact():
    """v_t = mu v_{t-1} + g; w_t = w_{t-1} - lr (g + mu v_t), all dyadic and exact."""
    g, lr, mu = Fr(1, 16), Fr(1, 8), Fr(1, 2)
    ws, vs, _ = run(oracle.NESTEROV, 1.0, 0.0, float(g), 6, float(lr), float(mu))
    w, v = Fr(1), Fr(0)
    for t in range(6):
        v = mu * v + g
        w = w - lr * (g + mu * v)
        assert Fr(vs[t]) == v and Fr(ws[t]) == w, t
    # a look-ahead on the previous velocity would give w_1 = 1 - lr g = 0.9921875 instead
    assert ws[0] == float(1 - lr * (g + mu * g)) == 0.98828125


def test_nesterov_without_momentum_is_plain_sgd():
    g, lr = 2.0 ** -6, 2.0 ** -4
    ws, _, h = run(oracle.NESTEROV, 0.5, 0.0, g, 4, lr, mu=0.0)
    assert ws == [0.5 - (t + 1) * lr * g for t in range(4)]
    assert h[0] == f16_bits(ws[-1])


def test_nesterov_weight_decay_enters_the_velocity():
    """g_eff = g + wd w with the FP32 master, before the momentum (exact dyadic case)."""
    g, lr, mu, wd = Fr(1, 16), Fr(1, 4), Fr(1, 2), Fr(1, 4)
    ws, vs, _ = run(oracle.NESTEROV, 1.0, 0.0, float(g), 3, float(lr), float(mu), float(wd))
    w, v = Fr(1), Fr(0)
    for t in range(3):
        ge = g + wd * w
        v = mu * v + ge
        w = w - lr * (ge + mu * v)
        assert Fr(vs[t]) == v and Fr(ws[t]) == w, t


def test_adagrad_first_step_is_a_sign_step():
    """From G = 0: G_1 = g^2 and g / sqrt(g^2) = sign(g) exactly (eps far below |g|)."""
    for g in (2.0 ** -4, -2.0 ** -9, 2.0 ** -14, -1.0):
        ws, vs, _ = run(oracle.ADAGRAD, 1.0, 0.0, g, 1, 2.0 ** -5, eps=2.0 ** -100)
        assert vs[0] == g * g
        assert ws[0] == 1.0 - math.copysign(2.0 ** -5, g)


def test_adagrad_constant_gradient_against_fp64():
    """G_t = t g^2 exactly; w_t = w_0 - lr sign(g) sum_{k<=t} 1/sqrt(k), within the FP32
    rounding of t steps (each step: sqrt, divide, multiply, subtract -> <= 4 ulps of ~lr,
    plus the subtraction's rounding of w ~ 2^-24)."""
    g, lr, T = 2.0 ** -4, 2.0 ** -6, 40
    ws, vs, _ = run(oracle.ADAGRAD, 1.0, 0.0, g, T, lr, eps=2.0 ** -100)
    acc = 0.0
    for t in range(1, T + 1):
        assert vs[t - 1] == t * g * g                      # exact accumulation
        acc += 1.0 / math.sqrt(t)
        assert abs(ws[t - 1] - (1.0 - lr * acc)) <= t * (4 * lr + 1.0) * 2.0 ** -24


def test_adagrad_eps_and_weight_decay():
    """Weight decay enters the accumulated square (exact: g_eff = 5/16, sqrt = 5/16); a large
    eps damps the step to lr g / (|g| + eps) (fp64 within one FP32 rounding per operation)."""
    ws, vs, _ = run(oracle.ADAGRAD, 1.0, 0.0, 2.0 ** -4, 1, 2.0 ** -3, wd=0.25, eps=2.0 ** -100)
    assert vs[0] == (5 / 16) ** 2 and ws[0] == 1.0 - 2.0 ** -3
    g, lr, eps = 0.375, 0.125, 1.0
    ws, _, _ = run(oracle.ADAGRAD, 2.0, 0.0, g, 1, lr, eps=eps, scale=8.0)
    assert abs(ws[0] - (2.0 - lr * g / (g + eps))) <= 4 * 2.0 ** -23


def test_adagrad_accumulator_never_decreases():
    rng = np.random.Generator(np.random.PCG64(5))
    n = 4096
    w = rng.standard_normal(n).astype(np.float32); G = np.zeros(n, np.float32)
    h = np.zeros(n, np.uint16)
    prev = G.copy()
    for _ in range(8):
        g16 = (rng.standard_normal(n) * 64).astype(np.float16).view(np.uint16)
        assert oracle.step_opt(oracle.ADAGRAD, [w], [G], [g16], [h], 0.01, 0.0, 1e-4, 1e-10, 2.0 ** -10) == 0
        assert np.all(G >= prev) and np.all(np.isfinite(w))
        prev = G.copy()


@pytest.mark.parametrize("kind", [oracle.NESTEROV, oracle.ADAGRAD])
def test_overflow_skips_every_kind(kind):
    """Step 6: one inf/NaN anywhere -> flag 1 and no element of any tensor changes."""
    rng = np.random.Generator(np.random.PCG64(kind))
    sizes = (7, 1000, 33)
    w = [rng.standard_normal(s).astype(np.float32) for s in sizes]
    v = [np.abs(rng.standard_normal(s)).astype(np.float32) for s in sizes]
    g = [rng.standard_normal(s).astype(np.float16).view(np.uint16) for s in sizes]
    h = [np.full(s, 0x1234, np.uint16) for s in sizes]
    g[1][999] = 0x7E00
    before = [a.copy() for a in w + v + h]
    assert oracle.step_opt(kind, w, v, g, h, 0.1, 0.9, 0.01, 1e-8, 0.5) == 1
    for a, b in zip(w + v + h, before):
        assert np.array_equal(a, b)


def test_sgd_kind_matches_the_original_sweep():
    """OR_OPT_SGD through the new entry point gives the bits of or_step (same rule)."""
    rng = np.random.Generator(np.random.PCG64(9))
    n = 5000
    base_w = rng.standard_normal(n).astype(np.float32)
    base_v = rng.standard_normal(n).astype(np.float32)
    g = (rng.standard_normal(n) * 100).astype(np.float16).view(np.uint16)
    w1, v1, h1 = base_w.copy(), base_v.copy(), np.zeros(n, np.uint16)
    w2, v2, h2 = base_w.copy(), base_v.copy(), np.zeros(n, np.uint16)
    oracle.step([w1], [v1], [g], [h1], 0.01, 0.9, 1e-4, 2.0 ** -8)
    oracle.step_opt(oracle.SGD, [w2], [v2], [g], [h2], 0.01, 0.9, 1e-4, 0.0, 2.0 ** -8)
    assert np.array_equal(w1.view(np.uint32), w2.view(np.uint32))
    assert np.array_equal(v1.view(np.uint32), v2.view(np.uint32)) and np.array_equal(h1, h2)


# ---------------------------------------------------------------- method 2
def test_absmax_matches_numpy_over_finite_elements():
    rng = np.random.Generator(np.random.PCG64(3))
    a = (rng.standard_normal(10000) * 2.0 ** rng.integers(-30, 10, 10000)).astype(np.float32)
    a[[5, 77]] = [np.inf, np.nan]
    a[100] = -0.0
    a[200] = np.float32(-1e-42)                               # subnormal
    b = rng.standard_normal(300).astype(np.float16).view(np.uint16)
    b[3] = 0xFC00                                             # -inf
    m, bad = oracle.absmax([a, b])
    fa = a[np.isfinite(a)]
    fb = b.view(np.float16).astype(np.float32)
    fb = fb[np.isfinite(fb)]
    assert m == max(np.max(np.abs(fa)), np.max(np.abs(fb))) and bad == 1
    m2, bad2 = oracle.absmax([fa])
    assert m2 == np.max(np.abs(fa)) and bad2 == 0
    assert oracle.absmax([], running=3.5) == (3.5, 0)
    assert oracle.absmax([np.zeros(4, np.float32)], running=0.25)[0] == 0.25


@pytest.mark.parametrize("amax,expect", [(1.0, 2.0 ** 14), (2.0 ** -10, 2.0 ** 24), (0.0, 2.0 ** 64),
                                         (32752.0, 1.0), (32753.0, 1.0), (1e30, 1.0),
                                         (2.0 ** -80, 2.0 ** 64), (16376.0, 2.0), (16376.5, 1.0)])
def test_scale_from_absmax_closed_forms(amax, expect):
    """S = largest power of two with S * 2 * amax <= 65504 (page: 65504 / (2 g_max)), in [1, 2^64]:
    amax = 1 -> 65504 / 2 = 32752 -> 2^14; 2^-10 -> 33,538,048 -> 2^24; 16376 -> 2 exactly fits."""
    assert oracle.scale_from_absmax(amax, 2.0) == expect


def test_scale_from_absmax_is_the_largest_fitting_power_of_two():
    """Maximality against the page's unrounded factor S* = 65504 / (h amax): S <= S* < 2 S,
    checked in fp64 over amax spread across 60 binades, for h = 1 and h = 2."""
    rng = np.random.Generator(np.random.PCG64(11))
    for amax in (2.0 ** rng.uniform(-45, 14, 2000)).astype(np.float32):
        for h in (1.0, 2.0):
            S = oracle.scale_from_absmax(float(amax), h)
            exact = 65504.0 / (h * float(amax))
            assert math.log2(S) == int(math.log2(S))
            if 1.0 < S < 2.0 ** 64:
                assert S <= exact < 2 * S
            elif S == 1.0:
                assert exact < 2.0
            else:
                assert exact >= 2.0 ** 64
