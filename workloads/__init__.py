"""Seeded synthetic inputs shared by the oracle tests, the GPU tests and the benchmark.

This module holds input recipes only: random draws (numpy PCG64), shapes,
injection positions and hyper-parameters. It contains none of the method's
arithmetic; the one conversion it performs, turning a synthetic FP32 gradient
into the binary16 tensor a backward pass would have stored, is numpy's own
``float16`` cast, a library routine that belongs to neither side under test.

The recipes stand in for the workloads of "Mixed Precision Training" (the
long-form analysis page, paper-graph-ui.vercel.app): the gradient range
[2^-34, 2^-4] follows the SSD activation-gradient histogram of its §3.4
"Loss Scaling" (original Figure 3), and the 5 % of magnitudes below 2^-24
follows the Mandarin speech weight-gradient histogram of §3.4 "FP32 Master
Copy of Weights" (original Figure 2b).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

F16_INF = np.uint16(0x7C00)
F16_QNAN = np.uint16(0x7E00)


def rng(seed: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def to_f16_bits(x: np.ndarray) -> np.ndarray:
    """numpy's float32 -> float16 cast, returned as uint16 bit patterns."""
    with np.errstate(over="ignore"):
        return np.asarray(x, np.float32).astype(np.float16).view(np.uint16)


def normal_f32(g: np.random.Generator, shape, std: float) -> np.ndarray:
    return (g.standard_normal(shape, dtype=np.float32) * np.float32(std)).astype(np.float32)


# --------------------------------------------------------------------- C1
@dataclass
class C1:
    """2-layer MLP 256 -> 512 -> 10, ReLU, softmax cross-entropy, batch 64."""
    W1: np.ndarray          # [512, 256] FP32 master
    W2: np.ndarray          # [10, 512]  FP32 master
    X16: np.ndarray         # [64, 256]  binary16 input
    labels: np.ndarray      # [64] int32 in [0, 10)
    lr: float = 0.01
    momentum: float = 0.9
    weight_decay: float = 0.0
    scale: float = 1024.0
    dynamic: bool = False
    growth_interval: int = 2000
    steps: int = 10


def c1(seed: int = 0) -> C1:
    g = rng(seed)
    W1 = normal_f32(g, (512, 256), 0.05)
    W2 = normal_f32(g, (10, 512), 0.05)
    X = g.standard_normal((64, 256), dtype=np.float32)
    labels = g.integers(0, 10, 64).astype(np.int32)
    return C1(W1, W2, to_f16_bits(X), labels)


# --------------------------------------------------------------------- C2
@dataclass
class C2:
    """Update-only sweep over one flat tensor."""
    w32: np.ndarray
    g_true: np.ndarray      # FP32 synthetic gradient, sign * 2^u, u ~ U(-34, -4)
    inf_step: int
    inf_index: int
    lr: float = 0.01
    momentum: float = 0.9
    weight_decay: float = 0.0
    scale: float = 2.0 ** 15
    dynamic: bool = True
    growth_interval: int = 2000
    steps: int = 50


def c2(n: int = 100_000_000, seed: int = 0, steps: int = 50, inf_step: int = 25) -> C2:
    g = rng(seed)
    w32 = normal_f32(g, n, 0.02)
    u = g.uniform(-34.0, -4.0, n)
    sign = np.where(g.integers(0, 2, n) == 1, 1.0, -1.0)
    g_true = (sign * np.exp2(u)).astype(np.float32)
    inf_index = int(g.integers(0, n))
    return C2(w32, g_true, inf_step, inf_index, steps=steps)


def grads_at_scale(g_true: np.ndarray, scale: float) -> np.ndarray:
    """The binary16 gradient a backward pass at loss scale ``scale`` would store."""
    return to_f16_bits(np.asarray(g_true, np.float32) * np.float32(scale))


# --------------------------------------------------------------------- C3
@dataclass
class C3:
    X16: np.ndarray         # [M, K]
    dY16: np.ndarray        # [M, N]
    W16: np.ndarray         # [N, K]


def c3(M: int = 8192, N: int = 4096, K: int = 4096, seed: int = 0) -> C3:
    g = rng(seed)
    X = g.standard_normal((M, K), dtype=np.float32)
    dY = g.standard_normal((M, N), dtype=np.float32)
    W = normal_f32(g, (N, K), 1.0 / math.sqrt(K))
    return C3(to_f16_bits(X), to_f16_bits(dY), to_f16_bits(W))


# --------------------------------------------------------------------- C4
@dataclass
class C4:
    """12-layer GELU MLP, width 4096, batch 4096, MSE loss to N(0,1) targets."""
    masters: list            # L x [width, width] FP32
    X16: np.ndarray          # [batch, width]
    T16: np.ndarray          # [batch, width]
    lr: float = 0.01
    momentum: float = 0.9
    weight_decay: float = 0.0
    scale: float = 2.0 ** 16
    dynamic: bool = True
    growth_interval: int = 2000
    steps: int = 20


def c4(width: int = 4096, batch: int = 4096, layers: int = 12, seed: int = 0,
       with_masters: bool = True) -> C4:
    g = rng(seed)
    masters = []
    for _ in range(layers):
        W = normal_f32(g, (width, width), 1.0 / math.sqrt(width))
        masters.append(W if with_masters else None)
    X = g.standard_normal((batch, width), dtype=np.float32)
    T = g.standard_normal((batch, width), dtype=np.float32)
    return C4(masters, to_f16_bits(X), to_f16_bits(T))


# --------------------------------------------------------------------- C5
C5_TOTAL = 1_500_000_000
C5_TENSORS = 500
C5_LOG2_MEDIAN = -20.0
C5_LOG2_SIGMA = 4.0 / 1.645     # 5 % of unscaled magnitudes below 2^-24


def c5_sizes(seed: int = 0, total: int = C5_TOTAL, count: int = C5_TENSORS,
             lo: float = 1e3, hi: float = 5e7) -> np.ndarray:
    """Log-uniform sizes in [lo, hi], rescaled until they sum to total +- 0.1 %."""
    g = rng(seed)
    while True:
        s = np.exp(g.uniform(math.log(lo), math.log(hi), count))
        s = np.clip(np.rint(s * (total / s.sum())), 1, None).astype(np.int64)
        if abs(int(s.sum()) - total) <= total // 1000:
            return s


@dataclass
class C5Tensor:
    w32: np.ndarray
    g_true: np.ndarray


def c5_tensor(t: int, size: int, seed: int = 0) -> C5Tensor:
    """Tensor t of C5, drawn from its own child stream so tensors can be made alone."""
    child = np.random.SeedSequence(seed).spawn(t + 1)[t]
    g = np.random.Generator(np.random.PCG64(child))
    w32 = normal_f32(g, int(size), 0.02)
    e = g.standard_normal(int(size)) * C5_LOG2_SIGMA + C5_LOG2_MEDIAN
    sign = np.where(g.integers(0, 2, int(size)) == 1, 1.0, -1.0)
    return C5Tensor(w32, (sign * np.exp2(e)).astype(np.float32))


def c5_nan_indices(total: int, frac: float = 1e-3, seed: int = 0) -> np.ndarray:
    """Sorted global indices (over the concatenated tensors) that receive NaN."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed).spawn(C5_TENSORS + 1)[-1]))
    k = int(round(total * frac))
    return np.sort(g.choice(total, size=k, replace=False))


@dataclass
class C5Hyper:
    lr: float = 1e-3
    momentum: float = 0.9
    weight_decay: float = 1e-4
    scale: float = 2.0 ** 12
    dynamic: bool = True
    growth_interval: int = 2000
    steps: int = 20
    nan_step: int = 7


# --------------------------------------------------------------------- ragged lists
def ragged_sizes(count: int, lo: int, hi: int, seed: int = 0) -> np.ndarray:
    """Log-uniform integer sizes in [lo, hi] for small ragged multi-tensor tests."""
    g = rng(seed)
    return np.exp(g.uniform(math.log(lo), math.log(hi), count)).astype(np.int64)
