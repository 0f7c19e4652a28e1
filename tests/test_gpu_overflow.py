"""The overflow flag of the weight-gradient epilogue on the 256 x 256 kernels the training step runs.

Source: "Mixed Precision Training", long-form analysis page, §3.4 "The Integrated Training
Procedure", Step 6 (weight gradients are checked for inf/NaN and the update is skipped when any
is found) and §3.4 "Choosing the Loss Scaling Factor", method 3 (on overflow skip the step and
halve S). mp_linear_wgrad(found_inf=...) ORs 1 into the flag when any stored binary16 output is
+-inf or NaN; the training step's sweep relies on that flag alone (MP_GRADS_PRECHECKED).

Each case poisons one element of dY (or X) with +inf, -inf or NaN, or with 65504, whose
products with the partner's elements of magnitude >= ~1 overflow binary16, on shapes whose
tiles take each reduction path of the 256 x 256 kernel:
  - 4096 x 4096 outputs, reduction 4096: whole tiles, the direct-to-LDS loop (the C4 layer);
  - 4352 x 2176 outputs, reduction 4096: whole tiles on the direct-to-LDS loop plus edge tiles on
    the general loop;
  - 4352 x 2176 outputs, reduction 4100: every tile on the general loop (ragged reduction);
  - 4096 x 4096 outputs, reduction 8192 (the C3 layer).
Checks: the flag is 1; every output outside the poisoned row (or column) has the bits of the
clean twin; the poisoned row agrees with the oracle's value class there (sampled: +inf, -inf,
NaN or finite, per element); the clean twin leaves the flag 0.
"""
import numpy as np
import pytest
import torch

import mixed_precision_neural_amd as mp
import oracle
from gpu_util import dev_f16, host_bits16, require_gpu

pytestmark = pytest.mark.gpu

POS_INF, NEG_INF, QNAN = 0x7C00, 0xFC00, 0x7E00


def value_class(h: np.ndarray) -> np.ndarray:
    """0 finite, 1 +inf, 2 -inf, 3 NaN, of binary16 bit patterns."""
    h = np.asarray(h, np.uint16)
    exp_all = (h & 0x7C00) == 0x7C00
    nan = exp_all & ((h & 0x3FF) != 0)
    inf = exp_all & ~nan
    return np.where(nan, 3, np.where(inf & (h >> 15 == 0), 1, np.where(inf, 2, 0)))


def f32_class(x: np.ndarray) -> np.ndarray:
    """The class of RNE16(x) for FP32 sums x: binary16 overflows where |x| >= 65520."""
    x = np.asarray(x, np.float64)
    big = np.abs(x) >= 65520.0
    return np.where(np.isnan(x), 3, np.where(big & (x > 0), 1, np.where(big, 2, 0)))


CASES = [
    # reduction M, outputs N x K, poisoned operand, value
    (4096, 4096, 4096, "dY", POS_INF),
    (4096, 4096, 4096, "dY", QNAN),
    (4096, 4096, 4096, "X", NEG_INF),
    (4096, 4096, 4096, "dY", "overflow"),
    (4096, 4352, 2176, "dY", NEG_INF),
    (4096, 4352, 2176, "X", "overflow"),
    (4100, 4352, 2176, "dY", POS_INF),
    (4100, 4352, 2176, "X", QNAN),
    (8192, 4096, 4096, "dY", POS_INF),
    (8192, 4096, 4096, "X", "overflow"),
]


@pytest.mark.timeout(300)
@pytest.mark.parametrize("M,N,K,where,value", CASES)
def test_wgrad_flag_on_large_tiles(M, N, K, where, value):
    require_gpu()
    rng = np.random.Generator(np.random.PCG64(M * 7 + N * 3 + K))
    dY = rng.standard_normal((M, N)).astype(np.float16).view(np.uint16)
    X = rng.standard_normal((M, K)).astype(np.float16).view(np.uint16)
    # the poisoned element: a row m0 of the reduction and an output row n0 (dY) or column k0 (X)
    m0 = int(rng.integers(0, M))
    n0, k0 = int(rng.integers(0, N)), int(rng.integers(0, K))
    print(f"wgrad flag: M={M} N={N} K={K} poison {where}[{m0}] value {value}", flush=True)
    dYp, Xp = dY.copy(), X.copy()
    if value == "overflow":
        # a finite input whose products overflow binary16: 65504 times the partner row's
        # elements of magnitude >= ~1 gives sums >= 65520, which round to +-inf
        value = 0x7BFF
    if where == "dY":
        dYp[m0, n0] = value
    else:
        Xp[m0, k0] = value
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    clean = mp.linear_wgrad(dev_f16(dY), dev_f16(X), found_inf=flag)
    torch.cuda.synchronize()
    assert int(flag.item()) == 0, "a clean wgrad set the flag"
    dirty = mp.linear_wgrad(dev_f16(dYp), dev_f16(Xp), found_inf=flag)
    torch.cuda.synchronize()
    assert int(flag.item()) == 1, "the flag was not set"
    c, d = host_bits16(clean), host_bits16(dirty)
    # outputs that do not involve the poisoned element keep the clean bits
    keep = np.ones_like(c, dtype=bool)
    if where == "dY":
        keep[n0, :] = False
    else:
        keep[:, k0] = False
    assert np.array_equal(c[keep], d[keep]), "outputs away from the poisoned element changed"
    # the poisoned row / column against the oracle's value class at every element of it
    if where == "dY":
        rows, cols = np.full(K, n0), np.arange(K)
        got = d[n0, :]
    else:
        rows, cols = np.arange(N), np.full(N, k0)
        got = d[:, k0]
    ref = oracle.linear_wgrad_at(dYp, Xp, rows, cols)
    assert np.array_equal(value_class(got), f32_class(ref))
    assert (value_class(got) != 0).mean() > (0.2 if value == 0x7BFF else 0.99)
