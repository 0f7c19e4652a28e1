"""Pin P1, device half: every one of the 2^32 FP32 bit patterns through the GPU's binary16
conversion (mp_round_f32_to_f16, the conversion of Step 1 that the update's write also uses)
against the oracle's software encoder, bit for bit; a NaN input must give a NaN (any payload).

Source: "Mixed Precision Training", long-form analysis page, §3.4 "The Integrated Training
Procedure", Step 1 (the master weights are rounded to the nearest binary16 value) and §6.5
"Single Hardware Architecture" (other hardware may round or treat subnormals differently, which
this sweep rules out on gfx950: gradual underflow, ties to even, overflow to +-inf at 65520).
The oracle's encoder is itself pinned over all 2^32 patterns (tests/test_oracle_codec.py).
Sixteen chunks of 2^28 patterns, one test each.
"""
import numpy as np
import pytest
import torch

import mixed_precision_neural_amd as mp
import oracle
from gpu_util import host_bits16, require_gpu

pytestmark = pytest.mark.gpu

CHUNK = 1 << 28


@pytest.mark.timeout(120)
@pytest.mark.parametrize("chunk", range(16))
def test_all_fp32_patterns_round_like_the_oracle(chunk):
    require_gpu()
    lo, hi = chunk * CHUNK, (chunk + 1) * CHUNK
    print(f"codec chunk {chunk}: patterns [{lo:#010x}, {hi:#010x})", flush=True)
    bits = torch.arange(lo, hi, dtype=torch.int64, device="cuda").to(torch.int32)
    w16 = mp.round_f32_to_f16(bits.view(torch.float32))
    del bits
    got = host_bits16(w16)
    del w16
    ref = oracle.f32bits_to_f16(lo, hi)
    # inputs that are NaN: exponent all ones, mantissa non-zero
    pat = np.arange(lo, hi, dtype=np.uint64).astype(np.uint32)
    src_nan = ((pat & 0x7F800000) == 0x7F800000) & ((pat & 0x007FFFFF) != 0)
    del pat
    is_nan = lambda h: ((h & 0x7C00) == 0x7C00) & ((h & 0x3FF) != 0)
    assert is_nan(got[src_nan]).all() and is_nan(ref[src_nan]).all()
    ok = ~src_nan
    bad = np.flatnonzero(got[ok] != ref[ok])
    assert bad.size == 0, [(hex(lo + int(np.flatnonzero(ok)[i])), hex(got[ok][i]), hex(ref[ok][i])) for i in bad[:8]]
