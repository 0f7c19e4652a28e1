"""Pins of the oracle's binary16 codec against numpy and the numbers the pages print.

Sources: "Mixed Precision Training", long-form analysis page, §2 and §3.4
("FP32 Master Copy of Weights", "Loss Scaling", "Choosing the Loss Scaling
Factor"); golden values in tests/golden/pages_constants.json.
"""
import json
import os

import numpy as np
import pytest

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_constants.json")))


def f16(x):
    return np.asarray(x, np.float16).view(np.uint16)


def test_decode_all_patterns_match_numpy(orc):
    h = np.arange(1 << 16, dtype=np.uint16)
    ours = orc.f16_to_f32(h)
    ref = h.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_encode_all_2p32_patterns_match_numpy(orc):
    """Pin P1: every float32 bit pattern. Where 2^-25 < |x| < 65520 the result must equal
    numpy's float16 cast (an RNE library routine). Outside that band the IEEE definition gives
    the answer in closed form (numpy's cast is very slow there): |x| <= 2^-25 rounds to a zero of
    the same sign, |x| >= 65520 to an infinity of the same sign, and NaN stays NaN."""
    zero_top = 0x33000000                  # bits of 2^-25
    inf_from = 0x477FF000                  # bits of 65520.0
    chunk = 1 << 26
    for sign in (0, 0x80000000):
        sbit = np.uint16(0x8000 if sign else 0)
        for lo in range(0, 1 << 31, chunk):
            hi = min(lo + chunk, 1 << 31)
            ours = orc.f32bits_to_f16(sign + lo, sign + hi)
            mag = np.arange(lo, hi, dtype=np.uint32)
            band = (mag > zero_top) & (mag < inf_from)
            if band.any():
                x = (mag[band] | np.uint32(sign)).view(np.float32)
                ref = x.astype(np.float16).view(np.uint16)
                bad = ours[band] != ref
                assert not bad.any(), f"first mismatch at {hex(int(x.view(np.uint32)[np.argmax(bad)]))}"
            low = mag <= zero_top
            assert (ours[low] == sbit).all()
            big = mag >= inf_from
            if big.any():
                out = ours[big]
                nan_in = mag[big] > 0x7F800000
                assert (out[~nan_in] == (sbit | np.uint16(0x7C00))).all()
                nan_out = ((out & 0x7C00) == 0x7C00) & ((out & 0x03FF) != 0)
                assert nan_out[nan_in].all()


def test_format_constants_from_pages(orc):
    """Pin P2: the largest finite value, the smallest normal and subnormal."""
    dec = lambda b: float(orc.f16_to_f32(np.array([b], np.uint16))[0])
    enc = lambda v: int(orc.f32_to_f16(np.array([v], np.float32))[0])
    assert dec(0x7BFF) == GOLD["f16_max"]["value"]
    assert dec(0x0400) == GOLD["f16_min_normal"]["value"] == 2.0 ** GOLD["f16_min_normal"]["log2"]
    assert dec(0x0001) == 2.0 ** GOLD["f16_min_subnormal_log2"]["value"]
    lo, hi = GOLD["f16_normal_exponent_range"]["value"]
    assert dec(((lo + 15) << 10)) == 2.0 ** lo and dec(((hi + 15) << 10)) == 2.0 ** hi
    assert dec(0x3C00 | 1) - 1.0 == 2.0 ** -GOLD["f16_mantissa_bits"]["value"]
    assert enc(65519.99) == 0x7BFF
    assert enc(65520.0) == 0x7C00
    assert enc(-65520.0) == 0xFC00
    assert enc(float("inf")) == 0x7C00
    assert enc(2.0 ** -14) == 0x0400
    assert enc(2.0 ** -24) == 0x0001


@pytest.mark.parametrize("value,bits", [
    (1.0 + 2.0 ** -11, 0x3C00),            # tie between 1 and 1+2^-10 -> even (1)
    (1.0 + 3 * 2.0 ** -11, 0x3C02),        # tie -> even significand (..10)
    (1.0 - 2.0 ** -12, 0x3C00),            # tie below 1 -> even (1.0)
    (1.0 - 2.0 ** -11, 0x3BFF),            # representable
    (2.0 ** -25, 0x0000),                  # exactly half the smallest subnormal -> 0
    (-(2.0 ** -25), 0x8000),               # sign kept
    (1.5 * 2.0 ** -25, 0x0001),            # above half -> smallest subnormal
    (3 * 2.0 ** -25, 0x0002),              # tie 1.5 subnormal quanta -> even (2)
    (5 * 2.0 ** -25, 0x0002),              # tie 2.5 quanta -> even (2)
    (2.0 ** -14 - 2.0 ** -25, 0x0400),     # tie at the top of the subnormals -> 2^-14
    (65504.0 + 15.0, 0x7BFF),
])
def test_round_to_nearest_even_cases(orc, value, bits):
    got = int(orc.f32_to_f16(np.array([value], np.float32))[0])
    assert got == bits, (value, hex(got))


def test_flush_without_scaling_and_survive_with_it(orc):
    """Pin P3: values no larger than 2^-25 become zero; scaling by 8 shifts [2^-27, 2^-24) into
    [2^-24, 2^-21), where every value survives with <= 2^-11 relative error (analysis page,
    §3.4 "Loss Scaling")."""
    ex = GOLD["loss_scale_shift_example"]
    g = np.random.Generator(np.random.PCG64(1))
    lo, hi = ex["from_log2"]
    x = np.exp2(g.uniform(lo, hi, 100000)).astype(np.float32)
    tiny = x[x <= 2.0 ** -25]
    assert tiny.size > 0 and not orc.f32_to_f16(tiny).any()
    scaled = (x * np.float32(ex["scale"])).astype(np.float32)
    assert np.log2(ex["scale"]) == ex["exponent_increase"]
    back = orc.f16_to_f32(orc.f32_to_f16(scaled))
    assert (back > 0).all()
    assert (back >= 2.0 ** ex["to_log2"][0]).all() and (back <= 2.0 ** ex["to_log2"][1]).all()
    # the subnormal spacing 2^-24 bounds the absolute error; relative error at most 1/2 ulp of
    # the smallest binade reached
    rel = np.abs(back.astype(np.float64) - scaled) / scaled
    assert rel.max() <= 0.5  # 2^-24-binade values keep at least their leading bit
    assert np.abs(back.astype(np.float64) - scaled).max() <= 2.0 ** -25


def test_swamping_threshold_in_f16_and_f32(orc):
    """Pin P5 (codec part): an addend 2048x smaller than a power-of-two weight is lost when the
    sum is rounded to binary16, kept when the sum is held in FP32 (analysis page, §3.4 "FP32
    Master Copy of Weights", failure mechanism 2)."""
    r = GOLD["swamping_ratio_f16"]["value"]
    w = np.float32(1.0)
    s = np.float32(w + np.float32(1.0 / r))          # FP32 sum, exact
    assert float(s) == 1.0 + 2.0 ** -11
    assert int(orc.f32_to_f16(np.array([s], np.float32))[0]) == 0x3C00     # lost in FP16
    # just below the threshold the update survives the FP16 rounding
    s2 = np.float32(w + np.float32(2.0 / r))
    assert int(orc.f32_to_f16(np.array([s2], np.float32))[0]) == 0x3C01
    # counter-examples of the plain ratio rule (see the design notes)
    s3 = np.float32(np.float32(1.5) + np.float32(1.5 / r))
    assert float(orc.f16_to_f32(orc.f32_to_f16(np.array([s3], np.float32)))[0]) == 1.5009765625
    assert int(orc.f32_to_f16(np.array([1.0 - 2.0 ** -11], np.float32))[0]) == 0x3BFF
    assert int(orc.f32_to_f16(np.array([1.0 - 2.0 ** -12], np.float32))[0]) == 0x3C00
    # FP32 loses an addend only at the ratio 2^24
    f32r = 2.0 ** GOLD["swamping_ratio_f32_log2"]["value"]
    assert np.float32(np.float32(1.0) + np.float32(1.0 / f32r)) == np.float32(1.0)
    assert np.float32(np.float32(1.0) + np.float32(2.0 / f32r)) != np.float32(1.0)
