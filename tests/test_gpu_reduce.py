"""GPU parity of the large reductions: batch-normalization statistics and normalization, and the
row softmax, all binary16 in and out with FP32 arithmetic.

Source: "Mixed Precision Training", long-form analysis page, §3.4 "FP16 Arithmetic with FP32
Accumulation": batch normalization's mean and variance over the batch and spatial positions and
the softmax normalization constant are summed in FP32 from binary16 tensors (the page's example
is 32 images of 112 x 112 positions and 64 channels, ~25.7M values), the arithmetic is FP32 and
binary16 results are written back. The softmax case at full size is a row of the 793K-word
vocabulary of the page's bigLSTM language model (§4.5).

Bars:
- Statistics: the oracle's fp64 values. Per-thread FP32 sums of shifted values (the shift a
  sample of the data, within a few std of the mean, so s2 - s1^2/n cancels at most ~17x) merged
  pairwise err by about eps32 * (17 + log2(n)) * (1 + |mean| / std) relative to the variance
  (eps32 = 2^-24, n <= 2^19, |mean| <= 4 std here: <= 2e-5), so |var - var*| <= 5e-5 var +
  1e-6 mean^2 and |mean - mean*| <= 1e-5 std + 1e-6 |mean|. Two runs give the same bits.
- Normalization: bit-exact against the oracle's FP32 evaluation in the same order, given the
  same FP32 mean, var, gamma, beta.
- Softmax: within one binary16 ulp of the oracle's fp64 result rounded once (2^-10 relative,
  2^-24 absolute): the FP32 sums and exp err by < 1e-5 relative, inside half an ulp (2^-11);
  two runs give the same bits.
"""
import ctypes as C

import numpy as np
import pytest
import torch

import mixed_precision_neural_amd as mp
import oracle
from gpu_util import dev_f16, dev_f32, f16_values, host_bits16, host_f32, require_gpu

pytestmark = pytest.mark.gpu


def normal_f16(rng, shape, mean_scale=0.0):
    """N(mu_c, s_c^2) per column, |mu_c| <= 4 s_c, s_c spread over 2^-6 .. 2^6."""
    s = 2.0 ** rng.uniform(-6, 6, shape[1])
    mu = s * rng.uniform(-4, 4, shape[1]) * mean_scale
    return (rng.standard_normal(shape) * s + mu).astype(np.float16).view(np.uint16)


def within_ulp(got, ref, ulps=1):
    g, r = f16_values(got), f16_values(ref)
    tol = np.maximum(np.abs(r) * 2.0 ** -10 * ulps, 2.0 ** -24 * ulps)
    both_nan = np.isnan(g) & np.isnan(r)
    return bool(np.all(both_nan | (np.abs(g - r) <= tol)))


def padded(bits, ld, fill=0x7E00):
    """A device matrix of the same values with row pitch ld (padding = NaN)."""
    rows, cols = bits.shape
    wide = np.full((rows, ld), fill, np.uint16)
    wide[:, :cols] = bits
    return dev_f16(wide)[:, :cols]


# ---------------------------------------------------------------- statistics
STAT_SHAPES = [(37, 5), (1000, 64), (4099, 72), (513, 260), (3000, 4096), (1, 16), (401408, 64)]


@pytest.mark.parametrize("rows,ch", STAT_SHAPES)
def test_bn_stats_against_oracle(rows, ch):
    """Both paths (16-byte: channels a multiple of 8; element-wise otherwise), one and several
    channel blocks, ragged row chunks, and the page's 32 x 112 x 112 x 64 case."""
    require_gpu()
    rng = np.random.Generator(np.random.PCG64(rows * 7 + ch))
    x = normal_f16(rng, (rows, ch), mean_scale=1.0)
    mean, var = mp.bn_stats(dev_f16(x))
    m2, v2 = mp.bn_stats(dev_f16(x))
    torch.cuda.synchronize()
    gm, gv = host_f32(mean).astype(np.float64), host_f32(var).astype(np.float64)
    rm, rv = oracle.bn_stats(x)
    sd = np.sqrt(rv)
    assert np.all(np.abs(gm - rm) <= 1e-5 * sd + 1e-6 * np.abs(rm) + 1e-30), np.max(np.abs(gm - rm) / (sd + 1e-30))
    assert np.all(np.abs(gv - rv) <= 5e-5 * rv + 1e-6 * rm * rm + 1e-30), np.max(np.abs(gv - rv) / (rv + 1e-30))
    assert np.array_equal(host_f32(m2).view(np.uint32), host_f32(mean).view(np.uint32))
    assert np.array_equal(host_f32(v2).view(np.uint32), host_f32(var).view(np.uint32))


def test_bn_stats_strided_and_constant():
    """A row pitch beyond the channels (NaN padding must not leak); constant channels give
    their value and variance 0 exactly."""
    require_gpu()
    rng = np.random.Generator(np.random.PCG64(3))
    x = normal_f16(rng, (777, 40))
    x[:, 3] = np.float16(2.5).view(np.uint16)
    for ld in (48, 43):                          # 16-byte path, then element-wise
        mean, var = mp.bn_stats(padded(x, ld))
        torch.cuda.synchronize()
        gm, gv = host_f32(mean).astype(np.float64), host_f32(var).astype(np.float64)
        rm, rv = oracle.bn_stats(x)
        assert np.all(np.isfinite(gm)) and np.all(np.isfinite(gv))
        assert np.all(np.abs(gm - rm) <= 1e-5 * np.sqrt(rv) + 1e-6 * np.abs(rm) + 1e-30)
        assert np.all(np.abs(gv - rv) <= 5e-5 * rv + 1e-6 * rm * rm + 1e-30)
        assert gm[3] == 2.5 and gv[3] == 0.0


def test_bn_stats_very_wide_pitch():
    """A row pitch of 2^20 values (2 MiB between rows; a chunk of rows spans over 2^31 bytes):
    the 16-byte path's addressing at pitches far beyond the channel count."""
    require_gpu()
    rng = np.random.Generator(np.random.PCG64(5))
    x = normal_f16(rng, (120, 40), mean_scale=1.0)
    mean, var = mp.bn_stats(padded(x, 1 << 20))
    torch.cuda.synchronize()
    gm, gv = host_f32(mean).astype(np.float64), host_f32(var).astype(np.float64)
    rm, rv = oracle.bn_stats(x)
    assert np.all(np.abs(gm - rm) <= 1e-5 * np.sqrt(rv) + 1e-6 * np.abs(rm) + 1e-30)
    assert np.all(np.abs(gv - rv) <= 5e-5 * rv + 1e-6 * rm * rm + 1e-30)


# ---------------------------------------------------------------- normalization
@pytest.mark.parametrize("rows,ch", [(37, 5), (1000, 64), (4099, 72), (513, 260), (401408, 64)])
def test_bn_apply_bit_exact(rows, ch):
    require_gpu()
    rng = np.random.Generator(np.random.PCG64(rows + 11 * ch))
    x = normal_f16(rng, (rows, ch), mean_scale=1.0)
    mean, var = [a.astype(np.float32) for a in oracle.bn_stats(x)]
    gamma = rng.uniform(0.5, 2.0, ch).astype(np.float32)
    beta = rng.uniform(-1, 1, ch).astype(np.float32)
    eps = np.float32(1e-5)
    y = mp.bn_apply(dev_f16(x), dev_f32(mean), dev_f32(var), dev_f32(gamma), dev_f32(beta), float(eps))
    torch.cuda.synchronize()
    ref = oracle.bn_apply(x, mean, var, gamma, beta, eps)
    got = host_bits16(y)
    bad = np.argwhere(got != ref)
    assert bad.size == 0, [(int(i), int(j), hex(got[i, j]), hex(ref[i, j])) for i, j in bad[:8]]


def test_bn_apply_strided_and_in_place():
    require_gpu()
    rng = np.random.Generator(np.random.PCG64(8))
    x = normal_f16(rng, (300, 24))
    mean, var = [a.astype(np.float32) for a in oracle.bn_stats(x)]
    gamma, beta = np.full(24, 1.5, np.float32), np.full(24, -0.25, np.float32)
    ref = oracle.bn_apply(x, mean, var, gamma, beta, 1e-3)
    args = (dev_f32(mean), dev_f32(var), dev_f32(gamma), dev_f32(beta), 1e-3)
    for ld in (32, 27):
        xd = padded(x, ld)
        yd = padded(np.zeros_like(x), ld + 1, fill=0x1234)
        mp.bn_apply(xd, *args, y=yd)
        assert np.array_equal(host_bits16(yd), ref)
        assert (host_bits16(yd.as_strided((300, 1), (ld + 1, 1), 24)) == 0x1234).all()   # pitch untouched
        mp.bn_apply(xd, *args, y=xd)                                                    # in place
        assert np.array_equal(host_bits16(xd), ref)


# ---------------------------------------------------------------- softmax
SOFTMAX_SHAPES = [
    (7, 10, 10),                 # element-wise two-pass form (odd pitch)
    (1000, 512, 512),            # two-pass: more rows than blocks of the single-read form
    (3, 3 * 8192 + 5, 3 * 8192 + 8),   # single read, one block per row, ragged tail
    (2, 50000, 50001),           # element-wise two-pass form, several segments
    (64, 793471, 793472),        # the page's vocabulary: single read, 4 blocks of 24,796 vectors per row
    (5, 1200003, 1200008),       # single read, 37 blocks per row of 4,055 vectors (8 per thread)
    (1, 40000005, 40000008),     # single read, 256 blocks of 19,532 vectors: a polling lane watches 4 slots
    (256, 204795, 204800),       # single read at capacity: one block per row, 50 vectors per thread
    (257, 1000, 1000),           # one row too many for one block per compute unit: two-pass
    (5, 7, 8),                   # single read, rows shorter than one 16-byte vector: the tail only
    (3, 8, 8),                   # single read, one vector per row and no tail
    (200, 300000, 300000),       # one block per row allowed, but a row exceeds 204,800 values: two-pass
]


@pytest.mark.parametrize("rows,cols,ld", SOFTMAX_SHAPES)
def test_softmax_against_oracle(rows, cols, ld):
    """Both forms (single read when the rows fit on chip, two-pass otherwise), 16-byte and
    element-wise paths, ragged tails, the single-read form's capacity limit, and the page's
    vocabulary size (64 rows of 793,471 with a row pitch of 793,472)."""
    require_gpu()
    rng = np.random.Generator(np.random.PCG64(rows + cols))
    x = (rng.standard_normal((rows, cols)) * 3.0).astype(np.float16).view(np.uint16)
    xd = padded(x, ld)
    y = mp.softmax(xd)
    y2 = mp.softmax(xd)
    torch.cuda.synchronize()
    got = host_bits16(y)
    ref = oracle.softmax(x)
    assert within_ulp(got, ref)
    assert np.array_equal(got, host_bits16(y2))


@pytest.mark.parametrize("rows,cols,ld", [(64, 793471, 793472), (1, 40000005, 40000008), (5, 1200003, 1200008)])
def test_softmax_single_read_without_waiting_gives_the_same_bits(rows, cols, ld):
    """With the wait set to 0 every block computes its row's other segments' (max, sum) from x
    itself: the path a block takes when the others are not resident. The bits must equal those
    of the blocks exchanging their pairs."""
    require_gpu()
    rng = np.random.Generator(np.random.PCG64(7 * rows + cols))
    x = (rng.standard_normal((rows, cols)) * 3.0).astype(np.float16).view(np.uint16)
    x[rows // 2, cols // 3] = 0x7BFF                          # one large value: a block's max
    xd = padded(x, ld)
    ref = host_bits16(mp.softmax(xd))
    prev = mp.softmax_wait_us(0)
    try:
        got = host_bits16(mp.softmax(xd))
    finally:
        mp.softmax_wait_us(prev)
    assert prev == mp.softmax_wait_us()
    assert np.array_equal(got, ref)


def test_softmax_concurrent_calls_on_two_streams():
    """Two single-read calls with their own workspaces on two streams: each grid wants every
    compute unit, so some blocks start only when the other call's blocks leave, and their
    row's resident blocks wait or compute the missing pairs themselves. The bits equal those of
    one call at a time."""
    require_gpu()
    rng = np.random.Generator(np.random.PCG64(11))
    xa = dev_f16((rng.standard_normal((64, 393216)) * 2.0).astype(np.float16).view(np.uint16))
    xb = dev_f16((rng.standard_normal((32, 800000)) * 4.0).astype(np.float16).view(np.uint16))
    ref_a, ref_b = host_bits16(mp.softmax(xa)), host_bits16(mp.softmax(xb))
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    ya, yb = torch.empty_like(xa), torch.empty_like(xb)
    torch.cuda.synchronize()
    for _ in range(3):
        with torch.cuda.stream(sa):
            mp.softmax(xa, y=ya, stream=sa)
        with torch.cuda.stream(sb):
            mp.softmax(xb, y=yb, stream=sb)
        torch.cuda.synchronize()
        assert np.array_equal(host_bits16(ya), ref_a)
        assert np.array_equal(host_bits16(yb), ref_b)


def test_softmax_captured_in_a_graph_and_replayed_on_new_inputs():
    """A call captured into a HIP graph takes the two-pass form (the single-read form's per-call
    tag would repeat on every replay, and a block could take an earlier replay's slots for this
    one's). Replayed on three different inputs written into the captured buffer, each replay is
    within one ulp of the oracle and equal to the two-pass form run eagerly (in place on a copy)."""
    require_gpu()
    rows, cols, ld = 64, 393216, 393216
    rng = np.random.Generator(np.random.PCG64(5))
    xd = dev_f16((rng.standard_normal((rows, cols)) * 3.0).astype(np.float16).view(np.uint16))
    yd = torch.empty_like(xd)
    mp.softmax(xd, y=yd)                       # warm-up outside capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        mp.softmax(xd, y=yd)                   # recorded, not run
    for t in range(3):
        x = (rng.standard_normal((rows, cols)) * (2.0 + t)).astype(np.float16).view(np.uint16)
        xd.copy_(dev_f16(x))
        g.replay()
        torch.cuda.synchronize()
        got = host_bits16(yd)
        assert within_ulp(got, oracle.softmax(x)), t
        two_pass = dev_f16(x)
        mp.softmax(two_pass, y=two_pass)       # in place: the two-pass form
        assert np.array_equal(got, host_bits16(two_pass)), t


def test_softmax_special_values_and_in_place():
    require_gpu()
    ninf, pinf, nan = 0xFC00, 0x7C00, 0x7E00
    rows = np.zeros((6, 24), np.uint16)
    rows[0, ::2] = ninf                       # -inf entries give 0
    rows[1, 5] = pinf                         # +inf: NaN throughout
    rows[2, 7] = nan                          # NaN: NaN throughout
    rows[3, :] = ninf                         # only -inf: NaN
    rows[4, :] = np.float16(60000.0).view(np.uint16)    # exp overflows without the max shift
    rows[5, :16] = ninf                       # a first vector of only -inf, then finite values
    ref = oracle.softmax(rows)
    for ld in (24, 25):
        xd = padded(rows, ld)
        got = host_bits16(mp.softmax(xd))
        assert within_ulp(got, ref), ld
        mp.softmax(xd, y=xd)
        assert within_ulp(host_bits16(xd), ref), ld


def test_argument_errors():
    """Invalid sizes, pitches and workspaces are rejected before any launch."""
    require_gpu()
    L = mp.lib()
    x = torch.zeros((4, 16), dtype=torch.float16, device="cuda")
    f = torch.zeros(16, dtype=torch.float32, device="cuda")
    ws = torch.zeros(1 << 16, dtype=torch.uint8, device="cuda")
    p = lambda t: C.c_void_p(t.data_ptr())
    s = C.c_void_p(torch.cuda.current_stream().cuda_stream)
    inval = 1                                  # MP_ERR_INVALID_ARGUMENT
    assert L.mp_bn_stats(p(x), 0, 16, 16, p(f), p(f), p(ws), 1 << 16, s) == inval          # no rows
    assert L.mp_bn_stats(p(x), 4, 16, 8, p(f), p(f), p(ws), 1 << 16, s) == inval           # ld < C
    assert L.mp_bn_stats(p(x), 4, 16, 16, p(f), p(f), p(ws), 4, s) == inval                # workspace
    assert L.mp_bn_stats(p(x), 4, 16, 16, None, p(f), p(ws), 1 << 16, s) == inval
    assert L.mp_bn_apply(p(x), -1, 16, 16, p(f), p(f), p(f), p(f), 0.0, p(x), 16, s) == inval
    assert L.mp_bn_apply(p(x), 4, 16, 16, p(f), p(f), None, p(f), 0.0, p(x), 16, s) == inval
    assert L.mp_softmax(p(x), 4, 16, 15, p(x), 16, p(ws), 1 << 16, s) == inval
    assert L.mp_softmax(p(x), 4, 16, 16, p(x), 16, None, 0, s) == inval
    assert L.mp_softmax(p(x), 0, 16, 16, p(x), 16, None, 0, s) == 0                       # nothing to do
    assert L.mp_bn_stats_workspace(0, 16) == 0 and L.mp_softmax_workspace(4, 0) == 0
