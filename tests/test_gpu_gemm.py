"""GPU parity of the three dot-product layers (forward, dgrad, wgrad) against the oracle.

Source: "Mixed Precision Training", long-form analysis page, §3.4 "FP16 Arithmetic
with FP32 Accumulation" and "The Integrated Training Procedure", Steps 2 and 4.

Tolerances: the error metric is max |y - r| / max(|r|, rms(r)) over the compared
outputs; FP32 outputs must be within 2e-3 of the oracle's ascending-order FP32
sum and binary16 outputs within 1e-2. Exactly representable problems (P8) must
match bit for bit.
"""
import numpy as np
import pytest
import torch

import mixed_precision_neural_amd as mp
import oracle
import workloads
from gpu_util import dev_f16, f16_values, host_bits16, host_f32, rel_err, require_gpu

pytestmark = pytest.mark.gpu

TOL_F32, TOL_F16 = 2e-3, 1e-2


def grid_bits(rng, shape, q_log2=-8, lim=2.0):
    q = 2.0 ** q_log2
    ints = rng.integers(-int(lim / q), int(lim / q) + 1, shape)
    return (ints * q).astype(np.float16).view(np.uint16), ints.astype(np.int64)


def gpu_all(X, W, dY, out=torch.float32):
    dX, dW_, dY_ = dev_f16(X), dev_f16(W), dev_f16(dY)
    y = mp.linear_fwd(dX, dW_, out_dtype=out)
    dx = mp.linear_dgrad(dY_, dW_, out_dtype=out)
    dw = mp.linear_wgrad(dY_, dX, out_dtype=out)
    torch.cuda.synchronize()
    if out == torch.float32:
        return host_f32(y), host_f32(dx), host_f32(dw)
    return host_bits16(y), host_bits16(dx), host_bits16(dw)


@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (3, 5, 7), (64, 10, 32), (17, 300, 24), (300, 257, 32),
                                   (2600, 3100, 32), (512, 768, 256), (1024, 512, 1536)])
def test_exact_integer_sums(M, N, K):
    """Grids of fewer than 128 tiles of 256 x 256 run the 64 x 64 kernel; the others the 256 x
    256 kernel's general loop here (reductions that are not multiples of 128). The direct-to-LDS
    loop is pinned the same way by test_exact_integer_sums_direct_to_lds.

    Pin P8: on a 2^-q grid with |x| <= 2 every product is a multiple of 2^-2q below 4, so a
    partial sum over R terms is a multiple of 2^-2q below 4R: exact in FP32 while 4R * 2^2q <= 2^24.
    The GPU result must then equal the integer sum bit for bit in any summation order. q = 8 for
    reductions up to 32, q = 4 up to 4096 (both tile paths)."""
    require_gpu()
    rng = np.random.Generator(np.random.PCG64(M + N + K))
    q = 8 if max(M, N, K) <= 32 else 4
    assert 4 * max(M, N, K) * 2 ** (2 * q) <= 2 ** 24
    X, Xi = grid_bits(rng, (M, K), -q); W, Wi = grid_bits(rng, (N, K), -q)
    dY, dYi = grid_bits(rng, (M, N), -q)
    y, dx, dw = gpu_all(X, W, dY)
    q2 = 2.0 ** (-2 * q)
    assert np.array_equal(y.astype(np.float64), (Xi @ Wi.T) * q2)
    assert np.array_equal(dx.astype(np.float64), (dYi @ Wi) * q2)
    assert np.array_equal(dw.astype(np.float64), (dYi.T @ Xi) * q2)


def test_exact_subnormal_inputs():
    """Pin P8, subnormal variant: binary16 subnormal operands must not be flushed by the MFMA."""
    require_gpu()
    rng = np.random.Generator(np.random.PCG64(11))
    M, N, K = 40, 24, 32
    Xi = rng.integers(-1023, 1024, (M, K))
    X = (np.abs(Xi) | np.where(Xi < 0, 0x8000, 0)).astype(np.uint16)
    Wi = rng.integers(-4, 5, (N, K))
    W = Wi.astype(np.float16).view(np.uint16)
    y = mp.linear_fwd(dev_f16(X), dev_f16(W), out_dtype=torch.float32)
    assert np.array_equal(host_f32(y).astype(np.float64), (Xi @ Wi.T) * 2.0 ** -24)


def test_fp32_accumulation_discriminator():
    """Pin P9: X = W = 1 with K = 4096 gives exactly 4096 (a binary16 accumulator stalls at 2048);
    random N(0,1) at K = 4096 stays within 2e-3 (a binary16 accumulator would be ~15x over)."""
    require_gpu()
    K = 4096
    ones = np.full((64, K), 0x3C00, np.uint16)
    y = host_f32(mp.linear_fwd(dev_f16(ones), dev_f16(ones[:48]), out_dtype=torch.float32))
    assert (y == 4096.0).all()
    rng = np.random.Generator(np.random.PCG64(1))
    X = rng.standard_normal((256, K)).astype(np.float16).view(np.uint16)
    W = rng.standard_normal((192, K)).astype(np.float16).view(np.uint16)
    got = host_f32(mp.linear_fwd(dev_f16(X), dev_f16(W), out_dtype=torch.float32))
    assert rel_err(got, oracle.linear_fwd(X, W)) <= TOL_F32


@pytest.mark.parametrize("M,N,K", [(4096, 4096, 2048), (4100, 4352, 2176), (2048, 8192, 128)])
def test_exact_integer_sums_direct_to_lds(M, N, K):
    """Pin P8 on the 256 x 256 kernel's direct-to-LDS loop (128 or more big tiles; whole tiles,
    reductions multiples of 128): 4096 x 4096 x 2048 sends all three layers through it;
    4100 x 4352 x 2176 mixes whole tiles with ragged edge tiles (general loop) in one launch, and
    its wgrad reduction (4100) is not a multiple of 128; 2048 x 8192 x 128 is the two-slab minimum
    for the forward layer. Integer sums below 2^53 are exact in float64, so the reference is a
    float64 product of the integer grids."""
    require_gpu()
    rng = np.random.Generator(np.random.PCG64(M + 2 * N + 3 * K))
    q = 4
    assert 4 * max(M, N, K) * 2 ** (2 * q) <= 2 ** 24
    X, Xi = grid_bits(rng, (M, K), -q); W, Wi = grid_bits(rng, (N, K), -q)
    dY, dYi = grid_bits(rng, (M, N), -q)
    y, dx, dw = gpu_all(X, W, dY)
    Xf, Wf, dYf = Xi.astype(np.float64), Wi.astype(np.float64), dYi.astype(np.float64)
    q2 = 2.0 ** (-2 * q)
    assert np.array_equal(y.astype(np.float64), (Xf @ Wf.T) * q2)
    assert np.array_equal(dx.astype(np.float64), (dYf @ Wf) * q2)
    assert np.array_equal(dw.astype(np.float64), (dYf.T @ Xf) * q2)


def test_exact_integer_sums_direct_to_lds_padded_rows():
    """P8 on the direct-to-LDS loop with row pitches above the row length (multiples of 8, so
    the loop still applies): every operand and output a view into a wider buffer. At 4096 x
    4096 x 2048 all three layers run the 256 x 256 loop; its slab offsets along the pitch (the
    reduction-strided operands step 64 pitches per slab) and the binary16 outputs' row stores
    must follow the pitch, and the columns past each row stay untouched. Binary16 outputs: the
    exact sums rounded once to nearest even."""
    require_gpu()
    M, N, K, q = 4096, 4096, 2048, 4
    rng = np.random.Generator(np.random.PCG64(17))
    X, Xi = grid_bits(rng, (M, K + 24), -q)
    W, Wi = grid_bits(rng, (N, K + 40), -q)
    dY, dYi = grid_bits(rng, (M, N + 8), -q)
    dX_, dW_, dY_ = dev_f16(X)[:, :K], dev_f16(W)[:, :K], dev_f16(dY)[:, :N]
    fill = 0x7E00                                          # a NaN pattern no GEMM output can take
    outs = {name: torch.from_numpy(np.full(shape, fill, np.uint16).view(np.int16)).cuda().view(torch.float16)
            for name, shape in (("y", (M, N + 16)), ("dx", (M, K + 32)), ("dw", (N, K + 8)))}
    mp.linear_fwd(dX_, dW_, Y=outs["y"][:, :N])
    mp.linear_dgrad(dY_, dW_, dX=outs["dx"][:, :K])
    mp.linear_wgrad(dY_, dX_, dW=outs["dw"][:, :K])
    torch.cuda.synchronize()
    Xf, Wf, dYf = (a.astype(np.float64) for a in (Xi[:, :K], Wi[:, :K], dYi[:, :N]))
    q2 = 2.0 ** (-2 * q)
    want = {"y": (Xf @ Wf.T) * q2, "dx": (dYf @ Wf) * q2, "dw": (dYf.T @ Xf) * q2}
    for name, ref in want.items():
        got = host_bits16(outs[name])
        cols = ref.shape[1]
        # the FP32 sums are exact (multiples of 2^-8 below 2^16), so the binary16 output is the
        # nearest-even binary16 of the exact sum (numpy rounds float64 to float16 that way)
        assert np.array_equal(got[:, :cols], ref.astype(np.float16).view(np.uint16)), name
        assert (got[:, cols:] == fill).all(), name


@pytest.mark.parametrize("M,N,K", [(64, 512, 256), (64, 10, 512), (300, 520, 200), (777, 1000, 333),
                                   (2600, 3100, 96), (4099, 2050, 130), (512, 768, 256),
                                   (1280, 1024, 384)])
def test_ragged_shapes_against_oracle(M, N, K):
    """Shapes spanning several tiles with ragged edges in every dimension, FP32 and binary16 out."""
    require_gpu()
    rng = np.random.Generator(np.random.PCG64(M * 7 + N * 3 + K))
    X = rng.standard_normal((M, K)).astype(np.float16).view(np.uint16)
    W = (rng.standard_normal((N, K)) / np.sqrt(K)).astype(np.float16).view(np.uint16)
    dY = rng.standard_normal((M, N)).astype(np.float16).view(np.uint16)
    refs = [oracle.linear_fwd(X, W), oracle.linear_dgrad(dY, W), oracle.linear_wgrad(dY, X)]
    got32 = gpu_all(X, W, dY, torch.float32)
    for g, r, name in zip(got32, refs, ("fwd", "dgrad", "wgrad")):
        assert g.shape == r.shape
        assert rel_err(g, r) <= TOL_F32, name
    got16 = gpu_all(X, W, dY, torch.float16)
    for g, r, name in zip(got16, refs, ("fwd", "dgrad", "wgrad")):
        assert rel_err(f16_values(g), r) <= TOL_F16, name


@pytest.mark.parametrize("M,N,K", [(64, 10, 512), (300, 520, 200), (1280, 1024, 384), (2048, 2048, 1024)])
def test_binary16_output_is_nearest_even_of_the_fp32_output(M, N, K):
    """The binary16 epilogue rounds the FP32 accumulator to nearest even (§3.4: FP32 sums,
    rounded to binary16 when stored): both outputs come from the same accumulation, so the
    binary16 result must equal the round-to-nearest-even of the FP32 result bit for bit, ties
    included (numpy's float16 cast, a library routine of neither side, rounds that way; the
    oracle's codec is pinned against it exhaustively)."""
    require_gpu()
    rng = np.random.Generator(np.random.PCG64(M + 3 * N + 7 * K))
    X = rng.standard_normal((M, K)).astype(np.float16).view(np.uint16)
    W = (rng.standard_normal((N, K)) / np.sqrt(K)).astype(np.float16).view(np.uint16)
    dY = rng.standard_normal((M, N)).astype(np.float16).view(np.uint16)
    f32 = gpu_all(X, W, dY, torch.float32)
    f16 = gpu_all(X, W, dY, torch.float16)
    for a, b, name in zip(f32, f16, ("fwd", "dgrad", "wgrad")):
        assert np.array_equal(b, np.ascontiguousarray(a, np.float32).astype(np.float16).view(np.uint16)), name


def test_unaligned_leading_dimensions():
    """Row pitches that are not multiples of 8 elements take the element-wise load path."""
    require_gpu()
    rng = np.random.Generator(np.random.PCG64(2))
    M, N, K = 333, 270, 77
    Xf = rng.standard_normal((M, K + 2)).astype(np.float16).view(np.uint16)
    Wf = rng.standard_normal((N, K + 5)).astype(np.float16).view(np.uint16)
    dYf = rng.standard_normal((M, N + 1)).astype(np.float16).view(np.uint16)
    X, W, dY = Xf[:, :K], Wf[:, :K], dYf[:, :N]
    dX_, dW_, dYd = dev_f16(Xf)[:, :K], dev_f16(Wf)[:, :K], dev_f16(dYf)[:, :N]
    y = mp.linear_fwd(dX_, dW_, out_dtype=torch.float32)
    dx = mp.linear_dgrad(dYd, dW_, out_dtype=torch.float32)
    dw = mp.linear_wgrad(dYd, dX_, out_dtype=torch.float32)
    assert rel_err(host_f32(y), oracle.linear_fwd(X.copy(), W.copy())) <= TOL_F32
    assert rel_err(host_f32(dx), oracle.linear_dgrad(dY.copy(), W.copy())) <= TOL_F32
    assert rel_err(host_f32(dw), oracle.linear_wgrad(dY.copy(), X.copy())) <= TOL_F32


def test_strided_output_and_k_zero():
    require_gpu()
    rng = np.random.Generator(np.random.PCG64(3))
    X = rng.standard_normal((70, 40)).astype(np.float16).view(np.uint16)
    W = rng.standard_normal((50, 40)).astype(np.float16).view(np.uint16)
    big = torch.full((70, 64), 7.0, dtype=torch.float32, device="cuda")
    mp.linear_fwd(dev_f16(X), dev_f16(W), Y=big[:, :50])
    out = host_f32(big)
    assert rel_err(out[:, :50], oracle.linear_fwd(X, W)) <= TOL_F32
    assert (out[:, 50:] == 7.0).all()                  # untouched beyond N
    e = torch.empty((70, 0), dtype=torch.float16, device="cuda")
    z = mp.linear_fwd(e, torch.empty((50, 0), dtype=torch.float16, device="cuda"), out_dtype=torch.float32)
    assert (host_f32(z) == 0).all()                     # K = 0 writes zeros


def test_empty_reduction_on_a_large_grid_writes_zeros():
    """A zero-length reduction with an output of 128 or more 256 x 256 tiles must take the
    general loop, which loads nothing, and write zeros. The operands are passed with row pitches
    that allow 16-byte loads (a pitch of 8 for the empty rows, n for the empty row lists), so
    that without the non-empty-reduction condition the launcher would pick the direct-to-LDS
    loop, whose prologue fetches a first slab the empty operands do not have. Forward with
    K = 0, dgrad with N = 0, wgrad with M = 0; binary16 and FP32 outputs, over a poisoned
    output buffer."""
    require_gpu()
    n = 4096
    no_cols = lambda: torch.empty((n, 8), dtype=torch.float16, device="cuda")[:, :0]   # [n, 0], pitch 8
    no_rows = lambda: torch.empty((0, n), dtype=torch.float16, device="cuda")           # [0, n], pitch n
    for dt in (torch.float16, torch.float32):
        out = torch.full((n, n), float("nan"), dtype=dt, device="cuda")
        mp.linear_fwd(no_cols(), no_cols(), Y=out)                     # K = 0
        torch.cuda.synchronize()
        assert (out == 0).all() and not torch.signbit(out).any()
        out.fill_(float("nan"))
        mp.linear_dgrad(no_cols(), no_rows(), dX=out)                  # N = 0
        torch.cuda.synchronize()
        assert (out == 0).all()
        out.fill_(float("nan"))
        flag = torch.zeros(1, dtype=torch.int32, device="cuda") if dt == torch.float16 else None
        mp.linear_wgrad(no_rows(), no_rows(), dW=out, found_inf=flag)  # M = 0
        torch.cuda.synchronize()
        assert (out == 0).all()
        if flag is not None:
            assert int(flag.item()) == 0


def test_overflow_becomes_inf_and_sets_wgrad_flag():
    """binary16 outputs overflow to +-inf (never 65504); wgrad ORs the flag when asked."""
    require_gpu()
    M, N, K = 128, 96, 64
    dY = np.full((M, N), 0x5BFF, np.uint16)          # 255.875
    X = np.full((M, K), 0x5BFF, np.uint16)
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    dw = mp.linear_wgrad(dev_f16(dY), dev_f16(X), found_inf=flag)
    assert (host_bits16(dw) == 0x7C00).all()
    assert int(flag.item()) == 1
    flag.zero_()
    small = np.full((M, N), 0x2000, np.uint16)
    mp.linear_wgrad(dev_f16(small), dev_f16(small[:, :K].copy()), found_inf=flag)
    assert int(flag.item()) == 0


def test_determinism():
    """Pin P10: the same inputs give the same bits twice."""
    require_gpu()
    c = workloads.c3(1024, 768, 512)
    a = gpu_all(c.X16, c.W16, c.dY16)
    b = gpu_all(c.X16, c.W16, c.dY16)
    for x, y in zip(a, b):
        assert np.array_equal(x.view(np.uint32), y.view(np.uint32))


def sample_points(rng, rows, cols, full_rows=64, full_cols=64, extra=4096):
    r = [np.repeat(rng.choice(rows, full_rows, replace=False), cols),
         np.tile(np.arange(rows), full_cols)]
    c = [np.tile(np.arange(cols), full_rows),
         np.repeat(rng.choice(cols, full_cols, replace=False), rows)]
    r.append(rng.integers(0, rows, extra)); c.append(rng.integers(0, cols, extra))
    r.append(np.array([rows - 1])); c.append(np.array([cols - 1]))
    return np.concatenate(r), np.concatenate(c)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("layer", ["fwd", "dgrad", "wgrad"])
def test_c3_full_size_sampled(layer):
    """C3 (M = 8192 tokens, N = K = 4096) in the launch configuration the benchmark times: 64 full
    rows, 64 full columns and 4096 random outputs against the oracle, FP32 and binary16 outputs."""
    require_gpu()
    c = workloads.c3()
    rng = np.random.Generator(np.random.PCG64(7))
    dX, dW, dY = dev_f16(c.X16), dev_f16(c.W16), dev_f16(c.dY16)
    if layer == "fwd":
        g32 = mp.linear_fwd(dX, dW, out_dtype=torch.float32); g16 = mp.linear_fwd(dX, dW)
        rows, cols = sample_points(rng, 8192, 4096)
        ref = oracle.linear_fwd_at(c.X16, c.W16, rows, cols)
    elif layer == "dgrad":
        g32 = mp.linear_dgrad(dY, dW, out_dtype=torch.float32); g16 = mp.linear_dgrad(dY, dW)
        rows, cols = sample_points(rng, 8192, 4096)
        ref = oracle.linear_dgrad_at(c.dY16, c.W16, rows, cols)
    else:
        g32 = mp.linear_wgrad(dY, dX, out_dtype=torch.float32); g16 = mp.linear_wgrad(dY, dX)
        rows, cols = sample_points(rng, 4096, 4096)
        ref = oracle.linear_wgrad_at(c.dY16, c.X16, rows, cols)
    ri, ci = torch.from_numpy(rows).cuda(), torch.from_numpy(cols).cuda()
    got32 = host_f32(g32[ri, ci])
    got16 = host_bits16(g16[ri, ci])
    assert rel_err(got32, ref) <= TOL_F32
    assert rel_err(f16_values(got16), ref) <= TOL_F16
