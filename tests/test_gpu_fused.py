"""GPU parity of the activation-fused dot-product layers.

Source: "Mixed Precision Training", long-form analysis page, §3.4 "The Integrated
Training Procedure", Steps 2 and 4: a layer's forward product followed by its
point-wise activation, and the activation gradient through it.

mp_linear_fwd_act must give the bits of mp_linear_fwd (binary16 out) followed by
mp_act_fwd, and mp_linear_dgrad_act the bits of mp_linear_dgrad followed by
mp_act_bwd. The point-wise ops themselves are pinned against the oracle over every
finite binary16 input (test_gpu_aux.py). Against the oracle, which only sees the
generated inputs: the product, and the activation (or its gradient) applied to the
oracle's own product, within the binary16 dot-product bar (max error / max(|ref|,
rms(ref)) <= 1e-2: the two products may round a value to neighbouring binary16 numbers
before the activation).

mp_linear_fwd_act_deriv stores act(Z) and RNE16(act'(Z)) instead of Z (the bits of mp_act_fwd
and of mp_act_bwd(Z, 1.0)); mp_linear_dgrad_mul multiplies the binary16 dgrad product by that
saved derivative in FP32 and rounds once, which is checked bit for bit against torch's FP32
product of the same two GPU tensors rounded to half, and against the oracle's exact
act'(Z) * (dY . W) from the generated inputs within the same bar.
"""
import numpy as np
import pytest
import torch

import mixed_precision_neural_amd as mp
import oracle
from gpu_util import dev_f16, f16_values, host_bits16, rel_err, require_gpu

pytestmark = pytest.mark.gpu

TOL_F16 = 1e-2


def act_ref(kind, z):
    return oracle.relu_fwd(z) if kind == mp.RELU else oracle.gelu_fwd(z)


def act_grad_ref(kind, z, dy):
    return oracle.relu_bwd(z, dy) if kind == mp.RELU else oracle.gelu_bwd(z, dy)


def sample_pts(rows, cols, seed):
    """Two full rows, two full columns and 4096 random outputs of a [rows, cols] result."""
    rng = np.random.Generator(np.random.PCG64(seed))
    r0, c0 = rng.choice(rows, 2, replace=False), rng.choice(cols, 2, replace=False)
    r = np.concatenate([np.repeat(r0, cols), np.tile(np.arange(rows), 2), rng.integers(0, rows, 4096)])
    c = np.concatenate([np.tile(np.arange(cols), 2), np.repeat(c0, rows), rng.integers(0, cols, 4096)])
    return r, c


def inputs(M, N, K, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    X = rng.standard_normal((M, K)).astype(np.float16).view(np.uint16)
    W = (rng.standard_normal((N, K)) / np.sqrt(K)).astype(np.float16).view(np.uint16)
    dY = rng.standard_normal((M, N)).astype(np.float16).view(np.uint16)
    Zs = rng.standard_normal((M, K)).astype(np.float16).view(np.uint16)   # saved pre-activation of dX
    return X, W, dY, Zs


def check_fwd(kind, X, W, Xd, Wd, Z=None, H=None, ref=True):
    Z, H = mp.linear_fwd_act(kind, Xd, Wd, Z=Z, H=H)
    Zu = mp.linear_fwd(Xd, Wd)
    Hu = mp.act_fwd(kind, Zu)
    torch.cuda.synchronize()
    z, h = host_bits16(Z), host_bits16(H)
    assert np.array_equal(z, host_bits16(Zu)), "Z differs from the unfused product"
    assert np.array_equal(h, host_bits16(Hu)), "H differs from the unfused activation"
    if ref == "sample":
        r, c = sample_pts(*z.shape, 1)
        z_o = oracle.f32_to_f16(oracle.linear_fwd_at(X, W, r, c))
        assert rel_err(f16_values(z[r, c]), f16_values(z_o)) <= TOL_F16
        assert rel_err(f16_values(h[r, c]), f16_values(act_ref(kind, z_o))) <= TOL_F16
    elif ref:
        z_o = oracle.linear_fwd(X, W, out_f16=True)
        assert rel_err(f16_values(z), f16_values(z_o)) <= TOL_F16
        assert rel_err(f16_values(h), f16_values(act_ref(kind, z_o))) <= TOL_F16


def check_dgrad(kind, dY, W, Zs, dYd, Wd, Zd, dZ=None, ref=True):
    dZ = mp.linear_dgrad_act(kind, dYd, Wd, Zd, dZ=dZ)
    dH = mp.linear_dgrad(dYd, Wd)
    dZu = mp.act_bwd(kind, Zd.contiguous(), dH)
    torch.cuda.synchronize()
    out, dh = host_bits16(dZ), host_bits16(dH)
    ref_u = host_bits16(dZu)
    bad = np.argwhere(out != ref_u)
    assert bad.size == 0, ("dZ differs from the unfused pair at %d of %d: " % (len(bad), out.size) +
                           "; ".join("z=%04x dh=%04x fused=%04x unfused=%04x" % (
                               host_bits16(Zd)[i, j], dh[i, j], out[i, j], ref_u[i, j]) for i, j in bad[:12]))
    if ref == "sample":
        r, c = sample_pts(*out.shape, 2)
        dh_o = oracle.f32_to_f16(oracle.linear_dgrad_at(dY, W, r, c))
        assert rel_err(f16_values(dh[r, c]), f16_values(dh_o)) <= TOL_F16
        dz_o = act_grad_ref(kind, np.ascontiguousarray(Zs[r, c]), dh_o)
        assert rel_err(f16_values(out[r, c]), f16_values(dz_o)) <= TOL_F16
    elif ref:
        dh_o = oracle.linear_dgrad(dY, W, out_f16=True)
        assert rel_err(f16_values(dh), f16_values(dh_o)) <= TOL_F16
        dz_o = act_grad_ref(kind, np.ascontiguousarray(Zs), dh_o)
        assert rel_err(f16_values(out), f16_values(dz_o)) <= TOL_F16


@pytest.mark.parametrize("kind", [mp.RELU, mp.GELU])
@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (64, 512, 256), (64, 10, 512), (300, 520, 200),
                                   (777, 1000, 333), (2600, 3100, 96), (1280, 1024, 384)])
def test_fused_matches_unfused_and_oracle(kind, M, N, K):
    """Small (64 x 64 tiles) and large (256 x 256 tiles) grids, ragged in every dimension."""
    require_gpu()
    X, W, dY, Zs = inputs(M, N, K, M * 5 + N * 3 + K + kind)
    Xd, Wd, dYd, Zd = dev_f16(X), dev_f16(W), dev_f16(dY), dev_f16(Zs)
    check_fwd(kind, X, W, Xd, Wd)
    check_dgrad(kind, dY, W, Zs, dYd, Wd, Zd)


@pytest.mark.parametrize("kind", [mp.RELU, mp.GELU])
def test_fused_unaligned_and_strided(kind):
    """Row pitches that are not multiples of 8 and outputs inside wider buffers take the
    element-wise epilogue; nothing beyond the output columns is written."""
    require_gpu()
    M, N, K = 333, 270, 77
    X, W, dY, Zs = inputs(M, N, K + 0, 9 + kind)
    Xf = np.zeros((M, K + 3), np.uint16); Xf[:, :K] = X
    Wf = np.zeros((N, K + 5), np.uint16); Wf[:, :K] = W
    Zf = np.zeros((M, K + 1), np.uint16); Zf[:, :K] = Zs
    Xd, Wd, Zd = dev_f16(Xf)[:, :K], dev_f16(Wf)[:, :K], dev_f16(Zf)[:, :K]
    Zbuf = torch.full((M, N + 9), 7.0, dtype=torch.float16, device="cuda")
    Hbuf = torch.full((M, N + 1), 7.0, dtype=torch.float16, device="cuda")
    check_fwd(kind, X, W, Xd, Wd, Z=Zbuf[:, :N], H=Hbuf[:, :N])
    assert (Zbuf[:, N:] == 7.0).all() and (Hbuf[:, N:] == 7.0).all()
    dZbuf = torch.full((M, K + 2), 7.0, dtype=torch.float16, device="cuda")
    check_dgrad(kind, dY, W, Zs, dev_f16(dY), Wd, Zd, dZ=dZbuf[:, :K])
    assert (dZbuf[:, K:] == 7.0).all()


def test_fused_c4_layer_shape():
    """The benchmark's launch configuration: one 4096^3 GELU layer. Bitwise equal to the unfused
    pair over all 16.8M outputs; against the oracle on two full rows, two full columns and 4096
    random outputs."""
    require_gpu()
    n = 4096
    X, W, dY, Zs = inputs(n, n, n, 4096)
    Xd, Wd, dYd, Zd = dev_f16(X), dev_f16(W), dev_f16(dY), dev_f16(Zs)
    check_fwd(mp.GELU, X, W, Xd, Wd, ref="sample")
    check_dgrad(mp.GELU, dY, W, Zs, dYd, Wd, Zd, ref="sample")


def test_fused_direct_to_lds_ragged():
    """Ragged grids of 256 x 256 tiles whose whole tiles take the direct-to-LDS loop and whose
    edge tiles take the general loop, in both fused layers (forward 17 x 17 tiles, K = 2176;
    dgrad 17 x 9 tiles, reduction 4352): bitwise equal to the unfused pair, and against the
    oracle on two full rows, two full columns and 4096 random outputs."""
    require_gpu()
    M, N, K = 4100, 4352, 2176
    X, W, dY, Zs = inputs(M, N, K, 4352)
    Xd, Wd, dYd, Zd = dev_f16(X), dev_f16(W), dev_f16(dY), dev_f16(Zs)
    check_fwd(mp.GELU, X, W, Xd, Wd, ref="sample")
    check_dgrad(mp.GELU, dY, W, Zs, dYd, Wd, Zd, ref="sample")


def check_fwd_deriv(kind, X, W, Xd, Wd, ref=True):
    """H and D of the derivative-saving forward: the bits of act_fwd(Z) and act_bwd(Z, 1.0), Z
    the binary16 product; against the oracle's activation of its own product."""
    H, D = mp.linear_fwd_act_deriv(kind, Xd, Wd)
    Z = mp.linear_fwd(Xd, Wd)
    ones = torch.ones_like(Z)
    Hu, Du = mp.act_fwd(kind, Z), mp.act_bwd(kind, Z, ones)
    torch.cuda.synchronize()
    h, d, z = host_bits16(H), host_bits16(D), host_bits16(Z)
    assert np.array_equal(h, host_bits16(Hu)), "H differs from act_fwd of the product"
    assert np.array_equal(d, host_bits16(Du)), "D differs from act_bwd(Z, 1) of the product"
    if ref:
        if ref == "sample":
            r, c = sample_pts(*h.shape, 3)
            z_o = oracle.f32_to_f16(oracle.linear_fwd_at(X, W, r, c))
            h, d = h[r, c], d[r, c]
        else:
            z_o = oracle.linear_fwd(X, W, out_f16=True)
        assert rel_err(f16_values(h), f16_values(act_ref(kind, z_o))) <= TOL_F16
        d_o = act_grad_ref(kind, z_o, np.full_like(z_o, 0x3C00))
        if kind == mp.RELU:
            # a step function: compared where the oracle's product is far from 0 (the two
            # products differ by far less than 2^-8), which must be nearly every element
            far = np.abs(f16_values(z_o)) >= 2.0 ** -8
            assert far.mean() >= 0.99 and np.array_equal(d[far], d_o[far])
        else:
            assert rel_err(f16_values(d), f16_values(d_o)) <= TOL_F16


def check_dgrad_mul(kind, dY, W, Zs, dYd, Wd, Zd, ref=True):
    """dZ = RNE16(f32(dgrad product) * f32(D)): bitwise against torch's FP32 product of the
    same two binary16 GPU tensors rounded to half (round to nearest even); against the oracle's
    exact act'(Z) * (dY . W) from the generated inputs."""
    Dd = mp.act_bwd(kind, Zd.contiguous(), torch.ones_like(Zd.contiguous()))
    dZ = mp.linear_dgrad_mul(dYd, Wd, Dd)
    dH = mp.linear_dgrad(dYd, Wd)
    prod = (dH.float() * Dd.float()).half()
    torch.cuda.synchronize()
    out, r = host_bits16(dZ), host_bits16(prod)
    nan = np.isnan(f16_values(out)) & np.isnan(f16_values(r))
    assert np.array_equal(out[~nan], r[~nan]), "dZ differs from the FP32 product rounded to binary16"
    if ref == "sample":
        r, c = sample_pts(*out.shape, 4)
        dh_o = oracle.f32_to_f16(oracle.linear_dgrad_at(dY, W, r, c))
        dz_o = act_grad_ref(kind, np.ascontiguousarray(Zs[r, c]), dh_o)
        assert rel_err(f16_values(out[r, c]), f16_values(dz_o)) <= TOL_F16
    elif ref:
        dz_o = act_grad_ref(kind, np.ascontiguousarray(Zs), oracle.linear_dgrad(dY, W, out_f16=True))
        assert rel_err(f16_values(out), f16_values(dz_o)) <= TOL_F16


@pytest.mark.parametrize("kind", [mp.RELU, mp.GELU])
@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (64, 512, 256), (64, 10, 512), (300, 520, 200),
                                   (777, 1000, 333), (2600, 3100, 96), (1280, 1024, 384)])
def test_derivative_saving_layers(kind, M, N, K):
    """mp_linear_fwd_act_deriv and mp_linear_dgrad_mul on small (64 x 64 tiles) and large
    (256 x 256 tiles) grids, ragged in every dimension."""
    require_gpu()
    X, W, dY, Zs = inputs(M, N, K, M * 3 + N * 5 + K + kind)
    Xd, Wd, dYd, Zd = dev_f16(X), dev_f16(W), dev_f16(dY), dev_f16(Zs)
    check_fwd_deriv(kind, X, W, Xd, Wd)
    check_dgrad_mul(kind, dY, W, Zs, dYd, Wd, Zd)


@pytest.mark.parametrize("M,N,K", [(4100, 4352, 2176), (4096, 4096, 4096)])
def test_derivative_saving_layers_direct_to_lds(M, N, K):
    """GELU, on grids whose whole tiles take the direct-to-LDS loop (edge tiles the general one),
    and the benchmark's 4096^3 layer; against the oracle on sampled outputs."""
    require_gpu()
    X, W, dY, Zs = inputs(M, N, K, M + N + K)
    Xd, Wd, dYd, Zd = dev_f16(X), dev_f16(W), dev_f16(dY), dev_f16(Zs)
    check_fwd_deriv(mp.GELU, X, W, Xd, Wd, ref="sample")
    check_dgrad_mul(mp.GELU, dY, W, Zs, dYd, Wd, Zd, ref="sample")


def test_fused_argument_errors():
    require_gpu()
    a = torch.zeros((8, 8), dtype=torch.float16, device="cuda")
    with pytest.raises(mp.MPError):
        mp.linear_fwd_act(7, a, a)
    with pytest.raises(mp.MPError):
        mp.linear_dgrad_act(-1, a, a, a)
    with pytest.raises(ValueError):
        mp.linear_dgrad_act(mp.GELU, a, a, torch.zeros((8, 4), dtype=torch.float16, device="cuda"))
