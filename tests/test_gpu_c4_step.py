"""The C4 training step exactly as the benchmark runs it, checked against the oracle.

C4 is the 12-layer GELU MLP of width 4096 and batch 4096 (MSE to N(0,1) targets, dynamic loss
scale 2^16, SGD lr 0.01 momentum 0.9; "Mixed Precision Training", long-form analysis page,
§3.4 "The Integrated Training Procedure", Steps 1-7, with GELU layers and the calibrated loss
multiplier of the workload). One step of `bench.Model` (the derivative-saving GELU layers,
the overflow flag from the weight-gradient epilogues, one update pass) runs on the GPU; the
oracle then checks, teacher-forced on the GPU's own inputs of each call:

- every forward layer on 8 sampled batch rows: H = GELU(Z) and D = GELU'(Z) (11 layers) and
  the last layer's Z against RNE16 of the oracle's FP32 dot products, within the dot-product
  bar (max error / max(|ref|, rms(ref)) <= 1e-2; GELU and GELU' are 1.13- and 0.4-Lipschitz,
  so a binary16 rounding difference in Z moves them by less than the bar);
- the MSE loss (times the workload's multiplier c) within 1e-5 relative (FP32 sums of 16.7M
  terms);
- the last dgrad (dZ0 = RNE16(RNE16(dZ1 . W1) * D0)) on 8 sampled rows, and the two weight
  gradients whose input gradients are still resident after the step (layers 0 and 1) on
  4096 sampled entries each, within 1e-2;
- the whole optimizer sweep over the 201,326,592 parameters, bit for bit, from host
  snapshots taken before the step.
"""
import numpy as np
import pytest
import torch

import bench
import mixed_precision_neural_amd as mp
import oracle
import workloads
from gpu_util import host_bits16, host_f32, rel_err, require_gpu

pytestmark = pytest.mark.gpu


def f16_rne(x32: np.ndarray) -> np.ndarray:
    return oracle.f32_to_f16(np.ascontiguousarray(x32, np.float32))


def test_c4_step_as_benchmarked():
    require_gpu()
    torch.cuda.set_device(0)
    c = bench.calibration_c()
    w = workloads.c4()
    model = bench.Model(mp, torch, w, c)
    assert model.gelu == "saved"
    L, n = bench.LAYERS, bench.WIDTH
    torch.cuda.synchronize()
    W0 = [host_f32(m).copy() for m in model.W]
    V0 = [host_f32(v).copy() for v in model.V]
    W16_0 = [host_bits16(h).copy() for h in model.W16]
    S0 = model.scaler.read()
    print("C4 step: 12 layers of 4096^3, one benchmark step", flush=True)
    model.step()
    torch.cuda.synchronize()
    S1 = model.scaler.read()
    assert S1["skipped_steps"] == 0, S1

    rng = np.random.Generator(np.random.PCG64(4))
    rows = np.unique(np.concatenate([[0, n - 1], rng.integers(0, n, 6)]))
    r_idx = np.repeat(np.arange(rows.size), n)
    c_idx = np.tile(np.arange(n), rows.size)

    # forward, layer by layer, on the GPU's own inputs
    X = w.X16
    inp = X[rows]
    for l in range(L):
        z = f16_rne(oracle.linear_fwd_at(inp, W16_0[l], r_idx, c_idx).reshape(rows.size, n))
        if l == L - 1:
            got = host_bits16(model.Z[l])[rows]
            assert rel_err(got.view(np.float16), z.view(np.float16)) <= 1e-2, l
            break
        h_ref = oracle.gelu_fwd(z)
        d_ref = oracle.gelu_bwd(z, np.full_like(z, 0x3C00))
        h_gpu = host_bits16(model.H[l])[rows]
        d_gpu = host_bits16(model.Z[l])[rows]          # the saved GELU'(Z)
        eh = rel_err(h_gpu.view(np.float16), h_ref.view(np.float16))
        ed = rel_err(d_gpu.view(np.float16), d_ref.view(np.float16))
        assert eh <= 1e-2 and ed <= 1e-2, (l, eh, ed)
        inp = h_gpu

    # the MSE loss on the GPU's output
    loss_ref, _ = oracle.mse(host_bits16(model.Z[L - 1]), w.T16, c, S0["scale"])
    loss_gpu = float(model.loss.cpu()[0])
    assert abs(loss_gpu - loss_ref) <= 1e-5 * abs(loss_ref), (loss_gpu, loss_ref)

    # dZ1 sits in dA and dZ0 in dB after the step (the two buffers alternate from dZ11 = dA)
    dZ1 = host_bits16(model.dA)
    dZ0 = host_bits16(model.dB)
    D0 = host_bits16(model.Z[0])
    dh = f16_rne(oracle.linear_dgrad_at(dZ1[rows], W16_0[1], r_idx, c_idx).reshape(rows.size, n))
    dz_ref = f16_rne(dh.view(np.float16).astype(np.float32) * D0[rows].view(np.float16).astype(np.float32))
    assert rel_err(dZ0[rows].view(np.float16), dz_ref.view(np.float16)) <= 1e-2

    H0 = host_bits16(model.H[0])
    wi = rng.integers(0, n, 4096); wj = rng.integers(0, n, 4096)
    for l, dz, prev in ((0, dZ0, X), (1, dZ1, H0)):
        g_ref = f16_rne(oracle.linear_wgrad_at(dz, prev, wi, wj))
        g_gpu = host_bits16(model.G[l])[wi, wj]
        assert rel_err(g_gpu.view(np.float16), g_ref.view(np.float16)) <= 1e-2, l

    # the sweep, bit for bit, over every parameter
    G = [host_bits16(g).reshape(-1).copy() for g in model.G]
    Wm = [x.reshape(-1) for x in W0]
    Vm = [x.reshape(-1) for x in V0]
    H16 = [x.reshape(-1).copy() for x in W16_0]
    flag = oracle.step(Wm, Vm, G, H16, w.lr, w.momentum, w.weight_decay, 1.0 / S0["scale"])
    assert flag == 0
    for l in range(L):
        assert np.array_equal(host_f32(model.W[l]).reshape(-1).view(np.uint32), Wm[l].view(np.uint32)), l
        assert np.array_equal(host_f32(model.V[l]).reshape(-1).view(np.uint32), Vm[l].view(np.uint32)), l
        assert np.array_equal(host_bits16(model.W16[l]).reshape(-1), H16[l]), l
    assert S1["scale"] == S0["scale"] and S1["count"] == S0["count"] + 1
