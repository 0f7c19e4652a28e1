"""The C4 training step exactly as the benchmark runs it, at full size.

C4 is the 12-layer GELU MLP of width 4096 and batch 4096 (MSE to N(0,1) targets, dynamic loss
scale 2^16, SGD lr 0.01 momentum 0.9; "Mixed Precision Training", long-form analysis page,
§3.4 "The Integrated Training Procedure", Steps 1-7, with GELU layers and the calibrated loss
multiplier of the workload). One step of `bench.Model` runs on the GPU: the derivative-saving
GELU layers, the overflow flag from the weight-gradient epilogues, one update pass.

Against the oracle, which only ever sees the generated inputs:
- the binary16 weights at step 0, bit for bit against the oracle's rounding of the masters;
- every forward layer on 8 sampled batch rows against the oracle's own 12-layer chain from
  the generated X and weights: H = GELU(Z) and D = GELU'(Z) for layers 0-10 and Z for layer
  11, within the dot-product bar (max error / max(|ref|, rms(ref)) <= 1e-2). Two chains that
  round differently at every layer drift apart (by layer 11 most elements differ by an ulp
  or more) but stay within 4.2e-3 of each other on this metric (measured between the oracle
  and an fp64-accumulating chain over the same rows).

Properties of the GPU's own outputs at any size (numpy, no oracle):
- the loss is c times the mean of (Z11 - T)^2 in float64 of the GPU's Z11, within 1e-5;
- every weight gradient is finite (the flag stays clear) and the step is not skipped;
- the update, bit for bit in the order of the method's rule (one float32 rounding per
  operation: g = f32(g16) * 2^-16; g = g + wd * w; v = mu * v0 + g; w' = w - lr * v;
  w16 = RNE(w') by numpy's float16 cast; v0 = 0 at step 0), over all 201,326,592 parameters.
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


def test_c4_step_as_benchmarked():
    require_gpu()
    torch.cuda.set_device(0)
    c = bench.calibration_c()
    w = workloads.c4()
    model = bench.Model(mp, torch, w, c)
    assert model.gelu == "saved"
    L, n = bench.LAYERS, bench.WIDTH
    torch.cuda.synchronize()
    W16_ref = [oracle.f32_to_f16(m) for m in w.masters]
    for l in range(L):
        assert np.array_equal(host_bits16(model.W16[l]), W16_ref[l]), l
    S0 = model.scaler.read()
    print("C4 step: 12 layers of 4096^3, one benchmark step", flush=True)
    model.step()
    torch.cuda.synchronize()
    S1 = model.scaler.read()
    assert S1["skipped_steps"] == 0 and S1["found_inf"] == 0, S1
    assert S1["scale"] == S0["scale"] and S1["count"] == S0["count"] + 1

    # the oracle's forward chain on sampled rows
    rng = np.random.Generator(np.random.PCG64(4))
    rows = np.unique(np.concatenate([[0, n - 1], rng.integers(0, n, 6)]))
    r_idx = np.repeat(np.arange(rows.size), n)
    c_idx = np.tile(np.arange(n), rows.size)
    inp = w.X16[rows]
    for l in range(L):
        z = oracle.f32_to_f16(oracle.linear_fwd_at(inp, W16_ref[l], r_idx, c_idx).reshape(rows.size, n))
        if l == L - 1:
            e = rel_err(host_bits16(model.Z[l])[rows].view(np.float16), z.view(np.float16))
            assert e <= 1e-2, (l, e)
            break
        h = oracle.gelu_fwd(z)
        d = oracle.gelu_bwd(z, np.full_like(z, 0x3C00))
        eh = rel_err(host_bits16(model.H[l])[rows].view(np.float16), h.view(np.float16))
        ed = rel_err(host_bits16(model.Z[l])[rows].view(np.float16), d.view(np.float16))   # saved GELU'(Z)
        assert eh <= 1e-2 and ed <= 1e-2, (l, eh, ed)
        inp = h

    # the loss on the GPU's output
    y = host_bits16(model.Z[L - 1]).view(np.float16).astype(np.float64)
    t = w.T16.view(np.float16).astype(np.float64)
    loss = c * float(np.mean((y - t) ** 2))
    assert abs(float(model.loss.cpu()[0]) - loss) <= 1e-5 * loss

    # the update from the GPU's gradients, one float32 rounding per operation of the rule
    lr, mu, wd = np.float32(w.lr), np.float32(w.momentum), np.float32(w.weight_decay)
    inv = np.float32(1.0 / S0["scale"])
    for l in range(L):
        g16 = host_bits16(model.G[l]).view(np.float16)
        assert np.all(np.isfinite(g16)), l
        w0 = w.masters[l]
        g = g16.astype(np.float32) * inv
        g = g + wd * w0
        v = mu * np.zeros_like(w0) + g
        w1 = w0 - lr * v
        assert np.array_equal(host_f32(model.V[l]).view(np.uint32), v.view(np.uint32)), l
        assert np.array_equal(host_f32(model.W[l]).view(np.uint32), w1.view(np.uint32)), l
        assert np.array_equal(host_bits16(model.W16[l]), w1.astype(np.float16).view(np.uint16)), l
