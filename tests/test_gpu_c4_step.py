"""The C4 training step exactly as the benchmark runs it, at full size.

C4 is the 12-layer GELU MLP of width 4096 and batch 4096 (MSE to N(0,1) targets, dynamic loss
scale 2^16, SGD lr 0.01 momentum 0.9; "Mixed Precision Training", long-form analysis page,
§3.4 "The Integrated Training Procedure", Steps 1-7, with GELU layers and the calibrated loss
multiplier of the workload). One step of `bench.Model` runs on the GPU: the derivative-saving
GELU layers, the overflow flag from the weight-gradient epilogues, one update pass.

Against the oracle, which only ever sees the generated inputs, on 8 sampled batch rows (every
step but the weight gradients is row-local: a row of Z, H, D or dZ depends only on the same row
of the layer's input):
- the binary16 weights at step 0, bit for bit against the oracle's rounding of the masters;
- every forward layer against the oracle's own 12-layer chain from the generated X and weights:
  H = GELU(Z) and D = GELU'(Z) for layers 0-10 and Z for layer 11, within the dot-product bar
  (max error / max(|ref|, rms(ref)) <= 1e-2). Two chains that round differently at every layer
  drift apart but stay within 4.2e-3 of each other on this metric (measured between the oracle
  and an fp64-accumulating chain over the same rows);
- every activation gradient of the backward pass against the oracle's own backward chain from
  its own Z11: the scaled loss gradient dZ11 and dZ_l = GELU'(Z_l) * (dZ_{l+1} . W_{l+1}) for
  l = 10 .. 0 (Step 4), within 1.5e-2. Between the oracle and the fp64-accumulating chain this
  drift grows from 8.6e-4 (dZ11) to 6.0e-3 (dZ0).

Properties of the GPU's own outputs at any size (numpy, no oracle):
- the loss is c times the mean of (Z11 - T)^2 in float64 of the GPU's Z11, within 1e-5;
- every weight gradient dW_l = dZ_l^T . H_{l-1} (H_{-1} = X) on one full row, one full column
  and 2048 random entries against the float64 sum of the GPU's own binary16 dZ_l and H_{l-1},
  within the binary16 dot-product bar 1e-2;
- every weight gradient is finite (the flag stays clear) and the step is not skipped;
- the update, bit for bit in the order of the method's rule (one float32 rounding per
  operation: g = f32(g16) * 2^-16; g = g + wd * w; v = mu * v0 + g; w' = w - lr * v;
  w16 = RNE(w') by numpy's float16 cast; v0 = 0 at step 0), over all 201,326,592 parameters.

A second test poisons one target element with +inf, so the loss gradient, and through it every
layer's weight gradient, holds non-finite values: the flag from the weight-gradient epilogues
must make the step skip (masters, momenta and binary16 weights keep every bit) and halve S, as
the oracle's scaler does (Step 6; §3.4 "Choosing the Loss Scaling Factor", method 3).
"""
import gc

import numpy as np
import pytest
import torch

import bench
import mixed_precision_neural_amd as mp
import oracle
import workloads
from gpu_util import host_bits16, host_f32, rel_err, require_gpu

pytestmark = pytest.mark.gpu

BAR_FWD, BAR_BWD, BAR_WGRAD = 1e-2, 1.5e-2, 1e-2


class Recording(bench.Model):
    """bench.Model whose step also keeps a copy of every activation gradient it produces."""

    def __init__(self, *a):
        super().__init__(*a)
        self.dz = {}
        self._next = None

    def _t(self, kind, fn, *a, **k):
        r = fn(*a, **k)
        if kind == "loss":
            self.dz[bench.LAYERS - 1] = self.dA.clone()
            self._next = bench.LAYERS - 2
        elif kind == "dgrad_mul":
            self.dz[self._next] = k["dZ"].clone()
            self._next -= 1
        return r


def f16(bits):
    return np.asarray(bits, np.uint16).view(np.float16)


def free_gpu():
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


@pytest.mark.timeout(600)
def test_c4_step_as_benchmarked():
    require_gpu()
    torch.cuda.set_device(0)
    c = bench.calibration_c()
    w = workloads.c4()
    model = Recording(mp, torch, w, c)
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
    assert sorted(model.dz) == list(range(L))

    # the oracle's forward chain on sampled rows
    rng = np.random.Generator(np.random.PCG64(4))
    rows = np.unique(np.concatenate([[0, n - 1], rng.integers(0, n, 6)]))
    r_idx = np.repeat(np.arange(rows.size), n)
    c_idx = np.tile(np.arange(n), rows.size)
    inp = w.X16[rows]
    Zo = []
    for l in range(L):
        z = oracle.f32_to_f16(oracle.linear_fwd_at(inp, W16_ref[l], r_idx, c_idx).reshape(rows.size, n))
        Zo.append(z)
        if l == L - 1:
            e = rel_err(f16(host_bits16(model.Z[l])[rows]), f16(z))
            assert e <= BAR_FWD, (l, e)
            break
        h = oracle.gelu_fwd(z)
        d = oracle.gelu_bwd(z, np.full_like(z, 0x3C00))
        eh = rel_err(f16(host_bits16(model.H[l])[rows]), f16(h))
        ed = rel_err(f16(host_bits16(model.Z[l])[rows]), f16(d))   # saved GELU'(Z)
        assert eh <= BAR_FWD and ed <= BAR_FWD, (l, eh, ed)
        inp = h
    print("forward chain within the bar on rows", rows.tolist(), flush=True)

    # the oracle's backward chain on the same rows, from its own Z11: the scaled MSE gradient
    # (the mean over all 4096 x 4096 elements, so c is rescaled for the row subset), then
    # dZ_{l-1} = GELU'(Z_{l-1}) * (dZ_l . W_l)
    _, dz = oracle.mse(Zo[-1], w.T16[rows], c * rows.size / bench.BATCH, S0["scale"])
    errs = {}
    for l in range(L - 1, -1, -1):
        got = f16(host_bits16(model.dz[l][torch.from_numpy(rows).cuda()]))
        errs[l] = rel_err(got, f16(dz))
        if l == 0:
            break
        dh = oracle.linear_dgrad(dz, W16_ref[l], out_f16=True)
        dz = oracle.gelu_bwd(Zo[l - 1], dh)
    print("backward drift per layer:", {k: f"{v:.2e}" for k, v in sorted(errs.items())}, flush=True)
    assert max(errs.values()) <= BAR_BWD, errs

    # the loss on the GPU's output
    y = f16(host_bits16(model.Z[L - 1])).astype(np.float64)
    t = f16(w.T16).astype(np.float64)
    loss = c * float(np.mean((y - t) ** 2))
    assert abs(float(model.loss.cpu()[0]) - loss) <= 1e-5 * loss
    del y, t

    # every weight gradient on sampled entries, from the GPU's own binary16 operands
    for l in range(L):
        dZ = f16(host_bits16(model.dz[l])).astype(np.float64)
        H = f16(w.X16 if l == 0 else host_bits16(model.H[l - 1])).astype(np.float64)
        G = f16(host_bits16(model.G[l])).astype(np.float64)
        n0, k0 = int(rng.integers(0, n)), int(rng.integers(0, n))
        ns, ks = rng.integers(0, n, 2048), rng.integers(0, n, 2048)
        ref = np.concatenate([dZ[:, n0] @ H, dZ.T @ H[:, k0], np.einsum("mi,mi->i", dZ[:, ns], H[:, ks])])
        got = np.concatenate([G[n0, :], G[:, k0], G[ns, ks]])
        e = rel_err(got, ref)
        assert e <= BAR_WGRAD, (l, e)
    del dZ, H, G

    # the update from the GPU's gradients, one float32 rounding per operation of the rule
    lr, mu, wd = np.float32(w.lr), np.float32(w.momentum), np.float32(w.weight_decay)
    inv = np.float32(1.0 / S0["scale"])
    for l in range(L):
        g16 = f16(host_bits16(model.G[l]))
        assert np.all(np.isfinite(g16)), l
        w0 = w.masters[l]
        g = g16.astype(np.float32) * inv
        g = g + wd * w0
        v = mu * np.zeros_like(w0) + g
        w1 = w0 - lr * v
        assert np.array_equal(host_f32(model.V[l]).view(np.uint32), v.view(np.uint32)), l
        assert np.array_equal(host_f32(model.W[l]).view(np.uint32), w1.view(np.uint32)), l
        assert np.array_equal(host_bits16(model.W16[l]), w1.astype(np.float16).view(np.uint16)), l
    del model
    free_gpu()


@pytest.mark.timeout(300)
def test_c4_overflowing_step_is_skipped():
    require_gpu()
    torch.cuda.set_device(0)
    c = bench.calibration_c()
    w = workloads.c4()
    model = bench.Model(mp, torch, w, c)
    L = bench.LAYERS
    rng = np.random.Generator(np.random.PCG64(25))
    m0, n0 = int(rng.integers(0, bench.BATCH)), int(rng.integers(0, bench.WIDTH))
    print(f"C4 step with T[{m0}, {n0}] = +inf", flush=True)
    T_clean = model.T.clone()
    model.T[m0, n0] = float("inf")
    torch.cuda.synchronize()
    before = ([host_f32(x).view(np.uint32) for x in model.W], [host_f32(x).view(np.uint32) for x in model.V],
              [host_bits16(x) for x in model.W16])
    S0 = model.scaler.read()
    model.step()
    torch.cuda.synchronize()
    S1 = model.scaler.read()
    # the oracle's scaler on the same flag
    ref = oracle.scaler_update(oracle.scaler_init(S0["scale"], 1, w.growth_interval), 1)
    assert S1["scale"] == ref.scale == S0["scale"] / 2, (S1, ref.as_dict())
    assert S1["count"] == ref.count == 0 and S1["skipped_steps"] == ref.skipped_steps == 1
    assert S1["found_inf"] == 0
    # the loss gradient holds the +inf; weight gradients of every layer are non-finite somewhere
    assert not np.isfinite(float(model.loss.cpu()[0]))
    for l in range(L):
        g = host_bits16(model.G[l])
        assert ((g & 0x7C00) == 0x7C00).any(), l
    after = ([host_f32(x).view(np.uint32) for x in model.W], [host_f32(x).view(np.uint32) for x in model.V],
             [host_bits16(x) for x in model.W16])
    for a, b in zip(before, after):
        for l in range(L):
            assert np.array_equal(a[l], b[l]), l
    # the next clean step runs at the halved scale and is not skipped
    model.T.copy_(T_clean)
    model.step()
    torch.cuda.synchronize()
    S2 = model.scaler.read()
    ref2 = oracle.scaler_update(ref, 0)
    assert S2["scale"] == ref2.scale and S2["count"] == ref2.count == 1
    assert S2["skipped_steps"] == ref2.skipped_steps == 1
    assert not np.array_equal(host_f32(model.W[L - 1]).view(np.uint32), before[0][L - 1])
    del model
    free_gpu()
