"""Benchmark of the mixed-precision training hot path on one MI355X.

One step = one full training step of the 12-layer GELU MLP (width 4096, batch 4096, MSE
loss to N(0,1) targets, FP16 storage, FP32 master weights and momentum, dynamic loss
scale starting at 2^16, SGD lr 0.01 momentum 0.9), i.e. every step of the method:
12 forward GEMMs, the scaled loss gradient, 12 weight-gradient and 11 activation-gradient
GEMMs, GELU and its derivative in the forward and dgrad epilogues (--gelu chooses how), the
optimizer sweep (overflow flag from the weight-gradient epilogues + one fused update pass over
201,326,592 parameters) and the scaler update. Inputs are synthetic, generated from seed 0,
and resident in HBM before the timed region starts. After the timed steps the line also
reports the other sweeps (Nesterov, Adagrad, two-pass), the |g| maximum, the large
reductions at the pages' sizes and the 2-layer MLP step's latency, eager and as a HIP graph.

Prints one JSON line. `value` is the GEMM throughput of the whole step (35 x 2 x 4096^3
FLOP per step / step time). `roofline` is for the GEMM kernel with the largest share of
the step, timed per launch with HIP events on the stream it runs on, over as many further
steps of the same workload as were timed (the timed steps themselves carry no per-launch
events, which would add queue markers to them); the sweep's HBM figures are reported beside
it. `cpu_baseline` times the CPU oracle on a bounded sample.
"""
from __future__ import annotations

import argparse
import gc
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "mp_step HBM GB/s + FP16/FP32-acc GEMM TFLOP/s, % of roofline, 1 MI355X"
PEAK_F16_TFLOPS = 2500.0          # MI355X dense FP16 MFMA
PEAK_HBM_GBPS = 8000.0            # MI355X HBM3E
WIDTH, BATCH, LAYERS = 4096, 4096, 12
SWEEP_BYTES_PER_PARAM = 20        # read g16 2 + w32 4 + v32 4, write w32 4 + v32 4 + w16 2
CHECK_BYTES_PER_PARAM = 2

# HBM-side bytes per launch from two rocprofv3 counter passes (FETCH_SIZE, then WRITE_SIZE, KiB
# per dispatch) over `bench.py --pmc-kernel <kind>`, at the bench's shapes. FETCH_SIZE reads half
# of the bytes a 1 GiB device copy moves and WRITE_SIZE all of them (`--pmc-kernel copy`), so the
# fetch figure is scaled by 2.0 and the write figure by 1.0. A figure holds only for the kernel
# source it was taken on: it is reported while the SHA-256 of those files still matches.
MEASURED_TRAFFIC = {
    "gemm": {"src": ["mp_gemm.hip", "mp_internal.h", "mp_act.h"],
             "sha256": "88fe50202f528eabafbfc0f38ef0fc6ba93db2c600812408147a641ac145ac78",
             "fwd": (98408.8, 32768.0), "fwd_act": (98481.7, 65536.0), "fwd_act_deriv": (98481.7, 65536.0),
             "dgrad_act": (114881.7, 32768.0), "dgrad_mul": (114808.5, 32768.0), "wgrad": (99453.4, 34816.0)},
    "update": {"src": ["mp_step.hip", "mp_internal.h"],
               "sha256": "675c7fca4abd374d5d1b1b91fee77a9c901bae463135c0c340572a03a10262f0",
               "update": (990844.1, 1972212.6), "nesterov": (990309.5, 1973116.0),
               "adagrad": (993440.6, 1969707.7)},
    "reduce": {"src": ["mp_reduce.hip", "mp_internal.h"],
               "sha256": "7109d62b3a4136e5de1a2c9267a43d3256f6dc012907ce095ee3a597a257069b",
               "bn_stats": (25340.3, 2021.7), "bn_apply": (25140.9, 50176.0), "softmax": (50773.2, 99331.0)},
    "stats": {"src": ["mp_stats.hip", "mp_internal.h"],
              "sha256": "4857ba544bf243d20e031caef561c1a496e998549740a7590313207240144019",
              "absmax": (394786.6, 7.5)},
}
FETCH_SCALE, WRITE_SCALE = 2.0, 1.0
# Matrix-core occupancy and shader clock of the 4096^3 GEMM kernels from one rocprofv3 counter pass each
# (SQ_VALU_MFMA_BUSY_CYCLES, SQ_BUSY_CU_CYCLES with the dispatch's start and end times, over
# `bench.py --pmc-kernel <kind>`): busy = MFMA-busy cycles / (4 SIMDs x CU-busy cycles), clock = CU-busy
# cycles per CU / kernel duration. Like MEASURED_TRAFFIC, reported while the GEMM sources are unchanged.
MEASURED_MFMA = {"sha256": MEASURED_TRAFFIC["gemm"]["sha256"],
                 "fwd": (0.827, 1437.0), "fwd_act_deriv": (0.720, 1492.0), "dgrad_mul": (0.818, 1400.0),
                 "wgrad": (0.839, 1398.0)}
# The large reductions at the pages' sizes: batch normalization over 32 images x 112 x 112
# positions x 64 channels, and the softmax over the 793,471-word vocabulary (64 rows, row pitch
# rounded up to 8 elements).
BN_ROWS, BN_CH = 32 * 112 * 112, 64
SM_ROWS, SM_COLS = 64, 793471


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-rows", type=int, default=32, help="batch rows of the oracle's sample step")
    p.add_argument("--gelu", choices=["saved", "recompute", "separate"], default="saved",
                   help="saved: the forward epilogue stores GELU(Z) and GELU'(Z), the dgrad epilogue "
                        "multiplies; recompute: the forward stores Z, the dgrad epilogue evaluates "
                        "GELU'(Z); separate: point-wise kernels beside plain GEMMs")
    p.add_argument("--unfused", action="store_true", help="the same as --gelu separate")
    p.add_argument("--pmc-kernel", choices=["fwd", "fwd_act", "fwd_act_deriv", "dgrad", "dgrad_act", "dgrad_mul",
                            "wgrad", "update", "update_nesterov",
                            "update_adagrad", "absmax", "bn_stats", "bn_apply", "softmax", "copy"],
                   help="only launch this kernel --pmc-reps times at the bench's shape (for counter passes)")
    p.add_argument("--pmc-reps", type=int, default=3)
    return p.parse_args()


def source_sha256(files) -> str:
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "mixed_precision_neural_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(group: str, kind: str):
    """Per-launch HBM bytes of the counter passes, or None once the kernel source has changed."""
    t = MEASURED_TRAFFIC[group]
    if source_sha256(t["src"]) != t["sha256"] or kind not in t:
        return None
    fetch_kib, write_kib = t[kind]
    return round((fetch_kib * FETCH_SCALE + write_kib * WRITE_SCALE) * 1024)


def measured_mfma(kind: str):
    """(MFMA-busy fraction, shader MHz) of a GEMM kind from the counter pass, or (None, None) once
    the GEMM sources have changed."""
    if source_sha256(MEASURED_TRAFFIC["gemm"]["src"]) != MEASURED_MFMA["sha256"] or kind not in MEASURED_MFMA:
        return None, None
    return MEASURED_MFMA[kind]


def pmc_kernel(args, mp, torch):
    """Launches one kernel kind a few times at the bench's shapes and nothing else of note."""
    n = WIDTH
    if args.pmc_kernel in ("fwd", "fwd_act", "fwd_act_deriv", "dgrad", "dgrad_act", "dgrad_mul", "wgrad"):
        g = torch.Generator(device="cuda").manual_seed(0)
        A = torch.randn(n, n, device="cuda", generator=g).half()
        B = torch.randn(n, n, device="cuda", generator=g).half()
        C = torch.empty(n, n, device="cuda", dtype=torch.float16)
        D = torch.randn(n, n, device="cuda", generator=g).half()
        flag = torch.zeros(1, dtype=torch.int32, device="cuda")
        f = {"fwd": lambda: mp.linear_fwd(A, B, Y=C),
             "fwd_act": lambda: mp.linear_fwd_act(mp.GELU, A, B, Z=C, H=D),
             "fwd_act_deriv": lambda: mp.linear_fwd_act_deriv(mp.GELU, A, B, H=C, D=D),
             "dgrad": lambda: mp.linear_dgrad(A, B, dX=C),
             "dgrad_act": lambda: mp.linear_dgrad_act(mp.GELU, A, B, D, dZ=C),
             "dgrad_mul": lambda: mp.linear_dgrad_mul(A, B, D, dZ=C),
             "wgrad": lambda: mp.linear_wgrad(A, B, dW=C, found_inf=flag)}[args.pmc_kernel]
    elif args.pmc_kernel.startswith("update"):
        N = LAYERS * n * n
        w = torch.randn(N, device="cuda"); v = torch.zeros(N, device="cuda")
        gr = (torch.randn(N, device="cuda") * 1e-3).half(); h = torch.empty(N, device="cuda", dtype=torch.float16)
        S = mp.Scaler(65536.0, True); pl = mp.ParamList([w], [v], [gr], [h])
        kind = {"update": mp.SGD, "update_nesterov": mp.NESTEROV, "update_adagrad": mp.ADAGRAD}[args.pmc_kernel]
        f = lambda: mp.step_opt(pl, S, kind, 0.01, 0.9, 0.0, 1e-10, flags=mp.MP_GRADS_PRECHECKED)
    elif args.pmc_kernel == "absmax":
        x = torch.randn(LAYERS * n * n, device="cuda")
        tl = mp.TensorList([x]); amax = torch.zeros(1, device="cuda")
        f = lambda: mp.absmax(tl, amax)
    elif args.pmc_kernel in ("bn_stats", "bn_apply", "softmax"):
        f = reduction_calls(mp, torch)[args.pmc_kernel]
    else:                                   # calibration: 1 GiB read + 1 GiB written per launch
        x = torch.randn(256 * 1024 * 1024, device="cuda"); y = torch.empty_like(x)
        f = lambda: y.copy_(x)
    for _ in range(args.pmc_reps):
        f()
    torch.cuda.synchronize()
    print(json.dumps({"pmc_kernel": args.pmc_kernel, "launches": args.pmc_reps}), flush=True)


def reduction_calls(mp, torch) -> dict:
    """One call of each large reduction on synthetic inputs of the pages' sizes (outputs
    preallocated; the first call of each is made here, untimed)."""
    g = torch.Generator(device="cuda").manual_seed(1)
    x = (torch.randn(BN_ROWS, BN_CH, device="cuda", generator=g) * 2.0 + 0.5).half()
    mean = torch.empty(BN_CH, device="cuda"); var = torch.empty(BN_CH, device="cuda")
    gamma = torch.ones(BN_CH, device="cuda"); beta = torch.zeros(BN_CH, device="cuda")
    y = torch.empty_like(x)
    ld = (SM_COLS + 7) // 8 * 8
    xs = (torch.randn(SM_ROWS, ld, device="cuda", generator=g) * 3.0).half()[:, :SM_COLS]
    ys = torch.empty(SM_ROWS, ld, device="cuda", dtype=torch.float16)[:, :SM_COLS]
    calls = {"bn_stats": lambda: mp.bn_stats(x, mean, var),
             "bn_apply": lambda: mp.bn_apply(x, mean, var, gamma, beta, 1e-5, y=y),
             "softmax": lambda: mp.softmax(xs, y=ys)}
    for f in calls.values():
        f()
    return calls


def gemm_backlog(mp, torch, count: int = 8):
    """Returns a function that queues `count` 4096^3 forward GEMMs (~1 ms of GPU work) on the
    current stream. Queued ahead of short timed calls, it keeps the GPU busy while the host
    issues them, so the host's per-call cost does not show up as idle time inside a pair of
    events."""
    a = torch.randn(WIDTH, WIDTH, device="cuda").half()
    b = torch.randn(WIDTH, WIDTH, device="cuda").half()
    c = torch.empty(WIDTH, WIDTH, device="cuda", dtype=torch.float16)

    def run():
        for _ in range(count):
            mp.linear_fwd(a, b, Y=c)
    return run


def c1_latency(mp, torch, workloads, steps: int = 200) -> dict:
    """The 2-layer MLP step (256 -> 512 -> 10, batch 64, fused ReLU epilogues, flag from the
    weight-gradient epilogues): nine launches of microsecond kernels, so the host's launch
    cost bounds it. Timed eagerly and as replays of one captured HIP graph, `steps` each."""
    cfg = workloads.c1()
    f16 = torch.float16
    S = mp.Scaler(cfg.scale, cfg.dynamic, cfg.growth_interval)
    W = [torch.from_numpy(cfg.W1).cuda(), torch.from_numpy(cfg.W2).cuda()]
    V = [torch.zeros_like(w) for w in W]
    W16 = [mp.round_f32_to_f16(w) for w in W]
    G = [torch.zeros(w.shape, dtype=f16, device="cuda") for w in W]
    pl = mp.ParamList(W, V, G, W16)
    import numpy as np
    X = torch.from_numpy(cfg.X16.view(np.int16)).cuda().view(f16)
    y = torch.from_numpy(cfg.labels).cuda()
    Z1 = torch.empty((64, 512), dtype=f16, device="cuda")
    H1, dZ1 = torch.empty_like(Z1), torch.empty_like(Z1)
    Z2 = torch.empty((64, 10), dtype=f16, device="cuda")
    dZ2 = torch.empty_like(Z2)
    loss = torch.zeros(1, dtype=torch.float32, device="cuda")
    ws = torch.empty(mp.loss_softmax_ce_workspace(64, 10), dtype=torch.uint8, device="cuda")

    def step():
        mp.linear_fwd_act(mp.RELU, X, W16[0], Z=Z1, H=H1)
        mp.linear_fwd(H1, W16[1], Y=Z2)
        mp.loss_softmax_ce(Z2, y, S, loss, dZ2, workspace=ws)
        mp.linear_wgrad(dZ2, H1, dW=G[1], found_inf=S.found_inf_ptr)
        mp.linear_dgrad_act(mp.RELU, dZ2, W16[1], Z1, dZ=dZ1)
        mp.linear_wgrad(dZ1, X, dW=G[0], found_inf=S.found_inf_ptr)
        mp.step(pl, S, cfg.lr, cfg.momentum, cfg.weight_decay, flags=mp.MP_GRADS_PRECHECKED)
        S.update()

    def timed(fn):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps * 1e3

    for _ in range(10):
        step()
    eager_us = timed(step)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for _ in range(10):
        g.replay()
    graph_us = timed(g.replay)
    st = S.read()
    pl.close()
    return {"workload": "C1: 2-layer MLP 256->512->10, batch 64, ReLU, softmax-CE, static scale 1024",
            "launches_per_step": 9, "eager_us": round(eager_us, 2), "graph_us": round(graph_us, 2),
            "steps": steps, "skipped_steps": st["skipped_steps"]}


def reductions(model, mp, torch) -> dict:
    """The large reductions, each queued behind ~1 ms of GEMMs (a call takes tens of
    microseconds, about what the host needs to issue one, so the backlog keeps the GPU busy
    while the host issues them): the time per call of 10 calls back to back between one pair of
    HIP events (`avg_us`, which the GB/s and fractions use), and the mean of 10 calls each
    between its own pair (`per_call_events_us`, which adds the event records). GB/s on the
    algorithmic bytes (statistics: 2 B per value read; normalization and softmax: 2 read + 2
    written). At the bench's shape the softmax takes its single-read form (x read once)."""
    calls = reduction_calls(mp, torch)
    backlog = gemm_backlog(mp, torch)
    out = {}
    for name, f in calls.items():
        model.start_events(10)
        backlog()
        for _ in range(10):
            model._t(name, f)
        torch.cuda.synchronize()
        per_call = model.kernel_ms()[name]["avg_ms"]
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        backlog()
        e0.record()
        for _ in range(10):
            f()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / 10
        n = BN_ROWS * BN_CH if name != "softmax" else SM_ROWS * SM_COLS
        nbytes = (2 if name == "bn_stats" else 4) * n
        gbps = nbytes / (ms * 1e-3) / 1e9
        out[name] = {"shape": [BN_ROWS, BN_CH] if name != "softmax" else [SM_ROWS, SM_COLS],
                     "avg_us": round(ms * 1e3, 2), "per_call_events_us": round(per_call * 1e3, 2),
                     "achieved_GBps": round(gbps, 1), "frac": round(gbps / PEAK_HBM_GBPS, 4),
                     "algorithmic_bytes": nbytes, "traffic": measured_traffic("reduce", name)}
    return out


def _event_avg_ms(torch, fn, reps: int, before=None) -> float:
    """Mean of `reps` launches of fn, each between two HIP events on the current stream (the
    stream the kernels run on); `before` runs untimed ahead of each launch."""
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    torch.cuda.synchronize()
    for a, b in pairs:
        if before is not None:
            before()
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    return sum(a.elapsed_time(b) for a, b in pairs) / reps


def hbm_ceiling(torch, probe, gib: int = 4) -> dict:
    """Achievable HBM rates over `gib` GiB with the stream probe (read only, write only, 1:1 copy),
    the best of eight launch shapes each (one block per 16 KiB or 1024-4096 persistent blocks;
    temporal or non-temporal accesses), 5 timed launches per shape."""
    nbytes = gib << 30
    src = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    dst = torch.empty_like(src)
    out = {}
    for mode, name, moved in ((probe.READ, "read", nbytes), (probe.WRITE, "write", nbytes),
                              (probe.COPY, "copy", 2 * nbytes)):
        best = None
        for blocks in (0, 1024, 2048, 4096):
            for nt in (False, True):
                f = lambda: probe.hbm(mode, src, dst, nbytes, blocks, nt)
                f()
                ms = _event_avg_ms(torch, f, 5)
                gbps = moved / (ms * 1e-3) / 1e9
                if best is None or gbps > best[0]:
                    best = (gbps, blocks, nt, ms)
        out[name] = {"GBps": round(best[0], 1), "frac": round(best[0] / PEAK_HBM_GBPS, 4),
                     "blocks": best[1] or "one per 16 KiB", "nontemporal": best[2],
                     "us": round(best[3] * 1e3, 1)}
    out["bytes"] = nbytes
    del src, dst
    return out


def mfma_clock(torch, probe, operands: int, shape: int, blocks: int = 256, ms_target: float = 25.0) -> dict:
    """The shader clock and the MFMA rate under a pure binary16 matrix-core load (one block of four
    waves per CU, independent MFMA chains, 16 x 32768 FLOP a round) of the form `shape`, with
    near-constant operands (probe.CONSTANT) or random ones like a GEMM's (probe.RANDOM)."""
    out_t = torch.zeros(4 * blocks, dtype=torch.int64, device="cuda")
    iters = 1000
    probe.mfma_clock(blocks, iters, out_t, operands, shape)       # warm-up and sizing
    ms = _event_avg_ms(torch, lambda: probe.mfma_clock(blocks, iters, out_t, operands, shape), 1)
    iters = max(1000, int(iters * ms_target / max(ms, 1e-3)))
    khz = probe.mfma_clock(blocks, iters, out_t, operands, shape)
    ms = _event_avg_ms(torch, lambda: probe.mfma_clock(blocks, iters, out_t, operands, shape), 1)
    t = out_t.cpu().numpy().reshape(blocks, 4).astype("float64")
    mhz = (t[:, 1] - t[:, 0]) / (t[:, 3] - t[:, 2]) * khz / 1000.0
    flop = blocks * 4 * iters * 16 * 2.0 * 32 * 32 * 16
    tf = flop / (ms * 1e-3) / 1e12
    mhz_med = float(sorted(mhz)[len(mhz) // 2])
    return {"clock_mhz": round(mhz_med, 1), "clock_mhz_min": round(float(mhz.min()), 1),
            "mfma_f16_TFLOPs": round(tf, 1), "frac_of_spec": round(tf / PEAK_F16_TFLOPS, 4),
            "clock_adjusted_peak_TFLOPs": round(PEAK_F16_TFLOPS * mhz_med / 2400.0, 1),
            "kernel_ms": round(ms, 3), "realtime_khz": khz,
            "load": f"{blocks} blocks x 4 waves, {iters} rounds of 16 x 32768 FLOP per wave"}


def sweep_config(mp, torch, name, tensors, scale, hyper, inject, reps, copy_gbps) -> dict:
    """The optimizer sweep over `tensors` (list of (w32, v32, g16, w16)) timed four ways: the two-
    pass step update-only callers use (check pass + update pass), the single update pass
    (MP_GRADS_PRECHECKED), the check pass alone (MP_CHECK_ONLY), and a step whose gradients hold
    the injected non-finite values (the check finds them, the update pass leaves at once)."""
    W, V, G, H = (list(x) for x in zip(*tensors))
    n = sum(w.numel() for w in W)
    pl = mp.ParamList(W, V, G, H)
    S = mp.Scaler(scale, True, 2000)
    lr, mu, wd = hyper
    mp.step(pl, S, lr, mu, wd)                            # untimed: waits for the list's upload
    S.update()
    two = _event_avg_ms(torch, lambda: mp.step(pl, S, lr, mu, wd), reps)
    one = _event_avg_ms(torch, lambda: mp.step(pl, S, lr, mu, wd, flags=mp.MP_GRADS_PRECHECKED), reps)
    chk = _event_avg_ms(torch, lambda: mp.step(pl, S, lr, mu, wd, flags=mp.MP_CHECK_ONLY), reps)
    restore = inject()
    reset = lambda: S.init(scale, True, 2000)
    skip = _event_avg_ms(torch, lambda: mp.step(pl, S, lr, mu, wd), reps, before=reset)
    st = S.read()
    restore()
    pl.close()
    alg = SWEEP_BYTES_PER_PARAM * n
    gb = lambda ms: alg / (ms * 1e-3) / 1e9
    return {"workload": name, "params": n, "tensors": len(W), "algorithmic_bytes": alg,
            "two_pass_us": round(two * 1e3, 1), "two_pass_GBps": round(gb(two), 1),
            "two_pass_frac": round(gb(two) / PEAK_HBM_GBPS, 4),
            "one_pass_us": round(one * 1e3, 1), "one_pass_GBps": round(gb(one), 1),
            "one_pass_frac": round(gb(one) / PEAK_HBM_GBPS, 4),
            "one_pass_frac_of_copy_ceiling": round(gb(one) / copy_gbps, 4) if copy_gbps else None,
            "check_only_us": round(chk * 1e3, 1),
            "check_only_GBps": round(CHECK_BYTES_PER_PARAM * n / (chk * 1e-3) / 1e9, 1),
            "skipped_step_us": round(skip * 1e3, 1), "skipped_flag": st["found_inf"]}


def c2_sweep(mp, torch, copy_gbps, reps=10, n=100_000_000) -> dict:
    """C2: one flat tensor of 10^8 parameters; w ~ N(0, 0.02^2), v = 0, g = RNE16(2^15 * sign *
    2^U(-34, -4)); +inf at one seeded index for the skipped step. Drawn on the GPU (the same
    distributions as the parity inputs; timing does not depend on the draw)."""
    g = torch.Generator(device="cuda").manual_seed(2)
    w = torch.randn(n, device="cuda", generator=g) * 0.02
    v = torch.zeros(n, device="cuda")
    u = torch.rand(n, device="cuda", generator=g) * 30.0 - 34.0
    sign = torch.randint(0, 2, (n,), device="cuda", generator=g).float() * 2 - 1
    g16 = (sign * torch.exp2(u) * 2.0 ** 15).half()
    del u, sign
    h = torch.empty(n, dtype=torch.float16, device="cuda")
    idx = int(torch.randint(0, n, (1,), generator=torch.Generator().manual_seed(25)))

    def inject():
        old = g16[idx].clone()
        g16[idx] = float("inf")
        return lambda: g16[idx].copy_(old)
    out = sweep_config(mp, torch, "C2: one tensor of 10^8 parameters, SGD lr 0.01 momentum 0.9, S = 2^15",
                       [(w, v, g16, h)], 2.0 ** 15, (0.01, 0.9, 0.0), inject, reps, copy_gbps)
    out["_host"] = (w, v, g16, h)
    return out


def c5_sweep(mp, torch, workloads, copy_gbps, reps=5) -> dict:
    """C5: 500 ragged tensors (log-uniform sizes rescaled to 1.5e9 parameters), w ~ N(0, 0.02^2),
    v = 0, log2|g| ~ N(-20, 2.43^2) times S = 2^12, 0.1 % NaN for the skipped step; SGD lr 1e-3
    momentum 0.9 weight decay 1e-4. Drawn on the GPU per tensor."""
    sizes = workloads.c5_sizes()
    g = torch.Generator(device="cuda").manual_seed(5)
    tensors = []
    for sz in sizes.tolist():
        w = torch.randn(sz, device="cuda", generator=g) * 0.02
        e = torch.randn(sz, device="cuda", generator=g) * workloads.C5_LOG2_SIGMA + workloads.C5_LOG2_MEDIAN
        sign = torch.randint(0, 2, (sz,), device="cuda", generator=g).float() * 2 - 1
        g16 = (sign * torch.exp2(e) * 2.0 ** 12).half()
        del e, sign
        tensors.append((w, torch.zeros_like(w), g16, torch.empty(sz, dtype=torch.float16, device="cuda")))
    torch.cuda.synchronize()

    def inject():
        saved = []
        for (_, _, g16, _) in tensors:
            m = torch.rand(g16.numel(), device="cuda", generator=g) < 1e-3
            saved.append((g16, m, g16[m].clone()))
            g16[m] = float("nan")

        def restore():
            for g16, m, old in saved:
                g16[m] = old
        return restore
    out = sweep_config(mp, torch, "C5: 500 ragged tensors, 1.5e9 parameters, SGD lr 1e-3 momentum 0.9 "
                       "weight decay 1e-4, S = 2^12", tensors, 2.0 ** 12, (1e-3, 0.9, 1e-4), inject, reps,
                       copy_gbps)
    out["_host"] = tensors
    return out


def c3_gemms(mp, torch, reps=25, M=8192, N=4096, K=4096) -> dict:
    """C3: one linear layer of 8192 tokens, 4096 -> 4096: forward, dgrad and wgrad with binary16
    outputs, each over `reps` launches after untimed ones (fifteen rounds of all three first, ~9 ms,
    then three of the kind: the chip's clock settles to the load over several milliseconds, and
    with five rounds the kind timed first still ran ~10 % slow). X, dY ~ N(0,1),
    W ~ N(0, 1/64^2)."""
    g = torch.Generator(device="cuda").manual_seed(3)
    X = torch.randn(M, K, device="cuda", generator=g).half()
    dY = torch.randn(M, N, device="cuda", generator=g).half()
    W = (torch.randn(N, K, device="cuda", generator=g) / 64.0).half()
    Y = torch.empty(M, N, dtype=torch.float16, device="cuda")
    dX = torch.empty(M, K, dtype=torch.float16, device="cuda")
    dW = torch.empty(N, K, dtype=torch.float16, device="cuda")
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    calls = {"fwd": lambda: mp.linear_fwd(X, W, Y=Y), "dgrad": lambda: mp.linear_dgrad(dY, W, dX=dX),
             "wgrad": lambda: mp.linear_wgrad(dY, X, dW=dW, found_inf=flag)}
    flop = 2.0 * M * N * K
    out = {"workload": f"C3: M={M} tokens, N={N}, K={K}, binary16 in and out, FP32 accumulation",
           "gflop_per_launch": round(flop / 1e9, 2)}
    for _ in range(15):                  # the GEMMs follow microsecond kernels: bring the chip to this load first
        for f in calls.values():
            f()
    for k, f in calls.items():
        for _ in range(3):
            f()
        ms = _event_avg_ms(torch, f, reps)
        tf = flop / (ms * 1e-3) / 1e12
        out[k] = {"us": round(ms * 1e3, 2), "TFLOPs": round(tf, 1), "frac": round(tf / PEAK_F16_TFLOPS, 4)}
    out["_host"] = (X, dY, W)
    return out


def cpu_c1_step(workloads, reps: int = 20) -> dict:
    """The oracle's C1 training step (forward with ReLU, softmax-CE at S = 1024, wgrad and dgrad of
    both layers, the sweep over 136,192 parameters), averaged over `reps` steps from the C1 inputs."""
    import numpy as np

    import oracle
    cfg = workloads.c1()
    W = [cfg.W1.reshape(-1).copy(), cfg.W2.reshape(-1).copy()]
    V = [np.zeros_like(w) for w in W]
    W16 = [oracle.f32_to_f16(w) for w in W]
    t0 = time.perf_counter()
    for _ in range(reps):
        w1, w2 = W16[0].reshape(512, 256), W16[1].reshape(10, 512)
        z1 = oracle.linear_fwd(cfg.X16, w1, out_f16=True)
        h1 = oracle.relu_fwd(z1)
        z2 = oracle.linear_fwd(h1, w2, out_f16=True)
        _, dz2 = oracle.softmax_ce(z2, cfg.labels, cfg.scale)
        g2 = oracle.linear_wgrad(dz2, h1, out_f16=True)
        dz1 = oracle.relu_bwd(z1, oracle.linear_dgrad(dz2, w2, out_f16=True))
        g1 = oracle.linear_wgrad(dz1, cfg.X16, out_f16=True)
        oracle.step(W, V, [g1.reshape(-1), g2.reshape(-1)], W16, cfg.lr, cfg.momentum, cfg.weight_decay,
                    1.0 / cfg.scale)
    dt = (time.perf_counter() - t0) / reps
    return {"sample": f"the full C1 step, {reps} steps", "us_per_step": round(dt * 1e6, 1),
            "cores": oracle.threads()}


def cpu_configs(c2, c3, c5) -> dict:
    """The oracle on bounded samples of C2, C3 and C5 (CPU threads of the host)."""
    import numpy as np

    import oracle
    res = {}
    w, v, g16, h = c2.pop("_host")
    hw, hv = w.cpu().numpy().copy(), v.cpu().numpy().copy()
    hg = g16.cpu().numpy().view(np.uint16).copy()
    hh = h.cpu().numpy().view(np.uint16).copy()
    t0 = time.perf_counter()
    oracle.step([hw], [hv], [hg], [hh], 0.01, 0.9, 0.0, 2.0 ** -15)
    dt = time.perf_counter() - t0
    res["c2"] = {"sample": "the full C2 step (two passes: check, then update) over 10^8 parameters",
                 "seconds": round(dt, 3), "GBps": round(SWEEP_BYTES_PER_PARAM * hw.size / dt / 1e9, 2)}
    del hw, hv, hg, hh
    tensors = c5.pop("_host")
    sel, total = [], 0
    for t in tensors:
        if total >= 100_000_000:
            break
        sel.append(t); total += t[0].numel()
    hw = [t[0].cpu().numpy().copy() for t in sel]
    hv = [t[1].cpu().numpy().copy() for t in sel]
    hg = [t[2].cpu().numpy().view(np.uint16).copy() for t in sel]
    hh = [np.zeros(t[0].numel(), np.uint16) for t in sel]
    t0 = time.perf_counter()
    oracle.step(hw, hv, hg, hh, 1e-3, 0.9, 1e-4, 2.0 ** -12)
    dt = time.perf_counter() - t0
    res["c5"] = {"sample": f"the C5 step over its first {len(sel)} tensors ({total} parameters)",
                 "seconds": round(dt, 3), "GBps": round(SWEEP_BYTES_PER_PARAM * total / dt / 1e9, 2)}
    del hw, hv, hg, hh
    X, dY, W = (np.ascontiguousarray(t.cpu().numpy().view(np.uint16)) for t in c3.pop("_host"))
    rows = 16
    t0 = time.perf_counter(); oracle.linear_fwd(X[:rows], W, out_f16=True); t_f = time.perf_counter() - t0
    t0 = time.perf_counter(); oracle.linear_dgrad(dY[:rows], W, out_f16=True); t_d = time.perf_counter() - t0
    rng = np.random.Generator(np.random.PCG64(6))
    pts = 32768
    r, cc = rng.integers(0, W.shape[0], pts), rng.integers(0, W.shape[1], pts)
    t0 = time.perf_counter(); oracle.linear_wgrad_at(dY, X, r, cc); t_w = time.perf_counter() - t0
    K = X.shape[1]
    res["c3"] = {"sample": f"forward and dgrad on {rows} of 8192 rows, wgrad on {pts} of 4096^2 outputs",
                 "fwd_TFLOPs": 2.0 * rows * W.shape[0] * K / t_f / 1e12,
                 "dgrad_TFLOPs": 2.0 * rows * W.shape[0] * K / t_d / 1e12,
                 "wgrad_TFLOPs": 2.0 * pts * X.shape[0] / t_w / 1e12,
                 "seconds": round(t_f + t_d + t_w, 2)}
    res["cores"] = oracle.threads()
    return res


def roofline_line(dom: str, g: dict, random_operand_tflops: float) -> dict:
    """The roofline object of the dominant GEMM kind: achieved TFLOP/s against the 2.5 PFLOP/s FP16
    dense peak, the counter traffic, from the counter pass how busy the matrix cores were and the
    shader clock the chip ran this kernel at (the spec peak assumes 2.4 GHz), and the fraction of the
    rate of the GEMMs' MFMA form (v_mfma_f32_16x16x32_f16) the chip sustains on random binary16
    operands with no memory traffic at all (the matrix-core probe measured in this run)."""
    busy, mhz = measured_mfma(dom)
    out = {"bound": "mfma", "kernel": f"gemm_{dom}", "achieved": g["TFLOPs"], "peak": PEAK_F16_TFLOPS,
           "unit": "TFLOP/s", "frac": g["frac"], "traffic": measured_traffic("gemm", dom),
           "mfma_busy_frac": busy, "clock_mhz_under_load": mhz,
           "random_operand_mfma_ceiling": random_operand_tflops,
           "frac_of_random_operand_ceiling": round(g["TFLOPs"] / random_operand_tflops, 4)}
    if mhz:
        adj = PEAK_F16_TFLOPS * mhz / 2400.0
        out["clock_adjusted_peak"] = round(adj, 1)
        out["frac_of_clock_adjusted_peak"] = round(g["TFLOPs"] / adj, 4)
    return out


def calibration_c() -> float:
    with open(os.path.join(ROOT, "tests", "golden", "c4_calibration.json")) as f:
        return float(json.load(f)["c"])


class Model:
    """Device state of the C4 workload and one training step through libmp."""

    def __init__(self, mp, torch, w, c):
        self.mp, self.torch, self.c = mp, torch, c
        dev = "cuda"
        f16 = torch.float16
        self.W = [torch.from_numpy(m).to(dev) for m in w.masters]
        self.V = [torch.zeros_like(m) for m in self.W]
        self.W16 = [mp.round_f32_to_f16(m) for m in self.W]
        self.G = [torch.empty((WIDTH, WIDTH), dtype=f16, device=dev) for _ in range(LAYERS)]
        import numpy as np
        self.X = torch.from_numpy(w.X16.view(np.int16)).to(dev).view(f16)
        self.T = torch.from_numpy(w.T16.view(np.int16)).to(dev).view(f16)
        # per layer: Z (last layer, recompute and separate modes) or GELU'(Z) (saved mode)
        self.Z = [torch.empty((BATCH, WIDTH), dtype=f16, device=dev) for _ in range(LAYERS)]
        self.H = [torch.empty((BATCH, WIDTH), dtype=f16, device=dev) for _ in range(LAYERS - 1)]
        self.dA = torch.empty((BATCH, WIDTH), dtype=f16, device=dev)
        self.dB = torch.empty((BATCH, WIDTH), dtype=f16, device=dev)
        self.dC = torch.empty((BATCH, WIDTH), dtype=f16, device=dev)   # unfused variant only
        self.loss = torch.zeros(1, dtype=torch.float32, device=dev)
        self.loss_ws = torch.empty(mp.loss_mse_workspace(BATCH, WIDTH), dtype=torch.uint8, device=dev)
        self.scaler = mp.Scaler(w.scale, w.dynamic, w.growth_interval)
        self.plist = mp.ParamList(self.W, self.V, self.G, self.W16)
        self.hp = (w.lr, w.momentum, w.weight_decay)
        self.events = None
        self.gelu = "saved"

    def start_events(self, pairs=128):
        """Per-launch timing from here on. The events are created and recorded once up front,
        so that a timed launch costs the host two event records and nothing else: a host stall
        long enough for the GPU to drain the queue would put idle time between a pair."""
        E = self.torch.cuda.Event
        self.pool = [(E(enable_timing=True), E(enable_timing=True)) for _ in range(pairs)]
        for a, b in self.pool:
            a.record(); b.record()
        self.torch.cuda.synchronize()
        self.pool.reverse()
        self.events = {}

    def _t(self, kind, fn, *a, **k):
        if self.events is None:
            return fn(*a, **k)
        if not self.pool:
            self.pool.append((self.torch.cuda.Event(enable_timing=True), self.torch.cuda.Event(enable_timing=True)))
        e0, e1 = self.pool.pop()
        e0.record()
        r = fn(*a, **k)
        e1.record()
        self.events.setdefault(kind, []).append((e0, e1))
        return r

    def step(self):
        mp, t = self.mp, self._t
        inp = self.X
        for l in range(LAYERS):
            if l == LAYERS - 1:
                t("fwd", mp.linear_fwd, inp, self.W16[l], Y=self.Z[l])
            elif self.gelu == "saved":
                t("fwd_act_deriv", mp.linear_fwd_act_deriv, mp.GELU, inp, self.W16[l], H=self.H[l], D=self.Z[l])
                inp = self.H[l]
            elif self.gelu == "recompute":
                t("fwd_act", mp.linear_fwd_act, mp.GELU, inp, self.W16[l], Z=self.Z[l], H=self.H[l])
                inp = self.H[l]
            else:
                t("fwd", mp.linear_fwd, inp, self.W16[l], Y=self.Z[l])
                t("gelu_fwd", mp.act_fwd, mp.GELU, self.Z[l], self.H[l])
                inp = self.H[l]
        t("loss", mp.loss_mse, self.Z[-1], self.T, self.c, self.scaler, self.loss, self.dA,
          workspace=self.loss_ws)
        dZ, other = self.dA, self.dB
        for l in range(LAYERS - 1, -1, -1):
            prev = self.X if l == 0 else self.H[l - 1]
            t("wgrad", mp.linear_wgrad, dZ, prev, dW=self.G[l], found_inf=self.scaler.found_inf_ptr)
            if l == 0:
                break
            if self.gelu == "saved":
                # dZ_{l-1} = GELU'(Z_{l-1}) * (dZ_l . W_l), the derivative saved by the forward
                t("dgrad_mul", mp.linear_dgrad_mul, dZ, self.W16[l], self.Z[l - 1], dZ=other)
            elif self.gelu == "recompute":
                # the same product with GELU'(Z_{l-1}) evaluated in the dgrad epilogue
                t("dgrad_act", mp.linear_dgrad_act, mp.GELU, dZ, self.W16[l], self.Z[l - 1], dZ=other)
            else:
                t("dgrad", mp.linear_dgrad, dZ, self.W16[l], dX=self.dC)
                t("gelu_bwd", mp.act_bwd, mp.GELU, self.Z[l - 1], self.dC, other)
            dZ, other = other, dZ
        lr, mu, wd = self.hp
        # the weight-gradient epilogues already set the overflow flag (Step 6
        # fused into the producer), so the sweep is the single update pass
        t("sweep", mp.step, self.plist, self.scaler, lr, mu, wd, flags=mp.MP_GRADS_PRECHECKED)
        t("scaler", self.scaler.update)

    def kernel_ms(self):
        out = {}
        for k, evs in self.events.items():
            d = sorted(a.elapsed_time(b) for a, b in evs)
            out[k] = {"launches": len(d), "avg_ms": sum(d) / len(d), "total_ms": sum(d),
                      "median_ms": d[len(d) // 2], "max_ms": d[-1]}
        return out


def cpu_baseline(w, c, rows):
    """The oracle on a bounded sample of the same step: all 35 GEMMs of the step on `rows` of the
    4096 batch rows (rows are independent in forward and dgrad; wgrad reduces over those rows),
    the point-wise ops and the loss on those rows, and the full optimizer sweep."""
    import numpy as np

    import oracle
    W16 = [oracle.f32_to_f16(m) for m in w.masters]
    X, T = w.X16[:rows].copy(), w.T16[:rows].copy()
    t0 = time.perf_counter()
    Z, H = [], [X]
    for l in range(LAYERS):
        Z.append(oracle.linear_fwd(H[-1], W16[l], out_f16=True))
        if l < LAYERS - 1:
            H.append(oracle.gelu_fwd(Z[-1]))
    _, dZ = oracle.mse(Z[-1], T, c * rows / BATCH, w.scale)
    grads = [None] * LAYERS
    for l in range(LAYERS - 1, -1, -1):
        grads[l] = oracle.linear_wgrad(dZ, H[l], out_f16=True)
        if l > 0:
            dH = oracle.linear_dgrad(dZ, W16[l], out_f16=True)
            dZ = oracle.gelu_bwd(Z[l - 1], dH)
    t_gemm = time.perf_counter() - t0
    masters = [m.reshape(-1).copy() for m in w.masters]
    moms = [np.zeros_like(m) for m in masters]
    w16 = [x.reshape(-1).copy() for x in W16]
    t1 = time.perf_counter()
    oracle.step(masters, moms, [g.reshape(-1) for g in grads], w16, w.lr, w.momentum,
                w.weight_decay, 1.0 / w.scale)
    t_sweep = time.perf_counter() - t1
    gemm_flops = 2.0 * rows * WIDTH * WIDTH * (3 * LAYERS - 1)
    nparam = LAYERS * WIDTH * WIDTH
    return {
        "value": gemm_flops / t_gemm / 1e12,
        "unit": "TFLOP/s",
        "cores": oracle.threads(),
        "kind": "oracle",
        "sample": f"C4 step on {rows} of {BATCH} batch rows: 35 GEMMs (2*{rows}*4096*4096 FLOP "
                  f"each), GELU and loss on those rows ({t_gemm:.2f} s); full optimizer sweep over "
                  f"{nparam} parameters ({t_sweep:.2f} s)",
        "sweep_GBps": SWEEP_BYTES_PER_PARAM * nparam / t_sweep / 1e9,
        "seconds": round(t_gemm + t_sweep, 2),
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import torch

    import mixed_precision_neural_amd as mp
    import workloads

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.pmc_kernel:
        pmc_kernel(args, mp, torch)
        return
    c = calibration_c()
    w = workloads.c4()
    model = Model(mp, torch, w, c)
    model.gelu = "separate" if args.unfused else args.gelu
    torch.cuda.synchronize()

    for _ in range(args.warmup):
        model.step()
    torch.cuda.synchronize()

    # The timed steps: nothing but the steps between the two bracketing events.
    model.events = None
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    gc.disable()
    t_wall = time.perf_counter()
    start.record()
    for _ in range(args.steps):
        model.step()
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    gc.enable()
    ms = start.elapsed_time(end) / args.steps

    # Median and minimum step: the same number of steps once more, each between its own pair
    # of HIP events (two queue markers per step of ~4.7 ms).
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(args.steps)]
    torch.cuda.synchronize()
    for a, b in pairs:
        a.record()
        model.step()
        b.record()
    torch.cuda.synchronize()
    per_step = sorted(a.elapsed_time(b) for a, b in pairs)
    step_stats = {"median_ms": round(per_step[len(per_step) // 2], 4), "min_ms": round(per_step[0], 4),
                  "max_ms": round(per_step[-1], 4), "steps": len(per_step),
                  "method": "one pair of HIP events around each of the same number of further steps"}

    # Per-launch durations: the same number of steps once more, each launch between two HIP
    # events on the stream it runs on. They are kept out of the timed steps because every
    # recorded event is a queue marker of its own (~0.25 ms per step for the 76 of a step).
    model.start_events(80 * args.steps)
    gc.disable()
    for _ in range(args.steps):
        model.step()
    torch.cuda.synchronize()
    gc.enable()
    kern = model.kernel_ms()
    st = model.scaler.read()

    # The two-pass sweep (read-only check pass + update pass) that update-only
    # callers use when the gradients were not produced by mp_linear_wgrad.
    model.start_events(5)
    lr, mu, wd = model.hp
    for _ in range(5):
        model._t("sweep2", mp.step, model.plist, model.scaler, lr, mu, wd)
    torch.cuda.synchronize()
    two_pass_ms = model.kernel_ms()["sweep2"]["avg_ms"]

    # The other update rules of the sweep (Nesterov, Adagrad) and the method-2
    # |g| maximum, at the same 201M parameters, on buffers of their own (the
    # model's masters stay intact): algorithmic 20 B/param for a sweep, 4 B per
    # FP32 element read for the maximum.
    variants = {}
    g_w = [w.clone() for w in model.W]
    g_s = [torch.zeros_like(w) for w in model.W]
    g_16 = [torch.empty_like(h) for h in model.W16]
    vlist = mp.ParamList(g_w, g_s, model.G, g_16)
    for name, kind in (("nesterov", mp.NESTEROV), ("adagrad", mp.ADAGRAD)):
        # one untimed call first: it also waits for the list's descriptor upload
        mp.step_opt(vlist, model.scaler, kind, lr, mu, wd, 1e-10, flags=mp.MP_GRADS_PRECHECKED)
        model.start_events(5)
        for _ in range(5):
            model._t(name, mp.step_opt, vlist, model.scaler, kind, lr, mu, wd, 1e-10,
                     flags=mp.MP_GRADS_PRECHECKED)
        torch.cuda.synchronize()
        v_ms = model.kernel_ms()[name]["avg_ms"]
        gbps = SWEEP_BYTES_PER_PARAM * LAYERS * WIDTH * WIDTH / (v_ms * 1e-3) / 1e9
        variants[name] = {"avg_us": round(v_ms * 1e3, 2), "achieved_GBps": round(gbps, 1),
                          "frac": round(gbps / PEAK_HBM_GBPS, 4),
                          "algorithmic_bytes": SWEEP_BYTES_PER_PARAM * LAYERS * WIDTH * WIDTH,
                          "traffic": measured_traffic("update", name)}
    vlist.close()
    tl = mp.TensorList(model.W)
    amax = torch.zeros(1, dtype=torch.float32, device="cuda")
    mp.absmax(tl, amax)                       # untimed: waits for the list's upload
    model.start_events(5)
    for _ in range(5):
        model._t("absmax", mp.absmax, tl, amax)
    torch.cuda.synchronize()
    a_ms = model.kernel_ms()["absmax"]["avg_ms"]
    a_gbps = 4 * LAYERS * WIDTH * WIDTH / (a_ms * 1e-3) / 1e9
    method2 = {"avg_us": round(a_ms * 1e3, 2), "achieved_GBps": round(a_gbps, 1),
               "frac": round(a_gbps / PEAK_HBM_GBPS, 4), "algorithmic_bytes": 4 * LAYERS * WIDTH * WIDTH,
               "traffic": measured_traffic("stats", "absmax"), "input": "FP32, 12 x 4096^2"}
    tl.close()
    del g_w, g_s, g_16
    fp32_reductions = reductions(model, mp, torch)
    c1 = c1_latency(mp, torch, workloads)

    # C3's single layer, the achievable denominators (stream probe; clock and MFMA rate under a
    # pure matrix-core load with constant and with random operands), then the C2 / C5 update-only
    # sweeps.
    from mixed_precision_neural_amd import probe
    c3 = c3_gemms(mp, torch)
    ceiling = hbm_ceiling(torch, probe)
    clock = {"v_mfma_f32_16x16x32_f16": {"constant_operands": mfma_clock(torch, probe, probe.CONSTANT, probe.MFMA_16X16X32),
                                         "random_operands": mfma_clock(torch, probe, probe.RANDOM, probe.MFMA_16X16X32)},
             "v_mfma_f32_32x32x16_f16": {"random_operands": mfma_clock(torch, probe, probe.RANDOM, probe.MFMA_32X32X16)}}
    copy_gbps = ceiling["copy"]["GBps"]
    c2 = c2_sweep(mp, torch, copy_gbps)
    c5 = c5_sweep(mp, torch, workloads, copy_gbps)
    if args.no_cpu_baseline:
        for d in (c2, c3, c5):
            d.pop("_host")
    else:
        cpu = cpu_configs(c2, c3, c5)
        for k, d in (("c2", c2), ("c3", c3), ("c5", c5)):
            d["cpu_oracle"] = dict(cpu[k], cores=cpu["cores"])
        c1["cpu_oracle"] = cpu_c1_step(workloads)
    torch.cuda.synchronize()

    gemm_flop = 2.0 * WIDTH * WIDTH * BATCH
    step_flop = gemm_flop * (3 * LAYERS - 1)
    value = step_flop / (ms * 1e-3) / 1e12
    gemm = {}
    kinds = [k for k in ("fwd_act_deriv", "fwd_act", "fwd", "dgrad_mul", "dgrad_act", "dgrad", "wgrad") if k in kern]
    for k in kinds:
        tf = gemm_flop / (kern[k]["avg_ms"] * 1e-3) / 1e12
        gemm[k] = {"avg_us": round(kern[k]["avg_ms"] * 1e3, 2), "median_us": round(kern[k]["median_ms"] * 1e3, 2),
                   "max_us": round(kern[k]["max_ms"] * 1e3, 2), "TFLOPs": round(tf, 1),
                   "frac": round(tf / PEAK_F16_TFLOPS, 4), "launches": kern[k]["launches"]}
    dom = max(kinds, key=lambda k: kern[k]["total_ms"])
    nparam = LAYERS * WIDTH * WIDTH
    sweep_ms = kern["sweep"]["avg_ms"]
    sweep_gbps = SWEEP_BYTES_PER_PARAM * nparam / (sweep_ms * 1e-3) / 1e9
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "step_ms": step_stats,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16/f32",
        "data": "synthetic",
        "config": {"workload": "C4: 12-layer GELU MLP, width 4096, batch 4096, MSE to N(0,1) targets, "
                               "FP16 storage, FP32 master + momentum, dynamic loss scale 2^16, "
                               "SGD lr 0.01 momentum 0.9",
                   "global_batch": BATCH, "params": nparam, "gemms_per_step": 3 * LAYERS - 1,
                   "gelu": {"saved": "in the GEMM epilogues, GELU'(Z) saved by the forward",
                            "recompute": "in the GEMM epilogues, GELU'(Z) evaluated in the backward",
                            "separate": "separate point-wise kernels"}[model.gelu],
                   "loss_multiplier_c": c},
        "roofline": roofline_line(dom, gemm[dom], clock["v_mfma_f32_16x16x32_f16"]["random_operands"]["mfma_f16_TFLOPs"]),
        "gemm": gemm,
        "mp_step": {"bound": "hbm", "mode": "flag from the wgrad epilogues, one update pass",
                    "avg_us": round(sweep_ms * 1e3, 2),
                    "achieved_GBps": round(sweep_gbps, 1), "peak": PEAK_HBM_GBPS,
                    "frac": round(sweep_gbps / PEAK_HBM_GBPS, 4),
                    "algorithmic_bytes": SWEEP_BYTES_PER_PARAM * nparam,
                    "traffic": measured_traffic("update", "update"),
                    "two_pass_us": round(two_pass_ms * 1e3, 2),
                    "two_pass_GBps": round(SWEEP_BYTES_PER_PARAM * nparam / (two_pass_ms * 1e-3) / 1e9, 1),
                    "check_pass_bytes": CHECK_BYTES_PER_PARAM * nparam,
                    "frac_of_copy_ceiling": round(sweep_gbps / copy_gbps, 4)},
        "mp_step_opt": variants,
        "absmax_method2": method2,
        "fp32_reductions": fp32_reductions,
        "c1_step_latency": c1,
        "c2": c2,
        "c3": c3,
        "c5": c5,
        "hbm_ceiling": ceiling,
        "mfma_probe": clock,
        "aux_us": {k: round(kern[k]["avg_ms"] * 1e3, 2) for k in ("gelu_fwd", "gelu_bwd", "loss", "scaler")
                   if k in kern},
        "scaler_after": {"scale": st["scale"], "skipped_steps": st["skipped_steps"]},
        "wall_s": round(wall, 3),
        "kernel_timing": f"HIP events around each launch over {args.steps} further steps of the same workload",
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, c, args.cpu_rows)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
