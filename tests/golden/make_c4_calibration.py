"""Writes tests/golden/c4_calibration.json: the loss multiplier c of the 12-layer MLP workload.

Recipe (a reading of "grads scaled so ~5 % of unscaled activation-gradients fall below
2^-24", after the Mandarin speech histogram of "Mixed Precision Training", long-form
analysis page, §3.4 "FP32 Master Copy of Weights", original Figure 2b): with c = 1, take
the activation gradients of one backward pass at step 0 (the loss gradient and every
dgrad output), find their 5th percentile magnitude q, and set c = 2^-24 / q.

Only the oracle computes. Rows of an MLP batch are independent in forward and dgrad, so
a subset of rows (with the mean still over the full 4096 x 4096 output) gives an unbiased
sample of the distribution. The backward runs at S = 2^24 so that every value sits well
inside the binary16 normal range, and the magnitudes are divided by S afterwards.
"""
import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
import workloads  # noqa: E402

ROWS = 32
S = 2.0 ** 24


def main():
    t0 = time.time()
    w = workloads.c4()
    W16 = [oracle.f32_to_f16(m) for m in w.masters]
    X = w.X16[:ROWS].copy()
    T = w.T16[:ROWS].copy()
    Z, H = [], [X]
    for l in range(12):
        z = oracle.linear_fwd(H[-1], W16[l], out_f16=True)
        Z.append(z)
        if l < 11:
            H.append(oracle.gelu_fwd(z))
    batch, width = w.X16.shape
    # loss gradient at c = 1, scaled by S and rounded once
    dY = oracle.mse_grad_f64(Z[11], T, batch, 1.0) * S
    mags = [np.abs(dY).ravel()]
    dZ = oracle.f32_to_f16(dY.astype(np.float32))
    for l in range(11, 0, -1):
        dH = oracle.linear_dgrad(dZ, W16[l], out_f16=False)
        mags.append(np.abs(dH.astype(np.float64)).ravel())
        dZ = oracle.gelu_bwd(Z[l - 1], oracle.f32_to_f16(dH))
    allm = np.concatenate(mags) / S
    q05 = float(np.quantile(allm, 0.05))
    c = float(np.float32(2.0 ** -24 / q05))
    out = {
        "c": c,
        "q05_unscaled": q05,
        "rows_sampled": ROWS,
        "values": int(allm.size),
        "fraction_below_2^-24_at_c": float(np.mean(allm * c < 2.0 ** -24)),
        "recipe": "12-layer GELU MLP, width 4096, batch 4096, seed 0; activation gradients "
                  "(loss gradient + 11 dgrad outputs) of step 0 at c = 1; c = 2^-24 / q05",
        "script": "tests/golden/make_c4_calibration.py (calls only the oracle)",
        "seconds": round(time.time() - t0, 1),
    }
    with open(os.path.join(HERE, "c4_calibration.json"), "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))


if __name__ == "__main__":
    main()
