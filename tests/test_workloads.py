"""Checks of the synthetic input recipes against the statistics they are built to have."""
import math

import numpy as np

import workloads


def test_c2_gradient_statistics(orc):
    """Pin P3 on the C2 recipe: log2|g| ~ U(-34, -4). Unscaled, |g| <= 2^-25 (9 of 30 binades)
    rounds to zero and (2^-25, 2^-24) (1 of 30) to 2^-24; at S = 2^15 nothing is lost."""
    w = workloads.c2(n=2_000_000)
    h = orc.f32_to_f16(w.g_true)
    n = h.size
    a = np.abs(w.g_true.astype(np.float64))
    zero = ((h & 0x7FFF) == 0)
    assert np.array_equal(zero, a <= 2.0 ** -25)
    sd = math.sqrt(0.3 * 0.7 / n)
    assert abs(zero.mean() - 9 / 30) < 6 * sd
    band = (a > 2.0 ** -25) & (a < 2.0 ** -24)
    assert ((h[band] & 0x7FFF) == 1).all()
    assert abs(band.mean() - 1 / 30) < 6 * math.sqrt((1 / 30) * (29 / 30) / n)
    scaled = orc.f32_to_f16((w.g_true * np.float32(2.0 ** 15)).astype(np.float32))
    assert not ((scaled & 0x7FFF) == 0).any()
    assert 0 <= w.inf_index < n


def test_grads_at_scale_agrees_with_oracle_codec(orc):
    w = workloads.c2(n=200_000)
    a = workloads.grads_at_scale(w.g_true, 2.0 ** 15)
    b = orc.f32_to_f16((w.g_true * np.float32(2.0 ** 15)).astype(np.float32))
    assert np.array_equal(a, b)


def test_c5_sizes_and_spread():
    s = workloads.c5_sizes()
    assert s.size == 500
    assert abs(int(s.sum()) - workloads.C5_TOTAL) <= workloads.C5_TOTAL // 1000
    assert s.min() >= 1 and (s % 8 != 0).any()
    t = workloads.c5_tensor(3, 400_000)
    below = (np.abs(t.g_true) < 2.0 ** -24).mean()
    assert abs(below - 0.05) < 0.005            # 5 % of unscaled magnitudes below 2^-24
    med = np.median(np.log2(np.abs(t.g_true)))
    assert abs(med - workloads.C5_LOG2_MEDIAN) < 0.05


def test_c5_nan_indices():
    idx = workloads.c5_nan_indices(10_000_000)
    assert idx.size == 10_000 and np.unique(idx).size == idx.size
    assert idx.min() >= 0 and idx.max() < 10_000_000


def test_generators_are_deterministic():
    a, b = workloads.c1(), workloads.c1()
    assert np.array_equal(a.W1, b.W1) and np.array_equal(a.X16, b.X16)
    assert np.array_equal(a.labels, b.labels)
    c, d = workloads.c3(64, 32, 48), workloads.c3(64, 32, 48)
    assert np.array_equal(c.W16, d.W16)
    assert abs(np.std(c.W16.view(np.float16).astype(np.float64)) - 1 / math.sqrt(48)) < 0.02
