"""Pins of the oracle's optimizer sweep, overflow flag and loss scaler.

Sources: "Mixed Precision Training", long-form analysis page, §3.4 "The
Integrated Training Procedure" (Steps 1 and 5-7, weight decay) and "Choosing
the Loss Scaling Factor" (methods 1 and 3).
"""
import numpy as np
import pytest


def f32bits(x):
    return int(np.asarray(x, np.float32).view(np.uint32))


def make(n, w=0.0, v=0.0, h=0):
    return (np.full(n, w, np.float32), np.full(n, v, np.float32),
            np.full(n, h, np.uint16), np.zeros(n, np.uint16))


def test_master_keeps_what_f16_loses(orc):
    """Pin P5: w = 1, lr = 2^-11, mu = 0, g = -1 at S = 1."""
    w, v, g, w16 = make(1, w=1.0, h=0xBC00)   # g16 = -1.0
    flag = orc.step([w], [v], [g], [w16], 2.0 ** -11, 0.0, 0.0, 1.0)
    assert flag == 0
    assert f32bits(w[0]) == 0x3F801000            # 1 + 2^-11 kept in FP32
    assert int(w16[0]) == 0x3C00                  # its binary16 copy still reads 1.0
    # the same update applied to a binary16 weight directly is lost
    s16 = orc.f32_to_f16(np.array([1.0 + 2.0 ** -11], np.float32))
    assert int(s16[0]) == 0x3C00
    orc.step([w], [v], [g], [w16], 2.0 ** -11, 0.0, 0.0, 1.0)
    assert float(w[0]) == 1.0 + 2.0 ** -10
    assert int(w16[0]) == 0x3C01


def test_exact_power_of_two_unscale_all_f16(orc):
    """Pin P4: f32(h) * 2^-k equals h / 2^k exactly for every finite binary16 h, k in [0, 64].
    With w = v = mu = wd = 0 and lr = -1 the master after one step is the unscaled gradient."""
    h = np.arange(1 << 16, dtype=np.uint16)
    finite = (h & 0x7C00) != 0x7C00
    h = h[finite]
    ref_all = h.view(np.float16).astype(np.float64)
    for k in range(0, 65):
        w, v, _, w16 = make(h.size)
        orc.sgd_update([w], [v], [h.copy()], [w16], -1.0, 0.0, 0.0, 2.0 ** -k)
        ref = ref_all / 2.0 ** k
        assert np.array_equal(w.astype(np.float64), ref), k
        nz = ref != 0        # -0 becomes +0 through the (+0) weight-decay term: see below
        assert np.array_equal(np.signbit(w[nz]), np.signbit(ref[nz])), k


def test_weight_decay_closed_form(orc):
    """g = 0, mu = 0, lr = 1, wd = 2^-k: w' = w - 2^-k w, one rounding (coupled L2 on the FP32
    master, applied before the update)."""
    rng = np.random.Generator(np.random.PCG64(3))
    w0 = rng.standard_normal(4096).astype(np.float32)
    for k in (1, 5, 13):
        w, v, g, w16 = w0.copy(), np.zeros(4096, np.float32), np.zeros(4096, np.uint16), np.zeros(4096, np.uint16)
        orc.sgd_update([w], [v], [g], [w16], 1.0, 0.0, 2.0 ** -k, 1.0)
        exact = w0.astype(np.float64) * (1.0 - 2.0 ** -k)
        assert np.array_equal(w, exact.astype(np.float32))
        assert np.array_equal(v, (w0.astype(np.float64) * 2.0 ** -k).astype(np.float32))


def test_momentum_closed_form_two_steps(orc):
    """v_1 = g, v_2 = mu v_1 + g; with mu = 1/2 and power-of-two lr: w_2 = w_0 - lr (1 + 3/2) g."""
    g16 = np.array([0x3C00, 0xC000, 0x0001, 0x3555], np.uint16)    # 1, -2, 2^-24, ~1/3
    gv = g16.view(np.float16).astype(np.float64)
    w, v, _, w16 = make(4, w=0.0)
    for _ in range(2):
        orc.step([w], [v], [g16], [w16], 2.0 ** -3, 0.5, 0.0, 1.0)
    assert np.array_equal(v.astype(np.float64), 1.5 * gv)
    assert np.array_equal(w.astype(np.float64), -(2.0 ** -3) * 2.5 * gv)


def test_full_step_closed_form_with_every_term(orc):
    """Every term non-zero and exactly representable: S = 4, wd = 1/4, mu = 1/2, lr = 1/8."""
    w, v, g, w16 = make(1, w=2.0, v=1.0, h=0x4400)   # g16 = 4.0 -> unscaled 1.0
    orc.step([w], [v], [g], [w16], 0.125, 0.5, 0.25, 0.25)
    # g = 1 + 0.25*2 = 1.5; v = 0.5*1 + 1.5 = 2.0; w = 2 - 0.125*2 = 1.75
    assert float(v[0]) == 2.0 and float(w[0]) == 1.75
    assert int(w16[0]) == 0x3F00


def test_signed_zero_rule(orc):
    """With v = -0 and g = -0 the weight-decay term +0 makes v = +0; dropping the term when
    wd = 0 would leave -0."""
    w, v, g, w16 = make(1, w=1.0, v=-0.0, h=0x8000)
    orc.step([w], [v], [g], [w16], 0.01, 0.9, 0.0, 1.0)
    assert f32bits(v[0]) == 0x00000000
    assert f32bits(w[0]) == f32bits(1.0)


@pytest.mark.parametrize("bad", [0x7C00, 0xFC00, 0x7E00, 0x7C01])
@pytest.mark.parametrize("where", ["first", "middle", "last"])
def test_overflow_step_leaves_state_untouched(orc, bad, where):
    """Pin P6: one non-finite gradient element anywhere skips the update of every tensor."""
    rng = np.random.Generator(np.random.PCG64(5))
    sizes = [7, 1000, 4099]                        # ragged tails
    ws = [rng.standard_normal(n).astype(np.float32) for n in sizes]
    vs = [rng.standard_normal(n).astype(np.float32) for n in sizes]
    gs = [(rng.standard_normal(n) * 0.1).astype(np.float16).view(np.uint16) for n in sizes]
    w16s = [np.full(n, 0x1234, np.uint16) for n in sizes]
    t = 2
    idx = {"first": 0, "middle": sizes[t] // 2, "last": sizes[t] - 1}[where]
    gs[t][idx] = bad
    before = [a.copy() for a in ws + vs + w16s]
    assert orc.check_overflow(gs) == 1
    flag = orc.step(ws, vs, gs, w16s, 0.01, 0.9, 1e-4, 2.0 ** -10)
    assert flag == 1
    for a, b in zip(ws + vs + w16s, before):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8))


def test_clean_step_flags_nothing(orc):
    h = np.arange(1 << 16, dtype=np.uint16)
    finite = h[(h & 0x7C00) != 0x7C00]
    assert orc.check_overflow([finite]) == 0
    assert orc.check_overflow([finite, np.array([0x7BFF, 0xFBFF], np.uint16)]) == 0
    assert orc.check_overflow([finite, np.array([0x7C00], np.uint16)]) == 1


def test_scaler_dynamic_overflow_halves_and_counts(orc):
    s = orc.scaler_init(2.0 ** 15, True, 2000)
    s = orc.scaler_update(s, 1)
    assert s.scale == 2.0 ** 14 and s.inv_scale == 2.0 ** -14 and s.count == 0
    assert s.skipped_steps == 1 and s.found_inf == 0


def test_scaler_static_overflow_keeps_scale(orc):
    s = orc.scaler_init(1024.0, False, 2000)
    for _ in range(5):
        s = orc.scaler_update(s, 0)
    s = orc.scaler_update(s, 1)
    assert s.scale == 1024.0 and s.skipped_steps == 1


def test_scaler_trace_c2(orc):
    """Pin P7 (C2): 2^15 for steps 0-24, step 25 skipped, 2^14 after, final count 24."""
    s = orc.scaler_init(2.0 ** 15, True, 2000)
    seen = []
    for t in range(50):
        seen.append(s.scale)
        s = orc.scaler_update(s, 1 if t == 25 else 0)
    assert seen[:26] == [2.0 ** 15] * 26 and seen[26:] == [2.0 ** 14] * 24
    assert s.count == 24 and s.skipped_steps == 1 and s.scale == 2.0 ** 14


def test_scaler_trace_c5(orc):
    s = orc.scaler_init(2.0 ** 12, True, 2000)
    for t in range(20):
        s = orc.scaler_update(s, 1 if t == 7 else 0)
    assert s.scale == 2.0 ** 11 and s.count == 12 and s.skipped_steps == 1


def test_scaler_growth_every_n_clean_steps(orc):
    """Growth interval 3: doubles after every 3 clean steps; an overflow resets the run."""
    s = orc.scaler_init(8.0, True, 3)
    trace = []
    for f in [0, 0, 0, 0, 0, 1, 0, 0, 0]:
        s = orc.scaler_update(s, f)
        trace.append((s.scale, s.count))
    assert trace == [(8, 1), (8, 2), (16, 0), (16, 1), (16, 2), (8, 0), (8, 1), (8, 2), (16, 0)]


def test_scaler_clamps(orc):
    s = orc.scaler_init(1.0, True, 1)
    s = orc.scaler_update(s, 1)
    assert s.scale == 1.0
    s = orc.scaler_init(2.0 ** 64, True, 1)
    s = orc.scaler_update(s, 0)
    assert s.scale == 2.0 ** 64 and s.inv_scale == 2.0 ** -64
