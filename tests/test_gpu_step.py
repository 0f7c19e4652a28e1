"""GPU parity of the optimizer sweep and the loss scaler against the oracle (bit-exact).

Source: "Mixed Precision Training", long-form analysis page, §3.4 "The Integrated
Training Procedure" (Steps 1, 5-7, weight decay) and "Choosing the Loss Scaling
Factor" (methods 1 and 3).
"""
import numpy as np
import pytest
import torch

import mixed_precision_neural_amd as mp
import oracle
import workloads
from gpu_util import (dev_f16, dev_f32, host_bits16, host_f32, require_gpu, same_f16_bits,
                      same_f32_bits)

pytestmark = pytest.mark.gpu


class Run:
    """The same tensors on the GPU and on the host, stepped by libmp and by the oracle."""

    def __init__(self, ws, vs, gs):
        self.h_w = [np.array(w, np.float32) for w in ws]
        self.h_v = [np.array(v, np.float32) for v in vs]
        self.h_g = [np.array(g, np.uint16) for g in gs]
        self.h_16 = [oracle.f32_to_f16(w) for w in self.h_w]
        self.d_w = [dev_f32(w) for w in self.h_w]
        self.d_v = [dev_f32(v) for v in self.h_v]
        self.d_g = [dev_f16(g) for g in self.h_g]
        self.d_16 = [mp.round_f32_to_f16(w) for w in self.d_w]

    def plist(self):
        return mp.ParamList(self.d_w, self.d_v, self.d_g, self.d_16)

    def set_grads(self, gs):
        for i, g in enumerate(gs):
            self.h_g[i][:] = g
            self.d_g[i].copy_(dev_f16(g))

    def oracle_step(self, lr, mu, wd, inv_scale):
        return oracle.step(self.h_w, self.h_v, self.h_g, self.h_16, lr, mu, wd, inv_scale)

    def assert_equal(self, what=""):
        torch.cuda.synchronize()
        for i in range(len(self.h_w)):
            assert same_f32_bits(host_f32(self.d_w[i]), self.h_w[i]), f"master {i} {what}"
            assert same_f32_bits(host_f32(self.d_v[i]), self.h_v[i]), f"momentum {i} {what}"
            assert same_f16_bits(host_bits16(self.d_16[i]), self.h_16[i]), f"weight16 {i} {what}"


def scaler_pair(scale, dynamic, interval=2000):
    return mp.Scaler(scale, dynamic, interval), oracle.scaler_init(scale, dynamic, interval)


def assert_scaler(d: mp.Scaler, o):
    got = d.read()
    for k in ("scale", "inv_scale", "count", "growth_interval", "found_inf", "dynamic", "skipped_steps"):
        assert got[k] == getattr(o, k), (k, got[k], getattr(o, k))


def test_round_init_matches_oracle():
    require_gpu()
    rng = np.random.Generator(np.random.PCG64(0))
    for n in (1, 7, 8, 1000, 65539):
        w = (rng.standard_normal(n) * rng.choice([1e-8, 1e-3, 1.0, 1e4, 7e4], n)).astype(np.float32)
        got = host_bits16(mp.round_f32_to_f16(dev_f32(w)))
        assert same_f16_bits(got, oracle.f32_to_f16(w)), n


@pytest.mark.parametrize("lr,mu,wd", [(0.01, 0.9, 0.0), (1e-3, 0.9, 1e-4), (2.0 ** -11, 0.0, 0.5)])
@pytest.mark.parametrize("scale_log2", [0, 10, 15, 24, 64])
def test_every_finite_f16_gradient_pattern(lr, mu, wd, scale_log2):
    """Pin P11: every finite binary16 gradient pattern, with masters and momenta drawn from edge
    values (signed zeros, FP32 subnormals, binary16 rounding ties and the overflow boundary)."""
    require_gpu()
    h = np.arange(1 << 16, dtype=np.uint16)
    g = h[(h & 0x7C00) != 0x7C00]
    edges = np.array([0.0, -0.0, 1.0, -1.0, 1.0 + 2 ** -11, 1.0 + 3 * 2 ** -11, 1.0 - 2 ** -12,
                      2.0 ** -25, 3 * 2.0 ** -26, 2.0 ** -14 - 2.0 ** -25, 1e-40, -1e-40, 65504.0,
                      65519.0, 65520.0, -65536.0, 1e30, 0.1, -0.3, 123.456], np.float32)
    n = g.size
    w = edges[np.arange(n) % edges.size]
    v = edges[(np.arange(n) // edges.size) % edges.size]
    r = Run([w], [v], [g])
    S = mp.Scaler(2.0 ** scale_log2, True)
    pl = r.plist()
    mp.step(pl, S, lr, mu, wd)
    flag = r.oracle_step(lr, mu, wd, 2.0 ** -scale_log2)
    assert flag == 0
    r.assert_equal()
    assert S.read()["found_inf"] == 0
    pl.close()


@pytest.mark.parametrize("bad", [0x7C00, 0xFC00, 0x7E00, 0xFE01, 0x7C01])
@pytest.mark.parametrize("where", ["first", "middle", "last"])
@pytest.mark.parametrize("tensor", [0, 2])
def test_overflow_anywhere_skips_everything(bad, where, tensor):
    """Pin P6: one non-finite gradient element anywhere in the ragged list: no bit of any master,
    momentum or binary16 copy changes; dynamic S halves, count resets, skipped_steps += 1."""
    require_gpu()
    rng = np.random.Generator(np.random.PCG64(5))
    sizes = [8193, 7, 20000]
    ws = [rng.standard_normal(n).astype(np.float32) for n in sizes]
    vs = [rng.standard_normal(n).astype(np.float32) for n in sizes]
    gs = [(rng.standard_normal(n) * 100).astype(np.float16).view(np.uint16) for n in sizes]
    idx = {"first": 0, "middle": sizes[tensor] // 2, "last": sizes[tensor] - 1}[where]
    gs[tensor][idx] = bad
    r = Run(ws, vs, gs)
    before = [host_f32(t).copy() for t in r.d_w + r.d_v] + [host_bits16(t).copy() for t in r.d_16]
    dS, oS = scaler_pair(2.0 ** 15, True)
    pl = r.plist()
    mp.step(pl, dS, 0.01, 0.9, 1e-4)
    assert dS.read()["found_inf"] == 1
    flag = r.oracle_step(0.01, 0.9, 1e-4, oS.inv_scale)
    assert flag == 1
    after = [host_f32(t) for t in r.d_w + r.d_v] + [host_bits16(t) for t in r.d_16]
    for a, b in zip(after, before):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8))
    dS.update(); oracle.scaler_update(oS, flag)
    assert_scaler(dS, oS)
    assert dS.read()["scale"] == 2.0 ** 14
    pl.close()


def test_static_scaler_overflow_keeps_scale():
    require_gpu()
    r = Run([np.ones(100, np.float32)], [np.zeros(100, np.float32)], [np.full(100, 0x7C00, np.uint16)])
    dS, oS = scaler_pair(1024.0, False)
    pl = r.plist()
    mp.step(pl, dS, 0.01, 0.9, 0.0)
    flag = r.oracle_step(0.01, 0.9, 0.0, oS.inv_scale)
    dS.update(); oracle.scaler_update(oS, flag)
    assert_scaler(dS, oS)
    assert dS.read()["scale"] == 1024.0 and dS.read()["skipped_steps"] == 1
    pl.close()


def test_scaler_growth_and_clamps():
    require_gpu()
    for init, dyn, interval, flags in [(8.0, True, 3, [0, 0, 0, 0, 0, 1, 0, 0, 0]),
                                       (1.0, True, 1, [1, 1, 0]),
                                       (2.0 ** 63, True, 1, [0, 0, 0]),
                                       (1024.0, False, 2, [0, 1, 0, 0])]:
        dS, oS = scaler_pair(init, dyn, interval)
        for f in flags:
            if f:
                dS.buf[4] = 1
            dS.update()
            oracle.scaler_update(oS, f)
            assert_scaler(dS, oS)


@pytest.mark.parametrize("sizes", [[1], [7, 8, 9], [8191, 8192, 8193], [1, 100000, 3, 65536 * 3 + 5]])
def test_ragged_lists_multi_step(sizes):
    """Several clean steps over ragged lists with tails shorter than a vector and a chunk."""
    require_gpu()
    rng = np.random.Generator(np.random.PCG64(len(sizes)))
    ws = [(rng.standard_normal(n) * 0.02).astype(np.float32) for n in sizes]
    vs = [np.zeros(n, np.float32) for n in sizes]
    g_true = [(rng.standard_normal(n) * 2.0 ** -12).astype(np.float32) for n in sizes]
    gs = [workloads.grads_at_scale(g, 2.0 ** 12) for g in g_true]
    r = Run(ws, vs, gs)
    dS, oS = scaler_pair(2.0 ** 12, True, 2)
    pl = r.plist()
    for t in range(5):
        mp.step(pl, dS, 1e-3, 0.9, 1e-4)
        flag = r.oracle_step(1e-3, 0.9, 1e-4, oS.inv_scale)
        dS.update(); oracle.scaler_update(oS, flag)
        r.assert_equal(f"step {t}")
        assert_scaler(dS, oS)
        r.set_grads([workloads.grads_at_scale(g, oS.scale) for g in g_true])
    pl.close()


def test_unaligned_tensors_take_the_scalar_path():
    """Views that start one element into an allocation break 16-byte alignment."""
    require_gpu()
    rng = np.random.Generator(np.random.PCG64(9))
    n = 50001
    base_w = dev_f32(rng.standard_normal(n + 1).astype(np.float32))
    base_v = dev_f32(rng.standard_normal(n + 1).astype(np.float32))
    g = (rng.standard_normal(n + 1) * 10).astype(np.float16).view(np.uint16)
    base_g = dev_f16(g)
    base_16 = torch.zeros(n + 1, dtype=torch.float16, device="cuda")
    d_w, d_v, d_g, d_16 = base_w[1:], base_v[1:], base_g[1:], base_16[1:]
    h_w = host_f32(d_w).copy(); h_v = host_f32(d_v).copy(); h_g = g[1:].copy()
    h_16 = np.zeros(n, np.uint16)
    dS = mp.Scaler(4.0, False)
    pl = mp.ParamList([d_w], [d_v], [d_g], [d_16])
    mp.step(pl, dS, 0.01, 0.9, 1e-4)
    oracle.step([h_w], [h_v], [h_g], [h_16], 0.01, 0.9, 1e-4, 0.25)
    torch.cuda.synchronize()
    assert same_f32_bits(host_f32(d_w), h_w) and same_f32_bits(host_f32(d_v), h_v)
    assert same_f16_bits(host_bits16(d_16), h_16)
    pl.close()


def test_prechecked_flag_skips_the_check_pass():
    """With MP_GRADS_PRECHECKED the sweep trusts found_inf: a clean flag updates, a set flag skips."""
    require_gpu()
    rng = np.random.Generator(np.random.PCG64(3))
    n = 30000
    w = rng.standard_normal(n).astype(np.float32)
    g = (rng.standard_normal(n)).astype(np.float16).view(np.uint16)
    r = Run([w], [np.zeros(n, np.float32)], [g])
    dS, oS = scaler_pair(1.0, True)
    pl = r.plist()
    mp.step(pl, dS, 0.01, 0.9, 0.0, flags=mp.MP_GRADS_PRECHECKED)
    r.oracle_step(0.01, 0.9, 0.0, 1.0)
    r.assert_equal()
    before = host_f32(r.d_w[0]).copy()
    dS.buf[4] = 1
    mp.step(pl, dS, 0.01, 0.9, 0.0, flags=mp.MP_GRADS_PRECHECKED)
    torch.cuda.synchronize()
    assert np.array_equal(host_f32(r.d_w[0]), before)
    pl.close()


@pytest.mark.parametrize("where", [None, "first", "last"])
def test_check_only_sets_the_flag_and_writes_nothing(where):
    """MP_CHECK_ONLY runs the check pass alone (Step 6): the flag equals the oracle's check over
    the ragged list, and no master, momentum or binary16 byte changes either way."""
    require_gpu()
    rng = np.random.Generator(np.random.PCG64(9))
    sizes = [4096 * 3 + 5, 13, 70001]
    ws = [rng.standard_normal(n).astype(np.float32) for n in sizes]
    vs = [rng.standard_normal(n).astype(np.float32) for n in sizes]
    gs = [(rng.standard_normal(n) * 100).astype(np.float16).view(np.uint16) for n in sizes]
    if where:
        gs[2][0 if where == "first" else sizes[2] - 1] = 0xFC00
    r = Run(ws, vs, gs)
    before = [host_f32(t).copy() for t in r.d_w + r.d_v] + [host_bits16(t).copy() for t in r.d_16]
    dS = mp.Scaler(2.0 ** 10, True)
    pl = r.plist()
    mp.step(pl, dS, 0.01, 0.9, 1e-4, flags=mp.MP_CHECK_ONLY)
    assert dS.read()["found_inf"] == oracle.check_overflow(r.h_g) == (1 if where else 0)
    after = [host_f32(t) for t in r.d_w + r.d_v] + [host_bits16(t) for t in r.d_16]
    for a, b in zip(after, before):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8))
    # with the flag already set, the check leaves it set; with PRECHECKED it does nothing
    mp.step(pl, dS, 0.01, 0.9, 1e-4, flags=mp.MP_CHECK_ONLY | mp.MP_GRADS_PRECHECKED)
    assert dS.read()["found_inf"] == (1 if where else 0)
    pl.close()


def test_determinism():
    """Pin P10: the same inputs give the same bits twice."""
    require_gpu()
    rng = np.random.Generator(np.random.PCG64(4))
    sizes = [100003, 5]
    outs = []
    for _ in range(2):
        r = Run([rng.standard_normal(n).astype(np.float32) * 0 + 1 for n in sizes],
                [np.zeros(n, np.float32) for n in sizes],
                [np.full(n, 0x3555, np.uint16) for n in sizes])
        dS = mp.Scaler(2.0, True)
        pl = r.plist()
        for _ in range(3):
            mp.step(pl, dS, 0.01, 0.9, 1e-4)
        torch.cuda.synchronize()
        outs.append([host_f32(t).copy() for t in r.d_w + r.d_v])
        pl.close()
    for a, b in zip(*outs):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.timeout(900)
def test_c2_update_sweep_full_size():
    """C2: one flat tensor of 10^8 parameters, 50 steps, +inf injected at step 25, dynamic scaler.
    The oracle runs its own trajectory from the same generated inputs; masters, momenta and binary16
    copies are compared bit for bit after steps 0, 1, 24, 25, 26 and 49, on a fixed sample of
    2^20 elements after every other step, and the scaler after every step."""
    require_gpu()
    cfg = workloads.c2()
    n = cfg.w32.size
    r = Run([cfg.w32], [np.zeros(n, np.float32)], [workloads.grads_at_scale(cfg.g_true, cfg.scale)])
    dS, oS = scaler_pair(cfg.scale, cfg.dynamic, cfg.growth_interval)
    pl = r.plist()
    sample = np.random.Generator(np.random.PCG64(99)).choice(n, 1 << 20, replace=False)
    g_scale = cfg.scale
    for t in range(cfg.steps):
        if oS.scale != g_scale or t == cfg.inf_step or t == cfg.inf_step + 1:
            g_scale = oS.scale
            g = workloads.grads_at_scale(cfg.g_true, g_scale)
            if t == cfg.inf_step:
                g[cfg.inf_index] = workloads.F16_INF
            r.set_grads([g])
        print(f"C2 step {t} scale {oS.scale}", flush=True)
        mp.step(pl, dS, cfg.lr, cfg.momentum, cfg.weight_decay)
        flag = r.oracle_step(cfg.lr, cfg.momentum, cfg.weight_decay, oS.inv_scale)
        assert flag == (1 if t == cfg.inf_step else 0)
        dS.update(); oracle.scaler_update(oS, flag)
        assert_scaler(dS, oS)
        if t in (0, 1, 24, 25, 26, cfg.steps - 1):
            r.assert_equal(f"step {t}")
        else:
            torch.cuda.synchronize()
            idx = torch.from_numpy(sample).cuda()
            assert same_f32_bits(host_f32(r.d_w[0][idx]), r.h_w[0][sample]), t
            assert same_f32_bits(host_f32(r.d_v[0][idx]), r.h_v[0][sample]), t
    s = dS.read()
    assert s["scale"] == 2.0 ** 14 and s["count"] == 24 and s["skipped_steps"] == 1
    pl.close()


@pytest.mark.timeout(1500)
def test_c5_ragged_step_full_size():
    """C5: 500 tensors with log-uniform sizes summing to 1.5e9 parameters, lr 1e-3, momentum 0.9,
    weight decay 1e-4, dynamic scale from 2^12, 0.1 % NaN injected at step 7, 20 steps. The oracle
    runs its own 20 steps from the same generated inputs; masters, momenta and binary16 copies are
    compared bit for bit in full after steps 0, 6, 7, 8 and 19 and on a fixed sample of 2^20
    elements per step otherwise; the scaler after every step."""
    import concurrent.futures as cf

    require_gpu()
    hp = workloads.C5Hyper()
    sizes = workloads.c5_sizes()
    total = int(sizes.sum())
    first = np.concatenate([[0], np.cumsum(sizes)[:-1]])
    print(f"C5 generating {sizes.size} tensors, {total} parameters", flush=True)
    with cf.ThreadPoolExecutor(16) as ex:
        tens = list(ex.map(lambda a: workloads.c5_tensor(a[0], a[1]), enumerate(sizes)))
    nan_idx = workloads.c5_nan_indices(total)
    nan_t = np.searchsorted(first, nan_idx, side="right") - 1
    h_w = [t.w32 for t in tens]
    h_v = [np.zeros(s, np.float32) for s in sizes]
    h_16 = [oracle.f32_to_f16(w) for w in h_w]
    h_g = [np.empty(s, np.uint16) for s in sizes]
    d_w = [dev_f32(w) for w in h_w]
    d_v = [torch.zeros(int(s), dtype=torch.float32, device="cuda") for s in sizes]
    d_g = [torch.empty(int(s), dtype=torch.float16, device="cuda") for s in sizes]
    d_16 = [mp.round_f32_to_f16(w) for w in d_w]
    pl = mp.ParamList(d_w, d_v, d_g, d_16)
    dS, oS = scaler_pair(hp.scale, hp.dynamic, hp.growth_interval)
    rng = np.random.Generator(np.random.PCG64(55))
    samp_t = rng.integers(0, sizes.size, 1 << 20)
    samp_i = (rng.random(1 << 20) * sizes[samp_t]).astype(np.int64)

    def set_grads(scale, inject):
        def one(t):
            g = workloads.grads_at_scale(tens[t].g_true, scale)
            if inject:
                sel = nan_idx[nan_t == t] - first[t]
                g[sel] = workloads.F16_QNAN
            h_g[t][:] = g
            d_g[t].copy_(torch.from_numpy(g.view(np.int16)).view(torch.float16))
        with cf.ThreadPoolExecutor(8) as ex:
            list(ex.map(one, range(sizes.size)))

    def full_compare(step):
        torch.cuda.synchronize()
        for t in range(sizes.size):
            assert same_f32_bits(host_f32(d_w[t]), h_w[t]), (step, t)
            assert same_f32_bits(host_f32(d_v[t]), h_v[t]), (step, t)
            assert same_f16_bits(host_bits16(d_16[t]), h_16[t]), (step, t)

    g_scale = None
    for step in range(hp.steps):
        inject = step == hp.nan_step
        if oS.scale != g_scale or inject or step == hp.nan_step + 1:
            g_scale = oS.scale
            set_grads(g_scale, inject)
        print(f"C5 step {step} scale {oS.scale}", flush=True)
        mp.step(pl, dS, hp.lr, hp.momentum, hp.weight_decay)
        flag = oracle.step(h_w, h_v, h_g, h_16, hp.lr, hp.momentum, hp.weight_decay, oS.inv_scale)
        assert flag == (1 if inject else 0)
        dS.update(); oracle.scaler_update(oS, flag)
        assert_scaler(dS, oS)
        if step in (0, hp.nan_step - 1, hp.nan_step, hp.nan_step + 1, hp.steps - 1):
            full_compare(step)
        else:
            torch.cuda.synchronize()
            for t in np.unique(samp_t)[:64]:
                sel = samp_i[samp_t == t]
                idx = torch.from_numpy(sel).cuda()
                assert same_f32_bits(host_f32(d_w[t][idx]), h_w[t][sel]), (step, t)
                assert same_f32_bits(host_f32(d_v[t][idx]), h_v[t][sel]), (step, t)
    s = dS.read()
    assert s["scale"] == 2.0 ** 11 and s["count"] == 12 and s["skipped_steps"] == 1
    pl.close()
