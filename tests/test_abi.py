"""The C-ABI library loads, exports every function include/mp.h declares, and rejects bad
arguments on the host before anything is launched (no GPU needed for these paths)."""
import ctypes as C
import subprocess

import pytest

import mixed_precision_neural_amd as mp


def test_header_declares_the_boundary():
    names = set(mp.header_functions())
    for n in ("mp_linear_fwd", "mp_linear_dgrad", "mp_linear_wgrad", "mp_step", "mp_scaler_update",
              "mp_scaler_init", "mp_param_list_create", "mp_param_list_destroy"):
        assert n in names


def test_library_exports_every_declared_symbol():
    L = mp.lib()
    for n in mp.header_functions():
        assert hasattr(L, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", mp.LIB_PATH], capture_output=True, text=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    missing = set(mp.header_functions()) - exported
    assert not missing, missing


def test_status_strings():
    L = mp.lib()
    assert L.mp_status_string(0) == b"MP_OK"
    assert L.mp_status_string(1) == b"MP_ERR_INVALID_ARGUMENT"
    assert L.mp_status_string(99) == b"MP_ERR_UNKNOWN"
    assert L.mp_version().startswith(b"libmp")


INVALID = 1
UNSUPPORTED = 3
P = C.c_void_p(0x1000)          # never dereferenced: every call below fails validation first


@pytest.mark.parametrize("args", [
    (P, 8, P, 8, P, 8, 0, -1, 8, 8),        # negative M
    (P, 8, P, 8, P, 8, 0, 8, 8, -1),        # negative K
    (P, 4, P, 8, P, 8, 0, 8, 8, 8),         # ldx < K
    (P, 8, P, 8, P, 4, 0, 8, 8, 8),         # ldy < N
    (None, 8, P, 8, P, 8, 0, 8, 8, 8),      # null X
    (P, 8, P, 8, P, 8, 7, 8, 8, 8),         # bad dtype
])
def test_linear_fwd_validation(args):
    assert mp.lib().mp_linear_fwd(*args, None) == INVALID


def test_dgrad_wgrad_validation():
    L = mp.lib()
    assert L.mp_linear_dgrad(P, 8, P, 4, P, 8, 0, 8, 8, 8, None) == INVALID      # ldw < K
    assert L.mp_linear_wgrad(P, 4, P, 8, P, 8, 0, 8, 8, 8, None, None) == INVALID  # lddy < N
    assert L.mp_linear_wgrad(P, 8, P, 8, P, 8, 1, 8, 8, 8, P, None) == INVALID     # flag with FP32 out


def test_empty_problems_are_no_ops():
    L = mp.lib()
    assert L.mp_linear_fwd(None, 0, None, 0, None, 0, 0, 0, 5, 5, None) == 0
    assert L.mp_linear_dgrad(None, 0, None, 0, None, 0, 0, 5, 5, 0, None) == 0
    assert L.mp_linear_wgrad(None, 0, None, 0, None, 0, 0, 5, 0, 5, None, None) == 0
    assert L.mp_round_f32_to_f16(None, None, 0, None) == 0
    assert L.mp_act_fwd(0, None, None, 0, None) == 0


def test_param_list_and_step_validation():
    L = mp.lib()
    h = C.c_void_p()
    assert L.mp_param_list_create(None, -1, C.byref(h), None) == INVALID
    bad = (mp._Param * 1)()
    bad[0] = mp._Param(None, 0x1000, 0x1000, 0x1000, 10)           # null master
    assert L.mp_param_list_create(bad, 1, C.byref(h), None) == INVALID
    bad[0] = mp._Param(0x1000, 0x1000, 0x1000, 0x1000, -5)         # negative numel
    assert L.mp_param_list_create(bad, 1, C.byref(h), None) == INVALID
    empty = (mp._Param * 1)()
    empty[0] = mp._Param(None, None, None, None, 0)                 # empty tensors are fine
    assert L.mp_param_list_create(empty, 1, C.byref(h), None) == 0
    assert L.mp_param_list_numel(h) == 0
    sgd = mp._Sgd(0.01, 0.9, 0.0)
    assert L.mp_step(None, sgd, P, 0, None) == INVALID
    assert L.mp_step(h, sgd, None, 0, None) == INVALID
    assert L.mp_step(h, sgd, P, 0x80, None) == UNSUPPORTED
    assert L.mp_step(h, sgd, P, 0, None) == 0                       # nothing to do
    assert L.mp_param_list_destroy(h) == 0
    assert L.mp_param_list_destroy(None) == 0


@pytest.mark.parametrize("scale", [0.0, -1.0, 3.0, 0.5, 2.0 ** 65, float("inf"), float("nan")])
def test_scaler_rejects_non_power_of_two(scale):
    assert mp.lib().mp_scaler_init(P, scale, 1, 2000, None) == INVALID


def test_scaler_rejects_bad_interval():
    assert mp.lib().mp_scaler_init(P, 1024.0, 1, 0, None) == INVALID
    assert mp.lib().mp_scaler_update(None, None) == INVALID


def test_product_package_does_not_touch_the_oracle():
    import os
    pkg = os.path.dirname(mp.__file__)
    for root, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(root, f)).read()
                assert "import oracle" not in text and "from oracle" not in text, f
                assert "oracle.h" not in text and "liboracle" not in text, f


def test_loss_workspace_sizes_and_validation():
    """The losses reduce through a caller workspace: its size is one FP32 partial per block (at
    most 1024 blocks), and a missing, short or misaligned workspace is rejected before launch."""
    L = mp.lib()
    assert L.mp_loss_mse_workspace(0, 5) == 0 and L.mp_loss_softmax_ce_workspace(3, 0) == 0
    assert L.mp_loss_mse_workspace(1, 8) == 4                       # one block
    assert L.mp_loss_mse_workspace(4096, 4096) == 4096               # capped at 1024 blocks
    assert L.mp_loss_softmax_ce_workspace(64, 10) == 64              # 4 rows per block
    assert L.mp_loss_softmax_ce_workspace(10 ** 6, 10) == 4096
    need = L.mp_loss_mse_workspace(8, 8)
    assert L.mp_loss_mse(P, P, 8, 8, C.c_float(1.0), P, P, P, None, need, None) == INVALID
    assert L.mp_loss_mse(P, P, 8, 8, C.c_float(1.0), P, P, P, P, need - 1, None) == INVALID
    assert L.mp_loss_mse(P, P, 8, 8, C.c_float(1.0), P, P, P, C.c_void_p(0x1002), need, None) == INVALID
    assert L.mp_loss_mse(None, None, 0, 8, C.c_float(1.0), P, P, None, None, 0, None) == 0
    need = L.mp_loss_softmax_ce_workspace(8, 10)
    assert L.mp_loss_softmax_ce(P, P, 8, 10, P, P, P, None, need, None) == INVALID
    assert L.mp_loss_softmax_ce(P, P, 8, 10, P, P, P, P, need - 4, None) == INVALID
    assert L.mp_loss_softmax_ce(P, P, -1, 10, P, P, P, P, need, None) == INVALID


def test_probe_library_exports_and_validation():
    """libmp_probe.so (the measurement probes of include/mp_probe.h) exports every function its
    header declares and rejects bad arguments on the host."""
    import re

    from mixed_precision_neural_amd import probe
    names = set(re.findall(r"^\s*mp_status\s+(mp_\w+)\s*\(", open(probe.HEADER_PATH).read(), re.M))
    assert names == {"mp_probe_hbm", "mp_probe_mfma_clock"}
    out = subprocess.run(["nm", "-D", "--defined-only", probe.LIB_PATH], capture_output=True, text=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    assert names <= exported
    L = probe.lib()
    assert L.mp_probe_hbm(7, P, P, 4096, 0, 0, None) == INVALID          # unknown mode
    assert L.mp_probe_hbm(0, P, P, 4000, 0, 0, None) == INVALID          # not a multiple of 4096
    assert L.mp_probe_hbm(0, None, P, 4096, 0, 0, None) == INVALID       # read needs a source
    assert L.mp_probe_hbm(2, P, C.c_void_p(0x1008), 4096, 0, 0, None) == INVALID   # misaligned
    khz = C.c_int32()
    k16 = probe.MFMA_16X16X32
    assert L.mp_probe_mfma_clock(0, 10, probe.CONSTANT, k16, P, C.byref(khz), None) == INVALID
    assert L.mp_probe_mfma_clock(1, 10, probe.RANDOM, k16, None, C.byref(khz), None) == INVALID
    assert L.mp_probe_mfma_clock(1, 10, 2, k16, P, C.byref(khz), None) == INVALID     # unknown operand kind
    assert L.mp_probe_mfma_clock(1, 10, probe.RANDOM, 2, P, C.byref(khz), None) == INVALID   # unknown MFMA form


def test_softmax_workspace_and_wait_setting():
    """The softmax workspace covers either form: the two-pass form's (max, sum) per (row, 32K
    segment) or the single-read form's 16-byte slot per block (at most 1024 blocks); a short,
    misaligned or mis-pitched call is rejected before any launch. The
    single-read wait is a process-wide setting in microseconds: 200 by default, clamped to
    100000, queried by a negative value, and every call returns the previous setting."""
    L = mp.lib()
    assert L.mp_softmax_workspace(0, 5) == 0 and L.mp_softmax_workspace(5, 0) == 0
    assert L.mp_softmax_workspace(1, 8) == 256 * 16                  # one row: 256 slots
    assert L.mp_softmax_workspace(64, 793471) == 1024 * 16           # slots capped at 1024 blocks
    assert L.mp_softmax_workspace(100000, 2 ** 20) == 100000 * 32 * 8  # two-pass pairs dominate
    nbn = L.mp_bn_stats_workspace(4, 16)
    assert L.mp_bn_stats(P, 4, 16, 16, P, P, C.c_void_p(0x1002), nbn, None) == INVALID   # misaligned
    need = L.mp_softmax_workspace(4, 16)
    assert L.mp_softmax(P, 4, 16, 16, P, 16, C.c_void_p(0x1004), need, None) == INVALID   # misaligned
    assert L.mp_softmax(P, 4, 16, 16, P, 16, P, need - 8, None) == INVALID               # short
    assert L.mp_softmax(P, 4, 16, 8, P, 16, P, need, None) == INVALID                    # ldx < cols
    prev = L.mp_softmax_wait_us(-1)
    try:
        assert prev == 200
        assert L.mp_softmax_wait_us(0) == 200 and L.mp_softmax_wait_us(-5) == 0
        assert L.mp_softmax_wait_us(10 ** 9) == 0 and L.mp_softmax_wait_us(-1) == 100000
    finally:
        L.mp_softmax_wait_us(prev)
    assert L.mp_softmax_wait_us(-1) == prev


def test_atomic_targets_must_be_word_aligned():
    """Words the kernels update atomically or read whole (the wgrad overflow flag, the scaler,
    the running |g| maximum and its non-finite flag, the loss) must be 4-byte aligned; a
    misaligned one is an argument error before any launch."""
    L = mp.lib()
    odd = C.c_void_p(0x1002)
    assert L.mp_linear_wgrad(P, 64, P, 64, P, 64, 0, 64, 64, 64, odd, None) == INVALID
    assert L.mp_scaler_init(odd, C.c_float(1024.0), 1, 2000, None) == INVALID
    assert L.mp_scaler_update(odd, None) == INVALID
    assert L.mp_loss_mse(P, P, 8, 8, C.c_float(1.0), odd, P, P, P, 1 << 12, None) == INVALID
    assert L.mp_loss_mse(P, P, 8, 8, C.c_float(1.0), P, odd, P, P, 1 << 12, None) == INVALID
    assert L.mp_loss_softmax_ce(P, P, 8, 10, odd, P, P, P, 1 << 12, None) == INVALID
    assert L.mp_scaler_init_from_absmax(odd, P, C.c_float(2.0), 1, 2000, None) == INVALID
    assert L.mp_scaler_init_from_absmax(P, odd, C.c_float(2.0), 1, 2000, None) == INVALID
    # the list handles below are never dereferenced: the pointer checks come first
    assert L.mp_absmax(P, odd, None, None) == INVALID
    assert L.mp_absmax(P, P, odd, None) == INVALID
