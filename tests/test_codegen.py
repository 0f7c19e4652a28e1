"""Instruction-level guarantees of the gfx950 build, checked on the generated assembly.

The update follows "Mixed Precision Training", long-form analysis page, §3.4 "The
Integrated Training Procedure", Step 7: each FP32 operation rounds on its own, so the
update kernel must contain no fused multiply-add of any kind. Every FP32 -> binary16
rounding is meant as "round the FP32 value": a mixed-precision v_fma_mix*_f16 (which
rounds the exact product once) must not appear in any kernel, or two kernels computing
the same expression can differ in the last bit on binary16 ties.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mixed_precision_neural_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


def build_flags():
    """The library's own compile flags (build.py loaded by path: no package import)."""
    import importlib.util
    spec = importlib.util.spec_from_file_location("_mp_build", os.path.join(ROOT, "mixed_precision_neural_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod.FLAGS


def device_asm(name, tmp_path):
    out = tmp_path / (name + ".s")
    cmd = [HIPCC, *build_flags(), "--cuda-device-only", "-S",
           os.path.join(CSRC, name + ".hip"), "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True)
    return out.read_text()


def kernel_bodies(asm):
    """{symbol: text} for every kernel in the assembly, from its label to its .Lfunc_end
    marker (a kernel can have several s_endpgm, e.g. an early return)."""
    bodies, name, cur = {}, None, []
    for line in asm.splitlines():
        m = re.match(r"^(_Z\w+):", line)
        if m:
            name, cur = m.group(1), []
            bodies[name] = cur
        elif name is not None:
            if line.startswith(".Lfunc_end"):
                name = None
            else:
                cur.append(line)
    return {k: "\n".join(v) for k, v in bodies.items()}


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
@pytest.mark.parametrize("name", ["mp_step", "mp_aux", "mp_gemm", "mp_reduce"])
def test_no_mixed_precision_fma(name, tmp_path):
    asm = device_asm(name, tmp_path)
    assert "v_fma_mix" not in asm and "v_mad_mix" not in asm


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_update_kernel_has_no_fused_multiply_add(tmp_path):
    """The SGD and Nesterov bodies (template kinds 0 and 1) are plain multiplies and adds. The
    Adagrad body (kind 2) needs a correctly rounded square root and division, whose expansions
    use fused operations internally; its bits are pinned against the oracle instead, and here it
    must contain the IEEE division sequence and no mixed-precision FMA."""
    bodies = kernel_bodies(device_asm("mp_step", tmp_path))
    kinds = {k: v for k, v in bodies.items() if "13update_kernel" in k}
    assert len(kinds) == 3, sorted(kinds)
    for sym, body in kinds.items():
        assert "global_load_dwordx4" in body and "global_store_dwordx4" in body, sym   # whole body read
        if "ILi0E" in sym or "ILi1E" in sym:
            assert not re.search(r"\bv_(fma|fmac|mad|mac|pk_fma|pk_mul|pk_add)\w*", body), sym
        else:
            assert "v_div_fixup_f32" in body and "v_div_fmas_f32" in body, sym
            assert "v_fma_mix" not in body, sym


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_bn_apply_uses_correctly_rounded_sqrt_and_division(tmp_path):
    """The batch-norm normalization computes 1 / sqrt(var + eps) with a correctly rounded square
    root (v_sqrt_f32 refined by its residual, with the scaling for small inputs) and the IEEE
    division sequence, so its bits match the oracle's FP32 sqrtf and division."""
    bodies = kernel_bodies(device_asm("mp_reduce", tmp_path))
    apply = {k: v for k, v in bodies.items() if "bn_apply_kernel" in k}
    assert len(apply) == 2, sorted(apply)
    for sym, body in apply.items():
        assert "v_sqrt_f32" in body and re.search(r"v_fma_f32 v\d+, -v\d+, v\d+, v\d+", body), sym
        assert "v_div_fixup_f32" in body and "v_div_fmas_f32" in body, sym


def back_edge_loops(body):
    """Bodies of the loops in one kernel's assembly: the lines from a label to a branch
    back to it."""
    lines = body.splitlines()
    labels = {}
    for i, line in enumerate(lines):
        m = re.match(r"^(\.LBB\w+):", line)
        if m:
            labels[m.group(1)] = i
    loops = []
    for i, line in enumerate(lines):
        m = re.search(r"s_c?branch\w* (\.LBB\w+)", line)
        if m and m.group(1) in labels and labels[m.group(1)] < i:
            loops.append("\n".join(lines[labels[m.group(1)]:i]))
    return loops


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_pipelined_gemm_loops_use_16x16x32_and_no_scratch(tmp_path):
    """The 256 x 256 kernels issue only v_mfma_f32_16x16x32_f16. In every kernel with a
    binary16 output (the ones the training step runs; FP32 output serves tests), neither
    pipelined loop (128 MFMAs per pass) touches scratch memory, and the forward and dgrad
    layouts (reduction-contiguous A) spill nothing at all. (Register spills of the
    computing waves once cost 5-15 MiB of scratch traffic per launch.)"""
    bodies = kernel_bodies(device_asm("mp_gemm", tmp_path))
    big = {k: v for k, v in bodies.items() if "gemm_kernel" in k and "ILi256ELi256ELi2ELi4E" in k}
    assert len(big) >= 10
    for name, body in big.items():
        m = re.search(r"ILi256ELi256ELi2ELi4ELb(\d)ELb(\d)ELi(\d)ELi(\d)E", name)
        a_kc, epi = m.group(1) == "1", int(m.group(3))
        mfmas = set(re.findall(r"v_mfma_\w+", body))
        assert mfmas == {"v_mfma_f32_16x16x32_f16"}, (name, mfmas)
        pipelined = [lp for lp in back_edge_loops(body) if lp.count("v_mfma_") == 128]
        assert len(pipelined) == 2, name                    # the loading and the computing waves' loop
        if epi == 0:
            continue
        for lp in pipelined:
            assert "scratch_" not in lp, name
        if a_kc and epi != 0:
            assert "scratch_" not in body, name
