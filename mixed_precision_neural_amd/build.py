"""Builds libmp.so (the HIP kernels and the C-ABI) in-tree for gfx950 with hipcc, and
libmp_probe.so (the measurement probes of include/mp_probe.h, linked against libmp.so).

Every translation unit is compiled with
  -ffp-contract=off   no fused multiply-add anywhere (the update is bit-exact
                      against a separately rounded multiply and add),
  -packed-fp32-ops off (target feature) the compiler emits no packed FP32 ops,
and never with fast-math or denormal flushing.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libmp.so")
PROBE_LIB = os.path.join(HERE, "libmp_probe.so")
SOURCES = ["mp_common.hip", "mp_step.hip", "mp_gemm.hip", "mp_aux.hip", "mp_stats.hip", "mp_reduce.hip",
           "mp_noalloc.hip"]
PROBE_SOURCES = ["mp_probe.hip"]
# Per-source flags. The matrix-core probe keeps its MFMA accumulators in VGPRs: with the
# compiler's default (AGPRs for a kernel of one block per CU) it shuffled the 16x16x32
# accumulators between register files around every MFMA and could not issue back to back.
SOURCE_FLAGS = {"mp_probe.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off", "-fno-fast-math",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def _compile(src: str, extra: list[str]) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *SOURCE_FLAGS.get(src, []), *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def _link(path: str, objs: list[str], libs: list[str]) -> None:
    tmp = path + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs, *libs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, path)


def build(verbose: bool = False, extra: list[str] | None = None) -> str:
    """Compiles every source, links libmp.so and libmp_probe.so next to this file. Returns the
    path of libmp.so."""
    os.makedirs(BUILD, exist_ok=True)
    extra = list(extra or [])
    srcs = SOURCES + PROBE_SOURCES
    with cf.ThreadPoolExecutor(max_workers=len(srcs)) as ex:
        objs = dict(zip(srcs, ex.map(lambda s: _compile(s, extra), srcs)))
    _link(LIB, [objs[s] for s in SOURCES], [])
    _link(PROBE_LIB, [objs[s] for s in PROBE_SOURCES], [f"-L{HERE}", "-lmp", "-Wl,-rpath,$ORIGIN"])
    if verbose:
        print(f"built {LIB} and {PROBE_LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])
