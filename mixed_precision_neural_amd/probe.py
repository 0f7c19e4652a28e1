"""Binding of libmp_probe.so (include/mp_probe.h): the achievable HBM stream rates, and the shader
clock and MFMA rate under a binary16 matrix-core load with constant or random operands, measured
beside the datasheet peaks. Argument marshalling only; the probes run in their own HIP kernels.
The import fails loudly when the library is missing.
"""
from __future__ import annotations

import ctypes as C
import os

import torch

from . import _check, _stream

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmp_probe.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "mp_probe.h")
READ, WRITE, COPY = 0, 1, 2
CONSTANT, RANDOM = 0, 1      # operand kinds of the matrix-core probe
MFMA_32X32X16, MFMA_16X16X32 = 0, 1   # its MFMA forms

_lib = None


def lib() -> C.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing; build it first (python -c "
                              "'import __graft_entry__ as g; g.build()')")
        L = C.CDLL(LIB_PATH)
        vp, i32 = C.c_void_p, C.c_int32
        L.mp_probe_hbm.argtypes = [i32, vp, vp, C.c_size_t, i32, i32, vp]
        L.mp_probe_hbm.restype = C.c_int
        L.mp_probe_mfma_clock.argtypes = [i32, i32, i32, i32, vp, C.POINTER(i32), vp]
        L.mp_probe_mfma_clock.restype = C.c_int
        _lib = L
    return _lib


def hbm(mode: int, src: torch.Tensor | None, dst: torch.Tensor, nbytes: int, blocks: int = 0,
        nontemporal: bool = False, stream=None) -> None:
    """One launch of the stream probe over nbytes (see mp_probe_hbm)."""
    _check(lib().mp_probe_hbm(int(mode), C.c_void_p(src.data_ptr() if src is not None else 0),
                              C.c_void_p(dst.data_ptr()), int(nbytes), int(blocks), int(bool(nontemporal)),
                              _stream(stream)), "mp_probe_hbm")


def mfma_clock(blocks: int, iters: int, out: torch.Tensor, operands: int = CONSTANT,
               shape: int = MFMA_16X16X32, stream=None) -> int:
    """One launch of the matrix-core probe (operands: CONSTANT or RANDOM; shape: MFMA_32X32X16 or
    MFMA_16X16X32); out: int64 GPU tensor of 4 * blocks entries. Returns the constant counter's
    rate in kHz."""
    if out.dtype != torch.int64 or out.numel() < 4 * blocks or not out.is_cuda:
        raise ValueError("out must be an int64 GPU tensor of 4 * blocks entries")
    khz = C.c_int32(0)
    _check(lib().mp_probe_mfma_clock(int(blocks), int(iters), int(operands), int(shape), C.c_void_p(out.data_ptr()),
                                     C.byref(khz), _stream(stream)), "mp_probe_mfma_clock")
    return int(khz.value)
