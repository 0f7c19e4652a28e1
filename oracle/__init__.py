"""Plain CPU oracle for the mixed-precision training hot path.

TEST INFRASTRUCTURE ONLY. The test-suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` are the only callers; the product package
never imports this module and shares no code with it.

The arithmetic lives in ``oracle.c`` (plain C11, built by ``build()`` with gcc
and ``-ffp-contract=off``); this module loads it with ctypes and marshals
numpy arrays. binary16 values travel as ``uint16`` bit patterns.

Sources, by page title: "Mixed Precision Training", the long-form analysis
page (paper-graph-ui.vercel.app), §3.4 — FP32 master copy, loss scaling,
FP16 arithmetic with FP32 accumulation, the integrated training procedure
(Steps 1-7) and the choice of the loss-scaling factor.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile ``liboracle.so`` next to its source with the host compiler."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math",
               "-fPIC", "-shared", "-pthread", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


class Param(C.Structure):
    _fields_ = [("master", C.c_void_p), ("momentum", C.c_void_p), ("grad", C.c_void_p),
                ("weight16", C.c_void_p), ("numel", C.c_int64)]


class Scaler(C.Structure):
    _fields_ = [("scale", C.c_float), ("inv_scale", C.c_float), ("count", C.c_int32),
                ("growth_interval", C.c_int32), ("found_inf", C.c_uint32),
                ("dynamic", C.c_uint32), ("skipped_steps", C.c_uint32)]

    def as_dict(self) -> dict:
        return {f: getattr(self, f) for f, _ in self._fields_}


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        L = C.CDLL(_LIB)
        vp, i64, i32, u16p = C.c_void_p, C.c_int64, C.c_int32, C.c_void_p
        L.or_f16_to_f32.argtypes = [C.c_uint16]; L.or_f16_to_f32.restype = C.c_float
        L.or_f32_to_f16.argtypes = [C.c_float]; L.or_f32_to_f16.restype = C.c_uint16
        L.or_f32_to_f16_array.argtypes = [vp, vp, i64]
        L.or_f16_to_f32_array.argtypes = [vp, vp, i64]
        L.or_f32bits_to_f16_range.argtypes = [C.c_uint64, C.c_uint64, vp]
        for n in ("or_linear_fwd", "or_linear_dgrad", "or_linear_wgrad"):
            getattr(L, n).argtypes = [vp, i64, vp, i64, vp, i64, C.c_int, i64, i64, i64]
        for n in ("or_linear_fwd_at", "or_linear_dgrad_at", "or_linear_wgrad_at"):
            getattr(L, n).argtypes = [vp, i64, vp, i64, i64, vp, vp, i64, vp]
        L.or_check_overflow.argtypes = [vp, i32]; L.or_check_overflow.restype = C.c_uint32
        L.or_sgd_update.argtypes = [vp, i32, C.c_float, C.c_float, C.c_float, C.c_float]
        L.or_step.argtypes = [vp, i32, C.c_float, C.c_float, C.c_float, C.c_float]
        L.or_step.restype = C.c_uint32
        L.or_opt_update.argtypes = [vp, i32, i32, C.c_float, C.c_float, C.c_float, C.c_float, C.c_float]
        L.or_step_opt.argtypes = [vp, i32, i32, C.c_float, C.c_float, C.c_float, C.c_float, C.c_float]
        L.or_step_opt.restype = C.c_uint32
        L.or_absmax_f32.argtypes = [vp, i64, C.c_float, C.POINTER(C.c_uint32)]
        L.or_absmax_f32.restype = C.c_float
        L.or_absmax_f16.argtypes = [vp, i64, C.c_float, C.POINTER(C.c_uint32)]
        L.or_absmax_f16.restype = C.c_float
        L.or_scale_from_absmax.argtypes = [C.c_float, C.c_float]
        L.or_scale_from_absmax.restype = C.c_float
        L.or_scaler_init.argtypes = [C.POINTER(Scaler), C.c_float, i32, i32]
        L.or_scaler_update.argtypes = [C.POINTER(Scaler)]
        L.or_relu_fwd.argtypes = [u16p, u16p, i64]
        L.or_relu_bwd.argtypes = [u16p, u16p, u16p, i64]
        L.or_gelu_fwd.argtypes = [u16p, u16p, i64]
        L.or_gelu_bwd.argtypes = [u16p, u16p, u16p, i64]
        L.or_softmax_ce.argtypes = [u16p, vp, i64, i64, C.c_double, u16p]
        L.or_softmax_ce.restype = C.c_double
        L.or_mse.argtypes = [u16p, u16p, i64, i64, C.c_double, C.c_double, u16p]
        L.or_mse.restype = C.c_double
        L.or_mse_grad_f64.argtypes = [u16p, u16p, i64, i64, i64, C.c_double, vp]
        L.or_bn_stats.argtypes = [u16p, i64, i64, i64, vp, vp]
        L.or_bn_apply.argtypes = [u16p, i64, i64, i64, vp, vp, vp, vp, C.c_float, u16p, i64]
        L.or_softmax.argtypes = [u16p, i64, i64, i64, u16p, i64]
        L.or_set_threads.argtypes = [i32]
        L.or_get_threads.restype = i32
        _lib = L
    return _lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(C.c_void_p)


def _c(a, dtype) -> np.ndarray:
    a = np.asarray(a)
    if a.dtype != dtype:
        raise TypeError(f"expected {dtype}, got {a.dtype}")
    return np.ascontiguousarray(a)


def set_threads(n: int) -> None:
    lib().or_set_threads(int(n))


def threads() -> int:
    return int(lib().or_get_threads())


# ---------------------------------------------------------------- codec
def f16_to_f32(h) -> np.ndarray:
    h = _c(h, np.uint16)
    out = np.empty(h.shape, np.float32)
    lib().or_f16_to_f32_array(_p(h), _p(out), h.size)
    return out


def f32_to_f16(x) -> np.ndarray:
    x = _c(x, np.float32)
    out = np.empty(x.shape, np.uint16)
    lib().or_f32_to_f16_array(_p(x), _p(out), x.size)
    return out


def f32bits_to_f16(lo: int, hi: int) -> np.ndarray:
    out = np.empty(hi - lo, np.uint16)
    lib().or_f32bits_to_f16_range(lo, hi, _p(out))
    return out


# ---------------------------------------------------------------- GEMMs
def _gemm(name, a, b, rows, cols, out_f16):
    a = _c(a, np.uint16); b = _c(b, np.uint16)
    out = np.empty((rows, cols), np.uint16 if out_f16 else np.float32)
    fn = getattr(lib(), name)
    return fn, a, b, out


def linear_fwd(X, W, out_f16=False):
    """Y[M,N] = X[M,K] . W[N,K]^T, FP32 accumulation in ascending k."""
    M, K = X.shape; N, K2 = W.shape
    assert K == K2
    fn, X, W, Y = _gemm("or_linear_fwd", X, W, M, N, out_f16)
    fn(_p(X), K, _p(W), K, _p(Y), N, int(out_f16), M, N, K)
    return Y


def linear_dgrad(dY, W, out_f16=False):
    """dX[M,K] = dY[M,N] . W[N,K], FP32 accumulation in ascending n."""
    M, N = dY.shape; N2, K = W.shape
    assert N == N2
    fn, dY, W, dX = _gemm("or_linear_dgrad", dY, W, M, K, out_f16)
    fn(_p(dY), N, _p(W), K, _p(dX), K, int(out_f16), M, N, K)
    return dX


def linear_wgrad(dY, X, out_f16=False):
    """dW[N,K] = dY[M,N]^T . X[M,K], FP32 accumulation in ascending m."""
    M, N = dY.shape; M2, K = X.shape
    assert M == M2
    fn, dY, X, dW = _gemm("or_linear_wgrad", dY, X, N, K, out_f16)
    fn(_p(dY), N, _p(X), K, _p(dW), K, int(out_f16), M, N, K)
    return dW


def _at(name, a, lda, b, ldb, red, rows, cols):
    a = _c(a, np.uint16); b = _c(b, np.uint16)
    rows = np.ascontiguousarray(rows, np.int64); cols = np.ascontiguousarray(cols, np.int64)
    out = np.empty(rows.size, np.float32)
    getattr(lib(), name)(_p(a), lda, _p(b), ldb, red, _p(rows), _p(cols), rows.size, _p(out))
    return out


def linear_fwd_at(X, W, rows, cols):
    return _at("or_linear_fwd_at", X, X.shape[1], W, W.shape[1], X.shape[1], rows, cols)


def linear_dgrad_at(dY, W, rows, cols):
    return _at("or_linear_dgrad_at", dY, dY.shape[1], W, W.shape[1], dY.shape[1], rows, cols)


def linear_wgrad_at(dY, X, rows, cols):
    return _at("or_linear_wgrad_at", dY, dY.shape[1], X, X.shape[1], dY.shape[0], rows, cols)


# ---------------------------------------------------------------- optimizer sweep
def _params(masters, moms, grads, w16s):
    n = len(masters)
    arr = (Param * max(n, 1))()
    for i in range(n):
        for a, dt in ((masters[i], np.float32), (moms[i], np.float32),
                      (grads[i], np.uint16), (w16s[i], np.uint16)):
            if a.dtype != dt or not a.flags.c_contiguous:
                raise TypeError("oracle tensors must be contiguous with the stated dtype")
        assert masters[i].size == moms[i].size == grads[i].size == w16s[i].size
        arr[i] = Param(masters[i].ctypes.data, moms[i].ctypes.data, grads[i].ctypes.data,
                       w16s[i].ctypes.data, masters[i].size)
    return arr, n


def check_overflow(grads) -> int:
    """1 if any element of any gradient tensor is +-inf or NaN (Step 6)."""
    grads = [_c(g, np.uint16) for g in grads]
    n = len(grads)
    arr = (Param * max(n, 1))()
    for i, g in enumerate(grads):
        arr[i] = Param(None, None, g.ctypes.data, None, g.size)
    return int(lib().or_check_overflow(arr, n))


def sgd_update(masters, moms, grads, w16s, lr, momentum, weight_decay, inv_scale):
    arr, n = _params(masters, moms, grads, w16s)
    lib().or_sgd_update(arr, n, lr, momentum, weight_decay, inv_scale)


def step(masters, moms, grads, w16s, lr, momentum, weight_decay, inv_scale) -> int:
    """Check, then update in place only when no gradient is +-inf/NaN. Returns the flag."""
    arr, n = _params(masters, moms, grads, w16s)
    return int(lib().or_step(arr, n, lr, momentum, weight_decay, inv_scale))


SGD, NESTEROV, ADAGRAD = 0, 1, 2      # optimizer kinds of the sweep


def opt_update(kind, masters, moms, grads, w16s, lr, momentum, weight_decay, eps, inv_scale):
    """The update rule `kind` on every element, unconditionally (moms: v, or G for Adagrad)."""
    arr, n = _params(masters, moms, grads, w16s)
    lib().or_opt_update(arr, n, int(kind), lr, momentum, weight_decay, eps, inv_scale)


def step_opt(kind, masters, moms, grads, w16s, lr, momentum, weight_decay, eps, inv_scale) -> int:
    """Check, then the update rule `kind` in place when no gradient is +-inf/NaN. Returns the flag."""
    arr, n = _params(masters, moms, grads, w16s)
    return int(lib().or_step_opt(arr, n, int(kind), lr, momentum, weight_decay, eps, inv_scale))


def absmax(tensors, running: float = 0.0):
    """(max(running, max |x| over the finite elements), 1 if any element is +-inf/NaN else 0)
    over a list of float32 arrays or binary16 bit-pattern (uint16) arrays."""
    nonfinite = C.c_uint32(0)
    m = float(running)
    for t in tensors:
        t = np.ascontiguousarray(t)
        if t.dtype == np.float32:
            m = lib().or_absmax_f32(_p(t), t.size, m, C.byref(nonfinite))
        elif t.dtype == np.uint16:
            m = lib().or_absmax_f16(_p(t), t.size, m, C.byref(nonfinite))
        else:
            raise TypeError("absmax takes float32 or uint16 (binary16 bits) arrays")
    return float(m), int(nonfinite.value)


def scale_from_absmax(amax: float, headroom: float = 2.0) -> float:
    """Largest power of two S with S * headroom * amax <= 65504, within [1, 2^64]."""
    return float(lib().or_scale_from_absmax(amax, headroom))


def scaler_init(init_scale, dynamic, growth_interval) -> Scaler:
    s = Scaler()
    lib().or_scaler_init(C.byref(s), init_scale, int(dynamic), int(growth_interval))
    return s


def scaler_update(s: Scaler, found_inf: int) -> Scaler:
    s.found_inf = int(found_inf)
    lib().or_scaler_update(C.byref(s))
    return s


# ---------------------------------------------------------------- point-wise and losses
def relu_fwd(x):
    x = _c(x, np.uint16); y = np.empty_like(x)
    lib().or_relu_fwd(_p(x), _p(y), x.size); return y


def relu_bwd(x, dy):
    x = _c(x, np.uint16); dy = _c(dy, np.uint16); dx = np.empty_like(x)
    lib().or_relu_bwd(_p(x), _p(dy), _p(dx), x.size); return dx


def gelu_fwd(x):
    x = _c(x, np.uint16); y = np.empty_like(x)
    lib().or_gelu_fwd(_p(x), _p(y), x.size); return y


def gelu_bwd(x, dy):
    x = _c(x, np.uint16); dy = _c(dy, np.uint16); dx = np.empty_like(x)
    lib().or_gelu_bwd(_p(x), _p(dy), _p(dx), x.size); return dx


def softmax_ce(logits, labels, scale):
    """Returns (mean cross-entropy, RNE16(scale * dL/dlogits))."""
    logits = _c(logits, np.uint16); labels = np.ascontiguousarray(labels, np.int32)
    B, Cn = logits.shape
    d = np.empty_like(logits)
    loss = lib().or_softmax_ce(_p(logits), _p(labels), B, Cn, float(scale), _p(d))
    return loss, d


def mse(y, t, c, scale):
    """Returns (c * mean((y-t)^2), RNE16(scale * dL/dy))."""
    y = _c(y, np.uint16); t = _c(t, np.uint16)
    M, N = y.shape
    d = np.empty_like(y)
    loss = lib().or_mse(_p(y), _p(t), M, N, float(c), float(scale), _p(d))
    return loss, d


def mse_grad_f64(y, t, m_total, c):
    y = _c(y, np.uint16); t = _c(t, np.uint16)
    M, N = y.shape
    d = np.empty((M, N), np.float64)
    lib().or_mse_grad_f64(_p(y), _p(t), M, N, int(m_total), float(c), _p(d))
    return d


# ---------------------------------------------------------------- large reductions
# [A] §3.4 "FP16 Arithmetic with FP32 Accumulation": batch-normalization statistics and
# softmax sums are large reductions done in FP32 from binary16 tensors, and the
# normalization arithmetic is FP32.
def _rows(a) -> tuple:
    """(array, rows, cols, row pitch in elements) of a 2-D uint16 array whose rows are
    contiguous; a row-strided view is passed as it is."""
    a = np.asarray(a)
    if a.dtype != np.uint16 or a.ndim != 2:
        raise TypeError("expected a 2-D uint16 array")
    if a.strides[1] != 2 or a.strides[0] % 2 or a.strides[0] < 2 * a.shape[1]:
        a = np.ascontiguousarray(a)
    ld = a.strides[0] // 2 if a.shape[0] > 1 else a.shape[1]
    return a, a.shape[0], a.shape[1], max(ld, a.shape[1])


def bn_stats(x):
    """Per-channel (mean, population variance) in float64 over the rows of x[rows, C]."""
    x, rows, cols, ld = _rows(x)
    mean = np.empty(cols, np.float64); var = np.empty(cols, np.float64)
    lib().or_bn_stats(_p(x), rows, cols, ld, _p(mean), _p(var))
    return mean, var


def bn_apply(x, mean, var, gamma, beta, eps):
    """y = RNE16(((x - mean) * (1 / sqrt(var + eps))) * gamma + beta) in FP32, in that order."""
    x, rows, cols, ld = _rows(x)
    f = [np.ascontiguousarray(a, np.float32) for a in (mean, var, gamma, beta)]
    if any(a.shape != (cols,) for a in f):
        raise ValueError("per-channel arrays must have one value per column")
    y = np.empty((rows, cols), np.uint16)
    lib().or_bn_apply(_p(x), rows, cols, ld, *[_p(a) for a in f], float(eps), _p(y), cols)
    return y


def softmax(x):
    """Row-wise softmax of x[rows, cols] in float64, rounded once to binary16."""
    x, rows, cols, ld = _rows(x)
    y = np.empty((rows, cols), np.uint16)
    lib().or_softmax(_p(x), rows, cols, ld, _p(y), cols)
    return y
