"""Python binding of libmp, the mixed-precision training hot path on MI355X (gfx950).

Argument marshalling only: every step runs in the HIP kernels of ``libmp.so``;
PyTorch provides device memory and the current stream. binary16 tensors are
``torch.float16`` (any 2-byte dtype is accepted and passed as raw bits), FP32
tensors ``torch.float32``; every tensor must live on a GPU and be row-major
(unit stride in its last dimension).

The import fails loudly when ``libmp.so`` has not been built: there is no
fallback path.
"""
from __future__ import annotations

import ctypes as C
import os
import re

import torch

__all__ = [
    "MPError", "lib", "header_functions", "LIB_PATH", "HEADER_PATH",
    "linear_fwd", "linear_dgrad", "linear_wgrad", "linear_fwd_act", "linear_dgrad_act",
    "linear_fwd_act_deriv", "linear_dgrad_mul",
    "Scaler", "ParamList", "step", "step_opt", "TensorList", "absmax", "scaler_init_from_absmax",
    "round_f32_to_f16", "act_fwd", "act_bwd", "loss_softmax_ce", "loss_mse",
    "loss_softmax_ce_workspace", "loss_mse_workspace", "loss_mse_noalloc",
    "bn_stats", "bn_apply", "softmax", "softmax_wait_us",
    "MP_GRADS_PRECHECKED", "MP_CHECK_ONLY", "RELU", "GELU", "SGD", "NESTEROV", "ADAGRAD",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmp.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "mp.h")

MP_F16, MP_F32 = 0, 1
MP_GRADS_PRECHECKED = 1
MP_CHECK_ONLY = 2
RELU, GELU = 0, 1
SGD, NESTEROV, ADAGRAD = 0, 1, 2          # mp_opt_kind
_STATUS = {0: "MP_OK", 1: "MP_ERR_INVALID_ARGUMENT", 2: "MP_ERR_MISALIGNED",
           3: "MP_ERR_UNSUPPORTED", 4: "MP_ERR_HIP", 5: "MP_ERR_OUT_OF_MEMORY"}


class MPError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str = ""):
        self.status = status
        super().__init__(f"{where}: {_STATUS.get(status, status)}" + (f" ({detail})" if detail else ""))


class _Param(C.Structure):
    _fields_ = [("master", C.c_void_p), ("momentum", C.c_void_p), ("grad", C.c_void_p),
                ("weight16", C.c_void_p), ("numel", C.c_int64)]


class _Sgd(C.Structure):
    _fields_ = [("lr", C.c_float), ("momentum", C.c_float), ("weight_decay", C.c_float)]


class _Optim(C.Structure):
    _fields_ = [("kind", C.c_int32), ("lr", C.c_float), ("momentum", C.c_float),
                ("weight_decay", C.c_float), ("eps", C.c_float)]


_lib = None


def lib() -> C.CDLL:
    """Loads libmp.so (raises if it is missing: build it with __graft_entry__.build())."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing; build it first (python -c "
                              "'import __graft_entry__ as g; g.build()')")
        L = C.CDLL(LIB_PATH)
        vp, i64, i32, u32 = C.c_void_p, C.c_int64, C.c_int32, C.c_uint32
        L.mp_linear_fwd.argtypes = [vp, i64, vp, i64, vp, i64, C.c_int, i64, i64, i64, vp]
        L.mp_linear_dgrad.argtypes = [vp, i64, vp, i64, vp, i64, C.c_int, i64, i64, i64, vp]
        L.mp_linear_wgrad.argtypes = [vp, i64, vp, i64, vp, i64, C.c_int, i64, i64, i64, vp, vp]
        L.mp_linear_fwd_act.argtypes = [C.c_int, vp, i64, vp, i64, vp, i64, vp, i64, i64, i64, i64, vp]
        L.mp_linear_dgrad_act.argtypes = [C.c_int, vp, i64, vp, i64, vp, i64, vp, i64, i64, i64, i64, vp]
        L.mp_linear_fwd_act_deriv.argtypes = [C.c_int, vp, i64, vp, i64, vp, i64, vp, i64, i64, i64, i64, vp]
        L.mp_linear_dgrad_mul.argtypes = [vp, i64, vp, i64, vp, i64, vp, i64, i64, i64, i64, vp]
        L.mp_param_list_create.argtypes = [vp, i32, C.POINTER(vp), vp]
        L.mp_param_list_destroy.argtypes = [vp]
        L.mp_param_list_numel.argtypes = [vp]
        L.mp_param_list_numel.restype = i64
        L.mp_step.argtypes = [vp, _Sgd, vp, u32, vp]
        L.mp_step_opt.argtypes = [vp, _Optim, vp, u32, vp]
        L.mp_tensor_list_create.argtypes = [vp, vp, i32, C.c_int, C.POINTER(vp), vp]
        L.mp_tensor_list_destroy.argtypes = [vp]
        L.mp_absmax.argtypes = [vp, vp, vp, vp]
        L.mp_scaler_init_from_absmax.argtypes = [vp, vp, C.c_float, i32, i32, vp]
        L.mp_scaler_init.argtypes = [vp, C.c_float, i32, i32, vp]
        L.mp_scaler_update.argtypes = [vp, vp]
        L.mp_round_f32_to_f16.argtypes = [vp, vp, i64, vp]
        L.mp_act_fwd.argtypes = [C.c_int, vp, vp, i64, vp]
        L.mp_act_bwd.argtypes = [C.c_int, vp, vp, vp, i64, vp]
        L.mp_loss_softmax_ce_workspace.argtypes = [i64, i64]
        L.mp_loss_softmax_ce_workspace.restype = C.c_size_t
        L.mp_loss_softmax_ce.argtypes = [vp, vp, i64, i64, vp, vp, vp, vp, C.c_size_t, vp]
        L.mp_loss_mse_workspace.argtypes = [i64, i64]
        L.mp_loss_mse_workspace.restype = C.c_size_t
        L.mp_loss_mse.argtypes = [vp, vp, i64, i64, C.c_float, vp, vp, vp, vp, C.c_size_t, vp]
        L.mp_loss_mse_noalloc.argtypes = [vp, vp, i64, i64, C.c_float, vp, vp, vp, vp]
        L.mp_loss_mse_noalloc.restype = C.c_int
        L.mp_bn_stats_workspace.argtypes = [i64, i64]
        L.mp_bn_stats_workspace.restype = C.c_size_t
        L.mp_bn_stats.argtypes = [vp, i64, i64, i64, vp, vp, vp, C.c_size_t, vp]
        L.mp_bn_apply.argtypes = [vp, i64, i64, i64, vp, vp, vp, vp, C.c_float, vp, i64, vp]
        L.mp_softmax_workspace.argtypes = [i64, i64]
        L.mp_softmax_workspace.restype = C.c_size_t
        L.mp_softmax.argtypes = [vp, i64, i64, i64, vp, i64, vp, C.c_size_t, vp]
        L.mp_softmax_wait_us.argtypes = [i64]
        L.mp_softmax_wait_us.restype = i64
        L.mp_status_string.argtypes = [C.c_int]
        L.mp_status_string.restype = C.c_char_p
        L.mp_last_hip_error.restype = C.c_char_p
        L.mp_version.restype = C.c_char_p
        for name in ("mp_linear_fwd", "mp_linear_dgrad", "mp_linear_wgrad", "mp_param_list_create",
                     "mp_param_list_destroy", "mp_step", "mp_scaler_init", "mp_scaler_update",
                     "mp_round_f32_to_f16", "mp_act_fwd", "mp_act_bwd", "mp_loss_softmax_ce",
                     "mp_loss_mse", "mp_bn_stats", "mp_bn_apply", "mp_softmax", "mp_linear_fwd_act_deriv",
                     "mp_linear_dgrad_mul"):
            getattr(L, name).restype = C.c_int
        _lib = L
    return _lib


def header_functions() -> list[str]:
    """Names of every function declared in include/mp.h."""
    text = open(HEADER_PATH).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+char\s*\*|mp_status|int64_t|size_t)\s+(mp_\w+)\s*\(",
                                 text, re.M)))


def _check(status: int, where: str) -> None:
    if status != 0:
        detail = lib().mp_last_hip_error().decode() if status == 4 else ""
        raise MPError(status, where, detail)


def _stream(stream) -> C.c_void_p:
    s = stream if stream is not None else torch.cuda.current_stream()
    return C.c_void_p(s.cuda_stream)


def _dev(t: torch.Tensor, name: str, elem: int) -> torch.Tensor:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a GPU tensor")
    if t.element_size() != elem:
        raise TypeError(f"{name} must have {elem}-byte elements, got {t.dtype}")
    return t


def _mat(t: torch.Tensor, name: str, elem: int = 2):
    _dev(t, name, elem)
    if t.dim() != 2 or (t.size(1) > 1 and t.stride(1) != 1):
        raise ValueError(f"{name} must be a row-major 2-D tensor")
    ld = t.stride(0) if t.size(0) > 1 else max(t.size(1), 1)
    return C.c_void_p(t.data_ptr()), ld


def _out(t, shape, dtype, device):
    if t is None:
        return torch.empty(shape, dtype=dtype, device=device)
    return t


# ------------------------------------------------------------------ dot products
def linear_fwd(X: torch.Tensor, W: torch.Tensor, Y: torch.Tensor | None = None,
               out_dtype=torch.float16, stream=None) -> torch.Tensor:
    """Y[M, N] = X[M, K] . W[N, K]^T, binary16 inputs, FP32 accumulation."""
    M, K = X.shape
    N = W.shape[0]
    if W.shape[1] != K:
        raise ValueError("W must be [N, K]")
    Y = _out(Y, (M, N), out_dtype, X.device)
    px, ldx = _mat(X, "X"); pw, ldw = _mat(W, "W"); py, ldy = _mat(Y, "Y", Y.element_size())
    dt = MP_F32 if Y.dtype == torch.float32 else MP_F16
    _check(lib().mp_linear_fwd(px, ldx, pw, ldw, py, ldy, dt, M, N, K, _stream(stream)), "mp_linear_fwd")
    return Y


def linear_dgrad(dY: torch.Tensor, W: torch.Tensor, dX: torch.Tensor | None = None,
                 out_dtype=torch.float16, stream=None) -> torch.Tensor:
    """dX[M, K] = dY[M, N] . W[N, K]."""
    M, N = dY.shape
    K = W.shape[1]
    if W.shape[0] != N:
        raise ValueError("W must be [N, K]")
    dX = _out(dX, (M, K), out_dtype, dY.device)
    pd, ldd = _mat(dY, "dY"); pw, ldw = _mat(W, "W"); px, ldx = _mat(dX, "dX", dX.element_size())
    dt = MP_F32 if dX.dtype == torch.float32 else MP_F16
    _check(lib().mp_linear_dgrad(pd, ldd, pw, ldw, px, ldx, dt, M, N, K, _stream(stream)),
           "mp_linear_dgrad")
    return dX


def linear_fwd_act(kind: int, X: torch.Tensor, W: torch.Tensor, Z: torch.Tensor | None = None,
                   H: torch.Tensor | None = None, stream=None):
    """Z = RNE16(X . W^T) and H = act(Z) in one kernel; returns (Z, H)."""
    M, K = X.shape
    N = W.shape[0]
    if W.shape[1] != K:
        raise ValueError("W must be [N, K]")
    Z = _out(Z, (M, N), torch.float16, X.device)
    H = _out(H, (M, N), torch.float16, X.device)
    px, ldx = _mat(X, "X"); pw, ldw = _mat(W, "W"); pz, ldz = _mat(Z, "Z"); ph, ldh = _mat(H, "H")
    _check(lib().mp_linear_fwd_act(int(kind), px, ldx, pw, ldw, pz, ldz, ph, ldh, M, N, K, _stream(stream)),
           "mp_linear_fwd_act")
    return Z, H


def linear_dgrad_act(kind: int, dY: torch.Tensor, W: torch.Tensor, Z: torch.Tensor,
                     dZ: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """dZ = RNE16(act'(Z) * RNE16(dY . W)) in one kernel."""
    M, N = dY.shape
    K = W.shape[1]
    if W.shape[0] != N:
        raise ValueError("W must be [N, K]")
    if tuple(Z.shape) != (M, K):
        raise ValueError("Z must be [M, K]")
    dZ = _out(dZ, (M, K), torch.float16, dY.device)
    pd, ldd = _mat(dY, "dY"); pw, ldw = _mat(W, "W"); pz, ldz = _mat(Z, "Z"); po, ldo = _mat(dZ, "dZ")
    _check(lib().mp_linear_dgrad_act(int(kind), pd, ldd, pw, ldw, pz, ldz, po, ldo, M, N, K, _stream(stream)),
           "mp_linear_dgrad_act")
    return dZ



def linear_fwd_act_deriv(kind: int, X: torch.Tensor, W: torch.Tensor, H: torch.Tensor | None = None,
                         D: torch.Tensor | None = None, stream=None):
    """H = act(Z) and D = RNE16(act'(Z)) with Z = RNE16(X . W^T) not stored; returns (H, D)."""
    M, K = X.shape
    N = W.shape[0]
    if W.shape[1] != K:
        raise ValueError("W must be [N, K]")
    H = _out(H, (M, N), torch.float16, X.device)
    D = _out(D, (M, N), torch.float16, X.device)
    px, ldx = _mat(X, "X"); pw, ldw = _mat(W, "W"); ph, ldh = _mat(H, "H"); pd, ldd = _mat(D, "D")
    _check(lib().mp_linear_fwd_act_deriv(int(kind), px, ldx, pw, ldw, ph, ldh, pd, ldd, M, N, K,
                                         _stream(stream)), "mp_linear_fwd_act_deriv")
    return H, D


def linear_dgrad_mul(dY: torch.Tensor, W: torch.Tensor, D: torch.Tensor, dZ: torch.Tensor | None = None,
                     stream=None) -> torch.Tensor:
    """dZ = RNE16(f32(RNE16(dY . W)) * f32(D)), D the derivative saved by linear_fwd_act_deriv."""
    M, N = dY.shape
    K = W.shape[1]
    if W.shape[0] != N or tuple(D.shape) != (M, K):
        raise ValueError("W must be [N, K] and D [M, K]")
    dZ = _out(dZ, (M, K), torch.float16, dY.device)
    pdy, lddy = _mat(dY, "dY"); pw, ldw = _mat(W, "W"); pd, ldd = _mat(D, "D"); pz, ldz = _mat(dZ, "dZ")
    _check(lib().mp_linear_dgrad_mul(pdy, lddy, pw, ldw, pd, ldd, pz, ldz, M, N, K, _stream(stream)),
           "mp_linear_dgrad_mul")
    return dZ

def linear_wgrad(dY: torch.Tensor, X: torch.Tensor, dW: torch.Tensor | None = None,
                 out_dtype=torch.float16, found_inf: torch.Tensor | None = None,
                 stream=None) -> torch.Tensor:
    """dW[N, K] = dY[M, N]^T . X[M, K]; found_inf (uint32/int32 device scalar) gets OR 1 on inf/NaN."""
    M, N = dY.shape
    K = X.shape[1]
    if X.shape[0] != M:
        raise ValueError("X must be [M, K]")
    dW = _out(dW, (N, K), out_dtype, dY.device)
    pd, ldd = _mat(dY, "dY"); px, ldx = _mat(X, "X"); pw, ldw = _mat(dW, "dW", dW.element_size())
    dt = MP_F32 if dW.dtype == torch.float32 else MP_F16
    fi = None
    if found_inf is not None:
        fi = C.c_void_p(found_inf.data_ptr()) if isinstance(found_inf, torch.Tensor) else C.c_void_p(found_inf)
    _check(lib().mp_linear_wgrad(pd, ldd, px, ldx, pw, ldw, dt, M, N, K, fi, _stream(stream)),
           "mp_linear_wgrad")
    return dW


# ------------------------------------------------------------------ loss scaler
class Scaler:
    """mp_scaler state in device memory (8 x 32-bit words)."""
    FIELDS = ("scale", "inv_scale", "count", "growth_interval", "found_inf", "dynamic",
              "skipped_steps", "reserved")

    def __init__(self, init_scale: float, dynamic: bool, growth_interval: int = 2000,
                 device="cuda", stream=None):
        self.buf = torch.zeros(8, dtype=torch.int32, device=device)
        self.init(init_scale, dynamic, growth_interval, stream)

    @property
    def ptr(self) -> C.c_void_p:
        return C.c_void_p(self.buf.data_ptr())

    @property
    def found_inf_ptr(self) -> int:
        return self.buf.data_ptr() + 16

    def init(self, init_scale: float, dynamic: bool, growth_interval: int = 2000, stream=None):
        _check(lib().mp_scaler_init(self.ptr, float(init_scale), int(bool(dynamic)),
                                    int(growth_interval), _stream(stream)), "mp_scaler_init")

    def update(self, stream=None):
        _check(lib().mp_scaler_update(self.ptr, _stream(stream)), "mp_scaler_update")

    def read(self) -> dict:
        """Copies the state to the host (synchronises)."""
        raw = self.buf.cpu().numpy()
        f = raw.view("float32")
        u = raw.view("uint32")
        return {"scale": float(f[0]), "inv_scale": float(f[1]), "count": int(raw[2]),
                "growth_interval": int(raw[3]), "found_inf": int(u[4]), "dynamic": int(u[5]),
                "skipped_steps": int(u[6])}

    def raw(self):
        return self.buf.cpu().numpy().view("uint32").copy()


# ------------------------------------------------------------------ optimizer sweep
class ParamList:
    """A library-owned descriptor table over (master, momentum, grad, weight16) tensors."""

    def __init__(self, masters, momenta, grads, weights16, stream=None):
        n = len(masters)
        if not (len(momenta) == len(grads) == len(weights16) == n):
            raise ValueError("the four tensor lists must have the same length")
        arr = (_Param * max(n, 1))()
        self._keep = []
        for i in range(n):
            m = _dev(masters[i], "master", 4); v = _dev(momenta[i], "momentum", 4)
            g = _dev(grads[i], "grad", 2); h = _dev(weights16[i], "weight16", 2)
            if not (m.numel() == v.numel() == g.numel() == h.numel()):
                raise ValueError(f"tensor {i}: sizes differ")
            for t in (m, v, g, h):
                if not t.is_contiguous():
                    raise ValueError(f"tensor {i} must be contiguous")
            arr[i] = _Param(m.data_ptr(), v.data_ptr(), g.data_ptr(), h.data_ptr(), m.numel())
            self._keep.append((m, v, g, h))
        handle = C.c_void_p()
        _check(lib().mp_param_list_create(arr, n, C.byref(handle), _stream(stream)),
               "mp_param_list_create")
        self.handle = handle
        self.numel = int(lib().mp_param_list_numel(handle))

    def close(self):
        if getattr(self, "handle", None) is not None and self.handle.value:
            _check(lib().mp_param_list_destroy(self.handle), "mp_param_list_destroy")
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def step(plist: ParamList, scaler: Scaler, lr: float, momentum: float, weight_decay: float = 0.0,
         flags: int = 0, stream=None) -> None:
    """One optimizer step over the list (check, then fused update unless overflow)."""
    _check(lib().mp_step(plist.handle, _Sgd(lr, momentum, weight_decay), scaler.ptr, int(flags),
                         _stream(stream)), "mp_step")


def step_opt(plist: ParamList, scaler: Scaler, kind: int, lr: float, momentum: float = 0.0,
             weight_decay: float = 0.0, eps: float = 1e-10, flags: int = 0, stream=None) -> None:
    """One optimizer step with the update rule `kind` (SGD, NESTEROV or ADAGRAD); for ADAGRAD
    the list's momentum tensors hold the running sum of squared gradients."""
    _check(lib().mp_step_opt(plist.handle, _Optim(int(kind), lr, momentum, weight_decay, eps),
                             scaler.ptr, int(flags), _stream(stream)), "mp_step_opt")


# ------------------------------------------------------------------ loss-scale method 2
class TensorList:
    """A library-owned table over float32 or binary16 device tensors (gradient statistics)."""

    def __init__(self, tensors, stream=None):
        n = len(tensors)
        if n and not all(t.dtype == tensors[0].dtype for t in tensors):
            raise ValueError("all tensors must have one dtype")
        dt = tensors[0].dtype if n else torch.float32
        if dt not in (torch.float32, torch.float16):
            raise ValueError("float32 or float16 tensors")
        self._keep = [_dev(t, "tensor", t.element_size()) for t in tensors]
        for t in self._keep:
            if not t.is_contiguous():
                raise ValueError("tensors must be contiguous")
        ptrs = (C.c_void_p * max(n, 1))(*[t.data_ptr() for t in self._keep])
        sizes = (C.c_int64 * max(n, 1))(*[t.numel() for t in self._keep])
        handle = C.c_void_p()
        _check(lib().mp_tensor_list_create(ptrs, sizes, n, MP_F32 if dt == torch.float32 else MP_F16,
                                           C.byref(handle), _stream(stream)), "mp_tensor_list_create")
        self.handle = handle

    def close(self):
        if getattr(self, "handle", None) is not None and self.handle.value:
            _check(lib().mp_tensor_list_destroy(self.handle), "mp_tensor_list_destroy")
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def absmax(tlist: TensorList, amax: torch.Tensor, nonfinite: torch.Tensor | None = None, stream=None):
    """amax (1-element float32 device tensor, >= 0) = max(amax, |x| over the finite elements);
    nonfinite (1-element int32 device tensor) gets 1 ORed in if any element is +-inf/NaN."""
    _dev(amax, "amax", 4)
    nf = None if nonfinite is None else C.c_void_p(_dev(nonfinite, "nonfinite", 4).data_ptr())
    _check(lib().mp_absmax(tlist.handle, C.c_void_p(amax.data_ptr()), nf, _stream(stream)), "mp_absmax")
    return amax


def scaler_init_from_absmax(scaler: Scaler, amax: torch.Tensor, headroom: float = 2.0,
                            dynamic: bool = False, growth_interval: int = 2000, stream=None):
    """Re-initialises `scaler` with S = largest power of two, S * headroom * amax <= 65504."""
    _check(lib().mp_scaler_init_from_absmax(scaler.ptr, C.c_void_p(_dev(amax, "amax", 4).data_ptr()),
                                            headroom, int(bool(dynamic)), int(growth_interval),
                                            _stream(stream)), "mp_scaler_init_from_absmax")
    return scaler


# ------------------------------------------------------------------ auxiliary steps
def round_f32_to_f16(w32: torch.Tensor, w16: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    _dev(w32, "w32", 4)
    w16 = _out(w16, tuple(w32.shape), torch.float16, w32.device)
    _dev(w16, "w16", 2)
    if w32.numel() != w16.numel() or not w32.is_contiguous() or not w16.is_contiguous():
        raise ValueError("w32 and w16 must be contiguous and the same size")
    _check(lib().mp_round_f32_to_f16(C.c_void_p(w32.data_ptr()), C.c_void_p(w16.data_ptr()),
                                     w32.numel(), _stream(stream)), "mp_round_f32_to_f16")
    return w16


def _flat2(*ts):
    for t in ts:
        _dev(t, "tensor", 2)
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
    if len({t.numel() for t in ts}) != 1:
        raise ValueError("sizes differ")


def act_fwd(kind: int, x: torch.Tensor, y: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    y = _out(y, tuple(x.shape), x.dtype, x.device)
    _flat2(x, y)
    _check(lib().mp_act_fwd(int(kind), C.c_void_p(x.data_ptr()), C.c_void_p(y.data_ptr()),
                            x.numel(), _stream(stream)), "mp_act_fwd")
    return y


def act_bwd(kind: int, x: torch.Tensor, dy: torch.Tensor, dx: torch.Tensor | None = None,
            stream=None) -> torch.Tensor:
    dx = _out(dx, tuple(x.shape), dy.dtype, x.device)
    _flat2(x, dy, dx)
    _check(lib().mp_act_bwd(int(kind), C.c_void_p(x.data_ptr()), C.c_void_p(dy.data_ptr()),
                            C.c_void_p(dx.data_ptr()), x.numel(), _stream(stream)), "mp_act_bwd")
    return dx


# ------------------------------------------------------------------ large reductions
def _f32vec(t: torch.Tensor, name: str, n: int) -> C.c_void_p:
    _dev(t, name, 4)
    if t.dtype != torch.float32 or t.numel() != n or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous float32 tensor of {n} elements")
    return C.c_void_p(t.data_ptr())


def bn_stats(x: torch.Tensor, mean: torch.Tensor | None = None, var: torch.Tensor | None = None,
             stream=None):
    """Per-channel mean and population variance (FP32) of x[rows, channels] (binary16)."""
    rows, ch = x.shape
    px, ldx = _mat(x, "x")
    mean = _out(mean, (ch,), torch.float32, x.device)
    var = _out(var, (ch,), torch.float32, x.device)
    nbytes = int(lib().mp_bn_stats_workspace(rows, ch))
    ws = torch.empty(max(nbytes, 4), dtype=torch.uint8, device=x.device)
    _check(lib().mp_bn_stats(px, rows, ch, ldx, _f32vec(mean, "mean", ch), _f32vec(var, "var", ch),
                             C.c_void_p(ws.data_ptr()), nbytes, _stream(stream)), "mp_bn_stats")
    return mean, var


def bn_apply(x: torch.Tensor, mean: torch.Tensor, var: torch.Tensor, gamma: torch.Tensor,
             beta: torch.Tensor, eps: float, y: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """y = RNE16(((x - mean) * (1 / sqrt(var + eps))) * gamma + beta), per channel, FP32."""
    rows, ch = x.shape
    y = _rows_out(y, rows, ch, x)
    px, ldx = _mat(x, "x"); py, ldy = _mat(y, "y")
    _check(lib().mp_bn_apply(px, rows, ch, ldx, _f32vec(mean, "mean", ch), _f32vec(var, "var", ch),
                             _f32vec(gamma, "gamma", ch), _f32vec(beta, "beta", ch), float(eps), py, ldy,
                             _stream(stream)), "mp_bn_apply")
    return y


def _rows_out(y, rows: int, cols: int, like: torch.Tensor) -> torch.Tensor:
    """y, or a new [rows, cols] matrix whose row pitch is cols rounded up to 8 elements, so
    its rows are 16-byte aligned (the kernels' 16-byte path)."""
    if y is not None:
        return y
    ld = (cols + 7) // 8 * 8
    return torch.empty((rows, ld), dtype=like.dtype, device=like.device)[:, :cols]


def softmax(x: torch.Tensor, y: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Row-wise softmax of x[rows, cols] (binary16 in and out, FP32 arithmetic)."""
    rows, cols = x.shape
    y = _rows_out(y, rows, cols, x)
    px, ldx = _mat(x, "x"); py, ldy = _mat(y, "y")
    nbytes = int(lib().mp_softmax_workspace(rows, cols))
    ws = torch.empty(max(nbytes, 8), dtype=torch.uint8, device=x.device)
    _check(lib().mp_softmax(px, rows, cols, ldx, py, ldy, C.c_void_p(ws.data_ptr()), nbytes,
                            _stream(stream)), "mp_softmax")
    return y


def softmax_wait_us(us: int = -1) -> int:
    """Sets how long (µs) a block of the single-read softmax waits for its row's other blocks
    before computing their (max, sum) itself (0: never waits); negative only queries. Returns
    the previous setting."""
    return int(lib().mp_softmax_wait_us(int(us)))


def _workspace(ws, nbytes: int, align: int, device) -> torch.Tensor:
    """ws (a GPU tensor of at least nbytes), or a new uint8 buffer of that size."""
    if ws is None:
        return torch.empty(max(nbytes, align), dtype=torch.uint8, device=device)
    if not isinstance(ws, torch.Tensor) or not ws.is_cuda or not ws.is_contiguous():
        raise TypeError("workspace must be a contiguous GPU tensor")
    if ws.numel() * ws.element_size() < nbytes:
        raise ValueError(f"workspace holds {ws.numel() * ws.element_size()} bytes, {nbytes} needed")
    return ws


def loss_softmax_ce_workspace(B: int, Cn: int) -> int:
    """Bytes of workspace mp_loss_softmax_ce needs (a reusable buffer for ``workspace=``)."""
    return int(lib().mp_loss_softmax_ce_workspace(B, Cn))


def loss_mse_workspace(M: int, N: int) -> int:
    """Bytes of workspace mp_loss_mse needs (a reusable buffer for ``workspace=``)."""
    return int(lib().mp_loss_mse_workspace(M, N))


def loss_softmax_ce(logits: torch.Tensor, labels: torch.Tensor, scaler: Scaler,
                    loss: torch.Tensor | None = None, dlogits: torch.Tensor | None = None,
                    stream=None, workspace: torch.Tensor | None = None):
    B, Cn = logits.shape
    _flat2(logits)
    if labels.dtype != torch.int32 or not labels.is_cuda or labels.numel() != B:
        raise TypeError("labels must be a GPU int32 tensor of length B")
    loss = _out(loss, (1,), torch.float32, logits.device)
    dlogits = _out(dlogits, (B, Cn), logits.dtype, logits.device)
    nbytes = loss_softmax_ce_workspace(B, Cn)
    ws = _workspace(workspace, nbytes, 4, logits.device)
    _check(lib().mp_loss_softmax_ce(C.c_void_p(logits.data_ptr()), C.c_void_p(labels.data_ptr()),
                                    B, Cn, scaler.ptr, C.c_void_p(loss.data_ptr()),
                                    C.c_void_p(dlogits.data_ptr()), C.c_void_p(ws.data_ptr()),
                                    ws.numel() * ws.element_size(), _stream(stream)),
           "mp_loss_softmax_ce")
    return loss, dlogits


def loss_mse(y: torch.Tensor, t: torch.Tensor, c: float, scaler: Scaler,
             loss: torch.Tensor | None = None, dy: torch.Tensor | None = None, stream=None,
             workspace: torch.Tensor | None = None):
    M, N = y.shape
    _flat2(y, t)
    loss = _out(loss, (1,), torch.float32, y.device)
    dy = _out(dy, (M, N), y.dtype, y.device)
    ws = _workspace(workspace, loss_mse_workspace(M, N), 4, y.device)
    _check(lib().mp_loss_mse(C.c_void_p(y.data_ptr()), C.c_void_p(t.data_ptr()), M, N, float(c),
                             scaler.ptr, C.c_void_p(loss.data_ptr()), C.c_void_p(dy.data_ptr()),
                             C.c_void_p(ws.data_ptr()), ws.numel() * ws.element_size(),
                             _stream(stream)), "mp_loss_mse")
    return loss, dy


def loss_mse_noalloc(y: torch.Tensor, t: torch.Tensor, c: float, scaler: Scaler, loss: torch.Tensor,
                     dy: torch.Tensor, stream=None):
    """mp_loss_mse_noalloc: loss_mse with the library's per-device scratch array instead of a
    workspace. The outputs are the caller's; nothing is allocated by this call."""
    M, N = y.shape
    _flat2(y, t, dy)
    if tuple(dy.shape) != (M, N) or loss.dtype != torch.float32 or loss.numel() < 1 or not loss.is_cuda:
        raise ValueError("dy must be [M, N] and loss a float32 GPU tensor")
    _check(lib().mp_loss_mse_noalloc(C.c_void_p(y.data_ptr()), C.c_void_p(t.data_ptr()), M, N, float(c),
                                     scaler.ptr, C.c_void_p(loss.data_ptr()), C.c_void_p(dy.data_ptr()),
                                     _stream(stream)), "mp_loss_mse_noalloc")
    return loss, dy
