"""Marshalling helpers for the GPU tests (host <-> device copies of bit patterns)."""
import numpy as np
import torch


def require_gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU; run them with -m gpu on an MI355X"


def dev_f16(bits: np.ndarray) -> torch.Tensor:
    """uint16 bit patterns -> a float16 GPU tensor holding the same bits."""
    t = torch.from_numpy(np.ascontiguousarray(bits, np.uint16).view(np.int16))
    return t.cuda().view(torch.float16)


def dev_f32(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).cuda()


def host_bits16(t: torch.Tensor) -> np.ndarray:
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def host_f32(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy().astype(np.float32, copy=False)


def bits32(x: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(x, np.float32).view(np.uint32)


def same_f32_bits(a: np.ndarray, b: np.ndarray) -> bool:
    """Bitwise equality, with any NaN matching any NaN."""
    a = np.ascontiguousarray(a, np.float32); b = np.ascontiguousarray(b, np.float32)
    na, nb = np.isnan(a), np.isnan(b)
    if not np.array_equal(na, nb):
        return False
    return np.array_equal(a.view(np.uint32)[~na], b.view(np.uint32)[~nb])


def same_f16_bits(a: np.ndarray, b: np.ndarray) -> bool:
    a = np.asarray(a, np.uint16); b = np.asarray(b, np.uint16)
    na = ((a & 0x7C00) == 0x7C00) & ((a & 0x3FF) != 0)
    nb = ((b & 0x7C00) == 0x7C00) & ((b & 0x3FF) != 0)
    if not np.array_equal(na, nb):
        return False
    return np.array_equal(a[~na], b[~nb])


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    """max |got - ref| / max(|ref|, rms(ref)) over all elements (the GEMM error metric)."""
    got = np.asarray(got, np.float64); ref = np.asarray(ref, np.float64)
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    den = np.maximum(np.abs(ref), rms if rms > 0 else 1.0)
    return float(np.max(np.abs(got - ref) / den)) if ref.size else 0.0


def f16_values(bits: np.ndarray) -> np.ndarray:
    return np.asarray(bits, np.uint16).view(np.float16).astype(np.float64)
