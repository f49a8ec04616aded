"""LSSAR causal attention forward on MI355X (gfx950).

Thin Python binding of the C ABI declared in ``include/lssar.h`` (library
``liblssar.so`` next to this file).  The functions carry the C names and do
argument marshalling only: shapes, dtype and pointers are read from the
tensors and every step of the computation runs in the HIP kernels.  PyTorch
supplies device memory and streams.  There is no fallback: if the library is
missing or fails to load, every call raises.

Method: paper note "Softplus Attention with Re-weighting Boosts Length
Extrapolation in Large Language Models", Method details, Key designs 1-3.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "LSSAR_F32", "LSSAR_BF16", "LSSAR_OK", "LSSAR_EINVAL", "LSSAR_EUNSUPPORTED",
    "LSSAR_EWORKSPACE", "LSSAR_EHIP", "LssarError", "lib", "lib_path",
    "lssar_workspace_bytes", "lssar_attn_fwd_ws", "lssar_attn_fwd",
    "lssar_key_inv_norms", "lssar_attn_fwd_prenormed", "lssar_status_str",
    "lssar_last_hip_error", "lssar_version", "DEFAULT_EPS",
]

LSSAR_F32, LSSAR_BF16 = 0, 1
LSSAR_OK, LSSAR_EINVAL, LSSAR_EUNSUPPORTED, LSSAR_EWORKSPACE, LSSAR_EHIP = 0, -1, -2, -3, -4
DEFAULT_EPS = 1e-4

_HERE = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_HERE, "liblssar.so")
_lib = None


class LssarError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = f"{where}: {lssar_status_str(status)} (status {status})"
        if status == LSSAR_EHIP:
            msg += f", hipError {lssar_last_hip_error()}"
        super().__init__(msg)


def lib():
    """The loaded C library (ctypes).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(lib_path):
            raise RuntimeError(f"{lib_path} is missing: build it with __graft_entry__.build() "
                               "(hipcc --offload-arch=gfx950); there is no fallback path")
        L = ctypes.CDLL(lib_path)
        vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
        L.lssar_workspace_bytes.argtypes = [i, i, i, i, i]
        L.lssar_workspace_bytes.restype = sz
        L.lssar_attn_fwd_ws.argtypes = [vp, vp, vp, vp, i, i, i, i, i, f, i, vp, sz, vp]
        L.lssar_attn_fwd_ws.restype = i
        L.lssar_attn_fwd.argtypes = [vp, vp, vp, vp, i, i, i, i, i, f, i, vp]
        L.lssar_attn_fwd.restype = i
        L.lssar_key_inv_norms.argtypes = [vp, vp, i, i, i, i, i, vp]
        L.lssar_key_inv_norms.restype = i
        L.lssar_attn_fwd_prenormed.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp]
        L.lssar_attn_fwd_prenormed.restype = i
        L.lssar_status_str.argtypes = [i]
        L.lssar_status_str.restype = ctypes.c_char_p
        L.lssar_last_hip_error.argtypes = []
        L.lssar_last_hip_error.restype = i
        L.lssar_version.argtypes = []
        L.lssar_version.restype = i
        _lib = L
    return _lib


def lssar_status_str(status: int) -> str:
    return lib().lssar_status_str(int(status)).decode()


def lssar_last_hip_error() -> int:
    return int(lib().lssar_last_hip_error())


def lssar_version() -> int:
    return int(lib().lssar_version())


def lssar_workspace_bytes(B: int, H: int, L: int, d: int, dtype: int) -> int:
    return int(lib().lssar_workspace_bytes(B, H, L, d, dtype))


# --------------------------------------------------------------------------
# tensor marshalling
# --------------------------------------------------------------------------

def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return LSSAR_BF16
    if t.dtype == torch.float32:
        return LSSAR_F32
    raise TypeError(f"unsupported dtype {t.dtype}: LSSAR takes float32 or bfloat16")


def _check_qkv(q, k, v, out=None):
    for name, t in (("q", q), ("k", k), ("v", v)) + ((("out", out),) if out is not None else ()):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if t.dim() != 4:
            raise ValueError(f"{name} must be [B, H, L, d]")
        if t.shape != q.shape or t.dtype != q.dtype:
            raise ValueError(f"{name} must match q in shape and dtype")
    B, H, L, d = q.shape
    return B, H, L, d, _dtype_code(q)


def _stream_ptr(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _raise(st, where):
    if st != LSSAR_OK:
        raise LssarError(st, where)


def lssar_attn_fwd_ws(q, k, v, out, workspace, *, p: int, eps: float = DEFAULT_EPS, stream=None):
    """out <- LSSAR(q, k, v) using a caller-owned workspace tensor (any dtype,
    at least lssar_workspace_bytes bytes, 256-byte aligned).  Returns out."""
    B, H, L, d, dt = _check_qkv(q, k, v, out)
    nbytes = workspace.numel() * workspace.element_size()
    st = lib().lssar_attn_fwd_ws(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, H, L, d, int(p),
                                 float(eps), dt, _ptr(workspace), nbytes, _stream_ptr(stream))
    _raise(st, "lssar_attn_fwd_ws")
    return out


def lssar_attn_fwd(q, k, v, out=None, *, p: int, eps: float = DEFAULT_EPS, stream=None):
    """out <- LSSAR(q, k, v); the workspace comes stream-ordered from the
    device memory pool.  Allocates `out` (with torch) if it is not given."""
    import torch
    if out is None:
        out = torch.empty_like(q)
    B, H, L, d, dt = _check_qkv(q, k, v, out)
    st = lib().lssar_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, H, L, d, int(p),
                              float(eps), dt, _stream_ptr(stream))
    _raise(st, "lssar_attn_fwd")
    return out


def lssar_key_inv_norms(k, fk, *, stream=None):
    """fk[b, h, j] <- 1 / max(|k[b, h, j]|_2, 1e-12); fk is a float32 device
    tensor with B*H*L elements."""
    import torch
    if not k.is_cuda or not k.is_contiguous() or k.dim() != 4:
        raise ValueError("k must be a contiguous [B, H, L, d] device tensor")
    B, H, L, d = k.shape
    if fk.dtype != torch.float32 or fk.numel() < B * H * L or not fk.is_cuda:
        raise ValueError("fk must be a float32 device tensor of B*H*L elements")
    st = lib().lssar_key_inv_norms(_ptr(k), _ptr(fk), B, H, L, d, _dtype_code(k),
                                   _stream_ptr(stream))
    _raise(st, "lssar_key_inv_norms")
    return fk


def lssar_attn_fwd_prenormed(q, k, v, fk, out, *, p: int, eps: float = DEFAULT_EPS, stream=None):
    """The fused attention kernel alone, given fk from lssar_key_inv_norms."""
    import torch
    B, H, L, d, dt = _check_qkv(q, k, v, out)
    if fk.dtype != torch.float32 or fk.numel() < B * H * L or not fk.is_cuda:
        raise ValueError("fk must be a float32 device tensor of B*H*L elements")
    st = lib().lssar_attn_fwd_prenormed(_ptr(q), _ptr(k), _ptr(v), _ptr(fk), _ptr(out), B, H,
                                        L, d, int(p), float(eps), dt, _stream_ptr(stream))
    _raise(st, "lssar_attn_fwd_prenormed")
    return out
