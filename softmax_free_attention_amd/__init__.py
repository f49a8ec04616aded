"""LSSAR causal attention forward on MI355X (gfx950).

Thin Python binding of the C ABI declared in ``include/lssar.h`` (library
``liblssar.so`` next to this file).  The functions carry the C names and do
argument marshalling only: shapes, dtype and pointers are read from the
tensors and every step of the computation runs in the HIP kernels.  PyTorch
supplies device memory and streams.  There is no fallback: if the library is
missing or fails to load, every call raises.

Method: paper note "Softplus Attention with Re-weighting Boosts Length
Extrapolation in Large Language Models", Method details, Key designs 1-3;
the two variants of its ablation table (Key experimental data, ablation):
the Sigmoid stage-1 map and stage 1 alone ("LSSA only").
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "LSSAR_F32", "LSSAR_BF16", "LSSAR_OK", "LSSAR_EINVAL", "LSSAR_EUNSUPPORTED",
    "LSSAR_EWORKSPACE", "LSSAR_EHIP", "LssarError", "lib", "lib_path",
    "lssar_workspace_bytes", "lssar_attn_fwd_ws", "lssar_attn_fwd",
    "lssar_prep", "lssar_attn_fwd_prepped", "lssar_status_str", "workspace_for",
    "lssar_last_hip_error", "lssar_version", "DEFAULT_EPS", "LSSAR_PHI_SOFTPLUS",
    "LSSAR_PHI_SIGMOID", "lssar_attn_fwd_phi_ws", "lssar_lssa_fwd_ws",
    "lssar_decode_workspace_bytes", "lssar_decode_ws", "decode_workspace_for",
    "lssar_bwd_workspace_bytes", "lssar_attn_bwd_ws", "bwd_workspace_for",
    "lssar_attn_fwd_stats_ws", "lssar_attn_bwd_stats_ws", "stats_for",
    "lssar_fwd_schedule", "lssar_attn_fwd_noalloc", "lssar_noalloc_scratch_bytes",
    "LSSAR_ESCRATCH",
]

LSSAR_F32, LSSAR_BF16 = 0, 1
LSSAR_PHI_SOFTPLUS, LSSAR_PHI_SIGMOID = 0, 1
LSSAR_OK, LSSAR_EINVAL, LSSAR_EUNSUPPORTED, LSSAR_EWORKSPACE, LSSAR_EHIP = 0, -1, -2, -3, -4
LSSAR_ESCRATCH = -5
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
        L.lssar_prep.argtypes = [vp, vp, sz, i, i, i, i, i, vp]
        L.lssar_prep.restype = i
        L.lssar_attn_fwd_prepped.argtypes = [vp, vp, vp, vp, sz, vp, i, i, i, i, i, f, i, vp]
        L.lssar_attn_fwd_prepped.restype = i
        L.lssar_attn_fwd_phi_ws.argtypes = [vp, vp, vp, vp, i, i, i, i, i, f, i, i, vp, sz, vp]
        L.lssar_attn_fwd_phi_ws.restype = i
        L.lssar_lssa_fwd_ws.argtypes = [vp, vp, vp, vp, i, i, i, i, i, vp, sz, vp]
        L.lssar_lssa_fwd_ws.restype = i
        L.lssar_decode_workspace_bytes.argtypes = [i, i, i, i, i]
        L.lssar_decode_workspace_bytes.restype = sz
        L.lssar_decode_ws.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp, sz, vp]
        L.lssar_decode_ws.restype = i
        L.lssar_bwd_workspace_bytes.argtypes = [i, i, i, i, i]
        L.lssar_bwd_workspace_bytes.restype = sz
        L.lssar_attn_bwd_ws.argtypes = [vp] * 7 + [i, i, i, i, i, f, i, vp, sz, vp]
        L.lssar_attn_bwd_ws.restype = i
        L.lssar_attn_fwd_stats_ws.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp, sz, vp]
        L.lssar_attn_fwd_stats_ws.restype = i
        L.lssar_attn_bwd_stats_ws.argtypes = [vp] * 9 + [i, i, i, i, i, f, i, vp, sz, vp]
        L.lssar_attn_bwd_stats_ws.restype = i
        L.lssar_status_str.argtypes = [i]
        L.lssar_status_str.restype = ctypes.c_char_p
        L.lssar_last_hip_error.argtypes = []
        L.lssar_last_hip_error.restype = i
        L.lssar_version.argtypes = []
        L.lssar_version.restype = i
        L.lssar_fwd_schedule.argtypes = [i, i, i, ctypes.POINTER(ctypes.c_int),
                                         ctypes.c_longlong]
        L.lssar_fwd_schedule.restype = ctypes.c_longlong
        L.lssar_attn_fwd_noalloc.argtypes = [vp, vp, vp, vp, i, i, i, i, i, f, i, vp]
        L.lssar_attn_fwd_noalloc.restype = i
        L.lssar_noalloc_scratch_bytes.argtypes = []
        L.lssar_noalloc_scratch_bytes.restype = sz
        _lib = L
    return _lib


def lssar_status_str(status: int) -> str:
    return lib().lssar_status_str(int(status)).decode()


def lssar_last_hip_error() -> int:
    return int(lib().lssar_last_hip_error())


def lssar_version() -> int:
    return int(lib().lssar_version())


def lssar_fwd_schedule(B: int, H: int, L: int):
    """The bf16 forward's dispatch order: a list with, for each workgroup,
    the query block (b H + h) nqb + qb it computes, or -1 (exits at once)."""
    n = int(lib().lssar_fwd_schedule(B, H, L, None, 0))
    if n < 0:
        raise LssarError(n, "lssar_fwd_schedule")
    buf = (ctypes.c_int * n)()
    rc = int(lib().lssar_fwd_schedule(B, H, L, buf, n))
    if rc != n:
        raise LssarError(rc, "lssar_fwd_schedule")
    return list(buf)


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


def lssar_attn_fwd_noalloc(q, k, v, out, *, p: int, eps: float = DEFAULT_EPS, stream=None):
    """out <- LSSAR(q, k, v) with the library's static per-GPU scratch as the
    workspace: no allocation (out must be given)."""
    B, H, L, d, dt = _check_qkv(q, k, v, out)
    st = lib().lssar_attn_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, H, L, d, int(p),
                                      float(eps), dt, _stream_ptr(stream))
    _raise(st, "lssar_attn_fwd_noalloc")
    return out


def lssar_noalloc_scratch_bytes() -> int:
    return int(lib().lssar_noalloc_scratch_bytes())


def workspace_for(q):
    """A device byte tensor of lssar_workspace_bytes for tensors shaped like q."""
    import torch
    B, H, L, d = q.shape
    n = lssar_workspace_bytes(B, H, L, d, _dtype_code(q))
    if n == 0:
        raise ValueError(f"unsupported shape {tuple(q.shape)} / dtype {q.dtype}")
    return torch.empty(n, dtype=torch.uint8, device=q.device)


def _ws_args(workspace):
    if not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous device tensor")
    return _ptr(workspace), workspace.numel() * workspace.element_size()


def lssar_prep(k, workspace, *, stream=None):
    """The prep step (prep kernel, K only): key-row inverse norms and, for bf16,
    the exact and the normalised f16 keys and the dispatch table, into the
    workspace."""
    B, H, L, d, dt = _check_qkv(k, k, k)
    wp, wn = _ws_args(workspace)
    st = lib().lssar_prep(_ptr(k), wp, wn, B, H, L, d, dt, _stream_ptr(stream))
    _raise(st, "lssar_prep")
    return workspace


def lssar_attn_fwd_prepped(q, k, v, workspace, out, *, p: int, eps: float = DEFAULT_EPS,
                           stream=None):
    """The attention kernel alone (fused), given a workspace filled by
    lssar_prep for this k."""
    B, H, L, d, dt = _check_qkv(q, k, v, out)
    wp, wn = _ws_args(workspace)
    st = lib().lssar_attn_fwd_prepped(_ptr(q), _ptr(k), _ptr(v), wp, wn, _ptr(out), B, H, L, d,
                                      int(p), float(eps), dt, _stream_ptr(stream))
    _raise(st, "lssar_attn_fwd_prepped")
    return out


def lssar_attn_fwd_phi_ws(q, k, v, out, workspace, *, p: int, eps: float = DEFAULT_EPS,
                          phi: int = LSSAR_PHI_SOFTPLUS, stream=None):
    """As lssar_attn_fwd_ws with the stage-1 map chosen by ``phi``
    (LSSAR_PHI_SOFTPLUS or the ablation's LSSAR_PHI_SIGMOID)."""
    B, H, L, d, dt = _check_qkv(q, k, v, out)
    wp, wn = _ws_args(workspace)
    st = lib().lssar_attn_fwd_phi_ws(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, H, L, d, int(p),
                                     float(eps), int(phi), dt, wp, wn, _stream_ptr(stream))
    _raise(st, "lssar_attn_fwd_phi_ws")
    return out


def lssar_lssa_fwd_ws(q, k, v, out, workspace, *, stream=None):
    """Stage 1 alone, then A V (the ablation's "LSSA only"), with a
    caller-owned workspace of lssar_workspace_bytes."""
    B, H, L, d, dt = _check_qkv(q, k, v, out)
    wp, wn = _ws_args(workspace)
    st = lib().lssar_lssa_fwd_ws(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, H, L, d, dt, wp, wn,
                                 _stream_ptr(stream))
    _raise(st, "lssar_lssa_fwd_ws")
    return out


def lssar_decode_workspace_bytes(B: int, H: int, Lmax: int, d: int, dtype: int) -> int:
    return int(lib().lssar_decode_workspace_bytes(B, H, Lmax, d, dtype))


def decode_workspace_for(k_cache):
    """A device byte tensor of lssar_decode_workspace_bytes for a cache shaped
    like k_cache ([B, H, Lmax, d])."""
    import torch
    B, H, Lmax, d = k_cache.shape
    n = lssar_decode_workspace_bytes(B, H, Lmax, d, _dtype_code(k_cache))
    if n == 0:
        raise ValueError(f"unsupported cache shape {tuple(k_cache.shape)} / dtype {k_cache.dtype}")
    return torch.empty(n, dtype=torch.uint8, device=k_cache.device)


def lssar_decode_ws(q, k_cache, v_cache, lens, out, workspace, *, p: int,
                    eps: float = DEFAULT_EPS, stream=None):
    """Decode step: q and out [B, H, d], caches [B, H, Lmax, d], lens a device
    int32 tensor [B] (1-based position of each sequence's query) or None (all
    Lmax rows).  Returns out."""
    import torch
    for name, t in (("q", q), ("out", out)):
        if not t.is_cuda or not t.is_contiguous() or t.dim() != 3 or t.dtype != q.dtype:
            raise ValueError(f"{name} must be a contiguous device tensor [B, H, d] of q's dtype")
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        if not t.is_cuda or not t.is_contiguous() or t.dim() != 4 or t.dtype != q.dtype:
            raise ValueError(f"{name} must be a contiguous device tensor [B, H, Lmax, d]")
    B, H, Lmax, d = k_cache.shape
    if v_cache.shape != k_cache.shape or tuple(q.shape) != (B, H, d) or out.shape != q.shape:
        raise ValueError("q/out [B, H, d] and caches [B, H, Lmax, d] must agree")
    lp = None
    if lens is not None:
        if not lens.is_cuda or lens.dtype != torch.int32 or lens.numel() != B or \
                not lens.is_contiguous():
            raise ValueError("lens must be a contiguous device int32 tensor of B entries")
        lp = _ptr(lens)
    wp, wn = _ws_args(workspace)
    st = lib().lssar_decode_ws(_ptr(q), _ptr(k_cache), _ptr(v_cache), lp, _ptr(out), B, H, Lmax,
                               d, int(p), float(eps), _dtype_code(q), wp, wn, _stream_ptr(stream))
    _raise(st, "lssar_decode_ws")
    return out


def lssar_bwd_workspace_bytes(B: int, H: int, L: int, d: int, dtype: int) -> int:
    return int(lib().lssar_bwd_workspace_bytes(B, H, L, d, dtype))


def bwd_workspace_for(q):
    """A device byte tensor of lssar_bwd_workspace_bytes for tensors shaped like q."""
    import torch
    B, H, L, d = q.shape
    n = lssar_bwd_workspace_bytes(B, H, L, d, _dtype_code(q))
    if n == 0:
        raise ValueError(f"unsupported shape {tuple(q.shape)} / dtype {q.dtype}")
    return torch.empty(n, dtype=torch.uint8, device=q.device)


def lssar_attn_bwd_ws(q, k, v, dout, dq, dk, dv, workspace, *, p: int,
                      eps: float = DEFAULT_EPS, stream=None):
    """Gradients (dq, dk, dv) of sum(dout * LSSAR(q, k, v)), written into the
    given tensors.  Returns (dq, dk, dv)."""
    B, H, L, d, dt = _check_qkv(q, k, v, dout)
    _check_qkv(dq, dk, dv)
    if dq.shape != q.shape or dq.dtype != q.dtype:
        raise ValueError("gradients must match q in shape and dtype")
    wp, wn = _ws_args(workspace)
    st = lib().lssar_attn_bwd_ws(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(dq), _ptr(dk),
                                 _ptr(dv), B, H, L, d, int(p), float(eps), dt, wp, wn,
                                 _stream_ptr(stream))
    _raise(st, "lssar_attn_bwd_ws")
    return dq, dk, dv


def _check_stats(stats, q):
    import torch
    B, H, L, _ = q.shape
    if not stats.is_cuda or not stats.is_contiguous() or stats.dtype != torch.float64 \
            or tuple(stats.shape) != (B, H, L, 2):
        raise ValueError("row statistics must be a contiguous float64 device tensor [B, H, L, 2]")


def stats_for(q):
    """A float64 device tensor [B, H, L, 2] for the row statistics of q's shape."""
    import torch
    B, H, L, _ = q.shape
    return torch.empty((B, H, L, 2), dtype=torch.float64, device=q.device)


def lssar_attn_fwd_stats_ws(q, k, v, out, stats, workspace, *, p: int,
                            eps: float = DEFAULT_EPS, stream=None):
    """Training forward: out <- LSSAR(q, k, v) and, per row, stats[..., 0] =
    sum_j Softplus(s_ij) and stats[..., 1] = max_j s_ij for the backward.
    Returns (out, stats)."""
    B, H, L, d, dt = _check_qkv(q, k, v, out)
    _check_stats(stats, q)
    wp, wn = _ws_args(workspace)
    st = lib().lssar_attn_fwd_stats_ws(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(stats), B, H,
                                       L, d, int(p), float(eps), dt, wp, wn, _stream_ptr(stream))
    _raise(st, "lssar_attn_fwd_stats_ws")
    return out, stats


def lssar_attn_bwd_stats_ws(q, k, v, out, dout, stats, dq, dk, dv, workspace, *, p: int,
                            eps: float = DEFAULT_EPS, stream=None):
    """lssar_attn_bwd_ws with the output and row statistics of
    lssar_attn_fwd_stats_ws (same q, k, v, p, eps).  Returns (dq, dk, dv)."""
    B, H, L, d, dt = _check_qkv(q, k, v, dout)
    _check_qkv(q, out, dout)
    _check_qkv(dq, dk, dv)
    if dq.shape != q.shape or dq.dtype != q.dtype:
        raise ValueError("gradients must match q in shape and dtype")
    _check_stats(stats, q)
    wp, wn = _ws_args(workspace)
    st = lib().lssar_attn_bwd_stats_ws(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout),
                                       _ptr(stats), _ptr(dq), _ptr(dk), _ptr(dv), B, H, L, d,
                                       int(p), float(eps), dt, wp, wn, _stream_ptr(stream))
    _raise(st, "lssar_attn_bwd_stats_ws")
    return dq, dk, dv
