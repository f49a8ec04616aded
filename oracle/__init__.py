"""fp64 CPU oracle for LSSAR causal attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The HIP library never calls it and the
two share no code.  The arithmetic lives in ``lssar_ref.c`` (plain C, fp64),
which follows the paper note "Softplus Attention with Re-weighting Boosts
Length Extrapolation in Large Language Models", Method details (Key designs
1-3); this module only builds it and marshals numpy arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "lssar_ref.c")
LIB = os.path.join(HERE, "liblssar_ref.so")

DEFAULT_EPS = 1e-4
PHI_SOFTPLUS = 0
PHI_SIGMOID = 1

_lib = None


def build(src: str = SRC, out: str = LIB) -> str:
    """Compile the oracle with gcc (fp64, OpenMP, no fast-math)."""
    tmp = f"{out}.{os.getpid()}.tmp"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                    "-o", tmp, src, "-lm"], check=True)
    os.replace(tmp, out)
    return out


def load(path: str | None = None):
    """Load (building if absent) the oracle library; returns the ctypes CDLL."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build()
        _lib = _bind(ctypes.CDLL(LIB))
    return _lib


def _bind(lib):
    dp = ctypes.POINTER(ctypes.c_double)
    ip = ctypes.POINTER(ctypes.c_int)
    lib.lssar_ref_fwd_f64.argtypes = [dp, dp, dp, dp] + [ctypes.c_int] * 5 + [
        ctypes.c_double, ctypes.c_int]
    lib.lssar_ref_fwd_f64.restype = ctypes.c_int
    lib.lssar_ref_head_rows_f64.argtypes = [dp, dp, dp, ctypes.c_int, ctypes.c_int,
                                            ctypes.c_int, ctypes.c_double, ip,
                                            ctypes.c_int, dp, ctypes.c_int]
    lib.lssar_ref_head_rows_f64.restype = ctypes.c_int
    lib.lssar_ref_fwd_ex_f64.argtypes = [dp, dp, dp, dp] + [ctypes.c_int] * 5 + [
        ctypes.c_double, ctypes.c_int, ctypes.c_int, ctypes.c_int]
    lib.lssar_ref_fwd_ex_f64.restype = ctypes.c_int
    lib.lssar_ref_head_rows_ex_f64.argtypes = [dp, dp, dp, ctypes.c_int, ctypes.c_int,
                                               ctypes.c_int, ctypes.c_double, ctypes.c_int,
                                               ctypes.c_int, ip, ctypes.c_int, dp,
                                               ctypes.c_int]
    lib.lssar_ref_head_rows_ex_f64.restype = ctypes.c_int
    lib.lssar_ref_bwd_f64.argtypes = [dp] * 7 + [ctypes.c_int] * 5 + [ctypes.c_double,
                                                                      ctypes.c_int]
    lib.lssar_ref_bwd_f64.restype = ctypes.c_int
    lib.lssar_ref_rowstats_f64.argtypes = [dp, dp, dp] + [ctypes.c_int] * 5
    lib.lssar_ref_rowstats_f64.restype = ctypes.c_int
    lib.lssar_ref_threads.argtypes = [ctypes.c_int]
    lib.lssar_ref_threads.restype = ctypes.c_int
    return lib


def _f64(x) -> np.ndarray:
    return np.ascontiguousarray(x, dtype=np.float64)


def _ptr(a: np.ndarray, t=ctypes.c_double):
    return a.ctypes.data_as(ctypes.POINTER(t))


def lssar_fwd(q, k, v, p: int, eps: float = DEFAULT_EPS, nthreads: int = 0,
              lib=None, phi: int = PHI_SOFTPLUS, reweight: bool = True) -> np.ndarray:
    """Oracle forward on [B,H,L,d] (or [L,d]) inputs; returns fp64 output.
    ``phi`` picks the stage-1 map (Softplus, or the ablation's Sigmoid);
    ``reweight=False`` stops after stage 1 (the ablation's LSSA only)."""
    lib = lib or load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    squeeze = q.ndim == 2
    if squeeze:
        q, k, v = q[None, None], k[None, None], v[None, None]
    B, H, L, d = q.shape
    assert k.shape == q.shape and v.shape == q.shape
    out = np.empty_like(q)
    rc = lib.lssar_ref_fwd_ex_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, H, L, d,
                                  int(p), float(eps), int(phi), int(bool(reweight)),
                                  int(nthreads))
    if rc != 0:
        raise ValueError(f"lssar_ref_fwd_ex_f64 failed with status {rc}")
    return out[0, 0] if squeeze else out


def lssar_rows(q, k, v, rows, p: int, eps: float = DEFAULT_EPS, nthreads: int = 0,
               lib=None, phi: int = PHI_SOFTPLUS, reweight: bool = True) -> np.ndarray:
    """Oracle output for chosen 0-based query rows of ONE head ([L,d] inputs)."""
    lib = lib or load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    L, d = q.shape
    r = np.ascontiguousarray(rows, dtype=np.int32)
    out = np.empty((len(r), d), dtype=np.float64)
    rc = lib.lssar_ref_head_rows_ex_f64(_ptr(q), _ptr(k), _ptr(v), L, d, int(p),
                                        float(eps), int(phi), int(bool(reweight)),
                                        _ptr(r, ctypes.c_int), len(r), _ptr(out),
                                        int(nthreads))
    if rc != 0:
        raise ValueError(f"lssar_ref_head_rows_ex_f64 failed with status {rc}")
    return out


def lssar_bwd(q, k, v, dout, p: int, eps: float = DEFAULT_EPS, nthreads: int = 0,
              lib=None):
    """Oracle backward on [B,H,L,d] (or [L,d]) inputs for the loss
    sum(dout * out); returns (dq, dk, dv) in fp64."""
    lib = lib or load()
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    squeeze = q.ndim == 2
    if squeeze:
        q, k, v, dout = q[None, None], k[None, None], v[None, None], dout[None, None]
    B, H, L, d = q.shape
    assert k.shape == q.shape and v.shape == q.shape and dout.shape == q.shape
    dq, dk, dv = np.empty_like(q), np.empty_like(q), np.empty_like(q)
    rc = lib.lssar_ref_bwd_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(dq), _ptr(dk),
                               _ptr(dv), B, H, L, d, int(p), float(eps), int(nthreads))
    if rc != 0:
        raise ValueError(f"lssar_ref_bwd_f64 failed with status {rc}")
    if squeeze:
        return dq[0, 0], dk[0, 0], dv[0, 0]
    return dq, dk, dv


def lssar_rowstats(q, k, nthreads: int = 0, lib=None) -> np.ndarray:
    """Oracle row statistics on [B,H,L,d] (or [L,d]) inputs: [..., L, 2] with
    S_i = sum_{j<=i} Softplus(s_ij) (stage 1's L1 norm before normalising)
    and m_i = max_{j<=i} s_ij (the largest unmasked scaled score)."""
    lib = lib or load()
    q, k = _f64(q), _f64(k)
    squeeze = q.ndim == 2
    if squeeze:
        q, k = q[None, None], k[None, None]
    B, H, L, d = q.shape
    assert k.shape == q.shape
    st = np.empty((B, H, L, 2), dtype=np.float64)
    rc = lib.lssar_ref_rowstats_f64(_ptr(q), _ptr(k), _ptr(st), B, H, L, d, int(nthreads))
    if rc != 0:
        raise ValueError(f"lssar_ref_rowstats_f64 failed with status {rc}")
    return st[0, 0] if squeeze else st


def threads(nthreads: int = 0, lib=None) -> int:
    lib = lib or load()
    return int(lib.lssar_ref_threads(int(nthreads)))
