"""Seeded synthetic inputs for LSSAR causal attention.

This module is shared by the fp64 oracle side (tests, bench baseline) and the
HIP side (tests, bench).  It holds none of the attention method's arithmetic:
only a counter-based random generator, the rounding of fp32 draws to bf16, and
the five workload recipes (shapes, value distributions and planted structure).

Generator
---------
Counter-based SplitMix64 (Steele, Lea & Flood, "Fast splittable pseudorandom
number generators", OOPSLA 2014): the n-th 64-bit word of stream ``s`` under
``seed`` is ``mix(base(seed, s) + (n + 1) * GAMMA)``, so any element can be
drawn without drawing the ones before it.  Pairs of words become two standard
normals by the Box-Muller transform, in fp64, then round to fp32 (and to bf16
with round-to-nearest-even for bf16 workloads).  Streams: Q = 0, K = 1, V = 2,
planted structure / shared factors = 3.

Workloads
---------
The pages measure a GPT-2-small (124M) model with RoPE trained at sequence
length 1024 on FineWeb-10B, then extrapolated to 8K and 16K (paper note
"Softplus Attention with Re-weighting Boosts Length Extrapolation in Large
Language Models", Training strategy and Main experiment).  Neither the data
set nor trained weights exist here, so each workload stands in for the
attention tensors of that model by a synthetic distribution of the same shape:
i.i.d. N(0,1) rows, one workload with planted sharp peaks and one wide-head
workload with low-rank correlated Q/K.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "workload", "normals", "uniforms", "words",
    "round_to_bf16", "bf16_bits", "make_inputs", "Inputs",
    "DecodeWorkload", "DECODE_WORKLOADS", "DecodeInputs", "make_decode_inputs", "decode_lens",
]

_GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_S30 = np.uint64(30)
_S27 = np.uint64(27)
_S31 = np.uint64(31)

STREAM_Q, STREAM_K, STREAM_V, STREAM_AUX = 0, 1, 2, 3

# Chunk size (in 64-bit words) for vectorised generation: bounds peak memory.
_CHUNK = 1 << 22


def _mix(z: np.ndarray) -> np.ndarray:
    """SplitMix64 output function (wrapping uint64 arithmetic)."""
    z = (z ^ (z >> _S30)) * _M1
    z = (z ^ (z >> _S27)) * _M2
    return z ^ (z >> _S31)


def _base(seed: int, stream: int) -> np.uint64:
    with np.errstate(over="ignore"):
        s = np.array([(seed * 0x100000001B3 + stream * 0x632BE59BD9B4E019)
                      & 0xFFFFFFFFFFFFFFFF], dtype=np.uint64)
        return _mix(s + _GAMMA)[0]


def words(seed: int, stream: int, start: int, count: int) -> np.ndarray:
    """64-bit words ``start .. start+count-1`` of one counter-based stream."""
    base = _base(seed, stream)
    out = np.empty(count, dtype=np.uint64)
    with np.errstate(over="ignore"):
        for c0 in range(0, count, _CHUNK):
            c1 = min(count, c0 + _CHUNK)
            n = np.arange(start + c0 + 1, start + c1 + 1, dtype=np.uint64)
            out[c0:c1] = _mix(base + n * _GAMMA)
    return out


def uniforms(seed: int, stream: int, start: int, count: int) -> np.ndarray:
    """Uniform fp64 draws in (0, 1]: top 53 bits of each word, plus one ulp."""
    w = words(seed, stream, start, count)
    return ((w >> np.uint64(11)).astype(np.float64) + 1.0) * (2.0 ** -53)


def _normals_into(out: np.ndarray, seed: int, stream: int, start: int, p0: int, p1: int) -> None:
    u = uniforms(seed, stream, start + 2 * p0, 2 * (p1 - p0))
    r = np.sqrt(-2.0 * np.log(u[0::2]))
    th = (2.0 * math.pi) * u[1::2]
    out[2 * p0:2 * p1:2] = r * np.cos(th)
    out[2 * p0 + 1:2 * p1:2] = r * np.sin(th)


def normals(seed: int, stream: int, start: int, count: int) -> np.ndarray:
    """Standard normal fp64 draws by Box-Muller over consecutive word pairs.

    Normal ``2m`` and ``2m+1`` of a stream both come from words ``2m, 2m+1``;
    ``start`` must be even so that a slice reproduces the full sequence.
    Large draws are split into chunks that threads fill independently (each
    element depends on its counter only, so the values do not change).
    """
    assert start % 2 == 0
    npairs = (count + 1) // 2
    out = np.empty(2 * npairs, dtype=np.float64)
    chunks = [(p0, min(npairs, p0 + _CHUNK // 2)) for p0 in range(0, npairs, _CHUNK // 2)]
    if len(chunks) > 1:
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(max_workers=min(len(chunks), _threads())) as ex:
            list(ex.map(lambda c: _normals_into(out, seed, stream, start, c[0], c[1]), chunks))
    else:
        for p0, p1 in chunks:
            _normals_into(out, seed, stream, start, p0, p1)
    return out[:count]


def _threads() -> int:
    import os
    try:
        return max(1, min(16, len(os.sched_getaffinity(0))))
    except AttributeError:
        return max(1, min(16, os.cpu_count() or 1))


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest, ties to even (finite input)."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((b >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((b + bias) >> np.uint32(16)).astype(np.uint16)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """fp32 values rounded to the nearest bf16 value, returned as fp32."""
    return (bf16_bits(x).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    L: int
    d: int
    dtype: str          # "f32" or "bf16"
    p: int
    structure: str      # "iid", "planted" or "lowrank"
    seed: int = 0
    note: str = ""

    @property
    def pairs(self) -> int:
        """Unmasked (query, key) pairs: B*H*L(L+1)/2."""
        return self.B * self.H * self.L * (self.L + 1) // 2

    @property
    def flops(self) -> int:
        """Algorithmic flops: QK^T once plus P.V once over the causal pairs."""
        return 4 * self.d * self.pairs

    def with_(self, **kw) -> "Workload":
        f = {k: getattr(self, k) for k in self.__dataclass_fields__}
        f.update(kw)
        return Workload(**f)


WORKLOADS = {
    "tiny": Workload("tiny", 1, 1, 128, 64, "f32", 3, "iid",
                     note="B1 H1 L128 d64 fp32 p=3, Q/K/V iid N(0,1)"),
    "gpt2s": Workload("gpt2s", 8, 12, 1024, 64, "bf16", 3, "iid",
                      note="GPT-2-small attention shape at its training length"),
    "x8_planted": Workload("x8_planted", 1, 12, 8192, 64, "bf16", 15, "planted",
                           note="8x extrapolation, 16 planted keys per head at cosine 0.9"),
    "x16": Workload("x16", 1, 12, 16384, 64, "bf16", 15, "iid",
                    note="16x extrapolation, iid N(0,1)"),
    "wide": Workload("wide", 2, 32, 4096, 128, "bf16", 15, "lowrank",
                     note="wide head, rank-8 correlated Q/K plus std-0.1 noise"),
}
WORKLOAD_ORDER = ["tiny", "gpt2s", "x8_planted", "x16", "wide"]


def workload(name: str) -> Workload:
    return WORKLOADS[name]


@dataclass
class Inputs:
    """Q, K, V as fp32 arrays [B,H,L,d] holding exactly representable values
    of the workload dtype (bf16-rounded for bf16 workloads)."""
    wl: Workload
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    meta: dict = field(default_factory=dict)

    def device_arrays(self):
        """Arrays in the storage dtype: fp32, or bf16 bit patterns (uint16)."""
        if self.wl.dtype == "f32":
            return self.q, self.k, self.v
        return bf16_bits(self.q), bf16_bits(self.k), bf16_bits(self.v)


def _finish(x: np.ndarray, dtype: str) -> np.ndarray:
    """fp64 draws -> fp32 (round to nearest) -> bf16 values for bf16 workloads;
    large arrays are converted in chunks by threads."""
    src = np.ascontiguousarray(x).reshape(-1)
    out = np.empty(src.shape, dtype=np.float32)

    def conv(c0):
        c1 = min(src.size, c0 + _CHUNK)
        y = src[c0:c1].astype(np.float32)
        out[c0:c1] = round_to_bf16(y) if dtype == "bf16" else y

    starts = range(0, src.size, _CHUNK)
    if len(starts) > 1:
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(max_workers=min(len(starts), _threads())) as ex:
            list(ex.map(conv, starts))
    else:
        for c0 in starts:
            conv(c0)
    return out.reshape(x.shape)


def _iid(wl: Workload, stream: int) -> np.ndarray:
    n = wl.B * wl.H * wl.L * wl.d
    return normals(wl.seed, stream, 0, n).reshape(wl.B, wl.H, wl.L, wl.d)


def _planted(wl: Workload, q: np.ndarray, k: np.ndarray, meta: dict) -> None:
    """Plant 16 keys per head aligned (cosine 0.9 before rounding) to one query.

    Per head: an index r uniform in [L/2, L); u = q_r/|q_r|; 16 distinct key
    positions j <= r; k_j <- |k_j| (0.9 u + sqrt(0.19) w_j) with w_j a unit
    vector orthogonal to u drawn from N(0, I).  Draws come from the auxiliary
    stream, in a fixed order per head.
    """
    B, H, L, d = q.shape
    npl = 16
    rows = []
    for b in range(B):
        for h in range(H):
            bh = b * H + h
            # per-head block of auxiliary words: 1 for r, 64 for positions,
            # npl*d normals for the orthogonal directions
            wbase = bh * (1 << 20)
            r = L // 2 + int(uniforms(wl.seed, STREAM_AUX, wbase, 1)[0] * (L - L // 2))
            r = min(r, L - 1)
            cand = uniforms(wl.seed, STREAM_AUX, wbase + 2, 4 * npl)
            pos = []
            for c in cand:
                j = min(int(c * (r + 1)), r)
                if j not in pos:
                    pos.append(j)
                if len(pos) == npl:
                    break
            assert len(pos) == npl
            u = q[b, h, r].astype(np.float64)
            u = u / np.linalg.norm(u)
            g = normals(wl.seed, STREAM_AUX, wbase + 4096, npl * d).reshape(npl, d)
            for t, j in enumerate(pos):
                w = g[t] - np.dot(g[t], u) * u
                w = w / np.linalg.norm(w)
                nk = np.linalg.norm(k[b, h, j].astype(np.float64))
                k[b, h, j] = nk * (0.9 * u + math.sqrt(0.19) * w)
            rows.append((b, h, r, sorted(pos)))
    meta["planted"] = rows


def _lowrank(wl: Workload):
    """Q = Z_q U / sqrt(8) + 0.1 E, K = Z_k U / sqrt(8) + 0.1 E' per (b,h).

    U (8 x d) is shared by Q and K of one head, from the auxiliary stream;
    Z and E come from the Q (resp. K) stream: first B*H*L*8 normals for Z,
    then B*H*L*d normals for E.
    """
    B, H, L, d = wl.B, wl.H, wl.L, wl.d
    R = 8
    U = normals(wl.seed, STREAM_AUX, 0, B * H * R * d).reshape(B, H, R, d)
    out = []
    for stream in (STREAM_Q, STREAM_K):
        nz = B * H * L * R
        nz_even = nz + (nz & 1)
        Z = normals(wl.seed, stream, 0, nz).reshape(B, H, L, R)
        E = normals(wl.seed, stream, nz_even, B * H * L * d).reshape(B, H, L, d)
        X = np.matmul(Z, U) / math.sqrt(R) + 0.1 * E
        out.append(X)
    return out


def make_inputs(wl: Workload | str, **overrides) -> Inputs:
    """Draw the inputs of a workload (optionally with fields overridden)."""
    if isinstance(wl, str):
        wl = WORKLOADS[wl]
    if overrides:
        wl = wl.with_(**overrides)
    meta: dict = {}
    if wl.structure == "lowrank":
        q, k = _lowrank(wl)
    else:
        q = _iid(wl, STREAM_Q)
        k = _iid(wl, STREAM_K)
    v = _iid(wl, STREAM_V)
    q = _finish(q, wl.dtype)
    k = np.array(_finish(k, wl.dtype))
    if wl.structure == "planted":
        kk = k.astype(np.float64)
        _planted(wl, q, kk, meta)
        k = _finish(kk, wl.dtype)
    v = _finish(v, wl.dtype)
    return Inputs(wl, q, k, v, meta)


# --------------------------------------------------------------------------
# Decode step: one new query per (batch, head) against a key/value cache
# --------------------------------------------------------------------------

@dataclass(frozen=True)
class DecodeWorkload:
    """A batch of B sequences, each with its own cache length lens[b] <= Lmax.
    lens: "full" (every sequence at Lmax) or "ragged" (uniform in
    [Lmax/2, Lmax] from the auxiliary stream)."""
    name: str
    B: int
    H: int
    Lmax: int
    d: int
    dtype: str
    p: int
    lens: str = "full"
    seed: int = 0
    note: str = ""

    def with_(self, **kw) -> "DecodeWorkload":
        f = {k: getattr(self, k) for k in self.__dataclass_fields__}
        f.update(kw)
        return DecodeWorkload(**f)


DECODE_WORKLOADS = {
    "x8_decode": DecodeWorkload("x8_decode", 16, 12, 8192, 64, "bf16", 15, "full",
                                note="8x extrapolation at inference: 16 sequences of 8192 "
                                     "cached tokens, GPT-2-small heads"),
    "x8_decode_ragged": DecodeWorkload("x8_decode_ragged", 16, 12, 8192, 64, "bf16", 15,
                                       "ragged", note="as x8_decode, lengths in [4096, 8192]"),
    "wide_decode": DecodeWorkload("wide_decode", 4, 32, 4096, 128, "bf16", 15, "ragged",
                                  note="wide heads, lengths in [2048, 4096]"),
}


@dataclass
class DecodeInputs:
    """q [B,H,d]; k, v [B,H,Lmax,d] (dtype-exact fp32 values); lens int32 [B]."""
    wl: DecodeWorkload
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    lens: np.ndarray


def make_decode_inputs(wl: DecodeWorkload | str, **overrides) -> DecodeInputs:
    """Cache rows and queries i.i.d. N(0,1) from streams K, V and Q; lengths
    from the auxiliary stream.  Rows past a sequence's length are drawn too
    (they must never be read)."""
    if isinstance(wl, str):
        wl = DECODE_WORKLOADS[wl]
    if overrides:
        wl = wl.with_(**overrides)
    B, H, L, d = wl.B, wl.H, wl.Lmax, wl.d
    q = normals(wl.seed, STREAM_Q, 0, B * H * d).reshape(B, H, d)
    k = normals(wl.seed, STREAM_K, 0, B * H * L * d).reshape(B, H, L, d)
    v = normals(wl.seed, STREAM_V, 0, B * H * L * d).reshape(B, H, L, d)
    return DecodeInputs(wl, _finish(q, wl.dtype), _finish(k, wl.dtype), _finish(v, wl.dtype),
                        decode_lens(wl))


def decode_lens(wl: DecodeWorkload) -> np.ndarray:
    """Cache length of each sequence (int32 [B])."""
    B, L = wl.B, wl.Lmax
    if wl.lens == "full":
        return np.full(B, L, dtype=np.int32)
    u = uniforms(wl.seed, STREAM_AUX, 0, B)
    return np.minimum(L // 2 + (u * (L - L // 2 + 1)).astype(np.int64), L).astype(np.int32)
