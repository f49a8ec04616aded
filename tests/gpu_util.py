"""Helpers for GPU tests: upload seeded inputs, run the HIP path, download."""
from __future__ import annotations

import numpy as np

# Parity bars (max-abs against the fp64 oracle): fp32 inputs 1e-5, bf16
# inputs with fp32 accumulation 3e-2.
F32_TOL = 1e-5
BF16_TOL = 3e-2


def tol_for(dtype: str) -> float:
    return F32_TOL if dtype == "f32" else BF16_TOL


def to_device(a: np.ndarray, dtype: str):
    """fp32 array holding dtype-exact values -> device tensor of that dtype."""
    import torch
    import lssar_inputs as gen
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()
    bits = gen.bf16_bits(a)
    return torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)


def to_host(t) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def run_ws(q, k, v, p, eps=1e-4, stream=None):
    """One call of lssar_attn_fwd_ws (the bench's launch configuration)."""
    import torch
    import softmax_free_attention_amd as sfa
    ws = sfa.workspace_for(q)
    out = torch.empty_like(q)
    sfa.lssar_attn_fwd_ws(q, k, v, out, ws, p=p, eps=eps, stream=stream)
    return out
