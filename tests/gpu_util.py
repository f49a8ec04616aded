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


# Gradient bars.  Gradients have no natural unit scale, so each tensor is
# held to two bars against its fp64 reference `want`:
#  * max-abs <= GRAD_MAXABS * max(1, max|want|): fp32 inputs run in fp64
#    (measured <= 5e-8); bf16 inputs round every output to bf16 (2^-9) and
#    feed bf16 weights and pair gradients to the matrix products (measured
#    <= 4.9e-3 on ordinary inputs);
#  * norm-wise ||got - want||_F <= GRAD_FRO * ||want||_F, which holds
#    ordinary entries of a tensor with a few large outliers to their own
#    size (the max-abs bar alone is set by the largest entry).  Measured:
#    2.0e-3 to 3.7e-3 for bf16 inputs (the output rounding alone gives about
#    2^-9 / sqrt(3) = 1.1e-3), 2.2e-8 to 2.9e-8 for fp32 inputs.
GRAD_MAXABS = {"f32": 1e-5, "bf16": 1e-2}
GRAD_FRO = {"f32": 2e-7, "bf16": 5e-3}


def check_grads(got, want, dtype, what, maxabs=None):
    """Assert both bars for (dq, dk, dv); returns the three max-abs errors
    relative to max(1, max|want|) and prints the norm-wise ones.  `maxabs`
    replaces the max-abs bar (a test that needs another states why)."""
    bar = GRAD_MAXABS[dtype] if maxabs is None else maxabs
    errs, fros, fails = [], [], []
    for name, a, b in zip(("dq", "dk", "dv"), got, want):
        scale = max(1.0, float(np.max(np.abs(b))))
        err = float(np.max(np.abs(a - b)))
        nb = float(np.linalg.norm(b))
        fro = float(np.linalg.norm(a - b))
        errs.append(err / scale)
        fros.append(fro / nb if nb > 0 else fro)
        if not err <= bar * scale:
            fails.append(f"{name}: max-abs {err:.3e} > {bar} * {scale:.3g}")
        if not fro <= GRAD_FRO[dtype] * nb + 1e-6 * np.sqrt(b.size):
            fails.append(f"{name}: norm-wise {fro:.3e} > {GRAD_FRO[dtype]} * {nb:.3g}")
    print(f"  {what}: max-abs/scale dq {errs[0]:.2e} dk {errs[1]:.2e} dv {errs[2]:.2e}; "
          f"norm-wise dq {fros[0]:.2e} dk {fros[1]:.2e} dv {fros[2]:.2e}", flush=True)
    assert not fails, f"{what}: " + "; ".join(fails)
    return errs
