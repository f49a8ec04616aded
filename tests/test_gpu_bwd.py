"""Backward (lssar_attn_bwd_ws) on the HIP path vs the fp64 oracle backward.

Bars (gpu_util.check_grads), per tensor: max-abs <= 1e-5 * max(1, g_max)
for fp32 inputs (the kernels compute in fp64) and <= 1e-2 * max(1, g_max)
for bf16 inputs, where every output element is rounded to bf16 (2^-9
relative) and the scores come from bf16 inputs with fp32 accumulation, as in
the forward; g_max is the tensor's largest reference entry.  Beside it a
norm-wise bar, ||err||_F <= 2e-7 (fp32) or 5e-3 (bf16) times ||want||_F,
holds the ordinary entries of a tensor with outliers to their own size.
"""
from __future__ import annotations

import numpy as np
import pytest

import lssar_inputs as gen
import oracle
from gpu_util import check_grads, to_device, to_host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import softmax_free_attention_amd as sfa
    sfa.lib()


def run_bwd(q, k, v, g, p, eps=1e-4):
    import softmax_free_attention_amd as sfa
    ws = sfa.bwd_workspace_for(q)
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    sfa.lssar_attn_bwd_ws(q, k, v, g, dq, dk, dv, ws, p=p, eps=eps)
    torch.cuda.synchronize()
    return dq, dk, dv


def _inputs(L, d, dtype, p, seed, H=2, name="gpt2s"):
    inp = gen.make_inputs(name, B=1, H=H, L=L, d=d, dtype=dtype, p=p, seed=seed)
    r = np.random.default_rng(seed + 77)
    g = r.standard_normal(inp.q.shape).astype(np.float32)
    if dtype == "bf16":
        g = gen.round_to_bf16(g)
    return inp.q, inp.k, inp.v, g


_check = check_grads


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("p", [1, 2, 3, 15, 7])
def test_small_shapes_bwd_parity(dtype, d, p):
    for L in (1, 2, 3, 4, 5, 17, 64, 65, 130, 257):
        q, k, v, g = _inputs(L, d, dtype, p, seed=L + 5)
        got = [to_host(t) for t in run_bwd(*(to_device(a, dtype) for a in (q, k, v, g)), p)]
        want = oracle.lssar_bwd(q, k, v, g, p)
        errs = _check(got, want, dtype, f"{dtype} d={d} p={p} L={L}")
        print(f"bwd {dtype} d={d} p={p} L={L}: rel max-abs dq {errs[0]:.2e} dk {errs[1]:.2e} "
              f"dv {errs[2]:.2e}", flush=True)


def test_scale_invariance_orthogonality():
    """q_i . dq_i = 0 and k_j . dk_j = 0 (rows of Q and K only enter through
    their directions)."""
    q, k, v, g = _inputs(300, 64, "f32", 15, seed=91)
    dq, dk, _ = (to_host(t) for t in run_bwd(*(to_device(a, "f32") for a in (q, k, v, g)), 15))
    for x, dx in ((q[0], dq[0]), (k[0], dk[0])):
        ortho = np.abs((x.astype(np.float64) * dx).sum(-1))
        scale = np.linalg.norm(x, axis=-1) * np.linalg.norm(dx, axis=-1) + 1e-30
        assert np.max(ortho / scale) < 1e-6


def test_dv_matches_forward_weights():
    """dv = W^T dout, with W read off the GPU forward on V = I."""
    import softmax_free_attention_amd as sfa
    for dtype in ("f32", "bf16"):
        L = 64
        q, k, v, g = _inputs(L, 64, dtype, 3, seed=93)
        qd, kd, vd, gd = (to_device(a, dtype) for a in (q, k, v, g))
        eye = to_device(np.broadcast_to(np.eye(L, dtype=np.float32), (1, 2, L, L)).copy(), dtype)
        W = torch.empty_like(qd)
        sfa.lssar_attn_fwd_ws(qd, kd, eye, W, sfa.workspace_for(qd), p=3)
        _, _, dv = run_bwd(qd, kd, vd, gd, 3)
        Wh = to_host(W)
        want = np.swapaxes(Wh, -1, -2) @ g.astype(np.float64)
        err = float(np.max(np.abs(to_host(dv) - want)))
        assert err <= (1e-5 if dtype == "f32" else 3e-2), f"{dtype}: {err:.3e}"


def test_degenerate_and_deep_rows():
    """Zero queries: rows >= 4 are degenerate and pass no gradient (dq = 0
    there).  Anti-aligned rows (every score far below 0) match the oracle."""
    for dtype in ("f32", "bf16"):
        q, k, v, g = _inputs(150, 64, dtype, 15, seed=95)
        q = q.copy()
        q[:, :, [4, 50, 149]] = 0.0
        got = [to_host(t) for t in run_bwd(*(to_device(a, dtype) for a in (q, k, v, g)), 15)]
        assert np.all(got[0][:, :, [4, 50, 149]] == 0.0)
        _check(got, oracle.lssar_bwd(q, k, v, g, 15), dtype, f"degenerate {dtype}")
    from test_gpu_deep_rows import anti_aligned
    for dtype in ("f32", "bf16"):
        q, k, v, _ = anti_aligned(200, 64, dtype, seed=7)
        g = np.random.default_rng(8).standard_normal(q.shape).astype(np.float32)
        if dtype == "bf16":
            g = gen.round_to_bf16(g)
        got = [to_host(t) for t in run_bwd(*(to_device(a, dtype) for a in (q, k, v, g)), 15)]
        errs = _check(got, oracle.lssar_bwd(q, k, v, g, 15), dtype, f"deep {dtype}")
        print(f"bwd deep {dtype}: rel max-abs {max(errs):.2e}", flush=True)


def test_deterministic():
    q, k, v, g = _inputs(500, 128, "bf16", 15, seed=97, H=3)
    dev = [to_device(a, "bf16") for a in (q, k, v, g)]
    a = run_bwd(*dev, 15)
    b = run_bwd(*dev, 15)
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))


@pytest.mark.parametrize("name,heads", [("gpt2s", [(0, 0), (3, 7), (7, 11)]),
                                        ("x8_planted", [(0, 5), (0, 11)])])
def test_full_workload_sampled_heads(name, heads):
    """Full-size workloads; the oracle backward on a few whole heads."""
    inp = gen.make_inputs(name)
    wl = inp.wl
    r = np.random.default_rng(99)
    g = gen.round_to_bf16(r.standard_normal(inp.q.shape).astype(np.float32))
    got = [to_host(t) for t in run_bwd(*(to_device(a, wl.dtype) for a in (inp.q, inp.k, inp.v, g)),
                                        wl.p)]
    worst = 0.0
    for b, h in heads:
        want = oracle.lssar_bwd(inp.q[b, h], inp.k[b, h], inp.v[b, h], g[b, h], wl.p)
        errs = _check([x[b, h] for x in got], want, wl.dtype, f"{name} b={b} h={h}")
        worst = max(worst, max(errs))
    assert all(np.all(np.isfinite(x)) for x in got)
    print(f"bwd {name}: sampled heads rel max-abs {worst:.2e}", flush=True)
