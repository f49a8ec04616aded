"""Rows whose every score is strongly negative ("deep" rows) vs the oracle.

When a query is anti-aligned with every key it sees, all its base-2 scores
t = log2(e) ln d ln i cos lie far below 0 and Softplus(t) ~ 2^t is lost to
fp32 rounding of 1 + 2^t (completely below t = -24).  The method's weights
are then a softmax-like row and far from degenerate; the kernels must not
return 0 or NaN there.  Inputs: per head, keys -u + noise and queries +u +
noise for one direction u (head 0: every query; head 1: every other query,
the rest random, so deep and ordinary rows share workgroups).
"""
from __future__ import annotations

import numpy as np
import pytest

import lssar_inputs as gen
import oracle
from gpu_util import to_device, to_host, tol_for
from test_gpu_variants import oracle_variant, run_variant

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import softmax_free_attention_amd as sfa
    sfa.lib()


def anti_aligned(L, d, dtype, seed, noise=0.03):
    """[1, 2, L, d] inputs (dtype-exact fp32 values) and the base-2 row maxima."""
    r = np.random.default_rng(seed)
    qs, ks, vs = [], [], []
    for head in range(2):
        u = r.standard_normal(d)
        u /= np.linalg.norm(u)
        K = -u[None] * r.uniform(0.5, 2.0, (L, 1)) + noise * r.standard_normal((L, d))
        Q = u[None] * r.uniform(0.5, 2.0, (L, 1)) + noise * r.standard_normal((L, d))
        if head == 1:
            Q[1::2] = r.standard_normal((len(Q[1::2]), d))
        qs.append(Q)
        ks.append(K)
        vs.append(r.standard_normal((L, d)))
    out = []
    for x in (qs, ks, vs):
        a = np.stack(x)[None].astype(np.float32)
        out.append(gen.round_to_bf16(a) if dtype == "bf16" else a)
    q, k, v = out
    qn = q[0].astype(np.float64) / np.linalg.norm(q[0], axis=-1, keepdims=True)
    kn = k[0].astype(np.float64) / np.linalg.norm(k[0], axis=-1, keepdims=True)
    cos = qn @ np.swapaxes(kn, -1, -2)
    i = np.arange(1, L + 1)
    t = np.log(d) * np.log(i)[None, :, None] * cos / np.log(2.0)
    t[:, np.triu_indices(L, 1)[0], np.triu_indices(L, 1)[1]] = -np.inf
    return q, k, v, t.max(-1)


MODES = [("lssar", 3), ("lssar", 15), ("lssa", 1), ("sigmoid", 15)]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("mode,p", MODES, ids=[f"{m}-p{p}" for m, p in MODES])
def test_deep_rows_parity(dtype, d, mode, p):
    L = 300
    q, k, v, tmax = anti_aligned(L, d, dtype, seed=d + p)
    deep = tmax < -4.0
    assert deep.sum() > 150 and (tmax < -24.0).sum() > 100, "construction lost its deep rows"
    qd, kd, vd = (to_device(a, dtype) for a in (q, k, v))
    if mode == "lssar":
        from gpu_util import run_ws
        got = to_host(run_ws(qd, kd, vd, p))
        want = oracle.lssar_fwd(q, k, v, p)
    else:
        got = to_host(run_variant(qd, kd, vd, mode, p))
        want = oracle_variant(q, k, v, mode, p)
    assert np.all(np.isfinite(got))
    err = np.abs(got - want).max(axis=-1)[0]             # [2, L] per-row max-abs
    print(f"{mode} {dtype} d={d} p={p}: deep rows {int(deep.sum())}, "
          f"max-abs deep {err[deep].max():.3e}, others {err[~deep].max():.3e}", flush=True)
    assert err.max() <= tol_for(dtype), f"max-abs {err.max():.3e}"
    # the method's deep rows are far from degenerate: their outputs are not 0
    nz = np.abs(want[0]).max(axis=-1) > 0.05
    assert np.all(np.abs(got[0]).max(axis=-1)[nz & deep] > 0.0)
