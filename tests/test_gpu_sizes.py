"""Size extremes of the forward and decode paths vs the oracle.

Long sequences (one head at L = 32768 and a ragged L = 20001: sampled rows,
including the last ones, computed one by one by the oracle) and very many
short heads (a large grid with L = 3 and L = 65, compared in full).
"""
from __future__ import annotations

import numpy as np
import pytest

import lssar_inputs as gen
import oracle
from gpu_util import BF16_TOL, run_ws, to_device, to_host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import softmax_free_attention_amd as sfa
    sfa.lib()


@pytest.mark.parametrize("L,d,p", [(32768, 64, 15), (20001, 128, 3)])
def test_long_sequence_sampled_rows(L, d, p):
    inp = gen.make_inputs("x16", B=1, H=1, L=L, d=d, p=p, seed=L)
    q, k, v = (to_device(a, "bf16") for a in (inp.q, inp.k, inp.v))
    got = to_host(run_ws(q, k, v, p))
    rows = sorted({0, 1, 2, 3, 63, 64, L // 3, L // 2, L - 65, L - 64, L - 2, L - 1}
                  | set(np.random.default_rng(L).integers(0, L, 8).tolist()))
    want = oracle.lssar_rows(inp.q[0, 0], inp.k[0, 0], inp.v[0, 0], rows, p)
    err = float(np.max(np.abs(got[0, 0, rows] - want)))
    print(f"L={L} d={d} p={p}: sampled max-abs {err:.3e}", flush=True)
    assert err <= BF16_TOL and np.all(np.isfinite(got))


@pytest.mark.parametrize("L,d,lo", [(5400, 128, 5120), (22200, 64, 21888)])
def test_pass1_forms_meet(L, d, lo):
    """The plain forward sums a block's Softplus values as the product of the
    factors 1 + 2^t (base 2) while every score is at most 60, that is while
    log2(e) ln d ln(last row) <= 60, and as max(t, 0) plus log2 of the
    factors 1 + 2^-|t| after that: rows 5276 on at d = 128, 22027 on at
    d = 64.  Every row of the four 64-row blocks around the switch against
    the oracle."""
    inp = gen.make_inputs("x16", B=1, H=1, L=L, d=d, p=15, seed=L + d)
    q, k, v = (to_device(a, "bf16") for a in (inp.q, inp.k, inp.v))
    got = to_host(run_ws(q, k, v, 15))
    rows = list(range(lo, lo + 256))
    want = oracle.lssar_rows(inp.q[0, 0], inp.k[0, 0], inp.v[0, 0], rows, 15)
    err = np.max(np.abs(got[0, 0, rows] - want), axis=1)
    print(f"L={L} d={d}: rows {lo}..{lo + 255} max-abs {err.max():.3e} (row {lo + int(err.argmax())})",
          flush=True)
    assert float(err.max()) <= BF16_TOL and np.all(np.isfinite(got))


@pytest.mark.parametrize("L", [3, 65])
def test_many_short_heads(L):
    B, H = 128, 16
    inp = gen.make_inputs("gpt2s", B=B, H=H, L=L, p=15, seed=5 + L)
    q, k, v = (to_device(a, "bf16") for a in (inp.q, inp.k, inp.v))
    got = to_host(run_ws(q, k, v, 15))
    want = oracle.lssar_fwd(inp.q, inp.k, inp.v, 15)
    err = float(np.max(np.abs(got - want)))
    print(f"B={B} H={H} L={L}: max-abs {err:.3e}", flush=True)
    assert err <= BF16_TOL


def test_long_decode_cache():
    """A 32768-row cache with ragged lengths, sampled heads."""
    import softmax_free_attention_amd as sfa
    inp = gen.make_decode_inputs("x8_decode_ragged", B=3, H=2, Lmax=32768)
    q, k, v = (to_device(a, "bf16") for a in (inp.q, inp.k, inp.v))
    out = torch.empty_like(q)
    lens = torch.from_numpy(inp.lens).cuda()
    sfa.lssar_decode_ws(q, k, v, lens, out, sfa.decode_workspace_for(k), p=15)
    got = to_host(out)
    err = 0.0
    for b, n in enumerate(inp.lens):
        for h in range(2):
            qf = np.zeros((n, 64))
            qf[n - 1] = inp.q[b, h]
            want = oracle.lssar_rows(qf, inp.k[b, h, :n], inp.v[b, h, :n], [n - 1], 15)[0]
            err = max(err, float(np.max(np.abs(got[b, h] - want))))
    print(f"decode Lmax=32768: max-abs {err:.3e}", flush=True)
    assert err <= BF16_TOL
