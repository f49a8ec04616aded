"""No kernel reads workspace memory that its own call did not write.

Each entry point runs twice on the same inputs: once with its workspace
filled with zero bytes, once with 0xFF bytes (NaN in every float and double
slot, -1 in every integer).  The outputs must be bitwise equal and finite.
A stale read (a dispatch-table slot, a key factor, a row record or a decode
score that the call itself did not store) shows up as a NaN or as a
difference between the two runs.
"""
from __future__ import annotations

import numpy as np
import pytest

import lssar_inputs as gen
from gpu_util import to_device

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import softmax_free_attention_amd as sfa
    sfa.lib()


def _same(a, b):
    if a.dtype == torch.bfloat16:
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    return torch.equal(a, b)


def _twice(run, ws):
    """run(ws) -> tuple of tensors, with ws zeroed and then 0xFF-filled."""
    ws.zero_()
    a = [t.clone() for t in run(ws)]
    torch.cuda.synchronize()
    ws.fill_(255)
    b = [t.clone() for t in run(ws)]
    torch.cuda.synchronize()
    for n, (x, y) in enumerate(zip(a, b)):
        assert bool(torch.isfinite(x.float()).all()), f"output {n} not finite"
        assert _same(x, y), f"output {n} depends on the workspace's prior contents"


def _inputs(dtype, d, L=333, H=3, seed=17):
    inp = gen.make_inputs("gpt2s", B=1, H=H, L=L, d=d, p=15, seed=seed, dtype=dtype)
    return tuple(to_device(a, dtype) for a in (inp.q, inp.k, inp.v))


@pytest.mark.parametrize("dtype,d", [("bf16", 64), ("bf16", 128), ("f32", 64)])
def test_forward_and_training_forward(dtype, d):
    import softmax_free_attention_amd as sfa
    q, k, v = _inputs(dtype, d)
    out = torch.empty_like(q)
    ws = sfa.workspace_for(q)

    def fwd(w):
        sfa.lssar_attn_fwd_ws(q, k, v, out, w, p=15)
        return (out,)

    _twice(fwd, ws)
    st = sfa.stats_for(q)

    def train(w):
        sfa.lssar_attn_fwd_stats_ws(q, k, v, out, st, w, p=15)
        return (out, st)

    _twice(train, ws)


@pytest.mark.parametrize("dtype,d,p", [("bf16", 64, 15), ("bf16", 64, 3), ("bf16", 128, 15),
                                       ("f32", 64, 15)])
def test_backward_both_paths(dtype, d, p):
    import softmax_free_attention_amd as sfa
    q, k, v = _inputs(dtype, d, seed=23)
    g = torch.randn(q.shape, generator=torch.Generator(device="cuda").manual_seed(5),
                    device="cuda").to(q.dtype)
    out, st = torch.empty_like(q), sfa.stats_for(q)
    sfa.lssar_attn_fwd_stats_ws(q, k, v, out, st, sfa.workspace_for(q), p=p)
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    ws = sfa.bwd_workspace_for(q)

    def saved(w):
        sfa.lssar_attn_bwd_stats_ws(q, k, v, out, g, st, dq, dk, dv, w, p=p)
        return (dq, dk, dv)

    def recompute(w):
        sfa.lssar_attn_bwd_ws(q, k, v, g, dq, dk, dv, w, p=p)
        return (dq, dk, dv)

    _twice(saved, ws)
    _twice(recompute, ws)


@pytest.mark.parametrize("d", [64, 128])
def test_decode(d):
    import softmax_free_attention_amd as sfa
    inp = gen.make_decode_inputs("x8_decode", B=4, H=3, Lmax=517, d=d, dtype="bf16", p=15, seed=9)
    q, k, v = (to_device(a, "bf16") for a in (inp.q, inp.k, inp.v))
    lens = torch.from_numpy(np.array([1, 200, 517, 300], np.int32)).cuda()
    out = torch.empty_like(q)
    ws = sfa.decode_workspace_for(k)

    def dec(w):
        sfa.lssar_decode_ws(q, k, v, lens, out, w, p=15)
        return (out,)

    _twice(dec, ws)
