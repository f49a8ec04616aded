"""The workspace entry points allocate nothing and issue only kernels, so a
caller can capture them in a HIP graph.  Each test captures once, then
replays three times with new inputs copied in by eager work between the
replays, and checks every replay bitwise against the eager calls on the
same inputs."""
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
    return torch.equal(a.view(torch.int16), b.view(torch.int16))


def _replays(graph, inputs, fresh, outputs, eager):
    """Copy fresh(n) into the captured inputs, replay, compare with eager()."""
    for n in range(3):
        for dst, src in zip(inputs, fresh(n)):
            dst.copy_(src)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [o.clone() for o in outputs]
        want = eager()
        torch.cuda.synchronize()
        for g, w in zip(got, want):
            assert (torch.equal(g, w) if g.dtype == torch.float64 else _same(g, w)), f"replay {n}"


def _bf16_inputs(name, seed, **kw):
    inp = gen.make_inputs(name, seed=seed, **kw)
    return [to_device(a, "bf16") for a in (inp.q, inp.k, inp.v)]


def test_forward_in_a_graph():
    import softmax_free_attention_amd as sfa
    q, k, v = _bf16_inputs("x8_planted", 1, H=3, L=700)
    ws, out = sfa.workspace_for(q), torch.empty_like(q)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):                 # warm up on the capture stream
        sfa.lssar_attn_fwd_ws(q, k, v, out, ws, p=15)
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sfa.lssar_attn_fwd_ws(q, k, v, out, ws, p=15)

    def eager():
        ref = torch.empty_like(q)
        sfa.lssar_attn_fwd_ws(q, k, v, ref, sfa.workspace_for(q), p=15)
        return [ref]
    _replays(g, [q, k, v], lambda n: _bf16_inputs("x8_planted", 10 + n, H=3, L=700), [out], eager)


def test_training_pair_in_a_graph():
    import softmax_free_attention_amd as sfa
    q, k, v = _bf16_inputs("gpt2s", 2, B=1, H=4, L=300, p=15)
    dout = to_device(gen.round_to_bf16(np.random.default_rng(3).standard_normal(q.shape)
                                       .astype(np.float32)), "bf16")
    fws, bws = sfa.workspace_for(q), sfa.bwd_workspace_for(q)
    out, st = torch.empty_like(q), sfa.stats_for(q)
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))

    def step(o, s_, g3, f_ws, b_ws):
        sfa.lssar_attn_fwd_stats_ws(q, k, v, o, s_, f_ws, p=15)
        sfa.lssar_attn_bwd_stats_ws(q, k, v, o, dout, s_, *g3, b_ws, p=15)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step(out, st, (dq, dk, dv), fws, bws)
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(out, st, (dq, dk, dv), fws, bws)

    def eager():
        o, s_ = torch.empty_like(q), sfa.stats_for(q)
        g3 = [torch.empty_like(q) for _ in range(3)]
        step(o, s_, g3, sfa.workspace_for(q), sfa.bwd_workspace_for(q))
        return [o, s_, *g3]

    def fresh(n):
        a = _bf16_inputs("gpt2s", 20 + n, B=1, H=4, L=300, p=15)
        d = to_device(gen.round_to_bf16(np.random.default_rng(30 + n).standard_normal(q.shape)
                                        .astype(np.float32)), "bf16")
        return [*a, d]
    _replays(g, [q, k, v, dout], fresh, [out, st, dq, dk, dv], eager)


@pytest.mark.parametrize("B,H", [(4, 3), (16, 12)])
def test_decode_in_a_graph(B, H):
    """B*H = 12 runs the three split kernels, B*H = 192 the one-launch kernel."""
    import softmax_free_attention_amd as sfa
    inp = gen.make_decode_inputs("x8_decode_ragged", B=B, H=H, Lmax=900)
    q, kc, vc = (to_device(a, "bf16") for a in (inp.q, inp.k, inp.v))
    lens = torch.from_numpy(np.ascontiguousarray(inp.lens, np.int32)).cuda()
    ws, out = sfa.decode_workspace_for(kc), torch.empty_like(q)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        sfa.lssar_decode_ws(q, kc, vc, lens, out, ws, p=15)
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sfa.lssar_decode_ws(q, kc, vc, lens, out, ws, p=15)

    def eager():
        ref = torch.empty_like(q)
        sfa.lssar_decode_ws(q, kc, vc, lens, ref, sfa.decode_workspace_for(kc), p=15)
        return [ref]

    def fresh(n):
        d = gen.make_decode_inputs("x8_decode_ragged", B=B, H=H, Lmax=900, seed=40 + n)
        new_lens = np.minimum(np.asarray(d.lens, np.int32) - 50 * n, 900).clip(1)
        return [to_device(d.q, "bf16"), to_device(d.k, "bf16"), to_device(d.v, "bf16"),
                torch.from_numpy(np.ascontiguousarray(new_lens, np.int32)).cuda()]
    _replays(g, [q, kc, vc, lens], fresh, [out], eager)
