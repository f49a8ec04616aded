"""lssar_attn_fwd_noalloc (the forward with the library's static per-GPU
scratch as its workspace) through the C ABI, against lssar_attn_fwd_ws on the
same inputs: the same kernels on the same data, so bitwise the same output.
Calls in a row share the scratch: a large input, then a smaller one, then
fp32 inputs; an input whose workspace exceeds the scratch is refused."""
from __future__ import annotations

import numpy as np
import pytest

import lssar_inputs as gen
from gpu_util import to_device, to_host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import softmax_free_attention_amd as sfa
    sfa.lib()


def _noalloc_c(q, k, v, out, p, eps=1e-4):
    """One call of the C entry point (ctypes, no Python wrapper)."""
    import softmax_free_attention_amd as sfa
    B, H, L, d = q.shape
    dt = sfa.LSSAR_BF16 if q.dtype == torch.bfloat16 else sfa.LSSAR_F32
    return sfa.lib().lssar_attn_fwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                            out.data_ptr(), B, H, L, d, p, eps, dt,
                                            torch.cuda.current_stream().cuda_stream)


def _ws(q, k, v, p):
    import softmax_free_attention_amd as sfa
    out = torch.empty_like(q)
    sfa.lssar_attn_fwd_ws(q, k, v, out, sfa.workspace_for(q), p=p)
    return out


@pytest.mark.parametrize("case", ["x8", "small", "f32"])
def test_noalloc_matches_ws(case):
    import softmax_free_attention_amd as sfa
    if case == "x8":
        inp = gen.make_inputs("x8_planted")
    elif case == "small":
        inp = gen.make_inputs("gpt2s", B=1, H=2, L=300, p=3, seed=5)
    else:
        inp = gen.make_inputs("tiny")
    wl = inp.wl
    q, k, v = (to_device(a, wl.dtype) for a in (inp.q, inp.k, inp.v))
    print(f"noalloc {case}: B{wl.B} H{wl.H} L{wl.L} d{wl.d} {wl.dtype} p{wl.p}", flush=True)
    out = torch.full_like(q, float("nan"))
    assert _noalloc_c(q, k, v, out, wl.p) == sfa.LSSAR_OK
    want = _ws(q, k, v, wl.p)
    torch.cuda.synchronize()
    if wl.dtype == "bf16":
        assert torch.equal(out.view(torch.int16), want.view(torch.int16))
    else:
        assert torch.equal(out, want)
    assert np.all(np.isfinite(to_host(out)))


def test_noalloc_refuses_input_beyond_scratch():
    import softmax_free_attention_amd as sfa
    shape = (1, 32, 8192, 128)
    assert sfa.lssar_workspace_bytes(*shape, sfa.LSSAR_BF16) > sfa.lssar_noalloc_scratch_bytes()
    q = torch.zeros(shape, dtype=torch.bfloat16, device="cuda")
    out = torch.empty_like(q)
    assert _noalloc_c(q, q.clone(), q.clone(), out, 3) == sfa.LSSAR_ESCRATCH
    # the scratch is still good for the next call
    inp = gen.make_inputs("gpt2s", B=1, H=1, L=130, p=15, seed=9)
    q2, k2, v2 = (to_device(a, "bf16") for a in (inp.q, inp.k, inp.v))
    out2 = torch.empty_like(q2)
    assert _noalloc_c(q2, k2, v2, out2, 15) == sfa.LSSAR_OK
    want = _ws(q2, k2, v2, 15)
    torch.cuda.synchronize()
    assert torch.equal(out2.view(torch.int16), want.view(torch.int16))
