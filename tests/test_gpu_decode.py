"""Decode step (lssar_decode_ws) on the HIP path vs the fp64 oracle.

The decode output of (b, h) is row i = lens[b] of the causal forward over the
cache prefix, so the oracle is its row function on that prefix (the new query
placed at row i).  Bars as for the forward: max-abs 1e-5 for fp32 inputs,
3e-2 for bf16 inputs.
"""
from __future__ import annotations

import numpy as np
import pytest

import lssar_inputs as gen
import oracle
from gpu_util import BF16_TOL, to_device, to_host, tol_for

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import softmax_free_attention_amd as sfa
    sfa.lib()


def run_decode(q, k, v, lens, p, eps=1e-4):
    """q [B,H,d], k/v [B,H,Lmax,d] device tensors; lens: numpy int32 or None."""
    import softmax_free_attention_amd as sfa
    ws = sfa.decode_workspace_for(k)
    out = torch.empty_like(q)
    lt = None if lens is None else torch.from_numpy(np.ascontiguousarray(lens, np.int32)).cuda()
    sfa.lssar_decode_ws(q, k, v, lt, out, ws, p=p, eps=eps)
    torch.cuda.synchronize()
    return out


def oracle_decode(q, k, v, lens, p, eps=1e-4, heads=None):
    """Oracle rows: {(b, h): out row} for the given heads (all by default)."""
    B, H, L, d = k.shape
    res = {}
    for b in range(B):
        n = int(min(max(lens[b], 0), L))
        for h in range(H):
            if heads is not None and (b, h) not in heads:
                continue
            if n == 0:
                res[(b, h)] = np.zeros(d)
                continue
            qf = np.zeros((n, d))
            qf[n - 1] = q[b, h]
            res[(b, h)] = oracle.lssar_rows(qf, k[b, h, :n], v[b, h, :n], [n - 1], p, eps)[0]
    return res


def _compare(got, want, tol, what):
    worst = 0.0
    for (b, h), row in want.items():
        err = float(np.max(np.abs(got[b, h] - row)))
        worst = max(worst, err)
        assert err <= tol, f"{what} b={b} h={h}: max-abs {err:.3e} > {tol}"
    return worst


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("p", [3, 15, 7])
def test_small_decode_parity(dtype, d, p):
    tol = tol_for(dtype)
    for Lmax in (1, 5, 256, 300, 513):
        inp = gen.make_decode_inputs("x8_decode", B=6, H=2, Lmax=Lmax, d=d, dtype=dtype, p=p,
                                     seed=Lmax)
        lens = np.array([1, 2, 3, 4, Lmax, max(1, Lmax // 2 + 7)], np.int32)
        lens = np.minimum(lens, Lmax)
        q, k, v = (to_device(a, dtype) for a in (inp.q, inp.k, inp.v))
        got = to_host(run_decode(q, k, v, lens, p))
        want = oracle_decode(inp.q, inp.k, inp.v, lens, p)
        worst = _compare(got, want, tol, f"{dtype} d={d} p={p} Lmax={Lmax}")
        print(f"decode {dtype} d={d} p={p} Lmax={Lmax}: max-abs {worst:.3e}", flush=True)


def test_lens_none_means_full_cache():
    inp = gen.make_decode_inputs("x8_decode", B=2, H=3, Lmax=700, dtype="bf16")
    q, k, v = (to_device(a, "bf16") for a in (inp.q, inp.k, inp.v))
    a = run_decode(q, k, v, None, 15)
    b = run_decode(q, k, v, np.full(2, 700, np.int32), 15)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_rows_past_length_never_read():
    """Cache rows at or past lens[b] hold NaN: the output is unchanged (bitwise)."""
    for dtype in ("bf16", "f32"):
        inp = gen.make_decode_inputs("x8_decode_ragged", B=5, H=2, Lmax=600, dtype=dtype)
        q, k, v = (to_device(a, dtype) for a in (inp.q, inp.k, inp.v))
        base = run_decode(q, k, v, inp.lens, 15)
        k2, v2 = k.clone(), v.clone()
        for b, n in enumerate(inp.lens):
            k2[b, :, n:] = float("nan")
            v2[b, :, n:] = float("nan")
        o2 = run_decode(q, k2, v2, inp.lens, 15)
        assert torch.equal(o2, base) and bool(torch.isfinite(o2).all())


def test_edge_lengths_and_degenerate_rows():
    """lens 0 gives zeros; lens above Lmax is clamped to Lmax; a zero query
    makes every score 0: degenerate (0) from row 4 on, mean of v before."""
    inp = gen.make_decode_inputs("x8_decode", B=6, H=2, Lmax=200, dtype="bf16")
    q = inp.q.copy()
    q[2:] = 0.0
    lens = np.array([0, 1000, 1, 3, 4, 200], np.int32)
    qd, k, v = (to_device(a, "bf16") for a in (q, inp.k, inp.v))
    got = to_host(run_decode(qd, k, v, lens, 3))
    assert np.all(got[0] == 0.0)
    want = oracle_decode(q, inp.k, inp.v, np.minimum(lens, 200), 3)
    _compare(got, want, BF16_TOL, "edge")
    assert np.all(got[4:] == 0.0)
    for b, n in ((2, 1), (3, 3)):
        assert np.max(np.abs(got[b] - inp.v[b, :, :n].astype(np.float64).mean(axis=1))) <= BF16_TOL


def test_decode_matches_forward_rows():
    """Decode at position i reproduces row i of the forward kernel (both are
    checked against the oracle elsewhere; here they agree with each other)."""
    import softmax_free_attention_amd as sfa
    L = 333
    inp = gen.make_inputs("gpt2s", B=1, H=4, L=L, d=64, p=15, seed=81)
    qf, kf, vf = (to_device(a, "bf16") for a in (inp.q, inp.k, inp.v))
    ws = sfa.workspace_for(qf)
    fwd = torch.empty_like(qf)
    sfa.lssar_attn_fwd_ws(qf, kf, vf, fwd, ws, p=15)
    for i in (1, 2, 4, 64, 65, 200, L):
        q = qf[:, :, i - 1].contiguous()
        out = run_decode(q, kf, vf, np.array([i], np.int32), 15)
        diff = float((out.float() - fwd[:, :, i - 1].float()).abs().max())
        assert diff <= 2e-2, f"row {i}: decode vs forward {diff:.3e}"


def test_deep_rows():
    """Every score far below 0 (query anti-aligned with the whole cache)."""
    from test_gpu_deep_rows import anti_aligned
    for dtype in ("bf16", "f32"):
        q4, k4, v4, _ = anti_aligned(400, 64, dtype, seed=5)
        # sequence b = head pair of the construction, query = its row lens[b]-1
        lens = np.array([400, 137], np.int32)
        k = np.concatenate([k4, k4], axis=0)             # [2, 2, 400, 64]
        v = np.concatenate([v4, v4], axis=0)
        q = np.stack([q4[0, :, lens[0] - 1], q4[0, :, lens[1] - 1]])   # [2, 2, 64]
        qd, kd, vd = (to_device(a, dtype) for a in (q, k, v))
        got = to_host(run_decode(qd, kd, vd, lens, 15))
        want = oracle_decode(q, k, v, lens, 15)
        worst = _compare(got, want, tol_for(dtype), f"deep {dtype}")
        print(f"decode deep {dtype}: max-abs {worst:.3e}", flush=True)


def test_deterministic():
    inp = gen.make_decode_inputs("wide_decode", B=2, H=4, Lmax=3000)
    q, k, v = (to_device(a, "bf16") for a in (inp.q, inp.k, inp.v))
    a = run_decode(q, k, v, inp.lens, 15)
    b = run_decode(q, k, v, inp.lens, 15)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


# From this many (batch, head) pairs on, bf16 decode runs as one launch with
# one workgroup per head; below it, as three launches over cache chunks.
FUSED_MIN_HEADS = 176


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("p", [3, 15, 7])
def test_one_launch_path_parity(d, p):
    """bf16 with B*H >= 176 (one workgroup per head): every head against the
    oracle, at lengths 0..4, one round of keys and the next (512 keys per
    round at d = 64, 256 at d = 128) and their ragged tails, a length above
    Lmax (clamped) and the full cache."""
    B, H = 16, -(-FUSED_MIN_HEADS // 16)
    for Lmax in (5, 513, 1100):
        inp = gen.make_decode_inputs("x8_decode", B=B, H=H, Lmax=Lmax, d=d, dtype="bf16", p=p,
                                     seed=Lmax + d)
        lens = np.array([0, 1, 2, 3, 4, 255, 256, 257, 511, 512, 513, 1000, 1023, 1100,
                         Lmax + 50, Lmax], np.int32)
        q, k, v = (to_device(a, "bf16") for a in (inp.q, inp.k, inp.v))
        got = to_host(run_decode(q, k, v, lens, p))
        eff = np.minimum(lens, Lmax)
        assert np.all(got[0] == 0.0)
        want = oracle_decode(inp.q, inp.k, inp.v, eff, p)
        worst = _compare(got, want, BF16_TOL, f"one launch d={d} p={p} Lmax={Lmax}")
        print(f"one-launch decode d={d} p={p} Lmax={Lmax}: max-abs {worst:.3e}", flush=True)


def test_one_launch_path_without_lens():
    """B*H >= 176 with lens = NULL: every head uses all Lmax rows."""
    B, H, Lmax = 16, 12, 700
    inp = gen.make_decode_inputs("x8_decode", B=B, H=H, Lmax=Lmax, d=64, dtype="bf16", seed=11)
    q, k, v = (to_device(a, "bf16") for a in (inp.q, inp.k, inp.v))
    got = to_host(run_decode(q, k, v, None, 15))
    want = oracle_decode(inp.q, inp.k, inp.v, np.full(B, Lmax, np.int32), 15)
    worst = _compare(got, want, BF16_TOL, "one launch, lens NULL")
    print(f"one-launch decode, lens NULL: max-abs {worst:.3e}", flush=True)


def test_one_launch_path_matches_split_path():
    """The same heads through both paths (B*H = 192 runs as one launch, the
    first two sequences alone, B*H = 24, as three): the outputs agree to the
    bf16 bar, and the one-launch path is deterministic."""
    for d in (64, 128):
        inp = gen.make_decode_inputs("x8_decode_ragged", B=16, H=12, Lmax=900, d=d, dtype="bf16",
                                     seed=d)
        q, k, v = (to_device(a, "bf16") for a in (inp.q, inp.k, inp.v))
        one = run_decode(q, k, v, inp.lens, 15)
        again = run_decode(q, k, v, inp.lens, 15)
        assert torch.equal(one.view(torch.int16), again.view(torch.int16))
        split = run_decode(q[:2].contiguous(), k[:2].contiguous(), v[:2].contiguous(),
                           inp.lens[:2], 15)
        diff = float((one[:2].float() - split.float()).abs().max())
        print(f"d={d}: one launch vs split max-abs {diff:.3e}", flush=True)
        assert diff <= BF16_TOL


def test_one_launch_path_edges():
    """B*H >= 176: rows past each length hold NaN and are never read (bitwise
    the same output); a zero query makes every score 0, so rows from 4 on are
    degenerate (0) and rows 1..3 the mean of their values."""
    B, H, Lmax = 16, 12, 600
    inp = gen.make_decode_inputs("x8_decode_ragged", B=B, H=H, Lmax=Lmax, dtype="bf16", seed=4)
    q, k, v = (to_device(a, "bf16") for a in (inp.q, inp.k, inp.v))
    base = run_decode(q, k, v, inp.lens, 15)
    k2, v2 = k.clone(), v.clone()
    for b, n in enumerate(inp.lens):
        k2[b, :, n:] = float("nan")
        v2[b, :, n:] = float("nan")
    o2 = run_decode(q, k2, v2, inp.lens, 15)
    assert torch.equal(o2.view(torch.int16), base.view(torch.int16))
    assert bool(torch.isfinite(o2.float()).all())
    qz = np.zeros_like(inp.q)
    lens = np.array([1, 2, 3, 4, 5, 600] + [300] * (B - 6), np.int32)
    got = to_host(run_decode(to_device(qz, "bf16"), k, v, lens, 3))
    assert np.all(got[3:] == 0.0)
    for b in range(3):
        n = int(lens[b])
        mean = inp.v[b, :, :n].astype(np.float64).mean(axis=1)
        assert np.max(np.abs(got[b] - mean)) <= BF16_TOL


@pytest.mark.parametrize("name", ["x8_decode", "x8_decode_ragged", "wide_decode"])
def test_full_decode_workload_sampled(name):
    """The bench's decode workloads at full size, sampled heads vs the oracle."""
    inp = gen.make_decode_inputs(name)
    wl = inp.wl
    q, k, v = (to_device(a, wl.dtype) for a in (inp.q, inp.k, inp.v))
    got = to_host(run_decode(q, k, v, inp.lens, wl.p))
    rng = np.random.default_rng(3)
    heads = {(int(b), int(h)) for b, h in zip(rng.integers(0, wl.B, 24), rng.integers(0, wl.H, 24))}
    heads |= {(0, 0), (wl.B - 1, wl.H - 1)}
    want = oracle_decode(inp.q, inp.k, inp.v, inp.lens, wl.p, heads=heads)
    worst = _compare(got, want, BF16_TOL, name)
    assert np.all(np.isfinite(got))
    print(f"{name}: sampled max-abs {worst:.3e}", flush=True)


def test_binding_rejects_bad_input():
    import softmax_free_attention_amd as sfa
    k = torch.zeros(2, 2, 64, 64, dtype=torch.bfloat16, device="cuda")
    q = torch.zeros(2, 2, 64, dtype=torch.bfloat16, device="cuda")
    ws = sfa.decode_workspace_for(k)
    with pytest.raises(ValueError):
        sfa.lssar_decode_ws(q, k, k, torch.zeros(2, dtype=torch.int64, device="cuda"),
                            torch.empty_like(q), ws, p=3)
    with pytest.raises(sfa.LssarError) as e:
        sfa.lssar_decode_ws(q, k, k, None, torch.empty_like(q), ws[:64], p=3)
    assert e.value.status == sfa.LSSAR_EWORKSPACE
