"""HIP path vs the fp64 oracle, element by element, through the C ABI.

Bars: max-abs 1e-5 for fp32 inputs, 3e-2 for bf16 inputs (fp32
accumulation).  Small shapes are compared in full (several 64-key tiles and
128-row query blocks, ragged tails, L = 1..5 edge cases).  At full size, in
the launch configuration the bench times: every row of the GPT-2-small and
8x-extrapolation workloads, whole heads of the 16x and wide-head workloads
plus sampled rows across their other heads, and invariants that hold at any
size.
"""
from __future__ import annotations

import numpy as np
import pytest

import lssar_inputs as gen
import oracle
from gpu_util import BF16_TOL, F32_TOL, run_ws, to_device, to_host, tol_for

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import softmax_free_attention_amd as sfa
    sfa.lib()


def _gpu_out(inp, p=None, eps=1e-4):
    wl = inp.wl
    q, k, v = (to_device(a, wl.dtype) for a in (inp.q, inp.k, inp.v))
    out = run_ws(q, k, v, p if p is not None else wl.p, eps)
    torch.cuda.synchronize()
    return to_host(out)


SMALL_L = [1, 2, 3, 4, 5, 17, 63, 64, 65, 127, 128, 129, 255, 300, 513]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("p", [1, 2, 3, 15, 7])
def test_small_shapes_full_parity(dtype, d, p):
    tol = tol_for(dtype)
    for L in SMALL_L:
        inp = gen.make_inputs("gpt2s", B=1, H=2, L=L, d=d, dtype=dtype, p=p, seed=L)
        got = _gpu_out(inp)
        want = oracle.lssar_fwd(inp.q, inp.k, inp.v, p)
        err = float(np.max(np.abs(got - want)))
        print(f"{dtype} d={d} p={p} L={L}: max-abs {err:.3e}", flush=True)
        assert err <= tol, f"{dtype} d={d} p={p} L={L}: max-abs {err:.3e} > {tol}"


def test_tiny_workload_full_parity():
    """B1 H1 L128 d64 fp32 p=3, the small case of the five workloads."""
    inp = gen.make_inputs("tiny")
    got = _gpu_out(inp)
    want = oracle.lssar_fwd(inp.q, inp.k, inp.v, inp.wl.p)
    err = float(np.max(np.abs(got - want)))
    print(f"tiny: max-abs {err:.3e}", flush=True)
    assert err <= F32_TOL


_FULL = {}


def _full(name):
    if name not in _FULL:
        _FULL.clear()
        inp = gen.make_inputs(name)
        _FULL[name] = inp
    return _FULL[name]


def _sample_rows(wl, meta, rng):
    """(b, h, rows) triples: the first five and last rows of every head, a
    random spread, and the planted query row where there is one."""
    out = []
    planted = {(b, h): r for b, h, r, _ in meta.get("planted", [])}
    heads = [(b, h) for b in range(wl.B) for h in range(wl.H)]
    if len(heads) > 16:
        idx = rng.choice(len(heads), size=16, replace=False)
        heads = [heads[i] for i in sorted(idx)]
    for b, h in heads:
        rows = {0, 1, 2, 3, 4, wl.L - 1, wl.L - 2}
        rows.update(int(x) for x in rng.integers(0, wl.L, size=12))
        if (b, h) in planted:
            rows.add(planted[(b, h)])
        out.append((b, h, sorted(rows)))
    return out


def _worst_row(got, want):
    """Largest per-row max-abs error and the (..., row) index where it is."""
    err = np.max(np.abs(got - want), axis=-1)
    idx = np.unravel_index(int(np.argmax(err)), err.shape)
    return float(err[idx]), tuple(int(x) for x in idx)


@pytest.mark.parametrize("name", ["gpt2s", "x8_planted"])
def test_full_workload_every_row(name):
    """Every row of the workload against the oracle's full forward."""
    inp = _full(name)
    wl = inp.wl
    print(f"{name}: B{wl.B} H{wl.H} L{wl.L} d{wl.d} p{wl.p}, every row", flush=True)
    got = _gpu_out(inp)
    want = oracle.lssar_fwd(inp.q, inp.k, inp.v, wl.p)
    err, (b, h, r) = _worst_row(got, want)
    print(f"{name}: all {wl.B * wl.H * wl.L} rows, max-abs {err:.3e} at b={b} h={h} row={r + 1}",
          flush=True)
    assert err <= BF16_TOL, f"{name}: max-abs {err:.3e} at b={b} h={h} row={r + 1}"
    assert np.array_equal(got[:, :, 0], inp.v[:, :, 0].astype(np.float64))


@pytest.mark.parametrize("name,heads", [
    ("x16", [(0, 0), (0, 11)]),
    ("wide", [(0, 0), (0, 9), (0, 17), (0, 31), (1, 2), (1, 15), (1, 24), (1, 31)])])
def test_full_workload_whole_heads(name, heads):
    """Whole heads of the larger workloads against the oracle's forward."""
    inp = _full(name)
    wl = inp.wl
    print(f"{name}: B{wl.B} H{wl.H} L{wl.L} d{wl.d} p{wl.p}, heads {heads}", flush=True)
    got = _gpu_out(inp)
    worst = (0.0, None)
    for b, h in heads:
        want = oracle.lssar_fwd(inp.q[b, h], inp.k[b, h], inp.v[b, h], wl.p)
        err, (r,) = _worst_row(got[b, h], want)
        print(f"{name} b={b} h={h}: {wl.L} rows, max-abs {err:.3e} at row {r + 1}", flush=True)
        assert err <= BF16_TOL, f"{name} b={b} h={h}: max-abs {err:.3e} at row {r + 1}"
        worst = max(worst, (err, (b, h, r + 1)), key=lambda x: x[0])
    print(f"{name}: whole heads max-abs {worst[0]:.3e} at (b, h, row) {worst[1]}", flush=True)


@pytest.mark.parametrize("name", ["x16", "wide"])
def test_full_workload_sampled_parity(name):
    inp = _full(name)
    wl = inp.wl
    print(f"{name}: B{wl.B} H{wl.H} L{wl.L} d{wl.d} p{wl.p}", flush=True)
    got = _gpu_out(inp)
    rng = np.random.default_rng(7)
    worst = 0.0
    for b, h, rows in _sample_rows(wl, inp.meta, rng):
        want = oracle.lssar_rows(inp.q[b, h], inp.k[b, h], inp.v[b, h], rows, wl.p)
        err = float(np.max(np.abs(got[b, h, rows] - want)))
        worst = max(worst, err)
        assert err <= BF16_TOL, f"{name} b={b} h={h}: max-abs {err:.3e}"
    # row 1 reproduces v_1 exactly (ln 1 = 0, o_1 = 0) in every head
    assert np.array_equal(got[:, :, 0], inp.v[:, :, 0].astype(np.float64))
    assert np.all(np.isfinite(got))
    print(f"{name}: sampled max-abs {worst:.3e}", flush=True)


@pytest.mark.parametrize("name", ["gpt2s", "x16"])
def test_full_workload_v_ones(name):
    """V = ones: every row is a convex combination, so out == 1 exactly after
    bf16 rounding (the weight sum rides the same contraction as P.V)."""
    inp = _full(name)
    wl = inp.wl
    q, k = to_device(inp.q, wl.dtype), to_device(inp.k, wl.dtype)
    v = torch.ones_like(q)
    out = to_host(run_ws(q, k, v, wl.p))
    assert np.all(out == 1.0)


def test_v_identity_probe():
    """V = I turns the output into the weight matrix: non-negative, exactly 0
    above the diagonal, rows summing to 1 (bf16 weights)."""
    for dtype, tol in (("bf16", 2e-2), ("f32", 1e-6)):
        inp = gen.make_inputs("gpt2s", B=1, H=3, L=64, d=64, dtype=dtype, p=3, seed=11)
        q, k = to_device(inp.q, dtype), to_device(inp.k, dtype)
        v = to_device(np.broadcast_to(np.eye(64, dtype=np.float32), (1, 3, 64, 64)).copy(), dtype)
        W = to_host(run_ws(q, k, v, 3))
        assert np.all(W >= 0.0)
        iu = np.triu_indices(64, 1)
        assert np.all(W[:, :, iu[0], iu[1]] == 0.0)
        assert np.max(np.abs(W.sum(axis=-1) - 1.0)) <= tol


def test_degenerate_rows():
    """Zero query rows: all scores equal.  Rows >= 4 give 0, rows 1-3 the
    mean of v_1..v_i (oracle and convention agree)."""
    for dtype in ("f32", "bf16"):
        inp = gen.make_inputs("gpt2s", B=1, H=2, L=200, d=64, dtype=dtype, p=15, seed=3)
        q = inp.q.copy()
        zero_rows = [0, 1, 2, 3, 4, 50, 127, 128, 199]
        q[:, :, zero_rows] = 0.0
        inp2 = gen.Inputs(inp.wl, q, inp.k, inp.v)
        got = _gpu_out(inp2)
        want = oracle.lssar_fwd(q, inp.k, inp.v, 15)
        assert np.max(np.abs(got - want)) <= tol_for(dtype)
        assert np.all(got[:, :, [3, 4, 50, 127, 128, 199]] == 0.0)
    # every key identical: rows >= 4 degenerate for any query
    inp = gen.make_inputs("gpt2s", B=1, H=1, L=130, d=128, dtype="bf16", p=3, seed=5)
    k = np.broadcast_to(inp.k[:, :, :1], inp.k.shape).copy()
    got = _gpu_out(gen.Inputs(inp.wl, inp.q, k, inp.v))
    assert np.all(got[:, :, 3:] == 0.0)


def test_bitwise_determinism_and_entry_points_agree():
    import softmax_free_attention_amd as sfa
    inp = gen.make_inputs("x8_planted", H=4, L=1500)
    q, k, v = (to_device(a, "bf16") for a in (inp.q, inp.k, inp.v))
    a = run_ws(q, k, v, 15)
    b = run_ws(q, k, v, 15)
    c = sfa.lssar_attn_fwd(q, k, v, p=15)
    ws = sfa.workspace_for(q)
    sfa.lssar_prep(k, ws)
    d = torch.empty_like(q)
    sfa.lssar_attn_fwd_prepped(q, k, v, ws, d, p=15)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        e = run_ws(q, k, v, 15, stream=s)
    s.synchronize()
    torch.cuda.synchronize()
    for t in (b, c, d, e):
        assert torch.equal(a.view(torch.int16), t.view(torch.int16))


def test_prep_workspace_contents():
    """The prep step writes 1/max(|k_j|, 1e-12) per key row (fp64 for fp32
    inputs, fp32 for bf16) and, for bf16: the normalised keys rounded to
    f16 and the attention kernel's dispatch table."""
    import softmax_free_attention_amd as sfa
    for dtype, d in (("bf16", 64), ("bf16", 128), ("f32", 64), ("f32", 128)):
        L = 77
        inp = gen.make_inputs("gpt2s", B=2, H=3, L=L, d=d, dtype=dtype, seed=9)
        k = inp.k.copy()
        k[0, 0, 5] = 0.0
        kt = to_device(k, dtype)
        ws = sfa.workspace_for(kt)
        sfa.lssar_prep(kt, ws)
        torch.cuda.synchronize()
        raw = ws.cpu().numpy()
        nrow = 2 * 3 * L
        fdt = np.float32 if dtype == "bf16" else np.float64
        fk = raw[:fdt().itemsize * nrow].view(fdt).reshape(2, 3, L)
        want = 1.0 / np.maximum(np.linalg.norm(k.astype(np.float64), axis=-1), 1e-12)
        if dtype == "f32":
            assert np.max(np.abs(fk / want - 1.0)) < 1e-14
        if dtype == "bf16":
            # one rounding of the fp64 factor to fp32
            assert np.max(np.abs(fk / want - 1.0)) <= 2.0 ** -24
            # KN16: k_j / max(|k_j|, 1e-12) rounded to f16 (within half an
            # f16 ulp of the fp64 value, plus the fp32 product's 2^-23
            # relative; zero rows stay zero)
            knoff = (4 * nrow + 255) // 256 * 256
            kn16 = raw[knoff:knoff + 2 * 3 * L * d * 2].view(np.float16).reshape(2, 3, L, d)
            kh = k.astype(np.float64) * want[..., None]
            half_ulp = np.ldexp(1.0, np.maximum(np.frexp(np.abs(kh))[1] - 12, -25))
            assert np.all(np.abs(kn16.astype(np.float64) - kh) <= half_ulp + np.abs(kh) * 2.0 ** -22)
            assert not np.any(kn16[0, 0, 5])
            # the attention kernel's dispatch table: (head, block) per
            # workgroup, as the host-side schedule query gives it
            items = sfa.lssar_fwd_schedule(2, 3, L)
            soff = knoff + (2 * 3 * L * d * 2 + 255) // 256 * 256
            tab = raw[soff:soff + 8 * len(items)].view(np.int32).reshape(-1, 2)
            nqb = (L + 63) // 64
            want_tab = np.array([[x // nqb, x % nqb] if x >= 0 else [-1, -1] for x in items])
            assert np.array_equal(tab, want_tab)
    for B, H, L in ((1, 12, 8192), (2, 32, 4096), (1, 5, 3000)):
        k = torch.zeros((B, H, L, 64), dtype=torch.bfloat16, device="cuda")
        ws = sfa.workspace_for(k)
        sfa.lssar_prep(k, ws)
        torch.cuda.synchronize()
        raw = ws.cpu().numpy()
        off = (4 * B * H * L + 255) // 256 * 256 + (B * H * L * 64 * 2 + 255) // 256 * 256
        items = sfa.lssar_fwd_schedule(B, H, L)
        tab = raw[off:off + 8 * len(items)].view(np.int32).reshape(-1, 2)
        nqb = (L + 63) // 64
        want_tab = np.array([[x // nqb, x % nqb] if x >= 0 else [-1, -1] for x in items])
        assert np.array_equal(tab, want_tab), (B, H, L)


def test_causality_and_scale_invariance():
    """Future keys/values never reach a row (bitwise), also when they make
    other rows of the row's 64-row block ask for the exact redo (a redone
    block stores only the rows that asked); scaling Q and K rows by powers
    of two changes nothing (bitwise: every factor is exact)."""
    inp = gen.make_inputs("gpt2s", B=1, H=2, L=400, d=64, p=15, seed=21)
    q, k, v = (to_device(a, "bf16") for a in (inp.q, inp.k, inp.v))
    base = run_ws(q, k, v, 15)
    g = torch.Generator(device="cuda").manual_seed(123)
    for trial in range(4):
        for cut in (0, 3, 63, 64, 65, 127, 200):
            k2, v2 = k.clone(), v.clone()
            n = k2[:, :, cut + 1:].shape
            k2[:, :, cut + 1:] = torch.randn(n, generator=g, device="cuda").to(k.dtype)
            v2[:, :, cut + 1:] = (torch.randn(n, generator=g, device="cuda") * 100).to(v.dtype)
            if trial == 3:
                # future keys that make every later row of the block nearly tied
                k2[:, :, cut + 1:] = k2[:, :, cut:cut + 1]
            o2 = run_ws(q, k2, v2, 15)
            same = torch.equal(o2[:, :, :cut + 1].view(torch.int16),
                               base[:, :, :cut + 1].view(torch.int16))
            assert same, (trial, cut)
    o3 = run_ws(q * 4.0, k * 0.25, v, 15)
    assert torch.equal(o3.view(torch.int16), base.view(torch.int16))


@pytest.mark.parametrize("d", [64, 128])
def test_row_scaling_over_a_wide_range(d):
    """Every factor of the scores is scale-free: scaling each row of Q and K
    by its own power of two in [2^-30, 2^30] changes neither the output of
    the plain forward (normalised f16 operands, and the exact operands of
    redone blocks) nor that of the training forward and its statistics,
    bitwise.  (Rows stay above the 1e-12 norm clamp and their squares in
    range.)"""
    import softmax_free_attention_amd as sfa
    inp = gen.make_inputs("x8_planted", B=1, H=2, L=700, d=d, p=15, seed=41)
    q, k, v = (to_device(a, "bf16") for a in (inp.q, inp.k, inp.v))
    r = np.random.default_rng(43)
    sq = torch.from_numpy(np.ldexp(1.0, r.integers(-30, 31, size=(1, 2, 700, 1)))).cuda()
    sk = torch.from_numpy(np.ldexp(1.0, r.integers(-30, 31, size=(1, 2, 700, 1)))).cuda()
    q2 = (q.double() * sq).to(torch.bfloat16)
    k2 = (k.double() * sk).to(torch.bfloat16)
    # the scaled rows are exact
    assert torch.equal((q2.double() / sq).to(torch.bfloat16).view(torch.int16), q.view(torch.int16))
    assert torch.equal((k2.double() / sk).to(torch.bfloat16).view(torch.int16), k.view(torch.int16))
    base, got = run_ws(q, k, v, 15), run_ws(q2, k2, v, 15)
    torch.cuda.synchronize()
    assert torch.equal(base.view(torch.int16), got.view(torch.int16))
    outs = []
    for a, b in ((q, k), (q2, k2)):
        out, st = torch.empty_like(a), sfa.stats_for(a)
        sfa.lssar_attn_fwd_stats_ws(a, b, v, out, st, sfa.workspace_for(a), p=15)
        outs.append((out, st))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0].view(torch.int16), outs[1][0].view(torch.int16))
    assert torch.equal(outs[0][1], outs[1][1])


def test_linearity_in_v():
    inp = gen.make_inputs("gpt2s", B=1, H=2, L=300, d=128, dtype="f32", p=3, seed=31)
    q, k, v = (to_device(a, "f32") for a in (inp.q, inp.k, inp.v))
    v2 = torch.randn(v.shape, generator=torch.Generator(device="cuda").manual_seed(32), device="cuda")
    a, b, c = run_ws(q, k, v, 3), run_ws(q, k, v2, 3), run_ws(q, k, 2 * v - 3 * v2, 3)
    assert float((c - (2 * a - 3 * b)).abs().max()) < 1e-4


def test_binding_rejects_bad_input():
    import softmax_free_attention_amd as sfa
    q = torch.zeros(1, 1, 8, 96, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(sfa.LssarError) as e:
        sfa.lssar_attn_fwd(q, q.clone(), q.clone(), p=3)
    assert e.value.status == sfa.LSSAR_EUNSUPPORTED
    q = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(sfa.LssarError) as e:
        sfa.lssar_attn_fwd(q, q.clone(), q.clone(), p=0)
    assert e.value.status == sfa.LSSAR_EINVAL
    with pytest.raises(TypeError):
        sfa.lssar_attn_fwd(q.half(), q.half(), q.half(), p=3)
