"""The C ABI library on the CPU: it loads, exports every declared symbol, and
rejects invalid arguments on the host before any HIP call (no GPU needed)."""
import ctypes
import os
import re
import subprocess

import pytest

import softmax_free_attention_amd as sfa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lssar.h")

# Fake device addresses: validation never dereferences them.
A = 0x7F0000000000
STEP = 1 << 30


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lssar_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(sfa.lib_path):
        from softmax_free_attention_amd import build
        build.build()
    return sfa.lib()


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("lssar_attn_fwd", "lssar_attn_fwd_ws", "lssar_workspace_bytes",
              "lssar_status_str", "lssar_prep", "lssar_attn_fwd_prepped",
              "lssar_attn_fwd_phi_ws", "lssar_lssa_fwd_ws", "lssar_decode_ws",
              "lssar_decode_workspace_bytes", "lssar_attn_bwd_ws", "lssar_bwd_workspace_bytes",
              "lssar_attn_fwd_stats_ws", "lssar_attn_bwd_stats_ws"):
        assert n in names


def test_library_exports_every_declared_symbol(L):
    raw = ctypes.CDLL(sfa.lib_path)
    for n in declared_functions():
        assert hasattr(raw, n), f"{n} declared in include/lssar.h but not exported"
    out = subprocess.run(["nm", "-D", "--defined-only", sfa.lib_path], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (lssar_[a-z0-9_]+)$", out, flags=re.M))
    assert exported == set(declared_functions()), "exported lssar_* symbols differ from the header"


def test_library_has_no_oracle_dependency(L):
    out = subprocess.run(["readelf", "-d", sfa.lib_path], capture_output=True, text=True,
                         check=True).stdout
    assert "lssar_ref" not in out
    assert "libamdhip64" in out
    for dirpath, _, files in os.walk(os.path.join(ROOT, "softmax_free_attention_amd")):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".h", ".cpp")):
                src = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(import|from)\s+oracle\b", src, flags=re.M), f
                assert "lssar_ref" not in src, f


def test_noalloc_host_checks(L):
    """lssar_attn_fwd_noalloc validates on the host before any HIP call: bad
    arguments, and an input whose workspace exceeds the 64 MiB scratch."""
    assert sfa.lssar_noalloc_scratch_bytes() == 64 << 20
    f = L.lssar_attn_fwd_noalloc
    q, k, v, o = A, A + STEP, A + 2 * STEP, A + 3 * STEP
    assert f(0, k, v, o, 1, 2, 64, 64, 3, 1e-4, 1, None) == sfa.LSSAR_EINVAL
    assert f(q, k, v, o, 1, 2, 64, 96, 3, 1e-4, 1, None) == sfa.LSSAR_EUNSUPPORTED
    assert f(q, k, v, o, 1, 2, 64, 64, 0, 1e-4, 1, None) == sfa.LSSAR_EINVAL
    assert f(q, k, v, o, 1, 32, 8192, 128, 3, 1e-4, 1, None) == sfa.LSSAR_ESCRATCH
    assert f(q, k, v, o, 2, 32, 4096, 128, 15, 1e-4, 1, None) == sfa.LSSAR_ESCRATCH


def test_version_and_status_strings(L):
    assert sfa.lssar_version() == 910
    assert sfa.lssar_status_str(0) == "ok"
    for st in (-1, -2, -3, -4, -5, 7):
        s = sfa.lssar_status_str(st)
        assert isinstance(s, str) and s
    assert sfa.lssar_last_hip_error() == 0


def test_workspace_bytes(L):
    # fp32: one fp64 factor per key row, rounded up to 256 bytes
    assert sfa.lssar_workspace_bytes(1, 1, 1, 64, sfa.LSSAR_F32) == 256
    assert sfa.lssar_workspace_bytes(2, 3, 5, 128, sfa.LSSAR_F32) == 256
    assert sfa.lssar_workspace_bytes(1, 1, 100, 64, sfa.LSSAR_F32) == 1024
    assert sfa.lssar_workspace_bytes(1, 1, 32, 64, sfa.LSSAR_F32) == 256
    # bf16: one fp32 factor per key row, the normalised rows of K in f16
    # and the attention kernel's dispatch table (8 bytes per workgroup),
    # each rounded up
    def r256(x):
        return (x + 255) // 256 * 256
    assert sfa.lssar_workspace_bytes(1, 12, 8192, 64, sfa.LSSAR_BF16) == \
        4 * 12 * 8192 + 12 * 64 * 8192 * 2 + r256(8 * 1536)
    assert sfa.lssar_workspace_bytes(2, 3, 77, 128, sfa.LSSAR_BF16) == \
        2048 + r256(6 * 77 * 128 * 2) + \
        r256(8 * len(sfa.lssar_fwd_schedule(2, 3, 77)))
    # the no-alloc scratch holds B1 H12 L32768 at d = 64
    assert sfa.lssar_workspace_bytes(1, 12, 32768, 64, sfa.LSSAR_BF16) <= 64 << 20
    assert sfa.lssar_workspace_bytes(0, 1, 1, 64, 0) == 0
    assert sfa.lssar_workspace_bytes(1, 1, 1, 96, 0) == 0
    assert sfa.lssar_workspace_bytes(1, 1, 1, 64, 5) == 0
    assert sfa.lssar_workspace_bytes(1, 1, (1 << 22) + 1, 64, 1) == 0


def _fwd_ws(L, q=A, k=A + STEP, v=A + 2 * STEP, o=A + 3 * STEP, B=1, H=2, Ln=64, d=64, p=3,
            eps=1e-4, dt=1, ws=A + 4 * STEP, wsb=1 << 20):
    return L.lssar_attn_fwd_ws(q, k, v, o, B, H, Ln, d, p, eps, dt, ws, wsb, None)


@pytest.mark.parametrize("kw,want", [
    (dict(q=0), sfa.LSSAR_EINVAL),
    (dict(k=0), sfa.LSSAR_EINVAL),
    (dict(v=0), sfa.LSSAR_EINVAL),
    (dict(o=0), sfa.LSSAR_EINVAL),
    (dict(B=0), sfa.LSSAR_EINVAL),
    (dict(H=-1), sfa.LSSAR_EINVAL),
    (dict(Ln=0), sfa.LSSAR_EINVAL),
    (dict(p=0), sfa.LSSAR_EINVAL),
    (dict(eps=-1.0), sfa.LSSAR_EINVAL),
    (dict(eps=float("nan")), sfa.LSSAR_EINVAL),
    (dict(eps=float("inf")), sfa.LSSAR_EINVAL),
    (dict(d=96), sfa.LSSAR_EUNSUPPORTED),
    (dict(d=32), sfa.LSSAR_EUNSUPPORTED),
    (dict(dt=2), sfa.LSSAR_EUNSUPPORTED),
    (dict(p=1025), sfa.LSSAR_EUNSUPPORTED),
    (dict(Ln=(1 << 22) + 1), sfa.LSSAR_EUNSUPPORTED),
    (dict(q=A + 8), sfa.LSSAR_EINVAL),                        # misaligned
    (dict(o=A + 64), sfa.LSSAR_EINVAL),                       # out overlaps q
    (dict(o=A + STEP + 2 * 64 * 64), sfa.LSSAR_EINVAL),       # out overlaps k
    (dict(B=1 << 16, H=1 << 16), sfa.LSSAR_EINVAL),           # B*H overflows
    (dict(ws=0), sfa.LSSAR_EWORKSPACE),
    (dict(ws=A + 4 * STEP + 16), sfa.LSSAR_EWORKSPACE),       # not 256-aligned
    (dict(wsb=100), sfa.LSSAR_EWORKSPACE),                    # too small
    (dict(ws=A + 3 * STEP - 256), sfa.LSSAR_EWORKSPACE),      # overlaps out
    (dict(ws=A + STEP + 256), sfa.LSSAR_EWORKSPACE),          # overlaps k
])
def test_validation_before_any_hip_call(L, kw, want):
    assert _fwd_ws(L, **kw) == want
    assert sfa.lssar_last_hip_error() == 0


def test_allocating_entry_validates(L):
    assert L.lssar_attn_fwd(0, A, A + STEP, A + 2 * STEP, 1, 1, 8, 64, 3, 1e-4, 1, None) == -1
    assert L.lssar_attn_fwd(A, A + STEP, A + 2 * STEP, A + 3 * STEP, 1, 1, 8, 80, 3, 1e-4, 1,
                            None) == -2


def test_stage_entries_validate(L):
    k, v, ws = A, A + STEP, A + 4 * STEP
    # prep (K only): null or misaligned k, bad d, bad workspace (null,
    # misaligned, small, overlapping k)
    assert L.lssar_prep(0, ws, 1 << 20, 1, 1, 8, 64, 1, None) == sfa.LSSAR_EINVAL
    assert L.lssar_prep(k + 8, ws, 1 << 20, 1, 1, 8, 64, 1, None) == sfa.LSSAR_EINVAL
    assert L.lssar_prep(k, ws, 1 << 20, 1, 1, 8, 72, 1, None) == sfa.LSSAR_EUNSUPPORTED
    assert L.lssar_prep(k, 0, 1 << 20, 1, 1, 8, 64, 1, None) == sfa.LSSAR_EWORKSPACE
    assert L.lssar_prep(k, ws + 16, 1 << 20, 1, 1, 8, 64, 1, None) == sfa.LSSAR_EWORKSPACE
    assert L.lssar_prep(k, ws, 64, 1, 1, 8, 64, 1, None) == sfa.LSSAR_EWORKSPACE
    assert L.lssar_prep(k, k - 256, 1 << 20, 1, 1, 8, 64, 1, None) == sfa.LSSAR_EWORKSPACE
    # prepped: the fused-call checks plus the workspace
    q, o = A + 2 * STEP, A + 3 * STEP
    assert L.lssar_attn_fwd_prepped(q, k, v, 0, 1 << 20, o, 1, 1, 8, 64, 3, 1e-4, 1,
                                    None) == sfa.LSSAR_EWORKSPACE
    assert L.lssar_attn_fwd_prepped(q, k, v, ws, 1 << 20, o, 1, 1, 8, 64, 0, 1e-4, 1,
                                    None) == sfa.LSSAR_EINVAL
    assert L.lssar_attn_fwd_prepped(q, k, v, o, 1 << 20, o, 1, 1, 8, 64, 3, 1e-4, 1,
                                    None) == sfa.LSSAR_EWORKSPACE
    assert sfa.lssar_last_hip_error() == 0


def test_variant_entries_validate(L):
    q, k, v, o, ws = A, A + STEP, A + 2 * STEP, A + 3 * STEP, A + 4 * STEP
    phi = L.lssar_attn_fwd_phi_ws
    assert phi(q, k, v, o, 1, 2, 64, 64, 3, 1e-4, 2, 1, ws, 1 << 20, None) == sfa.LSSAR_EUNSUPPORTED
    assert phi(q, k, v, o, 1, 2, 64, 64, 3, 1e-4, -1, 1, ws, 1 << 20, None) == sfa.LSSAR_EUNSUPPORTED
    assert phi(0, k, v, o, 1, 2, 64, 64, 3, 1e-4, 1, 1, ws, 1 << 20, None) == sfa.LSSAR_EINVAL
    assert phi(q, k, v, o, 1, 2, 64, 64, 0, 1e-4, 1, 1, ws, 1 << 20, None) == sfa.LSSAR_EINVAL
    assert phi(q, k, v, o, 1, 2, 64, 96, 3, 1e-4, 1, 1, ws, 1 << 20, None) == sfa.LSSAR_EUNSUPPORTED
    assert phi(q, k, v, o, 1, 2, 64, 64, 3, 1e-4, 1, 1, ws, 64, None) == sfa.LSSAR_EWORKSPACE
    lssa = L.lssar_lssa_fwd_ws
    assert lssa(q, k, v, 0, 1, 2, 64, 64, 1, ws, 1 << 20, None) == sfa.LSSAR_EINVAL
    assert lssa(q, k, v, o, 1, 2, 0, 64, 1, ws, 1 << 20, None) == sfa.LSSAR_EINVAL
    assert lssa(q, k, v, o, 1, 2, 64, 80, 1, ws, 1 << 20, None) == sfa.LSSAR_EUNSUPPORTED
    assert lssa(q, k, v, o, 1, 2, 64, 64, 3, ws, 1 << 20, None) == sfa.LSSAR_EUNSUPPORTED
    assert lssa(q, k, v, o, 1, 2, 64, 64, 1, 0, 1 << 20, None) == sfa.LSSAR_EWORKSPACE
    assert lssa(q, k, v, o, 1, 2, 64, 64, 1, o + 256, 1 << 20, None) == sfa.LSSAR_EWORKSPACE
    assert sfa.lssar_last_hip_error() == 0


def test_decode_workspace_bytes(L):
    # bf16: fp32 scores per cache row, 2 + (d + 1) fp32 partials per chunk of
    # 16384 / d rows
    r = lambda x: (x + 255) // 256 * 256
    assert sfa.lssar_decode_workspace_bytes(16, 12, 8192, 64, sfa.LSSAR_BF16) == \
        r(4 * 192 * 8192) + r(4 * 192 * 32 * 2) + r(4 * 192 * 32 * 65)
    assert sfa.lssar_decode_workspace_bytes(3, 2, 300, 128, sfa.LSSAR_F32) == \
        r(8 * 6 * 300) + r(8 * 6 * 3 * 2) + r(8 * 6 * 3 * 129)
    assert sfa.lssar_decode_workspace_bytes(1, 1, 1, 64, sfa.LSSAR_BF16) == 256 + 256 + 512
    assert sfa.lssar_decode_workspace_bytes(1, 1, 1, 96, sfa.LSSAR_BF16) == 0
    assert sfa.lssar_decode_workspace_bytes(0, 1, 1, 64, sfa.LSSAR_BF16) == 0


def test_decode_validates_before_any_hip_call(L):
    q, k, v, o, ws, ln = A, A + STEP, A + 2 * STEP, A + 3 * STEP, A + 4 * STEP, A + 5 * STEP
    dec = L.lssar_decode_ws
    big = 1 << 30

    def call(q=q, k=k, v=v, ln=ln, o=o, B=2, H=2, Lm=100, d=64, p=3, eps=1e-4, dt=1, ws=ws,
             wsb=big):
        return dec(q, k, v, ln, o, B, H, Lm, d, p, eps, dt, ws, wsb, None)

    assert call(q=0) == sfa.LSSAR_EINVAL
    assert call(k=0) == sfa.LSSAR_EINVAL
    assert call(o=0) == sfa.LSSAR_EINVAL
    assert call(p=0) == sfa.LSSAR_EINVAL
    assert call(eps=float("nan")) == sfa.LSSAR_EINVAL
    assert call(Lm=0) == sfa.LSSAR_EINVAL
    assert call(d=80) == sfa.LSSAR_EUNSUPPORTED
    assert call(dt=3) == sfa.LSSAR_EUNSUPPORTED
    assert call(p=2000) == sfa.LSSAR_EUNSUPPORTED
    assert call(q=q + 8) == sfa.LSSAR_EINVAL                    # misaligned
    assert call(ln=ln + 2) == sfa.LSSAR_EINVAL                  # lens misaligned
    assert call(o=q + 64) == sfa.LSSAR_EINVAL                   # out overlaps q
    assert call(o=k + 4096) == sfa.LSSAR_EINVAL                 # out inside the cache
    assert call(o=ln - 64) == sfa.LSSAR_EINVAL                  # out overlaps lens
    assert call(ws=0) == sfa.LSSAR_EWORKSPACE
    assert call(ws=ws + 128) == sfa.LSSAR_EWORKSPACE
    assert call(wsb=100) == sfa.LSSAR_EWORKSPACE
    assert call(ws=v + 256) == sfa.LSSAR_EWORKSPACE             # overlaps the V cache
    assert call(ws=ln - 256) == sfa.LSSAR_EWORKSPACE            # overlaps lens
    assert sfa.lssar_last_hip_error() == 0


def test_bwd_workspace_bytes(L):
    r = lambda x: (x + 255) // 256 * 256
    # bf16: fp32 factors and coefficients
    assert sfa.lssar_bwd_workspace_bytes(1, 12, 8192, 64, sfa.LSSAR_BF16) == \
        2 * r(4 * 12 * 8192) + r(4 * 8 * 12 * 8192)
    assert sfa.lssar_bwd_workspace_bytes(1, 1, 70, 128, sfa.LSSAR_BF16) == \
        2 * r(4 * 70) + r(32 * 70)
    assert sfa.lssar_bwd_workspace_bytes(2, 3, 5, 128, sfa.LSSAR_F32) == 2 * r(8 * 30) + r(64 * 30)
    assert sfa.lssar_bwd_workspace_bytes(1, 1, 1, 80, sfa.LSSAR_F32) == 0


def test_bwd_validates_before_any_hip_call(L):
    S = STEP
    base = dict(q=A, k=A + S, v=A + 2 * S, g=A + 3 * S, dq=A + 4 * S, dk=A + 5 * S, dv=A + 6 * S,
                B=1, H=2, Ln=64, d=64, p=3, eps=1e-4, dt=1, ws=A + 7 * S, wsb=1 << 24)

    def call(**kw):
        a = dict(base, **kw)
        return L.lssar_attn_bwd_ws(a["q"], a["k"], a["v"], a["g"], a["dq"], a["dk"], a["dv"],
                                   a["B"], a["H"], a["Ln"], a["d"], a["p"], a["eps"], a["dt"],
                                   a["ws"], a["wsb"], None)

    assert call(g=0) == sfa.LSSAR_EINVAL
    assert call(dv=0) == sfa.LSSAR_EINVAL
    assert call(q=0) == sfa.LSSAR_EINVAL
    assert call(p=0) == sfa.LSSAR_EINVAL
    assert call(d=96) == sfa.LSSAR_EUNSUPPORTED
    assert call(dk=A + 5 * S + 8) == sfa.LSSAR_EINVAL           # misaligned
    assert call(dq=A + 3 * S + 64) == sfa.LSSAR_EINVAL          # dq overlaps dout
    assert call(dv=A + 4 * S + 64) == sfa.LSSAR_EINVAL          # dv overlaps dq
    assert call(dk=A + 64) == sfa.LSSAR_EINVAL                  # dk overlaps q
    assert call(ws=0) == sfa.LSSAR_EWORKSPACE
    assert call(wsb=1000) == sfa.LSSAR_EWORKSPACE
    assert call(ws=A + 6 * S + 256) == sfa.LSSAR_EWORKSPACE     # overlaps dv
    assert sfa.lssar_last_hip_error() == 0


def test_stats_entries_validate_before_any_hip_call(L):
    """The training forward and the backward with saved statistics check the
    statistics buffer (null, misaligned, overlapping) on the host first."""
    S = STEP
    st0 = A + 9 * S
    fbase = dict(q=A, k=A + S, v=A + 2 * S, out=A + 3 * S, st=st0, B=1, H=2, Ln=64, d=64, p=3,
                 eps=1e-4, dt=1, ws=A + 7 * S, wsb=1 << 24)

    def fwd(**kw):
        a = dict(fbase, **kw)
        return L.lssar_attn_fwd_stats_ws(a["q"], a["k"], a["v"], a["out"], a["st"], a["B"],
                                         a["H"], a["Ln"], a["d"], a["p"], a["eps"], a["dt"],
                                         a["ws"], a["wsb"], None)

    assert fwd(st=0) == sfa.LSSAR_EINVAL
    assert fwd(st=st0 + 8) == sfa.LSSAR_EINVAL                  # misaligned
    assert fwd(st=A + 3 * S + 128) == sfa.LSSAR_EINVAL          # overlaps out
    assert fwd(st=A + 7 * S + 256) == sfa.LSSAR_EINVAL          # overlaps the workspace
    assert fwd(d=96) == sfa.LSSAR_EUNSUPPORTED
    assert fwd(out=0) == sfa.LSSAR_EINVAL
    assert fwd(wsb=1000) == sfa.LSSAR_EWORKSPACE

    bbase = dict(q=A, k=A + S, v=A + 2 * S, o=A + 8 * S, g=A + 3 * S, st=st0, dq=A + 4 * S,
                 dk=A + 5 * S, dv=A + 6 * S, B=1, H=2, Ln=64, d=64, p=3, eps=1e-4, dt=1,
                 ws=A + 7 * S, wsb=1 << 24)

    def bwd(**kw):
        a = dict(bbase, **kw)
        return L.lssar_attn_bwd_stats_ws(a["q"], a["k"], a["v"], a["o"], a["g"], a["st"],
                                         a["dq"], a["dk"], a["dv"], a["B"], a["H"], a["Ln"],
                                         a["d"], a["p"], a["eps"], a["dt"], a["ws"], a["wsb"],
                                         None)

    assert bwd(o=0) == sfa.LSSAR_EINVAL
    assert bwd(o=A + 8 * S + 8) == sfa.LSSAR_EINVAL              # misaligned
    assert bwd(o=A + 4 * S + 64) == sfa.LSSAR_EINVAL             # overlaps dq
    assert bwd(o=A + 7 * S + 256) == sfa.LSSAR_EINVAL            # overlaps the workspace
    assert bwd(st=0) == sfa.LSSAR_EINVAL
    assert bwd(st=st0 + 8) == sfa.LSSAR_EINVAL
    assert bwd(st=A + 5 * S + 64) == sfa.LSSAR_EINVAL           # overlaps dk
    assert bwd(st=A + 7 * S) == sfa.LSSAR_EINVAL                # overlaps the workspace
    assert bwd(g=0) == sfa.LSSAR_EINVAL
    assert bwd(p=0) == sfa.LSSAR_EINVAL
    assert bwd(ws=0) == sfa.LSSAR_EWORKSPACE
    assert sfa.lssar_last_hip_error() == 0


@pytest.mark.parametrize("B,H,Lq", [(1, 12, 8192), (8, 12, 1024), (2, 32, 4096), (1, 12, 16384),
                                   (1, 1, 1), (1, 1, 100), (3, 5, 1000), (1, 7, 2113),
                                   (16, 1, 65), (1, 200, 64)])
def test_forward_schedule(L, B, H, Lq):
    """The bf16 forward's dispatch order (host query of the kernels' own
    schedule code): every query block exactly once; workgroup w on XCD w % 8;
    each XCD runs its blocks largest first; the XCDs' work (key tiles) is
    equal up to one pair of blocks; each XCD touches about B H / 8 heads."""
    nqb = (Lq + 63) // 64
    items = sfa.lssar_fwd_schedule(B, H, Lq)
    real = [x for x in items if x >= 0]
    assert sorted(real) == list(range(B * H * nqb))
    assert len(items) % 8 == 0
    work = [0] * 8
    heads = [set() for _ in range(8)]
    for x in range(8):
        sizes = [items[w] % nqb + 1 for w in range(x, len(items), 8) if items[w] >= 0]
        assert sizes == sorted(sizes, reverse=True)
        # empty indices only after an XCD's last block
        tail = [items[w] for w in range(x, len(items), 8)]
        assert all(t < 0 for t in tail[len(sizes):])
        work[x] = sum(sizes)
        heads[x] = {items[w] // nqb for w in range(x, len(items), 8) if items[w] >= 0}
    assert max(work) - min(work) <= nqb + 1
    bh = B * H
    assert max(len(h) for h in heads) <= -(-bh // 8) + 2
