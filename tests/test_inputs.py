"""The seeded input generator (CPU only)."""
import numpy as np

import lssar_inputs as gen


def test_splitmix64_published_sequence():
    # SplitMix64 seeded with state 0 (Steele, Lea & Flood 2014): first outputs
    with np.errstate(over="ignore"):
        s = np.arange(1, 5, dtype=np.uint64) * gen._GAMMA
        got = [int(x) for x in gen._mix(s)]
    assert got == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F,
                   0xF88BB8A8724C81EC]


def test_counter_based_slices():
    full = gen.words(0, 1, 0, 1000)
    assert np.array_equal(gen.words(0, 1, 400, 100), full[400:500])
    n = gen.normals(3, 2, 0, 64)
    assert np.array_equal(gen.normals(3, 2, 10, 20), n[10:30])
    assert not np.array_equal(gen.words(0, 0, 0, 8), gen.words(0, 1, 0, 8))
    assert not np.array_equal(gen.words(0, 0, 0, 8), gen.words(1, 0, 0, 8))


def test_normal_moments():
    x = gen.normals(0, 0, 0, 1 << 20)
    assert abs(x.mean()) < 5e-3 and abs(x.std() - 1.0) < 5e-3
    u = gen.uniforms(0, 0, 0, 1 << 16)
    assert u.min() > 0.0 and u.max() <= 1.0


def test_bf16_round_to_nearest_even():
    one = np.float32(1.0)
    ulp = np.float32(2.0 ** -7)
    vals = np.array([1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -8 + 2.0 ** -20,
                     -2.5, 3.0e38], dtype=np.float32)
    want = np.array([1.0, 1.0, 1.0 + 2 * 2.0 ** -7, 1.0 + ulp, -2.5, 2.9908305e38],
                    dtype=np.float32)
    got = gen.round_to_bf16(vals)
    assert np.array_equal(got[:5], want[:5])
    assert got[5] == np.float32(gen.round_to_bf16(np.float32([3.0e38]))[0])
    assert one == gen.round_to_bf16(np.float32([1.0]))[0]


def test_workload_registry():
    assert [gen.WORKLOADS[n].L for n in gen.WORKLOAD_ORDER] == [128, 1024, 8192, 16384, 4096]
    w = gen.WORKLOADS["x8_planted"]
    assert w.flops == 4 * 64 * 12 * 8192 * 8193 // 2
    assert gen.WORKLOADS["tiny"].dtype == "f32"


def test_tiny_deterministic_and_iid():
    a = gen.make_inputs("tiny")
    b = gen.make_inputs("tiny")
    assert np.array_equal(a.q, b.q) and np.array_equal(a.v, b.v)
    assert a.q.shape == (1, 1, 128, 64) and a.q.dtype == np.float32
    assert not np.array_equal(a.q, a.k)


def test_planted_structure_small():
    inp = gen.make_inputs("x8_planted", L=512, H=2)
    for b, h, r, pos in inp.meta["planted"]:
        assert 256 <= r < 512 and len(pos) == 16 and max(pos) <= r
        u = inp.q[b, h, r].astype(np.float64)
        u /= np.linalg.norm(u)
        for j in pos:
            kj = inp.k[b, h, j].astype(np.float64)
            c = float(np.dot(kj, u) / np.linalg.norm(kj))
            assert abs(c - 0.9) < 0.01       # cosine 0.9 up to bf16 rounding
    assert np.array_equal(inp.k, gen.round_to_bf16(inp.k))


def test_lowrank_structure_small():
    inp = gen.make_inputs("wide", L=256, B=1, H=2)
    q = inp.q[0, 0].astype(np.float64)
    s = np.linalg.svd(q, compute_uv=False)
    # rank-8 signal plus std-0.1 noise: a clear gap after the 8th value
    assert s[7] > 5.0 * s[8]


def test_decode_inputs():
    a = gen.make_decode_inputs("x8_decode_ragged", B=8, Lmax=512, H=2)
    b = gen.make_decode_inputs("x8_decode_ragged", B=8, Lmax=512, H=2)
    assert a.q.shape == (8, 2, 64) and a.k.shape == (8, 2, 512, 64)
    assert np.array_equal(a.k, b.k) and np.array_equal(a.lens, b.lens)
    assert a.lens.dtype == np.int32 and np.all(a.lens >= 256) and np.all(a.lens <= 512)
    assert len(set(a.lens.tolist())) > 1
    assert np.array_equal(a.k, gen.round_to_bf16(a.k))
    f = gen.make_decode_inputs("x8_decode", B=2, Lmax=64, H=1)
    assert np.all(f.lens == 64)
