"""Pins for the fp64 oracle: facts the pages and mathematics fix on their own.

Every pin takes a loaded oracle library (``oracle.load()`` or a deliberately
broken copy built by ``test_oracle_mutants.py``) and raises AssertionError
when the oracle disagrees.  Only ``brute_force_matrix_form`` restates the
definition; every other pin is a closed form of a constructed special case,
an invariant or a limit, so it does not share the oracle's structure.

Source of the definition: paper note "Softplus Attention with Re-weighting
Boosts Length Extrapolation in Large Language Models", Method details,
Key design 1 (LSSA), Key design 2 (re-weighting), Key design 3 (mask).  The
two variants of the note's ablation table (Key experimental data, ablation)
are pinned alongside: the stage-1 map swapped for the logistic Sigmoid, and
stage 1 alone ("LSSA only").  A pin that holds for a variant runs it too.
"""
from __future__ import annotations

import json
import math
import os

import mpmath as mp
import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


SP, SIG = oracle.PHI_SOFTPLUS, oracle.PHI_SIGMOID
# (phi, reweight): the method, the Sigmoid swap, and stage 1 alone
MODES = [(SP, True), (SIG, True), (SP, False)]
RW_MODES = [m for m in MODES if m[1]]


def _fwd(lib, q, k, v, p, eps=oracle.DEFAULT_EPS, mode=(SP, True)):
    return oracle.lssar_fwd(q, k, v, p, eps, nthreads=2, lib=lib, phi=mode[0],
                            reweight=mode[1])


def _phi_mp(phi, x):
    """Softplus log(1 + e^x), or the logistic sigmoid 1/(1 + e^-x)."""
    if phi == SIG:
        return 1 / (1 + mp.exp(-x))
    return mp.log(1 + mp.exp(x))


def _rng(seed):
    return np.random.default_rng(seed)


# --------------------------------------------------------------------------
# Brute force: the literal matrix form at 50 digits, tiny L
# --------------------------------------------------------------------------

def brute_lssar(Q, K, V, p, eps=oracle.DEFAULT_EPS, dps=50, mode=(SP, True)):
    """Matrix form with explicit N, M' and O (Key designs 1-2) in mpmath."""
    phi, reweight = mode
    with mp.workdps(dps):
        L, d = Q.shape
        Qm = mp.matrix(Q.tolist())
        Km = mp.matrix(K.tolist())

        def rownorm(M):
            R = mp.matrix(M.rows, M.cols)
            for r in range(M.rows):
                n = mp.sqrt(mp.fsum(M[r, c] ** 2 for c in range(M.cols)))
                n = max(n, mp.mpf("1e-12"))
                for c in range(M.cols):
                    R[r, c] = M[r, c] / n
            return R

        Qn, Kn = rownorm(Qm), rownorm(Km)
        S = Qn * Kn.T
        N = mp.matrix(L, L)
        Mp = mp.matrix(L, L)
        O = mp.matrix(L, L)
        for i in range(L):
            for j in range(L):
                N[i, j] = i + 1
                Mp[i, j] = 1 if j <= i else 0
                O[i, j] = 0 if i < 3 else 1
        A = mp.matrix(L, L)
        for i in range(L):
            for j in range(L):
                A[i, j] = _phi_mp(phi, mp.log(d) * mp.log(N[i, j]) * S[i, j]) * Mp[i, j]
        for i in range(L):
            s = mp.fsum(abs(A[i, j]) for j in range(L))
            for j in range(L):
                A[i, j] = A[i, j] / s
        Vm = mp.matrix(V.tolist())
        if not reweight:
            out = A * Vm
            return np.array([[float(out[i, c]) for c in range(d)] for i in range(L)])
        X = mp.matrix(L, L)
        for i in range(L):
            for j in range(L):
                X[i, j] = A[i, j] * N[i, j] - O[i, j]
        W = mp.matrix(L, L)
        for i in range(L):
            m = max(X[i, j] for j in range(L))
            if m <= eps:
                continue            # degenerate row -> zero output
            for j in range(L):
                W[i, j] = max(X[i, j], 0) ** p
            s = mp.fsum(abs(W[i, j]) for j in range(L))
            for j in range(L):
                W[i, j] = W[i, j] / s
        out = W * Vm
        return np.array([[float(out[i, c]) for c in range(d)] for i in range(L)])


def brute_force_matrix_form(lib):
    for mode in MODES:
        cases = [(1, 4, 3), (5, 4, 1), (7, 8, 2), (9, 6, 3), (12, 8, 15), (10, 3, 5)]
        for seed, (L, d, p) in enumerate(cases if mode == (SP, True) else cases[1::2]):
            r = _rng(100 + seed)
            Q, K, V = (r.standard_normal((L, d)) for _ in range(3))
            got = _fwd(lib, Q, K, V, p, mode=mode)
            want = brute_lssar(Q, K, V, p, mode=mode)
            err = np.max(np.abs(got - want))
            assert err < 1e-12, f"brute force {mode} L={L} d={d} p={p}: max err {err:.3e}"


# --------------------------------------------------------------------------
# Closed forms of constructed special cases
# --------------------------------------------------------------------------

def _ortho(d, seed):
    r = _rng(seed)
    Qm, R = np.linalg.qr(r.standard_normal((d, d)))
    return Qm.T * np.sign(np.diag(R))[:, None]      # rows orthonormal


def row1_is_v1(lib):
    """Row 1: log 1 = 0 makes its single stage-1 entry 1; o_1 = 0 keeps it."""
    for mode in MODES:
        for seed, (L, d, p) in enumerate([(6, 8, 3), (33, 16, 15), (3, 64, 1)]):
            r = _rng(200 + seed)
            Q, K, V = (r.standard_normal((L, d)) for _ in range(3))
            out = _fwd(lib, Q, K, V, p, mode=mode)
            assert np.array_equal(out[0], V[0]) or np.max(np.abs(out[0] - V[0])) < 1e-15, \
                f"row 1 must reproduce v_1 ({mode})"


def _closed_form_row(i, d, cos, p, V, mode=(SP, True)):
    """Expected output of row i (1-based) whose cosines to keys 1..i are
    ``cos`` (orthonormal keys): sp_j = phi(ln d ln i c_j); A = sp/sum;
    w_j = ReLU(i A_j - o_i)^p; out = sum w v / sum w (0 if max <= eps).
    Stage 1 alone: out = sum A v."""
    with mp.workdps(40):
        lam = mp.log(d) * mp.log(i)
        sp = [_phi_mp(mode[0], lam * mp.mpf(c)) for c in cos]
        s1 = mp.fsum(sp)
        if not mode[1]:
            return np.array([float(mp.fsum(sp[j] * V[j, c] for j in range(len(sp))) / s1)
                             for c in range(V.shape[1])])
        o = 0 if i <= 3 else 1
        x = [i * s / s1 - o for s in sp]
        if max(x) <= oracle.DEFAULT_EPS:
            return np.zeros(V.shape[1])
        w = [max(t, 0) ** p for t in x]
        den = mp.fsum(w)
        return np.array([float(mp.fsum(w[j] * V[j, c] for j in range(len(w))) / den)
                         for c in range(V.shape[1])])


def _build_rows(L, d, cos_rows, seed):
    """Keys: orthonormal directions with random positive lengths.  Query i:
    unit vector with the given cosines to keys 1..len(c), completed with a
    direction orthogonal to every key, then a random positive length."""
    assert L < d
    E = _ortho(d, seed)
    r = _rng(seed + 1)
    K = E[:L] * r.uniform(0.25, 4.0, size=(L, 1))
    Q = np.zeros((L, d))
    for i in range(L):
        c = np.zeros(L)
        c[:len(cos_rows[i])] = cos_rows[i]
        rest = 1.0 - float(np.dot(c, c))
        assert rest >= -1e-15
        qv = c @ E[:L] + math.sqrt(max(rest, 0.0)) * E[L]
        Q[i] = qv * r.uniform(0.25, 4.0)
    V = r.standard_normal((L, d))
    return Q, K, V


def closed_form_rows(lib):
    """Rows 2..L with hand-chosen cosines, including rows 2-3 (o = 0), row 4
    (first row with o = 1) and rows where some entries fall below the mean."""
    L, d = 12, 16
    cos_rows = [[0.3], [1.0, 0.0], [0.2, 0.9, -0.1], [0.6, 0.5, 0.1, -0.3],
                [0.0, 0.7, 0.7, 0.0, 0.1], [0.5] * 3 + [0.1] * 3,
                [0.9, -0.4, 0.1], [0.2, 0.3, 0.4, 0.5, 0.6],
                [-0.5, 0.8], [0.1] * 10, [0.95], [0.4, 0.4, 0.4, 0.41]]
    for mode in MODES:
        for p in ((1, 3, 15) if mode[1] else (3,)):
            Q, K, V = _build_rows(L, d, cos_rows, seed=300 + p)
            out = _fwd(lib, Q, K, V, p, mode=mode)
            for i in range(2, L + 1):
                cos = list(cos_rows[i - 1]) + [0.0] * (i - len(cos_rows[i - 1]))
                cos = cos[:i]
                want = _closed_form_row(i, d, cos, p, V[:i], mode)
                err = np.max(np.abs(out[i - 1] - want))
                assert err < 1e-11, f"closed form row {i} p={p} {mode}: err {err:.3e}"


def golden_row2_value(lib):
    """Hand-derived value from the fixture (d=64, p=3, q_2 parallel to k_1,
    orthogonal to k_2): w_1 = sp(ln64 ln2)^3 / (sp(ln64 ln2)^3 + (ln 2)^3)."""
    with open(os.path.join(GOLDEN, "closed_forms.json")) as f:
        g = json.load(f)
    for case in g["cases"]:
        d, p, w1 = case["d"], case["p"], case["w1"]
        E = _ortho(d, 7)
        K = np.stack([E[0] * 2.5, E[1] * 0.75])
        Q = np.stack([E[3] * 1.5, E[0] * 3.0])
        V = np.stack([np.full(d, 1.0), np.zeros(d)])      # out_2 = w_1 * 1 + w_2 * 0
        out = _fwd(lib, Q, K, V, p)
        assert abs(out[1, 0] - w1) < 5e-7, f"row-2 golden d={d} p={p}: {out[1, 0]} vs {w1}"


def sigmoid_antisymmetric_pair(lib):
    """Sigmoid map, row 2 (o_2 = 0) with cosines +c and -c to two
    orthonormal keys: sigma(-x) = 1 - sigma(x) makes the re-weighted weight
    of key 1 exactly sigma(x)^p / (sigma(x)^p + sigma(-x)^p) = 1/(1 + e^(-p x)),
    x = ln d ln 2 c, so out_2 = w v_1 + (1 - w) v_2."""
    for d, p, c in [(8, 1, 0.7), (16, 3, 0.3), (64, 15, 0.05), (32, 2, -0.6), (4, 5, 0.7071)]:
        E = _ortho(d, 1400 + p)
        K = np.stack([E[0] * 1.7, E[1] * 0.6])
        u = c * E[0] - c * E[1] + math.sqrt(1.0 - 2.0 * c * c) * E[2]
        Q = np.stack([E[2], u * 2.5])
        V = np.stack([np.arange(d, dtype=float), np.full(d, -1.0)])
        out = _fwd(lib, Q, K, V, p, mode=(SIG, True))
        x = math.log(d) * math.log(2.0) * c
        w = 1.0 / (1.0 + math.exp(-p * x))
        err = np.max(np.abs(out[1] - (w * V[0] + (1.0 - w) * V[1])))
        assert err < 1e-13, f"sigmoid pair d={d} p={p} c={c}: err {err:.3e}"


def onehot_orthonormal(lib):
    """Rows i >= 4, orthonormal keys, q_i along key m(i): out_i = v_m(i)
    exactly (every other entry has phi(0) -- ln 2 for Softplus, 1/2 for
    Sigmoid -- below the row mean).  Stage 1 alone gives
    (phi(ln d ln i) v_m + phi(0) sum_(j != m) v_j) / (phi(ln d ln i) + (i-1) phi(0))."""
    for mode in MODES:
        for seed, (L, d, p) in enumerate([(16, 32, 3), (31, 32, 15), (40, 64, 1), (20, 64, 2)]):
            r = _rng(400 + seed)
            E = _ortho(d, 410 + seed)
            perm = r.permutation(d)[:L]
            K = E[perm] * r.uniform(0.5, 3.0, size=(L, 1))
            mi = [int(r.integers(0, i + 1)) for i in range(L)]
            Q = np.stack([K[mi[i]] * r.uniform(0.1, 5.0) for i in range(L)])
            V = r.standard_normal((L, d))
            out = _fwd(lib, Q, K, V, p, mode=mode)
            for i in range(3, L):
                if mode[1]:
                    want = V[mi[i]]
                else:
                    big = math.log1p(math.exp(math.log(d) * math.log(i + 1)))
                    rest = V[:i + 1].sum(axis=0) - V[mi[i]]
                    want = (big * V[mi[i]] + math.log(2.0) * rest) / (big + i * math.log(2.0))
                err = np.max(np.abs(out[i] - want))
                assert err < 1e-12, f"one-hot row {i + 1} p={p} {mode}: err {err:.3e}"


def two_way_tie(lib):
    """q_i = (e_a + e_b)/sqrt2 over orthonormal keys: out_i = (v_a + v_b)/2."""
    L, d = 24, 32
    r = _rng(500)
    E = _ortho(d, 501)
    K = E[:L] * r.uniform(0.5, 2.0, size=(L, 1))
    V = r.standard_normal((L, d))
    Q = np.zeros((L, d))
    pairs = {}
    for i in range(L):
        a, b = sorted(r.choice(i + 1, size=2, replace=False)) if i >= 1 else (0, 0)
        pairs[i] = (a, b)
        Q[i] = (E[a] + E[b]) * r.uniform(0.5, 2.0)
    for mode in RW_MODES:
        for p in (1, 3, 15):
            out = _fwd(lib, Q, K, V, p, mode=mode)
            for i in range(3, L):
                a, b = pairs[i]
                err = np.max(np.abs(out[i] - 0.5 * (V[a] + V[b])))
                assert err < 1e-12, f"tie row {i + 1} p={p} {mode}: err {err:.3e}"


def degenerate_rows(lib):
    """All scores of a row equal: rows >= 4 are degenerate (output 0);
    rows 1-3 have o = 0 and give the mean of v_1..v_i.  Stage 1 alone has
    no degenerate rows: every row gives the mean of v_1..v_i."""
    L, d = 10, 8
    r = _rng(600)
    V = r.standard_normal((L, d))
    # (a) zero query rows
    K = r.standard_normal((L, d))
    Q = np.zeros((L, d))
    # (b) every key identical, queries random
    K2 = np.tile(r.standard_normal((1, d)), (L, 1))
    Q2 = r.standard_normal((L, d))
    for mode in MODES:
        for (QQ, KK) in ((Q, K), (Q2, K2)):
            for p in (1, 3, 15):
                out = _fwd(lib, QQ, KK, V, p, mode=mode)
                for i in range(L):
                    want = V[:i + 1].mean(axis=0) if (i < 3 or not mode[1]) else np.zeros(d)
                    err = np.max(np.abs(out[i] - want))
                    assert err < 1e-12, f"degenerate row {i + 1} p={p} {mode}: err {err:.3e}"


# --------------------------------------------------------------------------
# Invariants
# --------------------------------------------------------------------------

def v_identity_probe(lib):
    """V = I turns the output into the weight matrix: non-negative, exactly 0
    above the diagonal (M' multiplies), rows sum to 1.  Stage 1 alone keeps
    every unmasked weight strictly positive."""
    for mode in MODES:
        for seed, (L, d, p) in enumerate([(16, 16, 3), (24, 32, 15), (9, 9, 2), (12, 12, 1)]):
            r = _rng(700 + seed)
            Q, K = r.standard_normal((L, d)), r.standard_normal((L, d))
            V = np.eye(L, d)
            W = _fwd(lib, Q, K, V, p, mode=mode)[:, :L]
            assert np.all(W >= 0.0), "weights must be non-negative"
            assert np.all(W[np.triu_indices(L, 1)] == 0.0), "masked weights must be exactly 0"
            if not mode[1]:
                assert np.all(W[np.tril_indices(L)] > 0.0), "stage-1 weights must be positive"
            err = np.max(np.abs(W.sum(axis=1) - 1.0))
            assert err < 1e-13, f"row sums {mode}: err {err:.3e}"


def v_ones(lib):
    r = _rng(800)
    L, d = 40, 16
    Q, K = r.standard_normal((L, d)), r.standard_normal((L, d))
    for mode in MODES:
        for p in (1, 3, 15):
            out = _fwd(lib, Q, K, np.ones((L, d)), p, mode=mode)
            err = np.max(np.abs(out - 1.0))
            assert err < 1e-13, f"V = ones {mode}: err {err:.3e}"


def scale_invariance(lib):
    """Rows of Q and K are L2-normalised, so rescaling them changes nothing."""
    r = _rng(900)
    L, d = 30, 16
    Q, K, V = (r.standard_normal((L, d)) for _ in range(3))
    sq = r.uniform(0.1, 10.0, size=(L, 1))
    sk = r.uniform(0.1, 10.0, size=(L, 1))
    for mode in MODES:
        for p in (3, 15):
            base = _fwd(lib, Q, K, V, p, mode=mode)
            s2 = _fwd(lib, Q * 8.0, K * 0.25, V, p, mode=mode)
            assert np.max(np.abs(s2 - base)) < 1e-13, "power-of-two rescale changed output"
            s3 = _fwd(lib, Q * sq, K * sk, V, p, mode=mode)
            err = np.max(np.abs(s3 - base))
            assert err < 1e-11, f"row rescale changed output by {err:.3e} ({mode})"


def linearity_in_v(lib):
    r = _rng(1000)
    L, d = 25, 8
    Q, K, V1, V2 = (r.standard_normal((L, d)) for _ in range(4))
    for mode in MODES:
        for p in (2, 15):
            a = _fwd(lib, Q, K, V1, p, mode=mode)
            b = _fwd(lib, Q, K, V2, p, mode=mode)
            c = _fwd(lib, Q, K, 2.0 * V1 - 3.0 * V2, p, mode=mode)
            assert np.max(np.abs(c - (2.0 * a - 3.0 * b))) < 1e-12, "output not linear in V"


def causality(lib):
    """out_i depends on keys/values 1..i only (bitwise)."""
    r = _rng(1100)
    L, d = 20, 8
    Q, K, V = (r.standard_normal((L, d)) for _ in range(3))
    for mode in MODES:
        for p in (1, 3, 15):
            base = _fwd(lib, Q, K, V, p, mode=mode)
            for cut in (0, 3, 10, 18):
                K2, V2 = K.copy(), V.copy()
                K2[cut + 1:] = r.standard_normal(K2[cut + 1:].shape)
                V2[cut + 1:] = r.standard_normal(V2[cut + 1:].shape) * 100.0
                o2 = _fwd(lib, Q, K2, V2, p, mode=mode)
                assert np.array_equal(o2[:cut + 1], base[:cut + 1]), \
                    f"row <= {cut + 1} saw the future ({mode})"


def permutation_invariance(lib):
    """Permuting (k_j, v_j) pairs among j <= i leaves out_i unchanged."""
    r = _rng(1200)
    L, d = 18, 8
    Q, K, V = (r.standard_normal((L, d)) for _ in range(3))
    i = L - 1
    perm = r.permutation(L)
    for mode in MODES:
        for p in (3, 15):
            a = _fwd(lib, Q, K, V, p, mode=mode)[i]
            b = _fwd(lib, Q, K[perm], V[perm], p, mode=mode)[i]
            assert np.max(np.abs(a - b)) < 1e-12, f"last row depends on key order ({mode})"


def hard_argmax_limit(lib):
    """Key design 2: as p grows the weights approach the one-hot argmax.
    For the normalised weights w(p) with ratios r_k = x_k/x_max < 1 of the
    positive entries: |w(p) - e_max|_1 = 2 sum_k r_k^p / (1 + sum_k r_k^p)
    exactly, which is at most 2 (n - 1) r_2^p; the max weight never drops.
    The ratios come from the p = 1 weights, which are proportional to x."""
    for mode in RW_MODES:
        _hard_argmax_limit(lib, mode)


def _hard_argmax_limit(lib, mode):
    r = _rng(1300)
    L, d = 14, 14
    Q, K = r.standard_normal((L, d)), r.standard_normal((L, d))
    V = np.eye(L, d)
    W1 = _fwd(lib, Q, K, V, 1, mode=mode)[:, :L]
    prev = np.zeros(L)
    for p in range(1, 65):
        W = _fwd(lib, Q, K, V, p, mode=mode)[:, :L]
        for i in range(3, L):
            w = W[i, :i + 1]
            wmax = w.max()
            assert wmax >= prev[i] - 1e-14, f"row {i + 1}: max weight fell at p={p}"
            prev[i] = wmax
            m = int(np.argmax(W1[i, :i + 1]))
            ratios = np.delete(W1[i, :i + 1], m) / W1[i, m]
            ratios = ratios[ratios > 0]
            exact = 2.0 * np.sum(ratios ** p) / (1.0 + np.sum(ratios ** p))
            dist = np.abs(w - np.eye(i + 1)[m]).sum()
            assert abs(dist - exact) < 1e-9, f"row {i + 1} p={p}: {dist} vs {exact}"
            if len(ratios):
                assert dist <= 2.0 * len(ratios) * ratios.max() ** p + 1e-12
    # at p = 64 every row's leader holds almost all the weight
    assert np.median(prev[3:]) > 0.99


# --------------------------------------------------------------------------
# Backward (lssar_ref_bwd_f64): pinned by the forward oracle it differentiates
# --------------------------------------------------------------------------

def _bwd(lib, q, k, v, g, p, eps=oracle.DEFAULT_EPS):
    return oracle.lssar_bwd(q, k, v, g, p, eps, nthreads=2, lib=lib)


def bwd_finite_differences(lib):
    """Central differences of sum(dout * forward) (the forward oracle, pinned
    above) against the backward, every entry of dq, dk and dv."""
    cases = [(6, 5, 3, 0), (7, 4, 1, 1), (5, 6, 2, 2), (8, 4, 15, 3), (3, 3, 3, 4), (9, 3, 5, 5)]
    h = 1e-6
    for L, d, p, seed in cases:
        r = _rng(1500 + seed)
        Q, K, V, G = (r.standard_normal((L, d)) for _ in range(4))
        dq, dk, dv = _bwd(lib, Q, K, V, G, p)

        def loss(Qx, Kx, Vx):
            return float(np.sum(G * _fwd(lib, Qx, Kx, Vx, p)))

        for name, X, D in (("q", Q, dq), ("k", K, dk), ("v", V, dv)):
            num = np.zeros_like(X)
            for idx in np.ndindex(X.shape):
                Xp, Xm = X.copy(), X.copy()
                Xp[idx] += h
                Xm[idx] -= h
                args = {"q": lambda Y: (Y, K, V), "k": lambda Y: (Q, Y, V),
                        "v": lambda Y: (Q, K, Y)}[name]
                num[idx] = (loss(*args(Xp)) - loss(*args(Xm))) / (2 * h)
            err = np.max(np.abs(num - D))
            assert err < 1e-6 * (1.0 + np.max(np.abs(D))), \
                f"d{name} vs finite differences L={L} d={d} p={p}: {err:.3e}"


def bwd_scale_invariance(lib):
    """The output does not change when a row of Q or K is rescaled, so each
    gradient row is orthogonal to its input row: q_i . dq_i = k_j . dk_j = 0."""
    r = _rng(1600)
    for L, d, p in ((20, 8, 3), (33, 16, 15)):
        Q, K, V, G = (r.standard_normal((L, d)) for _ in range(4))
        dq, dk, _ = _bwd(lib, Q, K, V, G, p)
        scale = 1e-12 * (np.max(np.abs(dq)) + np.max(np.abs(dk))) * np.max(np.abs(Q))
        assert np.max(np.abs((Q * dq).sum(axis=1))) < 100 * scale + 1e-13
        assert np.max(np.abs((K * dk).sum(axis=1))) < 100 * scale + 1e-13
        assert np.max(np.abs(dq)) > 1e-3                    # not trivially zero


def bwd_dv_is_weights_transposed(lib):
    """out = W V is linear in V, so dv = W^T dout; W comes from the forward
    with V = I."""
    r = _rng(1700)
    for L, d, p in ((12, 12, 3), (16, 20, 15), (9, 9, 1)):
        Q, K, V, G = (r.standard_normal((L, d)) for _ in range(4))
        W = _fwd(lib, Q, K, np.eye(L, d), p)[:, :L]
        _, _, dv = _bwd(lib, Q, K, V, G, p)
        assert np.max(np.abs(dv - W.T @ G)) < 1e-12


def bwd_causality_and_row1(lib):
    """dk_j and dv_j see dout_i for i >= j only; dq_i sees keys and values
    j <= i only (bitwise); row 1 (scale ln 1 = 0) passes no gradient to q."""
    r = _rng(1800)
    L, d, p = 14, 6, 3
    Q, K, V, G = (r.standard_normal((L, d)) for _ in range(4))
    dq, dk, dv = _bwd(lib, Q, K, V, G, p)
    assert np.max(np.abs(dq[0])) == 0.0
    cut = 6
    G2 = G.copy()
    G2[:cut] = r.standard_normal((cut, d))
    _, dk2, dv2 = _bwd(lib, Q, K, V, G2, p)
    assert np.array_equal(dk2[cut:], dk[cut:]) and np.array_equal(dv2[cut:], dv[cut:])
    K3, V3 = K.copy(), V.copy()
    K3[cut:] = r.standard_normal((L - cut, d))
    V3[cut:] = r.standard_normal((L - cut, d))
    dq3, _, _ = _bwd(lib, Q, K3, V3, G, p)
    assert np.array_equal(dq3[:cut], dq[:cut])


def bwd_degenerate_rows(lib):
    """Identical keys make rows >= 4 degenerate (constant output 0): they pass
    no gradient, so dq of those rows is 0 and dv gets rows 1-3 only."""
    r = _rng(1900)
    L, d = 10, 5
    K = np.tile(r.standard_normal((1, d)), (L, 1))
    Q, V, G = (r.standard_normal((L, d)) for _ in range(3))
    for p in (1, 3):
        dq, dk, dv = _bwd(lib, Q, K, V, G, p)
        assert np.all(dq[3:] == 0.0)
        G3 = G.copy()
        G3[3:] = 0.0
        _, _, dv3 = _bwd(lib, Q, K, V, G3, p)
        assert np.array_equal(dv, dv3)


# --------------------------------------------------------------------------
# Row statistics (lssar_ref_rowstats_f64): S_i = sum_{j<=i} Softplus(s_ij)
# and m_i = max_{j<=i} s_ij, what a training forward keeps for its backward
# --------------------------------------------------------------------------

def _stats(lib, q, k):
    return oracle.lssar_rowstats(q, k, nthreads=2, lib=lib)


def rowstats_closed_forms(lib):
    """Orthonormal keys and queries with chosen cosines: s_ij = ln d ln i c_j
    (c_j = 0 for keys past the chosen ones), so S_i = sum_j Softplus(s_ij) over
    j <= i and m_i = ln d ln i max_j c_j, at 40 digits.  Includes rows whose
    cosines are all negative (m_i < 0, while masked keys would score 0), and
    row 1 (S_1 = ln 2, m_1 = 0)."""
    L, d = 11, 16
    cos_rows = [[0.6], [-0.3, -0.8], [-0.5, -0.5, -0.5], [0.6, 0.5, 0.1, -0.3],
                [0.0, 0.7, 0.7, 0.0, 0.1], [-0.2] * 6, [0.9, -0.4, 0.1],
                [0.2, 0.3, 0.4, 0.5, 0.6], [-0.5, 0.8], [0.1] * 10, [-0.95]]
    for seed in (0, 1):
        Q, K, _ = _build_rows(L, d, cos_rows, seed=400 + seed)
        st = _stats(lib, Q, K)
        assert abs(st[0, 0] - math.log(2.0)) < 1e-15 and st[0, 1] == 0.0
        for i in range(2, L + 1):
            cos = (list(cos_rows[i - 1]) + [0.0] * i)[:i]
            with mp.workdps(40):
                lam = mp.log(d) * mp.log(i)
                S = mp.fsum(mp.log(1 + mp.exp(lam * mp.mpf(c))) for c in cos)
                m = lam * max(mp.mpf(c) for c in cos)
            assert abs(st[i - 1, 0] - float(S)) < 1e-12 * float(S), f"S_{i}"
            assert abs(st[i - 1, 1] - float(m)) < 1e-12, f"m_{i}"


def rowstats_invariants(lib):
    """Softplus(m_i) <= S_i <= i Softplus(m_i); row i ignores keys j > i
    (bitwise) and the order of keys j <= i; rows of Q and K enter through their
    directions only (powers of two rescale exactly)."""
    r = _rng(2000)
    L, d = 40, 8
    Q, K = r.standard_normal((L, d)), r.standard_normal((L, d))
    st = _stats(lib, Q, K)
    sp = np.logaddexp(0.0, st[:, 1])
    i = np.arange(1, L + 1)
    assert np.all(sp <= st[:, 0] * (1 + 1e-14)) and np.all(st[:, 0] <= i * sp * (1 + 1e-14))
    cut = 17
    K2 = K.copy()
    K2[cut:] = r.standard_normal((L - cut, d))
    assert np.array_equal(_stats(lib, Q, K2)[:cut], st[:cut])
    perm = np.concatenate([r.permutation(cut), np.arange(cut, L)])
    st3 = _stats(lib, Q, K[perm])
    assert np.max(np.abs(st3[cut - 1] - st[cut - 1])) < 1e-12 * max(1.0, abs(st[cut - 1, 0]))
    scale_q = 2.0 ** r.integers(-8, 9, size=(L, 1))
    scale_k = 2.0 ** r.integers(-8, 9, size=(L, 1))
    st4 = _stats(lib, Q * scale_q, K * scale_k)
    assert np.max(np.abs(st4 - st) / np.maximum(1.0, np.abs(st))) < 1e-13


# --------------------------------------------------------------------------
# The row-sampling entry, and the oracle's own stage-2 self-check
# --------------------------------------------------------------------------

def rows_entry_matches_forward(lib):
    """The row-sampling entry (the checker wherever a workload is too large
    for the full forward) returns bitwise the rows of the full forward, which
    every other pin checks, for sorted, unsorted and repeated row sets that
    include the first and the last row, in all three modes."""
    r = _rng(1500)
    for (L, d, p) in [(37, 8, 3), (64, 16, 15), (9, 4, 1), (130, 64, 15)]:
        Q, K, V = (r.standard_normal((L, d)) for _ in range(3))
        Q[L // 3] = 0.0                               # a degenerate row among them
        sets = [np.arange(L), r.permutation(L)[: max(1, L // 2)],
                np.array([L - 1, 0, min(3, L - 1), min(3, L - 1), L - 1, 1, 0]),
                np.array([L // 3, L - 1]), np.array([0])]
        for mode in MODES:
            full = _fwd(lib, Q, K, V, p, mode=mode)
            for rows in sets:
                got = oracle.lssar_rows(Q, K, V, rows, p, nthreads=2, lib=lib, phi=mode[0],
                                        reweight=mode[1])
                assert got.shape == (len(rows), d)
                assert np.array_equal(got, full[rows]), \
                    f"rows entry differs from the forward: L={L} p={p} {mode} rows={rows[:8]}"


def rescaled_form_self_check(lib):
    """Every re-weighted row is also computed with its entries divided by the
    row maximum m before the power (Key design 2: the factor m^-p cancels in
    the L1 normalisation), and the oracle refuses (status -3) when the two
    disagree.  One-hot rows over orthonormal keys at d = 64 reach
    m = i Softplus(ln 64 ln i) / S1_i - 1 = 13.5 at i = 40, whose literal
    400th power overflows fp64; at p = 15 both forms agree and the output is
    the one-hot closed form v_m(i).  (The Sigmoid map keeps m below 1 on
    these rows, sigma <= 1 against a row mean of at least 1/2, so its
    literal power cannot overflow and only the closed form is checked.)"""
    L, d = 40, 64
    r = _rng(1600)
    E = _ortho(d, 1601)
    K = E[:L] * r.uniform(0.5, 3.0, size=(L, 1))
    mi = [int(r.integers(0, i + 1)) for i in range(L)]
    Q = np.stack([K[mi[i]] * r.uniform(0.1, 5.0) for i in range(L)])
    V = r.standard_normal((L, d))
    for mode in RW_MODES:
        out = _fwd(lib, Q, K, V, 15, mode=mode)
        for i in range(3, L):
            assert np.max(np.abs(out[i] - V[mi[i]])) < 1e-12, f"one-hot row {i + 1} {mode}"
        if mode[0] != SP:
            continue
        refused = 0
        for call in (lambda: _fwd(lib, Q, K, V, 400, mode=mode),
                     lambda: oracle.lssar_rows(Q, K, V, [L - 1], 400, nthreads=2, lib=lib,
                                               phi=mode[0], reweight=mode[1])):
            try:
                call()
            except ValueError as e:
                assert "status -3" in str(e), str(e)
                refused += 1
        assert refused == 2, f"the literal 400th power overflowed unnoticed ({mode})"


PINS = [brute_force_matrix_form, row1_is_v1, closed_form_rows, golden_row2_value,
        sigmoid_antisymmetric_pair, onehot_orthonormal, two_way_tie, degenerate_rows,
        v_identity_probe, v_ones, scale_invariance, linearity_in_v, causality,
        permutation_invariance, hard_argmax_limit, bwd_finite_differences,
        bwd_scale_invariance, bwd_dv_is_weights_transposed, bwd_causality_and_row1,
        bwd_degenerate_rows, rowstats_closed_forms, rowstats_invariants,
        rows_entry_matches_forward, rescaled_form_self_check]
