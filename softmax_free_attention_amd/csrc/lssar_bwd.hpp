// lssar_bwd.hpp -- gfx950 kernels of the LSSAR causal attention backward.
//
// For the loss sum_i dO_i . out_i the gradients of q, k and v follow the
// forward (paper note "Softplus Attention with Re-weighting Boosts Length
// Extrapolation in Large Language Models", Method details, Key designs 1-3)
// step by step in reverse.  Per row i (1-based), keys j <= i, with the
// forward's base-2 quantities t_ij (score), sp_ij = log2(1 + 2^t) (Softplus
// / ln 2), S_i = sum_j sp_ij, the re-weighting y_ij = clamp((sp - tau) c, 0,
// 1) and Y_i = sum_j y^p (weights W_ij = y^p / Y):
//   dW_ij = dO_i . v_j                       (out = W V)
//   delta_i = sum_j W_ij dW_ij = dO_i . out_i
//   through W = r / sum r, r = ReLU(x)^p, x = i A - o (x = m y):
//       dA_ij = alpha_i y^(p-1) (dW_ij - delta_i),  alpha_i = p S_i / (gap_i Y_i)
//       (gap_i = sp_max - tau_i; y^(p-1) is the indicator y > 0 at p = 1)
//   through A = sp / S:  da_ij = (dA_ij - eps_i) / S,
//       eps_i = sum_j A_ij dA_ij = (alpha_i / S_i) (P2_i - delta_i Z_i),
//       P2_i = sum_j sp y^(p-1) dW_ij,  Z_i = sum_j sp y^(p-1)
//   through Softplus (derivative: the logistic sigmoid sigma(s) =
//       1 / (1 + 2^-t)) and s = ln d ln i q^.k^:
//       dc_ij = kappa_i sigma_ij (dA_ij - eps_i),  kappa_i = ln d ln i / (S_i ln 2)
//             = sigma_ij (Acoef_i y^(p-1) (dW_ij - delta_i) - Ecoef_i)
//   dq^_i = sum_j dc_ij k^_j,  dk^_j = sum_i dc_ij q^_i,  dv_j = sum_i W_ij dO_i
//   and through x^ = x / max(|x|, 1e-12): dx = (dx^ - (dx^ . x^) x^) / |x|
//   (dx^ / 1e-12 below the clamp).  A degenerate row (the forward's output 0)
//   passes no gradient: its coefficients are 0.
//
// Kernels (C = fp32 for bf16 inputs, fp64 for fp32 inputs; Softplus through
// softplus2_acc / softplus2_f64, exact for every t):
//   norms:    1 / max(|x|, 1e-12) for every row of Q and K;
//   rowstats: one wave per query row, lanes over keys: pass 1 S and the max
//             score, the row constants, pass 2 Y, P1 = sum y^p dW, P2, Z;
//             writes the row's coefficients;
//   dq:       one wave per query row: lanes over keys form dc_ij f_j for 64
//             keys in LDS, then lanes over dims accumulate dq^ from the key
//             rows (read whole);
//   dkdv:     one wave per key row: lanes over queries form W_ij and
//             dc_ij / |q_i| for 64 queries in LDS, then lanes over dims
//             accumulate dv and dk^ from the query and dO rows.
#pragma once

#include "lssar_decode.hpp"
#include "lssar_device.hpp"

namespace lssar {

constexpr int kBwdThreads = 256;   // 4 waves, one row each
// c, tc, invY, delta, Acoef, Ecoef, lam, rq per row (the bf16 kernels store
// c u, tc u, A Y u, -A delta Y u, E, lam, -, the largest score, u = Y^(-1/p))
constexpr int kBwdRowStats = 8;

template <typename C>
struct BwdMath;
template <>
struct BwdMath<float> {
    __device__ static float sp(float t) { return softplus2_acc(t); }
    __device__ static float sig(float t) { return sigmoid2(t); }
};
template <>
struct BwdMath<double> {
    __device__ static double sp(double t) { return softplus2_f64(t); }
    __device__ static double sig(double t) { return sigmoid2_f64(t); }
};

// Row of EPL-element pieces: lane `sub` of LPK holds elements sub*EPL..
template <typename T>
__device__ __forceinline__ void load_piece(const T* row, int sub, typename DecTraits<T>::C (&x)[DecTraits<T>::EPL])
{
    unpack(load_raw(row + sub * DecTraits<T>::EPL), x);
}

// Dot product of two rows held as EPL-element pieces by the LPK lanes of a
// group, reduced over the group.
template <typename C, int EPL, int LPK>
__device__ __forceinline__ C group_dot(const C (&a)[EPL], const C (&b)[EPL])
{
    C s = 0;
#pragma unroll
    for (int e = 0; e < EPL; ++e)
        s += a[e] * b[e];
#pragma unroll
    for (int o = 1; o < LPK; o <<= 1)
        s += __shfl_xor(s, o);
    return s;
}

template <typename C>
__device__ __forceinline__ C wave_sum(C x)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
        x += __shfl_xor(x, o);
    return x;
}
template <typename C>
__device__ __forceinline__ C wave_max(C x)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
        x = dmax(x, __shfl_xor(x, o));
    return x;
}

// y^(p-1): the derivative factor of y^p (indicator y > 0 at p = 1)
template <int P, typename C>
__device__ __forceinline__ C pow_m1(C y, int p)
{
    if constexpr (P == 1) {
        return y > (C)0 ? (C)1 : (C)0;
    } else if constexpr (P == 15) {
        const C y2 = y * y, y3 = y2 * y, y6 = y3 * y3, y7 = y6 * y;
        return y7 * y7;
    } else if constexpr (P == 0) {
        return p == 1 ? (y > (C)0 ? (C)1 : (C)0) : pow_chain<0>(y, p - 1);
    } else {
        return pow_chain<P - 1>(y, p - 1);
    }
}

// 1 / max(|x|, 1e-12) for every row of Q (rq) and K (fk): nrows rows each.
template <typename T, int D>
__global__ __launch_bounds__(kBwdThreads) void lssar_bwd_norms_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, typename DecTraits<T>::C* __restrict__ rq,
    typename DecTraits<T>::C* __restrict__ fk, long nrows)
{
    using C = typename DecTraits<T>::C;
    constexpr int EPL = DecTraits<T>::EPL;
    constexpr int LPK = D / EPL;
    constexpr int RPB = kBwdThreads / LPK;
    const long row = (long)blockIdx.x * RPB + threadIdx.x / LPK;
    const int sub = threadIdx.x % LPK;
    C xq[EPL], xk[EPL];
    for (int e = 0; e < EPL; ++e)
        xq[e] = xk[e] = 0;
    if (row < nrows) {
        load_piece(Q + row * D, sub, xq);
        load_piece(K + row * D, sub, xk);
    }
    const C sq = group_dot<C, EPL, LPK>(xq, xq), sk = group_dot<C, EPL, LPK>(xk, xk);
    if (row < nrows && sub == 0) {
        rq[row] = inv_norm(sq);
        fk[row] = inv_norm(sk);
    }
}

// Per query row: the forward's S, max score, row constants and Y, then the
// backward's delta, P2, Z and the row coefficients.  One wave per row.
template <typename T, int D, int P>
__global__ __launch_bounds__(kBwdThreads) void lssar_bwd_rowstats_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const T* __restrict__ dO, const typename DecTraits<T>::C* __restrict__ rq,
    const typename DecTraits<T>::C* __restrict__ fk, typename DecTraits<T>::C* __restrict__ stats,
    int L, long nrows, double lam_scale, float eps, int p_rt, const double* __restrict__ saved)
{
    using C = typename DecTraits<T>::C;
    using M = BwdMath<C>;
    constexpr int EPL = DecTraits<T>::EPL;
    constexpr int LPK = D / EPL;               // lanes per row piece
    constexpr int RPW = 64 / LPK;              // key rows per wave step
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int sub = lane % LPK, ksl = lane / LPK;
    const long grow = (long)blockIdx.x * 4 + wave;   // global query row
    if (grow >= nrows)
        return;                                // whole wave; no block barrier below
    const long bh = grow / L;
    const int row = (int)(grow % L), i = row + 1;
    const T* Kh = K + bh * L * D;
    const T* Vh = V + bh * L * D;
    const C* fkh = fk + bh * L;

    C qv[EPL], gv[EPL];
    load_piece(Q + grow * D, sub, qv);
    load_piece(dO + grow * D, sub, gv);
    // log2(e) ln d ln i / |q_i|  (Key design 1: log d . log N)
    const C lam = (C)(lam_scale * log((double)i)) * rq[grow];

    // pass 1: S and the max score, or the forward's saved statistics
    C s1 = 0, tmax = -INFINITY;
    if (saved) {
        load_row_stats(saved, (size_t)grow, s1, tmax);
    } else {
        for (int j0 = 0; j0 < i; j0 += RPW) {
            const int j = j0 + ksl;
            C kv[EPL];
            for (int e = 0; e < EPL; ++e)
                kv[e] = 0;
            if (j < i)
                load_piece(Kh + (size_t)j * D, sub, kv);
            const C dot = group_dot<C, EPL, LPK>(qv, kv);
            if (j < i && sub == 0) {
                const C t = dot * lam * fkh[j];
                s1 += M::sp(t);
                tmax = dmax(tmax, t);
            }
        }
        s1 = wave_sum(s1);
        tmax = wave_max(tmax);
    }
    const C o = i <= 3 ? (C)0 : (C)1;
    const C tau = o * s1 / (C)i;
    const C gap = M::sp(tmax) - tau;
    const bool degen = !((C)i * gap / s1 > (C)eps);
    const C c = degen ? (C)0 : (C)1 / gap;
    const C tc = tau * c;

    // pass 2: Y = sum y^p, P1 = sum y^p dW, P2 = sum sp y^(p-1) dW, Z = sum sp y^(p-1)
    C Y = 0, P1 = 0, P2 = 0, Z = 0;
    if (!degen) {
        for (int j0 = 0; j0 < i; j0 += RPW) {
            const int j = j0 + ksl;
            C kv[EPL], vv[EPL];
            for (int e = 0; e < EPL; ++e)
                kv[e] = vv[e] = 0;
            if (j < i) {
                load_piece(Kh + (size_t)j * D, sub, kv);
                load_piece(Vh + (size_t)j * D, sub, vv);
            }
            const C dot = group_dot<C, EPL, LPK>(qv, kv);
            const C dw = group_dot<C, EPL, LPK>(gv, vv);
            if (j < i && sub == 0) {
                const C t = dot * lam * fkh[j];
                const C sp = M::sp(t);
                C y = sp * c - tc;
                y = y < (C)0 ? (C)0 : (y > (C)1 ? (C)1 : y);
                const C yp = pow_chain<P>(y, p_rt);
                const C ym = pow_m1<P>(y, p_rt);
                Y += yp;
                P1 += yp * dw;
                P2 += sp * ym * dw;
                Z += sp * ym;
            }
        }
        Y = wave_sum(Y);
        P1 = wave_sum(P1);
        P2 = wave_sum(P2);
        Z = wave_sum(Z);
    }
    if (lane == 0) {
        C* st = stats + grow * kBwdRowStats;
        if (degen) {
            for (int e = 0; e < kBwdRowStats; ++e)
                st[e] = 0;
            st[6] = lam;
            st[7] = rq[grow];
        } else {
            const C delta = P1 / Y;
            const C alpha = (C)p_rt * s1 / (gap * Y);
            const C epsr = alpha / s1 * (P2 - delta * Z);
            const C kappa = (C)(log((double)D) * log((double)i) / 0.69314718055994530942) / s1;
            st[0] = c;
            st[1] = tc;
            st[2] = (C)1 / Y;
            st[3] = delta;
            st[4] = kappa * alpha;
            st[5] = kappa * epsr;
            st[6] = lam;
            st[7] = rq[grow];
        }
    }
}

// Per pair: (W_ij, dc_ij) from the score dot, dW and the row's coefficients.
template <typename C, int P>
struct PairGrad {
    C w, dc;
};
template <typename C, int P>
__device__ __forceinline__ PairGrad<C, P> pair_grad(C dot, C dw, C fkj, const C* st, int p_rt)
{
    using M = BwdMath<C>;
    const C t = dot * st[6] * fkj;
    const C sp = M::sp(t);
    C y = sp * st[0] - st[1];
    y = y < (C)0 ? (C)0 : (y > (C)1 ? (C)1 : y);
    PairGrad<C, P> g;
    g.w = pow_chain<P>(y, p_rt) * st[2];
    g.dc = M::sig(t) * (st[4] * pow_m1<P>(y, p_rt) * (dw - st[3]) - st[5]);
    return g;
}

// dq: one wave per query row; keys in steps of 64.
template <typename T, int D, int P>
__global__ __launch_bounds__(kBwdThreads) void lssar_bwd_dq_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const T* __restrict__ dO, const typename DecTraits<T>::C* __restrict__ fk,
    const typename DecTraits<T>::C* __restrict__ stats, T* __restrict__ dQ, int L, long nrows,
    int p_rt)
{
    using C = typename DecTraits<T>::C;
    constexpr int EPL = DecTraits<T>::EPL;
    constexpr int LPK = D / EPL;
    constexpr int RPW = 64 / LPK;
    constexpr int DPL = D / 64;                // dims per lane in the accumulation
    __shared__ C coef[4][64];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int sub = lane % LPK, ksl = lane / LPK;
    const long grow = (long)blockIdx.x * 4 + wave;
    if (grow >= nrows)
        return;
    const long bh = grow / L;
    const int i = (int)(grow % L) + 1;
    const T* Kh = K + bh * L * D;
    const T* Vh = V + bh * L * D;
    const C* fkh = fk + bh * L;
    C st[kBwdRowStats];
    for (int e = 0; e < kBwdRowStats; ++e)
        st[e] = stats[grow * kBwdRowStats + e];

    C qv[EPL], gv[EPL];
    load_piece(Q + grow * D, sub, qv);
    load_piece(dO + grow * D, sub, gv);
    C acc[DPL];
    for (int e = 0; e < DPL; ++e)
        acc[e] = 0;
    for (int j0 = 0; j0 < i; j0 += 64) {
        // coefficients dc_ij f_j of keys j0 .. j0 + 63 (0 past row i)
        for (int js = 0; js < 64; js += RPW) {
            const int j = j0 + js + ksl;
            C kv[EPL], vv[EPL];
            for (int e = 0; e < EPL; ++e)
                kv[e] = vv[e] = 0;
            if (j < i) {
                load_piece(Kh + (size_t)j * D, sub, kv);
                load_piece(Vh + (size_t)j * D, sub, vv);
            }
            const C dot = group_dot<C, EPL, LPK>(qv, kv);
            const C dw = group_dot<C, EPL, LPK>(gv, vv);
            if (sub == 0)
                coef[wave][js + ksl] =
                    j < i ? pair_grad<C, P>(dot, dw, fkh[j], st, p_rt).dc * fkh[j] : (C)0;
        }
        // lanes over dims: dq^ += sum_j coef_j k_j (rows read whole)
        const int jn = min(64, i - j0);
        for (int jj = 0; jj < jn; ++jj) {
            const C cj = coef[wave][jj];
            const T* kr = Kh + (size_t)(j0 + jj) * D;
#pragma unroll
            for (int e = 0; e < DPL; ++e)
                acc[e] += cj * (C)kr[lane + 64 * e];
        }
    }
    // dq = (dq^ - (dq^ . q^) q^) rq, or dq^ / 1e-12 below the norm clamp
    const C r = st[7];
    const T* qr = Q + grow * D;
    C qh[DPL], dd = 0;
    for (int e = 0; e < DPL; ++e) {
        qh[e] = (C)qr[lane + 64 * e] * r;
        dd += acc[e] * qh[e];
    }
    dd = wave_sum(dd);
    const bool clamped = !(r < (C)1e12);
    for (int e = 0; e < DPL; ++e)
        dQ[grow * D + lane + 64 * e] = (T)(clamped ? acc[e] * r : (acc[e] - dd * qh[e]) * r);
}

// dk and dv: one wave per key row; queries i >= j in steps of 64.
template <typename T, int D, int P>
__global__ __launch_bounds__(kBwdThreads) void lssar_bwd_dkdv_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const T* __restrict__ dO, const typename DecTraits<T>::C* __restrict__ fk,
    const typename DecTraits<T>::C* __restrict__ stats, T* __restrict__ dK, T* __restrict__ dV,
    int L, long nrows, int p_rt)
{
    using C = typename DecTraits<T>::C;
    constexpr int EPL = DecTraits<T>::EPL;
    constexpr int LPK = D / EPL;
    constexpr int RPW = 64 / LPK;
    constexpr int DPL = D / 64;
    __shared__ C cw[4][64], cq[4][64];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int sub = lane % LPK, ksl = lane / LPK;
    const long gkey = (long)blockIdx.x * 4 + wave;
    if (gkey >= nrows)
        return;
    const long bh = gkey / L;
    const int j = (int)(gkey % L);             // 0-based key row
    const T* Qh = Q + bh * L * D;
    const T* Gh = dO + bh * L * D;
    const C* sth = stats + bh * L * kBwdRowStats;
    const C fkj = fk[gkey];

    C kv[EPL], vv[EPL];
    load_piece(K + gkey * D, sub, kv);
    load_piece(V + gkey * D, sub, vv);
    C adv[DPL], adk[DPL];
    for (int e = 0; e < DPL; ++e)
        adv[e] = adk[e] = 0;
    for (int i0 = j; i0 < L; i0 += 64) {
        // W_ij and dc_ij / |q_i| of query rows i0 .. i0 + 63 (0 past L)
        for (int is = 0; is < 64; is += RPW) {
            const int r = i0 + is + ksl;        // 0-based query row
            C qv[EPL], gv[EPL];
            for (int e = 0; e < EPL; ++e)
                qv[e] = gv[e] = 0;
            if (r < L) {
                load_piece(Qh + (size_t)r * D, sub, qv);
                load_piece(Gh + (size_t)r * D, sub, gv);
            }
            const C dot = group_dot<C, EPL, LPK>(qv, kv);
            const C dw = group_dot<C, EPL, LPK>(gv, vv);
            if (sub == 0) {
                C w = 0, c = 0;
                if (r < L) {
                    const C* st = sth + (size_t)r * kBwdRowStats;
                    C s8[kBwdRowStats];
                    for (int e = 0; e < kBwdRowStats; ++e)
                        s8[e] = st[e];
                    const PairGrad<C, P> g = pair_grad<C, P>(dot, dw, fkj, s8, p_rt);
                    w = g.w;
                    c = g.dc * s8[7];
                }
                cw[wave][is + ksl] = w;
                cq[wave][is + ksl] = c;
            }
        }
        // lanes over dims: dv += sum_i W_ij dO_i, dk^ += sum_i (dc_ij / |q_i|) q_i
        const int in = min(64, L - i0);
        for (int ii = 0; ii < in; ++ii) {
            const C w = cw[wave][ii], c = cq[wave][ii];
            const T* qr = Qh + (size_t)(i0 + ii) * D;
            const T* gr = Gh + (size_t)(i0 + ii) * D;
#pragma unroll
            for (int e = 0; e < DPL; ++e) {
                adv[e] += w * (C)gr[lane + 64 * e];
                adk[e] += c * (C)qr[lane + 64 * e];
            }
        }
    }
    // dk = (dk^ - (dk^ . k^) k^) fk, or dk^ / 1e-12 below the norm clamp
    const T* kr = K + gkey * D;
    C kh[DPL], dd = 0;
    for (int e = 0; e < DPL; ++e) {
        kh[e] = (C)kr[lane + 64 * e] * fkj;
        dd += adk[e] * kh[e];
    }
    dd = wave_sum(dd);
    const bool clamped = !(fkj < (C)1e12);
    for (int e = 0; e < DPL; ++e) {
        dK[gkey * D + lane + 64 * e] = (T)(clamped ? adk[e] * fkj : (adk[e] - dd * kh[e]) * fkj);
        dV[gkey * D + lane + 64 * e] = (T)adv[e];
    }
}

}  // namespace lssar
