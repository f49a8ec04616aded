// lssar_decode.hpp -- gfx950 kernels of the LSSAR decode step.
//
// One new query per (batch b, head h) at 1-based position i = len_b attends
// to rows 1..i of a key/value cache.  What it computes is row i of the
// causal forward (paper note "Softplus Attention with Re-weighting Boosts
// Length Extrapolation in Large Language Models", Method details, Key
// designs 1-3): A_j = Softplus(ln d ln i q^ . k^_j) / S1 for j <= i, then
// ReLU(i A_j - o_i)^p normalised, times V.  The note's point is
// extrapolation to 8-16x the training length at inference, where this step
// reads the whole cache once per token.
//
// With one query there is no contraction worth a matrix core: every key costs
// 2d flops against 2d bytes (bf16), so the step is bound by HBM.  The kernels
// read K once and V once, split over workgroups of kDecChunk keys:
//   scores:  per key t_j = log2(e) ln d ln i (q . k_j) / (|q| |k_j|) (the key
//            norm is computed from the row being read, no prep step), stored
//            to the workspace; per chunk the partial S1 and max of t;
//   pv:      every workgroup of a head combines the chunk partials in the same
//            fixed order (so all agree), forms the row constants of the
//            re-weighting, and accumulates sum_j w_j v_j and sum_j w_j over
//            its chunk from the stored scores;
//   combine: per head, the chunk sums in order, out = U / D (0 for a
//            degenerate row, whose chunks write zeros).
// Softplus uses softplus2_acc (fp32) or softplus2_f64 (fp64) throughout:
// the decode step is memory-bound, so the exact form costs nothing.
//
// Lanes: a 16-byte load holds EPL elements of a row; LPK = d / EPL lanes
// share one key, and a wave reads 64 / LPK consecutive keys (1 KB) per load,
// so every load instruction reads whole cache lines.
#pragma once

#include "lssar_device.hpp"

namespace lssar {

constexpr int kDecChunk = 256;     // keys per workgroup
constexpr int kDecThreads = 256;

// Compute type per input type: fp32 inputs run the whole step in fp64 (the
// parity bar for fp32 inputs is 1e-5; see the fp32 forward kernel).
template <typename T>
struct DecTraits;
template <>
struct DecTraits<__bf16> {
    using C = float;
    static constexpr int EPL = 8;
};
template <>
struct DecTraits<float> {
    using C = double;
    static constexpr int EPL = 4;
};

__device__ __forceinline__ void load_row16(const __bf16* p, float (&x)[8])
{
    const u32x4 w = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        x[2 * e] = bf16lo(w[e]);
        x[2 * e + 1] = bf16hi(w[e]);
    }
}
__device__ __forceinline__ void load_row16(const float* p, double (&x)[4])
{
    const f32x4 w = *reinterpret_cast<const f32x4*>(p);
#pragma unroll
    for (int e = 0; e < 4; ++e)
        x[e] = (double)w[e];
}

__device__ __forceinline__ float softplus_dec(float t) { return softplus2_acc(t); }
__device__ __forceinline__ double softplus_dec(double t) { return softplus2_f64(t); }

template <typename C>
__device__ __forceinline__ C dmax(C a, C b)
{
    return a > b ? a : b;
}

// Cache rows in use for batch b: lens[b] clamped to [0, Lmax] (all Lmax
// rows when lens is null).
__device__ __forceinline__ int dec_len(const int* lens, int b, int Lmax)
{
    const int n = lens ? lens[b] : Lmax;
    return n < 0 ? 0 : (n > Lmax ? Lmax : n);
}

// Workgroup-wide sum and max of one value per thread, in a fixed order.
template <typename C>
__device__ __forceinline__ void block_sum_max(C& s, C& m, C* red)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        s += __shfl_xor(s, o);
        m = dmax(m, __shfl_xor(m, o));
    }
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
        red[2 * wave] = s;
        red[2 * wave + 1] = m;
    }
    __syncthreads();
    s = (red[0] + red[2]) + (red[4] + red[6]);
    m = dmax(dmax(red[1], red[3]), dmax(red[5], red[7]));
    __syncthreads();
}

// Scores and per-chunk (S1, max t).  Grid: nsplit * BH workgroups, item
// w -> (head w / nsplit, chunk w % nsplit).
template <typename T, int D>
__global__ __launch_bounds__(kDecThreads) void lssar_decode_scores_kernel(
    const T* __restrict__ Q, const T* __restrict__ Kc, const int* __restrict__ lens,
    typename DecTraits<T>::C* __restrict__ scores, typename DecTraits<T>::C* __restrict__ part1,
    int H, int Lmax, int nsplit, double lam_scale)
{
    using C = typename DecTraits<T>::C;
    constexpr int EPL = DecTraits<T>::EPL;
    constexpr int LPK = D / EPL;               // lanes per key
    constexpr int KPW = 64 / LPK;              // keys per wave per load
    __shared__ C red[8];

    const int bh = (int)(blockIdx.x / nsplit), split = (int)(blockIdx.x % nsplit);
    const int len = dec_len(lens, bh / H, Lmax);
    const int k0 = split * kDecChunk;
    if (k0 >= len)
        return;                                // whole workgroup: uniform
    const int kend = min(k0 + kDecChunk, len);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int sub = lane % LPK, ksl = lane / LPK;

    C qv[EPL];
    load_row16(Q + (size_t)bh * D + sub * EPL, qv);
    C qss = 0;
#pragma unroll
    for (int e = 0; e < EPL; ++e)
        qss += qv[e] * qv[e];
#pragma unroll
    for (int o = 1; o < LPK; o <<= 1)
        qss += __shfl_xor(qss, o);
    // log2(e) ln d ln i / max(|q|, 1e-12), i = len (Key design 1: log d . log N)
    const C lam = (C)(lam_scale * log((double)len) / fmax(sqrt((double)qss), 1e-12));

    const T* Kh = Kc + (size_t)bh * Lmax * D;
    C* sh = scores + (size_t)bh * Lmax;
    C s1 = 0, tmax = -INFINITY;
    for (int kb = k0 + wave * KPW; kb < kend; kb += 4 * KPW) {
        const int key = kb + ksl;
        C kv[EPL];
#pragma unroll
        for (int e = 0; e < EPL; ++e)
            kv[e] = 0;
        if (key < kend)
            load_row16(Kh + (size_t)key * D + sub * EPL, kv);
        C dot = 0, ss = 0;
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            dot += qv[e] * kv[e];
            ss += kv[e] * kv[e];
        }
#pragma unroll
        for (int o = 1; o < LPK; o <<= 1) {
            dot += __shfl_xor(dot, o);
            ss += __shfl_xor(ss, o);
        }
        if (key < kend && sub == 0) {
            const C t = dot * lam / (C)fmax(sqrt((double)ss), 1e-12);
            sh[key] = t;
            s1 += softplus_dec(t);
            tmax = dmax(tmax, t);
        }
    }
    block_sum_max(s1, tmax, red);
    if (threadIdx.x == 0) {
        part1[((size_t)bh * nsplit + split) * 2] = s1;
        part1[((size_t)bh * nsplit + split) * 2 + 1] = tmax;
    }
}

// Row constants of the re-weighting from the chunk partials of one head,
// combined in a fixed order by every thread of the workgroup.
template <typename C>
struct DecRow {
    C c, tc;
    bool degen;
};

template <typename C>
__device__ __forceinline__ DecRow<C> dec_row(const C* p1, int nvalid, int len, float eps, C* red)
{
    C s = 0, m = -INFINITY;
    for (int sp = threadIdx.x; sp < nvalid; sp += kDecThreads) {
        s += p1[2 * sp];
        m = dmax(m, p1[2 * sp + 1]);
    }
    block_sum_max(s, m, red);
    const C spmax = softplus_dec(m);
    const C o = len <= 3 ? (C)0 : (C)1;
    const C tau = o * s / (C)len;
    const C gap = spmax - tau;
    const C mrow = (C)len * gap / s;           // max_j (i A_j - o_i)
    DecRow<C> r;
    r.degen = !(mrow > (C)eps);
    r.c = r.degen ? (C)0 : (C)1 / gap;
    r.tc = tau * r.c;
    return r;
}

// Weights and the chunk's sums U = sum w v (d values) and D = sum w.
template <typename T, int D, int P>
__global__ __launch_bounds__(kDecThreads) void lssar_decode_pv_kernel(
    const T* __restrict__ Vc, const int* __restrict__ lens,
    const typename DecTraits<T>::C* __restrict__ scores,
    const typename DecTraits<T>::C* __restrict__ part1, typename DecTraits<T>::C* __restrict__ part2,
    int H, int Lmax, int nsplit, float eps, int p_rt)
{
    using C = typename DecTraits<T>::C;
    constexpr int EPL = DecTraits<T>::EPL;
    constexpr int LPK = D / EPL;
    constexpr int KPW = 64 / LPK;
    __shared__ C red[8];
    __shared__ C accs[4][D + 1];

    const int bh = (int)(blockIdx.x / nsplit), split = (int)(blockIdx.x % nsplit);
    const int len = dec_len(lens, bh / H, Lmax);
    const int k0 = split * kDecChunk;
    if (k0 >= len)
        return;
    const int kend = min(k0 + kDecChunk, len);
    const int nvalid = (len + kDecChunk - 1) / kDecChunk;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int sub = lane % LPK, ksl = lane / LPK;

    const DecRow<C> rc = dec_row<C>(part1 + (size_t)bh * nsplit * 2, nvalid, len, eps, red);
    C* out2 = part2 + ((size_t)bh * nsplit + split) * (D + 1);
    if (rc.degen) {                            // uniform: write zero sums
        for (int e = threadIdx.x; e <= D; e += kDecThreads)
            out2[e] = 0;
        return;
    }

    const T* Vh = Vc + (size_t)bh * Lmax * D;
    const C* sh = scores + (size_t)bh * Lmax;
    C acc[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e)
        acc[e] = 0;
    C dsum = 0;
    for (int kb = k0 + wave * KPW; kb < kend; kb += 4 * KPW) {
        const int key = kb + ksl;
        if (key < kend) {
            C y = softplus_dec(sh[key]) * rc.c - rc.tc;
            y = y < (C)0 ? (C)0 : (y > (C)1 ? (C)1 : y);
            const C w = pow_chain<P>(y, p_rt);
            C vv[EPL];
            load_row16(Vh + (size_t)key * D + sub * EPL, vv);
#pragma unroll
            for (int e = 0; e < EPL; ++e)
                acc[e] += w * vv[e];
            if (sub == 0)
                dsum += w;
        }
    }
    // lanes with the same sub hold the same dims: sum over the key slots
#pragma unroll
    for (int o = LPK; o < 64; o <<= 1) {
#pragma unroll
        for (int e = 0; e < EPL; ++e)
            acc[e] += __shfl_xor(acc[e], o);
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1)
        dsum += __shfl_xor(dsum, o);
    if (ksl == 0) {
#pragma unroll
        for (int e = 0; e < EPL; ++e)
            accs[wave][sub * EPL + e] = acc[e];
    }
    if (lane == 0)
        accs[wave][D] = dsum;
    __syncthreads();
    for (int e = threadIdx.x; e <= D; e += kDecThreads)
        out2[e] = (accs[0][e] + accs[1][e]) + (accs[2][e] + accs[3][e]);
}

// out = U / D over the chunks of each head (0 when D = 0: degenerate rows
// and empty caches).  One workgroup of D threads per head.
template <typename T, int D>
__global__ __launch_bounds__(D) void lssar_decode_combine_kernel(
    const int* __restrict__ lens, const typename DecTraits<T>::C* __restrict__ part2,
    T* __restrict__ out, int H, int Lmax, int nsplit)
{
    using C = typename DecTraits<T>::C;
    const int bh = blockIdx.x, e = threadIdx.x;
    const int len = dec_len(lens, bh / H, Lmax);
    const int nvalid = (len + kDecChunk - 1) / kDecChunk;
    const C* p2 = part2 + (size_t)bh * nsplit * (D + 1);
    C u = 0, den = 0;
    for (int sp = 0; sp < nvalid; ++sp) {
        u += p2[(size_t)sp * (D + 1) + e];
        den += p2[(size_t)sp * (D + 1) + D];
    }
    const C o = den > (C)0 ? u / den : (C)0;
    out[(size_t)bh * D + e] = (T)o;
}

}  // namespace lssar
