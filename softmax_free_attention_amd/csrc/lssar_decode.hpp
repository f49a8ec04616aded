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
// so every load instruction reads whole cache lines.  Each wave owns a
// quarter of its workgroup's chunk and issues all of its loads before using
// any (range-checked buffer loads: no branch around the chunk's tail).
#pragma once

#include "lssar_device.hpp"

namespace lssar {

constexpr int kDecThreads = 256;
// keys per workgroup: 32 KB of bf16 rows (256 keys at d = 64, 128 at d = 128)
__host__ __device__ constexpr int dec_chunk(int d) { return 16384 / d; }

// Compute type per input type: fp32 inputs run the whole step in fp64 (the
// parity bar for fp32 inputs is 1e-5; see the fp32 forward kernel).
template <typename T>
struct DecTraits;
template <>
struct DecTraits<__bf16> {
    using C = float;
    using Raw = u32x4;                         // 16 bytes as loaded
    static constexpr int EPL = 8;
};
template <>
struct DecTraits<float> {
    using C = double;
    using Raw = f32x4;
    static constexpr int EPL = 4;
};

// Buffer loads of base[voffset] with a range check: bytes at or past nbytes
// read as zero, so a chunk's tail needs no branch around its loads (kept out
// of kernel bodies, like the LDS-direct loads of the forward kernel).
// Cache rows are read once per step: the loads carry the non-temporal hint
// (cache-policy bit 1, `nt` on gfx950), measured 12% faster on a full
// 16 x 12 x 8192-row cache than default caching.
__device__ __forceinline__ u32x4 buf_load16(const void* base, unsigned nbytes, unsigned voffset)
{
    return __builtin_amdgcn_raw_buffer_load_b128(
        __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)nbytes,
                                          0x00020000),
        (int)voffset, 0, 2);
}
__device__ __forceinline__ float buf_load_c(const float* base, unsigned nbytes, unsigned voffset)
{
    return __builtin_bit_cast(
        float, __builtin_amdgcn_raw_buffer_load_b32(
                   __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), (short)0,
                                                     (int)nbytes, 0x00020000),
                   (int)voffset, 0, 0));
}
__device__ __forceinline__ double buf_load_c(const double* base, unsigned nbytes, unsigned voffset)
{
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(
        double, __builtin_amdgcn_raw_buffer_load_b64(
                    __builtin_amdgcn_make_buffer_rsrc(const_cast<double*>(base), (short)0,
                                                      (int)nbytes, 0x00020000),
                    (int)voffset, 0, 0));
}

__device__ __forceinline__ u32x4 as_raw(u32x4 w, const __bf16*) { return w; }
__device__ __forceinline__ f32x4 as_raw(u32x4 w, const float*) { return __builtin_bit_cast(f32x4, w); }

__device__ __forceinline__ u32x4 load_raw(const __bf16* p)
{
    return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ f32x4 load_raw(const float* p)
{
    return *reinterpret_cast<const f32x4*>(p);
}
__device__ __forceinline__ void unpack(const u32x4& w, float (&x)[8])
{
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        x[2 * e] = bf16lo(w[e]);
        x[2 * e + 1] = bf16hi(w[e]);
    }
}
__device__ __forceinline__ void unpack(const f32x4& w, double (&x)[4])
{
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

// 1 / max(sqrt(ss), 1e-12) in the compute type
__device__ __forceinline__ float inv_norm(float ss) { return 1.0f / fmaxf(sqrtf(ss), 1e-12f); }
__device__ __forceinline__ double inv_norm(double ss) { return 1.0 / fmax(sqrt(ss), 1e-12); }

// Cache rows in use for batch b: lens[b] clamped to [0, Lmax] (all Lmax
// rows when lens is null).
__device__ __forceinline__ int dec_len(const int* lens, int b, int Lmax)
{
    const int n = lens ? lens[b] : Lmax;
    return n < 0 ? 0 : (n > Lmax ? Lmax : n);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Elements 2E, 2E + 1 of eight bf16 values.  (A bit-cast of one element of
// a 32-bit vector was compiled as element 0 for every index; the whole
// vector is bit-cast and then shuffled instead.)
template <int E>
__device__ __forceinline__ bf16x2 bf16_pair(bf16x8 v)
{
    return __builtin_shufflevector(v, v, 2 * E, 2 * E + 1);
}

// sum_e a[e] b[e] + c over eight bf16 pairs by v_dot2c_f32_bf16
__device__ __forceinline__ float dot8_bf16(bf16x8 a, bf16x8 b, float c)
{
    c = __builtin_amdgcn_fdot2_f32_bf16(bf16_pair<0>(a), bf16_pair<0>(b), c, false);
    c = __builtin_amdgcn_fdot2_f32_bf16(bf16_pair<1>(a), bf16_pair<1>(b), c, false);
    c = __builtin_amdgcn_fdot2_f32_bf16(bf16_pair<2>(a), bf16_pair<2>(b), c, false);
    return __builtin_amdgcn_fdot2_f32_bf16(bf16_pair<3>(a), bf16_pair<3>(b), c, false);
}

// Sum of x over each aligned group of N lanes (8 or 16), in every lane of the
// group, by DPP moves folded into the adds: quad_perm [1,0,3,2] and [2,3,0,1]
// (lane ^ 1, lane ^ 2), then row_half_mirror (lane i <-> 7 - i within 8:
// quad against quad) and for 16 row_mirror (i <-> 15 - i).
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                                 0xf, 0xf, false));
}
template <int N>
__device__ __forceinline__ float lane_group_sum(float x)
{
    x += dpp_f32<0xB1>(x);
    x += dpp_f32<0x4E>(x);
    x += dpp_f32<0x141>(x);
    if constexpr (N == 16)
        x += dpp_f32<0x140>(x);
    return x;
}

// The value of lane n of each aligned group of N lanes (8 or 16), by
// ds_swizzle in bit mode: lane' = (lane & and_mask) | n within 32 lanes.
template <int PAT>
__device__ __forceinline__ float swizzle_f32(float v)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), PAT));
}
template <int N>
__device__ __forceinline__ float group_lane(float v, int n)
{
    constexpr int kAnd = 31 & ~(N - 1);
    switch (n) {                               // n is a constant after unrolling
    case 0: return swizzle_f32<kAnd | (0 << 5)>(v);
    case 1: return swizzle_f32<kAnd | (1 << 5)>(v);
    case 2: return swizzle_f32<kAnd | (2 << 5)>(v);
    case 3: return swizzle_f32<kAnd | (3 << 5)>(v);
    case 4: return swizzle_f32<kAnd | (4 << 5)>(v);
    case 5: return swizzle_f32<kAnd | (5 << 5)>(v);
    case 6: return swizzle_f32<kAnd | (6 << 5)>(v);
    default: return swizzle_f32<kAnd | (7 << 5)>(v);
    }
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
    constexpr int kDecChunk = dec_chunk(D);
    const int k0 = split * kDecChunk;
    if (k0 >= len)
        return;                                // whole workgroup: uniform
    const int kend = min(k0 + kDecChunk, len);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int sub = lane % LPK, ksl = lane / LPK;

    using Raw = typename DecTraits<T>::Raw;
    constexpr int NLD = kDecChunk / 4 / KPW;   // loads per lane
    constexpr unsigned RB = D * sizeof(T);     // bytes per cache row
    // the chunk's rows; keys past kend read as zeros
    const T* cbase = Kc + ((size_t)bh * Lmax + k0) * D;
    const unsigned cbytes = (unsigned)(kend - k0) * RB;
    const int kw = wave * (kDecChunk / 4);     // this wave's first key in the chunk
    Raw raw[NLD];
#pragma unroll
    for (int n = 0; n < NLD; ++n)
        raw[n] = as_raw(buf_load16(cbase, cbytes, (unsigned)(kw + n * KPW + ksl) * RB + sub * 16u),
                        cbase);

    C* sh = scores + (size_t)bh * Lmax;
    C s1 = 0, tmax = -INFINITY;
    if constexpr (std::is_same<T, __bf16>::value) {
        // bf16: q . k and |k|^2 of each 16-byte piece by v_dot2c_f32_bf16
        // (two products and the sum with one rounding: on random, tiny and
        // cancelling inputs as accurate as an fp32 fma chain), the LPK
        // lanes of a key summed by DPP moves, then one key per lane for the
        // rest: lane (sub, ksl) takes load n = sub mod NLD (d = 128: the
        // upper half of each key's 16 lanes repeats the lower and stores
        // nothing).  Per 64 keys at d = 64 this issues about 150 VALU
        // instructions instead of 800 with an fp32 fma per element, shuffles
        // through LDS and the tail on every eighth lane.
        static_assert(NLD == 8 && (LPK == 8 || LPK == 16), "decode lane layout");
        const bf16x8 q8 = __builtin_bit_cast(bf16x8, load_raw(Q + (size_t)bh * D + sub * EPL));
        const float qss = lane_group_sum<LPK>(dot8_bf16(q8, q8, 0.0f));
        // log2(e) ln d ln i / max(|q|, 1e-12), i = len (Key design 1: log d .
        // log N), in fp32: ln i = log2(i) ln 2
        const float lam = (float)lam_scale * (__builtin_amdgcn_logf((float)len) * 0.69314718055994531f) *
                          __builtin_amdgcn_rsqf(fmaxf(qss, 1e-24f));
        float dt[NLD], sq[NLD];
#pragma unroll
        for (int n = 0; n < NLD; ++n) {
            const bf16x8 k8 = __builtin_bit_cast(bf16x8, raw[n]);
            dt[n] = lane_group_sum<LPK>(dot8_bf16(q8, k8, 0.0f));
            sq[n] = lane_group_sum<LPK>(dot8_bf16(k8, k8, 0.0f));
        }
        const int n = sub & (NLD - 1);
        float dot = dt[0], ss = sq[0];
#pragma unroll
        for (int m = 1; m < NLD; ++m) {
            dot = n == m ? dt[m] : dot;
            ss = n == m ? sq[m] : ss;
        }
        const int key = k0 + kw + n * KPW + ksl;
        if (key < kend && sub < NLD) {
            // 1 / max(|k|, 1e-12) = rsqrt(max(|k|^2, 1e-24)), v_rsq_f32
            const float t = dot * lam * __builtin_amdgcn_rsqf(fmaxf(ss, 1e-24f));
            sh[key] = t;
            s1 = softplus_dec(t);
            tmax = t;
        }
    } else {
        C qv[EPL];
        unpack(load_raw(Q + (size_t)bh * D + sub * EPL), qv);
        C qss = 0;
#pragma unroll
        for (int e = 0; e < EPL; ++e)
            qss += qv[e] * qv[e];
#pragma unroll
        for (int o = 1; o < LPK; o <<= 1)
            qss += __shfl_xor(qss, o);
        // log2(e) ln d ln i / max(|q|, 1e-12), i = len (Key design 1: log d . log N)
        const C lam = (C)(lam_scale * log((double)len) / fmax(sqrt((double)qss), 1e-12));
#pragma unroll
        for (int n = 0; n < NLD; ++n) {
            const int key = k0 + kw + n * KPW + ksl;
            C kv[EPL];
            unpack(raw[n], kv);
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
                const C t = dot * lam * inv_norm(ss);
                sh[key] = t;
                s1 += softplus_dec(t);
                tmax = dmax(tmax, t);
            }
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
__device__ __forceinline__ DecRow<C> dec_row(const C* p1, int nvalid, int len, float eps)
{
    // every wave reduces all partials itself, in the same order: no barrier
    const int lane = threadIdx.x & 63;
    C s = 0, m = -INFINITY;
    for (int sp = lane; sp < nvalid; sp += 64) {
        s += p1[2 * sp];
        m = dmax(m, p1[2 * sp + 1]);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        s += __shfl_xor(s, o);
        m = dmax(m, __shfl_xor(m, o));
    }
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
    __shared__ C accs[4][D + 1];

    const int bh = (int)(blockIdx.x / nsplit), split = (int)(blockIdx.x % nsplit);
    const int len = dec_len(lens, bh / H, Lmax);
    constexpr int kDecChunk = dec_chunk(D);
    const int k0 = split * kDecChunk;
    if (k0 >= len)
        return;
    const int kend = min(k0 + kDecChunk, len);
    const int nvalid = (len + kDecChunk - 1) / kDecChunk;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int sub = lane % LPK, ksl = lane / LPK;

    using Raw = typename DecTraits<T>::Raw;
    constexpr int NLD = kDecChunk / 4 / KPW;
    constexpr unsigned RB = D * sizeof(T);
    const T* cbase = Vc + ((size_t)bh * Lmax + k0) * D;
    const unsigned cbytes = (unsigned)(kend - k0) * RB;
    const C* sbase = scores + (size_t)bh * Lmax + k0;
    const unsigned sbytes = (unsigned)(kend - k0) * (unsigned)sizeof(C);
    const int kw = wave * (kDecChunk / 4);
    constexpr bool kOwn = std::is_same<T, __bf16>::value;
    Raw raw[NLD];
    C tk[NLD];
    // bf16: each lane loads the score of one key, (n, ksl) with n = sub mod
    // NLD, and forms its weight once; the LPK lanes of key (n, ksl) take it
    // from lane n of their group by ds_swizzle.  (fp32: every lane forms
    // the weight of each key it multiplies.)
    C town = 0;
#pragma unroll
    for (int n = 0; n < NLD; ++n) {
        const unsigned lk = (unsigned)(kw + n * KPW + ksl);
        raw[n] = as_raw(buf_load16(cbase, cbytes, lk * RB + sub * 16u), cbase);
        if constexpr (!kOwn)
            tk[n] = buf_load_c(sbase, sbytes, lk * (unsigned)sizeof(C));
    }
    if constexpr (kOwn) {
        const unsigned lk = (unsigned)(kw + (sub & (NLD - 1)) * KPW + ksl);
        town = buf_load_c(sbase, sbytes, lk * (unsigned)sizeof(C));
    }

    const DecRow<C> rc = dec_row<C>(part1 + (size_t)bh * nsplit * 2, nvalid, len, eps);
    C* out2 = part2 + ((size_t)bh * nsplit + split) * (D + 1);
    if (rc.degen) {                            // uniform: write zero sums
        for (int e = threadIdx.x; e <= D; e += kDecThreads)
            out2[e] = 0;
        return;
    }

    // the weight of key (n, ksl): keys past the chunk (their rows read as
    // zeros) get weight 0
    auto weight = [&](C t, int n) {
        C y = softplus_dec(t) * rc.c - rc.tc;
        y = y < (C)0 ? (C)0 : (y > (C)1 ? (C)1 : y);
        const bool valid = kw + n * KPW + ksl < kend - k0;
        return valid ? pow_chain<P>(y, p_rt) : (C)0;
    };
    C acc[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e)
        acc[e] = 0;
    C dsum = 0;
    C wown = 0;
    if constexpr (kOwn) {
        wown = weight(town, sub & (NLD - 1));
        dsum = sub < NLD ? wown : (C)0;        // each key once
    }
#pragma unroll
    for (int n = 0; n < NLD; ++n) {
        C w;
        if constexpr (kOwn) {
            w = group_lane<LPK>(wown, n);
        } else {
            w = weight(tk[n], n);
            if (sub == 0)
                dsum += w;
        }
        C vv[EPL];
        unpack(raw[n], vv);
#pragma unroll
        for (int e = 0; e < EPL; ++e)
            acc[e] += w * vv[e];
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

// The whole decode step in one launch, one workgroup per (batch, head), for
// bf16 caches with many heads.  Phase A reads the head's K rows, stores
// each key's Softplus value (base 2) in the scores area of the workspace and
// reduces S1 and the largest score over the workgroup; phase B reads the V
// rows, forms each key's weight from its stored value and accumulates
// U = sum w v and D = sum w, and the workgroup writes out = U / D.  No
// partials leave the workgroup, so the chunk partials, the combine kernel
// and two kernel boundaries of the split path are gone.  With 192 heads,
// 192 workgroups of 512 threads with 8 loads in flight per lane read a
// cache at 7.1 TB/s in an in-bounds probe, against 6.6 TB/s for 12,288
// workgroups of 32 KB each; the split path is kept for fewer heads.
// Lanes: as in the split kernels, LPK lanes share a key and a wave-load
// reads KPW consecutive keys (1 KB); load n of wave w in a round covers
// keys (n NW + w) KPW + 0 .. KPW - 1.  Each round's loads are issued before
// the previous round is consumed.
constexpr int kDecFusedThreads = 512;

template <int D, int P>
__global__ __launch_bounds__(kDecFusedThreads) void lssar_decode_fused_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ Kc, const __bf16* __restrict__ Vc,
    const int* __restrict__ lens, float* __restrict__ sps, __bf16* __restrict__ out, int H,
    int Lmax, double lam_scale, float eps, int p_rt)
{
    constexpr int EPL = 8;                     // bf16 values per 16-byte load
    constexpr int LPK = D / EPL;               // lanes per key
    constexpr int KPW = 64 / LPK;              // keys per wave-load
    constexpr int NW = kDecFusedThreads / 64;  // waves
    constexpr int NLD = 8;                     // loads per lane and round
    constexpr int KPR = NW * KPW * NLD;        // keys per round
    constexpr unsigned RB = D * 2;             // bytes per cache row
    static_assert(LPK == 8 || LPK == 16, "decode lane layout");
    __shared__ float red[NW][2];
    __shared__ float accs[NW][D + 1];

    const int bh = (int)blockIdx.x;
    const int len = dec_len(lens, bh / H, Lmax);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int sub = lane % LPK, ksl = lane / LPK;
    __bf16* orow = out + (size_t)bh * D;
    if (len == 0) {                            // uniform: an empty cache gives 0
        for (int e = (int)threadIdx.x; e < D; e += kDecFusedThreads)
            orow[e] = (__bf16)0.0f;
        return;
    }
    const __bf16* kbase = Kc + (size_t)bh * Lmax * D;
    const __bf16* vbase = Vc + (size_t)bh * Lmax * D;
    const unsigned nbytes = (unsigned)len * RB;  // rows past len read as zeros
    float* sh = sps + (size_t)bh * Lmax;
    const unsigned sbytes = (unsigned)len * 4u;
    // the lane's own key of load n (one key per lane: load sub mod NLD;
    // at d = 128 the upper half of each key's lanes repeats the lower)
    const int nown = sub & (NLD - 1);
    auto key_of = [&](int k0, int n) { return k0 + (n * NW + wave) * KPW + ksl; };
    auto load_round = [&](const __bf16* base, int k0, u32x4 (&raw)[NLD]) {
#pragma unroll
        for (int n = 0; n < NLD; ++n)
            raw[n] = buf_load16(base, nbytes, (unsigned)key_of(k0, n) * RB + sub * 16u);
    };

    // the query and log2(e) ln d ln i / max(|q|, 1e-12), i = len (Key
    // design 1: log d . log N), as in the split scores kernel
    const bf16x8 q8 = __builtin_bit_cast(bf16x8, load_raw(Q + (size_t)bh * D + sub * EPL));
    const float qss = lane_group_sum<LPK>(dot8_bf16(q8, q8, 0.0f));
    const float lam = (float)lam_scale * (__builtin_amdgcn_logf((float)len) * 0.69314718055994531f) *
                      __builtin_amdgcn_rsqf(fmaxf(qss, 1e-24f));

    // ---- phase A: scores, their Softplus values, S1 and the largest score ----
    float s1 = 0.0f, tmax = -INFINITY;
    u32x4 cur[NLD], nxt[NLD];
    load_round(kbase, 0, nxt);
    for (int k0 = 0; k0 < len; k0 += KPR) {
#pragma unroll
        for (int n = 0; n < NLD; ++n)
            cur[n] = nxt[n];
        if (k0 + KPR < len)
            load_round(kbase, k0 + KPR, nxt);
        float dot = 0.0f, ss = 0.0f;
#pragma unroll
        for (int n = 0; n < NLD; ++n) {
            const bf16x8 k8 = __builtin_bit_cast(bf16x8, cur[n]);
            const float dn = lane_group_sum<LPK>(dot8_bf16(q8, k8, 0.0f));
            const float sn = lane_group_sum<LPK>(dot8_bf16(k8, k8, 0.0f));
            dot = n == nown ? dn : dot;
            ss = n == nown ? sn : ss;
        }
        const int key = key_of(k0, nown);
        if (key < len && sub < NLD) {
            // 1 / max(|k|, 1e-12) = rsqrt(max(|k|^2, 1e-24)), v_rsq_f32
            const float t = dot * lam * __builtin_amdgcn_rsqf(fmaxf(ss, 1e-24f));
            const float sp = softplus_dec(t);
            sh[key] = sp;
            s1 += sp;
            tmax = dmax(tmax, t);
        }
    }
    // phase B's first round in flight across the reduction
    load_round(vbase, 0, nxt);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        s1 += __shfl_xor(s1, o);
        tmax = dmax(tmax, __shfl_xor(tmax, o));
    }
    if (lane == 0) {
        red[wave][0] = s1;
        red[wave][1] = tmax;
    }
    __syncthreads();                           // also: every Softplus value stored
    float S = 0.0f, m = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) {             // a fixed order
        S += red[w][0];
        m = dmax(m, red[w][1]);
    }
    // row constants of the re-weighting (Key design 2)
    const float spmax = softplus_dec(m);
    const float o = len <= 3 ? 0.0f : 1.0f;
    const float tau = o * S / (float)len;
    const float gap = spmax - tau;
    const float mrow = (float)len * gap / S;   // max_j (i A_j - o_i)
    if (!(mrow > eps)) {                       // uniform: a degenerate row is 0
        for (int e = (int)threadIdx.x; e < D; e += kDecFusedThreads)
            orow[e] = (__bf16)0.0f;
        return;
    }
    const float c = 1.0f / gap, tc = tau * c;

    // ---- phase B: weights, U = sum w v and D = sum w ----
    float acc[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e)
        acc[e] = 0.0f;
    float dsum = 0.0f;
    for (int k0 = 0; k0 < len; k0 += KPR) {
#pragma unroll
        for (int n = 0; n < NLD; ++n)
            cur[n] = nxt[n];
        // the lane's own key's Softplus value (0 past len)
        const int key = key_of(k0, nown);
        const float sp = buf_load_c(sh, sbytes, (unsigned)key * 4u);
        if (k0 + KPR < len)
            load_round(vbase, k0 + KPR, nxt);
        const float y = __builtin_amdgcn_fmed3f(__builtin_fmaf(sp, c, -tc), 0.0f, 1.0f);
        const float wown = key < len ? pow_chain<P>(y, p_rt) : 0.0f;
        dsum += sub < NLD ? wown : 0.0f;       // each key once
#pragma unroll
        for (int n = 0; n < NLD; ++n) {
            const float w = group_lane<LPK>(wown, n);
            float vv[EPL];
            unpack(cur[n], vv);
#pragma unroll
            for (int e = 0; e < EPL; ++e)
                acc[e] = __builtin_fmaf(w, vv[e], acc[e]);
        }
    }
    // lanes with the same sub hold the same dims: sum over the key slots,
    // then over the waves in a fixed order
#pragma unroll
    for (int o2 = LPK; o2 < 64; o2 <<= 1) {
#pragma unroll
        for (int e = 0; e < EPL; ++e)
            acc[e] += __shfl_xor(acc[e], o2);
    }
#pragma unroll
    for (int o2 = 1; o2 < 64; o2 <<= 1)
        dsum += __shfl_xor(dsum, o2);
    if (ksl == 0) {
#pragma unroll
        for (int e = 0; e < EPL; ++e)
            accs[wave][sub * EPL + e] = acc[e];
    }
    if (lane == 0)
        accs[wave][D] = dsum;
    __syncthreads();
    for (int e = (int)threadIdx.x; e < D; e += kDecFusedThreads) {
        float u = 0.0f, den = 0.0f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            u += accs[w][e];
            den += accs[w][D];
        }
        orow[e] = (__bf16)(den > 0.0f ? u / den : 0.0f);
    }
}

// out = U / D over the chunks of each head (0 when D = 0: degenerate rows
// and empty caches).  One workgroup per head: thread (g, e) sums chunks
// g, g + G, ... of element e (G = 256 / (D + 1) rounded down, the element D
// being the weight sum), four loads in flight at a time; the G partial sums
// are then added in a fixed order.
template <typename T, int D>
__global__ __launch_bounds__(kDecThreads) void lssar_decode_combine_kernel(
    const int* __restrict__ lens, const typename DecTraits<T>::C* __restrict__ part2,
    T* __restrict__ out, int H, int Lmax, int nsplit)
{
    using C = typename DecTraits<T>::C;
    constexpr int E = D + 1;                   // elements per chunk record
    constexpr int G = kDecThreads / E;         // chunk groups
    __shared__ C red[G][E];
    const int bh = blockIdx.x;
    const int len = dec_len(lens, bh / H, Lmax);
    const int nvalid = (len + dec_chunk(D) - 1) / dec_chunk(D);
    const C* p2 = part2 + (size_t)bh * nsplit * E;
    const int g = threadIdx.x / E, e = threadIdx.x % E;
    if (g < G) {
        C a0 = 0, a1 = 0, a2 = 0, a3 = 0;
        int sp = g;
        for (; sp + 3 * G < nvalid; sp += 4 * G) {
            a0 += p2[(size_t)sp * E + e];
            a1 += p2[(size_t)(sp + G) * E + e];
            a2 += p2[(size_t)(sp + 2 * G) * E + e];
            a3 += p2[(size_t)(sp + 3 * G) * E + e];
        }
        for (; sp < nvalid; sp += G)
            a0 += p2[(size_t)sp * E + e];
        red[g][e] = (a0 + a1) + (a2 + a3);
    }
    __syncthreads();
    if (threadIdx.x < D) {
        C u = 0, den = 0;
#pragma unroll
        for (int k = 0; k < G; ++k) {
            u += red[k][threadIdx.x];
            den += red[k][D];
        }
        const C o = den > (C)0 ? u / den : (C)0;
        out[(size_t)bh * D + threadIdx.x] = (T)o;
    }
}

}  // namespace lssar
