// lssar_device.hpp -- gfx950 (CDNA4) kernels of the LSSAR causal attention
// forward.
//
// Method: paper note "Softplus Attention with Re-weighting Boosts Length
// Extrapolation in Large Language Models" (papernotes.org), Method details.
//   Key design 1 (LSSA): rows of Q and K L2-normalised; for j <= i,
//     A_ij = Softplus(ln d * ln i * q^_i . k^_j), masked entries multiplied
//     by 0 (Key design 3); each row divided by its L1 norm S1_i.
//   Key design 2 (re-weighting): A_ij <- ReLU(i A_ij - o_i)^p, o_i = 0 for
//     rows 1-3 else 1; each row divided by its L1 norm again; out = A V.
//
// How the kernels compute it (exact rearrangements of the definition):
//   * The norms are applied to the fp32 accumulator of the raw contraction:
//       s_ij = (ln d ln i / |q_i|) * (1/|k_j|) * (q_i . k_j).
//     The prep kernel stores 1/|k_j| per key row; the attention kernel
//     computes the query factor while loading its query block.
//   * Softplus runs in base 2: with t = s log2(e), log2(1 + 2^t) =
//     Softplus(s)/ln 2.  Every later quantity is a ratio of Softplus values,
//     so the constant factor cancels; log2(e) is folded into the query factor.
//   * With tau_i = o_i S1_i / i and sp_max the row's largest Softplus value,
//       i A_ij - o_i = (i / S1_i) (sp_ij - tau_i),
//     so the re-weighted row, after its L1 normalisation, equals the row of
//       y_ij = clamp((sp_ij - tau_i) / (sp_max,i - tau_i), 0, 1)^p
//     divided by its sum.  y stays in [0, 1], so y^p cannot overflow at any p
//     (the note lists ReLU^p overflow at large p as a limitation).
//   * m_i = max_j (i A_ij - o_i) = i (sp_max,i - tau_i) / S1_i decides the
//     degenerate rows (m_i <= eps: output 0).
//   * S1_i must be complete before any weight is known, so each workgroup
//     makes two passes over its keys: pass 1 accumulates S1 and the row max
//     of the scores; pass 2 recomputes the scores, re-weights and
//     accumulates P.V and the weight sum with MFMA, then divides.
//
// Variants (the note's ablation table, Key experimental data): the stage-1
// map phi may be the logistic Sigmoid instead of Softplus ("Sigmoid + L1 +
// re-weighting"; the same rearrangement holds with phi in place of
// Softplus), and stage 2 may be left out ("LSSA only": out = A V, one pass
// over the keys with weights phi(s_ij) normalised by their sum).
//
// Tiling (bf16): a workgroup of 4 waves owns one 64-row query block of one
// (batch, head), 16 rows per wave; each XCD takes a slice of the heads and
// runs its blocks largest first (lssar_sched.hpp).  Keys stream through LDS in tiles
// of 64 (double-buffered at d = 64, one buffer at d = 128).  Scores are
// computed transposed, S^T = K Q^T, with v_mfma_f32_16x16x32_bf16: each lane
// then holds 4 keys of ONE query row, so row sums stay per lane until one
// cross-lane reduction per pass, and the lane's weights are already the B
// operand of O^T = V^T P^T (V^T comes transposed from the prep kernel).  The
// weight sum is one more MFMA of the same weights against a block of ones.
//
// Training forward: when given a statistics buffer, the Softplus method
// stores each row's S1 and largest score after pass 1 (natural units) for
// the backward, which then need not recompute them.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "lssar_sched.hpp"

namespace lssar {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;   // 4 waves of 64
constexpr int kWaves = 4;
constexpr int kBK = 64;         // keys per tile
// bf16 kernel: 16 query rows per wave, 64 per workgroup
constexpr int kMQ16 = 16;
constexpr int kBQ16 = kWaves * kMQ16;
// fp32 kernel: 32 query rows per wave, 128 per workgroup
constexpr int kMQ32 = 32;
constexpr int kBQ32 = kWaves * kMQ32;

// ---------------------------------------------------------------------------
// Elementwise pieces shared by both dtypes
// ---------------------------------------------------------------------------

// log2(1 + 2^t) = Softplus(t ln 2) / ln 2 (Key design 1's Softplus, base 2).
// |t| <= log2(e) ln(d) ln(L) stays far below the exp2 overflow at 128 for
// every supported size.  For t < -24 the result rounds to 0, an absolute
// error below 2^-24 on values that are summed with O(1) terms.
__device__ __forceinline__ float softplus2(float t)
{
    return __builtin_amdgcn_logf(1.0f + __builtin_amdgcn_exp2f(t));
}

// Stage-1 maps.  Sigmoid(t ln 2) = 1 / (1 + 2^-t) needs no constant factor;
// a masked t = -inf gives 1 / inf = 0.
constexpr int kPhiSoftplus = 0;
constexpr int kPhiSigmoid = 1;

__device__ __forceinline__ float sigmoid2(float t)
{
    return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-t));
}

template <int PHI>
__device__ __forceinline__ float phi2(float t)
{
    if constexpr (PHI == kPhiSigmoid)
        return sigmoid2(t);
    else
        return softplus2(t);
}

// Deep rows.  fp32 evaluates log2(1 + 2^t) through the rounding of 1 + 2^t,
// whose absolute error 2^-24 is a relative error 2^-24 / 2^t of the result:
// for t below about -8 the value loses digits, and below -24 it is 0.  A row
// whose largest score is below kDeep (every Softplus2 value below
// log2(1 + 2^kDeep)) is only as good as these digits, so its block is
// computed again with softplus2_acc, which takes the series
// ln(1 + e) = e - e^2 / 2 + ... for e = 2^t < 2^-8 (dropped terms below
// 2^-17.6 relative) and the logarithm otherwise.  Stage 1 alone flags a row
// whose mean Softplus2 value is below kDeepMean instead (its largest score
// is not tracked there).
constexpr float kDeep = -4.0f;
constexpr float kDeepMean = 1.0f / 1024.0f;

// Conditioning of a re-weighted row.  The fast query operand (lambda_i q^_i
// rounded to f16, 2^-11 relative per element) moves a score by up to
// 2^-11 lambda_i, and the re-weighting turns a score error dt into a
// relative weight error of about p dt / (y (sp_max - tau)): the row's
// kappa_i = p lambda_i / (sp_max - tau) (base-2 units) scales it.  A row
// with kappa_i above kCondMax has its block computed again from the exact
// query rows.  Long rows of ordinary inputs have kappa near 40 at p = 15;
// rows of a few keys with nearly tied scores can have any kappa.
constexpr float kCondMax = 100.0f;

__device__ __forceinline__ float softplus2_acc(float t)
{
    constexpr float kLog2e = 1.4426950408889634f;
    const float e = __builtin_amdgcn_exp2f(t);
    const float series = kLog2e * e * __builtin_fmaf(-0.5f, e, 1.0f);
    return e < (1.0f / 256.0f) ? series : __builtin_amdgcn_logf(1.0f + e);
}

// Maxima of scores straight from the matrix cores.  fmaxf ignores a quiet
// NaN, and in IEEE mode the compiler quiets both operands first (one
// v_max_f32 x, x per score) unless it can prove them canonical, which it
// cannot for an MFMA result; the NaN-propagating maximum needs no quieting
// (v_maximum3_f32).  Scores of finite inputs are never NaN, and a masked
// pair's -inf behaves the same under both.
__device__ __forceinline__ float max_scores(float a, float b)
{
    return __builtin_elementwise_maximum(a, b);
}
__device__ __forceinline__ float max3_scores(float a, float b, float c)
{
    return __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b), c);
}

// What a run of pass 1 accumulates besides the row max.  kPass1Sum: S1 as
// max(t, 0) plus log2 of the product of the factors 1 + 2^-|t| (Softplus),
// or as a plain sum (Sigmoid); kPass1Acc: S1 from softplus2_acc (blocks
// computed again); kPass1Prod: S1 as log2 of the product of the factors
// 1 + 2^t themselves (scores at most kProdMaxT).
constexpr int kPass1Sum = 0;
constexpr int kPass1Acc = 1;
constexpr int kPass1Prod = 2;
// Largest base-2 score for which two factors 1 + 2^t times a mantissa below
// 1 stay finite in fp32 (2^121 < 2^128), with room for the f16 operands'
// rounding of lambda_i q^_i . k^_j above lambda_i.
constexpr float kProdMaxT = 60.0f;

// y^P for y in [0, 1] by a fixed multiplication chain (P = 0: runtime p).
template <int P, typename F>
__device__ __forceinline__ F pow_chain(F y, int p)
{
    if constexpr (P == 1) {
        return y;
    } else if constexpr (P == 2) {
        return y * y;
    } else if constexpr (P == 3) {
        return y * y * y;
    } else if constexpr (P == 15) {
        F y2 = y * y, y3 = y2 * y, y6 = y3 * y3, y12 = y6 * y6;
        return y12 * y3;
    } else {
        F r = 1, b = y;
        while (p) {
            if (p & 1)
                r *= b;
            b *= b;
            p >>= 1;
        }
        return r;
    }
}

// clamp(sp * c - tc, 0, 1): the rescaled ReLU argument; the clamp folds
// into the FMA's output modifier.
__device__ __forceinline__ float reweight_arg(float sp, float c, float tc)
{
    return __builtin_amdgcn_fmed3f(__builtin_fmaf(sp, c, -tc), 0.0f, 1.0f);
}

// Row constants after pass 1 (Key design 2).  i: 1-based row; s1: sum of
// the row's phi values (base-2 Softplus or Sigmoid, or relative Softplus for
// a deep row); spmax: the row's largest phi value.
struct RowConst {
    float c;      // 1 / (sp_max - tau), or 0 for a degenerate row
    float tc;     // tau * c
    bool degen;
};

__device__ __forceinline__ RowConst row_constants_sp(int i, float s1, float spmax, float eps)
{
    const float o = (i <= 3) ? 0.0f : 1.0f;
    const float tau = o * s1 / (float)i;
    const float gap = spmax - tau;
    const float m = (float)i * gap / s1;       // max_j (i A_ij - o_i)
    RowConst rc;
    rc.degen = !(m > eps);
    rc.c = rc.degen ? 0.0f : 1.0f / gap;
    rc.tc = tau * rc.c;
    return rc;
}

// ... from the row's largest scaled score tmax (phi is increasing)
template <int PHI>
__device__ __forceinline__ RowConst row_constants(int i, float s1, float tmax, float eps)
{
    return row_constants_sp(i, s1, phi2<PHI>(tmax), eps);
}

// fp64 versions for the fp32-input kernel.  With fp32 inputs the parity bar
// is 1e-5 absolute, and the re-weighting multiplies the absolute error of a
// Softplus value by about p / (sp_ij - tau_i): at p = 15 the fp32 spacing of
// scores and Softplus values near 30-70 (2^-19..2^-17) alone would use the
// whole budget.  The score -> Softplus -> re-weighting chain therefore runs
// in fp64 there; the contractions' inputs stay exact fp32 values.
typedef double f64x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ double softplus2_f64(double t)
{
    // log2(1 + 2^t), kept accurate for large |t| of either sign
    constexpr double kLog2e = 1.4426950408889634074;
    return t > 0.0 ? t + log1p(exp2(-t)) * kLog2e : log1p(exp2(t)) * kLog2e;
}

__device__ __forceinline__ double sigmoid2_f64(double t)
{
    return 1.0 / (1.0 + exp2(-t));
}

template <int PHI>
__device__ __forceinline__ double phi2_f64(double t)
{
    if constexpr (PHI == kPhiSigmoid)
        return sigmoid2_f64(t);
    else
        return softplus2_f64(t);
}

struct RowConstD {
    double c, tc;
    bool degen;
};

template <int PHI>
__device__ __forceinline__ RowConstD row_constants_f64(int i, double s1, double tmax, float eps)
{
    const double spmax = phi2_f64<PHI>(tmax);
    const double o = (i <= 3) ? 0.0 : 1.0;
    const double tau = o * s1 / (double)i;
    const double gap = spmax - tau;
    const double m = (double)i * gap / s1;
    RowConstD rc;
    rc.degen = !(m > (double)eps);
    rc.c = rc.degen ? 0.0 : 1.0 / gap;
    rc.tc = tau * rc.c;
    return rc;
}

// log2(e) ln(d) ln(i) / max(|q_i|, 1e-12) from the squared norm, in fp64
__device__ __forceinline__ double query_factor(double lam_scale, int i, double ss)
{
    return lam_scale * log((double)i) / fmax(sqrt(ss), 1e-12);
}

// Workgroup -> work-item map that keeps each XCD on a contiguous slice of the
// work.  Workgroups are dispatched round-robin over the 8 XCDs (workgroup w
// runs on XCD w % 8), and each XCD has its own L2; item order is head-major,
// so the heads whose K and V an XCD reads stay few and stay in its L2.
constexpr int kXcds = 8;
__device__ __forceinline__ int xcd_item(int w, int n)
{
    const int x = w % kXcds, local = w / kXcds;
    const int per = n / kXcds, rem = n % kXcds;
    return x * per + min(x, rem) + local;
}

__device__ __forceinline__ float bf16lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

// ---------------------------------------------------------------------------
// Prep kernels
// ---------------------------------------------------------------------------

// Prep for the fp32 kernel: fk[row] = 1 / max(|k_row|_2, 1e-12) in fp64 for
// every key row (Key design 1's K_j <- K_j / |K_j|_2, kept as a factor of
// the score).  fp64 because deep rows (every score far below 0) turn the
// absolute error of a score into a relative error of its Softplus value.
template <int D>
__global__ __launch_bounds__(kThreads) void lssar_knorm_f32_kernel(const float* __restrict__ K,
                                                                   double* __restrict__ fk,
                                                                   long nrows)
{
    constexpr int LPR = D / 4;                 // lanes per row, 4 floats per lane
    constexpr int RPB = kThreads / LPR;        // rows per block
    const long row = (long)blockIdx.x * RPB + threadIdx.x / LPR;
    const int sub = threadIdx.x % LPR;
    double ss = 0.0;
    if (row < nrows) {
        // loaded as a float vector: a bit-cast of an element of a u32x4 was
        // lowered as element 0 for every index by this compiler
        const f32x4 x = *reinterpret_cast<const f32x4*>(K + row * D + sub * 4);
#pragma unroll
        for (int e = 0; e < 4; ++e)
            ss = fma((double)x[e], (double)x[e], ss);
    }
#pragma unroll
    for (int m = LPR / 2; m >= 1; m >>= 1)
        ss += __shfl_xor(ss, m, LPR);
    if (row < nrows && sub == 0)
        fk[row] = 1.0 / fmax(sqrt(ss), 1e-12);
}

// Prep for the bf16 kernel, one workgroup per (64-key block kb, head bh):
//  * fk[bh*L + j] = 1 / max(|k_j|_2, 1e-12) for the block's keys (fp64 sum
//    of squares, one rounding to fp32): the exact scores' key factor;
//  * KN16[bh][j] = f16(k_j / max(|k_j|_2, 1e-12)) (unless KN16 is null): the
//    normalised key rounded to f16, the fast path's operand, whose scores
//    need no per-pair key factor;
//  * sched[w] = (bh, qb) for the attention kernel's workgroup w
//    (lssar_sched.hpp): each workgroup enters the query block qb = kb of
//    its head (the blocks and the 64-key blocks coincide), and the
//    workgroups (kb, 0) also mark the empty indices (-1, -1) of XCDs
//    kb, kb + nkb, ... up to per_xcd, the grid's indices per XCD (from the
//    host).  (One thread that counted all eight slices and wrote every
//    empty index set the end of the kernel.)
// The exact scores read K itself (bf16 products are exact in fp32).
template <int D>
__global__ __launch_bounds__(kThreads) void lssar_prep_bf16_kernel(
    const __bf16* __restrict__ K, float* __restrict__ fk, _Float16* __restrict__ KN16,
    int2* __restrict__ sched, int BH, int L, int Lp, int per_xcd)
{
    constexpr int LPR = D / 8;                 // lanes per key row for the norms
    const int kb = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
    const size_t hoff = (size_t)bh * L * D;

    if (tid == 0) {
        const FwdSched sc(BH, Lp / kBK);
        sched[sc.index_of(bh, kb)] = make_int2(bh, kb);
    }
    if (bh == 0 && tid < 64) {
        for (int x = kb; x < kSchedXcds; x += (int)gridDim.x) {
            const int n = FwdSched(BH, Lp / kBK).count(x);
            for (int l = n + tid; l < per_xcd; l += 64)
                sched[l * kSchedXcds + x] = make_int2(-1, -1);
        }
    }

    // key norms: 64 rows x LPR lanes, 16 bytes per lane per step
#pragma unroll
    for (int n = 0; n < 64 * LPR / kThreads; ++n) {
        const int c = tid + n * kThreads;
        const int key = c / LPR, sub = c % LPR;
        const int kg = kb * 64 + key;
        double ss = 0.0;
        float xv[8];
        u32x4 w = {0u, 0u, 0u, 0u};
        if (kg < L)
            w = *reinterpret_cast<const u32x4*>(K + hoff + (size_t)kg * D + sub * 8);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            xv[2 * e] = bf16lo(w[e]);
            xv[2 * e + 1] = bf16hi(w[e]);
            ss = fma((double)xv[2 * e], (double)xv[2 * e], ss);
            ss = fma((double)xv[2 * e + 1], (double)xv[2 * e + 1], ss);
        }
#pragma unroll
        for (int m = LPR / 2; m >= 1; m >>= 1)
            ss += __shfl_xor(ss, m, LPR);
        if (kg < L) {
            const double inv = 1.0 / fmax(sqrt(ss), 1e-12);
            if (sub == 0)
                fk[(size_t)bh * L + kg] = (float)inv;
            if (KN16) {
                // fp32 product, then f16 (a direct fp64 -> f16 conversion
                // is a long integer sequence on this part); the fp32 step
                // adds at most 2^-23 relative to the f16 rounding
                const float invf = (float)inv;
                f16x8 hn;
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    hn[i] = (_Float16)(xv[i] * invf);
                *reinterpret_cast<f16x8*>(KN16 + hoff + (size_t)kg * D + sub * 8) = hn;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// bf16 attention kernel
// ---------------------------------------------------------------------------
//
// A workgroup of 4 waves owns one query block of 64 rows of one (batch,
// head); each wave owns 16 rows (lane & 15).  The causal work of block qb
// grows with qb, so each XCD runs the blocks of its slice of heads largest
// first and the hardware fills freed slots with ever smaller blocks (greedy
// longest-first; lssar_sched.hpp).  Pairing blocks {nqb-1-pi, pi} per
// workgroup instead gives every workgroup the same work, but half as many
// waves: at B = 1, H = 12, L = 8192 that leaves 3 of the 4 wave slots per
// SIMD filled, and measured 15% slower.  Keys stream through LDS in tiles of 64 with
// buffer loads that write LDS directly (16 bytes per lane, zero past the end
// of the tensor), double-buffered.  LDS tiles are arrays of 16-byte slots,
// XOR-swizzled so that the 16 lanes reading one MFMA operand hit distinct
// banks.  Lane group grp = lane >> 4 holds keys 16 ks + 4 grp + r (r = 0..3)
// of every 16-key block ks of a tile.
//
// Pass 1 keeps, per lane and query row, the sum of Softplus2(t) =
// log2(1 + 2^t) in one of two product forms:
//  * while every score of the block is at most kProdMaxT: log2 of the
//    product of the factors 1 + 2^t_j, held as a mantissa in [0.5, 1) and
//    an exponent and renormalised after every two factors (one exp2 and
//    one fma per pair, one log2 per row);
//  * otherwise (long rows), as Softplus2(t) = max(t, 0) + log2(1 + 2^-|t|):
//    sum_j max(t_j, 0) plus log2 of the product of the factors
//    (1 + 2^-|t_j|), each in (1, 2] (one exp2 per pair and one log2 per
//    tile for its 16 factors, whose product stays below 2^16).
// Masked pairs get t = -inf, which adds exactly 0 to every sum in both
// passes (2^-inf = 0 and a factor 1, max(-inf, 0) = 0; in pass 2
// Softplus2 = 0 gives y = clamp(-tau c) = 0).

// One tile of BK keys: K and V (BK rows of D each, row-major) and the BK
// key factors (the area holds 64; the loader writes 64).
template <int D, int BK>
struct Bf16Tile {
    static constexpr int R = D / 8;                       // 16-byte slots per row
    static constexpr int KBYTES = BK * D * 2;             // K tile
    static constexpr int VBYTES = BK * D * 2;             // V tile
    static constexpr int FBYTES = 64 * 4;                 // key factors
    static constexpr int BYTES = KBYTES + VBYTES + FBYTES;
    static constexpr int KLOADS = KBYTES / 1024 / kWaves; // 1 KB wave-loads per wave
    static constexpr int VLOADS = VBYTES / 1024 / kWaves;
    // XOR swizzle of a K row's slots (key & 15 is all that matters)
    __device__ static int kswz(int key) { return R == 8 ? ((key >> 1) & 7) : (key & 15); }
    // XOR swizzle of a V row's slots.  V is read only by the LDS transpose
    // read (the A operand of O^T = V^T P^T: four consecutive keys of one
    // dim per lane); these are the swizzles an in-bounds microbenchmark
    // timed fastest for that read at 8 and 16 slots per row.
    __device__ static int vswz(int key)
    {
        return R == 8 ? (key & 7) : ((((key & 3) << 2) | ((key >> 2) & 3)) ^ ((key >> 1) & 2));
    }
};

typedef __attribute__((address_space(3))) void lds_void;
typedef short s16x4 __attribute__((ext_vector_type(4)));

// Four 16-bit elements by the LDS transpose read (ds_read_b64_tr_b16).  In
// each group of 16 lanes, lane j names 8 bytes (four consecutive elements
// of one row), and lane 4 q + e receives element e of the 8 bytes named by
// lanes q, q + 4, q + 8 and q + 12: with lane j naming row r0 + j / 4,
// columns c0 + 4 (j % 4) .. + 3, lane 4 q + e gets column c0 + 4 q + e of
// rows r0 .. r0 + 3.
__device__ __forceinline__ bf16x4 lds_read_tr16(const unsigned char* p)
{
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
    return __builtin_bit_cast(bf16x4, v);
}

// Buffer loads of base[voffset + soffset] written straight to LDS at
// lds + size * lane, 16 or 4 bytes per lane (reads at or past `nbytes`
// return zeros).  Kept out of kernel bodies: the host pass of a kernel that
// names the buffer-resource type drops the kernel's launch stub.
__device__ __forceinline__ void load16_to_lds(const void* base, unsigned nbytes, void* lds,
                                              unsigned voffset, unsigned soffset)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)nbytes,
                                          0x00020000),
        (lds_void*)lds, 16, (int)voffset, (int)soffset, 0, 0);
}
__device__ __forceinline__ void load4_to_lds(const void* base, unsigned nbytes, void* lds,
                                             unsigned voffset, unsigned soffset)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)nbytes,
                                          0x00020000),
        (lds_void*)lds, 4, (int)voffset, (int)soffset, 0, 0);
}

// Row statistics a training forward keeps for its backward: the stage-1 L1
// norm S_i = sum_{j<=i} Softplus(s_ij) and the largest unmasked scaled score
// m_i, in natural units (the kernels work in base 2: t = s log2(e) and
// Softplus2(t) = Softplus(s) / ln 2).  ST is [rows, 2] doubles.
__device__ __forceinline__ void save_row_stats(double* ST, size_t row, double s1_base2,
                                               double tmax_base2)
{
    constexpr double kLn2 = 0.69314718055994530942;
    *reinterpret_cast<double2*>(ST + 2 * row) = make_double2(s1_base2 * kLn2, tmax_base2 * kLn2);
}

// The backward's read of them, back in base 2.
template <typename C>
__device__ __forceinline__ void load_row_stats(const double* ST, size_t row, C& s1_base2,
                                               C& tmax_base2)
{
    constexpr double kLog2e = 1.4426950408889634074;
    const double2 sv = *reinterpret_cast<const double2*>(ST + 2 * row);
    s1_base2 = (C)(sv.x * kLog2e);
    tmax_base2 = (C)(sv.y * kLog2e);
}

// PHI: stage-1 map; RW: false = stage 1 only (no pass 1, weights phi(t)).
// ST: null, or where the Softplus method stores each row's statistics.
// Tiles: two buffers of 64 keys at d = 64 and of 32 keys at d = 128, 33 KB
// of LDS either way, so four workgroups (4 waves per SIMD) fit a CU.  At
// d = 128 a 32-key tile costs a wave as many MFMAs as a 64-key tile at
// d = 64; 64-key tiles there allowed one buffer only (two need 66 KB and
// halve the occupancy), which left every tile load exposed.
//
// Scores.  The prep kernel writes fk_j = 1 / |k_j| and the KN16 rows, the
// normalised keys rounded to f16.  The operands are either
//  * fast: f16(lambda_i q_i / |q_i|) against KN16 on the f16 MFMA, both
//    factors folded in and each operand rounded to f16 once, so that
//    t = acc: no multiply per pair (two before the factors were folded in);
//    or
//  * exact: q_i against k_j, the raw bf16 rows, on the bf16 MFMA (the
//    products are exact in fp32), with t = acc * (fk_j * lambda_i / |q_i|):
//    the scores of the raw inputs with fp32 accumulation.
// The deep-row redo and the training forward (EXACT: its row statistics
// feed the backward) take the exact operands; the plain Softplus forward the
// fast ones.  The Sigmoid map takes the exact operands throughout: with a
// map bounded by 1 the gap sigma_max - tau is below 1, so nearly every row
// of a long sequence has kappa_i = p lambda_i / gap_i far above kCondMax
// (about 1600 at L = 8192, d = 64, p = 15) and would be computed twice.
template <int D, int P, int PHI, bool RW, bool EXACT>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(D == 64 ? 1 : 4))) void lssar_fwd_bf16_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
    const _Float16* __restrict__ KN16, const __bf16* __restrict__ V, __bf16* __restrict__ O,
    const float* __restrict__ FK, const int2* __restrict__ sched, int L, double lam_scale,
    float eps, int p_rt, double* __restrict__ ST)
{
    static_assert(D == 64 || D == 128, "head dim");
    constexpr int BK = D == 64 ? 64 : 32;      // keys per tile
    using T = Bf16Tile<D, BK>;
    constexpr int DC = D / 32;                 // MFMA k-steps over d
    constexpr int DS = D / 16;                 // 16-row blocks of O^T
    constexpr int KS = BK / 16;                // 16-key score blocks per tile
    constexpr int C2 = BK / 32;                // 32-key P.V steps per tile

    // One LDS object: the NB tile buffers, then the deep-row flags.  (A
    // second __shared__ object makes the compiler wait for the in-flight
    // LDS-direct loads before every LDS read in the tile loops.)
    constexpr int NB = 2;
    __shared__ __attribute__((aligned(1024))) unsigned char lds[NB * T::BYTES + 16];
    auto smem = [&](int buf) { return lds + buf * T::BYTES; };
    int* const flags = reinterpret_cast<int*>(lds + NB * T::BYTES);

    const int tid = threadIdx.x;
    // wave index in a scalar register, so per-wave decisions are uniform branches
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int row16 = lane & 15, grp = lane >> 4;
    // one query block per workgroup, from the prep kernel's table: XCD-local
    // slices of the heads, the largest block first within each
    // (lssar_sched.hpp); an empty index exits
    const int2 it = sched[blockIdx.x];
    const int bh = it.x, qb = it.y;
    if (bh < 0)
        return;
    const size_t hoff = (size_t)bh * L * D;
    const __bf16* Qh = Q + hoff;
    __bf16* Oh = O + hoff;

    // this head's K (raw and normalised), V and key factors; buffer reads
    // past them return zeros
    const void* kbase = K + hoff;
    const void* knbase = EXACT ? kbase : KN16 + hoff;
    const unsigned kbytes = (unsigned)L * D * 2u;
    const void* vbase = V + hoff;
    const void* fbase = FK + (size_t)bh * L;
    const unsigned fbytes = (unsigned)L * 4u;

    // per-lane byte offsets (within a tile) of the 16-byte slots this lane loads
    int kld[T::KLOADS], vld[T::VLOADS];
#pragma unroll
    for (int n = 0; n < T::KLOADS; ++n) {
        const int slot = (wave * T::KLOADS + n) * 64 + lane;
        const int key = slot / T::R, c = (slot % T::R) ^ T::kswz(key);
        kld[n] = (key * D + c * 8) * 2;
    }
#pragma unroll
    for (int n = 0; n < T::VLOADS; ++n) {
        const int slot = (wave * T::VLOADS + n) * 64 + lane;
        const int key = slot / T::R, c = (slot % T::R) ^ T::vswz(key);
        vld[n] = (key * D + c * 8) * 2;
    }
    // per-lane LDS byte offsets of the MFMA operand slots (16 ks key rows
    // further on are constant offsets)
    int krd[DC], vrd[DS];
#pragma unroll
    for (int dc = 0; dc < DC; ++dc)
        krd[dc] = (row16 * T::R + ((4 * dc + grp) ^ T::kswz(row16))) * 16;
    // V by the transpose read: lane j of group grp names key 4 grp + j / 4
    // (plus 16 h + 32 c2) and dims 16 ds + 4 (j % 4) .. + 3, and receives
    // keys 4 grp .. 4 grp + 3 of dim 16 ds + j; the swizzle depends on the
    // key mod 16 only
    {
        const int x = 4 * grp + (row16 >> 2);
        const int X = ((row16 >> 1) & 1) ^ T::vswz(x);
#pragma unroll
        for (int ds = 0; ds < DS; ++ds)
            vrd[ds] = T::KBYTES + (x * T::R + ((2 * ds) ^ X)) * 16 + (row16 & 1) * 8;
    }

    // fast: the normalised keys and no key factors
    auto issue = [&](int kt, int buf, bool with_v, bool fast) {
        unsigned char* base = smem(buf);
#pragma unroll
        for (int n = 0; n < T::KLOADS; ++n)
            load16_to_lds(fast ? knbase : kbase, kbytes, base + (wave * T::KLOADS + n) * 1024,
                          kld[n], kt * BK * D * 2);
        if (with_v) {
#pragma unroll
            for (int n = 0; n < T::VLOADS; ++n)
                load16_to_lds(vbase, kbytes, base + T::KBYTES + (wave * T::VLOADS + n) * 1024,
                              vld[n], kt * BK * D * 2);
        }
        if (wave == 0 && !fast)
            load4_to_lds(fbase, fbytes, base + T::KBYTES + T::VBYTES, lane * 4, kt * BK * 4);
    };

    const __bf16 one = (__bf16)1.0f;
    const bf16x8 ones = {one, one, one, one, one, one, one, one};
    // the block's deep-row flag; the block's first barrier orders this store
    // before any lane sets it, and it is read after a barrier that follows
    // the block
    if (tid == 0)
        flags[0] = 0;
    // this lane's row asked for the redo: a redone block stores only such
    // rows, so that a row's output depends on its own keys alone (rows that
    // did not ask keep the first pass's results; which rows of a block ask
    // depends on later keys, and the two passes round differently)
    bool redo_me = false;

    // The query block; REDO: computed again from the exact query operand,
    // and for Softplus with softplus2_acc (deep or ill-conditioned rows).
    auto block_body = [&](auto redo_tag) {
        constexpr bool REDO = decltype(redo_tag)::value;
        // operands (see above)
        constexpr bool FAST = !REDO && !EXACT && PHI == kPhiSoftplus;
        const int q0 = qb * kBQ16;
        const int qw0 = q0 + wave * kMQ16;         // first query row of this wave
        const int qwl = min(qw0 + kMQ16 - 1, L - 1);  // last valid query row
        const bool wave_active = qw0 < L;
        // key tiles up to the block's last row; tiles from kdiag on reach
        // into the block (one at d = 64, up to two at d = 128)
        const int ntiles = (min(L, q0 + kBQ16) + BK - 1) / BK;
        const int kdiag = q0 / BK;
        const int qi = qw0 + row16;                // this lane's query row (0-based)

        // ---- query rows: B operand of S^T = K Q^T, and the row factor ----
        std::conditional_t<FAST, f16x8, bf16x8> qf[DC];
        float lam = 0.0f;
        float lam_row;                             // lambda_i = log2(e) ln d ln i
        {
            float ss = 0.0f;
            u32x4 w[DC];
#pragma unroll
            for (int dc = 0; dc < DC; ++dc) {
                w[dc] = u32x4{0u, 0u, 0u, 0u};
                if (qi < L)
                    w[dc] = *reinterpret_cast<const u32x4*>(Qh + (size_t)qi * D + 32 * dc + 8 * grp);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float a = bf16lo(w[dc][e]), b = bf16hi(w[dc][e]);
                    ss = __builtin_fmaf(a, a, ss);
                    ss = __builtin_fmaf(b, b, ss);
                }
            }
            ss += __shfl_xor(ss, 16);
            ss += __shfl_xor(ss, 32);
            // log2(e) ln d ln i / max(|q_i|, 1e-12)  (Key design 1: log d . log N)
            // in fp32: a few ulp of lambda_i against the fp32 scores' (d + 3)
            // ulp of ln d ln i; the fp64 log and divide cost a block about
            // 100 double-precision instructions per wave, noticeable on rows
            // of a few tiles
            constexpr float kLn2 = 0.693147180559945309f;
            lam_row = (float)lam_scale * (__builtin_amdgcn_logf((float)(qi + 1)) * kLn2);
            const float lamf = lam_row / fmaxf(sqrtf(ss), 1e-12f);
            // fast: lambda_i q^_i rounded to f16; exact: q_i itself and the
            // factor lambda_i / |q_i| applied to the accumulator
            if constexpr (FAST) {
#pragma unroll
                for (int dc = 0; dc < DC; ++dc)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        qf[dc][2 * e] = (_Float16)(bf16lo(w[dc][e]) * lamf);
                        qf[dc][2 * e + 1] = (_Float16)(bf16hi(w[dc][e]) * lamf);
                    }
            } else {
                lam = lamf;
#pragma unroll
                for (int dc = 0; dc < DC; ++dc)
                    qf[dc] = __builtin_bit_cast(bf16x8, w[dc]);
            }
        }

        // scores of 16-key block ks: acc[r] = k_(16ks+4grp+r) . q_(row16)
        auto qk_block = [&](const unsigned char* base, int ks) {
            f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int dc = 0; dc < DC; ++dc) {
                const unsigned char* a = base + krd[dc] + ks * 16 * T::R * 16;
                if constexpr (FAST)
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                        *reinterpret_cast<const f16x8*>(a), qf[dc], acc, 0, 0, 0);
                else
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        *reinterpret_cast<const bf16x8*>(a), qf[dc], acc, 0, 0, 0);
            }
            return acc;
        };
        // t = acc (fast) or acc * lam * f_key (exact); masked (t = -inf) on
        // diagonal tiles
        auto scale_block = [&](int kt, const unsigned char* base, int ks, f32x4 acc, bool diag) {
            f32x4 t;
            if constexpr (FAST) {
                t = acc;
            } else {
                const f32x4 f4 = *reinterpret_cast<const f32x4*>(
                    base + T::KBYTES + T::VBYTES + (16 * ks + 4 * grp) * 4);
                t = acc * (f4 * lam);
            }
            if (diag) {
                const int k0 = kt * BK + 16 * ks + 4 * grp;
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    t[r] = (k0 + r <= qi) ? t[r] : -INFINITY;
            }
            return t;
        };

        auto row_sum = [](float x) {
            x += __shfl_xor(x, 16);
            return x + __shfl_xor(x, 32);
        };
        auto row_max = [](float x) {
            x = fmaxf(x, __shfl_xor(x, 16));
            return fmaxf(x, __shfl_xor(x, 32));
        };

        // 16-key blocks of tile kt with a key at or before the wave's last
        // row (0 when the whole tile lies after it)
        auto diag_blocks = [&](int kt) {
            const int rel = qwl - kt * BK;
            return rel < 0 ? 0 : min(KS, rel / 16 + 1);
        };

        // ---------------- pass 1: S1 and the row max of the scores ----------------
        float s1 = 0.0f;
        float tmax = -INFINITY;
        // kPass1Prod: the running product of the factors 1 + 2^t as a
        // mantissa pm in [0.5, 1) and an exponent pe
        float pm = 1.0f;
        int pe = 0;
        auto pass1_tile = [&](int kt, const unsigned char* base, auto diag_tag, auto kind_tag) {
            constexpr bool DIAG = decltype(diag_tag)::value;
            constexpr int KIND = decltype(kind_tag)::value;
            // 16-key blocks with at least one key <= the wave's last row
            const int nks = DIAG ? diag_blocks(kt) : KS;
            f32x4 acc[KS];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                if (!DIAG || ks < nks)
                    acc[ks] = qk_block(base, ks);
            float pos_sum = 0.0f, prod = 1.0f;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                if (DIAG && ks >= nks)
                    continue;
                const f32x4 t = scale_block(kt, base, ks, acc[ks], DIAG);
                if constexpr (KIND == kPass1Acc) {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        pos_sum += softplus2_acc(t[r]);
                    tmax = max3_scores(tmax, t[0], t[1]);
                    tmax = max3_scores(tmax, t[2], t[3]);
                } else if constexpr (KIND == kPass1Prod) {
                    // log2(1 + 2^t) summed as log2 of the product of the
                    // factors, renormalised after every two of them (each
                    // at most 2^kProdMaxT + 1): one exp2 and one fma per
                    // pair, no max and add for the positive part
#pragma unroll
                    for (int r = 0; r < 4; r += 2) {
                        const float u0 = __builtin_amdgcn_exp2f(t[r]);
                        const float u1 = __builtin_amdgcn_exp2f(t[r + 1]);
                        pm = __builtin_fmaf(pm, u0, pm);
                        pm = __builtin_fmaf(pm, u1, pm);
                        pe += __builtin_amdgcn_frexp_expf(pm);
                        pm = __builtin_amdgcn_frexp_mantf(pm);
                    }
                    tmax = max3_scores(tmax, t[0], t[1]);
                    tmax = max3_scores(tmax, t[2], t[3]);
                } else if constexpr (PHI == kPhiSoftplus) {
                    f32x4 u;
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        u[r] = __builtin_amdgcn_exp2f(-fabsf(t[r]));
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        pos_sum += max_scores(t[r], 0.0f);
                    tmax = max3_scores(tmax, t[0], t[1]);
                    tmax = max3_scores(tmax, t[2], t[3]);
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        prod = __builtin_fmaf(prod, u[r], prod);
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        pos_sum += sigmoid2(t[r]);
                    tmax = max3_scores(tmax, t[0], t[1]);
                    tmax = max3_scores(tmax, t[2], t[3]);
                }
            }
            if constexpr (KIND == kPass1Sum && PHI == kPhiSoftplus)
                s1 += pos_sum + __builtin_amdgcn_logf(prod);
            else
                s1 += pos_sum;
        };
        // Tiles 0..ntiles-1 of K (and V^T) through LDS; body runs on every
        // tile that reaches the wave's rows (diagonal tiles masked).
        // Tiles 0..kdiag-1 lie wholly before every row of the block and the
        // rest hold its diagonal, so the loop runs the unmasked body and the
        // diagonal tiles follow it: with both bodies inside the loop, their
        // accumulators were copied back at every iteration (20 moves per
        // tile in pass 2).
        // Tile kt goes to buffer (kt + kdiag) & 1, so that the (first)
        // diagonal tile lands in buffer 0, and the loop runs two tiles per
        // iteration: every buffer index is then a constant, and the LDS
        // reads take the buffer's offset as an immediate (with the index
        // kt & 1 each tile paid a vector add per operand address).
        auto tile_loop = [&](bool with_v, auto body) {
            auto step = [&](int kt, auto buf_tag, auto diag_tag) {
                constexpr int buf = decltype(buf_tag)::value;
                __builtin_amdgcn_s_waitcnt(0);
                __syncthreads();                   // tile kt landed; buf^1 free
                if (kt + 1 < ntiles)
                    issue(kt + 1, buf ^ 1, with_v, FAST);
                if (wave_active)
                    body(kt, smem(buf), diag_tag);
            };
            using B0 = std::integral_constant<int, 0>;
            using B1 = std::integral_constant<int, 1>;
            __syncthreads();                       // earlier readers done with the buffers
            const bool odd = (kdiag & 1) != 0;
            issue(0, odd ? 1 : 0, with_v, FAST);
            int kt = 0;
            if (odd) {
                step(0, B1{}, std::false_type{});
                kt = 1;
            }
            for (; kt < kdiag; kt += 2) {          // kdiag - kt is even here
                step(kt, B0{}, std::false_type{});
                step(kt + 1, B1{}, std::false_type{});
            }
            step(kdiag, B0{}, std::true_type{});   // the diagonal tile(s)
            if constexpr (BK != kBQ16) {
                // 32-key tiles: the block's 64 rows span at most two
                if (kdiag + 1 < ntiles)
                    step(kdiag + 1, B1{}, std::true_type{});
            }
        };
        auto run_pass1 = [&](auto kind_tag) {
            tile_loop(false, [&](int kt, const unsigned char* base, auto diag_tag) {
                pass1_tile(kt, base, diag_tag, kind_tag);
            });
        };

        constexpr bool ACC = REDO && PHI == kPhiSoftplus;   // softplus2_acc
        RowConst rc = {0.0f, 0.0f, false};
        if constexpr (RW) {
            if constexpr (ACC) {
                run_pass1(std::integral_constant<int, kPass1Acc>{});
            } else if constexpr (PHI == kPhiSoftplus && (FAST || D == 64)) {
                // every score of the block is at most about lambda of its
                // last row (|q^ . k^| <= 1): the product form when that
                // stays within kProdMaxT (wave-uniform).  (The training
                // forward at d = 128 keeps the other form: with both, its
                // kernel spills 12 bytes per lane at 128 VGPRs.)
                constexpr float kLn2 = 0.693147180559945309f;
                const float lam_last = (float)lam_scale *
                    (__builtin_amdgcn_logf((float)min(L, q0 + kBQ16)) * kLn2);
                if (__builtin_amdgcn_readfirstlane((int)(lam_last <= kProdMaxT))) {
                    run_pass1(std::integral_constant<int, kPass1Prod>{});
                    s1 = __builtin_amdgcn_logf(pm) + (float)pe;
                } else {
                    run_pass1(std::integral_constant<int, kPass1Sum>{});
                }
            } else {
                run_pass1(std::integral_constant<int, kPass1Sum>{});
            }
            const float trow = row_max(tmax);
            const float s1r = row_sum(s1);
            if constexpr (ACC) {
                rc = row_constants_sp(qi + 1, s1r, softplus2_acc(trow), eps);
            } else {
                rc = row_constants<PHI>(qi + 1, s1r, trow, eps);
                if constexpr (PHI == kPhiSoftplus && !REDO)
                    if (qi < L && trow < kDeep) {
                        flags[0] = 1;
                        redo_me = true;
                    }
            }
            // kappa_i = p lambda_i c_i
            if constexpr (FAST) {
                const float pf = (float)(P > 0 ? P : p_rt);
                if (qi < L && pf * lam_row * rc.c > kCondMax) {
                    flags[0] = 1;
                    redo_me = true;
                }
            }
            // a redone block stores its asking rows again, after their
            // first store
            if constexpr (PHI == kPhiSoftplus)
                if (ST && qi < L && grp == 0 && (!REDO || redo_me))
                    save_row_stats(ST, (size_t)bh * L + qi, s1r, trow);
        }

        // ---------------- pass 2: re-weight, P.V and the weight sum ----------------
        f32x4 oacc[DS];
#pragma unroll
        for (int ds = 0; ds < DS; ++ds)
            oacc[ds] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        f32x4 dacc = {0.0f, 0.0f, 0.0f, 0.0f};

        auto weights = [&](f32x4 t) {
            f32x4 e, w;
            if constexpr (ACC) {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    e[r] = softplus2_acc(t[r]);
            } else if constexpr (PHI == kPhiSoftplus) {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    e[r] = __builtin_amdgcn_exp2f(t[r]);
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    e[r] = __builtin_amdgcn_logf(1.0f + e[r]);   // Softplus2
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    e[r] = sigmoid2(t[r]);
            }
            if constexpr (!RW)
                return e;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                w[r] = pow_chain<P>(reweight_arg(e[r], rc.c, rc.tc), p_rt);
            return w;
        };

        auto pass2_tile = [&](int kt, const unsigned char* base, auto diag_tag) {
            constexpr bool DIAG = decltype(diag_tag)::value;
            const int nks = DIAG ? diag_blocks(kt) : KS;
            f32x4 acc[KS];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                if (!DIAG || ks < nks)
                    acc[ks] = qk_block(base, ks);
#pragma unroll
            for (int c2 = 0; c2 < C2; ++c2) {
                if (DIAG && 2 * c2 >= nks)
                    continue;
                const f32x4 w0 = weights(scale_block(kt, base, 2 * c2, acc[2 * c2], DIAG));
                const f32x4 w1 =
                    (!DIAG || 2 * c2 + 1 < nks)
                        ? weights(scale_block(kt, base, 2 * c2 + 1, acc[2 * c2 + 1], DIAG))
                        : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
                const bf16x4 lo = __builtin_convertvector(w0, bf16x4);
                const bf16x4 hi = __builtin_convertvector(w1, bf16x4);
                const bf16x8 bfr = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
                for (int ds = 0; ds < DS; ++ds) {
                    // keys 32 c2 + 4 grp + 0..3, then 32 c2 + 16 + 4 grp + 0..3
                    // of dim 16 ds + row16: the order of bfr
                    const unsigned char* vp = base + vrd[ds] + 32 * c2 * T::R * 16;
                    const bf16x4 v0 = lds_read_tr16(vp), v1 = lds_read_tr16(vp + 16 * T::R * 16);
                    const bf16x8 a = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
                    oacc[ds] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bfr, oacc[ds], 0, 0, 0);
                }
                dacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, bfr, dacc, 0, 0, 0);
            }
        };

        tile_loop(true, pass2_tile);
        if constexpr (!RW && PHI == kPhiSoftplus && !REDO)
            if (qi < L && dacc[0] < (float)(qi + 1) * kDeepMean) {
                flags[0] = 1;
                redo_me = true;
            }

        // ---------------- finalize: out_i = U_i / D_i (0 if degenerate) ----------------
        if (qi < L && (!REDO || redo_me)) {
            const float inv = rc.degen ? 0.0f : 1.0f / dacc[0];
#pragma unroll
            for (int ds = 0; ds < DS; ++ds) {
                const f32x4 o = oacc[ds] * inv;
                const bf16x4 ob = __builtin_convertvector(o, bf16x4);
                *reinterpret_cast<bf16x4*>(Oh + (size_t)qi * D + 16 * ds + 4 * grp) = ob;
            }
        }
    };

    block_body(std::false_type{});
    if constexpr (PHI == kPhiSoftplus) {
        __syncthreads();                           // every lane's flag store is done
        if (flags[0])
            block_body(std::true_type{});
    }
}

// ---------------------------------------------------------------------------
// fp32 attention kernel: the same two passes.  Scores come from
// v_mfma_f64_16x16x4_f64 on the exact fp32 inputs widened to fp64, and the
// score -> Softplus -> row sums -> re-weighting chain runs in fp64 (see
// softplus2_f64); the weights are rounded to fp32 once and P.V runs on
// v_mfma_f32_16x16x4_f32.  K and V stay row-major in LDS (one element per
// lane per MFMA operand); tiles are single-buffered.
// ---------------------------------------------------------------------------
template <int D, int P, int PHI, bool RW>
__global__ __launch_bounds__(kThreads, 1) void lssar_fwd_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K,
    const float* __restrict__ V, float* __restrict__ O,
    const double* __restrict__ FK, int BH, int L, int nqb, double lam_scale,
    float eps, int p_rt, double* __restrict__ ST)
{
    static_assert(D == 64 || D == 128, "head dim");
    constexpr int DK = D / 4;                  // MFMA k-steps over d
    constexpr int DS = D / 16;
    constexpr int KS = D + 4;                  // row stride (floats) for K and V tiles
    constexpr int CH = kBK * D / 4 / kThreads; // 16-byte chunks per thread per tile

    __shared__ __attribute__((aligned(16))) float Ks[kBK * KS];
    __shared__ __attribute__((aligned(16))) float Vs[kBK * KS];
    __shared__ __attribute__((aligned(16))) double Fs[kBK];

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int row16 = lane & 15, grp = lane >> 4;
    const int qb = nqb - 1 - (int)(blockIdx.x / BH);
    const int bh = (int)(blockIdx.x % BH);
    const int q0 = qb * kBQ32;
    const size_t hoff = (size_t)bh * L * D;
    const float* Qh = Q + hoff;
    const float* Kh = K + hoff;
    const float* Vh = V + hoff;
    float* Oh = O + hoff;
    const double* Fh = FK + (size_t)bh * L;

    const int qw0 = q0 + wave * kMQ32;
    const int qwl = min(qw0 + kMQ32 - 1, L - 1);
    const bool wave_active = qw0 < L;
    const int kend = min(q0 + kBQ32, L);
    const int ntiles = (kend + kBK - 1) / kBK;

    float qf[2][DK];
    int qi[2];
    double lam[2];
#pragma unroll
    for (int qs = 0; qs < 2; ++qs) {
        qi[qs] = qw0 + 16 * qs + row16;
        double ss = 0.0;
#pragma unroll
        for (int kk = 0; kk < DK; ++kk) {
            const float x = qi[qs] < L ? Qh[(size_t)qi[qs] * D + 4 * kk + grp] : 0.0f;
            qf[qs][kk] = x;
            ss = fma((double)x, (double)x, ss);
        }
        ss += __shfl_xor(ss, 16);
        ss += __shfl_xor(ss, 32);
        lam[qs] = query_factor(lam_scale, qi[qs] + 1, ss);
    }

    auto stage = [&](int kt, bool with_v) {
#pragma unroll
        for (int n = 0; n < CH; ++n) {
            const int c = tid + n * kThreads;
            const int key = c / (D / 4), col4 = c % (D / 4);
            const int kg = kt * kBK + key;
            const f32x4 z = {0.0f, 0.0f, 0.0f, 0.0f};
            *reinterpret_cast<f32x4*>(&Ks[key * KS + col4 * 4]) =
                kg < L ? *reinterpret_cast<const f32x4*>(Kh + (size_t)kg * D + col4 * 4) : z;
            if (with_v)
                *reinterpret_cast<f32x4*>(&Vs[key * KS + col4 * 4]) =
                    kg < L ? *reinterpret_cast<const f32x4*>(Vh + (size_t)kg * D + col4 * 4) : z;
        }
        if (tid < kBK) {
            const int kg = kt * kBK + tid;
            Fs[tid] = kg < L ? Fh[kg] : 0.0;
        }
    };

    // S^T block in fp64.  v_mfma_f64_16x16x4_f64 returns output row
    // 4 r + grp in register r (measured; the fp32/bf16 16x16 forms return
    // row 4 grp + r), so acc[ks][qs][r] = k_(16ks+grp+4r) . q_(16qs+row16).
    auto key_of = [&](int ks, int r) { return 16 * ks + grp + 4 * r; };
    auto qk_tile = [&](f64x4 (&acc)[4][2]) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
            for (int qs = 0; qs < 2; ++qs)
                acc[ks][qs] = f64x4{0.0, 0.0, 0.0, 0.0};
#pragma unroll
        for (int kk = 0; kk < DK; ++kk) {
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const double a = Ks[(16 * ks + row16) * KS + 4 * kk + grp];
#pragma unroll
                for (int qs = 0; qs < 2; ++qs)
                    acc[ks][qs] = __builtin_amdgcn_mfma_f64_16x16x4f64(a, (double)qf[qs][kk],
                                                                       acc[ks][qs], 0, 0, 0);
            }
        }
    };

    // pass 1 (both stages only)
    RowConstD rc[2] = {{0.0, 0.0, false}, {0.0, 0.0, false}};
    if constexpr (RW) {
        double s1[2] = {0.0, 0.0};
        double tmax[2] = {-INFINITY, -INFINITY};
        for (int kt = 0; kt < ntiles; ++kt) {
            __syncthreads();
            stage(kt, false);
            __syncthreads();
            if (!(wave_active && kt * kBK <= qwl))
                continue;
            f64x4 acc[4][2];
            qk_tile(acc);
            double part[2] = {0.0, 0.0};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
                for (int qs = 0; qs < 2; ++qs) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int key = key_of(ks, r);
                        const bool ok = kt * kBK + key <= qi[qs];
                        if (ok) {
                            const double t = acc[ks][qs][r] * (lam[qs] * Fs[key]);
                            part[qs] += phi2_f64<PHI>(t);
                            tmax[qs] = fmax(tmax[qs], t);
                        }
                    }
                }
            }
            s1[0] += part[0];
            s1[1] += part[1];
        }
#pragma unroll
        for (int qs = 0; qs < 2; ++qs) {
            double s = s1[qs];
            s += __shfl_xor(s, 16);
            s += __shfl_xor(s, 32);
            double t = tmax[qs];
            t = fmax(t, __shfl_xor(t, 16));
            t = fmax(t, __shfl_xor(t, 32));
            rc[qs] = row_constants_f64<PHI>(qi[qs] + 1, s, t, eps);
            if constexpr (PHI == kPhiSoftplus)
                if (ST && qi[qs] < L && grp == 0)
                    save_row_stats(ST, (size_t)bh * L + qi[qs], s, t);
        }
    }

    // pass 2
    f32x4 oacc[DS][2];
#pragma unroll
    for (int ds = 0; ds < DS; ++ds)
#pragma unroll
        for (int qs = 0; qs < 2; ++qs)
            oacc[ds][qs] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    float dsum[2] = {0.0f, 0.0f};
    for (int kt = 0; kt < ntiles; ++kt) {
        __syncthreads();
        stage(kt, true);
        __syncthreads();
        if (!(wave_active && kt * kBK <= qwl))
            continue;
        f64x4 acc[4][2];
        qk_tile(acc);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            float w[2][4];
#pragma unroll
            for (int qs = 0; qs < 2; ++qs) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int key = key_of(ks, r);
                    const bool ok = kt * kBK + key <= qi[qs];
                    float wv = 0.0f;
                    if (ok) {
                        const double t = acc[ks][qs][r] * (lam[qs] * Fs[key]);
                        if constexpr (RW) {
                            double y = phi2_f64<PHI>(t) * rc[qs].c - rc[qs].tc;
                            y = fmin(fmax(y, 0.0), 1.0);
                            wv = (float)pow_chain<P>(y, p_rt);
                        } else {
                            wv = (float)phi2_f64<PHI>(t);
                        }
                    }
                    w[qs][r] = wv;
                    dsum[qs] += wv;
                }
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
#pragma unroll
                for (int ds = 0; ds < DS; ++ds) {
                    // P.V step r: k-slot grp carries key key_of(ks, r)
                    const float a = Vs[key_of(ks, r) * KS + 16 * ds + row16];
#pragma unroll
                    for (int qs = 0; qs < 2; ++qs)
                        oacc[ds][qs] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, w[qs][r],
                                                                            oacc[ds][qs], 0, 0, 0);
                }
            }
        }
    }

#pragma unroll
    for (int qs = 0; qs < 2; ++qs) {
        float s = dsum[qs];
        s += __shfl_xor(s, 16);
        s += __shfl_xor(s, 32);
        if (qi[qs] >= L)
            continue;
        const float inv = rc[qs].degen ? 0.0f : 1.0f / s;
#pragma unroll
        for (int ds = 0; ds < DS; ++ds) {
            const f32x4 o = oacc[ds][qs] * inv;
            *reinterpret_cast<f32x4*>(Oh + (size_t)qi[qs] * D + 16 * ds + 4 * grp) = o;
        }
    }
}

}  // namespace lssar
