// lssar_bwd_mfma.hpp -- matrix-core kernels of the LSSAR backward for bf16
// inputs on gfx950.
//
// The gradient formulas are those of lssar_bwd.hpp (the chain rule through
// Key designs 1-3 of the paper note "Softplus Attention with Re-weighting
// Boosts Length Extrapolation in Large Language Models", Method details);
// these kernels evaluate them on the matrix cores:
//   prep:     key factors f_j = 1/|k_j| and query factors 1/|q_i|;
//   rowstats: per query block, the scores S^T = K Q^T and dW^T = V dO^T on
//             v_mfma_f32_16x16x32_bf16, pass 1 the row's S and max score,
//             pass 2 the sums Y, P1, P2, Z; writes the row coefficients
//             with u = Y^(-1/p): (c u, tau c u, A Y u/|q|, -delta A Y u/|q|,
//             E/|q|, the score factor, -, the largest score).  With them
//             y' = clamp((sp - tau) c u, 0, 1) = y u, the weight y^p / Y is
//             y'^p, and the pair gradient sigma (y^(p-1) (A dW - A delta) -
//             E) is sigma (y'^(p-1) (A Y u dW - A Y u delta) - E): two fma
//             and a multiply;
//   dq:       per query block, S^T, dW^T, the pair gradients dc_ij f_j, and
//             dQ^ = (dc f) K on v_mfma_f32_16x16x16_bf16, whose output
//             layout (lane = one query, four keys) is exactly its A operand;
//   one pass (d = 64, from a training forward's row statistics and output):
//             rowstats' second pass and dq together, the row coefficients
//             applied to accumulated vectors at the end;
//   dkdv:     per key block, S = Q K^T and dW = dO V^T (lane = one key, four
//             queries), then dV = W^T dO and dK^ = (dc / |q|)^T Q on
//             v_mfma_f32_16x16x16_bf16.
// A workgroup is 4 waves x 16 rows (queries, or keys in dkdv) of a 64-row
// block; at d = 64 paired blocks {n-1-pi, pi} give every workgroup the same
// number of 64-row tiles, at d = 128 single blocks run largest first in the
// forward's XCD-local order (bwd_blocks).  Tiles of the other side stream
// through LDS by LDS-direct buffer loads, row-major only: the 16x16x16 B
// operands (K in dq, Q and dO in dkdv; four consecutive rows of one dim)
// come from the same tiles by the LDS transpose read (ds_read_b64_tr_b16).
// Softplus is exact (softplus2_acc, or sp_sig with its derivative from the
// same exp2), except that query blocks without a deep row take plain
// log2(1 + 2^t), the forward's rule, and at d = 64 so do key blocks whose
// query blocks have none (at every p: p = 3 training backward 139 -> 129 us
// at B8 H12 L1024, recomputing 178 -> 164 us; the query side at d = 128:
// B2 H32 L4096 p = 15 training backward 1864 -> 1813 us, recomputing
// 2067 -> 2014 us, gradients bitwise unchanged).
#pragma once

#include "lssar_bwd.hpp"
#include "lssar_device.hpp"

namespace lssar {


// Softplus2(t) (exact for every t, as softplus2_acc) and its derivative
// sigma(t ln 2) = e / (1 + e), e = 2^t, from one exp2.
__device__ __forceinline__ void sp_sig(float t, float& sp, float& sig)
{
    constexpr float kLog2e = 1.4426950408889634f;
    const float e = __builtin_amdgcn_exp2f(t);
    const float ope = 1.0f + e;
    const float series = e * __builtin_fmaf(-0.5f * kLog2e, e, kLog2e);
    sp = e < (1.0f / 256.0f) ? series : __builtin_amdgcn_logf(ope);
    sig = e * __builtin_amdgcn_rcpf(ope);
}

// The same with Softplus2 as plain log2(1 + 2^t), the forward's evaluation
// for rows whose largest score is at least kDeep: there it differs from the
// exact value only where 2^t < 1/256, by at most 2^-24 log2(e) absolute,
// and such scores lie far below the row's largest.
__device__ __forceinline__ void sp_sig_plain(float t, float& sp, float& sig)
{
    const float e = __builtin_amdgcn_exp2f(t);
    const float ope = 1.0f + e;
    sp = __builtin_amdgcn_logf(ope);
    sig = e * __builtin_amdgcn_rcpf(ope);
}

// Four fp32 values as the bf16 operand of the 16x16x16 MFMA (round to
// nearest even).  Packed two by two into 32-bit words: a bf16x4 bit-cast to
// the operand type compiles to one conversion per element plus merges.
__device__ __forceinline__ s16x4 pack_bf16x4(f32x4 x)
{
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
    const bf16x2 lo = __builtin_convertvector(f32x2{x[0], x[1]}, bf16x2);
    const bf16x2 hi = __builtin_convertvector(f32x2{x[2], x[3]}, bf16x2);
    const u32x2 u = {__builtin_bit_cast(unsigned, lo), __builtin_bit_cast(unsigned, hi)};
    return __builtin_bit_cast(s16x4, u);
}

__device__ __forceinline__ f32x4 mfma16k16(s16x4 a, bf16x4 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
}

// Two 16x16x16 products into one accumulator, a0 b0 + a1 b1, as one
// 16x16x32: each lane's eight k-slots hold its four of the first product
// and then its four of the second, on both operands alike.  On gfx950 the
// 16x16x16 instruction takes as many cycles as the 16x16x32.
__device__ __forceinline__ f32x4 mfma16k16x2(s16x4 a0, s16x4 a1, bf16x4 b0, bf16x4 b1, f32x4 c)
{
    const bf16x8 a = __builtin_shufflevector(__builtin_bit_cast(bf16x4, a0),
                                             __builtin_bit_cast(bf16x4, a1), 0, 1, 2, 3, 4, 5, 6, 7);
    const bf16x8 b = __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// LDS layout of one 64-row tile: 64 rows x D bf16 as 16-byte slots, slot
// c of row r at r * R + (c ^ swz(r)), R = D / 8.  The 16x16x32 A operands
// read 16-byte slots of 16 rows; the 16x16x16 B operands (four consecutive
// rows of one dim) come from the same tile by the LDS transpose read.  The
// swizzle serves both: in-bounds microbenchmarks of the two read patterns
// on gfx950 timed the row reads equal to the best of the candidates tried
// and the transpose reads 1.4x (d = 64) and 1.5x (d = 128) faster than with
// swz = (r >> 1) & 7 and r & 15.  It depends on r mod 16 only.
template <int D>
struct BwdTiles {
    static constexpr int R = D / 8;
    static constexpr int RM = 64 * D * 2;        // bytes of a tile
    static constexpr int RM_LOADS = RM / 1024 / kWaves;   // wave-loads per wave
    __device__ static int swz(int r)
    {
        return R == 8 ? (r & 7) : ((((r & 3) << 2) | ((r >> 2) & 3)) ^ ((r >> 1) & 2));
    }
};

// Bytes of the tile's 16-byte slot s in the global tensor [rows][D] (row
// stride D*2).
template <int D>
__device__ __forceinline__ unsigned rm_src(int s)
{
    using T = BwdTiles<D>;
    const int r = s / T::R, c = (s % T::R) ^ T::swz(r);
    return (unsigned)((r * D + c * 8) * 2);
}

// The 64-row blocks of head bh that a workgroup w takes, the one with more
// work first (b1 < 0: one block).  Block b of the query side has the work of
// b + 1 key tiles, key block b of the key side that of nb - b query tiles.
//  d = 64: the pair {pi, nb - 1 - pi} (equal work for every workgroup), in
//          the XCD-local order of xcd_item; npair * BH workgroups.
//  d = 128: one block per workgroup, in the forward's dispatch order
//          (FwdSched: balanced slices of heads per XCD, largest block first),
//          FwdSched(BH, nb).grid() workgroups; false for an empty index.
//  (At d = 128, 3 waves per SIMD, the smaller workgroups ended the key-side
//  kernel 2.7% sooner; at d = 64 the pairs were faster.)
template <int D>
__device__ __forceinline__ bool bwd_blocks(int w, int BH, int nb, bool key_side, int& bh, int& b0,
                                           int& b1)
{
    if constexpr (D == 64) {
        const int npair = (nb + 1) / 2;
        const int item = xcd_item(w, npair * BH);
        bh = item / npair;
        const int pi = item % npair;
        b0 = key_side ? pi : nb - 1 - pi;
        b1 = pi == nb - 1 - pi ? -1 : nb - 1 - b0;
        return true;
    } else {
        int qbx;
        if (!FwdSched(BH, nb).item(w, bh, qbx))
            return false;
        b0 = key_side ? nb - 1 - qbx : qbx;
        b1 = -1;
        return true;
    }
}

// ---------------------------------------------------------------------------
// Prep: row factors, one workgroup per (64-row block, head)
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreads) void lssar_bwd_prep_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, float* __restrict__ rq,
    float* __restrict__ fk, int L)
{
    constexpr int LPR = D / 8;
    const int kb = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
    const size_t hoff = (size_t)bh * L * D;

    // factors 1 / max(|x|, 1e-12) of the block's Q and K rows (fp64 sums)
#pragma unroll
    for (int n = 0; n < 64 * LPR / kThreads; ++n) {
        const int c = tid + n * kThreads;
        const int row = c / LPR, sub = c % LPR;
        const int rg = kb * 64 + row;
        double sq = 0.0, sk = 0.0;
        if (rg < L) {
            const u32x4 wq = *reinterpret_cast<const u32x4*>(Q + hoff + (size_t)rg * D + sub * 8);
            const u32x4 wk = *reinterpret_cast<const u32x4*>(K + hoff + (size_t)rg * D + sub * 8);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const double a = bf16lo(wq[e]), b = bf16hi(wq[e]);
                const double x = bf16lo(wk[e]), y = bf16hi(wk[e]);
                sq = fma(a, a, fma(b, b, sq));
                sk = fma(x, x, fma(y, y, sk));
            }
        }
#pragma unroll
        for (int m = LPR / 2; m >= 1; m >>= 1) {
            sq += __shfl_xor(sq, m, LPR);
            sk += __shfl_xor(sk, m, LPR);
        }
        if (rg < L && sub == 0) {
            rq[(size_t)bh * L + rg] = (float)(1.0 / fmax(sqrt(sq), 1e-12));
            fk[(size_t)bh * L + rg] = (float)(1.0 / fmax(sqrt(sk), 1e-12));
        }
    }
}

// ---------------------------------------------------------------------------
// Query-side kernels (rowstats, dq): lane (row16, grp) owns query row16 of its
// wave and keys 16 ks + 4 grp + r of each 16-key block ks of a tile.
// ---------------------------------------------------------------------------

// MODE 0: rowstats (writes 8 coefficients per query row; saved: null, or
// the training forward's row statistics, which replace pass 1); MODE 1: dq
// (reads the coefficients); MODE 2 (d = 64): both in one pass, from the
// training forward's row statistics (saved) and output (O).
// One key-tile buffer in LDS: a double-buffered loop measured slower, since
// its LDS and registers cost workgroups per CU that hide the loads better.
// MODE 2 keeps three d-wide accumulators and four row sums beside the
// scores; capped for 3 waves per SIMD it fits without spills (164 VGPRs)
// and runs faster than at 2 (x8 9% faster; and faster than MODE 0 +
// MODE 1).  At d = 128 the accumulators alone take 96 VGPRs, and the
// two-kernel path is faster.
template <int D, int P, int MODE>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(MODE == 2 ? 3 : 1))) void lssar_bwd_qside_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    const __bf16* __restrict__ G, const float* __restrict__ rq, const float* __restrict__ fk,
    float* __restrict__ stats, __bf16* __restrict__ dQ, int BH, int L, int nqb, int npair,
    double lam_scale, float eps, int p_rt,
    const double* __restrict__ saved, const __bf16* __restrict__ O)
{
    static_assert(D == 64 || D == 128, "head dim");
    static_assert(MODE != 2 || D == 64, "the one-pass mode is for d = 64");
    using T = BwdTiles<D>;
    constexpr int DC = D / 32;                 // 32-deep MFMA steps over d
    constexpr int DS = D / 16;                 // 16-wide output blocks over d
    constexpr int KOFF = 0, VOFF = T::RM;
    constexpr int FOFF = 2 * T::RM;
    constexpr int BYTES = FOFF + 256;
    // one LDS object: the tiles, then (MODE 0, 2) the block's deep-row flag
    __shared__ __attribute__((aligned(1024))) unsigned char lds[BYTES + 16];
    int* const deep_flag = reinterpret_cast<int*>(lds + BYTES);

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, row16 = lane & 15, grp = lane >> 4;
    int bh, blk0, blk1;
    if (!bwd_blocks<D>((int)blockIdx.x, BH, nqb, false, bh, blk0, blk1))
        return;
    const size_t hoff = (size_t)bh * L * D;

    const void* kbase = K + hoff;
    const void* vbase = V + hoff;
    const unsigned rmbytes = (unsigned)L * D * 2u;
    const void* fbase = fk + (size_t)bh * L;
    const unsigned fbytes = (unsigned)L * 4u;

    int rm_ld[T::RM_LOADS];
#pragma unroll
    for (int n = 0; n < T::RM_LOADS; ++n)
        rm_ld[n] = (int)rm_src<D>((wave * T::RM_LOADS + n) * 64 + lane);

    // tile kt of K (and V as the pass needs) into LDS
    auto issue = [&](int kt, bool with_v) {
        unsigned char* base = lds;
#pragma unroll
        for (int n = 0; n < T::RM_LOADS; ++n)
            load16_to_lds(kbase, rmbytes, base + KOFF + (wave * T::RM_LOADS + n) * 1024, rm_ld[n],
                          kt * 64 * D * 2);
        if (with_v) {
#pragma unroll
            for (int n = 0; n < T::RM_LOADS; ++n)
                load16_to_lds(vbase, rmbytes, base + VOFF + (wave * T::RM_LOADS + n) * 1024,
                              rm_ld[n], kt * 64 * D * 2);
        }
        if (wave == 0)
            load4_to_lds(fbase, fbytes, base + FOFF, lane * 4, kt * 64 * 4);
    };

    int ard[DC];                               // A-operand slot offsets of row-major tiles
#pragma unroll
    for (int dc = 0; dc < DC; ++dc)
        ard[dc] = (row16 * T::R + ((4 * dc + grp) ^ T::swz(row16))) * 16;

    const int nblk = blk1 < 0 ? 1 : 2;
    for (int blk = 0; blk < nblk; ++blk) {
        const int qb = blk == 0 ? blk0 : blk1;
        const int qw0 = qb * 64 + wave * 16;
        const int qwl = min(qw0 + 15, L - 1);
        const bool wave_active = qw0 < L;
        const int ntiles = qb + 1;
        const int qi = qw0 + row16;
        const bool qvalid = qi < L;

        // query and dO rows of this lane's query (B operands), the row factor
        bf16x8 qf[DC], gf[DC];
#pragma unroll
        for (int dc = 0; dc < DC; ++dc) {
            u32x4 w = {0u, 0u, 0u, 0u}, x = {0u, 0u, 0u, 0u};
            if (qvalid) {
                w = *reinterpret_cast<const u32x4*>(Q + hoff + (size_t)qi * D + 32 * dc + 8 * grp);
                x = *reinterpret_cast<const u32x4*>(G + hoff + (size_t)qi * D + 32 * dc + 8 * grp);
            }
            qf[dc] = __builtin_bit_cast(bf16x8, w);
            gf[dc] = __builtin_bit_cast(bf16x8, x);
        }
        const float rqi = qvalid ? rq[(size_t)bh * L + qi] : 0.0f;
        // log2(e) ln d ln i / |q_i|  (Key design 1: log d . log N), in fp32
        // as in the forward (a few ulp against the scores' fp32 error)
        constexpr float kLn2 = 0.693147180559945309f;
        const float lam_i = (float)lam_scale * (__builtin_amdgcn_logf((float)(qi + 1)) * kLn2);
        const float lam = lam_i * rqi;

        // (init: the accumulator's starting value)
        auto mm_block = [&](const unsigned char* base, int off, const bf16x8 (&b)[DC], int ks,
                            float init = 0.0f) {
            f32x4 acc = {init, init, init, init};
#pragma unroll
            for (int dc = 0; dc < DC; ++dc) {
                const bf16x8 a =
                    *reinterpret_cast<const bf16x8*>(base + off + ard[dc] + ks * 16 * T::R * 16);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[dc], acc, 0, 0, 0);
            }
            return acc;
        };
        // scaled scores t (masked: -inf) of block ks, and the key factors
        auto scores = [&](int kt, const unsigned char* base, int ks, f32x4 acc, bool diag,
                          f32x4& f4) {
            f4 = *reinterpret_cast<const f32x4*>(base + FOFF + (16 * ks + 4 * grp) * 4);
            f32x4 t = acc * (f4 * lam);
            if (diag) {
                const int k0 = kt * 64 + 16 * ks + 4 * grp;
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    t[r] = (k0 + r <= qi) ? t[r] : -INFINITY;
            }
            return t;
        };

        // ---------------- pass 1 (rowstats): S and the max score ----------------
        float s1 = 0.0f, tmax = -INFINITY;
        float c = 0.0f, tc = 0.0f;
        bool degen = true;
        // row coefficients (dq reads them; rowstats computes them)
        float adl = 0.0f, Ac = 0.0f, Ec = 0.0f;    // adl = -A delta

        // tiles 0..ntiles-2 lie before every row of the block, the last one
        // holds its diagonal: the loop runs the unmasked body only (with both
        // bodies in the loop their accumulators were copied at every tile)
        auto tile_loop = [&](bool with_v, auto body) {
            auto step = [&](int kt, auto diag_tag) {
                __syncthreads();                   // readers of the previous tile done
                issue(kt, with_v);
                __builtin_amdgcn_s_waitcnt(0);
                __syncthreads();                   // tile kt landed
                if (wave_active)
                    body(kt, lds, diag_tag);
            };
            for (int kt = 0; kt + 1 < ntiles; ++kt)
                step(kt, std::false_type{});
            step(ntiles - 1, std::true_type{});
        };

        // stage-2 row constants from S and the max score (degenerate: c = 0)
        float gap = 0.0f;
        auto row_consts = [&]() {
            const float o = (qi + 1) <= 3 ? 0.0f : 1.0f;
            const float tau = o * s1 / (float)(qi + 1);
            gap = softplus2_acc(tmax) - tau;
            degen = !((float)(qi + 1) * gap / s1 > eps) || !qvalid;
            c = degen ? 0.0f : 1.0f / gap;
            tc = tau * c;
        };
        // the 8 coefficients of the row for the dq and key-side kernels, from
        // Y = sum y^p, delta = dO . out and Pd = sum sp y^(p-1) (dW - delta)
        // (exact: the block evaluates Softplus exactly, stored in field 6 of
        // every row for the key side's choice of path)
        auto row_coefs = [&](float Y, float dl, float Pd, bool exact) {
            const float alpha = (float)p_rt * s1 / (gap * Y);
            const float epsr = alpha / s1 * Pd;
            // ln d ln i / (S ln 2), S in base 2: lam_scale ln i / S
            const float kappa = lam_i / s1;
            // A and E carry 1 / |q_i|: dk^ sums (dc_ij / |q_i|) q_i, and dq
            // = (dq^ - (dq^ . q^) q^) / |q_i| takes the factor from them
            const float a_ = degen ? 0.0f : kappa * alpha * rqi;
            const float e_ = degen ? 0.0f : kappa * epsr * rqi;
            if (qvalid && grp == 0) {
                // u = Y^(-1/p) (Y >= 1: the row's largest score gives y = 1);
                // (y u)^p = y^p / Y and (y u)^(p-1) Y u = y^(p-1), so the
                // key side forms the weight with one multiply.  The kernels
                // clamp y u at 1, not at u (a clamp at 1 is free on the fma):
                // y u exceeds u only where rounding puts y above 1, and by the
                // same factor.
                const float u = degen ? 0.0f
                                      : __builtin_amdgcn_exp2f(-__builtin_amdgcn_logf(Y) / (float)p_rt);
                const float yu = Y * u;
                float* st = stats + ((size_t)bh * L + qi) * kBwdRowStats;
                const float4 a = degen ? make_float4(0.0f, 0.0f, 0.0f, 0.0f)
                                       : make_float4(c * u, tc * u, a_ * yu, -dl * a_ * yu);
                *reinterpret_cast<float4*>(st) = a;
                *reinterpret_cast<float2*>(st + 4) = make_float2(e_, lam);
                st[6] = exact ? 1.0f : 0.0f;
            }
            Ac = a_;
            Ec = e_;
        };
        // the row's largest score, stored as soon as it is known (kept to the
        // end it would cost a register through the pass-2 loop)
        auto store_tmax = [&]() {
            if (qvalid && grp == 0)
                stats[((size_t)bh * L + qi) * kBwdRowStats + 7] = tmax;
        };
        // B operand of 16x16x16 (four consecutive keys 16 ks + 4 grp + 0..3
        // of dim 16 ds + row16) from the row-major K tile by the LDS
        // transpose read, as in the key-side kernel: lane j of group grp
        // names key 16 ks + 4 grp + j / 4, dims 16 ds + 4 (j % 4) + 0..3
        int trr[DS];
        {
            const int x = 4 * grp + (row16 >> 2);
            const int X = ((row16 >> 1) & 1) ^ T::swz(x);
#pragma unroll
            for (int ds = 0; ds < DS; ++ds)
                trr[ds] = (x * T::R + ((2 * ds) ^ X)) * 16 + (row16 & 1) * 8;
        }
        auto mm_kt = [&](const unsigned char* base, int ks, s16x4 g, f32x4 (&acc)[DS]) {
#pragma unroll
            for (int ds = 0; ds < DS; ++ds) {
                const bf16x4 bk = lds_read_tr16(base + KOFF + ks * 16 * T::R * 16 + trr[ds]);
                acc[ds] = mfma16k16(g, bk, acc[ds]);
            }
        };
        // key blocks ks and ks + 1 together
        auto mm_kt2 = [&](const unsigned char* base, int ks, s16x4 g0, s16x4 g1, f32x4 (&acc)[DS]) {
#pragma unroll
            for (int ds = 0; ds < DS; ++ds) {
                const unsigned char* b = base + KOFF + ks * 16 * T::R * 16 + trr[ds];
                acc[ds] = mfma16k16x2(g0, g1, lds_read_tr16(b), lds_read_tr16(b + 16 * T::R * 16),
                                      acc[ds]);
            }
        };
        // acc[ds][r] = dQ^[query 4 grp + r of the wave][dim 16 ds + row16], with
        // 1 / |q| carried by the coefficients;
        // dq = (dq^ - (dq^ . q^) q^) / |q|, or dq^ / 1e-12 below the clamp
        auto store_dq = [&](const f32x4 (&acc)[DS]) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int qr = qw0 + 4 * grp + r;
                const bool ok = qr < L;
                const float rr = ok ? rq[(size_t)bh * L + qr] : 0.0f;
                float qh[DS], dd = 0.0f;
#pragma unroll
                for (int ds = 0; ds < DS; ++ds) {
                    qh[ds] = ok ? (float)Q[hoff + (size_t)qr * D + 16 * ds + row16] * rr : 0.0f;
                    dd = __builtin_fmaf(acc[ds][r], qh[ds], dd);
                }
#pragma unroll
                for (int m = 1; m < 16; m <<= 1)
                    dd += __shfl_xor(dd, m);
                const bool clamped = !(rr < 1e12f);
                if (ok) {
#pragma unroll
                    for (int ds = 0; ds < DS; ++ds) {
                        const float v = clamped ? acc[ds][r] : acc[ds][r] - dd * qh[ds];
                        dQ[hoff + (size_t)qr * D + 16 * ds + row16] = (__bf16)v;
                    }
                }
            }
        };

        if constexpr (MODE == 0) {
            if (saved) {
                // the training forward's statistics replace pass 1; the
                // block's deep-row flag from their largest scores
                if (qvalid)
                    load_row_stats(saved, (size_t)bh * L + qi, s1, tmax);
                __syncthreads();                   // earlier readers of the flag done
                if (tid == 0)
                    *deep_flag = 0;
                __syncthreads();
                if (qvalid && tmax < kDeep)
                    *deep_flag = 1;
                __syncthreads();
            } else {
                // pass 1 as in the forward: sum max(t, 0) plus log2 of the
                // product of the factors 1 + 2^-|t| (one exp2 per pair), and
                // for a block with a deep row the exact Softplus (softplus2_acc)
                // PROD: log2 of the product of the factors 1 + 2^t, a
                // mantissa and an exponent renormalised after every two, as
                // in the forward while the block's scores stay within
                // kProdMaxT
                auto pass1 = [&](auto acc_tag, auto prod_tag) {
                    constexpr bool ACC = decltype(acc_tag)::value;
                    constexpr bool PROD = decltype(prod_tag)::value;
                    s1 = 0.0f;
                    tmax = -INFINITY;
                    float pm = 1.0f;
                    int pe = 0;
                    tile_loop(false, [&](int kt, const unsigned char* base, auto diag_tag) {
                        constexpr bool DIAG = decltype(diag_tag)::value;
                        const int nks = DIAG ? min(4, (qwl - kt * 64) / 16 + 1) : 4;
                        float pos = 0.0f, prod = 1.0f;
#pragma unroll
                        for (int ks = 0; ks < 4; ++ks) {
                            if (DIAG && ks >= nks)
                                continue;
                            f32x4 f4;
                            const f32x4 t =
                                scores(kt, base, ks, mm_block(base, KOFF, qf, ks), DIAG, f4);
                            if constexpr (PROD) {
#pragma unroll
                                for (int r = 0; r < 4; r += 2) {
                                    pm = __builtin_fmaf(pm, __builtin_amdgcn_exp2f(t[r]), pm);
                                    pm = __builtin_fmaf(pm, __builtin_amdgcn_exp2f(t[r + 1]), pm);
                                    pe += __builtin_amdgcn_frexp_expf(pm);
                                    pm = __builtin_amdgcn_frexp_mantf(pm);
                                }
                            }
#pragma unroll
                            for (int r = 0; r < 4; ++r) {
                                if constexpr (ACC) {
                                    pos += softplus2_acc(t[r]);
                                } else if constexpr (!PROD) {
                                    pos += fmaxf(t[r], 0.0f);
                                    prod = __builtin_fmaf(prod, __builtin_amdgcn_exp2f(-fabsf(t[r])),
                                                          prod);
                                }
                                tmax = fmaxf(tmax, t[r]);
                            }
                        }
                        if constexpr (ACC)
                            s1 += pos;
                        else if constexpr (!PROD)
                            s1 += pos + __builtin_amdgcn_logf(prod);
                    });
                    if constexpr (PROD)
                        s1 = __builtin_amdgcn_logf(pm) + (float)pe;
                    s1 += __shfl_xor(s1, 16);
                    s1 += __shfl_xor(s1, 32);
                    tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
                    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
                };
                // the block's flag: cleared before the first tile barrier,
                // set by lanes of deep rows, read after one more barrier
                if (tid == 0)
                    *deep_flag = 0;
                // every score of the block is at most about lambda of its
                // last row (wave-uniform)
                const float lam_last = (float)lam_scale *
                    (__builtin_amdgcn_logf((float)min(L, qb * 64 + 64)) * kLn2);
                if (__builtin_amdgcn_readfirstlane((int)(lam_last <= kProdMaxT)))
                    pass1(std::false_type{}, std::true_type{});
                else
                    pass1(std::false_type{}, std::false_type{});
                if (qvalid && tmax < kDeep)
                    *deep_flag = 1;
                __syncthreads();
                if (*deep_flag)
                    pass1(std::true_type{}, std::false_type{});
            }
            store_tmax();
            row_consts();

            // ---------------- pass 2: Y, P1, P2, Z ----------------
            // (a block without a deep row takes plain log2(1 + 2^t); the
            // flag is final after pass 1)
            const bool exact = *deep_flag;
            float Y = 0.0f, P1 = 0.0f, P2 = 0.0f, Z = 0.0f;
            auto pass2 = [&](auto exact_tag) {
              tile_loop(true, [&](int kt, const unsigned char* base, auto diag_tag) {
                constexpr bool DIAG = decltype(diag_tag)::value;
                const int nks = DIAG ? min(4, (qwl - kt * 64) / 16 + 1) : 4;
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    if (DIAG && ks >= nks)
                        continue;
                    f32x4 f4;
                    const f32x4 t = scores(kt, base, ks, mm_block(base, KOFF, qf, ks), DIAG, f4);
                    const f32x4 dw = mm_block(base, VOFF, gf, ks);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float sp = decltype(exact_tag)::value
                                             ? softplus2_acc(t[r])
                                             : __builtin_amdgcn_logf(1.0f + __builtin_amdgcn_exp2f(t[r]));
                        const float y = __builtin_amdgcn_fmed3f(__builtin_fmaf(sp, c, -tc), 0.0f, 1.0f);
                        const float ym = pow_m1<P>(y, p_rt);
                        const float yp = ym * y;
                        Y += yp;
                        P1 = __builtin_fmaf(yp, dw[r], P1);
                        const float sym = sp * ym;
                        P2 = __builtin_fmaf(sym, dw[r], P2);
                        Z += sym;
                    }
                }
              });
            };
            if (exact)
                pass2(std::true_type{});
            else
                pass2(std::false_type{});
#pragma unroll
            for (int m = 16; m <= 32; m <<= 1) {
                Y += __shfl_xor(Y, m);
                P1 += __shfl_xor(P1, m);
                P2 += __shfl_xor(P2, m);
                Z += __shfl_xor(Z, m);
            }
            const float dl = P1 / Y;
            row_coefs(Y, dl, P2 - dl * Z, exact);
        } else if constexpr (MODE == 1) {
            // ---------------- dq: dQ^ = sum_j (dc_ij f_j) k_j ----------------
            if (qvalid) {
                // (c u, tau c u, A Y u, -A delta Y u, E): y u and the pair
                // gradient as from (c, tau c, A, -A delta, E), see row_coefs
                const float* st = stats + ((size_t)bh * L + qi) * kBwdRowStats;
                const float4 a = *reinterpret_cast<const float4*>(st);
                c = a.x;
                tc = a.y;
                Ac = a.z;
                adl = a.w;
                Ec = st[4];
            }
            // (a block without a deep row, by the largest scores in
            // the coefficient records, takes plain log2(1 + 2^t))
            const float tm = qvalid ? stats[((size_t)bh * L + qi) * kBwdRowStats + 7] : 0.0f;
            __syncthreads();                       // earlier readers of the flag done
            if (tid == 0)
                deep_flag[0] = 0;
            __syncthreads();
            if (tm < kDeep)
                deep_flag[0] = 1;
            __syncthreads();
            const bool exact = deep_flag[0] != 0;
            f32x4 acc[DS];
#pragma unroll
            for (int ds = 0; ds < DS; ++ds)
                acc[ds] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            auto dq_pass = [&](auto exact_tag) {
              tile_loop(true, [&](int kt, const unsigned char* base, auto diag_tag) {
                constexpr bool DIAG = decltype(diag_tag)::value;
                const int nks = DIAG ? min(4, (qwl - kt * 64) / 16 + 1) : 4;
                // the pair gradients of key block ks as the bf16 A operand
                auto grad = [&](int ks) {
                    f32x4 f4;
                    const f32x4 t = scores(kt, base, ks, mm_block(base, KOFF, qf, ks), DIAG, f4);
                    const f32x4 dw = mm_block(base, VOFF, gf, ks);
                    f32x4 g;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        float sp, sg;
                        if constexpr (decltype(exact_tag)::value)
                            sp_sig(t[r], sp, sg);
                        else
                            sp_sig_plain(t[r], sp, sg);
                        const float y = __builtin_amdgcn_fmed3f(__builtin_fmaf(sp, c, -tc), 0.0f, 1.0f);
                        const float ym = pow_m1<P>(y, p_rt);
                        const float dcv = sg * __builtin_fmaf(ym, __builtin_fmaf(Ac, dw[r], adl), -Ec);
                        g[r] = dcv * f4[r];
                    }
                    return pack_bf16x4(g);
                };
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int ks = 2 * h;
                    if (DIAG && ks >= nks)
                        continue;
                    const s16x4 g0 = grad(ks);
                    if (DIAG && ks + 1 >= nks) {
                        mm_kt(base, ks, g0, acc);
                        continue;
                    }
                    const s16x4 g1 = grad(ks + 1);
                    mm_kt2(base, ks, g0, g1, acc);
                }
              });
            };
            if (exact)
                dq_pass(std::true_type{});
            else
                dq_pass(std::false_type{});
            store_dq(acc);
        } else {
            // ------- rowstats and dq in one pass, from the training forward's
            // row statistics.  delta = sum_j W_ij dW_ij must be the one of
            // this pass's own weights (on peaked rows an error in it is
            // multiplied by A_i), so the forward's output gives only an
            // offset d0 = dO . out, and with h = y^(p-1) (dW - d0):
            //   delta - d0 = sum y h / Y                       (= Dl)
            //   dq^_i = A_i (sum sigma h k^ - Dl sum sigma y^(p-1) k^)
            //           - E_i sum sigma k^
            // A_i and E_i need the row's full sums, so they and Dl scale the
            // three accumulated vectors at the end.  A block without a deep
            // row (largest score below kDeep) takes plain log2(1 + 2^t), as
            // the forward does, and a block with one the exact Softplus (a
            // uniform branch) -------
            if (qvalid)
                load_row_stats(saved, (size_t)bh * L + qi, s1, tmax);
            store_tmax();
            __syncthreads();                       // earlier readers of the flag done
            if (tid == 0)
                deep_flag[0] = 0;
            __syncthreads();
            if (qvalid && tmax < kDeep)
                deep_flag[0] = 1;
            __syncthreads();
            const bool blk_deep = deep_flag[0] != 0;
            float d0 = 0.0f;
            if (qvalid) {
#pragma unroll
                for (int dc = 0; dc < DC; ++dc) {
                    const u32x4 w =
                        *reinterpret_cast<const u32x4*>(O + hoff + (size_t)qi * D + 32 * dc + 8 * grp);
                    const u32x4 x = __builtin_bit_cast(u32x4, gf[dc]);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        d0 = __builtin_fmaf(bf16lo(w[e]), bf16lo(x[e]), d0);
                        d0 = __builtin_fmaf(bf16hi(w[e]), bf16hi(x[e]), d0);
                    }
                }
            }
            d0 += __shfl_xor(d0, 16);
            d0 += __shfl_xor(d0, 32);
            row_consts();

            f32x4 acc1[DS], acc2[DS], acc3[DS];
#pragma unroll
            for (int ds = 0; ds < DS; ++ds)
                acc1[ds] = acc2[ds] = acc3[ds] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            float Y = 0.0f, P1 = 0.0f, Pd = 0.0f, Z = 0.0f;
            auto one_pass = [&](auto exact_tag) {
              tile_loop(true, [&](int kt, const unsigned char* base, auto diag_tag) {
                constexpr bool DIAG = decltype(diag_tag)::value;
                const int nks = DIAG ? min(4, (qwl - kt * 64) / 16 + 1) : 4;
                // the three pair-gradient products of key block ks as bf16 A
                // operands; the row sums are taken in key order
                auto grads = [&](int ks, s16x4& p1, s16x4& p2, s16x4& p3) {
                    f32x4 f4;
                    const f32x4 t = scores(kt, base, ks, mm_block(base, KOFF, qf, ks), DIAG, f4);
                    // dW - d0, the offset as the accumulator's start
                    const f32x4 dw = mm_block(base, VOFF, gf, ks, -d0);
                    f32x4 g1, g2, g3;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        float sp, sg;
                        if constexpr (decltype(exact_tag)::value)
                            sp_sig(t[r], sp, sg);
                        else
                            sp_sig_plain(t[r], sp, sg);
                        const float y = __builtin_amdgcn_fmed3f(__builtin_fmaf(sp, c, -tc), 0.0f, 1.0f);
                        const float ym = pow_m1<P>(y, p_rt);
                        Y = __builtin_fmaf(ym, y, Y);
                        Z = __builtin_fmaf(sp, ym, Z);
                        const float h = ym * dw[r];
                        P1 = __builtin_fmaf(y, h, P1);
                        Pd = __builtin_fmaf(sp, h, Pd);
                        g2[r] = sg * f4[r];
                        g1[r] = g2[r] * h;
                        g3[r] = g2[r] * ym;
                    }
                    p1 = pack_bf16x4(g1);
                    p2 = pack_bf16x4(g2);
                    p3 = pack_bf16x4(g3);
                };
                // the first product one key block at a time, the other two
                // for pairs of blocks (all three paired would need six
                // operands live and spill at this register cap)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int ks = 2 * h;
                    if (DIAG && ks >= nks)
                        continue;
                    s16x4 p1, p2, p3;
                    grads(ks, p1, p2, p3);
                    const bool one = DIAG && ks + 1 >= nks;
#pragma unroll
                    for (int ds = 0; ds < DS; ++ds) {
                        const bf16x4 bk = lds_read_tr16(base + KOFF + ks * 16 * T::R * 16 + trr[ds]);
                        acc1[ds] = mfma16k16(p1, bk, acc1[ds]);
                        if (one) {
                            acc2[ds] = mfma16k16(p2, bk, acc2[ds]);
                            acc3[ds] = mfma16k16(p3, bk, acc3[ds]);
                        }
                    }
                    if (one)
                        continue;
                    s16x4 q1, q2, q3;
                    grads(ks + 1, q1, q2, q3);
#pragma unroll
                    for (int ds = 0; ds < DS; ++ds) {
                        const unsigned char* b = base + KOFF + ks * 16 * T::R * 16 + trr[ds];
                        const bf16x4 b0 = lds_read_tr16(b), b1 = lds_read_tr16(b + 16 * T::R * 16);
                        acc1[ds] = mfma16k16(q1, b1, acc1[ds]);
                        acc2[ds] = mfma16k16x2(p2, q2, b0, b1, acc2[ds]);
                        acc3[ds] = mfma16k16x2(p3, q3, b0, b1, acc3[ds]);
                    }
                }
              });
            };
            if (blk_deep)
                one_pass(std::true_type{});
            else
                one_pass(std::false_type{});
#pragma unroll
            for (int m = 16; m <= 32; m <<= 1) {
                Y += __shfl_xor(Y, m);
                Z += __shfl_xor(Z, m);
                P1 += __shfl_xor(P1, m);
                Pd += __shfl_xor(Pd, m);
            }
            const float Dl = degen ? 0.0f : P1 / Y;
            row_coefs(Y, d0 + Dl, Pd - Dl * Z, blk_deep);
            // the coefficients of query 4 grp + r sit in lane 4 grp + r
            f32x4 acc[DS];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int src = 4 * grp + r;
                const float a = __shfl(Ac, src), e = __shfl(Ec, src), ad = a * __shfl(Dl, src);
#pragma unroll
                for (int ds = 0; ds < DS; ++ds)
                    acc[ds][r] = a * acc1[ds][r] - ad * acc3[ds][r] - e * acc2[ds][r];
            }
            store_dq(acc);
        }
    }
}

// ---------------------------------------------------------------------------
// Key-side kernel (dk, dv): lane (row16, grp) owns key row16 of its wave and
// queries 16 c + 4 grp + r of each 16-query block c of a query tile.
// ---------------------------------------------------------------------------
// Query tiles stream through LDS, double-buffered at d = 64 (one buffer at
// d = 128, as in the query-side kernels).
template <int D, int P>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(3))) void lssar_bwd_kside_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    const __bf16* __restrict__ G, const float* __restrict__ fk, const float* __restrict__ stats,
    __bf16* __restrict__ dK, __bf16* __restrict__ dV, int BH, int L, int nkb, int npair, int p_rt)
{
    static_assert(D == 64 || D == 128, "head dim");
    using T = BwdTiles<D>;
    constexpr int DC = D / 32;
    constexpr int DS = D / 16;
    constexpr int QOFF = 0, GOFF = T::RM;
    constexpr int SOFF = 2 * T::RM;
    constexpr int BYTES = SOFF + 64 * kBwdRowStats * 4;   // one tile buffer
    // d = 64: two buffers (36 KB); d = 128: one.  Capped for 3 waves per
    // SIMD: uncapped, the p = 15 instantiation took 236 VGPRs (2 waves, 13%
    // slower); capped for 4 it spills inside the tile loop (46% slower)
    constexpr int NB = D == 64 ? 2 : 1;
    // the tile buffers, then the key block's deep-block flag
    __shared__ __attribute__((aligned(1024))) unsigned char lds[NB * BYTES + 16];
    int* const deep_flag = reinterpret_cast<int*>(lds + NB * BYTES);

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, row16 = lane & 15, grp = lane >> 4;
    int bh, blk0, blk1;
    if (!bwd_blocks<D>((int)blockIdx.x, BH, nkb, true, bh, blk0, blk1))
        return;
    const size_t hoff = (size_t)bh * L * D;

    const void* qbase = Q + hoff;
    const void* gbase = G + hoff;
    const unsigned rmbytes = (unsigned)L * D * 2u;
    const void* sbase = stats + (size_t)bh * L * kBwdRowStats;
    const unsigned sbytes = (unsigned)L * kBwdRowStats * 4u;

    int rm_ld[T::RM_LOADS];
#pragma unroll
    for (int n = 0; n < T::RM_LOADS; ++n)
        rm_ld[n] = (int)rm_src<D>((wave * T::RM_LOADS + n) * 64 + lane);
    // the tile's coefficient rows in LDS in the order (r, c, g) of query
    // 16 c + 4 g + r: the four lane groups, which read rows 4 apart at
    // once, then read 128 consecutive bytes instead of one bank four times
    int st_src;
    {
        const int u = wave * 64 + lane;        // 16-byte unit of the LDS copy
        const int pos = u >> 1, r = pos >> 4, c = (pos >> 2) & 3, g = pos & 3;
        st_src = (16 * c + 4 * g + r) * kBwdRowStats * 4 + (u & 1) * 16;
    }

    // query tile qt: Q, dO (row-major) and the 64 rows' coefficients
    auto issue = [&](int qt, int buf) {
        unsigned char* base = lds + buf * BYTES;
#pragma unroll
        for (int n = 0; n < T::RM_LOADS; ++n) {
            load16_to_lds(qbase, rmbytes, base + QOFF + (wave * T::RM_LOADS + n) * 1024, rm_ld[n],
                          qt * 64 * D * 2);
            load16_to_lds(gbase, rmbytes, base + GOFF + (wave * T::RM_LOADS + n) * 1024, rm_ld[n],
                          qt * 64 * D * 2);
        }
        if (wave < 2)
            load16_to_lds(sbase, sbytes, base + SOFF + wave * 1024, st_src,
                          qt * 64 * kBwdRowStats * 4);
    };

    int ard[DC];
#pragma unroll
    for (int dc = 0; dc < DC; ++dc)
        ard[dc] = (row16 * T::R + ((4 * dc + grp) ^ T::swz(row16))) * 16;
    // B operands of the 16x16x16 products (four consecutive queries of one
    // dim) straight from the row-major tiles by the LDS transpose read: in
    // each 16-lane group, lane j names four consecutive dims of one query
    // row, and lane 4q + e receives element e of lanes q, q + 4, q + 8 and
    // q + 12.  Lane j of group grp names query 16 c + 4 grp + j / 4, dims
    // 16 ds + 4 (j % 4) + 0..3; the rows' slot swizzle does not depend on c.
    int trr[DS];
    {
        const int x = 4 * grp + (row16 >> 2);
        const int X = ((row16 >> 1) & 1) ^ T::swz(x);
#pragma unroll
        for (int ds = 0; ds < DS; ++ds)
            trr[ds] = (x * T::R + ((2 * ds) ^ X)) * 16 + (row16 & 1) * 8;
    }

    const int nblk = blk1 < 0 ? 1 : 2;
    for (int blk = 0; blk < nblk; ++blk) {
        // blk 0: the earlier key block (more query tiles), blk 1: the later
        const int kb = blk == 0 ? blk0 : blk1;
        const int kw0 = kb * 64 + wave * 16;       // first key row of this wave
        const int kj = kw0 + row16;                // this lane's key (0-based)
        const bool kvalid = kj < L;
        const int qt0 = kb, ntiles = (L + 63) / 64 - kb;

        bf16x8 kf[DC], vf[DC];
#pragma unroll
        for (int dc = 0; dc < DC; ++dc) {
            u32x4 w = {0u, 0u, 0u, 0u}, x = {0u, 0u, 0u, 0u};
            if (kvalid) {
                w = *reinterpret_cast<const u32x4*>(K + hoff + (size_t)kj * D + 32 * dc + 8 * grp);
                x = *reinterpret_cast<const u32x4*>(V + hoff + (size_t)kj * D + 32 * dc + 8 * grp);
            }
            kf[dc] = __builtin_bit_cast(bf16x8, w);
            vf[dc] = __builtin_bit_cast(bf16x8, x);
        }
        const float fj = kvalid ? fk[(size_t)bh * L + kj] : 0.0f;

        f32x4 adv[DS], adk[DS];
#pragma unroll
        for (int ds = 0; ds < DS; ++ds)
            adv[ds] = adk[ds] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

        auto mm_block = [&](const unsigned char* base, int off, const bf16x8 (&b)[DC], int c) {
            f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int dc = 0; dc < DC; ++dc) {
                const bf16x8 a =
                    *reinterpret_cast<const bf16x8*>(base + off + ard[dc] + c * 16 * T::R * 16);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[dc], acc, 0, 0, 0);
            }
            return acc;
        };

        auto tile = [&](int qt, const unsigned char* base, auto diag_tag, auto exact_tag) {
            constexpr bool DIAG = decltype(diag_tag)::value;
            // weights and pair gradients of 16-query block c as bf16 A operands
            auto operands = [&](int c, s16x4& wb, s16x4& gb) {
                const f32x4 sc = mm_block(base, QOFF, kf, c);   // S[query][key]
                const f32x4 dw = mm_block(base, GOFF, vf, c);   // dW[query][key]
                f32x4 w4, g4;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int qrow = 16 * c + 4 * grp + r;       // query in the tile
                    const float* st = reinterpret_cast<const float*>(base + SOFF) +
                                      (16 * r + 4 * c + grp) * kBwdRowStats;
                    // (c u, tau c u, A Y u, -A delta Y u), (E, lam)
                    const float4 a = *reinterpret_cast<const float4*>(st);
                    const float2 b = *reinterpret_cast<const float2*>(st + 4);
                    float t = sc[r] * b.y * fj;                  // lam_i f_j (q . k)
                    if (DIAG && qt * 64 + qrow < kj)
                        t = -INFINITY;
                    float sp, sg;
                    if constexpr (decltype(exact_tag)::value)
                        sp_sig(t, sp, sg);
                    else
                        sp_sig_plain(t, sp, sg);
                    const float y = __builtin_amdgcn_fmed3f(__builtin_fmaf(sp, a.x, -a.y), 0.0f, 1.0f);
                    const float ym = pow_m1<P>(y, p_rt);
                    w4[r] = ym * y;                              // y^p / Y
                    g4[r] = sg * __builtin_fmaf(ym, __builtin_fmaf(a.z, dw[r], a.w), -b.x);
                }
                wb = pack_bf16x4(w4);
                gb = pack_bf16x4(g4);
            };
            auto mm_one = [&](int c, s16x4 wb, s16x4 gb) {
#pragma unroll
                for (int ds = 0; ds < DS; ++ds) {
                    const int off = c * 16 * T::R * 16 + trr[ds];
                    adv[ds] = mfma16k16(wb, lds_read_tr16(base + GOFF + off), adv[ds]);
                    adk[ds] = mfma16k16(gb, lds_read_tr16(base + QOFF + off), adk[ds]);
                }
            };
            // d = 128: one block at a time (pairs need 256 VGPRs there)
            if constexpr (D != 64) {
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    if (DIAG && qt * 64 + 16 * c + 15 < kw0)
                        continue;
                    s16x4 wb, gb;
                    operands(c, wb, gb);
                    mm_one(c, wb, gb);
                }
                return;
            }
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int c = 2 * h;
                // query blocks entirely before this wave's first key see none
                // of it (a leading run of blocks)
                if (DIAG && qt * 64 + 16 * (c + 1) + 15 < kw0)
                    continue;
                s16x4 wb1, gb1;
                if (DIAG && qt * 64 + 16 * c + 15 < kw0) {
                    operands(c + 1, wb1, gb1);
                    mm_one(c + 1, wb1, gb1);
                    continue;
                }
                s16x4 wb0, gb0;
                operands(c, wb0, gb0);
                operands(c + 1, wb1, gb1);
#pragma unroll
                for (int ds = 0; ds < DS; ++ds) {
                    const int off = c * 16 * T::R * 16 + trr[ds];
                    const int off1 = off + 16 * T::R * 16;
                    adv[ds] = mfma16k16x2(wb0, wb1, lds_read_tr16(base + GOFF + off),
                                          lds_read_tr16(base + GOFF + off1), adv[ds]);
                    adk[ds] = mfma16k16x2(gb0, gb1, lds_read_tr16(base + QOFF + off),
                                          lds_read_tr16(base + QOFF + off1), adk[ds]);
                }
            }
        };

        // at d = 64 a key block all of whose query blocks (kb and later)
        // are without a deep row takes plain log2(1 + 2^t) for every tile,
        // a workgroup-uniform choice made once from the blocks' flags
        // (record field 6, stored by the query-side kernels); at d = 128
        // the second path spills in the tile loop, and every tile is
        // exact.  (Chosen per tile inside the loop, the two paths'
        // accumulators met in different registers: 16 64-bit copies per
        // tile.)
        constexpr bool kPlain = D == 64;
        bool exact = true;
        if constexpr (kPlain) {
            bool deep = false;
            for (int b = kb + tid; b < nkb; b += kThreads)
                deep = deep || stats[((size_t)bh * L + (size_t)b * 64) * kBwdRowStats + 6] != 0.0f;
            __syncthreads();                       // earlier readers of the flag done
            if (tid == 0)
                *deep_flag = 0;
            __syncthreads();
            if (deep)
                *deep_flag = 1;
            __syncthreads();
            exact = *deep_flag != 0;
        }
        // the first query tile (qt = kb) holds the diagonal, the later ones
        // lie wholly after every key of the block: it is peeled off the loop.
        // Double-buffered, tile n sits in buffer n & 1 and the loop runs two
        // tiles per iteration, so that every buffer index is a constant and
        // the LDS reads take the buffer's offset as an immediate (a runtime
        // index cost a vector add per operand address and tile).
        auto tile_loop = [&](auto exact_tag) {
            auto step = [&](int n, auto buf_tag, auto diag_tag) {
                if constexpr (NB == 2) {
                    constexpr int buf = decltype(buf_tag)::value;
                    __builtin_amdgcn_s_waitcnt(0);
                    __syncthreads();               // tile n landed; buffer buf ^ 1 free
                    if (n + 1 < ntiles)
                        issue(qt0 + n + 1, buf ^ 1);
                    if (kw0 < L)
                        tile(qt0 + n, lds + buf * BYTES, diag_tag, exact_tag);
                } else {
                    __syncthreads();               // readers of the previous tile done
                    issue(qt0 + n, 0);
                    __builtin_amdgcn_s_waitcnt(0);
                    __syncthreads();               // tile landed
                    if (kw0 < L)
                        tile(qt0 + n, lds, diag_tag, exact_tag);
                }
            };
            using B0 = std::integral_constant<int, 0>;
            using B1 = std::integral_constant<int, 1>;
            if constexpr (NB == 2) {
                __syncthreads();                   // earlier readers done with both buffers
                issue(qt0, 0);
            }
            step(0, B0{}, std::true_type{});
            for (int n = 1; n < ntiles; n += 2) {
                step(n, B1{}, std::false_type{});
                if (n + 1 < ntiles)
                    step(n + 1, B0{}, std::false_type{});
            }
        };
        if (exact)
            tile_loop(std::true_type{});
        else if constexpr (kPlain)
            tile_loop(std::false_type{});

        // adv/adk[ds][r] = grad[key 4 grp + r of the wave][dim 16 ds + row16]
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int kr = kw0 + 4 * grp + r;
            const bool ok = kr < L;
            const float ff = ok ? fk[(size_t)bh * L + kr] : 0.0f;
            float kh[DS], dd = 0.0f;
#pragma unroll
            for (int ds = 0; ds < DS; ++ds) {
                kh[ds] = ok ? (float)K[hoff + (size_t)kr * D + 16 * ds + row16] * ff : 0.0f;
                dd = __builtin_fmaf(adk[ds][r], kh[ds], dd);
            }
#pragma unroll
            for (int m = 1; m < 16; m <<= 1)
                dd += __shfl_xor(dd, m);
            const bool clamped = !(ff < 1e12f);
            if (ok) {
#pragma unroll
                for (int ds = 0; ds < DS; ++ds) {
                    const float v = clamped ? adk[ds][r] * ff : (adk[ds][r] - dd * kh[ds]) * ff;
                    dK[hoff + (size_t)kr * D + 16 * ds + row16] = (__bf16)v;
                    dV[hoff + (size_t)kr * D + 16 * ds + row16] = (__bf16)adv[ds][r];
                }
            }
        }
    }
}

}  // namespace lssar
