// lssar.hip -- C ABI of the LSSAR causal attention forward on gfx950.
//
// Declarations, argument meaning, layout, ownership and error behaviour are
// documented in include/lssar.h.  Method: paper note "Softplus Attention with
// Re-weighting Boosts Length Extrapolation in Large Language Models",
// Method details, Key designs 1-3.  This file validates arguments on the
// host (before any HIP call), lays out the workspace, picks the kernel
// instantiation and launches the prep and attention kernels on the caller's
// stream.
#include "lssar.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <initializer_list>
#include <mutex>
#include <type_traits>

#include "lssar_bwd.hpp"
#include "lssar_bwd_mfma.hpp"
#include "lssar_decode.hpp"
#include "lssar_device.hpp"

namespace {

thread_local int g_last_hip_error = 0;

constexpr int kMaxL = 1 << 22;
constexpr int kMaxP = 1024;

int hip_fail(hipError_t e)
{
    g_last_hip_error = (int)e;
    return LSSAR_EHIP;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// [a, a + na) and [b, b + nb) share a byte
bool overlaps(const void* a, size_t na, const void* b, size_t nb)
{
    auto x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

// Workspace layout: [fk: key factor per key row, fp32 for bf16 inputs and
// fp64 for fp32 inputs][KN16: the normalised keys in f16, bf16 inputs only]
// [sched: the attention kernel's (head, block) per workgroup, int2, bf16
// inputs only]
struct Layout {
    size_t fk_bytes, kn16_bytes, sched_bytes;
    int Lp;
    size_t total() const { return fk_bytes + kn16_bytes + sched_bytes; }
};

Layout layout(long long B, long long H, long long L, int d, int dtype)
{
    Layout w;
    w.Lp = (int)((L + lssar::kBK - 1) / lssar::kBK * lssar::kBK);
    w.fk_bytes = round256((size_t)((dtype == LSSAR_F32 ? 8 : 4) * B * H * L));
    w.kn16_bytes = dtype == LSSAR_BF16 ? round256((size_t)(B * H * d) * (size_t)L * 2) : 0;
    w.sched_bytes = 0;
    if (dtype == LSSAR_BF16) {
        const int nqb = (int)((L + lssar::kBQ16 - 1) / lssar::kBQ16);
        w.sched_bytes = round256((size_t)lssar::FwdSched((int)(B * H), nqb).grid() * 8);
    }
    return w;
}

size_t elem_bytes(int dtype) { return dtype == LSSAR_F32 ? 4 : 2; }

// Sizes, dtype and head dimension.
int validate_shape(int B, int H, int L, int d, int dtype)
{
    if (B < 1 || H < 1 || L < 1)
        return LSSAR_EINVAL;
    if (dtype != LSSAR_F32 && dtype != LSSAR_BF16)
        return LSSAR_EUNSUPPORTED;
    if (d != 64 && d != 128)
        return LSSAR_EUNSUPPORTED;
    if (L > kMaxL)
        return LSSAR_EUNSUPPORTED;
    const long long bh = (long long)B * H;
    const long long nqb = (L + lssar::kBQ16 - 1) / lssar::kBQ16;
    // the forward's grid (lssar_sched.hpp) has at most B H (nqb + 1) + 16
    // workgroups
    if (bh > (1LL << 31) - 1 || bh * (nqb + 1) + 16 > (1LL << 31) - 1 || bh * L * d > (1LL << 46))
        return LSSAR_EINVAL;
    return LSSAR_OK;
}

int validate(const void* q, const void* k, const void* v, const void* out, int B, int H,
             int L, int d, int p, float eps, int dtype)
{
    if (!q || !k || !v || !out)
        return LSSAR_EINVAL;
    if (p < 1 || !(eps >= 0.0f) || !std::isfinite(eps))
        return LSSAR_EINVAL;
    int st = validate_shape(B, H, L, d, dtype);
    if (st != LSSAR_OK)
        return st;
    if (p > kMaxP)
        return LSSAR_EUNSUPPORTED;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
        return LSSAR_EINVAL;
    const size_t bytes = (size_t)B * H * L * d * elem_bytes(dtype);
    if (overlaps(out, bytes, q, bytes) || overlaps(out, bytes, k, bytes) ||
        overlaps(out, bytes, v, bytes))
        return LSSAR_EINVAL;
    return LSSAR_OK;
}

// The workspace must be 256-byte aligned, large enough, and overlap none of
// the tensors.
int validate_ws(const void* ws, size_t ws_bytes, const Layout& w, size_t tbytes,
                const void* a, const void* b, const void* c, const void* d)
{
    if (!ws || (reinterpret_cast<uintptr_t>(ws) & 255u) != 0 || ws_bytes < w.total())
        return LSSAR_EWORKSPACE;
    for (const void* t : {a, b, c, d})
        if (t && overlaps(ws, w.total(), t, tbytes))
            return LSSAR_EWORKSPACE;
    return LSSAR_OK;
}

template <int D>
void launch_knorm_f32(const void* k, double* fk, long nrows, hipStream_t s)
{
    constexpr int rpb = lssar::kThreads / (D / 4);
    const unsigned grid = (unsigned)((nrows + rpb - 1) / rpb);
    hipLaunchKernelGGL((lssar::lssar_knorm_f32_kernel<D>), dim3(grid), dim3(lssar::kThreads), 0,
                       s, static_cast<const float*>(k), fk, nrows);
}

template <int D>
void launch_prep_bf16(const void* k, float* fk, void* kn16, int2* sched, int BH, int L, int Lp,
                      hipStream_t s)
{
    const int per_xcd =
        (int)(lssar::FwdSched(BH, Lp / lssar::kBK).grid() / lssar::kSchedXcds);
    hipLaunchKernelGGL((lssar::lssar_prep_bf16_kernel<D>), dim3(Lp / lssar::kBK, BH),
                       dim3(lssar::kThreads), 0, s, static_cast<const __bf16*>(k), fk,
                       static_cast<_Float16*>(kn16), sched, BH, L, Lp, per_xcd);
}

// Where the bf16 workspace parts start.
struct WsParts {
    float* fk;
    _Float16* kn16;
    int2* sched;
};
WsParts ws_parts(void* ws, const Layout& w)
{
    unsigned char* b = static_cast<unsigned char*>(ws);
    const size_t o_kn16 = w.fk_bytes;
    return {reinterpret_cast<float*>(b), reinterpret_cast<_Float16*>(b + o_kn16),
            reinterpret_cast<int2*>(b + o_kn16 + w.kn16_bytes)};
}

// fast_keys: also write the normalised f16 keys, which the bf16 Softplus
// kernels read, except the training forward's (exact scores throughout)
int run_prep(const void* k, void* ws, int B, int H, int L, int d, int dtype,
             hipStream_t s, bool fast_keys = true)
{
    const Layout w = layout(B, H, L, d, dtype);
    const long nrows = (long)B * H * L;
    if (dtype == LSSAR_BF16) {
        const WsParts pt = ws_parts(ws, w);
        void* kn16 = fast_keys ? pt.kn16 : nullptr;
        if (d == 64)
            launch_prep_bf16<64>(k, pt.fk, kn16, pt.sched, B * H, L, w.Lp, s);
        else
            launch_prep_bf16<128>(k, pt.fk, kn16, pt.sched, B * H, L, w.Lp, s);
    } else {
        double* fk = static_cast<double*>(ws);
        if (d == 64)
            launch_knorm_f32<64>(k, fk, nrows, s);
        else
            launch_knorm_f32<128>(k, fk, nrows, s);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return hip_fail(e);
    return LSSAR_OK;
}

template <int D, int P, int PHI, bool RW>
void launch_fwd(const void* q, const void* k, const void* v, void* ws, void* out, int BH, int L,
                int dtype, double lam_scale, float eps, int p, double* stats, hipStream_t s)
{
    const Layout w = layout(1, BH, L, D, dtype);
    if (dtype == LSSAR_BF16) {
        const int nqb = (L + lssar::kBQ16 - 1) / lssar::kBQ16;
        const WsParts pt = ws_parts(ws, w);
        const dim3 grid((unsigned)lssar::FwdSched(BH, nqb).grid());
        // the training forward (row statistics) computes exact scores
        if constexpr (PHI == lssar::kPhiSoftplus && RW) {
            if (stats) {
                hipLaunchKernelGGL((lssar::lssar_fwd_bf16_kernel<D, P, PHI, RW, true>), grid,
                                   dim3(lssar::kThreads), 0, s, static_cast<const __bf16*>(q),
                                   static_cast<const __bf16*>(k), nullptr,
                                   static_cast<const __bf16*>(v),
                                   static_cast<__bf16*>(out), pt.fk, pt.sched, L, lam_scale, eps,
                                   p, stats);
                return;
            }
        }
        hipLaunchKernelGGL((lssar::lssar_fwd_bf16_kernel<D, P, PHI, RW, false>), grid,
                           dim3(lssar::kThreads), 0, s, static_cast<const __bf16*>(q),
                           static_cast<const __bf16*>(k), pt.kn16, static_cast<const __bf16*>(v),
                           static_cast<__bf16*>(out),
                           pt.fk, pt.sched, L, lam_scale, eps, p, nullptr);
    } else {
        const int nqb = (L + lssar::kBQ32 - 1) / lssar::kBQ32;
        hipLaunchKernelGGL((lssar::lssar_fwd_f32_kernel<D, P, PHI, RW>),
                           dim3((unsigned)(nqb * BH)),
                           dim3(lssar::kThreads), 0, s, static_cast<const float*>(q),
                           static_cast<const float*>(k), static_cast<const float*>(v),
                           static_cast<float*>(out), static_cast<const double*>(ws), BH, L, nqb,
                           lam_scale, eps, p, stats);
    }
}

// What the attention kernel computes: the stage-1 map and whether stage 2
// (re-weighting) runs.
struct Variant {
    int phi;        // LSSAR_PHI_SOFTPLUS or LSSAR_PHI_SIGMOID
    bool reweight;  // false: stage 1 only, p and eps unused
};
constexpr Variant kLssar = {LSSAR_PHI_SOFTPLUS, true};

template <int D, int PHI>
void dispatch_p(const void* q, const void* k, const void* v, void* ws, void* out, int BH, int L,
                int dtype, double lam_scale, float eps, int p, double* stats, hipStream_t s)
{
#define LSSAR_LAUNCH(PV) \
    launch_fwd<D, PV, PHI, true>(q, k, v, ws, out, BH, L, dtype, lam_scale, eps, p, stats, s)
    if constexpr (PHI == lssar::kPhiSoftplus) {
        switch (p) {
        case 1: LSSAR_LAUNCH(1); break;
        case 2: LSSAR_LAUNCH(2); break;
        case 3: LSSAR_LAUNCH(3); break;
        case 15: LSSAR_LAUNCH(15); break;
        default: LSSAR_LAUNCH(0); break;
        }
    } else {
        switch (p) {
        case 3: LSSAR_LAUNCH(3); break;
        case 15: LSSAR_LAUNCH(15); break;
        default: LSSAR_LAUNCH(0); break;
        }
    }
#undef LSSAR_LAUNCH
}

// stats: null, or (the Softplus method only) where the rows' statistics go.
template <int D>
void dispatch_variant(const void* q, const void* k, const void* v, void* ws, void* out, int BH,
                      int L, int dtype, double lam_scale, float eps, int p, Variant var,
                      double* stats, hipStream_t s)
{
    if (!var.reweight)
        launch_fwd<D, 1, lssar::kPhiSoftplus, false>(q, k, v, ws, out, BH, L, dtype, lam_scale,
                                                     eps, p, nullptr, s);
    else if (var.phi == LSSAR_PHI_SIGMOID)
        dispatch_p<D, lssar::kPhiSigmoid>(q, k, v, ws, out, BH, L, dtype, lam_scale, eps, p,
                                          nullptr, s);
    else
        dispatch_p<D, lssar::kPhiSoftplus>(q, k, v, ws, out, BH, L, dtype, lam_scale, eps, p,
                                           stats, s);
}

int run_fwd(const void* q, const void* k, const void* v, void* ws, void* out, int B, int H, int L,
            int d, int p, float eps, int dtype, hipStream_t s, Variant var = kLssar,
            double* stats = nullptr)
{
    // log2(e) * ln(d): the per-row factor is this times ln(i) / |q_i|
    const double lam_scale = std::log((double)d) / std::log(2.0);
    if (d == 64)
        dispatch_variant<64>(q, k, v, ws, out, B * H, L, dtype, lam_scale, eps, p, var, stats, s);
    else
        dispatch_variant<128>(q, k, v, ws, out, B * H, L, dtype, lam_scale, eps, p, var, stats,
                              s);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return hip_fail(e);
    return LSSAR_OK;
}

// Row statistics buffer ([B, H, L, 2] doubles): non-null, 16-byte aligned,
// overlapping none of the other buffers.
int validate_stats(const void* stats, int B, int H, int L, std::initializer_list<const void*> ts,
                   size_t tbytes, const void* ws, size_t ws_bytes)
{
    if (!stats || !aligned16(stats))
        return LSSAR_EINVAL;
    const size_t sb = (size_t)B * H * L * 2 * sizeof(double);
    for (const void* t : ts)
        if (overlaps(stats, sb, t, tbytes))
            return LSSAR_EINVAL;
    if (overlaps(stats, sb, ws, ws_bytes))
        return LSSAR_EINVAL;
    return LSSAR_OK;
}

// Validation, prep and attention kernel on a caller-owned workspace; stats
// (the Softplus method only): null, or where the rows' statistics go.
int fwd_ws(const void* q, const void* k, const void* v, void* out, int B, int H, int L, int d,
           int p, float eps, int dtype, void* workspace, size_t workspace_bytes, void* stream,
           Variant var, double* stats = nullptr)
{
    int st = validate(q, k, v, out, B, H, L, d, p, eps, dtype);
    if (st != LSSAR_OK)
        return st;
    const size_t tbytes = (size_t)B * H * L * d * elem_bytes(dtype);
    st = validate_ws(workspace, workspace_bytes, layout(B, H, L, d, dtype), tbytes, q, k, v, out);
    if (st != LSSAR_OK)
        return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    // the training forward and the Sigmoid map (exact scores) do not read
    // the normalised keys
    const bool training = stats && var.phi == LSSAR_PHI_SOFTPLUS && var.reweight;
    st = run_prep(k, workspace, B, H, L, d, dtype, s, var.phi == LSSAR_PHI_SOFTPLUS && !training);
    if (st != LSSAR_OK)
        return st;
    return run_fwd(q, k, v, workspace, out, B, H, L, d, p, eps, dtype, s, var, stats);
}

// ---------------------------------------------------------------------------
// Decode step
// ---------------------------------------------------------------------------

// Workspace: [scores: C per cache row][part1: 2 C per chunk][part2: d+1 C per
// chunk], C = fp32 for bf16 inputs and fp64 for fp32 inputs, each part
// rounded up to 256 bytes.  Chunks: 16384 / d cache rows.
struct DecLayout {
    size_t scores_bytes, part1_bytes, part2_bytes;
    int nsplit;
    size_t total() const { return scores_bytes + part1_bytes + part2_bytes; }
};

DecLayout dec_layout(long long B, long long H, long long Lmax, int d, int dtype)
{
    DecLayout w;
    const size_t cb = dtype == LSSAR_F32 ? 8 : 4;
    const int chunk = lssar::dec_chunk(d);
    w.nsplit = (int)((Lmax + chunk - 1) / chunk);
    const size_t bh = (size_t)(B * H);
    w.scores_bytes = round256(cb * bh * (size_t)Lmax);
    w.part1_bytes = round256(cb * bh * (size_t)w.nsplit * 2);
    w.part2_bytes = round256(cb * bh * (size_t)w.nsplit * (size_t)(d + 1));
    return w;
}

int validate_decode_shape(int B, int H, int Lmax, int d, int dtype)
{
    int st = validate_shape(B, H, Lmax, d, dtype);
    if (st != LSSAR_OK)
        return st;
    const long long nsplit = (Lmax + lssar::dec_chunk(d) - 1) / lssar::dec_chunk(d);
    if ((long long)B * H * nsplit > (1LL << 31) - 1)
        return LSSAR_EINVAL;
    return LSSAR_OK;
}

// Heads from which the bf16 decode step runs as one launch with one
// workgroup per head (lssar_decode_fused_kernel).  One such workgroup reads
// about 37 GB/s, the split path about 6.6 TB/s in all, so below about 180
// heads the split path is faster: with 192 heads (B16 H12, 8192 rows,
// d = 64) the one-launch path took 63.2 us against 68.0 us, with 128 heads
// (B4 H32, 4096 rows, d = 128) 46.7 us against 43.8 us.  (Lmax <= 2^22
// keeps a head's cache, at most 2^30 bytes, within the 32-bit byte offsets
// of its buffer loads.)
constexpr int kDecFusedMinHeads = 176;

template <typename T, int D, int P>
void launch_decode(const void* q, const void* kc, const void* vc, const int* lens, void* out,
                   void* ws, int B, int H, int Lmax, int p, float eps, double lam_scale,
                   hipStream_t s)
{
    using C = typename lssar::DecTraits<T>::C;
    const DecLayout w = dec_layout(B, H, Lmax, D, std::is_same<T, float>::value ? LSSAR_F32
                                                                                 : LSSAR_BF16);
    auto* base = static_cast<unsigned char*>(ws);
    C* scores = reinterpret_cast<C*>(base);
    C* part1 = reinterpret_cast<C*>(base + w.scores_bytes);
    C* part2 = reinterpret_cast<C*>(base + w.scores_bytes + w.part1_bytes);
    const int BH = B * H;
    // bf16 with enough heads to fill the part: one workgroup per head, one
    // launch (the Softplus values go to the scores area)
    if constexpr (std::is_same<T, __bf16>::value) {
        if (BH >= kDecFusedMinHeads) {
            hipLaunchKernelGGL((lssar::lssar_decode_fused_kernel<D, P>), dim3((unsigned)BH),
                               dim3(lssar::kDecFusedThreads), 0, s, static_cast<const T*>(q),
                               static_cast<const T*>(kc), static_cast<const T*>(vc), lens,
                               scores, static_cast<T*>(out), H, Lmax, lam_scale, eps, p);
            return;
        }
    }
    const unsigned grid = (unsigned)((long long)BH * w.nsplit);
    hipLaunchKernelGGL((lssar::lssar_decode_scores_kernel<T, D>), dim3(grid),
                       dim3(lssar::kDecThreads), 0, s, static_cast<const T*>(q),
                       static_cast<const T*>(kc), lens, scores, part1, H, Lmax, w.nsplit,
                       lam_scale);
    hipLaunchKernelGGL((lssar::lssar_decode_pv_kernel<T, D, P>), dim3(grid),
                       dim3(lssar::kDecThreads), 0, s, static_cast<const T*>(vc), lens,
                       scores, part1, part2, H, Lmax, w.nsplit, eps, p);
    hipLaunchKernelGGL((lssar::lssar_decode_combine_kernel<T, D>), dim3((unsigned)BH),
                       dim3(lssar::kDecThreads), 0, s, lens, part2, static_cast<T*>(out), H, Lmax,
                       w.nsplit);
}

template <typename T, int D>
void decode_dispatch_p(const void* q, const void* kc, const void* vc, const int* lens, void* out,
                       void* ws, int B, int H, int Lmax, int p, float eps, double lam_scale,
                       hipStream_t s)
{
    switch (p) {
    case 3: launch_decode<T, D, 3>(q, kc, vc, lens, out, ws, B, H, Lmax, p, eps, lam_scale, s); break;
    case 15: launch_decode<T, D, 15>(q, kc, vc, lens, out, ws, B, H, Lmax, p, eps, lam_scale, s); break;
    default: launch_decode<T, D, 0>(q, kc, vc, lens, out, ws, B, H, Lmax, p, eps, lam_scale, s); break;
    }
}

// ---------------------------------------------------------------------------
// Backward
// ---------------------------------------------------------------------------

// Workspace: [rq: C per query row][fk: C per key row][stats: 8 C per query
// row], C = fp32 for bf16 inputs and fp64 for fp32 inputs; each part rounded
// up to 256 bytes.
struct BwdLayout {
    size_t rq_bytes, fk_bytes, st_bytes;
    size_t total() const { return rq_bytes + fk_bytes + st_bytes; }
};

BwdLayout bwd_layout(long long B, long long H, long long L, int d, int dtype)
{
    const size_t cb = dtype == LSSAR_F32 ? 8 : 4;
    const size_t rows = (size_t)(B * H * L);
    BwdLayout w;
    w.rq_bytes = round256(cb * rows);
    w.fk_bytes = round256(cb * rows);
    w.st_bytes = round256(cb * rows * lssar::kBwdRowStats);
    return w;
}

// saved, out: null (the row statistics are recomputed), or the training
// forward's row statistics and output.
template <typename T, int D, int P>
void launch_bwd(const void* q, const void* k, const void* v, const void* dout, void* dq, void* dk,
                void* dv, void* ws, int BH, int L, int p, float eps, double lam_scale,
                const double* saved, const void* out, hipStream_t s)
{
    using C = typename lssar::DecTraits<T>::C;
    constexpr bool BF = std::is_same<T, __bf16>::value;
    const BwdLayout w = bwd_layout(1, BH, L, D, BF ? LSSAR_BF16 : LSSAR_F32);
    const long nrows = (long)BH * L;
    auto* base = static_cast<unsigned char*>(ws);
    C* rq = reinterpret_cast<C*>(base);
    C* fk = reinterpret_cast<C*>(base + w.rq_bytes);
    C* st = reinterpret_cast<C*>(base + w.rq_bytes + w.fk_bytes);
    const T* Q = static_cast<const T*>(q);
    const T* K = static_cast<const T*>(k);
    const T* V = static_cast<const T*>(v);
    const T* G = static_cast<const T*>(dout);
    const unsigned g4 = (unsigned)((nrows + 3) / 4);
    if constexpr (BF) {
        const int nqb = (L + 63) / 64, npair = (nqb + 1) / 2;
        hipLaunchKernelGGL((lssar::lssar_bwd_prep_kernel<D>), dim3((unsigned)nqb, BH),
                           dim3(lssar::kThreads), 0, s, Q, K, rq, fk, L);
        // d = 64: block pairs; d = 128: single blocks in the forward's order
        const dim3 grid(D == 64 ? (unsigned)(npair * BH) : (unsigned)lssar::FwdSched(BH, nqb).grid());
        bool fused = false;
        if constexpr (D == 64) {
            if (saved) {
                // row coefficients and dq in one pass over the keys
                hipLaunchKernelGGL((lssar::lssar_bwd_qside_kernel<D, P, 2>), grid,
                                   dim3(lssar::kThreads), 0, s, Q, K, V, G, rq, fk, st,
                                   static_cast<__bf16*>(dq), BH, L, nqb, npair, lam_scale, eps, p,
                                   saved, static_cast<const __bf16*>(out));
                fused = true;
            }
        }
        if (!fused) {
            hipLaunchKernelGGL((lssar::lssar_bwd_qside_kernel<D, P, 0>), grid,
                               dim3(lssar::kThreads), 0, s, Q, K, V, G, rq, fk, st,
                               static_cast<__bf16*>(dq), BH, L, nqb, npair, lam_scale, eps, p,
                               saved, nullptr);
            hipLaunchKernelGGL((lssar::lssar_bwd_qside_kernel<D, P, 1>), grid,
                               dim3(lssar::kThreads), 0, s, Q, K, V, G, rq, fk, st,
                               static_cast<__bf16*>(dq), BH, L, nqb, npair, lam_scale, eps, p,
                               nullptr, nullptr);
        }
        hipLaunchKernelGGL((lssar::lssar_bwd_kside_kernel<D, P>), grid, dim3(lssar::kThreads), 0,
                           s, Q, K, V, G, fk, st, static_cast<__bf16*>(dk),
                           static_cast<__bf16*>(dv), BH, L, nqb, npair, p);
        return;
    } else {
        constexpr int rpb = lssar::kBwdThreads / (D / lssar::DecTraits<T>::EPL);
        hipLaunchKernelGGL((lssar::lssar_bwd_norms_kernel<T, D>),
                           dim3((unsigned)((nrows + rpb - 1) / rpb)), dim3(lssar::kBwdThreads), 0,
                           s, Q, K, rq, fk, nrows);
        hipLaunchKernelGGL((lssar::lssar_bwd_rowstats_kernel<T, D, P>), dim3(g4),
                           dim3(lssar::kBwdThreads), 0, s, Q, K, V, G, rq, fk, st, L, nrows,
                           lam_scale, eps, p, saved);
        hipLaunchKernelGGL((lssar::lssar_bwd_dq_kernel<T, D, P>), dim3(g4),
                           dim3(lssar::kBwdThreads), 0, s, Q, K, V, G, fk, st,
                           static_cast<T*>(dq), L, nrows, p);
    }
    hipLaunchKernelGGL((lssar::lssar_bwd_dkdv_kernel<T, D, P>), dim3(g4),
                       dim3(lssar::kBwdThreads), 0, s, Q, K, V, G, fk, st, static_cast<T*>(dk),
                       static_cast<T*>(dv), L, nrows, p);
}

template <typename T, int D>
void bwd_dispatch_p(const void* q, const void* k, const void* v, const void* dout, void* dq,
                    void* dk, void* dv, void* ws, int BH, int L, int p, float eps,
                    double lam_scale, const double* saved, const void* out, hipStream_t s)
{
#define LSSAR_BWD(PV) \
    launch_bwd<T, D, PV>(q, k, v, dout, dq, dk, dv, ws, BH, L, p, eps, lam_scale, saved, out, s)
    switch (p) {
    case 1: LSSAR_BWD(1); break;
    case 2: LSSAR_BWD(2); break;
    case 3: LSSAR_BWD(3); break;
    case 15: LSSAR_BWD(15); break;
    default: LSSAR_BWD(0); break;
    }
#undef LSSAR_BWD
}

}  // namespace

extern "C" {

size_t lssar_workspace_bytes(int B, int H, int L, int d, int dtype)
{
    if (validate_shape(B, H, L, d, dtype) != LSSAR_OK)
        return 0;
    return layout(B, H, L, d, dtype).total();
}

int lssar_attn_fwd_ws(const void* q, const void* k, const void* v, void* out, int B, int H, int L,
                      int d, int p, float eps, int dtype, void* workspace, size_t workspace_bytes,
                      void* stream)
{
    return fwd_ws(q, k, v, out, B, H, L, d, p, eps, dtype, workspace, workspace_bytes, stream,
                  kLssar);
}

int lssar_attn_fwd_stats_ws(const void* q, const void* k, const void* v, void* out,
                            double* row_stats, int B, int H, int L, int d, int p, float eps,
                            int dtype, void* workspace, size_t workspace_bytes, void* stream)
{
    int st = validate_shape(B, H, L, d, dtype);
    if (st != LSSAR_OK)
        return st;
    const size_t tb = (size_t)B * H * L * d * elem_bytes(dtype);
    st = validate_stats(row_stats, B, H, L, {q, k, v, out}, tb, workspace,
                        workspace ? layout(B, H, L, d, dtype).total() : 0);
    if (st != LSSAR_OK)
        return st;
    return fwd_ws(q, k, v, out, B, H, L, d, p, eps, dtype, workspace, workspace_bytes, stream,
                  kLssar, row_stats);
}

int lssar_attn_fwd_phi_ws(const void* q, const void* k, const void* v, void* out, int B, int H,
                          int L, int d, int p, float eps, int phi, int dtype, void* workspace,
                          size_t workspace_bytes, void* stream)
{
    if (phi != LSSAR_PHI_SOFTPLUS && phi != LSSAR_PHI_SIGMOID)
        return LSSAR_EUNSUPPORTED;
    return fwd_ws(q, k, v, out, B, H, L, d, p, eps, dtype, workspace, workspace_bytes, stream,
                  Variant{phi, true});
}

int lssar_lssa_fwd_ws(const void* q, const void* k, const void* v, void* out, int B, int H, int L,
                      int d, int dtype, void* workspace, size_t workspace_bytes, void* stream)
{
    // p and eps take no part in stage 1; valid placeholders pass validation
    return fwd_ws(q, k, v, out, B, H, L, d, 1, 0.0f, dtype, workspace, workspace_bytes, stream,
                  Variant{LSSAR_PHI_SOFTPLUS, false});
}

int lssar_attn_fwd(const void* q, const void* k, const void* v, void* out, int B, int H, int L,
                   int d, int p, float eps, int dtype, void* stream)
{
    int st = validate(q, k, v, out, B, H, L, d, p, eps, dtype);
    if (st != LSSAR_OK)
        return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const size_t bytes = layout(B, H, L, d, dtype).total();
    void* ws = nullptr;
    hipError_t e = hipMallocAsync(&ws, bytes, s);
    if (e != hipSuccess)
        return hip_fail(e);
    st = run_prep(k, ws, B, H, L, d, dtype, s);
    if (st == LSSAR_OK)
        st = run_fwd(q, k, v, ws, out, B, H, L, d, p, eps, dtype, s);
    e = hipFreeAsync(ws, s);
    if (st == LSSAR_OK && e != hipSuccess)
        return hip_fail(e);
    return st;
}

// Workspace of lssar_attn_fwd_noalloc: a file-scope device array, one copy
// per GPU the library runs on, held until the process ends.  Host code never
// uses its name as an address (on the host it is only a stand-in): each
// device's address comes from hipGetSymbolAddress, taken once per device
// with that device current, and is what the kernels receive.
constexpr size_t kScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];
std::once_flag g_scratch_once[kMaxDevices];

// The current device's copy of `scratch`.
int scratch_of_current_device(void** ptr)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return hip_fail(e);
    if (dev < 0 || dev >= kMaxDevices)
        return LSSAR_EUNSUPPORTED;
    std::call_once(g_scratch_once[dev], [dev] {
        g_scratch_err[dev] = hipGetSymbolAddress(&g_scratch_ptr[dev], HIP_SYMBOL(scratch));
    });
    if (g_scratch_err[dev] != hipSuccess)
        return hip_fail(g_scratch_err[dev]);
    *ptr = g_scratch_ptr[dev];
    return LSSAR_OK;
}
}  // namespace

int lssar_attn_fwd_noalloc(const void* q, const void* k, const void* v, void* out, int B, int H,
                           int L, int d, int p, float eps, int dtype, void* stream)
{
    int st = validate(q, k, v, out, B, H, L, d, p, eps, dtype);
    if (st != LSSAR_OK)
        return st;
    if (layout(B, H, L, d, dtype).total() > kScratchBytes)
        return LSSAR_ESCRATCH;
    void* ws = nullptr;
    st = scratch_of_current_device(&ws);
    if (st != LSSAR_OK)
        return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    st = run_prep(k, ws, B, H, L, d, dtype, s);
    if (st != LSSAR_OK)
        return st;
    return run_fwd(q, k, v, ws, out, B, H, L, d, p, eps, dtype, s);
}

size_t lssar_noalloc_scratch_bytes(void) { return kScratchBytes; }

int lssar_prep(const void* k, void* workspace, size_t workspace_bytes, int B, int H, int L,
               int d, int dtype, void* stream)
{
    if (!k)
        return LSSAR_EINVAL;
    int st = validate_shape(B, H, L, d, dtype);
    if (st != LSSAR_OK)
        return st;
    if (!aligned16(k))
        return LSSAR_EINVAL;
    const size_t tbytes = (size_t)B * H * L * d * elem_bytes(dtype);
    st = validate_ws(workspace, workspace_bytes, layout(B, H, L, d, dtype), tbytes, k, nullptr,
                     nullptr, nullptr);
    if (st != LSSAR_OK)
        return st;
    return run_prep(k, workspace, B, H, L, d, dtype, static_cast<hipStream_t>(stream));
}

int lssar_attn_fwd_prepped(const void* q, const void* k, const void* v, void* workspace,
                           size_t workspace_bytes, void* out, int B, int H, int L, int d, int p,
                           float eps, int dtype, void* stream)
{
    int st = validate(q, k, v, out, B, H, L, d, p, eps, dtype);
    if (st != LSSAR_OK)
        return st;
    const size_t tbytes = (size_t)B * H * L * d * elem_bytes(dtype);
    st = validate_ws(workspace, workspace_bytes, layout(B, H, L, d, dtype), tbytes, q, k, v, out);
    if (st != LSSAR_OK)
        return st;
    return run_fwd(q, k, v, workspace, out, B, H, L, d, p, eps, dtype,
                   static_cast<hipStream_t>(stream));
}

size_t lssar_decode_workspace_bytes(int B, int H, int Lmax, int d, int dtype)
{
    if (validate_decode_shape(B, H, Lmax, d, dtype) != LSSAR_OK)
        return 0;
    return dec_layout(B, H, Lmax, d, dtype).total();
}

int lssar_decode_ws(const void* q, const void* k_cache, const void* v_cache, const int* lens,
                    void* out, int B, int H, int Lmax, int d, int p, float eps, int dtype,
                    void* workspace, size_t workspace_bytes, void* stream)
{
    if (!q || !k_cache || !v_cache || !out)
        return LSSAR_EINVAL;
    if (p < 1 || !(eps >= 0.0f) || !std::isfinite(eps))
        return LSSAR_EINVAL;
    int st = validate_decode_shape(B, H, Lmax, d, dtype);
    if (st != LSSAR_OK)
        return st;
    if (p > kMaxP)
        return LSSAR_EUNSUPPORTED;
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out) ||
        (reinterpret_cast<uintptr_t>(lens) & 3u) != 0)
        return LSSAR_EINVAL;
    const size_t eb = elem_bytes(dtype);
    const size_t qbytes = (size_t)B * H * d * eb;
    const size_t cbytes = (size_t)B * H * Lmax * d * eb;
    const size_t lbytes = lens ? (size_t)B * sizeof(int) : 0;
    if (overlaps(out, qbytes, q, qbytes) || overlaps(out, qbytes, k_cache, cbytes) ||
        overlaps(out, qbytes, v_cache, cbytes) || (lens && overlaps(out, qbytes, lens, lbytes)))
        return LSSAR_EINVAL;
    const DecLayout w = dec_layout(B, H, Lmax, d, dtype);
    if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0 ||
        workspace_bytes < w.total())
        return LSSAR_EWORKSPACE;
    if (overlaps(workspace, w.total(), q, qbytes) || overlaps(workspace, w.total(), k_cache, cbytes) ||
        overlaps(workspace, w.total(), v_cache, cbytes) || overlaps(workspace, w.total(), out, qbytes) ||
        (lens && overlaps(workspace, w.total(), lens, lbytes)))
        return LSSAR_EWORKSPACE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const double lam_scale = std::log((double)d) / std::log(2.0);
    if (dtype == LSSAR_BF16) {
        if (d == 64)
            decode_dispatch_p<__bf16, 64>(q, k_cache, v_cache, lens, out, workspace, B, H, Lmax,
                                          p, eps, lam_scale, s);
        else
            decode_dispatch_p<__bf16, 128>(q, k_cache, v_cache, lens, out, workspace, B, H, Lmax,
                                           p, eps, lam_scale, s);
    } else {
        if (d == 64)
            decode_dispatch_p<float, 64>(q, k_cache, v_cache, lens, out, workspace, B, H, Lmax,
                                         p, eps, lam_scale, s);
        else
            decode_dispatch_p<float, 128>(q, k_cache, v_cache, lens, out, workspace, B, H, Lmax,
                                          p, eps, lam_scale, s);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return hip_fail(e);
    return LSSAR_OK;
}

size_t lssar_bwd_workspace_bytes(int B, int H, int L, int d, int dtype)
{
    if (validate_shape(B, H, L, d, dtype) != LSSAR_OK)
        return 0;
    return bwd_layout(B, H, L, d, dtype).total();
}

}  // extern "C"

namespace {

// Validation and launch of the backward; saved, out: null, or the training
// forward's row statistics and output (validated by the caller).
int bwd_ws(const void* q, const void* k, const void* v, const void* dout, void* dq, void* dk,
           void* dv, int B, int H, int L, int d, int p, float eps, int dtype, void* workspace,
           size_t workspace_bytes, void* stream, const double* saved, const void* out)
{
    if (!dout || !dq || !dk || !dv)
        return LSSAR_EINVAL;
    // q, k, v, sizes, p, eps, dtype and alignment as for the forward, with dq
    // standing in for out (it must not overlap q, k or v)
    int st = validate(q, k, v, dq, B, H, L, d, p, eps, dtype);
    if (st != LSSAR_OK)
        return st;
    if (!aligned16(dout) || !aligned16(dk) || !aligned16(dv))
        return LSSAR_EINVAL;
    const size_t tb = (size_t)B * H * L * d * elem_bytes(dtype);
    const void* ins[4] = {q, k, v, dout};
    const void* outs[3] = {dq, dk, dv};
    for (const void* o : outs) {
        for (const void* in : ins)
            if (overlaps(o, tb, in, tb))
                return LSSAR_EINVAL;
    }
    if (overlaps(dq, tb, dk, tb) || overlaps(dq, tb, dv, tb) || overlaps(dk, tb, dv, tb))
        return LSSAR_EINVAL;
    const BwdLayout w = bwd_layout(B, H, L, d, dtype);
    if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0 ||
        workspace_bytes < w.total())
        return LSSAR_EWORKSPACE;
    for (const void* t : {q, k, v, dout, static_cast<const void*>(dq), static_cast<const void*>(dk),
                          static_cast<const void*>(dv)})
        if (overlaps(workspace, w.total(), t, tb))
            return LSSAR_EWORKSPACE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const double lam_scale = std::log((double)d) / std::log(2.0);
    const int BH = B * H;
    if (dtype == LSSAR_BF16) {
        if (d == 64)
            bwd_dispatch_p<__bf16, 64>(q, k, v, dout, dq, dk, dv, workspace, BH, L, p, eps,
                                       lam_scale, saved, out, s);
        else
            bwd_dispatch_p<__bf16, 128>(q, k, v, dout, dq, dk, dv, workspace, BH, L, p, eps,
                                        lam_scale, saved, out, s);
    } else {
        if (d == 64)
            bwd_dispatch_p<float, 64>(q, k, v, dout, dq, dk, dv, workspace, BH, L, p, eps,
                                      lam_scale, saved, out, s);
        else
            bwd_dispatch_p<float, 128>(q, k, v, dout, dq, dk, dv, workspace, BH, L, p, eps,
                                       lam_scale, saved, out, s);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return hip_fail(e);
    return LSSAR_OK;
}

}  // namespace

extern "C" {

int lssar_attn_bwd_ws(const void* q, const void* k, const void* v, const void* dout, void* dq,
                      void* dk, void* dv, int B, int H, int L, int d, int p, float eps, int dtype,
                      void* workspace, size_t workspace_bytes, void* stream)
{
    return bwd_ws(q, k, v, dout, dq, dk, dv, B, H, L, d, p, eps, dtype, workspace,
                  workspace_bytes, stream, nullptr, nullptr);
}

int lssar_attn_bwd_stats_ws(const void* q, const void* k, const void* v, const void* out,
                            const void* dout, const double* row_stats, void* dq, void* dk,
                            void* dv, int B, int H, int L, int d, int p, float eps, int dtype,
                            void* workspace, size_t workspace_bytes, void* stream)
{
    int st = validate_shape(B, H, L, d, dtype);
    if (st != LSSAR_OK)
        return st;
    if (!dq || !dk || !dv || !out || !aligned16(out))
        return LSSAR_EINVAL;
    // inputs: they may share memory with other inputs, not with outputs or the workspace
    const size_t tb = (size_t)B * H * L * d * elem_bytes(dtype);
    const size_t wsb = workspace ? bwd_layout(B, H, L, d, dtype).total() : 0;
    st = validate_stats(row_stats, B, H, L, {dq, dk, dv}, tb, workspace, wsb);
    if (st != LSSAR_OK)
        return st;
    for (const void* o : {dq, dk, dv})
        if (overlaps(out, tb, o, tb))
            return LSSAR_EINVAL;
    if (overlaps(out, tb, workspace, wsb))
        return LSSAR_EINVAL;
    return bwd_ws(q, k, v, dout, dq, dk, dv, B, H, L, d, p, eps, dtype, workspace,
                  workspace_bytes, stream, row_stats, out);
}

const char* lssar_status_str(int status)
{
    switch (status) {
    case LSSAR_OK: return "ok";
    case LSSAR_EINVAL: return "invalid argument";
    case LSSAR_EUNSUPPORTED: return "unsupported head dimension, dtype, p or length";
    case LSSAR_EWORKSPACE: return "workspace missing, misaligned, too small or overlapping";
    case LSSAR_EHIP: return "HIP runtime error (see lssar_last_hip_error)";
    case LSSAR_ESCRATCH:
        return "input needs more workspace than lssar_attn_fwd_noalloc's static scratch "
               "(lssar_noalloc_scratch_bytes)";
    default: return "unknown status";
    }
}

int lssar_last_hip_error(void) { return g_last_hip_error; }

int lssar_version(void) { return 910; }

long long lssar_fwd_schedule(int B, int H, int L, int* items, long long capacity)
{
    if (validate_shape(B, H, L, 64, LSSAR_BF16) != LSSAR_OK)
        return LSSAR_EINVAL;
    const int BH = B * H, nqb = (L + lssar::kBQ16 - 1) / lssar::kBQ16;
    const lssar::FwdSched sc(BH, nqb);
    const long long grid = sc.grid();
    if (items) {
        if (capacity < grid)
            return LSSAR_EINVAL;
        for (long long w = 0; w < grid; ++w) {
            int bh, qb;
            items[w] = sc.item((int)w, bh, qb) ? bh * nqb + qb : -1;
        }
    }
    return grid;
}

}  // extern "C"
