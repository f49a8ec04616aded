// lssar.hip -- C ABI of the LSSAR causal attention forward on gfx950.
//
// Declarations, argument meaning, layout, ownership and error behaviour are
// documented in include/lssar.h.  Method: paper note "Softplus Attention with
// Re-weighting Boosts Length Extrapolation in Large Language Models",
// Method details, Key designs 1-3.  This file validates arguments on the
// host (before any HIP call), picks the kernel instantiation and launches
// the prep kernel and the attention kernel on the caller's stream.
#include "lssar.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <type_traits>

#include "lssar_device.hpp"

namespace {

thread_local int g_last_hip_error = 0;

constexpr int kMaxL = 1 << 24;
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

size_t ws_bytes(long long B, long long H, long long L)
{
    const size_t raw = (size_t)(4 * B * H * L);
    return (raw + 255) & ~(size_t)255;
}

int validate(const void* q, const void* k, const void* v, const void* out, int B, int H,
             int L, int d, int p, float eps, int dtype)
{
    if (!q || !k || !v || !out)
        return LSSAR_EINVAL;
    if (B < 1 || H < 1 || L < 1 || p < 1 || !(eps >= 0.0f) || !std::isfinite(eps))
        return LSSAR_EINVAL;
    if (dtype != LSSAR_F32 && dtype != LSSAR_BF16)
        return LSSAR_EUNSUPPORTED;
    if (d != 64 && d != 128)
        return LSSAR_EUNSUPPORTED;
    if (p > kMaxP || L > kMaxL)
        return LSSAR_EUNSUPPORTED;
    const long long bh = (long long)B * H;
    const long long nqb = (L + lssar::kBQ - 1) / lssar::kBQ;
    if (bh > (1LL << 31) - 1 || bh * nqb > (1LL << 31) - 1)
        return LSSAR_EINVAL;
    const long long elems = bh * L * d;
    if (elems > (1LL << 46))
        return LSSAR_EINVAL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
        return LSSAR_EINVAL;
    const size_t bytes = (size_t)elems * (dtype == LSSAR_F32 ? 4 : 2);
    if (overlaps(out, bytes, q, bytes) || overlaps(out, bytes, k, bytes) ||
        overlaps(out, bytes, v, bytes))
        return LSSAR_EINVAL;
    return LSSAR_OK;
}

template <typename T, int D>
void launch_prep(const void* k, float* fk, long nrows, hipStream_t s)
{
    constexpr int lpr = D / (16 / (int)sizeof(T));
    constexpr int rpb = lssar::kThreads / lpr;
    const unsigned grid = (unsigned)((nrows + rpb - 1) / rpb);
    hipLaunchKernelGGL((lssar::lssar_prep_kernel<T, D>), dim3(grid), dim3(lssar::kThreads), 0, s,
                       static_cast<const T*>(k), fk, nrows);
}

template <int D, int P>
void launch_fwd(const void* q, const void* k, const void* v, void* out, const float* fk, int BH,
                int L, int dtype, double lam_scale, float eps, int p, hipStream_t s)
{
    const int nqb = (L + lssar::kBQ - 1) / lssar::kBQ;
    const dim3 grid((unsigned)(nqb * BH));
    if (dtype == LSSAR_BF16) {
        hipLaunchKernelGGL((lssar::lssar_fwd_bf16_kernel<D, P>), grid, dim3(lssar::kThreads), 0, s,
                           static_cast<const __bf16*>(q), static_cast<const __bf16*>(k),
                           static_cast<const __bf16*>(v), static_cast<__bf16*>(out), fk, BH, L,
                           nqb, lam_scale, eps, p);
    } else {
        hipLaunchKernelGGL((lssar::lssar_fwd_f32_kernel<D, P>), grid, dim3(lssar::kThreads), 0, s,
                           static_cast<const float*>(q), static_cast<const float*>(k),
                           static_cast<const float*>(v), static_cast<float*>(out), fk, BH, L, nqb,
                           lam_scale, eps, p);
    }
}

template <int D>
void dispatch_p(const void* q, const void* k, const void* v, void* out, const float* fk, int BH,
                int L, int dtype, double lam_scale, float eps, int p, hipStream_t s)
{
    switch (p) {
    case 1: launch_fwd<D, 1>(q, k, v, out, fk, BH, L, dtype, lam_scale, eps, p, s); break;
    case 2: launch_fwd<D, 2>(q, k, v, out, fk, BH, L, dtype, lam_scale, eps, p, s); break;
    case 3: launch_fwd<D, 3>(q, k, v, out, fk, BH, L, dtype, lam_scale, eps, p, s); break;
    case 15: launch_fwd<D, 15>(q, k, v, out, fk, BH, L, dtype, lam_scale, eps, p, s); break;
    default: launch_fwd<D, 0>(q, k, v, out, fk, BH, L, dtype, lam_scale, eps, p, s); break;
    }
}

int run_prep(const void* k, float* fk, int B, int H, int L, int d, int dtype, hipStream_t s)
{
    const long nrows = (long)B * H * L;
    if (dtype == LSSAR_BF16) {
        if (d == 64)
            launch_prep<__bf16, 64>(k, fk, nrows, s);
        else
            launch_prep<__bf16, 128>(k, fk, nrows, s);
    } else {
        if (d == 64)
            launch_prep<float, 64>(k, fk, nrows, s);
        else
            launch_prep<float, 128>(k, fk, nrows, s);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return hip_fail(e);
    return LSSAR_OK;
}

int run_fwd(const void* q, const void* k, const void* v, const float* fk, void* out, int B, int H,
            int L, int d, int p, float eps, int dtype, hipStream_t s)
{
    const int BH = B * H;
    // log2(e) * ln(d): the per-row factor is this times ln(i) / |q_i|
    const double lam_scale = std::log((double)d) / std::log(2.0);
    if (d == 64)
        dispatch_p<64>(q, k, v, out, fk, BH, L, dtype, lam_scale, eps, p, s);
    else
        dispatch_p<128>(q, k, v, out, fk, BH, L, dtype, lam_scale, eps, p, s);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return hip_fail(e);
    return LSSAR_OK;
}

int run(const void* q, const void* k, const void* v, void* out, int B, int H, int L, int d, int p,
        float eps, int dtype, void* ws, hipStream_t s)
{
    float* fk = static_cast<float*>(ws);
    int st = run_prep(k, fk, B, H, L, d, dtype, s);
    if (st != LSSAR_OK)
        return st;
    return run_fwd(q, k, v, fk, out, B, H, L, d, p, eps, dtype, s);
}

}  // namespace

extern "C" {

size_t lssar_workspace_bytes(int B, int H, int L, int d, int dtype)
{
    if (B < 1 || H < 1 || L < 1 || (d != 64 && d != 128) ||
        (dtype != LSSAR_F32 && dtype != LSSAR_BF16) || L > kMaxL)
        return 0;
    return ws_bytes(B, H, L);
}

int lssar_attn_fwd_ws(const void* q, const void* k, const void* v, void* out, int B, int H, int L,
                      int d, int p, float eps, int dtype, void* workspace, size_t workspace_bytes,
                      void* stream)
{
    int st = validate(q, k, v, out, B, H, L, d, p, eps, dtype);
    if (st != LSSAR_OK)
        return st;
    const size_t need = ws_bytes(B, H, L);
    if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0 ||
        workspace_bytes < need)
        return LSSAR_EWORKSPACE;
    const size_t bytes = (size_t)B * H * L * d * (dtype == LSSAR_F32 ? 4 : 2);
    if (overlaps(workspace, need, q, bytes) || overlaps(workspace, need, k, bytes) ||
        overlaps(workspace, need, v, bytes) || overlaps(workspace, need, out, bytes))
        return LSSAR_EWORKSPACE;
    return run(q, k, v, out, B, H, L, d, p, eps, dtype, workspace, static_cast<hipStream_t>(stream));
}

int lssar_attn_fwd(const void* q, const void* k, const void* v, void* out, int B, int H, int L,
                   int d, int p, float eps, int dtype, void* stream)
{
    int st = validate(q, k, v, out, B, H, L, d, p, eps, dtype);
    if (st != LSSAR_OK)
        return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    void* ws = nullptr;
    hipError_t e = hipMallocAsync(&ws, ws_bytes(B, H, L), s);
    if (e != hipSuccess)
        return hip_fail(e);
    st = run(q, k, v, out, B, H, L, d, p, eps, dtype, ws, s);
    e = hipFreeAsync(ws, s);
    if (st == LSSAR_OK && e != hipSuccess)
        return hip_fail(e);
    return st;
}

int lssar_key_inv_norms(const void* k, float* fk, int B, int H, int L, int d, int dtype,
                        void* stream)
{
    if (!k)
        return LSSAR_EINVAL;
    if (B < 1 || H < 1 || L < 1)
        return LSSAR_EINVAL;
    if (dtype != LSSAR_F32 && dtype != LSSAR_BF16)
        return LSSAR_EUNSUPPORTED;
    if (d != 64 && d != 128)
        return LSSAR_EUNSUPPORTED;
    if (L > kMaxL)
        return LSSAR_EUNSUPPORTED;
    const long long bh = (long long)B * H;
    if (bh > (1LL << 31) - 1 || bh * L * d > (1LL << 46))
        return LSSAR_EINVAL;
    if (!aligned16(k))
        return LSSAR_EINVAL;
    if (!fk || !aligned16(fk))
        return LSSAR_EWORKSPACE;
    const size_t kbytes = (size_t)(bh * L * d) * (dtype == LSSAR_F32 ? 4 : 2);
    const size_t fbytes = (size_t)(bh * L) * 4;
    if (overlaps(k, kbytes, fk, fbytes))
        return LSSAR_EWORKSPACE;
    return run_prep(k, fk, B, H, L, d, dtype, static_cast<hipStream_t>(stream));
}

int lssar_attn_fwd_prenormed(const void* q, const void* k, const void* v, const float* fk,
                             void* out, int B, int H, int L, int d, int p, float eps, int dtype,
                             void* stream)
{
    int st = validate(q, k, v, out, B, H, L, d, p, eps, dtype);
    if (st != LSSAR_OK)
        return st;
    if (!fk || !aligned16(fk))
        return LSSAR_EWORKSPACE;
    const size_t obytes = (size_t)B * H * L * d * (dtype == LSSAR_F32 ? 4 : 2);
    if (overlaps(out, obytes, fk, (size_t)B * H * L * 4))
        return LSSAR_EWORKSPACE;
    return run_fwd(q, k, v, fk, out, B, H, L, d, p, eps, dtype, static_cast<hipStream_t>(stream));
}

const char* lssar_status_str(int status)
{
    switch (status) {
    case LSSAR_OK: return "ok";
    case LSSAR_EINVAL: return "invalid argument";
    case LSSAR_EUNSUPPORTED: return "unsupported head dimension, dtype, p or length";
    case LSSAR_EWORKSPACE: return "workspace missing, misaligned or too small";
    case LSSAR_EHIP: return "HIP runtime error (see lssar_last_hip_error)";
    default: return "unknown status";
    }
}

int lssar_last_hip_error(void) { return g_last_hip_error; }

int lssar_version(void) { return 100; }

}  // extern "C"
