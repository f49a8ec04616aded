// issue_rates.hip -- instruction issue rates of a gfx950 (MI355X) SIMD, the
// basis of the attention kernels' issue roofline.
//
// For fp32 FMA, v_exp_f32, v_log_f32, v_pk_mul_f16 and the 16x16x32 bf16 and
// f16 MFMA, alone and mixed (in one wave, and in different waves on one
// SIMD), at 1, 2, 4 and 8 waves per SIMD: nanoseconds per instruction per
// SIMD from the kernel time (one launch of 256 or 512 workgroups covering
// every SIMD equally), plus each wave's own cycle count (clock64).
// ALU work only: each thread writes one float of its result and one wave
// counter; no other memory access.
//
// Build and run (one MI355X):
//   hipcc -O3 -std=c++17 --offload-arch=gfx950 -Xclang -target-feature \
//       -Xclang -packed-fp32-ops issue_rates.hip -o /tmp/issue_rates
//   /tmp/issue_rates
#include <hip/hip_runtime.h>
#include <cstdio>
#include <vector>
#include <algorithm>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

#define FMA8(a) \
    asm volatile("v_fma_f32 %0, %0, %1, %2" : "+v"(a[0]) : "v"(b), "v"(c)); \
    asm volatile("v_fma_f32 %0, %0, %1, %2" : "+v"(a[1]) : "v"(b), "v"(c)); \
    asm volatile("v_fma_f32 %0, %0, %1, %2" : "+v"(a[2]) : "v"(b), "v"(c)); \
    asm volatile("v_fma_f32 %0, %0, %1, %2" : "+v"(a[3]) : "v"(b), "v"(c)); \
    asm volatile("v_fma_f32 %0, %0, %1, %2" : "+v"(a[4]) : "v"(b), "v"(c)); \
    asm volatile("v_fma_f32 %0, %0, %1, %2" : "+v"(a[5]) : "v"(b), "v"(c)); \
    asm volatile("v_fma_f32 %0, %0, %1, %2" : "+v"(a[6]) : "v"(b), "v"(c)); \
    asm volatile("v_fma_f32 %0, %0, %1, %2" : "+v"(a[7]) : "v"(b), "v"(c));
#define EXP8(a) \
    asm volatile("v_exp_f32 %0, %0" : "+v"(a[0])); asm volatile("v_exp_f32 %0, %0" : "+v"(a[1])); \
    asm volatile("v_exp_f32 %0, %0" : "+v"(a[2])); asm volatile("v_exp_f32 %0, %0" : "+v"(a[3])); \
    asm volatile("v_exp_f32 %0, %0" : "+v"(a[4])); asm volatile("v_exp_f32 %0, %0" : "+v"(a[5])); \
    asm volatile("v_exp_f32 %0, %0" : "+v"(a[6])); asm volatile("v_exp_f32 %0, %0" : "+v"(a[7]));
#define LOG8(a) \
    asm volatile("v_log_f32 %0, %0" : "+v"(a[0])); asm volatile("v_log_f32 %0, %0" : "+v"(a[1])); \
    asm volatile("v_log_f32 %0, %0" : "+v"(a[2])); asm volatile("v_log_f32 %0, %0" : "+v"(a[3])); \
    asm volatile("v_log_f32 %0, %0" : "+v"(a[4])); asm volatile("v_log_f32 %0, %0" : "+v"(a[5])); \
    asm volatile("v_log_f32 %0, %0" : "+v"(a[6])); asm volatile("v_log_f32 %0, %0" : "+v"(a[7]));
#define PKF16_8(h) \
    asm volatile("v_pk_mul_f16 %0, %0, %1" : "+v"(h[0]) : "v"(hb)); asm volatile("v_pk_mul_f16 %0, %0, %1" : "+v"(h[1]) : "v"(hb)); \
    asm volatile("v_pk_mul_f16 %0, %0, %1" : "+v"(h[2]) : "v"(hb)); asm volatile("v_pk_mul_f16 %0, %0, %1" : "+v"(h[3]) : "v"(hb)); \
    asm volatile("v_pk_mul_f16 %0, %0, %1" : "+v"(h[4]) : "v"(hb)); asm volatile("v_pk_mul_f16 %0, %0, %1" : "+v"(h[5]) : "v"(hb)); \
    asm volatile("v_pk_mul_f16 %0, %0, %1" : "+v"(h[6]) : "v"(hb)); asm volatile("v_pk_mul_f16 %0, %0, %1" : "+v"(h[7]) : "v"(hb));

// MODE: 0 fma; 1 exp; 2 log; 3 mfma bf16 (4 independent accumulators);
// 4 mfma f16; 5 fma + mfma interleaved in one wave (8 fma : 1 mfma);
// 6 waves < nv do fma, the others mfma (split waves); 7 pk_mul_f16;
// 8 mfma bf16 dependent chain (1 accumulator); 9 exp + fma interleaved (1:1).
template <int MODE>
__global__ __launch_bounds__(1024) void kern(float* out, long long* cyc, int iters, int nv)
{
    const int tid = threadIdx.x, wave = tid >> 6;
    float a[8];
    for (int i = 0; i < 8; ++i) a[i] = 1.0f + 1e-3f * (tid + i);
    float b = 0.999f, c = 1e-3f;
    unsigned h[8];
    for (int i = 0; i < 8; ++i) h[i] = 0x3c003c00u + tid;
    unsigned hb = 0x3bff3bffu;
    f32x4 acc[4] = {};
    bf16x8 x, y;
    f16x8 xh, yh;
    for (int i = 0; i < 8; ++i) {
        x[i] = (__bf16)(0.01f * (tid & 7) + i);
        y[i] = (__bf16)(0.02f * i);
        xh[i] = (_Float16)(0.01f * (tid & 7) + i);
        yh[i] = (_Float16)(0.02f * i);
    }
    const bool do_valu = (MODE == 6 || MODE == 11) ? wave < nv : true;
    long long t0 = clock64();
    for (int it = 0; it < iters; ++it) {
        if constexpr (MODE == 0) { FMA8(a) FMA8(a) }
        if constexpr (MODE == 1) { EXP8(a) EXP8(a) }
        if constexpr (MODE == 2) { LOG8(a) LOG8(a) }
        if constexpr (MODE == 3)
            for (int k = 0; k < 4; ++k) acc[k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x, y, acc[k], 0, 0, 0);
        if constexpr (MODE == 4)
            for (int k = 0; k < 4; ++k) acc[k] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xh, yh, acc[k], 0, 0, 0);
        if constexpr (MODE == 5) {
            for (int k = 0; k < 4; ++k) {
                acc[k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x, y, acc[k], 0, 0, 0);
                FMA8(a)
            }
        }
        if constexpr (MODE == 6) {
            if (do_valu) { FMA8(a) FMA8(a) FMA8(a) FMA8(a) }
            else for (int k = 0; k < 4; ++k) acc[k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x, y, acc[k], 0, 0, 0);
        }
        if constexpr (MODE == 7) { PKF16_8(h) PKF16_8(h) }
        if constexpr (MODE == 8)
            for (int k = 0; k < 4; ++k) acc[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x, y, acc[0], 0, 0, 0);
        if constexpr (MODE == 9) { EXP8(a) FMA8(a) }
        if constexpr (MODE == 10)
            for (int k = 0; k < 4; ++k)
                asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc[k]) : "v"(x), "v"(y));
        if constexpr (MODE == 11) {
            if (do_valu) { FMA8(a) FMA8(a) FMA8(a) FMA8(a) }
            else
                for (int k = 0; k < 4; ++k)
                    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc[k]) : "v"(x), "v"(y));
        }
        if constexpr (MODE == 12) {
            for (int k = 0; k < 4; ++k) {
                asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc[k]) : "v"(x), "v"(y));
                FMA8(a)
            }
        }
    }
    long long t1 = clock64();
    float s = 0.0f;
    for (int i = 0; i < 8; ++i) s += a[i] + (float)(h[i] & 1);
    for (int k = 0; k < 4; ++k) s += acc[k][0] + acc[k][1] + acc[k][2] + acc[k][3];
    const long long g = (long long)blockIdx.x * blockDim.x + tid;
    out[g] = s;
    if ((tid & 63) == 0)
        cyc[g >> 6] = t1 - t0;
}

template <int MODE>
void run(const char* name, int threads, int blocks, int iters, int nv, double insts_per_iter,
         float* out, long long* cyc)
{
    hipLaunchKernelGGL(kern<MODE>, dim3(blocks), dim3(threads), 0, 0, out, cyc, iters / 10, nv);
    hipEvent_t e0, e1;
    hipEventCreate(&e0);
    hipEventCreate(&e1);
    hipEventRecord(e0);
    hipLaunchKernelGGL(kern<MODE>, dim3(blocks), dim3(threads), 0, 0, out, cyc, iters, nv);
    hipEventRecord(e1);
    hipEventSynchronize(e1);
    float ms;
    hipEventElapsedTime(&ms, e0, e1);
    const int nw = blocks * threads / 64;
    std::vector<long long> c(nw);
    hipMemcpy(c.data(), cyc, sizeof(long long) * nw, hipMemcpyDeviceToHost);
    if (MODE == 6 || MODE == 11) {
        // waves < nv of each workgroup ran 32 fma per iteration, the others 4 mfma
        const int wpg = threads / 64;
        std::vector<long long> cv, cm;
        for (int w = 0; w < nw; ++w) ((w % wpg) < nv ? cv : cm).push_back(c[w]);
        std::sort(cv.begin(), cv.end());
        std::sort(cm.begin(), cm.end());
        printf("%-44s waves/SIMD %d: fma waves %.2f cycles/fma, mfma waves %.2f cycles/mfma, kernel %.3f ms\n",
               name, nw / 1024, (double)cv[cv.size() / 2] / (iters * 32.0),
               (double)cm[cm.size() / 2] / (iters * 4.0), ms);
        return;
    }
    std::sort(c.begin(), c.end());
    const double med = (double)c[nw / 2];
    // per-wave cycles per instruction (shader clock), and SIMD-level time
    // SIMD-level rate from the kernel time at the clock the waves' own
    // counters show (median wave cycles / kernel time at 1 wave per SIMD)
    const double per_simd = (double)nw / 1024 * iters * insts_per_iter;
    printf("%-44s waves/SIMD %d: %7.2f ns/inst per SIMD (median wave %.0f cycles), kernel %.3f ms\n",
           name, nw / 1024, ms * 1e6 / per_simd, med, ms);
}

int main()
{
    const int maxw = 1024 * 8;   // up to 8 waves per SIMD
    float* out;
    long long* cyc;
    hipMalloc(&out, sizeof(float) * maxw * 64);
    hipMalloc(&cyc, sizeof(long long) * maxw);
    const int it = 20000;
    for (int wps : {1, 2, 4, 8}) {
        // wps waves per SIMD: workgroups of 4*wps waves (at most 16), 256 per
        // 4-wave share of the CUs
        const int th = 256 * (wps > 4 ? 4 : wps), bl = 256 * (wps > 4 ? wps / 4 : 1);
        printf("--- %d wave(s) per SIMD ---\n", wps);
        run<0>("v_fma_f32 (8 chains)", th, bl, it, 0, 16, out, cyc);
        run<1>("v_exp_f32 (8 chains)", th, bl, it, 0, 16, out, cyc);
        run<2>("v_log_f32 (8 chains)", th, bl, it, 0, 16, out, cyc);
        run<9>("v_exp_f32 + v_fma_f32 1:1 (per pair)", th, bl, it, 0, 8, out, cyc);
        run<7>("v_pk_mul_f16 (8 chains)", th, bl, it, 0, 16, out, cyc);
        run<3>("mfma_f32_16x16x32_bf16 (4 accumulators)", th, bl, it / 4, 0, 4, out, cyc);
        run<4>("mfma_f32_16x16x32_f16 (4 accumulators)", th, bl, it / 4, 0, 4, out, cyc);
        run<8>("mfma_f32_16x16x32_bf16 (1 chain)", th, bl, it / 4, 0, 4, out, cyc);
        run<5>("1 mfma + 8 fma per group (per group)", th, bl, it / 4, 0, 4, out, cyc);
        run<10>("mfma bf16, AGPR accumulators", th, bl, it / 4, 0, 4, out, cyc);
        run<12>("1 mfma (AGPR acc) + 8 fma per group", th, bl, it / 4, 0, 4, out, cyc);
        if (wps >= 2) {
            run<6>("split: half waves 32 fma, half 4 mfma (per it)", th, bl, it / 4, th / 128, 1, out, cyc);
            run<11>("split, mfma with AGPR accumulators", th, bl, it / 4, th / 128, 1, out, cyc);
        }
    }
    hipFree(out);
    hipFree(cyc);
    return 0;
}
