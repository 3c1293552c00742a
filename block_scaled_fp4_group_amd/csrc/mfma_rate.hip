// mfma_rate.hip -- sustained matrix-core throughput and shader clock of the
// device, for the roofline peaks the benchmark reports against.  Not part of
// the GEMM: bench.py --mfma-rates loads it (libnvfp4gg_probe.so) and prints
// what it measures.
//
// Every probe keeps its operands in registers and runs one workgroup per
// compute unit for a few milliseconds per launch, 40 launches back to back;
// throughput is the launches' flops over their wall time (HIP events), and
// the clock is the shader-clock counter (s_memtime) over the 100 MHz
// constant counter (s_memrealtime) of the same waves.  All stores are in
// bounds: out[] has one float per thread, times[] two words per wave.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>

namespace {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

// Probe kinds: per iteration and wave,
//  0: 8 x v_mfma_f32_32x32x16_f16
//  1: 16 x v_mfma_f32_16x16x32_f16
//  2: 8 x v_mfma_scale_f32_32x32x64_f8f6f4 on FP8 (E4M3) operands
//  3: 8 x v_mfma_scale_f32_32x32x64_f8f6f4 on FP4 (E2M1) operands
//  4: kind 0 plus the exact FP4 -> fp16 decode of 24 code dwords' worth of
//     pairs (one convert and one packed multiply per pair), the VALU work a
//     decode-to-fp16 path issues beside those MFMAs
//  5: the FP4-MFMA alternative with a register rescale: 8 x
//     v_mfma_scale_f32_32x32x64_f8f6f4 on FP4 operands, each covering one
//     16-element NVFP4 scale block (the other 48 k zero, since the
//     instruction's own scales are powers of two per 32 k), its 32 x 32
//     partial started from zero and added into the accumulator times the
//     per-output scale product: 16 multiplies (row scale x column scale) and
//     16 fused multiply-adds per lane.  Counted flops are the useful ones
//     (16 k per instruction).
template <int KIND>
__global__ __launch_bounds__(512, 1) void probe(float *out, unsigned long long *times, int iters, uint32_t seed)
{
    const int lane = threadIdx.x & 63;
    f16x8 a[2], b[2];
    for (int i = 0; i < 2; ++i)
        for (int j = 0; j < 8; ++j) {
            a[i][j] = (_Float16)(0.01f * (float)((lane + i + j + seed) & 7));
            b[i][j] = (_Float16)(0.02f * (float)((lane * 3 + i + j + seed) & 7));
        }
    i32x8 xa, xb;
    for (int j = 0; j < 8; ++j) {
        xa[j] = (int)((seed + lane + j) * 0x01010101u);
        xb[j] = (int)((seed * 3 + lane + j) * 0x01010101u);
    }
    uint32_t codes[6];
    for (int i = 0; i < 6; ++i)
        codes[i] = seed * 2654435761u + lane * 97u + i;
    const f16x2 sc = {(_Float16)1.125f, (_Float16)1.125f};
    float sa16[16];                // row scales of the lane's 16 outputs (kind 5)
    for (int j = 0; j < 16; ++j)
        sa16[j] = 0.5f + 0.0625f * (float)((lane + j + seed) & 15);
    float sbv = 1.125f;            // the lane's column scale (kind 5)
    f32x16 acc32[8];
    f32x4 acc16[16];
    for (int i = 0; i < 8; ++i)
        acc32[i] = f32x16{};
    for (int i = 0; i < 16; ++i)
        acc16[i] = f32x4{};
    const unsigned long long t0 = __builtin_amdgcn_s_memtime();
    const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; ++it) {
        if constexpr (KIND == 0 || KIND == 4) {
#pragma unroll
            for (int i = 0; i < 8; ++i)
                acc32[i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i & 1], b[(i >> 1) & 1], acc32[i], 0, 0, 0);
        } else if constexpr (KIND == 1) {
#pragma unroll
            for (int i = 0; i < 16; ++i)
                acc16[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[i & 1], b[(i >> 1) & 1], acc16[i], 0, 0, 0);
        } else if constexpr (KIND == 5) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                asm volatile("" : "+v"(xa));       // a new block of codes every MFMA
                const f32x16 part = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(xa, xb, f32x16{}, 4, 4, 0, 0x7f,
                                                                                    0, 0x7f);
                asm volatile("" : "+v"(sbv));     // a new column scale every block
#pragma unroll
                for (int j = 0; j < 16; ++j)
                    acc32[i & 3][j] = __builtin_fmaf(part[j], sa16[j] * sbv, acc32[i & 3][j]);
            }
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i)
                acc32[i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(xa, xb, acc32[i], KIND == 2 ? 0 : 4,
                                                                           KIND == 2 ? 0 : 4, 0, 0x7f, 0, 0x7f);
        }
        if constexpr (KIND == 4) {
            // 24 pairs: six code dwords, four pairs each, decoded and kept live
#pragma unroll
            for (int i = 0; i < 6; ++i) {
                uint32_t c = codes[i];
                asm volatile("" : "+v"(c));
                const f16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c, 1.0f, 0) * sc;
                const f16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c, 1.0f, 1) * sc;
                const f16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c, 1.0f, 2) * sc;
                const f16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c, 1.0f, 3) * sc;
                const f16x8 d = {p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
                if (i < 2)
                    b[i] = d;
                else
                    asm volatile("" :: "v"(d));
            }
        }
    }
    const unsigned long long t1 = __builtin_amdgcn_s_memtime();
    const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
    float s = 0.0f;
    for (int i = 0; i < 8; ++i)
        for (int j = 0; j < 16; ++j)
            s += acc32[i][j];
    for (int i = 0; i < 16; ++i)
        for (int j = 0; j < 4; ++j)
            s += acc16[i][j];
    out[blockIdx.x * blockDim.x + threadIdx.x] = s;
    if (lane == 0) {
        const int gw = (int)(blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6));
        times[2 * gw] = t1 - t0;
        times[2 * gw + 1] = r1 - r0;
    }
}

constexpr double kFlopsPerIter[6] = {8.0 * 32 * 32 * 16 * 2, 16.0 * 16 * 16 * 32 * 2, 8.0 * 32 * 32 * 64 * 2,
                                     8.0 * 32 * 32 * 64 * 2, 8.0 * 32 * 32 * 16 * 2, 8.0 * 32 * 32 * 16 * 2};
constexpr const char *kNames[6] = {"f16 32x32x16", "f16 16x16x32", "fp8 32x32x64 (scaled)", "fp4 32x32x64 (scaled)",
                                   "f16 32x32x16 + fp4->f16 decode of 48 values per 8 MFMA",
                                   "fp4 32x32x64, one 16-k scale block per MFMA + register rescale (useful flops)"};

template <int KIND>
int run(int waves, int iters, int launches, double &tflops, double &ghz)
{
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, 0) != hipSuccess || cus <= 0)
        return 1;
    const int threads = 64 * waves;
    float *out = nullptr;
    unsigned long long *times = nullptr;
    if (hipMalloc(&out, sizeof(float) * cus * threads) != hipSuccess)
        return 1;
    if (hipMalloc(&times, sizeof(unsigned long long) * cus * waves * 2) != hipSuccess) {
        (void)hipFree(out);
        return 1;
    }
    hipEvent_t e0, e1;
    (void)hipEventCreate(&e0);
    (void)hipEventCreate(&e1);
    for (int i = 0; i < 3; ++i)
        hipLaunchKernelGGL(probe<KIND>, dim3(cus), dim3(threads), 0, 0, out, times, iters, 1u + i);
    (void)hipDeviceSynchronize();
    (void)hipEventRecord(e0, 0);
    for (int i = 0; i < launches; ++i)
        hipLaunchKernelGGL(probe<KIND>, dim3(cus), dim3(threads), 0, 0, out, times, iters, 7u + i);
    (void)hipEventRecord(e1, 0);
    (void)hipEventSynchronize(e1);
    int rc = hipGetLastError() == hipSuccess ? 0 : 1;
    float ms = 0.0f;
    (void)hipEventElapsedTime(&ms, e0, e1);
    unsigned long long *h = new unsigned long long[(size_t)cus * waves * 2];
    if (hipMemcpy(h, times, sizeof(unsigned long long) * cus * waves * 2, hipMemcpyDeviceToHost) != hipSuccess)
        rc = 1;
    double clk = 0, rt = 0;
    for (int w = 0; w < cus * waves; ++w) {
        clk += (double)h[2 * w];
        rt += (double)h[2 * w + 1];
    }
    delete[] h;
    const double fl = kFlopsPerIter[KIND] * iters * (double)cus * waves * launches;
    tflops = fl / (ms * 1e-3) / 1e12;
    ghz = rt > 0 ? clk / (rt / 100e6) / 1e9 : 0.0;
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    (void)hipFree(out);
    (void)hipFree(times);
    return rc;
}

}  // namespace

// Runs every probe on device 0 (the current device) and writes one JSON
// object per line into `buf` (at most `cap` bytes, NUL-terminated).  Returns 0,
// or 1 if a HIP call failed.
extern "C" int nvfp4_probe_mfma_rates(char *buf, int cap)
{
    int len = 0, rc = 0;
    auto emit = [&](int kind, int waves, double tf, double ghz) {
        if (len < cap)
            len += snprintf(buf + len, (size_t)(cap - len),
                            "{\"probe\": \"%s\", \"waves_per_cu\": %d, \"tflops\": %.1f, \"clock_ghz\": %.3f}\n",
                            kNames[kind], waves, tf, ghz);
    };
    double tf = 0, ghz = 0;
    const int it = 20000, launches = 40;
    rc |= run<0>(4, it, launches, tf, ghz);
    emit(0, 4, tf, ghz);
    rc |= run<0>(8, it / 2, launches, tf, ghz);
    emit(0, 8, tf, ghz);
    rc |= run<1>(8, it / 2, launches, tf, ghz);
    emit(1, 8, tf, ghz);
    rc |= run<2>(4, it / 2, launches, tf, ghz);
    emit(2, 4, tf, ghz);
    rc |= run<3>(4, it / 2, launches, tf, ghz);
    emit(3, 4, tf, ghz);
    rc |= run<4>(4, it, launches, tf, ghz);
    emit(4, 4, tf, ghz);
    rc |= run<5>(4, it / 2, launches, tf, ghz);
    emit(5, 4, tf, ghz);
    rc |= run<5>(8, it / 4, launches, tf, ghz);
    emit(5, 8, tf, ghz);
    return rc;
}
