// spa_probe.hip -- rate probes for the benchmark's roofline context: the sustained rate of
// the bf16 matrix core (32x32x16 MFMA), of fp32 VALU FMAs, and the engine clock while each
// runs. Not part of the attention path.
//
// The MFMA probe launches one workgroup of 256 threads per CU (one wave per SIMD: a single
// wave keeps the matrix core busy), the FMA probe four (four waves per SIMD: one wave alone
// cannot issue VALU work back to back); every wave runs a fixed number of independent
// operations. The elapsed time comes from HIP events around the launch, the engine clock
// from the shader-clock counter (s_memtime) against the constant 100 MHz counter
// (s_memrealtime), read by wave 0 of each workgroup at its start and end.
#include <hip/hip_runtime.h>

#include <vector>

#include "spa_device.h"

namespace spa {
namespace {

constexpr int kProbeThreads = 256;
constexpr int kMfmaIters = 4096;  // x 8 MFMAs per wave
constexpr int kFmaIters = 4096;   // x 16 FMAs per lane

// out[2 * block] = shader clocks, out[2 * block + 1] = 100 MHz ticks (wave 0 of the block).
__global__ __launch_bounds__(kProbeThreads, 1) void probe_mfma_kernel(float* sink,
                                                                      long long* ticks,
                                                                      float seed) {
    bf16x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = (__bf16)(seed * (float)(i + 1));
        b[i] = (__bf16)(seed * (float)(8 - i));
    }
    f32x16 c[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) c[j] = f32x16_fill(0.0f);
    const long long t0 = __builtin_amdgcn_s_memtime();
    const long long r0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < kMfmaIters; ++it) {
#pragma unroll
        for (int j = 0; j < 8; ++j) c[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[j], 0, 0, 0);
    }
    const long long t1 = __builtin_amdgcn_s_memtime();
    const long long r1 = __builtin_amdgcn_s_memrealtime();
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int i = 0; i < 16; ++i) s += c[j][i];
    sink[blockIdx.x * kProbeThreads + threadIdx.x] = s;
    if (threadIdx.x == 0) {
        ticks[2 * blockIdx.x] = t1 - t0;
        ticks[2 * blockIdx.x + 1] = r1 - r0;
    }
}

__global__ __launch_bounds__(kProbeThreads) void probe_fma_kernel(float* sink,
                                                                     long long* ticks,
                                                                     float seed) {
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = seed * (float)(threadIdx.x + i);
    const long long t0 = __builtin_amdgcn_s_memtime();
    const long long r0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < kFmaIters; ++it) {
#pragma unroll
        for (int i = 0; i < 16; ++i) x[i] = __builtin_fmaf(x[i], 0.9999f, 1e-7f);
    }
    const long long t1 = __builtin_amdgcn_s_memtime();
    const long long r1 = __builtin_amdgcn_s_memrealtime();
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) s += x[i];
    sink[blockIdx.x * kProbeThreads + threadIdx.x] = s;
    if (threadIdx.x == 0) {
        ticks[2 * blockIdx.x] = t1 - t0;
        ticks[2 * blockIdx.x + 1] = r1 - r0;
    }
}

}  // namespace

// Runs one probe (kind 0: MFMA, 1: fp32 FMA) `reps` times after a warm-up; returns the best
// rate in TFLOP/s and the mean engine clock in GHz over the waves of that launch.
hipError_t run_probe(int kind, int reps, hipStream_t stream, double* tflops, double* ghz) {
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    const int blocks = kind == 0 ? cus : 4 * cus;
    float* sink = nullptr;
    long long* ticks = nullptr;
    e = hipMalloc(&sink, sizeof(float) * kProbeThreads * blocks);
    if (e == hipSuccess) e = hipMalloc(&ticks, sizeof(long long) * 2 * blocks);
    hipEvent_t e0 = nullptr, e1 = nullptr;
    if (e == hipSuccess) e = hipEventCreate(&e0);
    if (e == hipSuccess) e = hipEventCreate(&e1);
    std::vector<long long> h(2 * (size_t)blocks);
    double best_ms = 1e30, clk = 0.0;
    for (int r = -1; e == hipSuccess && r < reps; ++r) {
        e = hipEventRecord(e0, stream);
        if (e != hipSuccess) break;
        if (kind == 0)
            probe_mfma_kernel<<<blocks, kProbeThreads, 0, stream>>>(sink, ticks, 1e-3f);
        else
            probe_fma_kernel<<<blocks, kProbeThreads, 0, stream>>>(sink, ticks, 1e-3f);
        e = hipGetLastError();
        if (e == hipSuccess) e = hipEventRecord(e1, stream);
        if (e == hipSuccess) e = hipEventSynchronize(e1);
        float ms = 0.0f;
        if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
        if (e == hipSuccess) e = hipMemcpy(h.data(), ticks, sizeof(long long) * 2 * blocks, hipMemcpyDeviceToHost);
        if (e != hipSuccess || r < 0) continue;  // r = -1: warm-up
        if (ms < best_ms) {
            best_ms = ms;
            double sum = 0.0;
            for (int i = 0; i < blocks; ++i) sum += (double)h[2 * i] / ((double)h[2 * i + 1] * 10.0);
            clk = sum / blocks;  // shader clocks per ns
        }
    }
    if (e == hipSuccess) {
        const double flops = kind == 0
                                 ? (double)cus * 4 * kMfmaIters * 8 * 32.0 * 32.0 * 16.0 * 2.0
                                 : (double)blocks * kProbeThreads * kFmaIters * 16 * 2.0;
        *tflops = flops / (best_ms * 1e-3) / 1e12;
        *ghz = clk;
    }
    if (e0) (void)hipEventDestroy(e0);
    if (e1) (void)hipEventDestroy(e1);
    if (sink) (void)hipFree(sink);
    if (ticks) (void)hipFree(ticks);
    return e;
}

}  // namespace spa
