// spa_probe.hip -- rate probes for the benchmark's roofline context: the sustained rate of
// the bf16 matrix core (32x32x16 MFMA), of fp32 VALU FMAs, and the engine clock while each
// runs. Not part of the attention path.
//
// The MFMA probe launches one workgroup of 256 threads per CU (one wave per SIMD: a single
// wave keeps the matrix core busy), the FMA probe four (four waves per SIMD: one wave alone
// cannot issue VALU work back to back); every wave runs a fixed number of independent
// operations. The MFMA operands are random bf16 values in [-1, 1) (a per-lane linear
// congruential sequence), four operand sets cycled so that consecutive MFMAs see different
// inputs: the matrix core's power, and with it the clock the chip holds, depends on the data
// (tiny constant operands run it some 25 % faster than random ones). Each probe is launched
// back to back for about 50 ms, long enough for the clock to settle at its sustained value;
// the rate is the work of the second half of the launches over their time (HIP events), the
// engine clock the shader-clock counter (s_memtime) against the constant 100 MHz counter
// (s_memrealtime), read by wave 0 of each workgroup of the last launch at its start and end.
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
                                                                      unsigned seed) {
    bf16x8 a[4], b[4];
    uint32_t x = seed ^ (threadIdx.x * 2654435761u) ^ (blockIdx.x * 40503u);
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            x = x * 1664525u + 1013904223u;
            a[q][i] = (__bf16)((float)(x >> 16) * 0x1p-15f - 1.0f);
            x = x * 1664525u + 1013904223u;
            b[q][i] = (__bf16)((float)(x >> 16) * 0x1p-15f - 1.0f);
        }
    f32x16 c[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) c[j] = f32x16_fill(0.0f);
    const long long t0 = __builtin_amdgcn_s_memtime();
    const long long r0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < kMfmaIters; it += 2) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int j = 0; j < 8; ++j)
                c[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[(j + h) & 3], b[(j + 2 * h + 1) & 3],
                                                               c[j], 0, 0, 0);
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
                                                                     unsigned seed) {
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = 1e-3f * (float)((seed + threadIdx.x + i) & 1023);
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

// Runs one probe (kind 0: MFMA, 1: fp32 FMA) `launches` times back to back (at least 2);
// returns the rate of the second half of the launches in TFLOP/s and the mean engine clock in
// GHz over the waves of the last launch.
hipError_t run_probe(int kind, int launches, hipStream_t stream, double* tflops, double* ghz) {
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    if (launches < 2) launches = 2;
    const int blocks = kind == 0 ? cus : 4 * cus;
    float* sink = nullptr;
    long long* ticks = nullptr;
    e = hipMalloc(&sink, sizeof(float) * kProbeThreads * blocks);
    if (e == hipSuccess) e = hipMalloc(&ticks, sizeof(long long) * 2 * blocks);
    hipEvent_t e0 = nullptr, e1 = nullptr;
    if (e == hipSuccess) e = hipEventCreate(&e0);
    if (e == hipSuccess) e = hipEventCreate(&e1);
    const int timed_from = launches / 2;
    for (int l = 0; e == hipSuccess && l < launches; ++l) {
        if (l == timed_from) e = hipEventRecord(e0, stream);
        if (e != hipSuccess) break;
        if (kind == 0)
            probe_mfma_kernel<<<blocks, kProbeThreads, 0, stream>>>(sink, ticks, 12345u + l);
        else
            probe_fma_kernel<<<blocks, kProbeThreads, 0, stream>>>(sink, ticks, 12345u + l);
        e = hipGetLastError();
    }
    if (e == hipSuccess) e = hipEventRecord(e1, stream);
    if (e == hipSuccess) e = hipEventSynchronize(e1);
    float ms = 0.0f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
    std::vector<long long> h(2 * (size_t)blocks);
    if (e == hipSuccess) e = hipMemcpy(h.data(), ticks, sizeof(long long) * 2 * blocks, hipMemcpyDeviceToHost);
    if (e == hipSuccess) {
        double sum = 0.0;
        for (int i = 0; i < blocks; ++i) sum += (double)h[2 * i] / ((double)h[2 * i + 1] * 10.0);
        const double per_launch = kind == 0
                                      ? (double)cus * 4 * kMfmaIters * 8 * 32.0 * 32.0 * 16.0 * 2.0
                                      : (double)blocks * kProbeThreads * kFmaIters * 16 * 2.0;
        *tflops = per_launch * (launches - timed_from) / (ms * 1e-3) / 1e12;
        *ghz = sum / blocks;  // shader clocks per ns
    }
    if (e0) (void)hipEventDestroy(e0);
    if (e1) (void)hipEventDestroy(e1);
    if (sink) (void)hipFree(sink);
    if (ticks) (void)hipFree(ticks);
    return e;
}

}  // namespace spa
