// spa_sfa.hip -- Top-k feature selection for sparse feature attention.
//
// What it computes ("Scaling Attention via Feature Sparsity", key design 1): for every row x
// of Q and of K, Topk_k(x)_u = x_u when u is among the k coordinates of largest |x|, else 0
// (ties in |x|: the lower coordinate index first). The selected rows are written in the
// streamed attention kernel's operand layout -- fp16 [BH, N, d], queries times
// scale*log2(e) -- with the largest selected key norm per 256-key block, so the attention
// kernel runs unchanged with m = d: its score MFMA over d features is exactly the sum over
// the shared support (every other product has a zero factor; key design 3 asks for exact
// results). Dense 32x32x16 MFMAs over d <= 128 features cost d/16 instructions per 32x32
// score tile, far less than scattering the support intersections.
//
// A workgroup of 256 threads per (head, 256 tokens), one thread per row: the row's d
// features sit in the thread's registers as packed bf16 pairs, so every count below is plain
// vector arithmetic (the earlier layout, a row spread over a wave with ballot counts, was
// bound by the one scalar unit per CU that summed the ballots). The k-th largest magnitude T
// is found by a bitwise search over the 15 magnitude bits of bf16; features above T are
// kept, and of those equal to T the (k - #above) of lowest index.
#include "spa_device.h"
#include "spa_internal.h"

namespace spa {
namespace {

constexpr int kTopkThreads = kProjBlockTokens;  // one thread per row of a 256-row block

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// Number of features among the packed pairs mag[0 .. W) whose magnitude is >= cand, times 8.
// Per 16-bit half, mag + (0x8000 - cand) has bit 15 set exactly when mag >= cand (both terms
// are below 0x8000, so nothing carries out of the half); the permute's sign-replicating
// selectors turn the four indicator bits of two pairs into four 0x00 / 0xff bytes, and one
// bit count with accumulate adds them.
template <int W>
__device__ __forceinline__ uint32_t count_ge8(const uint32_t (&mag)[W], uint32_t cand) {
    const uint32_t c = (0x8000u - cand) * 0x10001u;
    const u16x2 cv = __builtin_bit_cast(u16x2, c);
    uint32_t n = 0;
#pragma unroll
    for (int j = 0; j < W; j += 2) {
        const uint32_t a = __builtin_bit_cast(uint32_t, __builtin_bit_cast(u16x2, mag[j]) + cv);
        const uint32_t b = __builtin_bit_cast(uint32_t, __builtin_bit_cast(u16x2, mag[j + 1]) + cv);
        n += __builtin_popcount(__builtin_amdgcn_perm(b, a, 0x0b0a0908u));
    }
    return n;
}

template <int D>
__global__ __launch_bounds__(kTopkThreads) void sfa_topk_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, uint16_t* __restrict__ Qt,
    uint16_t* __restrict__ Kt, float* __restrict__ kmax, int N, int k, float qscale, int nblk) {
    constexpr int W = D / 2;   // packed bf16 pairs per row
    constexpr int L = D / 8;   // 16-byte pieces per row
    static_assert(W % 4 == 0, "rows move in 16-byte pieces");
    __shared__ float wave_max[kTopkThreads / 64];
    const int z = blockIdx.x & 1;  // 0: queries, 1: keys
    const int rest = blockIdx.x >> 1;
    const int blk = rest % nblk;
    const int bh = rest / nblk;
    const int tok = blk * kProjBlockTokens + (int)threadIdx.x;
    const bool live = tok < N;
    const size_t row = ((size_t)bh * N + (live ? tok : 0)) * D;
    const float sc = z ? 1.0f : qscale;

    uint32_t raw[W], mag[W];
    if (live) {
        const uint4* src = reinterpret_cast<const uint4*>((z ? K : Q) + row);
#pragma unroll
        for (int i = 0; i < L; ++i) {
            const uint4 v = src[i];
            raw[4 * i] = v.x;
            raw[4 * i + 1] = v.y;
            raw[4 * i + 2] = v.z;
            raw[4 * i + 3] = v.w;
        }
    } else {
#pragma unroll
        for (int j = 0; j < W; ++j) raw[j] = 0u;
    }
#pragma unroll
    for (int j = 0; j < W; ++j) mag[j] = raw[j] & 0x7fff7fffu;

    // T = the largest t with #{features with magnitude >= t} >= k; n8 = 8 * that count.
    const uint32_t k8 = 8u * (uint32_t)k;
    uint32_t t = 0, n8 = 8u * D;
#pragma unroll 1
    for (int bit = 14; bit >= 0; --bit) {
        const uint32_t cand = t | (1u << bit);
        const uint32_t n = count_ge8(mag, cand);
        const bool take = n >= k8;
        t = take ? cand : t;
        n8 = take ? n : n8;
    }

    // Keep every feature of magnitude >= T except the last (#{>= T} - k) of those equal to T,
    // i.e. the ties of highest index: walk the features from the end with that many drops.
    int drop = (int)((n8 - k8) >> 3);
    const int ti = (int)t;
    uint32_t outw[W];
    float n2 = 0.0f;
#pragma unroll
    for (int j = W - 1; j >= 0; --j) {
        const int shi = (int)(mag[j] >> 16) - ti;
        const int keep_hi = shi - min(max(drop, 0), 1);  // >= 0: kept
        drop -= shi == 0 ? 1 : 0;
        const int slo = (int)(mag[j] & 0xffffu) - ti;
        const int keep_lo = slo - min(max(drop, 0), 1);
        drop -= slo == 0 ? 1 : 0;
        const float vlo = keep_lo >= 0 ? __uint_as_float(raw[j] << 16) * sc : 0.0f;
        const float vhi = keep_hi >= 0 ? __uint_as_float(raw[j] & 0xffff0000u) * sc : 0.0f;
        outw[j] = pack_f16x2(vlo, vhi);
        if (z) {
            const float hlo = (float)__builtin_bit_cast(_Float16, (uint16_t)(outw[j] & 0xffffu));
            const float hhi = (float)__builtin_bit_cast(_Float16, (uint16_t)(outw[j] >> 16));
            n2 += hlo * hlo + hhi * hhi;
        }
    }
    if (live) {
        uint4* dst = reinterpret_cast<uint4*>((z ? Kt : Qt) + row);
#pragma unroll
        for (int i = 0; i < L; ++i)
            dst[i] = make_uint4(outw[4 * i], outw[4 * i + 1], outw[4 * i + 2], outw[4 * i + 3]);
    }
    if (z) {
        const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
        if (!live) n2 = 0.0f;
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) n2 = fmaxf(n2, __shfl_xor(n2, o, 64));
        if (lane == 0) wave_max[wave] = n2;
        __syncthreads();
        if (threadIdx.x == 0) {
            float b = wave_max[0];
#pragma unroll
            for (int w = 1; w < kTopkThreads / 64; ++w) b = fmaxf(b, wave_max[w]);
            kmax[(size_t)bh * nblk + blk] = sqrtf(b);
        }
    }
}

}  // namespace

hipError_t launch_sfa_topk(const void* Q, const void* K, void* Qt, void* Kt, float* kmax,
                           int BH, int N, int d, int k, float qscale, hipStream_t stream) {
    const int nblk = proj_blocks(N);
    const long long grid = 2LL * BH * nblk;
    if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    const auto* q = static_cast<const uint16_t*>(Q);
    const auto* kk = static_cast<const uint16_t*>(K);
    auto* qt = static_cast<uint16_t*>(Qt);
    auto* kt = static_cast<uint16_t*>(Kt);
    switch (d) {
        case 64:
            sfa_topk_kernel<64><<<dim3((unsigned)grid), kTopkThreads, 0, stream>>>(q, kk, qt, kt, kmax, N, k, qscale, nblk);
            break;
        case 128:
            sfa_topk_kernel<128><<<dim3((unsigned)grid), kTopkThreads, 0, stream>>>(q, kk, qt, kt, kmax, N, k, qscale, nblk);
            break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace spa
