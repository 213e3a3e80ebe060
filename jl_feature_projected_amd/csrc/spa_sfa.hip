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
// A workgroup of 16 waves per (head, 256 tokens), each wave 16 rows, loaded eight at a
// time. Per row the lanes hold d/64 consecutive features each; the k-th largest magnitude T
// is found by a bitwise search over the 15 magnitude bits of bf16 with wave ballots
// counting the features at or above a candidate (wave-uniform, scalar counts), eight rows'
// searches interleaved; features above T are kept, and of those equal to T the
// (k - #above) of lowest index.
#include "spa_device.h"
#include "spa_internal.h"

namespace spa {
namespace {

constexpr int kTopkThreads = 1024;
constexpr int kTopkRows = kProjBlockTokens / (kTopkThreads / 64);  // rows per wave

__device__ __forceinline__ int popc64(uint64_t x) { return __builtin_popcountll(x); }

template <int D>
__global__ __launch_bounds__(kTopkThreads) void sfa_topk_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, uint16_t* __restrict__ Qt,
    uint16_t* __restrict__ Kt, float* __restrict__ kmax, int N, int k, float qscale, int nblk) {
    constexpr int E = D / 64;  // features per lane
    __shared__ float wave_max[kTopkThreads / 64];
    const int z = blockIdx.x & 1;  // 0: queries, 1: keys
    const int rest = blockIdx.x >> 1;
    const int blk = rest % nblk;
    const int bh = rest / nblk;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const uint16_t* X = (z ? K : Q) + (size_t)bh * N * D;
    uint16_t* Y = (z ? Kt : Qt) + (size_t)bh * N * D;
    const float sc = z ? 1.0f : qscale;
    const uint64_t below = (1ull << lane) - 1ull;
    float nmax = 0.0f;  // largest squared norm of a selected key row in this wave

    const int tok0 = blk * kProjBlockTokens + wave * kTopkRows;
    // Rows in groups of RG: the groups' bitwise searches run side by side, so their chains
    // of wave-uniform counts and selects overlap instead of waiting on each other.
    constexpr int RG = 8;
    static_assert(kTopkRows % RG == 0, "row groups");
#pragma unroll 1
    for (int r0 = 0; r0 < kTopkRows; r0 += RG) {
        if (tok0 + r0 >= N) break;  // wave-uniform
        uint32_t raw[RG];           // this lane's d/64 features of each row of the group
#pragma unroll
        for (int g = 0; g < RG; ++g) {
            const int tok = tok0 + r0 + g;
            raw[g] = 0u;
            if (tok < N)
                raw[g] = E == 2 ? *reinterpret_cast<const uint32_t*>(X + (size_t)tok * D + 2 * lane)
                                : (uint32_t)X[(size_t)tok * D + lane];
        }
        uint16_t x[RG][E];
        uint32_t mag[RG][E], t[RG];
#pragma unroll
        for (int g = 0; g < RG; ++g) {
            x[g][0] = (uint16_t)(raw[g] & 0xffffu);
            if (E == 2) x[g][E - 1] = (uint16_t)(raw[g] >> 16);
#pragma unroll
            for (int e = 0; e < E; ++e) mag[g][e] = x[g][e] & 0x7fffu;
            t[g] = 0;
        }
        // T = the largest t with #{mag >= t} >= k, per row
#pragma unroll 1
        for (int bit = 14; bit >= 0; --bit) {
#pragma unroll
            for (int g = 0; g < RG; ++g) {
                const uint32_t cand = t[g] | (1u << bit);
                int cnt = 0;
#pragma unroll
                for (int e = 0; e < E; ++e) cnt += popc64(__ballot(mag[g][e] >= cand));
                t[g] = __builtin_amdgcn_readfirstlane(cnt >= k ? cand : t[g]);
            }
        }
#pragma unroll
        for (int g = 0; g < RG; ++g) {
            const int tok = tok0 + r0 + g;
            if (tok >= N) break;  // wave-uniform
            int above = 0;
            uint64_t tie[E];
#pragma unroll
            for (int e = 0; e < E; ++e) {
                above += popc64(__ballot(mag[g][e] > t[g]));
                tie[e] = __ballot(mag[g][e] == t[g]);
            }
            const int need = k - above;  // ties to keep, lowest feature index first
            int rank = 0;                // ties at lower feature indices than this lane's first
#pragma unroll
            for (int e = 0; e < E; ++e) rank += popc64(tie[e] & below);
            float n2 = 0.0f;
            uint16_t out[E];
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const bool is_tie = mag[g][e] == t[g];
                const bool keep = mag[g][e] > t[g] || (is_tie && rank < need);
                rank += is_tie ? 1 : 0;
                const float v = keep ? __uint_as_float((uint32_t)x[g][e] << 16) * sc : 0.0f;
                const uint32_t h = pack_f16x2(v, 0.0f) & 0xffffu;
                out[e] = (uint16_t)h;
                const float hv = (float)__builtin_bit_cast(_Float16, (uint16_t)h);
                n2 += hv * hv;
            }
            if (E == 2)
                *reinterpret_cast<uint32_t*>(Y + (size_t)tok * D + 2 * lane) =
                    (uint32_t)out[0] | ((uint32_t)out[E - 1] << 16);
            else
                Y[(size_t)tok * D + lane] = out[0];
            if (z) {
#pragma unroll
                for (int o = 32; o > 0; o >>= 1) n2 += __shfl_xor(n2, o, 64);
                nmax = fmaxf(nmax, n2);
            }
        }
    }
    if (z) {
        if (lane == 0) wave_max[wave] = nmax;
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
