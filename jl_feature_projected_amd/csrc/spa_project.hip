// spa_project.hip -- the projection step X~ = X P on bf16 MFMA (gfx950).
//
// "Sparse Projection Attention" page, Sec. 3.1.2 and Algorithm 1 steps 2-3: queries and keys
// are mapped from d to m features by one shared matrix. "Projection-Decomposition Attention
// (PDA)", Algorithm 2.1 step 1, and Sec. 4.1 (cost O(L d m), small next to the O(L^2 m)
// scores): the launch is bound by reading X from HBM.
//
// Each wave computes X~^T for 32 tokens: D[c][t] = sum_k P^T[c][k] X^T[k][t], with P^T
// staged once per workgroup in LDS as the A operand and 16-byte loads of X rows as the B
// operand. In the D layout a lane owns one token and 4 consecutive output columns per
// group, so every store is one 8-byte write of 4 values. The result is rounded once, to
// bf16 for the exported projection or to fp16 for the attention path's score operands.
// When asked (kmax != null), the launch also records, per (head, 256-token block) of the
// second tensor (the keys), the largest row norm of the projected values: the attention
// launch bounds every score of a row by the query norm times that maximum.
#include "spa_device.h"
#include "spa_internal.h"

namespace spa {
namespace {

constexpr int kProjThreads = 256;
constexpr int kProjTokensPerWave = 32;
constexpr int kProjIters = 2;  // token blocks per wave: amortises the P^T staging
constexpr int kProjTokensPerBlock = kProjThreads / 64 * kProjTokensPerWave * kProjIters;
static_assert(kProjTokensPerBlock == kProjBlockTokens, "projection block size");

// Round-to-nearest-even of two floats to the output type, packed into one dword.
template <bool F16>
__device__ __forceinline__ uint32_t pack_out(float lo, float hi) {
    return F16 ? pack_f16x2(lo, hi) : pack_bf16x2(lo, hi);
}

template <int D, int MB, bool F16>
__global__ __launch_bounds__(kProjThreads) void project_bf16_kernel(
    const bf16_t* __restrict__ X0, const bf16_t* __restrict__ X1, const bf16_t* __restrict__ P,
    uint16_t* __restrict__ Y0, uint16_t* __restrict__ Y1, int N, int BH, int H, int m,
    int out_stride, int out_cols, float out_scale0, float out_scale1, float* __restrict__ kmax) {
    constexpr int PROW = D + 8;  // LDS row pitch in bf16: 16 bytes of padding per row
    constexpr int KS = D / 16;   // MFMA k-steps over the input features
    __shared__ __attribute__((aligned(16))) bf16_t Pt[MB * 32 * PROW];
    __shared__ float wave_max[kProjThreads / 64];

    // blockIdx.x = (z * BH + bh) * nblk + token block; z picks the tensor (queries/keys).
    const int nblk = (N + kProjTokensPerBlock - 1) / kProjTokensPerBlock;
    const int blk = blockIdx.x % nblk;
    const int zbh = blockIdx.x / nblk;
    const int z = zbh / BH;
    const int bh = zbh - z * BH;
    const bf16_t* X = z ? X1 : X0;
    uint16_t* Y = z ? Y1 : Y0;
    const float out_scale = z ? out_scale1 : out_scale0;
    const int h = bh % H;
    const int tid = threadIdx.x;

    // P^T[c][k] = P[h][k][c] for c < m; rows m .. 32*MB-1 are zero.
    const bf16_t* Ph = P + (size_t)h * D * m;
    for (int idx = tid; idx < MB * 32 * D; idx += kProjThreads) {
        const int c = idx / D, k = idx % D;
        Pt[c * PROW + k] = c < m ? Ph[k * m + c] : (bf16_t)0.0f;
    }
    __syncthreads();

    const int wave = tid / 64, lane = tid % 64, col = lane % 32, half = lane / 32;
    const bf16_t* Xh = X + (size_t)bh * N * D;
    uint16_t* Yh = Y + (size_t)bh * N * out_stride;
    const bool vec_store = (out_stride % 4) == 0;
    const bool want_norm = kmax != nullptr && z == 1;
    float norm2_max = 0.0f;  // largest squared row norm among this lane's tokens

#pragma unroll 1
    for (int it = 0; it < kProjIters; ++it) {
        const int tok = blk * kProjTokensPerBlock + (it * 4 + wave) * kProjTokensPerWave + col;
        const bool valid = tok < N;
        bf16x8 xf[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            uint4 v = make_uint4(0, 0, 0, 0);
            if (valid) v = load16(Xh + (size_t)tok * D + ks * 16 + half * 8);
            xf[ks] = as_bf16x8(v);
        }
        float norm2 = 0.0f;  // squared norm over this lane's half of the columns
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            f32x16 acc = f32x16_fill(0.0f);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const bf16x8 a = as_bf16x8(load16(Pt + (mb * 32 + col) * PROW + ks * 16 + half * 8));
                acc = mfma32x32x16(a, xf[ks], acc);
            }
            if (want_norm) {
#pragma unroll
                for (int i = 0; i < 16; ++i) norm2 += acc[i] * acc[i];
            }
            if (!valid) continue;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int c0 = mb * 32 + 8 * g + 4 * half;
                if (c0 >= out_cols) continue;
                uint16_t* dst = Yh + (size_t)tok * out_stride + c0;
                uint2 w;
                w.x = pack_out<F16>(acc[4 * g + 0] * out_scale, acc[4 * g + 1] * out_scale);
                w.y = pack_out<F16>(acc[4 * g + 2] * out_scale, acc[4 * g + 3] * out_scale);
                if (vec_store && c0 + 4 <= out_cols) {
                    *reinterpret_cast<uint2*>(dst) = w;
                } else {
                    const uint16_t v[4] = {(uint16_t)(w.x & 0xffffu), (uint16_t)(w.x >> 16),
                                           (uint16_t)(w.y & 0xffffu), (uint16_t)(w.y >> 16)};
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (c0 + r < out_cols) dst[r] = v[r];
                }
            }
        }
        if (want_norm) {
            // lanes l and l ^ 32 hold the two halves of one token's columns
            const float full = halves_sum(norm2) * out_scale * out_scale;
            if (valid) norm2_max = fmaxf(norm2_max, full);
        }
    }
    if (want_norm) {
        float v = norm2_max;
#pragma unroll
        for (int o = 16; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
        if (lane == 0) wave_max[wave] = v;
        __syncthreads();
        if (tid == 0) {
            float b = wave_max[0];
#pragma unroll
            for (int w = 1; w < kProjThreads / 64; ++w) b = fmaxf(b, wave_max[w]);
            kmax[(size_t)bh * nblk + blk] = sqrtf(b);
        }
    }
}

template <int D, int MB, bool F16>
hipError_t launch(const void* X0, const void* X1, const void* P, void* Y0, void* Y1, int nz,
                  int BH, int H, int N, int m, int out_stride, int out_cols, float s0, float s1,
                  float* kmax, hipStream_t stream) {
    const long long nblk = (N + kProjTokensPerBlock - 1) / kProjTokensPerBlock;
    const long long blocks = nblk * BH * nz;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    project_bf16_kernel<D, MB, F16><<<dim3((unsigned)blocks), kProjThreads, 0, stream>>>(
        static_cast<const bf16_t*>(X0), static_cast<const bf16_t*>(X1),
        static_cast<const bf16_t*>(P), static_cast<uint16_t*>(Y0), static_cast<uint16_t*>(Y1),
        N, BH, H, m, out_stride, out_cols, s0, s1, kmax);
    return hipGetLastError();
}

template <int D, bool F16>
hipError_t launch_d(const void* X0, const void* X1, const void* P, void* Y0, void* Y1, int nz,
                    int BH, int H, int N, int m, int out_stride, int out_cols, float s0,
                    float s1, float* kmax, hipStream_t stream) {
    const int cols = out_cols > m ? out_cols : m;
    const int mb = (cols + 31) / 32;
    switch (mb) {
        case 1: return launch<D, 1, F16>(X0, X1, P, Y0, Y1, nz, BH, H, N, m, out_stride, out_cols, s0, s1, kmax, stream);
        case 2: return launch<D, 2, F16>(X0, X1, P, Y0, Y1, nz, BH, H, N, m, out_stride, out_cols, s0, s1, kmax, stream);
        case 3:
        case 4: return launch<D, 4, F16>(X0, X1, P, Y0, Y1, nz, BH, H, N, m, out_stride, out_cols, s0, s1, kmax, stream);
        default: return hipErrorInvalidValue;
    }
}

template <int D>
hipError_t launch_t(const void* X0, const void* X1, const void* P, void* Y0, void* Y1, int nz,
                    int BH, int H, int N, int m, int out_stride, int out_cols, float s0,
                    float s1, bool out_f16, float* kmax, hipStream_t stream) {
    return out_f16 ? launch_d<D, true>(X0, X1, P, Y0, Y1, nz, BH, H, N, m, out_stride, out_cols, s0, s1, kmax, stream)
                   : launch_d<D, false>(X0, X1, P, Y0, Y1, nz, BH, H, N, m, out_stride, out_cols, s0, s1, kmax, stream);
}

}  // namespace

hipError_t launch_project_bf16(const void* X0, const void* X1, const void* P, void* Y0,
                               void* Y1, int nz, int BH, int H, int N, int d, int m,
                               int out_stride, int out_cols, float out_scale0,
                               float out_scale1, bool out_f16, float* kmax,
                               hipStream_t stream) {
    switch (d) {
        case 64: return launch_t<64>(X0, X1, P, Y0, Y1, nz, BH, H, N, m, out_stride, out_cols, out_scale0, out_scale1, out_f16, kmax, stream);
        case 128: return launch_t<128>(X0, X1, P, Y0, Y1, nz, BH, H, N, m, out_stride, out_cols, out_scale0, out_scale1, out_f16, kmax, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace spa
