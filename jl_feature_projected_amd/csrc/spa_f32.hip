// spa_f32.hip -- the fp32 path: projection and projected attention in fp32 on the VALU.
//
// Same operation as the bf16 path ("Sparse Projection Attention" page, Sec. 3.1.2-3.1.3 and
// Algorithm 1; "Projection-Decomposition Attention (PDA)" page, Algorithm 2.1 steps 1-3
// and 5), for inputs that must not be rounded to bf16. It is the small, latency-bound path:
// no MFMA, straightforward tiling, an exact (non-lazy) online softmax in natural-exponent
// units, every product and sum in fp32.
#include <hip/hip_runtime.h>
#include <math.h>

#include "spa_internal.h"

namespace spa {
namespace {

__global__ __launch_bounds__(256) void project_f32_kernel(const float* __restrict__ X,
                                                          const float* __restrict__ P,
                                                          float* __restrict__ Y, int N, int H,
                                                          int d, int m, float out_scale) {
    const long per_head = ((long)N * m + 255) / 256;  // blocks per head
    const int bh = (int)(blockIdx.x / per_head);
    const long idx = (long)(blockIdx.x % per_head) * blockDim.x + threadIdx.x;
    if (idx >= (long)N * m) return;
    const int n = (int)(idx / m), c = (int)(idx % m);
    const float* x = X + ((size_t)bh * N + n) * d;
    const float* p = P + (size_t)(bh % H) * d * m + c;
    float acc = 0.0f;
    for (int k = 0; k < d; ++k) acc = fmaf(x[k], p[(size_t)k * m], acc);
    Y[((size_t)bh * N + n) * m + c] = acc * out_scale;
}

constexpr int kQ = 64;      // queries per workgroup
constexpr int kKeys = 64;   // keys per LDS tile
constexpr int kParts = 4;   // threads per query, each owning every 4th output column
constexpr int kMaxDv = 128;

// One workgroup: 64 queries of one head. Thread (q, part) keeps its query's projected row
// (MM floats, zero past m) and the output columns part, part+4, ... in registers.
template <int MM>
__global__ __launch_bounds__(256) void attn_f32_kernel(const float* __restrict__ Qt,
                                                       const float* __restrict__ Kt,
                                                       const float* __restrict__ V,
                                                       float* __restrict__ O,
                                                       float* __restrict__ lse, int N, int m,
                                                       int dv, int causal, float scale) {
    constexpr int OC = kMaxDv / kParts;
    __shared__ float Ks[kKeys * MM];
    __shared__ float Vs[kKeys * kMaxDv];

    const int nqb = (N + kQ - 1) / kQ;
    const int bh = blockIdx.x / nqb;
    const int q0 = (blockIdx.x % nqb) * kQ;
    const int tid = threadIdx.x;
    const int qi = tid % kQ, part = tid / kQ;
    const int q = q0 + qi;
    const float* Qh = Qt + (size_t)bh * N * m;
    const float* Kh = Kt + (size_t)bh * N * m;
    const float* Vh = V + (size_t)bh * N * dv;

    float qr[MM];
#pragma unroll
    for (int c = 0; c < MM; ++c) qr[c] = (q < N && c < m) ? Qh[(size_t)q * m + c] : 0.0f;
    float o[OC];
#pragma unroll
    for (int i = 0; i < OC; ++i) o[i] = 0.0f;
    float mx = -INFINITY, l = 0.0f;

    const int kend = causal ? min(N, q0 + kQ) : N;
    for (int k0 = 0; k0 < kend; k0 += kKeys) {
        __syncthreads();
        for (int e = tid; e < kKeys * MM; e += 256) {
            const int j = e / MM, c = e % MM;
            Ks[e] = (k0 + j < N && c < m) ? Kh[(size_t)(k0 + j) * m + c] : 0.0f;
        }
        for (int e = tid; e < kKeys * dv; e += 256) {
            const int j = e / dv;
            Vs[j * kMaxDv + e % dv] = (k0 + j < N) ? Vh[(size_t)k0 * dv + e] : 0.0f;
        }
        __syncthreads();
        float s[kKeys];
        float tmax = -INFINITY;
#pragma unroll
        for (int j = 0; j < kKeys; ++j) {
            float acc = 0.0f;
#pragma unroll
            for (int c = 0; c < MM; ++c) acc = fmaf(qr[c], Ks[j * MM + c], acc);
            const int key = k0 + j;
            s[j] = (key >= N || (causal && key > q)) ? -INFINITY : acc * scale;
            tmax = fmaxf(tmax, s[j]);
        }
        if (tmax == -INFINITY) continue;  // every key of this tile is masked for q
        const float mnew = fmaxf(mx, tmax);
        const float corr = expf(mx - mnew);  // 0 on the first contributing tile
        l *= corr;
#pragma unroll
        for (int i = 0; i < OC; ++i) o[i] *= corr;
        mx = mnew;
#pragma unroll
        for (int j = 0; j < kKeys; ++j) {
            const float p = expf(s[j] - mx);
            l += p;
#pragma unroll
            for (int i = 0; i < OC; ++i) {
                const int cc = part + kParts * i;
                if (cc < dv) o[i] = fmaf(p, Vs[j * kMaxDv + cc], o[i]);
            }
        }
    }
    if (q >= N) return;
    const float inv = 1.0f / l;
#pragma unroll
    for (int i = 0; i < OC; ++i) {
        const int cc = part + kParts * i;
        if (cc < dv) O[((size_t)bh * N + q) * dv + cc] = o[i] * inv;
    }
    if (lse && part == 0) lse[(size_t)bh * N + q] = mx + logf(l);
}

}  // namespace

hipError_t launch_project_f32(const float* X, const float* P, float* Y, int BH, int H, int N,
                              int d, int m, float out_scale, hipStream_t stream) {
    const long long blocks = (((long long)N * m + 255) / 256) * BH;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    project_f32_kernel<<<dim3((unsigned)blocks), 256, 0, stream>>>(X, P, Y, N, H, d, m, out_scale);
    return hipGetLastError();
}

hipError_t launch_attn_f32(const float* Qt, const float* Kt, const float* V, float* O,
                           float* lse, int BH, int N, int m, int dv, bool causal, float scale,
                           hipStream_t stream) {
    if (dv > kMaxDv) return hipErrorInvalidValue;
    const long long blocks = (long long)((N + kQ - 1) / kQ) * BH;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)blocks);
    const int c = causal ? 1 : 0;
    if (m <= 16) attn_f32_kernel<16><<<grid, 256, 0, stream>>>(Qt, Kt, V, O, lse, N, m, dv, c, scale);
    else if (m <= 32) attn_f32_kernel<32><<<grid, 256, 0, stream>>>(Qt, Kt, V, O, lse, N, m, dv, c, scale);
    else if (m <= 64) attn_f32_kernel<64><<<grid, 256, 0, stream>>>(Qt, Kt, V, O, lse, N, m, dv, c, scale);
    else if (m <= 128) attn_f32_kernel<128><<<grid, 256, 0, stream>>>(Qt, Kt, V, O, lse, N, m, dv, c, scale);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace spa
