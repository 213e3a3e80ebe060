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

// Y = X P for one or two tensors (blockIdx.y selects X0 -> Y0 or X1 -> Y1): one thread per
// output element, a plain fp32 dot product over d in order.
__global__ __launch_bounds__(256) void project_f32_kernel(const float* __restrict__ X0,
                                                          const float* __restrict__ X1,
                                                          const float* __restrict__ P,
                                                          float* __restrict__ Y0,
                                                          float* __restrict__ Y1, int N, int H,
                                                          int d, int m, float out_scale) {
    const float* X = blockIdx.y ? X1 : X0;
    float* Y = blockIdx.y ? Y1 : Y0;
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

constexpr int kQ = 16;      // queries per workgroup
constexpr int kKeys = 64;   // keys per LDS tile
constexpr int kParts = 16;  // threads per query
constexpr int kKP = kKeys / kParts;  // keys of a tile scored by each thread
constexpr int kMaxDv = 128;
constexpr int kOC = kMaxDv / kParts;  // output columns owned by each thread

// One workgroup: 16 queries of one head, 16 threads per query. Per 64-key tile, thread
// (q, part) scores keys part*4 .. part*4+3 of the tile for its query (MM-float projected row
// in registers, zero past m); the tile maximum of each query is combined through LDS; the
// thread exponentiates its 4 scores against the new running maximum and publishes the
// weights in LDS; then it accumulates output columns part*8 .. part*8+7 over all 64 keys
// (LDS reads of the key and value rows are 16-byte vectors, the same address across the
// lanes of a query group). The normaliser is kept per thread over its own keys and summed
// at the end.
template <int MM>
__global__ __launch_bounds__(256) void attn_f32_kernel(const float* __restrict__ Qt,
                                                       const float* __restrict__ Kt,
                                                       const float* __restrict__ V,
                                                       float* __restrict__ O,
                                                       float* __restrict__ lse, int N, int m,
                                                       int dv, int causal, float scale) {
    __shared__ __attribute__((aligned(16))) float Ks[kKeys * MM];
    __shared__ __attribute__((aligned(16))) float Vs[kKeys * kMaxDv];
    __shared__ float Ps[kKeys * kQ];
    __shared__ float red[kParts * kQ];

    const int nqb = (N + kQ - 1) / kQ;
    const int bh = blockIdx.x / nqb;
    const int q0 = (blockIdx.x % nqb) * kQ;
    const int tid = threadIdx.x;
    const int qi = tid % kQ, part = tid / kQ;
    const int q = q0 + qi;
    const int c0 = part * kOC;  // first owned output column
    const float* Qh = Qt + (size_t)bh * N * m;
    const float* Kh = Kt + (size_t)bh * N * m;
    const float* Vh = V + (size_t)bh * N * dv;

    float qr[MM];
#pragma unroll
    for (int c = 0; c < MM; ++c) qr[c] = (q < N && c < m) ? Qh[(size_t)q * m + c] : 0.0f;
    float o[kOC];
#pragma unroll
    for (int i = 0; i < kOC; ++i) o[i] = 0.0f;
    float mx = -INFINITY, lpart = 0.0f;

    const int kend = causal ? min(N, q0 + kQ) : N;
    for (int k0 = 0; k0 < kend; k0 += kKeys) {
        __syncthreads();
        for (int e = tid; e < kKeys * MM; e += 256) {
            const int j = e / MM, c = e % MM;
            Ks[e] = (k0 + j < N && c < m) ? Kh[(size_t)(k0 + j) * m + c] : 0.0f;
        }
        for (int e = tid; e < kKeys * kMaxDv; e += 256) {
            const int j = e / kMaxDv, c = e % kMaxDv;
            Vs[e] = (k0 + j < N && c < dv) ? Vh[(size_t)(k0 + j) * dv + c] : 0.0f;
        }
        __syncthreads();
        float s[kKP];
        float pmax = -INFINITY;
#pragma unroll
        for (int jj = 0; jj < kKP; ++jj) {
            const int j = part * kKP + jj, key = k0 + j;
            float acc = 0.0f;
#pragma unroll
            for (int c = 0; c < MM; c += 4) {
                const float4 k4 = *reinterpret_cast<const float4*>(&Ks[j * MM + c]);
                acc = fmaf(qr[c], k4.x, acc);
                acc = fmaf(qr[c + 1], k4.y, acc);
                acc = fmaf(qr[c + 2], k4.z, acc);
                acc = fmaf(qr[c + 3], k4.w, acc);
            }
            s[jj] = (key >= N || (causal && key > q)) ? -INFINITY : acc * scale;
            pmax = fmaxf(pmax, s[jj]);
        }
        red[part * kQ + qi] = pmax;
        __syncthreads();
        float tmax = -INFINITY;
#pragma unroll
        for (int p = 0; p < kParts; ++p) tmax = fmaxf(tmax, red[p * kQ + qi]);
        const float mnew = fmaxf(mx, tmax);
        // every key so far masked (only for queries past N): nothing to add
        const bool none = mnew == -INFINITY;
        const float corr = none ? 1.0f : expf(mx - mnew);  // 0 on the first contributing tile
        lpart *= corr;
#pragma unroll
        for (int jj = 0; jj < kKP; ++jj) {
            const float p = none ? 0.0f : expf(s[jj] - mnew);
            lpart += p;
            Ps[(part * kKP + jj) * kQ + qi] = p;
        }
        mx = mnew;
#pragma unroll
        for (int i = 0; i < kOC; ++i) o[i] *= corr;
        __syncthreads();
        if (c0 < dv) {
#pragma unroll 4
            for (int j = 0; j < kKeys; ++j) {
                const float p = Ps[j * kQ + qi];
#pragma unroll
                for (int i = 0; i < kOC; i += 4) {
                    const float4 v4 = *reinterpret_cast<const float4*>(&Vs[j * kMaxDv + c0 + i]);
                    o[i] = fmaf(p, v4.x, o[i]);
                    o[i + 1] = fmaf(p, v4.y, o[i + 1]);
                    o[i + 2] = fmaf(p, v4.z, o[i + 2]);
                    o[i + 3] = fmaf(p, v4.w, o[i + 3]);
                }
            }
        }
    }
    __syncthreads();
    red[part * kQ + qi] = lpart;
    __syncthreads();
    float l = 0.0f;
#pragma unroll
    for (int p = 0; p < kParts; ++p) l += red[p * kQ + qi];
    if (q >= N) return;
    const float inv = 1.0f / l;
#pragma unroll
    for (int i = 0; i < kOC; ++i)
        if (c0 + i < dv) O[((size_t)bh * N + q) * dv + c0 + i] = o[i] * inv;
    if (lse && part == 0) lse[(size_t)bh * N + q] = mx + logf(l);
}

}  // namespace

hipError_t launch_project_f32(const float* X, const float* P, float* Y, int BH, int H, int N,
                              int d, int m, float out_scale, hipStream_t stream,
                              const float* X1, float* Y1) {
    const long long blocks = (((long long)N * m + 255) / 256) * BH;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)blocks, X1 ? 2u : 1u);
    project_f32_kernel<<<grid, 256, 0, stream>>>(X, X1, P, Y, Y1, N, H, d, m, out_scale);
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
