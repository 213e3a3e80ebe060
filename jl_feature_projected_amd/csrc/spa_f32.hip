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

constexpr int kQW = 4;      // queries per workgroup (one per wave)
constexpr int kKeys = 64;   // keys per tile (one per lane)
constexpr int kMaxDv = 128;

// Maximum over the 64 lanes of a wave.
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
    return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
    return x;
}

// One workgroup: 4 queries of one head, one wave per query. Per 64-key tile (staged in LDS,
// the next tile's loads in flight in registers while this one is computed), lane k scores
// key k0 + k for the wave's query (MM-float projected row in registers, zero past m); the
// tile maximum is a wave reduction; the lane exponentiates its score against the new running
// maximum (exact online softmax) and the wave accumulates output columns lane and lane + 64
// (DVC of them) over the tile's 64 keys, each weight broadcast from its lane, the V columns
// read four keys at a time from a transposed LDS copy. The normaliser is kept per lane over
// its own keys and summed at the end.
template <int MM, int DVC>
__global__ __launch_bounds__(256) void attn_f32_kernel(const float* __restrict__ Qt,
                                                       const float* __restrict__ Kt,
                                                       const float* __restrict__ V,
                                                       float* __restrict__ O,
                                                       float* __restrict__ lse, int N, int m,
                                                       int dv, int causal, float scale) {
    constexpr int KS = MM + 1;               // LDS row stride of the key tile (floats)
    constexpr int VS = kKeys + 4;            // LDS row stride of the transposed value tile
    constexpr int KPT = kKeys * MM / 256;    // key-tile floats per thread (at most)
    constexpr int VPT = kKeys * 64 * DVC / 256;  // value-tile floats per thread (at most)
    // (one spare float after each tile takes the loads that fall past it)
    __shared__ __attribute__((aligned(16))) float Ks[kKeys * KS + 4];
    __shared__ __attribute__((aligned(16))) float Vs[64 * DVC * VS + 4];

    const int nqb = (N + kQW - 1) / kQW;
    const int bh = blockIdx.x / nqb;
    const int q0 = (blockIdx.x % nqb) * kQW;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int q = q0 + wave;
    const float* Qh = Qt + (size_t)bh * N * m;
    const float* Kh = Kt + (size_t)bh * N * m;
    const float* Vh = V + (size_t)bh * N * dv;

    // Columns m .. MM-1 of the key tile stay zero (the query row is zero there too).
    for (int e = tid; e < kKeys * KS; e += 256) Ks[e] = 0.0f;
    float qr[MM];
#pragma unroll
    for (int c = 0; c < MM; ++c) qr[c] = (q < N && c < m) ? Qh[(size_t)q * m + c] * scale : 0.0f;

    // The tile [k0, k0 + 64) of K~ (64 m floats) and of V (64 dv floats) is contiguous in
    // memory; thread tid loads elements tid, tid + 256, ... of each into registers.
    const int kend = causal ? min(N, q0 + kQW) : N;
    const int ntiles = (kend + kKeys - 1) / kKeys;
    // Two register sets of tile loads: the loads of tile t + 2 go out while tile t is
    // computed, and tile t + 1 is staged from the other set after it.
    struct TileRegs {
        float k[KPT], v[VPT];
    };
    TileRegs ra, rb;
    // Buffer resources from the tile's first row to the head's end: loads past it read as
    // zero, with no branch (at most N * 128 * 4 <= 2^31 bytes, a 32-bit record count).
    auto load = [&](TileRegs& r, int t) __attribute__((always_inline)) {
        const int r0 = t * kKeys;
        const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(Kh + (size_t)r0 * m), (short)0, (int)((unsigned)(N - r0) * (unsigned)m * 4u),
            0x00020000);
        const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(Vh + (size_t)r0 * dv), (short)0, (int)((unsigned)(N - r0) * (unsigned)dv * 4u),
            0x00020000);
#pragma unroll
        for (int i = 0; i < KPT; ++i)
            r.k[i] = __builtin_bit_cast(
                float, __builtin_amdgcn_raw_buffer_load_b32(krs, 4 * (tid + 256 * i), 0, 0));
#pragma unroll
        for (int i = 0; i < VPT; ++i)
            r.v[i] = __builtin_bit_cast(
                float, __builtin_amdgcn_raw_buffer_load_b32(vrs, 4 * (tid + 256 * i), 0, 0));
    };
    // LDS slots of those elements (the same for every tile; past the tile: the spare float).
    int kslot[KPT], vslot[VPT];
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
        const int e = tid + 256 * i;
        kslot[i] = e < kKeys * m ? (e / m) * KS + e % m : kKeys * KS;
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
        const int e = tid + 256 * i;
        vslot[i] = e < kKeys * dv ? (e % dv) * VS + e / dv : 64 * DVC * VS;
    }
    auto stage = [&](const TileRegs& r) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < KPT; ++i) Ks[kslot[i]] = r.k[i];
#pragma unroll
        for (int i = 0; i < VPT; ++i) Vs[vslot[i]] = r.v[i];
    };

    float o[DVC];
#pragma unroll
    for (int j = 0; j < DVC; ++j) o[j] = 0.0f;
    float mx = -INFINITY, lpart = 0.0f;
    load(ra, 0);
    if (ntiles > 1) load(rb, 1);
    __syncthreads();  // the zeroed key tile before it is staged over
    stage(ra);
    __syncthreads();
    // Tile t from LDS; `cur` held its loads (now free), `nxt` holds tile t + 1's.
    auto step = [&](int t, TileRegs& cur, const TileRegs& nxt) __attribute__((always_inline)) {
        if (t + 2 < ntiles) load(cur, t + 2);
        const int key = t * kKeys + lane;
        float sc = 0.0f;
#pragma unroll
        for (int c = 0; c < MM; ++c) sc = fmaf(qr[c], Ks[lane * KS + c], sc);
        if (key >= N || (causal && key > q)) sc = -INFINITY;
        const float mnew = fmaxf(mx, wave_max(sc));
        // every key so far masked (only for queries past N): nothing to add
        const bool none = mnew == -INFINITY;
        const float corr = none ? 1.0f : expf(mx - mnew);  // 0 on the first contributing tile
        const float p = none ? 0.0f : expf(sc - mnew);
        lpart = fmaf(lpart, corr, p);
        mx = mnew;
#pragma unroll
        for (int j = 0; j < DVC; ++j) o[j] *= corr;
        const float* vrow[DVC];
#pragma unroll
        for (int j = 0; j < DVC; ++j) vrow[j] = Vs + (lane + 64 * j) * VS;
#pragma unroll 4
        for (int k = 0; k < kKeys; k += 4) {
            float pk[4];
#pragma unroll
            for (int u = 0; u < 4; ++u)
                pk[u] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(p), k + u));
#pragma unroll
            for (int j = 0; j < DVC; ++j) {
                const float4 v4 = *reinterpret_cast<const float4*>(vrow[j] + k);
                o[j] = fmaf(pk[0], v4.x, o[j]);
                o[j] = fmaf(pk[1], v4.y, o[j]);
                o[j] = fmaf(pk[2], v4.z, o[j]);
                o[j] = fmaf(pk[3], v4.w, o[j]);
            }
        }
        if (t + 1 < ntiles) {
            __syncthreads();  // every wave is done with this tile
            stage(nxt);
            __syncthreads();
        }
    };
    for (int t = 0; t < ntiles; t += 2) {
        step(t, ra, rb);
        if (t + 1 < ntiles) step(t + 1, rb, ra);
    }
    const float l = wave_sum(lpart);
    if (q >= N) return;
    const float inv = 1.0f / l;
#pragma unroll
    for (int j = 0; j < DVC; ++j)
        if (lane + 64 * j < dv) O[((size_t)bh * N + q) * dv + lane + 64 * j] = o[j] * inv;
    if (lse && lane == 0) lse[(size_t)bh * N + q] = mx + logf(l);
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
    const long long blocks = (long long)((N + kQW - 1) / kQW) * BH;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)blocks);
    const int c = causal ? 1 : 0;
#define SPA_F32_LAUNCH(MMV)                                                                  \
    (dv <= 64 ? (attn_f32_kernel<MMV, 1><<<grid, 256, 0, stream>>>(Qt, Kt, V, O, lse, N, m, dv, c, scale), 0) \
              : (attn_f32_kernel<MMV, 2><<<grid, 256, 0, stream>>>(Qt, Kt, V, O, lse, N, m, dv, c, scale), 0))
    if (m <= 16) (void)SPA_F32_LAUNCH(16);
    else if (m <= 32) (void)SPA_F32_LAUNCH(32);
    else if (m <= 64) (void)SPA_F32_LAUNCH(64);
    else if (m <= 128) (void)SPA_F32_LAUNCH(128);
    else return hipErrorInvalidValue;
#undef SPA_F32_LAUNCH
    return hipGetLastError();
}

}  // namespace spa
