// spa_bwd_f32.hip -- the backward of the fp32 path: every product and sum in fp32 on the VALU.
//
// The gradients of the projected attention: the chain rule through the forward's definition
// ("Sparse Projection Attention" page, Sec. 3.1.3 and Algorithm 1; its Sec. 3.4.1 Gradient
// Flow writes the query term of the projection's gradient, which Algorithm 2 trains the
// projection with; the key term enters the same way). With A = softmax(scale Qt Kt^T [+ mask]) recomputed from
// the forward's natural-log lse:
//   D_i = <dO_i, O_i>,  dS_ij = A_ij (<dO_i, V_j> - D_i),  dV_j = sum_i A_ij dO_i,
//   dQt = scale dS Kt,  dKt = scale dS^T Qt,  dQ = dQt P^T,  dK = dKt P^T,
//   dP_h = sum over batches and tokens of Q^T dQt + K^T dKt.
// Like the fp32 forward it is the small, latency-bound path: no MFMA, straightforward
// tiling. A row (a query or a key) is owned by eight adjacent lanes, lane `part` holding the
// feature columns part, part + 8, ...; dot products over the features are the eight partial
// sums added by three lane exchanges. Every sum runs in a fixed order, so the results are
// deterministic.
#include <hip/hip_runtime.h>
#include <math.h>

#include "spa_internal.h"

namespace spa {
namespace {

constexpr int kThreads = 256;
constexpr int kParts = 8;                   // lanes per row
constexpr int kRows = kThreads / kParts;    // rows (queries or keys) per workgroup
constexpr int kTile = 32;                   // rows of the other side per LDS tile
constexpr int kMaxDv = 128;
constexpr int VC = kMaxDv / kParts;         // value columns per lane

__device__ __forceinline__ float sum8(float x) {
    x += __shfl_xor(x, 1, kParts);
    x += __shfl_xor(x, 2, kParts);
    x += __shfl_xor(x, 4, kParts);
    return x;
}

// Query-major: D_i and dQt_i = scale sum_j dS_ij Kt_j for kRows queries of one head.
template <int MM>
__global__ __launch_bounds__(kThreads) void bwd_q_f32_kernel(
    const float* __restrict__ Qt, const float* __restrict__ Kt, const float* __restrict__ V,
    const float* __restrict__ O, const float* __restrict__ dO, const float* __restrict__ lse,
    float* __restrict__ Dout, float* __restrict__ dQt, int N, int m, int dv, int causal,
    float scale) {
    constexpr int MC = MM / kParts;
    __shared__ float Ks[kTile][MM];
    __shared__ float Vs[kTile][kMaxDv];
    const int nb = (N + kRows - 1) / kRows;
    const int bh = blockIdx.x / nb;
    const int q0 = (blockIdx.x % nb) * kRows;
    const int tid = threadIdx.x, qi = tid / kParts, part = tid % kParts;
    const int q = q0 + qi;
    const bool valid = q < N;
    const size_t row = (size_t)bh * N + q;

    float qr[MC], dq[MC], dor[VC];
    float dpart = 0.0f;
#pragma unroll
    for (int k = 0; k < MC; ++k) {
        const int c = part + kParts * k;
        qr[k] = (valid && c < m) ? Qt[row * m + c] : 0.0f;
        dq[k] = 0.0f;
    }
#pragma unroll
    for (int k = 0; k < VC; ++k) {
        const int c = part + kParts * k;
        dor[k] = (valid && c < dv) ? dO[row * dv + c] : 0.0f;
        if (valid && c < dv) dpart = fmaf(dor[k], O[row * dv + c], dpart);
    }
    const float Di = sum8(dpart);
    if (valid && part == 0) Dout[row] = Di;
    const float L = valid ? lse[row] : 0.0f;

    const float* Kh = Kt + (size_t)bh * N * m;
    const float* Vh = V + (size_t)bh * N * dv;
    const int kend = causal ? min(N, q0 + kRows) : N;
    for (int k0 = 0; k0 < kend; k0 += kTile) {
        __syncthreads();
        for (int e = tid; e < kTile * MM; e += kThreads) {
            const int j = e / MM, c = e % MM;
            Ks[j][c] = (k0 + j < N && c < m) ? Kh[(size_t)(k0 + j) * m + c] : 0.0f;
        }
        for (int e = tid; e < kTile * kMaxDv; e += kThreads) {
            const int j = e / kMaxDv, c = e % kMaxDv;
            Vs[j][c] = (k0 + j < N && c < dv) ? Vh[(size_t)(k0 + j) * dv + c] : 0.0f;
        }
        __syncthreads();
        for (int j = 0; j < kTile; ++j) {
            const int key = k0 + j;
            float sp = 0.0f, pp = 0.0f;
#pragma unroll
            for (int k = 0; k < MC; ++k) sp = fmaf(qr[k], Ks[j][part + kParts * k], sp);
#pragma unroll
            for (int k = 0; k < VC; ++k) pp = fmaf(dor[k], Vs[j][part + kParts * k], pp);
            const float s = sum8(sp), dp = sum8(pp);
            const bool masked = !valid || key >= N || (causal && key > q);
            const float a = masked ? 0.0f : expf(scale * s - L);
            const float ds = a * (dp - Di);
#pragma unroll
            for (int k = 0; k < MC; ++k) dq[k] = fmaf(ds, Ks[j][part + kParts * k], dq[k]);
        }
    }
    if (!valid) return;
#pragma unroll
    for (int k = 0; k < MC; ++k) {
        const int c = part + kParts * k;
        if (c < m) dQt[row * m + c] = scale * dq[k];
    }
}

// Key-major: dV_j = sum_i A_ij dO_i and dKt_j = scale sum_i dS_ij Qt_i for kRows keys.
template <int MM>
__global__ __launch_bounds__(kThreads) void bwd_kv_f32_kernel(
    const float* __restrict__ Qt, const float* __restrict__ Kt, const float* __restrict__ V,
    const float* __restrict__ dO, const float* __restrict__ lse, const float* __restrict__ Din,
    float* __restrict__ dKt, float* __restrict__ dV, int N, int m, int dv, int causal,
    float scale) {
    constexpr int MC = MM / kParts;
    __shared__ float Qs[kTile][MM];
    __shared__ float dOs[kTile][kMaxDv];
    __shared__ float Ls[kTile], Ds[kTile];
    const int nb = (N + kRows - 1) / kRows;
    const int bh = blockIdx.x / nb;
    const int k0 = (blockIdx.x % nb) * kRows;
    const int tid = threadIdx.x, kj = tid / kParts, part = tid % kParts;
    const int key = k0 + kj;
    const bool valid = key < N;
    const size_t row = (size_t)bh * N + key;

    float kr[MC], dk[MC], vr[VC], dvv[VC];
#pragma unroll
    for (int k = 0; k < MC; ++k) {
        const int c = part + kParts * k;
        kr[k] = (valid && c < m) ? Kt[row * m + c] : 0.0f;
        dk[k] = 0.0f;
    }
#pragma unroll
    for (int k = 0; k < VC; ++k) {
        const int c = part + kParts * k;
        vr[k] = (valid && c < dv) ? V[row * dv + c] : 0.0f;
        dvv[k] = 0.0f;
    }

    const float* Qh = Qt + (size_t)bh * N * m;
    const float* dOh = dO + (size_t)bh * N * dv;
    const int qbeg = causal ? k0 : 0;  // queries before the block's first key see none of it
    for (int t0 = qbeg; t0 < N; t0 += kTile) {
        __syncthreads();
        for (int e = tid; e < kTile * MM; e += kThreads) {
            const int i = e / MM, c = e % MM;
            Qs[i][c] = (t0 + i < N && c < m) ? Qh[(size_t)(t0 + i) * m + c] : 0.0f;
        }
        for (int e = tid; e < kTile * kMaxDv; e += kThreads) {
            const int i = e / kMaxDv, c = e % kMaxDv;
            dOs[i][c] = (t0 + i < N && c < dv) ? dOh[(size_t)(t0 + i) * dv + c] : 0.0f;
        }
        if (tid < kTile) {
            const bool in = t0 + tid < N;
            Ls[tid] = in ? lse[(size_t)bh * N + t0 + tid] : 0.0f;
            Ds[tid] = in ? Din[(size_t)bh * N + t0 + tid] : 0.0f;
        }
        __syncthreads();
        for (int i = 0; i < kTile; ++i) {
            const int q = t0 + i;
            float sp = 0.0f, pp = 0.0f;
#pragma unroll
            for (int k = 0; k < MC; ++k) sp = fmaf(kr[k], Qs[i][part + kParts * k], sp);
#pragma unroll
            for (int k = 0; k < VC; ++k) pp = fmaf(vr[k], dOs[i][part + kParts * k], pp);
            const float s = sum8(sp), dp = sum8(pp);
            const bool masked = !valid || q >= N || (causal && key > q);
            const float a = masked ? 0.0f : expf(scale * s - Ls[i]);
            const float ds = a * (dp - Ds[i]);
#pragma unroll
            for (int k = 0; k < VC; ++k) dvv[k] = fmaf(a, dOs[i][part + kParts * k], dvv[k]);
#pragma unroll
            for (int k = 0; k < MC; ++k) dk[k] = fmaf(ds, Qs[i][part + kParts * k], dk[k]);
        }
    }
    if (!valid) return;
#pragma unroll
    for (int k = 0; k < MC; ++k) {
        const int c = part + kParts * k;
        if (c < m) dKt[row * m + c] = scale * dk[k];
    }
#pragma unroll
    for (int k = 0; k < VC; ++k) {
        const int c = part + kParts * k;
        if (c < dv) dV[row * dv + c] = dvv[k];
    }
}

// Y[bh, n, k] = sum_c G[bh, n, c] P[h, k, c]  (G P^T: the projection's gradient back to d).
__global__ __launch_bounds__(kThreads) void unproject_f32_kernel(const float* __restrict__ G,
                                                                 const float* __restrict__ P,
                                                                 float* __restrict__ Y, int N,
                                                                 int H, int d, int m) {
    const long long per_head = ((long long)N * d + kThreads - 1) / kThreads;
    const int bh = (int)(blockIdx.x / per_head);
    const long long idx = (long long)(blockIdx.x % per_head) * kThreads + threadIdx.x;
    if (idx >= (long long)N * d) return;
    const int n = (int)(idx / d), k = (int)(idx % d);
    const float* g = G + ((size_t)bh * N + n) * m;
    const float* p = P + ((size_t)(bh % H) * d + k) * m;
    float acc = 0.0f;
    for (int c = 0; c < m; ++c) acc = fmaf(g[c], p[c], acc);
    Y[((size_t)bh * N + n) * d + k] = acc;
}

// dP[h, k, c] = sum over batches b and tokens n of Q[b,h,n,k] dQt[b,h,n,c] + K[b,h,n,k]
// dKt[b,h,n,c]. One workgroup per (h, k): lane t takes column t % m and every G-th token of
// the flattened (batch, token) range from t / m (G = 256 / m groups); the groups' partial
// sums are then added in group order.
__global__ __launch_bounds__(kThreads) void dp_f32_kernel(const float* __restrict__ Q,
                                                          const float* __restrict__ K,
                                                          const float* __restrict__ dQt,
                                                          const float* __restrict__ dKt,
                                                          float* __restrict__ dP, int B, int H,
                                                          int N, int d, int m) {
    __shared__ float part[kThreads];
    const int h = blockIdx.x / d, k = blockIdx.x % d;
    const int groups = kThreads / m;
    const int t = threadIdx.x, c = t % m, g = t / m;
    float acc = 0.0f;
    if (g < groups) {
        const long long rows = (long long)B * N;
        for (long long r = g; r < rows; r += groups) {
            const int b = (int)(r / N), n = (int)(r % N);
            const size_t row = ((size_t)b * H + h) * N + n;
            acc = fmaf(Q[row * d + k], dQt[row * m + c], acc);
            acc = fmaf(K[row * d + k], dKt[row * m + c], acc);
        }
    }
    part[t] = acc;
    __syncthreads();
    if (t < m) {
        float s = 0.0f;
        for (int gg = 0; gg < groups; ++gg) s += part[gg * m + t];
        dP[((size_t)h * d + k) * m + t] = s;
    }
}

template <int MM>
hipError_t launch_core(const BwdF32Args& a, hipStream_t s) {
    const int nb = (a.N + kRows - 1) / kRows;
    const long long grid = (long long)nb * a.B * a.H;
    if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    bwd_q_f32_kernel<MM><<<dim3((unsigned)grid), kThreads, 0, s>>>(
        a.Qt, a.Kt, a.V, a.O, a.dO, a.lse, a.D, a.dQt, a.N, a.m, a.dv, a.causal, a.scale);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    bwd_kv_f32_kernel<MM><<<dim3((unsigned)grid), kThreads, 0, s>>>(
        a.Qt, a.Kt, a.V, a.dO, a.lse, a.D, a.dKt, a.dV, a.N, a.m, a.dv, a.causal, a.scale);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bwd_f32(const BwdF32Args& a, hipStream_t s) {
    if (a.m < 1 || a.m > 128 || a.dv < 1 || a.dv > kMaxDv || a.d < 1) return hipErrorInvalidValue;
    const int BH = a.B * a.H;
    hipError_t e = launch_project_f32(a.Q, a.P, a.Qt, BH, a.H, a.N, a.d, a.m, 1.0f, s, a.K, a.Kt);
    if (e != hipSuccess) return e;
    if (a.m <= 16) e = launch_core<16>(a, s);
    else if (a.m <= 32) e = launch_core<32>(a, s);
    else if (a.m <= 64) e = launch_core<64>(a, s);
    else e = launch_core<128>(a, s);
    if (e != hipSuccess) return e;
    const long long ublocks = (((long long)a.N * a.d + kThreads - 1) / kThreads) * BH;
    if (ublocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    unproject_f32_kernel<<<dim3((unsigned)ublocks), kThreads, 0, s>>>(a.dQt, a.P, a.dQ, a.N, a.H,
                                                                      a.d, a.m);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    unproject_f32_kernel<<<dim3((unsigned)ublocks), kThreads, 0, s>>>(a.dKt, a.P, a.dK, a.N, a.H,
                                                                      a.d, a.m);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    dp_f32_kernel<<<dim3((unsigned)(a.H * a.d)), kThreads, 0, s>>>(a.Q, a.K, a.dQt, a.dKt, a.dP,
                                                                   a.B, a.H, a.N, a.d, a.m);
    return hipGetLastError();
}

}  // namespace spa
