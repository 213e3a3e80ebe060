// spa_decode.hip -- a few queries against a cache of projected keys (decode / inference).
//
// What it computes: the forward of the projected attention ("Sparse Projection Attention"
// page, Sec. 3.1.3 and Algorithm 1; "Projection-Decomposition Attention" Algorithm 2.1 steps
// 1-3 and 5) for Nq queries against Nk cached keys. Keys enter the scores only through
// Kt = K P, so the cache holds Kt (fp16, m per key) instead of K (d per key), next to V.
// The causal mask is aligned to the end of the cache: query i (of Nq) sits at position
// Nk - Nq + i and sees keys j <= Nk - Nq + i.
//
// decode_attn_kernel: one workgroup per (head, group of up to QN queries, key split). It
//   projects its queries (fp32, times scale*log2 e; Q rows and P staged in LDS), then
//   streams its split of the cache in blocks of 256 keys: one key per thread for the
//   scores, an exact online softmax per query (running max and sum in base-2 units), and
//   the weights times V with fp32 FMAs, each thread owning COLS columns of V (16-byte row
//   loads for COLS = 8). Writes per (query, split) the unnormalised output, the running
//   max and the sum.
// decode_combine_kernel: per query, merges the splits in a fixed order (log-sum-exp).
// Both are HBM-bound: every cache byte is read once per (head, query group).
#include "spa_device.h"
#include "spa_internal.h"

namespace spa {
namespace {

constexpr int kDecThreads = 256;
constexpr int kDecKeys = 256;  // keys per block: one per thread in the score phase
constexpr int kDecMaxM = 128;

template <int DV, int QN>
__global__ __launch_bounds__(kDecThreads) void decode_attn_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ Kc,
    const uint16_t* __restrict__ Vc, const uint16_t* __restrict__ P, float qscale, int causal,
    int H, int Nq, int Nk, int rows, int d, int m, int nqg, int nsplit, int chunk,
    float* __restrict__ partO, float* __restrict__ partML) {
    constexpr int COLS = QN <= 4 ? 8 : QN <= 8 ? 4 : 2;  // V columns per thread
    constexpr int CT = DV / COLS;            // threads per V row
    constexpr int KG = kDecThreads / CT;     // key groups
    constexpr int KPG = kDecKeys / KG;       // keys per group per block
    static_assert(KPG % 4 == 0, "weights are read four keys at a time");
    // LDS (dynamic, decode_lds_bytes): the projected queries [QN][kDecMaxM], then either the
    // projection's staging (P [d][m] and the Q rows [QN][d], bf16) or the score / weight tile
    // [QN][kDecKeys] followed by the key groups' partial outputs [KG][QN][DV].
    extern __shared__ __attribute__((aligned(16))) char dsm[];
    float(*qt)[kDecMaxM] = reinterpret_cast<float(*)[kDecMaxM]>(dsm);
    char* un = dsm + QN * kDecMaxM * sizeof(float);
    float(*S)[kDecKeys] = reinterpret_cast<float(*)[kDecKeys]>(un);
    float(*red)[QN][DV] = reinterpret_cast<float(*)[QN][DV]>(un + QN * kDecKeys * sizeof(float));
    __shared__ float Mrun[QN], Lrun[QN], alpha[QN];

    const int sp = blockIdx.x % nsplit;
    const int rest = blockIdx.x / nsplit;
    const int qg = rest % nqg;
    const int bh = rest / nqg;
    const int h = bh % H;
    const int q0 = qg * QN;
    const int nq = min(QN, Nq - q0);
    const int kbeg = sp * chunk;
    const int kend = min(Nk, kbeg + chunk);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int ct = tid % CT, kgi = tid / CT;
    const int last = Nk - Nq + q0;  // absolute position of query q0 (causal limit)

    // projected queries (zero rows past nq): Q rows and P staged in LDS (in the space of the
    // score tile and of the final reduction, not yet in use), then 8 threads per output,
    // each summing d/8 products, and a shuffle reduction
    {
        uint16_t* Ps = reinterpret_cast<uint16_t*>(un);  // [d][m]
        uint16_t* Qs = Ps + d * m;                         // [QN][d]
        const uint16_t* Ph = P + (size_t)h * d * m;
        for (int i = tid; i < d * m; i += kDecThreads) Ps[i] = Ph[i];
        const uint16_t* Qh = Q + ((size_t)bh * Nq + q0) * d;
        for (int i = tid; i < nq * d; i += kDecThreads) Qs[i] = Qh[i];
        __syncthreads();
        const int slice = tid & 7, per = d / 8;
        for (int o0 = 0; o0 < QN * m; o0 += kDecThreads / 8) {
            const int o = o0 + (tid >> 3);
            const int q = o / m, c = o - q * m;
            float a = 0.0f;
            if (o < nq * m) {
                for (int k = slice * per; k < slice * per + per; ++k)
                    a += __uint_as_float((uint32_t)Qs[q * d + k] << 16) *
                         __uint_as_float((uint32_t)Ps[k * m + c] << 16);
            }
            a += __shfl_xor(a, 1, 8);
            a += __shfl_xor(a, 2, 8);
            a += __shfl_xor(a, 4, 8);
            if (slice == 0 && o < QN * m) qt[q][c] = a * qscale;
        }
        __syncthreads();  // the staging space is reused below
    }
    if (tid < QN) {
        Mrun[tid] = -INFINITY;
        Lrun[tid] = 0.0f;
    }
    float acc[QN][COLS];
#pragma unroll
    for (int q = 0; q < QN; ++q)
#pragma unroll
        for (int e = 0; e < COLS; ++e) acc[q][e] = 0.0f;
    __syncthreads();

    const uint16_t* Kh = Kc + (size_t)bh * rows * m;
    const uint16_t* Vh = Vc + (size_t)bh * rows * DV;
    const bool kvec = (m & 7) == 0;
#pragma unroll 1
    for (int kb0 = kbeg; kb0 < kend; kb0 += kDecKeys) {
        // V columns of this thread's keys, requested first so they arrive during the scores
        uint32_t vb[KPG][COLS / 2];
#pragma unroll
        for (int j = 0; j < KPG; ++j) {
            const int key = kb0 + kgi * KPG + j;
            if constexpr (COLS == 8) {
                u32x4 v = {0u, 0u, 0u, 0u};
                if (key < kend) v = *reinterpret_cast<const u32x4*>(Vh + (size_t)key * DV + COLS * ct);
#pragma unroll
                for (int e = 0; e < COLS / 2; ++e) vb[j][e] = v[e];
            } else if constexpr (COLS == 4) {
                u32x2 v = {0u, 0u};
                if (key < kend) v = *reinterpret_cast<const u32x2*>(Vh + (size_t)key * DV + COLS * ct);
                vb[j][0] = v[0];
                vb[j][1] = v[1];
            } else {
                vb[j][0] = key < kend ? *reinterpret_cast<const uint32_t*>(Vh + (size_t)key * DV + COLS * ct) : 0u;
            }
        }
        // scores of key kb0 + tid against every query of the group
        const int key = kb0 + tid;
        float s[QN];
#pragma unroll
        for (int q = 0; q < QN; ++q) s[q] = 0.0f;
        if (key < kend) {
            const uint16_t* kr = Kh + (size_t)key * m;
            if (kvec) {
                for (int c = 0; c < m; c += 8) {
                    const u32x4 raw = *reinterpret_cast<const u32x4*>(kr + c);
                    const f16x8 kv = __builtin_bit_cast(f16x8, raw);
#pragma unroll
                    for (int q = 0; q < QN; ++q) {
                        const float4 a = *reinterpret_cast<const float4*>(&qt[q][c]);
                        const float4 b = *reinterpret_cast<const float4*>(&qt[q][c + 4]);
                        s[q] += a.x * (float)kv[0] + a.y * (float)kv[1] + a.z * (float)kv[2] +
                                a.w * (float)kv[3] + b.x * (float)kv[4] + b.y * (float)kv[5] +
                                b.z * (float)kv[6] + b.w * (float)kv[7];
                    }
                }
            } else {
                for (int c = 0; c < m; ++c) {
                    const float kv = (float)__builtin_bit_cast(_Float16, kr[c]);
#pragma unroll
                    for (int q = 0; q < QN; ++q) s[q] += qt[q][c] * kv;
                }
            }
        }
#pragma unroll
        for (int q = 0; q < QN; ++q) {
            const bool ok = key < kend && q < nq && (!causal || key <= last + q);
            S[q][tid] = ok ? s[q] : -INFINITY;
        }
        __syncthreads();

        // online softmax per query: wave w takes queries w, w + 4, ...
        for (int q = wave; q < QN; q += kDecThreads / 64) {
            float x[kDecKeys / 64];
            float bm = -INFINITY;
#pragma unroll
            for (int i = 0; i < kDecKeys / 64; ++i) {
                x[i] = S[q][lane + 64 * i];
                bm = fmaxf(bm, x[i]);
            }
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) bm = fmaxf(bm, __shfl_xor(bm, o, 64));
            const float mo = Mrun[q];
            const float mn = fmaxf(mo, bm);
            float ps = 0.0f;
#pragma unroll
            for (int i = 0; i < kDecKeys / 64; ++i) {
                const float p = x[i] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(x[i] - mn);
                S[q][lane + 64 * i] = p;
                ps += p;
            }
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) ps += __shfl_xor(ps, o, 64);
            if (lane == 0) {
                const float al = mo == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mo - mn);
                Lrun[q] = Lrun[q] * al + ps;
                Mrun[q] = mn;
                alpha[q] = al;
            }
        }
        __syncthreads();

        // weights x V for this thread's keys and columns
#pragma unroll
        for (int q = 0; q < QN; ++q) {
            const float al = alpha[q];
#pragma unroll
            for (int e = 0; e < COLS; ++e) acc[q][e] *= al;
        }
#pragma unroll
        for (int j = 0; j < KPG; j += 4) {
            float v[4][COLS];
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
#pragma unroll
                for (int e = 0; e < COLS / 2; ++e) {
                    v[jj][2 * e] = __uint_as_float(vb[j + jj][e] << 16);
                    v[jj][2 * e + 1] = __uint_as_float(vb[j + jj][e] & 0xffff0000u);
                }
#pragma unroll
            for (int q = 0; q < QN; ++q) {
                const float4 p4 = *reinterpret_cast<const float4*>(&S[q][kgi * KPG + j]);
#pragma unroll
                for (int e = 0; e < COLS; ++e)
                    acc[q][e] += p4.x * v[0][e] + p4.y * v[1][e] + p4.z * v[2][e] + p4.w * v[3][e];
            }
        }
        __syncthreads();
    }

    // sum the key groups' partial outputs; write this split's partial results
#pragma unroll
    for (int q = 0; q < QN; ++q)
#pragma unroll
        for (int e = 0; e < COLS; ++e) red[kgi][q][COLS * ct + e] = acc[q][e];
    __syncthreads();
    for (int i = tid; i < QN * DV; i += kDecThreads) {
        const int q = i / DV, c = i - q * DV;
        if (q < nq) {
            float o = 0.0f;
#pragma unroll
            for (int g = 0; g < KG; ++g) o += red[g][q][c];
            partO[(((size_t)bh * Nq + q0 + q) * nsplit + sp) * DV + c] = o;
        }
    }
    if (tid < nq) {
        float* ml = partML + (((size_t)bh * Nq + q0 + tid) * nsplit + sp) * 2;
        ml[0] = Mrun[tid];
        ml[1] = Lrun[tid];
    }
}

// One workgroup of DV threads per (head, query): the splits merged in split order. The
// per-split maxima and sums are loaded by all threads at once and their weights staged in
// LDS, so only the DV-wide partial outputs are read in the (unrolled) loop.
constexpr int kCombineMaxSplits = 1024;
template <int DV>
__global__ __launch_bounds__(DV) void decode_combine_kernel(
    const float* __restrict__ partO, const float* __restrict__ partML, void* __restrict__ O,
    int o_f32, float* __restrict__ lse, int nsplit) {
    __shared__ float wsp[kCombineMaxSplits];
    __shared__ float wmax[DV / 64], wsum[DV / 64];
    const size_t row = blockIdx.x;
    const int c = threadIdx.x, wave = c >> 6, lane = c & 63;
    const float* ml = partML + row * nsplit * 2;
    float mx = -INFINITY;
    for (int s = c; s < nsplit; s += DV) mx = fmaxf(mx, ml[2 * s]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
    if (lane == 0) wmax[wave] = mx;
    __syncthreads();
    float M = wmax[0];
#pragma unroll
    for (int w = 1; w < DV / 64; ++w) M = fmaxf(M, wmax[w]);
    float ls = 0.0f;
    for (int s = c; s < nsplit; s += DV) {
        const float ms = ml[2 * s];
        const float w = ms == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(ms - M);
        wsp[s] = w;
        ls += w * ml[2 * s + 1];
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) ls += __shfl_xor(ls, o, 64);
    if (lane == 0) wsum[wave] = ls;
    __syncthreads();
    float L = 0.0f;
#pragma unroll
    for (int w = 0; w < DV / 64; ++w) L += wsum[w];
    const float* po = partO + row * nsplit * DV + c;
    float o = 0.0f;
#pragma unroll 8
    for (int s = 0; s < nsplit; ++s) o += wsp[s] * po[(size_t)s * DV];
    o /= L;
    if (o_f32)
        static_cast<float*>(O)[row * DV + c] = o;
    else
        static_cast<uint16_t*>(O)[row * DV + c] = (uint16_t)(pack_bf16x2(o, 0.0f) & 0xffffu);
    if (lse && c == 0) lse[row] = (M + __log2f(L)) * 0.69314718055994530942f;
}

template <int DV, int QN>
size_t decode_lds_bytes(int d, int m) {
    constexpr int COLS = QN <= 4 ? 8 : QN <= 8 ? 4 : 2;
    constexpr int KG = kDecThreads / (DV / COLS);
    const size_t main = sizeof(float) * ((size_t)QN * kDecKeys + (size_t)KG * QN * DV);
    const size_t stage = sizeof(uint16_t) * ((size_t)d * m + (size_t)QN * d);
    return sizeof(float) * QN * kDecMaxM + (main > stage ? main : stage);
}

template <int DV, int QN>
hipError_t launch_qn(const DecodeArgs& a, hipStream_t s) {
    const int nqg = (a.Nq + QN - 1) / QN;
    const long long grid = (long long)a.BH * nqg * a.nsplit;
    if (grid > 0x7fffffffLL || a.nsplit > kCombineMaxSplits) return hipErrorInvalidConfiguration;
    const size_t lds = decode_lds_bytes<DV, QN>(a.d, a.m);
    decode_attn_kernel<DV, QN><<<dim3((unsigned)grid), kDecThreads, lds, s>>>(
        a.Q, a.Kc, a.Vc, a.P, a.qscale, a.causal, a.H, a.Nq, a.Nk, a.rows, a.d, a.m, nqg,
        a.nsplit, a.chunk, a.partO, a.partML);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    decode_combine_kernel<DV><<<dim3((unsigned)((long long)a.BH * a.Nq)), DV, 0, s>>>(
        a.partO, a.partML, a.O, a.o_f32, a.lse, a.nsplit);
    return hipGetLastError();
}

template <int DV>
hipError_t launch_dv(const DecodeArgs& a, hipStream_t s) {
    if (a.Nq == 1) return launch_qn<DV, 1>(a, s);
    if (a.Nq <= 4) return launch_qn<DV, 4>(a, s);
    if (a.Nq <= 8) return launch_qn<DV, 8>(a, s);
    return launch_qn<DV, 16>(a, s);
}

}  // namespace

DecodeSplit decode_split(int BH, int Nq, int Nk) {
    const int qn = Nq == 1 ? 1 : Nq <= 4 ? 4 : Nq <= 8 ? 8 : 16;
    const long long base = (long long)BH * ((Nq + qn - 1) / qn);
    const int blocks = (Nk + kDecKeys - 1) / kDecKeys;
    // about four workgroups per CU in total, at least two key blocks per split (a split's
    // second block of rows is requested while its first is reduced), one if there is one
    long long want = (1024 + base - 1) / base;
    if (want > blocks) want = blocks;
    if (want < 1) want = 1;
    int per = (int)((blocks + want - 1) / want);
    if (per < 2) per = blocks < 2 ? blocks : 2;
    DecodeSplit r;
    r.chunk = per * kDecKeys;
    r.nsplit = (Nk + r.chunk - 1) / r.chunk;
    return r;
}

hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t stream) {
    if (a.m > kDecMaxM || a.m < 1) return hipErrorInvalidValue;
    switch (a.dv) {
        case 64: return launch_dv<64>(a, stream);
        case 128: return launch_dv<128>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace spa
