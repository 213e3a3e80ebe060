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
// decode_mq_kernel: the same work and outputs for more than four queries per head when m is
//   a multiple of 8, on 16x16x32 MFMAs (scores against the fp16 cache rows, weights times the
//   V rows through transposing LDS reads), 16 queries per workgroup.
// decode_combine_kernel: per query, merges the splits in a fixed order (log-sum-exp).
// Both are HBM-bound: every cache byte is read once per (head, query group).
#include <algorithm>

#include "spa_device.h"
#include "spa_internal.h"

namespace spa {
namespace {

constexpr int kDecThreads = 256;
constexpr int kDecKeys = 256;  // keys per block: one per thread in the score phase
constexpr int kDecMaxM = 128;

// The group's projected queries, qt[q][c] = scale*log2(e) * sum_k Q[q][k] P[k][c] in fp32
// (rows past nq zero): the Q rows and P staged in LDS at `stage` (free space of the caller),
// then 8 threads per output, each summing d/8 products, and a shuffle reduction. Ends with
// a barrier (the staging space may be reused at once).
template <int QN>
__device__ __forceinline__ void project_queries(float (*qt)[kDecMaxM], char* stage,
                                                const uint16_t* __restrict__ Q,
                                                const uint16_t* __restrict__ P, float qscale,
                                                int bh, int h, int Nq, int q0, int nq, int d,
                                                int m, int tid) {
    uint16_t* Ps = reinterpret_cast<uint16_t*>(stage);  // [d][m]
    uint16_t* Qs = Ps + d * m;                            // [QN][d]
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
    __syncthreads();
}

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

    project_queries<QN>(qt, un, Q, P, qscale, bh, h, Nq, q0, nq, d, m, tid);
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

typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef short i16x4 __attribute__((ext_vector_type(4)));

// 16-key x 16-query block products on the 16x16x32 MFMAs. Operand layouts (wave64, lane l,
// j = l % 16, g = l / 16): A (16 x 32) lane l holds A[j][8g .. 8g+7]; B (32 x 16) lane l holds
// B[8g .. 8g+7][j]; D (16 x 16) lane l holds D[4g + r][j] at index r.
__device__ __forceinline__ f32x4 mfma16(f16x8 a, f16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// decode_mq_kernel: the work and the outputs of decode_attn_kernel<DV, 16> (a workgroup per
// head, group of 16 queries and key split) on the matrix cores, for m a multiple of 8 (MK =
// m rounded up to 32, over 32). Each wave streams its own 32-key chunks of the split (chunk
// w, w + 4, ...) with its own exact online softmax, and the four waves' results are merged
// at the end. Per chunk, on fp16/bf16 16x16x32 MFMAs with fp32 accumulation:
//   S^T (16 keys x 16 queries) = Kt rows . qt^T   (per 16-key half, MK k-steps)
//   O^T (DV x 16 queries)     += V^T . P^T       (32 keys as one k-step)
// The score accumulator gives lane (g, j) keys 4g .. 4g+3 of each half for query j, which is
// used directly as the B operand of the value product in that key order (half 0's four keys,
// then half 1's). The V^T operand in the same order comes from the V rows staged in LDS
// row-major, by transposing reads (ds_read_b64_tr_b16: within each 16 lanes, output lane j
// gets element j % 4 of the 8 bytes addressed by lanes 4e + j / 4, e = 0..3). The chunk's Kt
// and V rows are copied HBM -> LDS into a buffer of the wave's own (a second buffer, to copy
// the next chunk during this one, was slower: the larger footprint costs more workgroups per
// CU than the overlap gains); rows at or past the split's end read as zero.
template <int DV, int MK>
__global__ __launch_bounds__(kDecThreads) void decode_mq_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ Kc,
    const uint16_t* __restrict__ Vc, const uint16_t* __restrict__ P, float qscale, int causal,
    int H, int Nq, int Nk, int rows, int d, int m, int nqg, int nsplit, int chunk,
    float* __restrict__ partO, float* __restrict__ partML) {
    constexpr int QN = 16;
    constexpr int CK = 32;                      // keys per wave step
    constexpr int VB = CK * DV * 2;             // V rows of a chunk (bytes)
    constexpr int NVC = VB / 1024;              // their 64-lane x 16-byte copies
    constexpr int DB = DV / 16;
    constexpr int NW = kDecThreads / 64;
    extern __shared__ __attribute__((aligned(16))) char dsm[];
    float(*qt)[kDecMaxM] = reinterpret_cast<float(*)[kDecMaxM]>(dsm);
    char* un = dsm + QN * kDecMaxM * sizeof(float);

    const int sp = blockIdx.x % nsplit;
    const int rest = blockIdx.x / nsplit;
    const int qg = rest % nqg;
    const int bh = rest / nqg;
    const int h = bh % H;
    const int q0 = qg * QN;
    const int nq = min(QN, Nq - q0);
    const int kbeg = sp * chunk;
    const int kend = min(Nk, kbeg + chunk);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, j = lane & 15, g = lane >> 4;
    const int last = Nk - Nq + q0;  // absolute position of query q0 (causal limit)

    project_queries<QN>(qt, un, Q, P, qscale, bh, h, Nq, q0, nq, d, m, tid);
    // B operands of the scores: features 32 kk + 8g .. +7 of query j (fp16, zero past m)
    f16x8 qb[MK];
#pragma unroll
    for (int kk = 0; kk < MK; ++kk)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int c = 32 * kk + 8 * g + e;
            qb[kk][e] = (_Float16)(c < m ? qt[j][c] : 0.0f);
        }
    __syncthreads();  // qt and the staging space are reused below

    // this wave's two buffers: [Kt rows of a chunk (KB bytes)][V rows (VB bytes)], from the
    // start of the shared space (the projected queries are in registers now)
    // Kt rows of a chunk: CK * m * 2 <= 2048 * MK bytes in 2 * MK copies; copies past the
    // chunk's last kilobyte repeat it (same bytes to the same place), so every wave issues
    // the same number of copies per chunk and the waits below are constants
    constexpr int NKC = 2 * MK;
    constexpr int KB = 1024 * NKC;
    const int nkc = (CK * m * 2 + 1023) / 1024;
    const uint32_t wbuf = lds_address(dsm) + (uint32_t)(wave * (KB + VB));
    const char* wbuf_p = dsm + wave * (KB + VB);
    const uint16_t* Kh = Kc + (size_t)bh * rows * m;
    const uint16_t* Vh = Vc + (size_t)bh * rows * DV;
    const u32x4 kr = make_rsrc(Kh, (uint32_t)kend * (uint32_t)m * 2u);
    const u32x4 vr = make_rsrc(Vh, (uint32_t)kend * (uint32_t)DV * 2u);
    auto copy_chunk = [&](int key0, int b) {
        const uint32_t base = wbuf + (uint32_t)(b * (KB + VB));
#pragma unroll
        for (int i = 0; i < NKC; ++i) {
            const int c = min(i, nkc - 1);
            copy16_to_lds(kr, base + 1024 * c, (uint32_t)key0 * m * 2 + 1024 * c + 16 * lane);
        }
#pragma unroll
        for (int i = 0; i < NVC; ++i) {
            const int c = 64 * i + lane;
            copy16_to_lds(vr, base + KB + 1024 * i,
                          (uint32_t)(key0 + c / (DV / 8)) * DV * 2 + 16 * (c % (DV / 8)));
        }
    };

    float mrun = -INFINITY, lrun = 0.0f;  // query j, this wave's keys
    f32x4 acc[DB];
#pragma unroll
    for (int b = 0; b < DB; ++b) acc[b] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    const int first = kbeg + CK * wave;
    const int nck = first < kend ? (kend - first + NW * CK - 1) / (NW * CK) : 0;
#pragma unroll 1
    for (int i = 0; i < nck; ++i) {
        const int key0 = first + NW * CK * i;
        // the buffer was last read a step ago, by reads the MFMAs have consumed
        __builtin_amdgcn_s_waitcnt(0);
        asm volatile("" ::: "memory");
        copy_chunk(key0, 0);
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        asm volatile("" ::: "memory");
        typedef __attribute__((address_space(3))) const char lds_char;
        lds_char* kb = (lds_char*)wbuf_p;
        lds_char* vb = kb + KB;

        // scores (base 2) of keys key0 + 16 hf + 4g + r, query j
        f32x4 s[2];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            s[hf] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int kk = 0; kk < MK; ++kk) {
                u32x4 a = {0u, 0u, 0u, 0u};
                if (32 * kk + 8 * g < m)
                    a = *(const __attribute__((address_space(3))) u32x4*)(kb + (16 * hf + j) * m * 2 + (32 * kk + 8 * g) * 2);
                s[hf] = mfma16(__builtin_bit_cast(f16x8, a), qb[kk], s[hf]);
            }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int key = key0 + 16 * hf + 4 * g + r;
                if (key >= kend || j >= nq || (causal && key > last + j)) s[hf][r] = -INFINITY;
                mx = fmaxf(mx, s[hf][r]);
            }
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const float mn = fmaxf(mrun, mx);
        // weights (bf16, as the value product consumes them) and their sum
        bf16x8 pw;
        float ps = 0.0f;
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float x = s[hf][r];
                const float p = x == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(x - mn);
                const bf16_t pb = (bf16_t)p;
                pw[4 * hf + r] = pb;
                ps += (float)pb;
            }
        ps += __shfl_xor(ps, 16, 64);
        ps += __shfl_xor(ps, 32, 64);
        const float al = mrun == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mrun - mn);
        lrun = lrun * al + ps;
        mrun = mn;
#pragma unroll
        for (int b = 0; b < DB; ++b) acc[b] *= al;
        // V^T operand of dv block b: lane (g, 4e + q) addresses row 16 hf + 4g + e, columns
        // 16b + 4q .. +3 of the staged V rows; hf = 0 gives the operand's first four keys
#pragma unroll
        for (int b = 0; b < DB; ++b) {
            const int e = j >> 2, q = j & 3;
            typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
            const i16x4 t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_i16x4*)(vb + ((4 * g + e) * DV + 16 * b + 4 * q) * 2));
            const i16x4 t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_i16x4*)(vb + ((16 + 4 * g + e) * DV + 16 * b + 4 * q) * 2));
            // whole registers reinterpreted (inserting the 16-bit elements one by one has
            // been compiled into a wrong permute)
            const u32x2 w0 = __builtin_bit_cast(u32x2, t0), w1 = __builtin_bit_cast(u32x2, t1);
            const bf16x8 va = __builtin_bit_cast(bf16x8, u32x4{w0.x, w0.y, w1.x, w1.y});
            acc[b] = mfma16(va, pw, acc[b]);
        }
    }

    // merge the four waves: M = max, L = sum of l 2^(m - M), O = sum of O 2^(m - M)
    __syncthreads();  // every wave is done with its buffers
    float* wm = reinterpret_cast<float*>(dsm);      // [NW][QN]
    float* wl = wm + NW * QN;                        // [NW][QN]
    float* wo = wl + NW * QN;                        // [NW][QN][DV]
    if (g == 0) {
        wm[wave * QN + j] = mrun;
        wl[wave * QN + j] = lrun;
    }
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r) wo[(wave * QN + j) * DV + 16 * b + 4 * g + r] = acc[b][r];
    __syncthreads();
    for (int i = tid; i < QN * DV; i += kDecThreads) {
        const int q = i / DV, c = i - q * DV;
        if (q < nq) {
            float M = -INFINITY;
#pragma unroll
            for (int w = 0; w < NW; ++w) M = fmaxf(M, wm[w * QN + q]);
            float o = 0.0f;
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                const float mw = wm[w * QN + q];
                const float f = mw == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mw - M);
                o += f * wo[(w * QN + q) * DV + c];
            }
            partO[(((size_t)bh * Nq + q0 + q) * nsplit + sp) * DV + c] = o;
        }
    }
    if (tid < nq) {
        float M = -INFINITY, L = 0.0f;
#pragma unroll
        for (int w = 0; w < NW; ++w) M = fmaxf(M, wm[w * QN + tid]);
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const float mw = wm[w * QN + tid];
            L += mw == -INFINITY ? 0.0f : wl[w * QN + tid] * __builtin_amdgcn_exp2f(mw - M);
        }
        float* ml = partML + (((size_t)bh * Nq + q0 + tid) * nsplit + sp) * 2;
        ml[0] = M;
        ml[1] = L;
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

// Shared bytes of decode_mq_kernel: the projection's (queries and staging), the four waves'
// buffers, or the final merge, whichever is largest (64 KiB at most: d = m = dv = 128).
template <int DV>
size_t decode_mq_lds_bytes(int d, int m) {
    const size_t proj = sizeof(float) * 16 * kDecMaxM + sizeof(uint16_t) * ((size_t)d * m + 16 * (size_t)d);
    const size_t kb = 2048 * (size_t)((m + 31) / 32);
    const size_t bufs = 4 * (kb + (size_t)32 * DV * 2);
    const size_t merge = sizeof(float) * (2 * 4 * 16 + 4 * 16 * (size_t)DV);
    return std::max(proj, std::max(bufs, merge));
}

template <int DV, int MK>
hipError_t launch_mq(const DecodeArgs& a, hipStream_t s) {
    const int nqg = (a.Nq + 15) / 16;
    const long long grid = (long long)a.BH * nqg * a.nsplit;
    if (grid > 0x7fffffffLL || a.nsplit > kCombineMaxSplits) return hipErrorInvalidConfiguration;
    const size_t lds = decode_mq_lds_bytes<DV>(a.d, a.m);
    if (lds > 64 * 1024) return hipErrorInvalidConfiguration;  // at most 64 KiB for d, m <= 128
    decode_mq_kernel<DV, MK><<<dim3((unsigned)grid), kDecThreads, lds, s>>>(
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
    // more than four queries per head and m a multiple of 8: the matrix-core kernel
    if (a.Nq > 4 && a.m % 8 == 0) {
        switch ((a.m + 31) / 32) {
            case 1: return launch_mq<DV, 1>(a, s);
            case 2: return launch_mq<DV, 2>(a, s);
            case 3: return launch_mq<DV, 3>(a, s);
            default: return launch_mq<DV, 4>(a, s);
        }
    }
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
    // about four workgroups per CU in total (two for more than four queries per head, whose
    // matrix-core kernel does more per workgroup), at least two key blocks per split (a
    // split's second block of rows is requested while its first is reduced), one if there
    // is one
    const long long target = Nq > 4 ? 512 : 1024;
    long long want = (target + base - 1) / base;
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
