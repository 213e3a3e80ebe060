// spa_bwd.hip -- backward of the projected attention for bf16 inputs on gfx950 MFMA.
//
// What it computes: the chain rule of the forward ("Sparse Projection Attention" page,
// Sec. 3.1.3 and Algorithm 1; Sec. 3.2 and Algorithm 2 train the projection by
// backpropagation, with the query term of the projection's gradient written out; the key
// term enters the same way). With A the row softmax of the forward, O = A V, dO = dL/dO:
//   D_i = <dO_i, O_i>,  dA_ij = <dO_i, V_j>,  dS_ij = A_ij (dA_ij - D_i)
//   dV_j = sum_i A_ij dO_i,  dQt_i = scale sum_j dS_ij Kt_j,  dKt_j = scale sum_i dS_ij Qt_i
//   dQ = dQt P^T,  dK = dKt P^T,  dP_h = sum over batches and rows of Q^T dQt + K^T dKt.
// The weights A are recomputed from the forward's log-sum-exp: the projected queries and keys
// are prepared exactly as in the forward (fp16, queries pre-scaled by scale*log2(e)), so the
// recomputed base-2 scores are the forward's, bit for bit.
//
// Kernels (all on 32x32x16 MFMA; see the forward for the operand layouts):
//   bwd_q_kernel   query-major: per 32-query wave, a loop over 32-key tiles computes
//                  dQt^T = Kt^T . dS^T, after D_i from the wave's own dO and O rows.
//   bwd_kv_kernel  key-major: per 32-key wave, a loop over 32-query tiles computes
//                  dV^T = dO^T . A and dKt^T = Qt^T . dS. Needs D from bwd_q_kernel.
//   proj_back_kernel   dQ = dQt P^T and dK = dKt P^T.
//   dp_partial_kernel / dp_reduce_kernel   the projection gradient, per 256-row chunk and
//                  then summed over chunks and batches in a fixed order (deterministic).
// In the transposed (A-operand) tiles the rows are V^T-ordered: within every 16 tokens the
// order 0-3, 8-11, 4-7, 12-15, which is the order in which a score accumulator lane holds
// its 8 tokens of a 16-token k-step. So every MFMA operand is one 16-byte LDS read or a
// register, as in the forward.
#include "spa_device.h"
#include "spa_internal.h"

namespace spa {
namespace {

constexpr int kThreads = 256;
constexpr int kTile = 32;  // keys (query-major kernel) or queries (key-major kernel) per step
constexpr float kLog2e = 1.44269504088896340736f;

// Linear workgroup index with the grid split into 8 contiguous ranges, range x on XCD x
// (the dispatcher hands workgroups to the XCDs round-robin); identity unless 8 divides it.
__device__ __forceinline__ int xcd_local_index() {
    const int total = gridDim.x;
    return (total & 7) == 0 ? (blockIdx.x & 7) * (total >> 3) + (blockIdx.x >> 3) : blockIdx.x;
}

// Tag for compile-time variants of a loop step.
template <bool B>
struct Flag {
    static constexpr bool value = B;
};

// Byte offset that is out of range for every tile resource below (loads read zero).
constexpr uint32_t kOutOfRange = 0x80000000u;

// Raw buffer resource over max(bytes, 0) bytes from `base`: loads at offsets past the end
// return zero instead of touching memory. base and bytes must be wave-uniform.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const void* base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, max(bytes, 0),
                                             0x00020000);
}

// fp32 score-layout values (slots 8*half + j of k-step tt) -> packed pairs
template <bool F16>
__device__ __forceinline__ u32x4 pack_kstep(const f32x16& x, int tt) {
    u32x4 w;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float lo = x[8 * tt + 2 * j], hi = x[8 * tt + 2 * j + 1];
        w[j] = F16 ? pack_f16x2(lo, hi) : pack_bf16x2(lo, hi);
    }
    return w;
}

// ---------------------------------------------------------------------------------------
// Query-major kernel: dQt and D.
// Inputs: Qs [BH,N,MP] fp16 (scaled), Kt [BH,N,MP] fp16, Ktt [BH,MP,Np] fp16 (transposed,
// permuted), V [BH,N,DV] bf16, O, dO [BH,N,DV] bf16, lse [BH,N] (natural log).
// Outputs: dQt [BH,N,MP] fp32 (scaled by `scale`), D [BH,N] fp32.
template <int MP, int DV, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void bwd_q_kernel(
    const uint16_t* __restrict__ Qs, const uint16_t* __restrict__ Kt,
    const uint16_t* __restrict__ Ktt, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ O, const uint16_t* __restrict__ dO,
    const float* __restrict__ lse, float* __restrict__ dQt, float* __restrict__ Dout, int N,
    int Np, int nqb, float scale) {
    constexpr int KS = MP / 16;                // score k-steps
    constexpr int MB = (MP + 31) / 32;         // 32-row blocks of dQt^T
    constexpr int CS = DV / 16;                // dA k-steps
    // LDS tiles, rows padded by 16 bytes so that 16-byte reads of one chunk column across
    // consecutive rows hit distinct banks.
    constexpr int KP = MP * 2 + 16;            // Kt tile row pitch (bytes)
    constexpr int TP = kTile * 2 + 16;         // transposed tile row pitch: 32 tokens
    constexpr int VP = DV * 2 + 16;            // V tile row pitch
    constexpr int K_B = kTile * KP;
    constexpr int KT_B = MB * 32 * TP;         // rows past MP zero
    constexpr int V_B = kTile * VP;
    constexpr int BUF = K_B + KT_B + V_B;
    // 16-byte chunks per region (each a multiple of 64, so one wave's slot is in one region)
    constexpr int NK = kTile * MP / 8, NKT = MB * 32 * 4, NV = kTile * DV / 8;
    constexpr int NCH = NK + NKT + NV;
    constexpr int CPT = (NCH + kThreads - 1) / kThreads;
    static_assert(NK % 64 == 0 && NKT % 64 == 0 && NV % 64 == 0, "region sizes");
    __shared__ __attribute__((aligned(16))) char lds[2 * BUF];

    // Workgroup -> (head, query block) as in the forward: XCD x (workgroups are handed to
    // the 8 XCDs round-robin) gets a contiguous range of pairs, so a head's key tiles stay
    // in one XCD's L2; causal blocks run heaviest (last) first.
    const int li = xcd_local_index();
    const int bh = li / nqb;
    const int qbi = li - bh * nqb;
    const int qb = CAUSAL ? nqb - 1 - qbi : qbi;
    const int q0 = qb * 128;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, col = lane & 31, half = lane >> 5;
    const int myq = q0 + wave * 32 + col;
    const bool qvalid = myq < N;

    const uint16_t* Qh = Qs + (size_t)bh * N * MP;
    const char* Kh = reinterpret_cast<const char*>(Kt + (size_t)bh * N * MP);
    const char* Kth = reinterpret_cast<const char*>(Ktt + (size_t)bh * MP * Np);
    const char* Vh = reinterpret_cast<const char*>(V + (size_t)bh * N * DV);

    // This lane's query (B operand of the scores) and dO row (B operand of dA).
    f16x8 qf[KS];
    bf16x8 dof[CS];
    float dpart = 0.0f;  // this lane's half of <dO_q, O_q>
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        u32x4 v = {0u, 0u, 0u, 0u};
        if (qvalid) v = *reinterpret_cast<const u32x4*>(Qh + (size_t)myq * MP + ks * 16 + half * 8);
        qf[ks] = __builtin_bit_cast(f16x8, v);
    }
#pragma unroll
    for (int cs = 0; cs < CS; ++cs) {
        u32x4 v = {0u, 0u, 0u, 0u}, o = {0u, 0u, 0u, 0u};
        if (qvalid) {
            const size_t off = ((size_t)bh * N + myq) * DV + cs * 16 + half * 8;
            v = *reinterpret_cast<const u32x4*>(dO + off);
            o = *reinterpret_cast<const u32x4*>(O + off);
        }
        dof[cs] = __builtin_bit_cast(bf16x8, v);
        const bf16x8 ob = __builtin_bit_cast(bf16x8, o);
#pragma unroll
        for (int i = 0; i < 8; ++i) dpart += (float)dof[cs][i] * (float)ob[i];
    }
    const float Dq = halves_sum(dpart);
    const float lse2 = qvalid ? lse[(size_t)bh * N + myq] * kLog2e : INFINITY;

    const int kend = CAUSAL ? min(N, q0 + 128) : N;
    const int ntiles = (kend + kTile - 1) / kTile;
    // Tiles before `nfree` need no mask: causal, all their keys precede the block's first
    // query; otherwise every tile but a ragged last one.
    const int nfree = CAUSAL ? min(ntiles, q0 / kTile) : N / kTile;

    // Staging slots: chunk i * kThreads + tid -> region (wave-uniform), byte offset from the
    // tile's first token, LDS byte offset. Per region, the head's array, its bytes per token
    // step and its size in bytes. Region 0: Kt rows; 1: Kt^T feature rows (rows past MP read
    // zero); 2: V rows; none (slots past the tile).
    const int wu = __builtin_amdgcn_readfirstlane(wave);
    const char* sbase[CPT];
    int sstep[CPT], stot[CPT];
    bool slive[CPT];
    uint32_t voff[CPT], loff[CPT];
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
        const int cw = i * kThreads + wu * 64;
        const int c = cw + lane;
        slive[i] = cw < NCH;
        if (cw < NK) {
            const int row = c / (MP / 8), cc = c % (MP / 8);
            sbase[i] = Kh, sstep[i] = MP * 2, stot[i] = N * MP * 2;
            voff[i] = row * MP * 2 + cc * 16, loff[i] = row * KP + cc * 16;
        } else if (cw < NK + NKT) {
            const int row = (c - NK) / 4, cc = (c - NK) % 4;
            sbase[i] = Kth, sstep[i] = 2, stot[i] = MP * Np * 2;
            voff[i] = row < MP ? row * Np * 2 + cc * 16 : kOutOfRange;
            loff[i] = K_B + row * TP + cc * 16;
        } else {
            const int row = (c - NK - NKT) / (DV / 8), cc = (c - NK - NKT) % (DV / 8);
            sbase[i] = Vh, sstep[i] = DV * 2, stot[i] = slive[i] ? N * DV * 2 : 0;
            voff[i] = row * DV * 2 + cc * 16, loff[i] = K_B + KT_B + row * VP + cc * 16;
        }
    }
    u32x4 stage[CPT];
    auto load_tile = [&](int k0) {
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int skip = k0 * sstep[i];
            stage[i] = __builtin_amdgcn_raw_buffer_load_b128(
                tile_rsrc(sbase[i] + skip, stot[i] - skip), voff[i], 0, 0);
        }
    };
    auto store_tile = [&](int buf) {
#pragma unroll
        for (int i = 0; i < CPT; ++i)
            if ((i + 1) * kThreads <= NCH || slive[i])
                *reinterpret_cast<u32x4*>(lds + buf * BUF + loff[i]) = stage[i];
    };

    f32x16 acc[MB];
#pragma unroll
    for (int b = 0; b < MB; ++b) acc[b] = f32x16_fill(0.0f);

    // One barrier per step: step t stores tile t+1 (loaded during step t-1) into the buffer
    // step t-1 read, requests tile t+2 (past the end: all reads out of range, zero), then
    // computes tile t.
    auto step = [&](int t, auto mask_tag) {
        constexpr bool MASK = decltype(mask_tag)::value;
        const int k0 = t * kTile;
        store_tile((t + 1) & 1);
        load_tile(k0 + 2 * kTile);
        const char* Ks = lds + (t & 1) * BUF;
        const char* Kts = Ks + K_B;
        const char* Vs = Kts + KT_B;
        // causal: a wave whose queries all precede the tile has nothing to do in it
        if (!(MASK && CAUSAL) || k0 <= q0 + wave * 32 + 31) {
            // scores^T (32 keys x 32 queries), base-2 units
            f32x16 s = f32x16_fill(0.0f);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const f16x8 a = __builtin_bit_cast(
                    f16x8, *reinterpret_cast<const u32x4*>(Ks + col * KP + (ks * 16 + half * 8) * 2));
                s = mfma32x32x16(a, qf[ks], s);
            }
            // dA^T (32 keys x 32 queries) = V . dO^T
            f32x16 da = f32x16_fill(0.0f);
#pragma unroll
            for (int cs = 0; cs < CS; ++cs) {
                const bf16x8 a = __builtin_bit_cast(
                    bf16x8, *reinterpret_cast<const u32x4*>(Vs + col * VP + (cs * 16 + half * 8) * 2));
                da = mfma32x32x16(a, dof[cs], da);
            }
            // dS = A (dA - D), masked entries (later keys, keys past N) zero
            f32x16 ds;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float w = __builtin_amdgcn_exp2f(s[i] - lse2);
                if (MASK) {
                    const int key = k0 + 8 * (i >> 2) + 4 * half + (i & 3);
                    if ((CAUSAL && key > myq) || key >= N) w = 0.0f;
                }
                ds[i] = w * (da[i] - Dq);
            }
            // dQt^T (MP x 32 queries) += Kt^T . dS^T
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                const f16x8 b = __builtin_bit_cast(f16x8, pack_kstep<true>(ds, tt));
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) {
                    const f16x8 a = __builtin_bit_cast(
                        f16x8, *reinterpret_cast<const u32x4*>(Kts + (mb * 32 + col) * TP + (tt * 16 + half * 8) * 2));
                    acc[mb] = mfma32x32x16(a, b, acc[mb]);
                }
            }
        }
        __syncthreads();
    };

    load_tile(0);
    store_tile(0);
    load_tile(kTile);
    __syncthreads();
    int t = 0;
#pragma unroll 1
    for (; t < nfree; ++t) step(t, Flag<false>{});
#pragma unroll 1
    for (; t < ntiles; ++t) step(t, Flag<true>{});

    if (qvalid) {
        float* dst = dQt + ((size_t)bh * N + myq) * MP;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int c0 = mb * 32 + 8 * g + 4 * half;
                if (c0 < MP)
                    *reinterpret_cast<float4*>(dst + c0) =
                        make_float4(acc[mb][4 * g] * scale, acc[mb][4 * g + 1] * scale,
                                    acc[mb][4 * g + 2] * scale, acc[mb][4 * g + 3] * scale);
            }
        if (half == 0) Dout[(size_t)bh * N + myq] = Dq;
    }
}

// ---------------------------------------------------------------------------------------
// Key-major kernel: dV and dKt.
// Inputs: Qs [BH,N,MP] fp16 (scaled), Qst [BH,MP,Np] fp16 (transposed, permuted), Kt
// [BH,N,MP] fp16, V [BH,N,DV] bf16, dO [BH,N,DV] bf16, dOt [BH,DV,Np] bf16 (transposed,
// permuted), lse [BH,N], D [BH,N].
// Outputs: dV [BH,N,DV] (fp32 or bf16), dKt [BH,N,MP] fp32 (scale applied).
template <int MP, int DV, bool CAUSAL>
__global__ __launch_bounds__(kThreads, (MP >= 64 && DV >= 128) ? 1 : 2) void bwd_kv_kernel(
    const uint16_t* __restrict__ Qs, const uint16_t* __restrict__ Qst,
    const uint16_t* __restrict__ Kt, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const uint16_t* __restrict__ dOt,
    const float* __restrict__ lse, const float* __restrict__ Din, void* __restrict__ dV,
    int dv_f32, float* __restrict__ dKt, int N, int Np, int nkb) {
    constexpr int KS = MP / 16;
    constexpr int MB = (MP + 31) / 32;
    constexpr int CS = DV / 16;
    constexpr int DB = DV / 32;
    // LDS tiles, rows padded by 16 bytes (see the query-major kernel).
    constexpr int QP = MP * 2 + 16;            // Qs tile row pitch
    constexpr int TP = kTile * 2 + 16;         // transposed tiles' row pitch: 32 tokens
    constexpr int OP = DV * 2 + 16;            // dO tile row pitch
    constexpr int Q_B = kTile * QP;
    constexpr int QT_B = MB * 32 * TP;         // rows past MP zero
    constexpr int DO_B = kTile * OP;
    constexpr int DOT_B = DV * TP;
    constexpr int L_B = kTile * 4;             // lse2 (then D) of the tile
    constexpr int BUF = Q_B + QT_B + DO_B + DOT_B + 2 * L_B;
    constexpr int NQ = kTile * MP / 8, NQT = MB * 32 * 4, NO = kTile * DV / 8, NOT = DV * 4;
    constexpr int NCH = NQ + NQT + NO + NOT;
    constexpr int CPT = (NCH + kThreads - 1) / kThreads;
    static_assert(NQ % 64 == 0 && NQT % 64 == 0 && NO % 64 == 0 && NOT % 64 == 0, "region sizes");
    __shared__ __attribute__((aligned(16))) char lds[2 * BUF];

    // Workgroup -> (head, key block), XCD-contiguous as in the query-major kernel; causal
    // key blocks are heaviest first already (block 0 meets every query).
    const int li = xcd_local_index();
    const int bh = li / nkb;
    const int kb = li - bh * nkb;
    const int k0 = kb * 128;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, col = lane & 31, half = lane >> 5;
    const int k0w = k0 + wave * 32;
    const int myk = k0w + col;
    const bool kvalid = myk < N;

    const char* Qh = reinterpret_cast<const char*>(Qs + (size_t)bh * N * MP);
    const char* Qth = reinterpret_cast<const char*>(Qst + (size_t)bh * MP * Np);
    const char* dOh = reinterpret_cast<const char*>(dO + (size_t)bh * N * DV);
    const char* dOth = reinterpret_cast<const char*>(dOt + (size_t)bh * DV * Np);
    const float* lseh = lse + (size_t)bh * N;
    const float* Dh = Din + (size_t)bh * N;

    // This lane's key (B operand of the scores) and value row (B operand of dA).
    f16x8 kf[KS];
    bf16x8 vf[CS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        u32x4 v = {0u, 0u, 0u, 0u};
        if (kvalid) v = *reinterpret_cast<const u32x4*>(Kt + ((size_t)bh * N + myk) * MP + ks * 16 + half * 8);
        kf[ks] = __builtin_bit_cast(f16x8, v);
    }
#pragma unroll
    for (int cs = 0; cs < CS; ++cs) {
        u32x4 v = {0u, 0u, 0u, 0u};
        if (kvalid) v = *reinterpret_cast<const u32x4*>(V + ((size_t)bh * N + myk) * DV + cs * 16 + half * 8);
        vf[cs] = __builtin_bit_cast(bf16x8, v);
    }

    const int qstart = CAUSAL ? k0 : 0;
    const int ntiles = (N - qstart + kTile - 1) / kTile;
    // causal: the first four tiles meet the block's keys and need the mask
    const int nmask = CAUSAL ? min(ntiles, 128 / kTile) : 0;

    // Staging slots as in the query-major kernel. Region 0: Qs rows; 1: Qs^T feature rows
    // (rows past MP read zero); 2: dO rows; 3: dO^T rows; none (slots past the tile).
    const int wu = __builtin_amdgcn_readfirstlane(wave);
    const char* sbase[CPT];
    int sstep[CPT], stot[CPT];
    bool slive[CPT];
    uint32_t voff[CPT], loff[CPT];
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
        const int cw = i * kThreads + wu * 64;
        const int c = cw + lane;
        slive[i] = cw < NCH;
        if (cw < NQ) {
            const int row = c / (MP / 8), cc = c % (MP / 8);
            sbase[i] = Qh, sstep[i] = MP * 2, stot[i] = N * MP * 2;
            voff[i] = row * MP * 2 + cc * 16, loff[i] = row * QP + cc * 16;
        } else if (cw < NQ + NQT) {
            const int row = (c - NQ) / 4, cc = (c - NQ) % 4;
            sbase[i] = Qth, sstep[i] = 2, stot[i] = MP * Np * 2;
            voff[i] = row < MP ? row * Np * 2 + cc * 16 : kOutOfRange;
            loff[i] = Q_B + row * TP + cc * 16;
        } else if (cw < NQ + NQT + NO) {
            const int row = (c - NQ - NQT) / (DV / 8), cc = (c - NQ - NQT) % (DV / 8);
            sbase[i] = dOh, sstep[i] = DV * 2, stot[i] = N * DV * 2;
            voff[i] = row * DV * 2 + cc * 16, loff[i] = Q_B + QT_B + row * OP + cc * 16;
        } else {
            const int row = (c - NQ - NQT - NO) / 4, cc = (c - NQ - NQT - NO) % 4;
            sbase[i] = dOth, sstep[i] = 2, stot[i] = slive[i] ? DV * Np * 2 : 0;
            voff[i] = row * Np * 2 + cc * 16;
            loff[i] = Q_B + QT_B + DO_B + row * TP + cc * 16;
        }
    }
    u32x4 stage[CPT];
    float lstage, dstage;
    const int ql = tid & (kTile - 1);  // every thread stages the lse and D of query ql
    auto load_tile = [&](int q0) {
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int skip = q0 * sstep[i];
            stage[i] = __builtin_amdgcn_raw_buffer_load_b128(
                tile_rsrc(sbase[i] + skip, stot[i] - skip), voff[i], 0, 0);
        }
        const int nl = (N - q0) * 4;
        const float l = __uint_as_float(
            __builtin_amdgcn_raw_buffer_load_b32(tile_rsrc(lseh + q0, nl), ql * 4, 0, 0));
        dstage = __uint_as_float(
            __builtin_amdgcn_raw_buffer_load_b32(tile_rsrc(Dh + q0, nl), ql * 4, 0, 0));
        lstage = q0 + ql < N ? l * kLog2e : INFINITY;  // rows past N get zero weight
    };
    auto store_tile = [&](int buf) {
        char* base = lds + buf * BUF;
#pragma unroll
        for (int i = 0; i < CPT; ++i)
            if ((i + 1) * kThreads <= NCH || slive[i])
                *reinterpret_cast<u32x4*>(base + loff[i]) = stage[i];
        // identical values from the threads that share ql
        reinterpret_cast<float*>(base + BUF - 2 * L_B)[ql] = lstage;
        reinterpret_cast<float*>(base + BUF - L_B)[ql] = dstage;
    };

    f32x16 dva[DB], dka[MB];
#pragma unroll
    for (int b = 0; b < DB; ++b) dva[b] = f32x16_fill(0.0f);
#pragma unroll
    for (int b = 0; b < MB; ++b) dka[b] = f32x16_fill(0.0f);

    // One barrier per step, as in the query-major kernel.
    auto step = [&](int t, auto mask_tag) {
        constexpr bool MASK = decltype(mask_tag)::value;
        const int q0 = qstart + t * kTile;
        store_tile((t + 1) & 1);
        load_tile(q0 + 2 * kTile);
        const char* Qts = lds + (t & 1) * BUF;  // Qs tile (rows = queries)
        const char* QTs = Qts + Q_B;            // Qs^T tile (rows = features)
        const char* dOs = QTs + QT_B;           // dO tile (rows = queries)
        const char* dOTs = dOs + DO_B;          // dO^T tile (rows = V columns)
        const float* L2s = reinterpret_cast<const float*>(Qts + BUF - 2 * L_B);
        const float* Ds = reinterpret_cast<const float*>(Qts + BUF - L_B);
        // causal: nothing to do if every query of the tile precedes every key of the wave
        if (!MASK || q0 + kTile - 1 >= k0w) {
            // scores^T (32 queries x 32 keys)
            f32x16 s = f32x16_fill(0.0f);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const f16x8 a = __builtin_bit_cast(
                    f16x8, *reinterpret_cast<const u32x4*>(Qts + col * QP + (ks * 16 + half * 8) * 2));
                s = mfma32x32x16(a, kf[ks], s);
            }
            // dA^T (32 queries x 32 keys) = dO . V^T
            f32x16 da = f32x16_fill(0.0f);
#pragma unroll
            for (int cs = 0; cs < CS; ++cs) {
                const bf16x8 a = __builtin_bit_cast(
                    bf16x8, *reinterpret_cast<const u32x4*>(dOs + col * OP + (cs * 16 + half * 8) * 2));
                da = mfma32x32x16(a, vf[cs], da);
            }
            // weights and dS; the row (query) of slot i is 8*(i/4) + 4*half + i%4
            f32x16 w, ds;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const float4 l4 = *reinterpret_cast<const float4*>(L2s + 8 * g + 4 * half);
                const float4 d4 = *reinterpret_cast<const float4*>(Ds + 8 * g + 4 * half);
                const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
                const float dv4[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = 4 * g + r;
                    float a = __builtin_amdgcn_exp2f(s[i] - lv[r]);
                    if (MASK && myk > q0 + 8 * g + 4 * half + r) a = 0.0f;
                    w[i] = a;
                    ds[i] = a * (da[i] - dv4[r]);
                }
            }
            // dV^T (DV x 32 keys) += dO^T . A ; dKt^T (MP x 32 keys) += Qs^T . dS
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                const bf16x8 bw = __builtin_bit_cast(bf16x8, pack_kstep<false>(w, tt));
                const f16x8 bs = __builtin_bit_cast(f16x8, pack_kstep<true>(ds, tt));
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    const bf16x8 a = __builtin_bit_cast(
                        bf16x8, *reinterpret_cast<const u32x4*>(dOTs + (db * 32 + col) * TP + (tt * 16 + half * 8) * 2));
                    dva[db] = mfma32x32x16(a, bw, dva[db]);
                }
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) {
                    const f16x8 a = __builtin_bit_cast(
                        f16x8, *reinterpret_cast<const u32x4*>(QTs + (mb * 32 + col) * TP + (tt * 16 + half * 8) * 2));
                    dka[mb] = mfma32x32x16(a, bs, dka[mb]);
                }
            }
        }
        __syncthreads();
    };

    load_tile(qstart);
    store_tile(0);
    load_tile(qstart + kTile);
    __syncthreads();
    int t = 0;
#pragma unroll 1
    for (; t < nmask; ++t) step(t, Flag<true>{});
#pragma unroll 1
    for (; t < ntiles; ++t) step(t, Flag<false>{});

    if (kvalid) {
        const size_t row = (size_t)bh * N + myk;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int c0 = db * 32 + 8 * g + 4 * half;
                const float x0 = dva[db][4 * g], x1 = dva[db][4 * g + 1];
                const float x2 = dva[db][4 * g + 2], x3 = dva[db][4 * g + 3];
                if (dv_f32) {
                    *reinterpret_cast<float4*>(static_cast<float*>(dV) + row * DV + c0) = make_float4(x0, x1, x2, x3);
                } else {
                    u32x2 p;
                    p.x = pack_bf16x2(x0, x1);
                    p.y = pack_bf16x2(x2, x3);
                    *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(dV) + row * DV + c0) = p;
                }
            }
        // dKt = scale * sum dS Qt = sum dS Qs / log2(e)
        float* dst = dKt + row * MP;
        constexpr float inv = 1.0f / kLog2e;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int c0 = mb * 32 + 8 * g + 4 * half;
                if (c0 < MP)
                    *reinterpret_cast<float4*>(dst + c0) =
                        make_float4(dka[mb][4 * g] * inv, dka[mb][4 * g + 1] * inv,
                                    dka[mb][4 * g + 2] * inv, dka[mb][4 * g + 3] * inv);
            }
    }
}

// ---------------------------------------------------------------------------------------
// dX[bh, n, k] = sum_{c < m} dXt[bh, n, c] P[h, k, c] for X in {Q, K} (z = blockIdx.y).
// One workgroup per (head, 64 rows); P^T and the rows' dXt staged in LDS; each thread
// computes a block of RT rows x 4 features with fp32 FMAs (RT = D / 16).
constexpr int kBackRows = 64;
template <int D>
__global__ __launch_bounds__(kThreads) void proj_back_kernel(
    const float* __restrict__ dQt, const float* __restrict__ dKt, const uint16_t* __restrict__ P,
    void* __restrict__ dQ, void* __restrict__ dK, int out_f32, int N, int H, int m, int mp,
    int nrb) {
    constexpr int KG = D / 4;                 // feature groups of 4
    constexpr int RT = kBackRows * KG / kThreads;  // rows per thread
    extern __shared__ __attribute__((aligned(16))) float sm[];
    float* Ps = sm;                           // [m][D]: P^T of the head
    float* Xs = sm + m * D;                   // [kBackRows][m]
    const int bh = blockIdx.x / nrb;
    const int n0 = (blockIdx.x - bh * nrb) * kBackRows;
    const int z = blockIdx.y;
    const float* src = (z ? dKt : dQt) + (size_t)bh * N * mp;
    const int h = bh % H;
    for (int i = threadIdx.x; i < D * m; i += kThreads) {
        const int k = i / m, c = i - k * m;
        Ps[c * D + k] = __uint_as_float((uint32_t)P[(size_t)h * D * m + i] << 16);
    }
    for (int i = threadIdx.x; i < kBackRows * m; i += kThreads) {
        const int r = i / m, c = i - r * m;
        Xs[i] = n0 + r < N ? src[(size_t)(n0 + r) * mp + c] : 0.0f;
    }
    __syncthreads();
    const int kg = threadIdx.x % KG, rg = threadIdx.x / KG;
    float acc[RT][4];
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[r][j] = 0.0f;
    for (int c = 0; c < m; ++c) {
        const float4 p4 = *reinterpret_cast<const float4*>(Ps + c * D + 4 * kg);
#pragma unroll
        for (int r = 0; r < RT; ++r) {
            const float x = Xs[(rg * RT + r) * m + c];
            acc[r][0] += x * p4.x;
            acc[r][1] += x * p4.y;
            acc[r][2] += x * p4.z;
            acc[r][3] += x * p4.w;
        }
    }
    void* dst = z ? dK : dQ;
#pragma unroll
    for (int r = 0; r < RT; ++r) {
        const int n = n0 + rg * RT + r;
        if (n >= N) continue;
        const size_t o = ((size_t)bh * N + n) * D + 4 * kg;
        if (out_f32) {
            *reinterpret_cast<float4*>(static_cast<float*>(dst) + o) =
                make_float4(acc[r][0], acc[r][1], acc[r][2], acc[r][3]);
        } else {
            u32x2 w;
            w.x = pack_bf16x2(acc[r][0], acc[r][1]);
            w.y = pack_bf16x2(acc[r][2], acc[r][3]);
            *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(dst) + o) = w;
        }
    }
}

// partial[bh, chunk, k, c] = sum over the chunk's rows n of Q[n,k] dQt[n,c] + K[n,k] dKt[n,c].
// Thread t owns features 4*(t % (D/4)) .. +3 and columns c = t / (D/4) + CG * i (CG = 1024 /
// D column groups, TC = D / 16 columns each, m <= 64), accumulated over rows in fp32.
constexpr int kDpRows = 256;
constexpr int kDpSub = 32;
template <int D>
__global__ __launch_bounds__(kThreads) void dp_partial_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const float* __restrict__ dQt,
    const float* __restrict__ dKt, float* __restrict__ part, int N, int m, int mp, int nch) {
    constexpr int KG = D / 4;
    constexpr int CG = kThreads / KG;
    constexpr int TC = 64 / CG;
    extern __shared__ __attribute__((aligned(16))) float sm[];
    float* Qs = sm;                      // [kDpSub][D]
    float* Ks = Qs + kDpSub * D;         // [kDpSub][D]
    float* dQs = Ks + kDpSub * D;        // [kDpSub][m]
    float* dKs = dQs + kDpSub * m;       // [kDpSub][m]
    const int bh = blockIdx.x / nch;
    const int ch = blockIdx.x - bh * nch;
    const int n0 = ch * kDpRows;
    const int kg = threadIdx.x % KG, cg = threadIdx.x / KG;
    float acc[4][TC];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < TC; ++i) acc[j][i] = 0.0f;
    for (int s0 = n0; s0 < n0 + kDpRows && s0 < N; s0 += kDpSub) {
        __syncthreads();
        for (int i = threadIdx.x; i < kDpSub * D; i += kThreads) {
            const int r = i / D, kk = i - r * D;
            const bool ok = s0 + r < N;
            const size_t o = ((size_t)bh * N + s0 + r) * D + kk;
            Qs[i] = ok ? __uint_as_float((uint32_t)Q[o] << 16) : 0.0f;
            Ks[i] = ok ? __uint_as_float((uint32_t)K[o] << 16) : 0.0f;
        }
        for (int i = threadIdx.x; i < kDpSub * m; i += kThreads) {
            const int r = i / m, c = i - r * m;
            const bool ok = s0 + r < N;
            const size_t o = ((size_t)bh * N + s0 + r) * mp + c;
            dQs[i] = ok ? dQt[o] : 0.0f;
            dKs[i] = ok ? dKt[o] : 0.0f;
        }
        __syncthreads();
        for (int r = 0; r < kDpSub; ++r) {
            const float4 q = *reinterpret_cast<const float4*>(Qs + r * D + 4 * kg);
            const float4 kv = *reinterpret_cast<const float4*>(Ks + r * D + 4 * kg);
#pragma unroll
            for (int i = 0; i < TC; ++i) {
                const int c = cg + CG * i;
                if (c < m) {
                    const float a = dQs[r * m + c], b = dKs[r * m + c];
                    acc[0][i] += q.x * a + kv.x * b;
                    acc[1][i] += q.y * a + kv.y * b;
                    acc[2][i] += q.z * a + kv.z * b;
                    acc[3][i] += q.w * a + kv.w * b;
                }
            }
        }
    }
    float* dst = part + ((size_t)bh * nch + ch) * D * m;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < TC; ++i) {
            const int c = cg + CG * i;
            if (c < m) dst[(size_t)(4 * kg + j) * m + c] = acc[j][i];
        }
}

// dP[h, k, c] = sum over b (ascending) and chunks (ascending) of the partials.
__global__ __launch_bounds__(kThreads) void dp_reduce_kernel(const float* __restrict__ part,
                                                             float* __restrict__ dP, int B,
                                                             int H, int nout, int nch) {
    const int i = blockIdx.x * kThreads + threadIdx.x;
    if (i >= H * nout) return;
    const int h = i / nout, e = i - h * nout;
    float acc = 0.0f;
    for (int b = 0; b < B; ++b)
        for (int ch = 0; ch < nch; ++ch) acc += part[(((size_t)(b * H + h)) * nch + ch) * nout + e];
    dP[i] = acc;
}

template <int MP, int DV, bool CAUSAL>
hipError_t launch_main(const BwdArgs& a, hipStream_t s) {
    const int nqb = (a.N + 127) / 128;
    bwd_q_kernel<MP, DV, CAUSAL><<<dim3(a.BH * nqb), kThreads, 0, s>>>(
        a.Qs, a.Kt, a.Ktt, a.V, a.O, a.dO, a.lse, a.dQt, a.D, a.N, a.Np, nqb, a.scale);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    bwd_kv_kernel<MP, DV, CAUSAL><<<dim3(a.BH * nqb), kThreads, 0, s>>>(
        a.Qs, a.Qst, a.Kt, a.V, a.dO, a.dOt, a.lse, a.D, a.dV, a.g_f32, a.dKt, a.N, a.Np, nqb);
    return hipGetLastError();
}

template <int MP, int DV>
hipError_t launch_c(const BwdArgs& a, hipStream_t s) {
    return a.causal ? launch_main<MP, DV, true>(a, s) : launch_main<MP, DV, false>(a, s);
}

template <int MP>
hipError_t launch_dv(const BwdArgs& a, hipStream_t s) {
    switch (a.dv) {
        case 64: return launch_c<MP, 64>(a, s);
        case 128: return launch_c<MP, 128>(a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_attn_bwd_bf16(const BwdArgs& a, hipStream_t stream) {
    if ((long long)a.BH * ((a.N + 127) / 128) > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipError_t e;
    switch (a.mp) {
        case 16: e = launch_dv<16>(a, stream); break;
        case 32: e = launch_dv<32>(a, stream); break;
        case 64: e = launch_dv<64>(a, stream); break;
        default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess) return e;
    // back through the projection
    const int nrb = (a.N + kBackRows - 1) / kBackRows;
    const size_t sm_back = sizeof(float) * ((size_t)a.m * a.d + (size_t)kBackRows * a.m);
    if (a.d == 128)
        proj_back_kernel<128><<<dim3(a.BH * nrb, 2), kThreads, sm_back, stream>>>(
            a.dQt, a.dKt, a.P, a.dQ, a.dK, a.g_f32, a.N, a.H, a.m, a.mp, nrb);
    else
        proj_back_kernel<64><<<dim3(a.BH * nrb, 2), kThreads, sm_back, stream>>>(
            a.dQt, a.dKt, a.P, a.dQ, a.dK, a.g_f32, a.N, a.H, a.m, a.mp, nrb);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int nch = (a.N + kDpRows - 1) / kDpRows;
    const size_t sm_dp = sizeof(float) * (2 * (size_t)kDpSub * a.d + 2 * (size_t)kDpSub * a.m);
    if (a.d == 128)
        dp_partial_kernel<128><<<dim3(a.BH * nch), kThreads, sm_dp, stream>>>(
            a.Q, a.K, a.dQt, a.dKt, a.dPpart, a.N, a.m, a.mp, nch);
    else
        dp_partial_kernel<64><<<dim3(a.BH * nch), kThreads, sm_dp, stream>>>(
            a.Q, a.K, a.dQt, a.dKt, a.dPpart, a.N, a.m, a.mp, nch);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int nout = a.d * a.m;
    dp_reduce_kernel<<<dim3((a.H * nout + kThreads - 1) / kThreads), kThreads, 0, stream>>>(
        a.dPpart, a.dP, a.BH / a.H, a.H, nout, nch);
    return hipGetLastError();
}

}  // namespace spa
