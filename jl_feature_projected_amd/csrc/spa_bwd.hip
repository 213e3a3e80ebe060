// spa_bwd.hip -- backward of the projected attention for bf16 inputs on gfx950 MFMA.
//
// What it computes: the chain rule of the forward ("Sparse Projection Attention" page,
// Sec. 3.1.3 and Algorithm 1; its Sec. 3.4.1 Gradient Flow writes out the query term of the
// projection's gradient, which Algorithm 2 trains the projection with; the key term enters
// the same way). With A the row softmax of the forward, O = A V, dO = dL/dO:
//   D_i = <dO_i, O_i>,  dA_ij = <dO_i, V_j>,  dS_ij = A_ij (dA_ij - D_i)
//   dV_j = sum_i A_ij dO_i,  dQt_i = scale sum_j dS_ij Kt_j,  dKt_j = scale sum_i dS_ij Qt_i
//   dQ = dQt P^T,  dK = dKt P^T,  dP_h = sum over batches and rows of Q^T dQt + K^T dKt.
// The weights A are recomputed from the forward's log-sum-exp: the projected queries and keys
// are prepared exactly as in the forward (fp16, queries pre-scaled by scale*log2(e)), so the
// recomputed base-2 scores are the forward's, bit for bit.
//
// Kernels (on 32x32x16 MFMA unless noted; see the forward for the operand layouts):
//   bwd_kv_kernel  key-major: per 32-key wave, a loop over 32-query tiles computes
//                  dV^T = dO^T . A and dKt^T = Qt^T . dS; with DQ (mp <= 64) also
//                  dQt += dS Kt over the workgroup's 128 keys (dS through LDS, 16x16x32
//                  MFMAs, fp32 atomic adds), with D_i and lse from the preparation launch.
//   bwd_q_kernel   query-major (mp = 128 only): per 32-query wave, a loop over 32-key tiles
//                  computes dQt^T = Kt^T . dS^T, after D_i from the wave's own dO and O
//                  rows, which the key-major kernel then reads.
//   proj_grad_kernel   dQ = dQt P^T, dK = dKt P^T and the projection gradient's partial
//                  per 256-row chunk (bf16 MFMAs, fp32 factors split hi + lo).
//   dp_reduce_kernel   the partials summed over chunks and batches in a fixed order.
// In the transposed (A-operand) tiles the rows are V^T-ordered: within every 16 tokens the
// order 0-3, 8-11, 4-7, 12-15, which is the order in which a score accumulator lane holds
// its 8 tokens of a 16-token k-step. So every MFMA operand is one 16-byte LDS read or a
// register, as in the forward.
#include "spa_device.h"
#include "spa_internal.h"

namespace spa {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kBufs = 3;   // tile buffers of the MFMA kernels' loops
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

// Key-major kernel with the projected-query gradient: one dS tile in LDS, 128 key rows of 32
// f16 queries (64 bytes). Within every 16 queries the row holds them in the order 0-3, 8-11,
// 4-7, 12-15, the order in which a score accumulator lane holds them, so a lane's 8 values of
// a k-step are one 16-byte chunk; chunk c of row r sits at c ^ ds_swz(r). A half-wave's 16-byte
// store then covers every bank twice (the minimum for 512 bytes), and the 4 rows of a 16-lane
// transposing read lie in 4 distinct quarters of the banks.
constexpr int kDsBytes = 128 * 64;
__device__ __forceinline__ int ds_swz(int row) { return (row >> 2) & 3; }
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

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
// Query-major kernel: dQt, and per query -lse2 and -D for the key-major kernel.
// Inputs: Qs [BH,N,MP] fp16 (scaled), Kt [BH,N,MP] fp16, Ktt [BH,MP,Np] fp16 (transposed,
// permuted), V [BH,N,DV] bf16, O, dO [BH,N,DV] bf16, lse [BH,N] (natural log).
// Outputs: dQt [BH,N,MP] fp32 (scaled by `scale`); LD [BH, Np/32, 2, 32] fp32: per 32
// queries, -lse*log2(e) then -D (-inf and 0 for queries past N).
template <int MP, int DV, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void bwd_q_kernel(
    const uint16_t* __restrict__ Qs, const uint16_t* __restrict__ Kt,
    const uint16_t* __restrict__ Ktt, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ O, const uint16_t* __restrict__ dO,
    const float* __restrict__ lse, float* __restrict__ dQt, float* __restrict__ LD, int N,
    int Np, int nqb, float scale) {
    constexpr int KS = MP / 16;                // score k-steps
    constexpr int MB = (MP + 31) / 32;         // 32-row blocks of dQt^T
    constexpr int CS = DV / 16;                // dA k-steps
    // Tile buffer: Kt rows (32 keys x MP fp16), Kt^T rows (MB*32 feature rows x 32 keys,
    // rows past MP zero), V rows (32 keys x DV bf16). Rows unpadded, 16-byte chunks
    // swizzled (kswz of the row's element count); every region a whole number of 1 KiB
    // wave copies.
    constexpr int K_B = kTile * MP * 2;
    constexpr int KT_B = MB * 32 * kTile * 2;
    constexpr int V_B = kTile * DV * 2;
    constexpr int BUF = K_B + KT_B + V_B;
    constexpr int NCP = BUF / 1024;                    // wave copies per tile
    constexpr int CPW = (NCP + kWaves - 1) / kWaves;   // ... per wave
    static_assert(K_B % 1024 == 0 && KT_B % 1024 == 0 && V_B % 1024 == 0, "copy regions");
    __shared__ __attribute__((aligned(16))) char lds[kBufs * BUF];

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

    const int kend = CAUSAL ? min(N, q0 + 128) : N;
    const int ntiles = (kend + kTile - 1) / kTile;
    // Tiles before `nfree` need no mask: causal, all their keys precede the block's first
    // query; otherwise every tile but a ragged last one.
    const int nfree = CAUSAL ? min(ntiles, q0 / kTile) : N / kTile;

    // ---- HBM -> LDS tile copies ------------------------------------------------------
    // Wave copy j (j = wave, wave + 4, ...) fills buffer chunks 64j .. 64j+63; lane l writes
    // chunk c = 64j + l, which holds global chunk (slot ^ swizzle(row)) of its region's row.
    // Per copy: the head's array, its bytes per token of tile advance and its size (loads
    // past it read zero), the lane's byte offset from the tile's first token. A wave past
    // the last copy repeats it (same bytes to the same place).
    const int wu = __builtin_amdgcn_readfirstlane(wave);
    const char* cbase[CPW];
    int cstep[CPW], ctot[CPW];
    uint32_t coff[CPW], cdst[CPW];
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
        const int j = min(wu + kWaves * i, NCP - 1);
        const int c = 64 * j + lane;
        cdst[i] = 1024 * j;
        if (64 * j < K_B / 16) {
            const int row = c / (MP / 8), slot = c % (MP / 8);
            cbase[i] = Kh, cstep[i] = MP * 2, ctot[i] = N * MP * 2;
            coff[i] = row * MP * 2 + 16 * (slot ^ kswz<MP>(row));
        } else if (64 * j < (K_B + KT_B) / 16) {
            const int cc = c - K_B / 16, row = cc >> 2, slot = cc & 3;
            cbase[i] = Kth, cstep[i] = 2, ctot[i] = MP * Np * 2;
            coff[i] = row < MP ? row * Np * 2 + 16 * (slot ^ kswz<kTile>(row)) : kOutOfRange;
        } else {
            const int cc = c - (K_B + KT_B) / 16, row = cc / (DV / 8), slot = cc % (DV / 8);
            cbase[i] = Vh, cstep[i] = DV * 2, ctot[i] = N * DV * 2;
            coff[i] = row * DV * 2 + 16 * (slot ^ kswz<DV>(row));
        }
    }
    const uint32_t lds0 = lds_address(lds);
    auto copy_tile = [&](int k0, int buf) {
#pragma unroll
        for (int i = 0; i < CPW; ++i) {
            const int skip = k0 * cstep[i];
            copy16_to_lds(make_rsrc(cbase[i] + skip, (uint32_t)max(ctot[i] - skip, 0)),
                          lds0 + buf * BUF + cdst[i], coff[i]);
        }
    };
    // Tile 0's copies go out before the lane's own rows are loaded; the wait for both
    // comes before tile 1's copies (a wait left to the compiler would land inside the tile
    // loop, where it would also wait for the copies in flight).
    copy_tile(0, 0);

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
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    copy_tile(kTile, 1);
    // The score accumulator starts at -lse2 and the dA accumulator at -D, so the MFMAs
    // leave s - lse2 and dA - D.
    const f32x16 sinit = f32x16_fill(-lse2);
    const f32x16 dinit = f32x16_fill(-Dq);

    // Per-lane LDS read offsets (fixed across tiles). Kt tile: row col, chunk 2ks + half;
    // V tile: row col, chunk 2cs + half; Kt^T tile: row mb*32 + col (same swizzle for
    // every mb), chunk 2tt + half.
    uint32_t kread[KS], vread[CS], tread[2];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) kread[ks] = col * MP * 2 + 16 * ((2 * ks + half) ^ kswz<MP>(col));
#pragma unroll
    for (int cs = 0; cs < CS; ++cs) vread[cs] = col * DV * 2 + 16 * ((2 * cs + half) ^ kswz<DV>(col));
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) tread[tt] = col * kTile * 2 + 16 * ((2 * tt + half) ^ kswz<kTile>(col));

    f32x16 acc[MB];
#pragma unroll
    for (int b = 0; b < MB; ++b) acc[b] = f32x16_fill(0.0f);

    // Three buffers, one barrier per step: step t requests tile t+2 into the buffer step t-1
    // read, computes tile t, then waits for its own copies of tile t+1 before the barrier
    // that hands tile t+1 to every wave. Copies past the last tile read real or zero bytes
    // into a buffer no step reads.
    auto step = [&](int t, int cur, auto mask_tag) {
        constexpr bool MASK = decltype(mask_tag)::value;
        const int k0 = t * kTile;
        copy_tile(k0 + 2 * kTile, cur == 0 ? kBufs - 1 : cur - 1);
        const char* Ks = lds + cur * BUF;
        const char* Kts = Ks + K_B;
        const char* Vs = Kts + KT_B;
        // causal: a wave whose queries all precede the tile has nothing to do in it
        if (!(MASK && CAUSAL) || k0 <= q0 + wave * 32 + 31) {
            // scores^T (32 keys x 32 queries), base-2 units, minus lse2
            f32x16 s = sinit;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                s = mfma32x32x16(__builtin_bit_cast(f16x8, *reinterpret_cast<const u32x4*>(Ks + kread[ks])),
                                 qf[ks], s);
            // dA^T (32 keys x 32 queries) = V . dO^T, minus D
            f32x16 da = dinit;
#pragma unroll
            for (int cs = 0; cs < CS; ++cs)
                da = mfma32x32x16(__builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(Vs + vread[cs])),
                                  dof[cs], da);
            // dS = A (dA - D), masked entries (later keys, keys past N) zero
            f32x16 ds;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float w = __builtin_amdgcn_exp2f(s[i]);
                if (MASK) {
                    const int key = k0 + 8 * (i >> 2) + 4 * half + (i & 3);
                    if ((CAUSAL && key > myq) || key >= N) w = 0.0f;
                }
                ds[i] = w * da[i];
            }
            // dQt^T (MP x 32 queries) += Kt^T . dS^T
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                const f16x8 b = __builtin_bit_cast(f16x8, pack_kstep<true>(ds, tt));
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) {
                    const f16x8 a = __builtin_bit_cast(
                        f16x8, *reinterpret_cast<const u32x4*>(Kts + mb * 32 * kTile * 2 + tread[tt]));
                    acc[mb] = mfma32x32x16(a, b, acc[mb]);
                }
            }
        }
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(CPW));
        __syncthreads();
    };

    __syncthreads();  // tile 0 from every wave
    int t = 0, cur = 0;
#pragma unroll 1
    for (; t < nfree; ++t, cur = cur == kBufs - 1 ? 0 : cur + 1) step(t, cur, Flag<false>{});
#pragma unroll 1
    for (; t < ntiles; ++t, cur = cur == kBufs - 1 ? 0 : cur + 1) step(t, cur, Flag<true>{});
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // no copy may land after the workgroup ends

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
    }
    if (half == 0 && myq < Np) {
        float* dst = LD + ((size_t)bh * Np + (myq & ~(kTile - 1))) * 2 + (myq & (kTile - 1));
        dst[0] = -lse2;
        dst[kTile] = -Dq;
    }
}

// ---------------------------------------------------------------------------------------
// Key-major kernel: dV and dKt.
// Inputs: Qs [BH,N,MP] fp16 (scaled), Qst [BH,MP,Np] fp16 (transposed, permuted), Kt
// [BH,N,MP] fp16, V [BH,N,DV] bf16, dO [BH,N,DV] bf16, dOt [BH,DV,Np] bf16 (transposed,
// permuted), LD (from the query-major kernel).
// Outputs: dV [BH,N,DV] (fp32 or bf16), dKt [BH,N,MP] fp32 (scale applied).
template <int MP, int DV, bool CAUSAL, bool DQ>
__global__ __launch_bounds__(kThreads, (MP >= 64 && DV >= 128) ? 1 : 2) void bwd_kv_kernel(
    const uint16_t* __restrict__ Qs, const uint16_t* __restrict__ Qst,
    const uint16_t* __restrict__ Kt, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const uint16_t* __restrict__ dOt,
    const float* __restrict__ LD, void* __restrict__ dV, int dv_f32, float* __restrict__ dKt,
    float* __restrict__ dQt, float scale, int N, int Np, int nkb) {
    constexpr int KS = MP / 16;
    constexpr int MB = (MP + 31) / 32;
    constexpr int CS = DV / 16;
    constexpr int DB = DV / 32;
    // Tile buffer: Qs rows (32 queries x MP fp16), Qs^T rows (MB*32 feature rows x 32
    // queries, rows past MP zero), dO rows (32 x DV bf16), dO^T rows (DV x 32 queries), all
    // as in the query-major kernel; then -lse2 and -D of the 32 queries.
    constexpr int Q_B = kTile * MP * 2;
    constexpr int QT_B = MB * 32 * kTile * 2;
    constexpr int DO_B = kTile * DV * 2;
    constexpr int DOT_B = DV * kTile * 2;
    constexpr int B16 = Q_B + QT_B + DO_B + DOT_B;     // bytes copied 16 per lane
    constexpr int BUF = B16 + 2 * kTile * 4;
    constexpr int NCP = B16 / 1024;
    constexpr int CPW = (NCP + kWaves - 1) / kWaves;
    static_assert(Q_B % 1024 == 0 && QT_B % 1024 == 0 && DO_B % 1024 == 0 && DOT_B % 1024 == 0,
                  "copy regions");
    // DQ: two dS tiles (one being written, the previous one being read), kDsBytes each
    __shared__ __attribute__((aligned(16))) char lds[kBufs * BUF + (DQ ? 2 * kDsBytes : 0)];
    char* dsl = lds + kBufs * BUF;

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
    const float* LDh = LD + (size_t)bh * Np * 2;

    const int qstart = CAUSAL ? k0 : 0;
    const int ntiles = (N - qstart + kTile - 1) / kTile;
    // causal: the first four tiles meet the block's keys and need the mask
    const int nmask = CAUSAL ? min(ntiles, 128 / kTile) : 0;

    // ---- HBM -> LDS tile copies, as in the query-major kernel ---------------------------
    const int wu = __builtin_amdgcn_readfirstlane(wave);
    const char* cbase[CPW];
    int cstep[CPW], ctot[CPW];
    uint32_t coff[CPW], cdst[CPW];
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
        const int j = min(wu + kWaves * i, NCP - 1);
        const int c = 64 * j + lane;
        cdst[i] = 1024 * j;
        if (64 * j < Q_B / 16) {
            const int row = c / (MP / 8), slot = c % (MP / 8);
            cbase[i] = Qh, cstep[i] = MP * 2, ctot[i] = N * MP * 2;
            coff[i] = row * MP * 2 + 16 * (slot ^ kswz<MP>(row));
        } else if (64 * j < (Q_B + QT_B) / 16) {
            const int cc = c - Q_B / 16, row = cc >> 2, slot = cc & 3;
            cbase[i] = Qth, cstep[i] = 2, ctot[i] = MP * Np * 2;
            coff[i] = row < MP ? row * Np * 2 + 16 * (slot ^ kswz<kTile>(row)) : kOutOfRange;
        } else if (64 * j < (Q_B + QT_B + DO_B) / 16) {
            const int cc = c - (Q_B + QT_B) / 16, row = cc / (DV / 8), slot = cc % (DV / 8);
            cbase[i] = dOh, cstep[i] = DV * 2, ctot[i] = N * DV * 2;
            coff[i] = row * DV * 2 + 16 * (slot ^ kswz<DV>(row));
        } else {
            const int cc = c - (Q_B + QT_B + DO_B) / 16, row = cc >> 2, slot = cc & 3;
            cbase[i] = dOth, cstep[i] = 2, ctot[i] = DV * Np * 2;
            coff[i] = row * Np * 2 + 16 * (slot ^ kswz<kTile>(row));
        }
    }
    const uint32_t lds0 = lds_address(lds);
    // CPW 16-byte copies, then the tile's -lse2 and -D (one 4-byte copy, the same in every
    // wave).
    auto copy_tile = [&](int q0, int buf) {
#pragma unroll
        for (int i = 0; i < CPW; ++i) {
            const int skip = q0 * cstep[i];
            copy16_to_lds(make_rsrc(cbase[i] + skip, (uint32_t)max(ctot[i] - skip, 0)),
                          lds0 + buf * BUF + cdst[i], coff[i]);
        }
        copy4_to_lds(make_rsrc(LDh + 2 * q0, (uint32_t)max(Np - q0, 0) * 8), lds0 + buf * BUF + B16,
                     4 * lane);
    };
    copy_tile(qstart, 0);  // then the lane's rows, then one wait, as in the query-major kernel

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
    // DQ: this wave's share of dQt (32 queries x MP) per tile: 16x16 output
    // blocks u (query half u & 1, features 16 (u >> 1) ..), each a sum over the workgroup's
    // 128 keys in four 32-key k-steps; the wave takes the (block, k-step) pairs
    // dq_block(p), dq_kstep(p). Their B operands (Kt of 8 keys for one feature) stay in
    // registers.
    constexpr int NT = DQ ? 2 * (MP / 16) : 0;           // 16x16 output blocks per tile
    constexpr int NPAIR = DQ ? NT : 1;                    // (block, k-step) pairs per wave
    const int g16 = lane >> 4, j16 = lane & 15;
    auto dq_block = [&](int p) { return NT >= 4 ? wave + 4 * (p >> 2) : (wave & 1); };
    auto dq_kstep = [&](int p) { return NT >= 4 ? (p & 3) : 2 * (wave >> 1) + p; };
    f16x8 kq[NPAIR];
    if constexpr (DQ) {
#pragma unroll
        for (int p = 0; p < NPAIR; ++p) {
            const int f = 16 * (dq_block(p) >> 1) + j16;
            const int key0 = k0 + 32 * dq_kstep(p) + 8 * g16;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int key = key0 + e;
                kq[p][e] = key < N ? __builtin_bit_cast(_Float16, Kt[((size_t)bh * N + key) * MP + f])
                                   : (_Float16)0.0f;
            }
        }
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    copy_tile(qstart + kTile, 1);

    // Per-lane LDS read offsets: Qs tile row col, chunk 2ks + half; dO tile row col, chunk
    // 2cs + half; transposed tiles (Qs^T, dO^T) row blk*32 + col, chunk 2tt + half.
    uint32_t kread[KS], oread[CS], tread[2];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) kread[ks] = col * MP * 2 + 16 * ((2 * ks + half) ^ kswz<MP>(col));
#pragma unroll
    for (int cs = 0; cs < CS; ++cs) oread[cs] = col * DV * 2 + 16 * ((2 * cs + half) ^ kswz<DV>(col));
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) tread[tt] = col * kTile * 2 + 16 * ((2 * tt + half) ^ kswz<kTile>(col));

    f32x16 dva[DB], dka[MB];
#pragma unroll
    for (int b = 0; b < DB; ++b) dva[b] = f32x16_fill(0.0f);
#pragma unroll
    for (int b = 0; b < MB; ++b) dka[b] = f32x16_fill(0.0f);

    // DQ: the tile's dS (f16) in the layout above. The lane's packed dS of k-step tt (queries
    // 16tt + 4half .. +3 and 16tt + 8 + 4half .. +3 of its key) is chunk 2tt + half of its
    // key's row. A wave with nothing to do in a tile stores zeros, as do keys past N.
    const int dsrow = wave * 32 + col;
    auto ds_store = [&](int buf, int tt, u32x4 w) {
        *reinterpret_cast<u32x4*>(dsl + buf * kDsBytes + dsrow * 64 +
                                  16 * ((2 * tt + half) ^ ds_swz(dsrow))) = w;
    };
    // dQt += scale * dS Kt for the tile in dS buffer buf (queries from qd0): the A operand of
    // block u, k-step ks is two transposing reads; lane (g, 4e + a) of the 16x16x32 layout
    // addresses key row 32ks + 8g + 4s + e, queries 16 (u & 1) + 4a .. +3 (s = 0, 1 for the
    // operand's first and last four keys), which the row holds at chunk 2 (u & 1) + (a & 1),
    // bytes 8 (a >> 1) .. +7. The results go to dQt by fp32 atomic adds through a buffer
    // resource of the head's N rows, which drops the adds of queries past N.
    const __amdgpu_buffer_rsrc_t dqr =
        __builtin_amdgcn_make_buffer_rsrc(dQt + (size_t)bh * N * MP, (short)0, N * MP * 4, 0x00020000);
    auto dq_phase = [&](int buf, int qd0) {
        const char* base = dsl + buf * kDsBytes;
        f32x4 acc[NT >= 4 ? NT / 4 : 1];
#pragma unroll
        for (int b = 0; b < (NT >= 4 ? NT / 4 : 1); ++b) acc[b] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int p = 0; p < NPAIR; ++p) {
            const int u = dq_block(p), ks = dq_kstep(p);
            const int e = j16 >> 2, a = j16 & 3;
            u32x2 h[2];
#pragma unroll
            for (int sh = 0; sh < 2; ++sh) {
                const int row = 32 * ks + 8 * g16 + 4 * sh + e;
                const int c = 2 * (u & 1) + (a & 1);
                typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
                const i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_i16x4*)(base + row * 64 + 16 * (c ^ ds_swz(row)) + 8 * (a >> 1)));
                h[sh] = __builtin_bit_cast(u32x2, r);
            }
            const f16x8 af = __builtin_bit_cast(f16x8, u32x4{h[0].x, h[0].y, h[1].x, h[1].y});
            f32x4& c = acc[NT >= 4 ? p >> 2 : 0];
            c = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, kq[p], c, 0, 0, 0);
        }
#pragma unroll
        for (int b = 0; b < (NT >= 4 ? NT / 4 : 1); ++b) {
            const int u = dq_block(NT >= 4 ? 4 * b : 0);
            const int f = 16 * (u >> 1) + j16;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int q = qd0 + 16 * (u & 1) + 4 * g16 + i;
                __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(acc[b][i] * scale, dqr,
                                                                 (q * MP + f) * 4, 0, 0);
            }
        }
    };

    // Three buffers, one barrier per step, as in the query-major kernel. DQ: step t first
    // takes tile t-1's dS (stored before the last barrier) into dQt, before the step's tile
    // copies: the atomic adds count in the same in-order vector-memory counter, so issued
    // after the copies they would make the step's closing wait also wait for those copies.
    auto step = [&](int t, int cur, auto mask_tag) {
        constexpr bool MASK = decltype(mask_tag)::value;
        const int q0 = qstart + t * kTile;
        if constexpr (DQ) {
            if (t > 0) dq_phase((t - 1) & 1, q0 - kTile);
            __builtin_amdgcn_sched_barrier(0);
        }
        copy_tile(q0 + 2 * kTile, cur == 0 ? kBufs - 1 : cur - 1);
        const char* Qts = lds + cur * BUF;      // Qs tile (rows = queries)
        const char* QTs = Qts + Q_B;            // Qs^T tile (rows = features)
        const char* dOs = QTs + QT_B;           // dO tile (rows = queries)
        const char* dOTs = dOs + DO_B;          // dO^T tile (rows = V columns)
        const float* Ls = reinterpret_cast<const float*>(Qts + B16);  // -lse2 [32], -D [32]
        // causal: nothing to do if every query of the tile precedes every key of the wave
        const bool active = !MASK || q0 + kTile - 1 >= k0w;
        if constexpr (DQ) {
            if (!active)
#pragma unroll
                for (int tt = 0; tt < 2; ++tt) ds_store(t & 1, tt, u32x4{0u, 0u, 0u, 0u});
        }
        if (active) {
            // accumulators start at -lse2 and -D of the slot's query (8*(i/4) + 4*half + i%4)
            f32x16 s, da;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const float4 l4 = *reinterpret_cast<const float4*>(Ls + 8 * g + 4 * half);
                const float4 d4 = *reinterpret_cast<const float4*>(Ls + kTile + 8 * g + 4 * half);
                s[4 * g] = l4.x, s[4 * g + 1] = l4.y, s[4 * g + 2] = l4.z, s[4 * g + 3] = l4.w;
                da[4 * g] = d4.x, da[4 * g + 1] = d4.y, da[4 * g + 2] = d4.z, da[4 * g + 3] = d4.w;
            }
            // scores^T (32 queries x 32 keys) - lse2
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                s = mfma32x32x16(__builtin_bit_cast(f16x8, *reinterpret_cast<const u32x4*>(Qts + kread[ks])),
                                 kf[ks], s);
            // dA^T (32 queries x 32 keys) = dO . V^T, minus D
#pragma unroll
            for (int cs = 0; cs < CS; ++cs)
                da = mfma32x32x16(__builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(dOs + oread[cs])),
                                  vf[cs], da);
            // weights and dS
            f32x16 w, ds;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float a = __builtin_amdgcn_exp2f(s[i]);
                if (MASK && myk > q0 + 8 * (i >> 2) + 4 * half + (i & 3)) a = 0.0f;
                w[i] = a;
                ds[i] = a * da[i];
            }
            // dV^T (DV x 32 keys) += dO^T . A ; dKt^T (MP x 32 keys) += Qs^T . dS
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                const bf16x8 bw = __builtin_bit_cast(bf16x8, pack_kstep<false>(w, tt));
                const u32x4 bsu = pack_kstep<true>(ds, tt);
                const f16x8 bs = __builtin_bit_cast(f16x8, bsu);
                if constexpr (DQ) ds_store(t & 1, tt, kvalid ? bsu : u32x4{0u, 0u, 0u, 0u});
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    const bf16x8 a = __builtin_bit_cast(
                        bf16x8, *reinterpret_cast<const u32x4*>(dOTs + db * 32 * kTile * 2 + tread[tt]));
                    dva[db] = mfma32x32x16(a, bw, dva[db]);
                }
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) {
                    const f16x8 a = __builtin_bit_cast(
                        f16x8, *reinterpret_cast<const u32x4*>(QTs + mb * 32 * kTile * 2 + tread[tt]));
                    dka[mb] = mfma32x32x16(a, bs, dka[mb]);
                }
            }
        }
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(CPW + 1));
        __syncthreads();
    };

    __syncthreads();  // tile 0 from every wave
    int t = 0, cur = 0;
#pragma unroll 1
    for (; t < nmask; ++t, cur = cur == kBufs - 1 ? 0 : cur + 1) step(t, cur, Flag<true>{});
#pragma unroll 1
    for (; t < ntiles; ++t, cur = cur == kBufs - 1 ? 0 : cur + 1) step(t, cur, Flag<false>{});
    if constexpr (DQ) {
        if (ntiles > 0) dq_phase((ntiles - 1) & 1, qstart + (ntiles - 1) * kTile);
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // no copy may land after the workgroup ends

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
// Back through the projection, one pass over the rows of a head:
//   dQ = dQt P^T, dK = dKt P^T                (rows of the workgroup's chunk)
//   partial[bh, chunk] = Q^T dQt + K^T dKt    (the chunk's share of the projection gradient)
// on bf16 MFMAs with each fp32 factor of dQt and dKt split as hi + lo (both bf16, hi the
// rounded value, lo the rounded remainder): the products keep about 16 significant bits of
// the fp32 factor, the accumulation is fp32. Q, K and P are bf16 already.
// Workgroup: kPgRows rows of one head, in passes of kPgSub rows staged in LDS transposed
// (feature-major) for the products that contract over rows.
constexpr int kPgRows = 256;
constexpr int kPgSub = 64;

__device__ __forceinline__ void split_bf16(float x, uint16_t& hi, uint16_t& lo) {
    const uint32_t h = pack_bf16x2(x, 0.0f) & 0xffffu;
    hi = (uint16_t)h;
    lo = (uint16_t)(pack_bf16x2(x - __uint_as_float(h << 16), 0.0f) & 0xffffu);
}

template <int D, int MP>
__global__ __launch_bounds__(kThreads, MP >= 128 ? 1 : 2) void proj_grad_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const float* __restrict__ dQt,
    const float* __restrict__ dKt, const uint16_t* __restrict__ P, void* __restrict__ dQ,
    void* __restrict__ dK, int out_f32, float* __restrict__ part, int N, int H, int m, int nch) {
    constexpr int KB = D / 32;                 // 32-feature blocks
    constexpr int KS = MP / 16;                // k-steps over the projected columns
    constexpr int MB = (MP + 31) / 32;         // 32-column blocks of the partial
    constexpr int TP = kPgSub * 2 + 16;        // transposed tile row pitch (bytes), padded
    constexpr int QT_B = D * TP;               // Q^T or K^T: D feature rows x kPgSub rows
    constexpr int XT_B = MB * 32 * TP;         // one bf16 plane of dQt^T or dKt^T
    constexpr int ZW = KB == 4 ? 1 : 2;        // waves per feature block (D = 64: one per term)
    static_assert(KB * ZW == kWaves, "one feature block (and term) per wave");
    // MP <= 32: dQt and dKt rows also kept row-major in LDS (fp32, rows padded by 16 bytes),
    // the B operands of dQ and dK; wider rows read them from global memory instead.
    constexpr bool XROW = MP <= 32;
    constexpr int XRP = MP + 4;                // row pitch (floats)
    constexpr int XR_B = XROW ? kPgSub * XRP * 4 : 0;
    __shared__ __attribute__((aligned(16))) char lds[2 * QT_B + 4 * XT_B + 2 * XR_B];
    // Q^T (z = 0) and K^T (z = 1); then the hi (p = 0) and lo planes of dQt^T and dKt^T
    auto QTs = [&](int z) { return lds + z * QT_B; };
    auto XTs = [&](int z, int p) { return lds + 2 * QT_B + (2 * z + p) * XT_B; };
    auto XRs = [&](int z) { return reinterpret_cast<float*>(lds + 2 * QT_B + 4 * XT_B + z * XR_B); };

    const int bh = blockIdx.x / nch;
    const int ch = blockIdx.x - bh * nch;
    const int h = bh % H;
    const int r0 = ch * kPgRows;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, col = lane & 31, half = lane >> 5;
    const int kb = wave % KB;                  // this wave's feature block

    // Feature rows past MP of the dQt^T planes stay zero.
    if (MB * 32 > MP) {
        for (int i = tid; i < (MB * 32 - MP) * TP / 4; i += kThreads)
#pragma unroll
            for (int z = 0; z < 2; ++z)
#pragma unroll
                for (int p = 0; p < 2; ++p) reinterpret_cast<uint32_t*>(XTs(z, p) + MP * TP)[i] = 0u;
    }

    // A operands of dX = dXt P^T: P[k][c] for k = kb*32 + col, c = 16ks + 8half .. +7 (zero
    // past m).
    bf16x8 pa[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        const uint16_t* prow = P + ((size_t)h * D + kb * 32 + col) * m;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int c = ks * 16 + half * 8 + e;
            pa[ks][e] = __builtin_bit_cast(bf16_t, c < m ? prow[c] : (uint16_t)0);
        }
    }

    f32x16 accp[MB];  // this wave's share of the partial: features kb*32.., columns mb*32..
#pragma unroll
    for (int b = 0; b < MB; ++b) accp[b] = f32x16_fill(0.0f);

    // This thread's share of a pass's rows, loaded a pass ahead: Q and K rows (thread =
    // (row, 16-byte chunk column)) and dQt and dKt rows (thread = (row, 4-column chunk)).
    constexpr int XC = (MP / 4 + kWaves - 1) / kWaves;  // 4-column chunks per thread and term
    const int row = tid % kPgSub;
    u32x4 qv[2][D / 32];
    float4 xv[2][XC];
    auto load_pass = [&](int rs) {
        const bool rok = rs + row < N;
#pragma unroll
        for (int z = 0; z < 2; ++z) {
            const uint16_t* X = (z ? K : Q) + ((size_t)bh * N + rs + row) * D;
#pragma unroll
            for (int i = 0; i < D / 32; ++i) {
                const int cc = tid / kPgSub + kWaves * i;
                qv[z][i] = u32x4{0u, 0u, 0u, 0u};
                if (rok) qv[z][i] = *reinterpret_cast<const u32x4*>(X + cc * 8);
            }
            const float* Xt = (z ? dKt : dQt) + ((size_t)bh * N + rs + row) * MP;
#pragma unroll
            for (int i = 0; i < XC; ++i) {
                const int cc = tid / kPgSub + kWaves * i;
                xv[z][i] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
                if (rok && cc < MP / 4) xv[z][i] = *reinterpret_cast<const float4*>(Xt + cc * 4);
            }
        }
    };
    load_pass(r0);

#pragma unroll 1
    for (int rs = r0; rs < r0 + kPgRows && rs < N; rs += kPgSub) {
        __syncthreads();  // the previous pass's tiles are read
        // Q^T and K^T: 8 two-byte transposed writes per 16-byte chunk.
#pragma unroll
        for (int z = 0; z < 2; ++z) {
#pragma unroll
            for (int i = 0; i < D / 32; ++i) {
                const int cc = tid / kPgSub + kWaves * i;
                const u32x4 v = qv[z][i];
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    *reinterpret_cast<uint16_t*>(QTs(z) + (cc * 8 + e) * TP + row * 2) =
                        (uint16_t)(v[e >> 1] >> (16 * (e & 1)));
            }
        }
        // dQt^T and dKt^T, hi and lo planes (and the row-major copy).
#pragma unroll
        for (int z = 0; z < 2; ++z) {
#pragma unroll
            for (int i = 0; i < XC; ++i) {
                const int cc = tid / kPgSub + kWaves * i;
                if (cc < MP / 4) {
                    const float4 v = xv[z][i];
                    if constexpr (XROW) *reinterpret_cast<float4*>(XRs(z) + row * XRP + cc * 4) = v;
                    const float f[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        uint16_t hi, lo;
                        split_bf16(f[e], hi, lo);
                        *reinterpret_cast<uint16_t*>(XTs(z, 0) + (cc * 4 + e) * TP + row * 2) = hi;
                        *reinterpret_cast<uint16_t*>(XTs(z, 1) + (cc * 4 + e) * TP + row * 2) = lo;
                    }
                }
            }
        }
        __syncthreads();
        // The next pass's rows are requested now, to arrive during this pass's products.
        const bool more = rs + kPgSub < r0 + kPgRows && rs + kPgSub < N;
        if (XROW && more) load_pass(rs + kPgSub);

        // dQ, dK: output block (term z, 32-row block rb, feature block kb):
        // D[k][row] = sum_c P[k][c] Xt[row][c], B operand = lane row's 8 columns, hi and lo.
#pragma unroll
        for (int i = 0; i < 4 / ZW; ++i) {
            const int bz = (wave / KB) + ZW * i;   // 0..3 over (z, rb)
            const int z = bz >> 1, rb = bz & 1;
            const int orow = rs + rb * 32 + col;
            const bool ook = orow < N;
            const float* X = (z ? dKt : dQt) + ((size_t)bh * N + orow) * MP;
            f32x16 o = f32x16_fill(0.0f);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                float4 a = make_float4(0.0f, 0.0f, 0.0f, 0.0f), b = a;
                if constexpr (XROW) {
                    // rows past N were staged as zeros
                    const float* xr = XRs(z) + (rb * 32 + col) * XRP + ks * 16 + half * 8;
                    a = *reinterpret_cast<const float4*>(xr);
                    b = *reinterpret_cast<const float4*>(xr + 4);
                } else if (ook) {
                    a = *reinterpret_cast<const float4*>(X + ks * 16 + half * 8);
                    b = *reinterpret_cast<const float4*>(X + ks * 16 + half * 8 + 4);
                }
                const float f[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
                bf16x8 bh8, bl8;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    uint16_t hi, lo;
                    split_bf16(f[e], hi, lo);
                    bh8[e] = __builtin_bit_cast(bf16_t, hi);
                    bl8[e] = __builtin_bit_cast(bf16_t, lo);
                }
                o = mfma32x32x16(pa[ks], bh8, o);
                o = mfma32x32x16(pa[ks], bl8, o);
            }
            if (ook) {
                void* dst = z ? dK : dQ;
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const size_t at = ((size_t)bh * N + orow) * D + kb * 32 + 8 * g + 4 * half;
                    if (out_f32) {
                        *reinterpret_cast<float4*>(static_cast<float*>(dst) + at) =
                            make_float4(o[4 * g], o[4 * g + 1], o[4 * g + 2], o[4 * g + 3]);
                    } else {
                        u32x2 w;
                        w.x = pack_bf16x2(o[4 * g], o[4 * g + 1]);
                        w.y = pack_bf16x2(o[4 * g + 2], o[4 * g + 3]);
                        *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(dst) + at) = w;
                    }
                }
            }
        }

        // (Wider rows: their B operands above came from global memory, so the next pass's
        // loads go out only now, behind them.)
        if (!XROW && more) load_pass(rs + kPgSub);

        // Partial: D[k][c] += sum_rows X^T[k][row] Xt[row][c] over this wave's term(s).
#pragma unroll
        for (int zi = 0; zi < 2 / ZW; ++zi) {
            const int z = ZW == 1 ? zi : wave / KB;
#pragma unroll
            for (int s4 = 0; s4 < kPgSub / 16; ++s4) {
                const bf16x8 a = __builtin_bit_cast(
                    bf16x8, *reinterpret_cast<const u32x4*>(QTs(z) + (kb * 32 + col) * TP + (16 * s4 + 8 * half) * 2));
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                    for (int p = 0; p < 2; ++p) {
                        const bf16x8 b = __builtin_bit_cast(
                            bf16x8, *reinterpret_cast<const u32x4*>(XTs(z, p) + (mb * 32 + col) * TP + (16 * s4 + 8 * half) * 2));
                        accp[mb] = mfma32x32x16(a, b, accp[mb]);
                    }
            }
        }
    }

    // D = 64: the K-term waves hand their partial to the Q-term waves of the same block.
    if (ZW == 2) {
        __syncthreads();
        float* red = reinterpret_cast<float*>(lds);
        if (wave >= KB) {
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int i = 0; i < 16; ++i) red[((kb * MB + mb) * 16 + i) * 64 + lane] = accp[mb][i];
        }
        __syncthreads();
        if (wave < KB) {
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int i = 0; i < 16; ++i) accp[mb][i] += red[((kb * MB + mb) * 16 + i) * 64 + lane];
        }
    }
    if (wave < KB) {
        float* dst = part + ((size_t)bh * nch + ch) * D * m;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            const int c = mb * 32 + col;
            if (c < m) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int k = kb * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
                    dst[(size_t)k * m + c] = accp[mb][i];
                }
            }
        }
    }
}

// dP[h, k, c] = sum over b (ascending) and chunks (ascending) of the partials.
__global__ __launch_bounds__(kThreads) void dp_reduce_kernel(const float* __restrict__ part,
                                                             float* __restrict__ dP, int B,
                                                             int H, int nout, int nch) {
    const int i = blockIdx.x * kThreads + threadIdx.x;
    if (i >= H * nout) return;
    const int h = i / nout, e = i - h * nout;
    // Sixteen loads in flight before their adds (same order of the sums): the partials come
    // from L2 or HBM, and one wave per SIMD cannot hide one latency per add.
    constexpr int U = 16;
    float acc = 0.0f;
    for (int b = 0; b < B; ++b) {
        const float* p = part + ((size_t)(b * H + h) * nch) * nout + e;
        int ch = 0;
        for (; ch + U <= nch; ch += U) {
            float v[U];
#pragma unroll
            for (int u = 0; u < U; ++u) v[u] = p[(size_t)(ch + u) * nout];
#pragma unroll
            for (int u = 0; u < U; ++u) acc += v[u];
        }
        for (; ch < nch; ++ch) acc += p[(size_t)ch * nout];
    }
    dP[i] = acc;
}

template <int MP, int DV, bool CAUSAL>
hipError_t launch_main(const BwdArgs& a, hipStream_t s) {
    const int nqb = (a.N + 127) / 128;
    if (a.fused_dq) {
        // LD and the zeroed dQt come from the preparation launch
        if constexpr (MP <= 64) {
            bwd_kv_kernel<MP, DV, CAUSAL, true><<<dim3(a.BH * nqb), kThreads, 0, s>>>(
                a.Qs, a.Qst, a.Kt, a.V, a.dO, a.dOt, a.LD, a.dV, a.g_f32, a.dKt, a.dQt, a.scale,
                a.N, a.Np, nqb);
            return hipGetLastError();
        } else {
            return hipErrorInvalidValue;
        }
    }
    bwd_q_kernel<MP, DV, CAUSAL><<<dim3(a.BH * nqb), kThreads, 0, s>>>(
        a.Qs, a.Kt, a.Ktt, a.V, a.O, a.dO, a.lse, a.dQt, a.LD, a.N, a.Np, nqb, a.scale);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    bwd_kv_kernel<MP, DV, CAUSAL, false><<<dim3(a.BH * nqb), kThreads, 0, s>>>(
        a.Qs, a.Qst, a.Kt, a.V, a.dO, a.dOt, a.LD, a.dV, a.g_f32, a.dKt, nullptr, a.scale, a.N,
        a.Np, nqb);
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

bool bwd_fuses_dq(int mp, int dv) { return mp <= 64 && (dv == 64 || dv == 128); }

hipError_t launch_attn_bwd_bf16(const BwdArgs& a, hipStream_t stream) {
    if ((long long)a.BH * ((a.N + 127) / 128) > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipError_t e;
    switch (a.mp) {
        case 16: e = launch_dv<16>(a, stream); break;
        case 32: e = launch_dv<32>(a, stream); break;
        case 64: e = launch_dv<64>(a, stream); break;
        case 128: e = launch_dv<128>(a, stream); break;
        default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess) return e;
    // back through the projection
    const int nch = (a.N + kPgRows - 1) / kPgRows;
    const dim3 grid(a.BH * nch);
#define SPA_PG(D_, MP_)                                                                  \
    proj_grad_kernel<D_, MP_><<<grid, kThreads, 0, stream>>>(a.Q, a.K, a.dQt, a.dKt, a.P, \
                                                            a.dQ, a.dK, a.g_f32, a.dPpart, \
                                                            a.N, a.H, a.m, nch)
    if (a.d == 128) {
        if (a.mp == 16) SPA_PG(128, 16);
        else if (a.mp == 32) SPA_PG(128, 32);
        else if (a.mp == 64) SPA_PG(128, 64);
        else SPA_PG(128, 128);
    } else {
        if (a.mp == 16) SPA_PG(64, 16);
        else if (a.mp == 32) SPA_PG(64, 32);
        else if (a.mp == 64) SPA_PG(64, 64);
        else SPA_PG(64, 128);
    }
#undef SPA_PG
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int nout = a.d * a.m;
    dp_reduce_kernel<<<dim3((a.H * nout + kThreads - 1) / kThreads), kThreads, 0, stream>>>(
        a.dPpart, a.dP, a.BH / a.H, a.H, nout, nch);
    return hipGetLastError();
}

}  // namespace spa
