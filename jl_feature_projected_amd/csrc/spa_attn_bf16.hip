// spa_attn_bf16.hip -- projected softmax attention for bf16 inputs on gfx950 MFMA, streamed
// over key tiles so the N x N score matrix never reaches memory.
//
// What it computes: "Sparse Projection Attention" page, Sec. 3.1.3 and Algorithm 1 steps 4-6
// (scores of projected queries and keys, row softmax, weights times V); "Projection-
// Decomposition Attention (PDA)" page, Algorithm 2.1 steps 2, 3, 5 and Sec. 4.2 (the
// projected score matrix can be streamed instead of stored). The streaming itself (query
// tile x key tile, scores kept on chip and folded at once into an online softmax) follows
// the FlashSFA description in the "Scaling Attention via Feature Sparsity" notes, Key
// design 3, with the dense projected contraction in place of the sparse intersection.
//
// Work decomposition: a workgroup of 4 waves owns 128 queries of one (batch, head); each
// wave owns 32 of them. Key tiles of 64 (projected keys, and the matching 64 columns of
// V^T) are copied HBM -> LDS by buffer loads that write LDS directly (no registers, no VALU;
// rows past the end read as zero), double buffered: a copy is issued one step before the
// step that reads it. Per tile and wave:
//   scores^T (64 keys x 32 queries) = Kt_tile . Qt^T on 32x32x16 MFMA. The accumulator starts
//     at -mu (the running row maximum), so the MFMA output is already score - mu; a lane
//     owns one query and 16 keys per 32-key block, so row reductions are in-lane plus one
//     exchange with lane l xor 32.
//   softmax without a running maximum: by Cauchy-Schwarz every score of a row is at most
//     M = |q_i| * max_j |k_j| (the key norm maxima come from the projection launch), so the
//     accumulator starts at -M and exp2 of the MFMA output is a weight in (0, 1]: no max,
//     no cross-lane exchange, no rescale, no branch in the tile loop. If M overshoots a
//     row's true maximum so far that its normaliser falls below 2^-64 (weights would start
//     to underflow), the whole workgroup recomputes its rows with an exact online softmax
//     (lazy: the running maximum only moves when a tile exceeds it by more than kTau base-2
//     units, rescaling what was accumulated).
//   O^T (dv x 32 queries) += V^T_tile . p^T on 32x32x16 MFMA. The weights p go from the
//     score accumulator straight into the B operand: the k-order of the contraction is the
//     key order the score layout already has. V arrives transposed (a separate launch
//     writes V^T with the keys of each 16-key group in that same order), so each A operand
//     is one 16-byte LDS read: 8 keys of one V column.
// LDS tiles are XOR-swizzled in 16-byte chunks (the copy picks, per lane, which global chunk
// lands in its LDS slot), so no read of the score or PV operands hits a bank twice.
// Queries arrive pre-scaled by scale*log2(e), so exp2 of the MFMA output is the softmax
// numerator. The projected queries and keys are fp16 (the score MFMA runs in fp16, whose
// 11-bit significand keeps the score error small); V and the weights are bf16. The
// normaliser is summed from the bf16-rounded weights, the same values the PV MFMA consumes.
#include <type_traits>

#include "spa_device.h"
#include "spa_internal.h"

namespace spa {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kBR = 128;  // queries per workgroup (4 waves x 32)
constexpr int kBC = 64;   // keys per tile
constexpr float kTau = 8.0f;

template <int MP, int DV, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void attn_bf16_kernel(
    const uint16_t* __restrict__ Qt, const uint16_t* __restrict__ Kt, const bf16_t* __restrict__ Vt,
    const float* __restrict__ kmax, void* __restrict__ O, float* __restrict__ lse, int N, int nqb,
    int out_f32) {
    constexpr int KS = MP / 16;              // score MFMA k-steps
    constexpr int KCH = MP / 8;              // 16-byte chunks per projected-key row
    constexpr int K_BYTES = kBC * MP * 2;    // one K tile
    constexpr int V_BYTES = kBC * DV * 2;    // one V^T tile (DV rows of 64 keys)
    constexpr int BUF = K_BYTES + V_BYTES;   // one LDS buffer
    constexpr int KINS = K_BYTES / 1024;     // 64-lane x 16-byte copies per K tile (2 .. 16)
    constexpr int VINS = V_BYTES / 1024;     // ... per V tile (8 or 16)
    constexpr int DB = DV / 32;              // 32-row blocks of V^T / O^T
    static_assert(KINS >= 2 && VINS % kWaves == 0, "tile copy split");

    __shared__ __attribute__((aligned(16))) char lds[2 * BUF];

    // Workgroup -> (head, query block). Workgroups are handed to the 8 XCDs round-robin;
    // when the grid divides evenly, XCD x gets a contiguous range of (head, block) pairs so
    // a head's projected keys and values stay in one XCD's L2. Causal blocks run heaviest
    // (last) first.
    const int total = gridDim.x;
    int li = blockIdx.x;
    if ((total & 7) == 0) li = (blockIdx.x & 7) * (total >> 3) + (blockIdx.x >> 3);
    const int bh = li / nqb;
    const int qbi = li - bh * nqb;
    const int qb = CAUSAL ? (nqb - 1 - qbi) : qbi;
    const int q0 = qb * kBR;

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, col = lane & 31, half = lane >> 5;
    const int qw0 = q0 + wave * 32;
    const int myq = qw0 + col;

    const uint16_t* Qh = Qt + (size_t)bh * N * MP;
    const uint16_t* Kh = Kt + (size_t)bh * N * MP;
    const int Np = vt_padded_keys(N);  // row length of V^T
    const bf16_t* Vh = Vt + (size_t)bh * DV * Np;

    const int kend = CAUSAL ? min(N, q0 + kBR) : N;
    const int ntiles = (kend + kBC - 1) / kBC;

    // ---- HBM -> LDS tile copy ---------------------------------------------------------
    // Copy j (64 lanes x 16 bytes) fills LDS chunks 64j .. 64j+63 of the tile; lane l writes
    // chunk c = 64j + l, which holds global chunk (c % CH) ^ swizzle(row) of row c / CH (CH
    // chunks per row: MP/8 for a K row, 8 for a V^T row of 64 keys).
    // Copies are dealt round-robin to the waves (wave w issues j = w, w + 4, ...); the
    // global byte offsets are fixed per lane, a tile only moves the descriptor's base.
    constexpr int KPW = (KINS + kWaves - 1) / kWaves;  // K copies per wave (the last may idle)
    constexpr int VPW = VINS / kWaves;                 // V copies per wave
    uint32_t koff[KPW], voff[VPW];
#pragma unroll
    for (int i = 0; i < KPW; ++i) {
        const int c = 64 * (wave + kWaves * i) + lane;
        const int row = c / KCH;
        koff[i] = row * MP * 2 + 16 * ((c % KCH) ^ kswz<MP>(row));
    }
#pragma unroll
    for (int i = 0; i < VPW; ++i) {
        const int c = 64 * (wave + kWaves * i) + lane;
        const int row = c >> 3;  // V column
        voff[i] = row * Np * 2 + 16 * ((c & 7) ^ vtswz(row));
    }
    // LDS byte address of this wave's first copy slot in buffer 0 (wave-uniform; the M0
    // values below are this plus constants).
    const uint32_t lds_wave = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)lds + 1024 * wave);
    auto copy_k = [&](int k0, int buf) {
        const u32x4 kr = make_rsrc(Kh + (size_t)k0 * MP, (uint32_t)(N - k0) * MP * 2);
#pragma unroll
        for (int i = 0; i < KPW; ++i) {
            const int j = wave + kWaves * i;
            if (j < KINS) copy16_to_lds(kr, lds_wave + buf * BUF + 1024 * kWaves * i, koff[i]);
        }
    };
    auto copy_v = [&](int k0, int buf) {
        const u32x4 vr = make_rsrc(Vh + k0, (uint32_t)(DV * Np - k0) * 2);
#pragma unroll
        for (int i = 0; i < VPW; ++i)
            copy16_to_lds(vr, lds_wave + buf * BUF + K_BYTES + 1024 * kWaves * i, voff[i]);
    };

    // The first tiles' copies go out before anything else is loaded, so their latency
    // overlaps that of the query and key-norm loads below (the fast path starts from tile 0
    // in buffer 0 and, when pipelined, the keys of tile 1 in buffer 1).
    // (At MP = DV = 128 the pipelined loop does not fit the register budget of two
    // workgroups per CU; that shape runs every tile through tile_loop.)
    constexpr bool PIPELINED = !(MP == 128 && DV == 128);
    // Tiles with no masked key for any query of the workgroup.
    const int nfull = CAUSAL ? min(ntiles, q0 / kBC) : N / kBC;
    copy_k(0, 0);
    copy_v(0, 0);
    if (PIPELINED && ntiles > 1) copy_k(kBC, 1);

    // This lane's query as the B operand of the score MFMA (zero past N).
    f16x8 qf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        u32x4 v = {0u, 0u, 0u, 0u};
        if (myq < N) v = *reinterpret_cast<const u32x4*>(Qh + (size_t)myq * MP + ks * 16 + half * 8);
        qf[ks] = __builtin_bit_cast(f16x8, v);
    }

    // Per-lane LDS read offsets, fixed across tiles.
    // Score operand: key row kb*32 + col, global chunk 2*ks + half.
    int kread[2][KS];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int row = kb * 32 + col;
            kread[kb][ks] = row * MP * 2 + 16 * ((2 * ks + half) ^ kswz<MP>(row));
        }
    // PV operand: V^T row db*32 + col (a V column), 16-byte chunk 4*kb + 2*tt + half (keys
    // kb*32 + 16*tt + {4*half .. 4*half+3, 8+4*half .. 8+4*half+3}, in the slot order of the
    // score accumulator). The swizzle of row db*32 + col does not depend on db.
    int vread[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
            vread[kb][tt] = col * 128 + 16 * ((4 * kb + 2 * tt + half) ^ vtswz(col));

    // ---- score bound: M = |q| * max |k| over the key blocks this workgroup reads -------
    float kmx = 0.0f;
    {
        const int nkb = proj_blocks(N);
        const int kblocks = (kend + kProjBlockTokens - 1) / kProjBlockTokens;
        for (int b = lane; b < kblocks; b += 64) kmx = fmaxf(kmx, kmax[(size_t)bh * nkb + b]);
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) kmx = fmaxf(kmx, __shfl_xor(kmx, o, 64));
    }
    float qn2 = 0.0f;  // squared norm of the query as the MFMA sees it (fp16 values)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float v = (float)qf[ks][i];
            qn2 += v * v;
        }
    // The slack covers fp16 rounding of the keys and fp32 rounding of norms and sums.
    const float bound = sqrtf(halves_sum(qn2)) * kmx * (1.0f + 0x1p-8f) + 0x1p-8f;

    // ---- per-lane softmax state (query myq) --------------------------------------------
    f32x16 acc[DB];
    float mu;        // the exponent offset (base-2 units), identical in both half-waves
    float lsum;      // partial normaliser over this half-wave's keys
    f32x16 cinit;    // the score accumulator's start value, -mu

    // Scores^T of one key tile (64 keys x this wave's 32 queries), minus mu.
    auto scores = [&](const char* Ks, f32x16 (&s)[2]) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            s[kb] = cinit;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const f16x8 a = __builtin_bit_cast(
                    f16x8, *reinterpret_cast<const u32x4*>(Ks + kread[kb][ks]));
                s[kb] = mfma32x32x16(a, qf[ks], s[kb]);
            }
        }
    };
    // Weights of k-step tt of key block kb, pair j (keys 2j, 2j+1 of the lane's 8 slots):
    // exp2, rounded to bf16, packed, and added to the normaliser. With a mask, slot i of
    // key block kb (key k0 + kb*32 + 8*(i/4) + 4*half + i%4) is dropped when kb*32 + 8*(i/4)
    // + i%4 > rel, rel being the lane's last admissible key minus k0 + 4*half.
    auto weight_pair = [&](const f32x16 (&s)[2], int kb, int tt, int j, auto masked,
                           int rel) -> uint32_t {
        constexpr bool MASKED = decltype(masked)::value;
        float x0 = s[kb][8 * tt + 2 * j], x1 = s[kb][8 * tt + 2 * j + 1];
        if constexpr (MASKED) {
            const int i0 = 8 * tt + 2 * j;
            if (kb * 32 + 8 * (i0 >> 2) + (i0 & 3) > rel) x0 = -INFINITY;
            if (kb * 32 + 8 * (i0 >> 2) + (i0 & 3) + 1 > rel) x1 = -INFINITY;
        }
        const float p0 = __builtin_amdgcn_exp2f(x0);
        const float p1 = __builtin_amdgcn_exp2f(x1);
        const uint32_t w = pack_bf16x2(p0, p1);
        lsum = add_bf16x2(w, lsum);
        return w;
    };
    // One PV MFMA: O^T block db += V^T_tile(key block kb, k-step tt) . p^T. Slot 8*half + j
    // of k-step tt in key block kb holds key kb*32 + 16*tt + 8*(j/4) + 4*half + j%4, in the
    // score accumulator and in the V^T tile alike.
    auto pv_step = [&](const char* Vs, const u32x4 (&p)[2][2], int db, int kb, int tt) {
        const bf16x8 a = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const u32x4*>(Vs + db * 32 * 128 + vread[kb][tt]));
        acc[db] = mfma32x32x16(a, __builtin_bit_cast(bf16x8, p[kb][tt]), acc[db]);
    };
    auto pv = [&](const char* Vs, const u32x4 (&p)[2][2]) {
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int tt = 0; tt < 2; ++tt) pv_step(Vs, p, db, kb, tt);
    };
    auto weights = [&](const f32x16 (&s)[2], u32x4 (&p)[2][2]) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    p[kb][tt][j] = weight_pair(s, kb, tt, j, std::false_type{}, 0);
    };
    // One pipelined step: scores of the next tile (K tile Kn) and PV of this one (V^T tile
    // Vs, weights p), with the next tile's weights (out pn) computed while the PV MFMAs run.
    // The schedule is fixed explicitly (scheduling fences between slots), since the LDS
    // reads and the MFMA -> exp dependency each take about three MFMA issue slots to come
    // back: all K operands and the first PF V operands are read up front; the score MFMAs
    // follow; PV MFMA i is preceded by the read of V operand i + PF; the weights start
    // WSTART PV MFMAs after the score MFMAs (their inputs are ready by then) and are spread
    // evenly over the remaining PV MFMAs.
    auto pipelined_step = [&](const char* Kn, const char* Vs, const u32x4 (&p)[2][2],
                              u32x4 (&pn)[2][2], auto masked, int rel) {
        constexpr int NPV = 4 * DB;  // PV MFMAs per tile
        constexpr int PF = 4;        // V operand prefetch distance, in MFMAs
        constexpr int WSTART = 3;    // first PV MFMA that weight work is placed after
        constexpr int NW = NPV - WSTART;
        u32x4 ka[2][KS];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                ka[kb][ks] = *reinterpret_cast<const u32x4*>(Kn + kread[kb][ks]);
        u32x4 va[NPV];
        auto vload = [&](int i) {
            const int db = i / 4, kb = (i >> 1) & 1, tt = i & 1;
            va[i] = *reinterpret_cast<const u32x4*>(Vs + db * 32 * 128 + vread[kb][tt]);
        };
#pragma unroll
        for (int i = 0; i < PF; ++i) vload(i);
        f32x16 sn[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            sn[kb] = cinit;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                sn[kb] = mfma32x32x16(__builtin_bit_cast(f16x8, ka[kb][ks]), qf[ks], sn[kb]);
        }
        __builtin_amdgcn_sched_barrier(0);  // nothing below moves above the score MFMAs
#pragma unroll
        for (int i = 0; i < NPV; ++i) {
            if (i + PF < NPV) vload(i + PF);
            const int db = i / 4, kb = (i >> 1) & 1, tt = i & 1;
            acc[db] = mfma32x32x16(__builtin_bit_cast(bf16x8, va[i]),
                                   __builtin_bit_cast(bf16x8, p[kb][tt]), acc[db]);
            if (i >= WSTART) {
#pragma unroll
                for (int u = (i - WSTART) * 16 / NW; u < (i - WSTART + 1) * 16 / NW; ++u)
                    pn[u >> 3][(u >> 2) & 1][u & 3] =
                        weight_pair(sn, u >> 3, (u >> 2) & 1, u & 3, masked, rel);
            }
            // Slot fence: the compiler keeps this order (it would otherwise bunch the exps).
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    auto init_state = [&](float mu0) {
#pragma unroll
        for (int db = 0; db < DB; ++db) acc[db] = f32x16_fill(0.0f);
        lsum = 0.0f;
        mu = mu0;
        cinit = f32x16_fill(-mu);
    };

    // Tiles [t0, ntiles), one at a time: the next tile's copy is issued first; keys past N
    // and after the query (causal) are masked; waves whose queries all precede a tile skip
    // it. The exact variant keeps a lazy running maximum.
    auto tile_loop = [&](auto exact_tag, int t0) {
        constexpr bool EXACT = decltype(exact_tag)::value;
#pragma unroll 1
        for (int t = t0; t < ntiles; ++t) {
            const int k0 = t * kBC;
            if (t + 1 < ntiles) {
                copy_k(k0 + kBC, (t + 1) & 1);
                copy_v(k0 + kBC, (t + 1) & 1);
            }
            const char* Ks = lds + (t & 1) * BUF;
            const char* Vs = Ks + K_BYTES;

            if (!CAUSAL || k0 <= qw0 + 31) {
                f32x16 s[2];
                scores(Ks, s);
                const bool edge = (k0 + kBC > N) || (CAUSAL && k0 + kBC - 1 > qw0);
                if (edge) {
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                        for (int i = 0; i < 16; ++i) {
                            const int key = k0 + kb * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
                            if (key >= N || (CAUSAL && key > myq)) s[kb][i] = -INFINITY;
                        }
                }
                if constexpr (EXACT) {
                    float tmax = -INFINITY;
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                        for (int i = 0; i < 16; ++i) tmax = fmaxf(tmax, s[kb][i]);
                    tmax = halves_max(tmax);
                    // The first tile sets mu to its maximum (key 0 is unmasked for every
                    // query, so that maximum is finite, and nothing has been accumulated
                    // yet); later tiles move mu only past the kTau slack, rescaling what was
                    // accumulated by 2^-delta <= 1.
                    if (t == 0 || __any(tmax > kTau)) {
                        const float delta = (t == 0) ? tmax : fmaxf(tmax, 0.0f);
                        if (t != 0) {
                            const float alpha = __builtin_amdgcn_exp2f(-delta);
                            lsum *= alpha;
#pragma unroll
                            for (int db = 0; db < DB; ++db)
#pragma unroll
                                for (int i = 0; i < 16; ++i) acc[db][i] *= alpha;
                        }
                        mu += delta;
#pragma unroll
                        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                            for (int i = 0; i < 16; ++i) s[kb][i] -= delta;
                        cinit = f32x16_fill(-mu);
                    }
                }
                u32x4 p[2][2];
                weights(s, p);
                pv(Vs, p);
            }
            // This wave's copies into the other buffer are done, and (barrier) everyone's
            // are, and everyone has finished reading this buffer.
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
        }
    };

    // Fast path (every tile when the shape is pipelined): the score MFMAs of tile t+1 are
    // issued, then the PV MFMAs of tile t run while the wave computes tile t+1's weights. K
    // and V copies are issued separately, each one step before the step that reads it:
    //   step t reads K[t+1] (buffer (t+1)&1) and V[t] (buffer t&1), and copies V[t+1] into
    //   buffer (t+1)&1 and K[t+2] into buffer t&1.
    // Tiles [0, nfull) have no masked key for any query of the workgroup; their steps run in
    // a loop of two steps with the buffer parity as a template constant (every LDS offset an
    // immediate) and no branch around the MFMAs. The at most three steps after it mask the
    // keys past N and past each query (causal) as the weights are formed, and a wave skips
    // the score or PV half of a step whose tile lies wholly after its queries. Returns the
    // number of tiles done (all, or none for the shapes that are not pipelined). The copies
    // of tile 0 (and of tile 1's keys) were issued at the top of the kernel.
    auto fast_phase = [&]() -> int {
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if constexpr (!PIPELINED) {
            return 0;
        } else {
            // The lane's last admissible key (ragged tail, causal diagonal).
            const int klim = CAUSAL ? min(myq, N - 1) : N - 1;
            auto rel_of = [&](int k0) { return klim - k0 - 4 * half; };
            // Does this wave have an admissible key in tile t?
            auto wave_needs = [&](int t) { return !CAUSAL || t * kBC <= qw0 + 31; };
            u32x4 pa[2][2], pb[2][2];
            {
                f32x16 s[2];
                scores(lds, s);
                if (nfull == 0) {
                    const int rel = rel_of(0);
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                            for (int j = 0; j < 4; ++j)
                                pa[kb][tt][j] = weight_pair(s, kb, tt, j, std::true_type{}, rel);
                } else {
                    weights(s, pa);
                }
            }
            __syncthreads();  // K[0] read by every wave before step 0 refills buffer 0
            // Step t of the unmasked loop, weights p of tile t in, pn of tile t+1 out.
            auto step = [&](auto parity, int t, const u32x4 (&p)[2][2], u32x4 (&pn)[2][2]) {
                constexpr int PAR = decltype(parity)::value;
                copy_v((t + 1) * kBC, 1 - PAR);  // t + 1 < nfull <= ntiles
                if (t + 2 < ntiles) copy_k((t + 2) * kBC, PAR);
                pipelined_step(lds + (1 - PAR) * BUF, lds + PAR * BUF + K_BYTES, p, pn,
                               std::false_type{}, 0);
                // The weights are plain register arithmetic, which the compiler may sink past
                // the barrier to their use in the next step; pin them here, beside the MFMAs
                // they are meant to overlap.
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int tt = 0; tt < 2; ++tt) asm volatile("" : "+v"(pn[kb][tt]));
                asm volatile("" : "+v"(lsum));
                __builtin_amdgcn_s_waitcnt(0);
                __syncthreads();
            };
            using P0 = std::integral_constant<int, 0>;
            using P1 = std::integral_constant<int, 1>;
            int t = 0;
#pragma unroll 1
            for (; t + 2 < nfull; t += 2) {
                step(P0{}, t, pa, pb);
                step(P1{}, t + 1, pb, pa);
            }
            // The rest, t .. ntiles - 1 (at most three steps and the last PV: t + 2 >= nfull,
            // ntiles <= nfull + 2), with the buffer parity at run time and tile t's weights
            // always in pa.
#pragma unroll 1
            for (; t + 1 < ntiles; ++t) {
                const int par = t & 1;
                const char* Kn = lds + (1 - par) * BUF;
                const char* Vs = lds + par * BUF + K_BYTES;
                copy_v((t + 1) * kBC, 1 - par);
                if (t + 2 < ntiles) copy_k((t + 2) * kBC, par);
                if (wave_needs(t + 1)) {
                    if (t + 1 < nfull)
                        pipelined_step(Kn, Vs, pa, pb, std::false_type{}, 0);
                    else
                        pipelined_step(Kn, Vs, pa, pb, std::true_type{}, rel_of((t + 1) * kBC));
                } else {
                    if (wave_needs(t)) pv(Vs, pa);
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                        for (int tt = 0; tt < 2; ++tt) pb[kb][tt] = u32x4{0u, 0u, 0u, 0u};
                }
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int tt = 0; tt < 2; ++tt) pa[kb][tt] = pb[kb][tt];
                __builtin_amdgcn_s_waitcnt(0);
                __syncthreads();
            }
            if (wave_needs(t)) pv(lds + (t & 1) * BUF + K_BYTES, pa);
            return ntiles;
        }
    };

    init_state(bound);
    tile_loop(std::false_type{}, fast_phase());
    float ltot = halves_sum(lsum);
    if (__syncthreads_or(myq < N && ltot < 0x1p-64f)) {
        init_state(0.0f);
        copy_k(0, 0);
        copy_v(0, 0);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        tile_loop(std::true_type{}, 0);
        ltot = halves_sum(lsum);
    }

    // ---- epilogue: O = O_acc / l (both half-waves' key subsets summed) ------------------
    const float inv = 1.0f / ltot;
    if (myq < N) {
        const size_t row = (size_t)bh * N + myq;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            if (out_f32) {
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int c0 = db * 32 + 8 * g + 4 * half;
                    float* dst = static_cast<float*>(O) + row * DV + c0;
                    *reinterpret_cast<float4*>(dst) =
                        make_float4(acc[db][4 * g] * inv, acc[db][4 * g + 1] * inv,
                                    acc[db][4 * g + 2] * inv, acc[db][4 * g + 3] * inv);
                }
            } else {
                // 16-byte stores: of each pair of 8-column groups (g0, g1) the lower half-wave
                // writes g0 and the upper g1, each taking the partner's four columns of it
#pragma unroll
                for (int g0 = 0; g0 < 4; g0 += 2) {
                    u32x2 a, b;
                    a.x = pack_bf16x2(acc[db][4 * g0] * inv, acc[db][4 * g0 + 1] * inv);
                    a.y = pack_bf16x2(acc[db][4 * g0 + 2] * inv, acc[db][4 * g0 + 3] * inv);
                    b.x = pack_bf16x2(acc[db][4 * g0 + 4] * inv, acc[db][4 * g0 + 5] * inv);
                    b.y = pack_bf16x2(acc[db][4 * g0 + 6] * inv, acc[db][4 * g0 + 7] * inv);
                    const u32x2 send = half ? a : b;
                    u32x2 recv;
                    recv.x = __shfl_xor(send.x, 32, 64);
                    recv.y = __shfl_xor(send.y, 32, 64);
                    const u32x4 v = half ? u32x4{recv.x, recv.y, b.x, b.y} : u32x4{a.x, a.y, recv.x, recv.y};
                    bf16_t* dst = static_cast<bf16_t*>(O) + row * DV + db * 32 + 8 * (g0 + half);
                    *reinterpret_cast<u32x4*>(dst) = v;
                }
            }
        }
        if (lse && half == 0) lse[row] = (mu + __log2f(ltot)) * 0.69314718055994530942f;
    }
}

template <int MP, int DV, bool CAUSAL>
hipError_t launch(const void* Qt, const void* Kt, const void* Vt, const float* kmax, void* O,
                  float* lse, int BH, int N, bool out_f32, hipStream_t stream) {
    const int nqb = (N + kBR - 1) / kBR;
    attn_bf16_kernel<MP, DV, CAUSAL><<<dim3(nqb * BH), kThreads, 0, stream>>>(
        static_cast<const uint16_t*>(Qt), static_cast<const uint16_t*>(Kt),
        static_cast<const bf16_t*>(Vt), kmax, O, lse, N, nqb, out_f32 ? 1 : 0);
    return hipGetLastError();
}

template <int MP, int DV>
hipError_t launch_c(const void* Qt, const void* Kt, const void* V, const float* kmax, void* O,
                    float* lse, int BH, int N, bool causal, bool out_f32, hipStream_t stream) {
    return causal ? launch<MP, DV, true>(Qt, Kt, V, kmax, O, lse, BH, N, out_f32, stream)
                  : launch<MP, DV, false>(Qt, Kt, V, kmax, O, lse, BH, N, out_f32, stream);
}

template <int MP>
hipError_t launch_dv(const void* Qt, const void* Kt, const void* V, const float* kmax, void* O,
                     float* lse, int BH, int N, int dv, bool causal, bool out_f32,
                     hipStream_t stream) {
    switch (dv) {
        case 64: return launch_c<MP, 64>(Qt, Kt, V, kmax, O, lse, BH, N, causal, out_f32, stream);
        case 128: return launch_c<MP, 128>(Qt, Kt, V, kmax, O, lse, BH, N, causal, out_f32, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_attn_bf16(const void* Qt, const void* Kt, const void* V, const float* kmax,
                            void* O, float* lse, int BH, int N, int mp, int dv, bool causal,
                            bool out_f32, hipStream_t stream) {
    switch (mp) {
        case 16: return launch_dv<16>(Qt, Kt, V, kmax, O, lse, BH, N, dv, causal, out_f32, stream);
        case 32: return launch_dv<32>(Qt, Kt, V, kmax, O, lse, BH, N, dv, causal, out_f32, stream);
        case 64: return launch_dv<64>(Qt, Kt, V, kmax, O, lse, BH, N, dv, causal, out_f32, stream);
        case 128: return launch_dv<128>(Qt, Kt, V, kmax, O, lse, BH, N, dv, causal, out_f32, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace spa
