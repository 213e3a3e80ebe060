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
// Work decomposition: a workgroup of 4 waves owns 128 * QB queries of one (batch, head);
// each wave owns QB blocks of 32 of them. QB = 1: two workgroups per CU (two waves per
// SIMD, <= 256 registers each). QB = 2: one workgroup per CU, one wave per SIMD with the
// whole register file; every LDS operand read and every tile copy then serves two query
// blocks (half the LDS and L2 traffic per MFMA). Key tiles of 64 (projected keys, and the
// matching 64 columns of V^T) are copied HBM -> LDS by buffer loads that write LDS directly
// (no registers, no VALU; rows past the end read as zero), double buffered: a copy is
// issued one step before the step that reads it. Per tile, wave and query block:
//   scores^T (64 keys x 32 queries) = Kt_tile . Qt^T on 32x32x16 MFMA. The accumulator starts
//     at -mu (the row's score bound), so the MFMA output is already score - mu; a lane
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
constexpr int kBC = 64;   // keys per tile
constexpr float kTau = 8.0f;

// The query projection folded into the attention launch (one-wave variant): raw queries
// [BH, N, d] (bf16, d in {64, 128}), the projection P [H, d, m] (bf16, m <= MP) and the
// factor the projected queries carry (scale * log2 e). Q == null: the projected queries
// come from Qt instead.
struct QueryFold {
    const uint16_t* Q;
    const uint16_t* P;
    float scale;
    int d, H, m;
};

template <int MP, int DV, bool CAUSAL, int QB>
__global__ __launch_bounds__(kThreads, QB == 1 ? 2 : 1) void attn_bf16_kernel(
    const uint16_t* __restrict__ Qt, const uint16_t* __restrict__ Kt, const bf16_t* __restrict__ Vt,
    const bf16_t* __restrict__ Vrow, const float* __restrict__ kmax, void* __restrict__ O,
    float* __restrict__ lse, int N, int nqb, int out_f32, QueryFold fq) {
    constexpr int kBR = kWaves * 32 * QB;    // queries per workgroup
    constexpr int WQ = 32 * QB;              // queries per wave
    constexpr int KS = MP / 16;              // score MFMA k-steps
    constexpr int KCH = MP / 8;              // 16-byte chunks per projected-key row
    constexpr int K_BYTES = kBC * MP * 2;    // one K tile
    // VDIRECT (QB = 2, DV = 128): V tiles are row-major V as stored, one key per row, and
    // each PV operand is two transposing LDS reads (ds_read_b64_tr_b16). Within a row the
    // 16-byte slots are permuted by an XOR with vxswz(row % 4), so that the four rows one
    // transposing read touches fall on disjoint banks. Otherwise V^T tiles as the
    // preparation launch writes them, each operand one 16-byte read.
    constexpr bool VDIRECT = QB == 2 && DV == 128;
    constexpr int VP = DV * 2;               // VDIRECT: LDS bytes per key row
    constexpr int V_BYTES = VDIRECT ? kBC * VP : kBC * DV * 2;  // one V (or V^T) tile
    constexpr int BUF = K_BYTES + V_BYTES;   // one LDS buffer
    constexpr int KINS = K_BYTES / 1024;     // 64-lane x 16-byte copies per K tile (2 .. 16)
    constexpr int VINS = V_BYTES / 1024;     // ... per V tile (8 or 16)
    constexpr int DB = DV / 32;              // 32-row blocks of V^T / O^T
    static_assert(KINS >= 2 && VINS % kWaves == 0, "tile copy split");
    static_assert(V_BYTES % 1024 == 0, "whole copies per V tile");
    static_assert(QB == 1 || QB == 2, "query blocks per wave");
    // With one wave per SIMD the weight stages (exp, pack, sum) of a pair are spread over
    // consecutive MFMA slots; with two, the other wave fills their latency.
    constexpr bool kSkewWeights = QB != 1;
    // With one wave per SIMD the normaliser of the pipelined steps is summed on the matrix
    // core (16x16x32 MFMAs over the packed weights), off the VALU.
    constexpr bool kNormMfma = QB != 1;

    // Two buffers, each one K tile and one V^T tile, at TWO_BUF (the per-tile loop; for
    // QB = 1 also the pipelined steps). QB = 2 adds rings of three K tiles (at offset 0) and
    // three V^T tiles (at RING_V) ahead of them, so that a pipelined step can read the
    // operands of the next one before its closing barrier, and has four buffers at TWO_BUF
    // (the first two are the per-tile loop's): the tiles with masked keys (at most
    // kBR / kBC), all copied at the start.
    constexpr int NBUF = QB == 1 ? 2 : 7;
    constexpr int RING_V = 3 * K_BYTES;
    constexpr int TWO_BUF = QB == 1 ? 0 : 3 * BUF;
    // QB = 2 with the query projection folded in: P^T (32 rows, d <= 128 columns, rows
    // padded by 16 bytes) after the buffers.
    constexpr int PTP = 136;
    constexpr int PT_BYTES = QB == 2 ? 32 * PTP * 2 : 0;
    __shared__ __attribute__((aligned(16))) char lds[NBUF * BUF + PT_BYTES];

    // Workgroup -> (head, query block). Workgroups are handed to the 8 XCDs round-robin;
    // when the grid divides evenly, XCD x gets a contiguous range of (head, block) pairs so
    // a head's projected keys and values stay in one XCD's L2. Causal blocks run heaviest
    // (last) first: head by head, or, when the range is whole heads whose keys and values
    // fit in the XCD's L2 together, across those heads (every head's heaviest block, then
    // every head's next one, ...), which balances the CUs' loads better.
    const int total = gridDim.x;
    int li = blockIdx.x;
    int bh, qbi;
    if ((total & 7) == 0) {
        const int per_xcd = total >> 3, x = blockIdx.x & 7, j = blockIdx.x >> 3;
        const int hpx = per_xcd / nqb;  // whole heads per XCD (0: not whole heads)
        constexpr long long kRowBytes = MP * 2 + DV * 2;  // projected key + value row
        if (CAUSAL && hpx > 0 && hpx * nqb == per_xcd &&
            (long long)hpx * N * kRowBytes <= (3ll << 20)) {
            bh = x * hpx + j % hpx;
            qbi = j / hpx;
        } else {
            li = x * per_xcd + j;
            bh = li / nqb;
            qbi = li - bh * nqb;
        }
    } else {
        bh = li / nqb;
        qbi = li - bh * nqb;
    }
    const int qb_ = CAUSAL ? (nqb - 1 - qbi) : qbi;
    const int q0 = qb_ * kBR;

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, col = lane & 31, half = lane >> 5;
    const int qw0 = q0 + wave * WQ;
    int myq[QB];
#pragma unroll
    for (int b = 0; b < QB; ++b) myq[b] = qw0 + 32 * b + col;

    const uint16_t* Qh = Qt + (size_t)bh * N * MP;
    const uint16_t* Kh = Kt + (size_t)bh * N * MP;
    const int Np = vt_padded_keys(N);  // row length of V^T
    const bf16_t* Vh = VDIRECT ? Vrow + (size_t)bh * N * DV : Vt + (size_t)bh * DV * Np;

    const int kend = CAUSAL ? min(N, q0 + kBR) : N;
    const int ntiles = (kend + kBC - 1) / kBC;
    // The key-norm maxima of the key blocks this workgroup reads (the first 64 requested
    // before anything else, so their latency overlaps the tile copies').
    const int nkb = proj_blocks(N);
    const int kblocks = (kend + kProjBlockTokens - 1) / kProjBlockTokens;
    float kmx = lane < kblocks ? kmax[(size_t)bh * nkb + lane] : 0.0f;

    // ---- HBM -> LDS tile copy ---------------------------------------------------------
    // Copy j (64 lanes x 16 bytes) fills LDS chunks 64j .. 64j+63 of the tile; lane l writes
    // chunk c = 64j + l, which holds global chunk (c % CH) ^ swizzle(row) of row c / CH (CH
    // chunks per row: MP/8 for a K row, 8 for a V^T row of 64 keys).
    // Copies are dealt round-robin to the waves (wave w issues j = w, w + 4, ...); the
    // global byte offsets are fixed per lane, a tile only moves the descriptor's base.
    constexpr int KPW = (KINS + kWaves - 1) / kWaves;  // K copies per wave (the last may idle)
    constexpr int VPW = (VINS + kWaves - 1) / kWaves;  // V copies per wave (the last may idle)
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
        if constexpr (VDIRECT) {
            // LDS slot c of the tile: key row c / 16, bytes 16 * (c % 16) of that row, which
            // hold the row's bytes at that offset XOR vxswz(row % 4)
            const int row = c >> 4;
            voff[i] = row * VP + ((16 * (c & 15)) ^ vxswz(row & 3));
        } else {
            const int row = c >> 3;  // V column
            voff[i] = row * Np * 2 + 16 * ((c & 7) ^ vtswz(row));
        }
    }
    // LDS byte address of this wave's first copy slot in buffer 0 (wave-uniform; the M0
    // values below are this plus constants).
    const uint32_t lds_wave = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)lds + 1024 * wave);
    // Copies of the K tile at key k0 to LDS byte offset `at`, and of the V^T tile.
    auto copy_k_to = [&](int k0, int at) {
        const u32x4 kr = make_rsrc(Kh + (size_t)k0 * MP, (uint32_t)(N - k0) * MP * 2);
#pragma unroll
        for (int i = 0; i < KPW; ++i) {
            const int j = wave + kWaves * i;
            if (j < KINS) copy16_to_lds(kr, lds_wave + at + 1024 * kWaves * i, koff[i]);
        }
    };
    auto copy_v_to = [&](int k0, int at) {
        const u32x4 vr = VDIRECT ? make_rsrc(Vh + (size_t)k0 * DV, (uint32_t)(N - k0) * DV * 2)
                                 : make_rsrc(Vh + k0, (uint32_t)(DV * Np - k0) * 2);
#pragma unroll
        for (int i = 0; i < VPW; ++i) {
            const int j = wave + kWaves * i;
            if (j < VINS) copy16_to_lds(vr, lds_wave + at + 1024 * kWaves * i, voff[i]);
        }
    };
    auto copy_k = [&](int k0, int buf) { copy_k_to(k0, TWO_BUF + buf * BUF); };
    auto copy_v = [&](int k0, int buf) { copy_v_to(k0, TWO_BUF + buf * BUF + K_BYTES); };
    // Ring slots (QB = 2): tile t's keys at kslot(t % 3), its V^T at vslot(t % 3).
    auto kslot = [](int r) { return r * K_BYTES; };
    auto vslot = [](int r) { return RING_V + r * V_BYTES; };

    // Query projection (QB = 2, raw queries given): this lane's query rows and the
    // workgroup's share of P are requested before the tile copies, which they then overlap.
    // P^T is staged in LDS with its 32 rows permuted by fold_row (an involution), so that
    // the MFMA result lands in the layout of the score MFMA's B operand: lane half h holds
    // rows 4h..4h+3 + 8j, i.e. features 8h..8h+7 (+16 for the second k-step).
    const bool fold = QB == 2 && fq.Q != nullptr;
    auto fold_row = [](int r) {
        const int b4 = r >> 2;
        return 4 * ((b4 & 4) | ((b4 & 1) << 1) | ((b4 >> 1) & 1)) + (r & 3);
    };
    constexpr int XK = QB == 2 ? 8 : 1;  // 16-k-steps over d <= 128
    u32x4 xq[QB][XK];
    u32x4 pvec[2];      // 16-byte vectors of P rows (m a multiple of 8): d*m/8 <= 2 per thread
    uint16_t pel[16];   // otherwise single elements of P^T: 32*d <= 16 per thread
    const int fks = fq.d >> 4;
    const int pvr = fq.m >> 3;  // 16-byte vectors per row of P
    const bool pvecs = (fq.m & 7) == 0;
    const uint16_t* Pf = fq.P + (size_t)(fold ? bh % fq.H : 0) * fq.d * fq.m;
    if constexpr (QB == 2) {
        if (fold) {
            if (pvecs) {
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const int v = tid + kThreads * i;
                    pvec[i] = u32x4{0u, 0u, 0u, 0u};
                    if (v < fq.d * pvr) {
                        const int k = v / pvr, c8 = (v - k * pvr) * 8;
                        pvec[i] = *reinterpret_cast<const u32x4*>(Pf + (size_t)k * fq.m + c8);
                    }
                }
            } else {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int idx = tid + kThreads * i;
                    pel[i] = 0;
                    if (idx < 32 * fq.d) {
                        const int r = idx / fq.d, k = idx - r * fq.d, c = fold_row(r);
                        if (c < fq.m) pel[i] = Pf[(size_t)k * fq.m + c];
                    }
                }
            }
            const uint16_t* Qb = fq.Q + (size_t)bh * N * fq.d;
#pragma unroll
            for (int b = 0; b < QB; ++b)
#pragma unroll
                for (int ks = 0; ks < XK; ++ks) {
                    xq[b][ks] = u32x4{0u, 0u, 0u, 0u};
                    if (ks < fks && myq[b] < N)
                        xq[b][ks] = *reinterpret_cast<const u32x4*>(
                            Qb + (size_t)myq[b] * fq.d + ks * 16 + half * 8);
                }
        }
    }

    // The first tiles' copies go out before anything else is loaded, so their latency
    // overlaps that of the query and key-norm loads below (the fast path starts from tile 0
    // in buffer 0 and, when pipelined, the keys of tile 1 in buffer 1).
    // (At MP = DV = 128 the pipelined loop does not fit the register budget of two
    // workgroups per CU; that shape runs every tile through tile_loop.)
    constexpr bool PIPELINED = !(QB == 1 && MP == 128 && DV == 128);
    // Tiles with no masked key for any query of the workgroup.
    const int nfull = CAUSAL ? min(ntiles, q0 / kBC) : N / kBC;
    // The copies of the ring's first tiles: K and V of tiles 0 and 1, K of tile 2.
    auto copy_ring_start = [&]() {
        if (nfull > 0) {
            copy_k_to(0, kslot(0));
            copy_v_to(0, vslot(0));
        }
        if (nfull > 1) {
            copy_k_to(kBC, kslot(1));
            copy_v_to(kBC, vslot(1));
        }
        if (nfull > 2) copy_k_to(2 * kBC, kslot(2));
    };
    if constexpr (QB == 1) {
        copy_k(0, 0);
        copy_v(0, 0);
        if (PIPELINED && ntiles > 1) copy_k(kBC, 1);
    } else {
        // Every tile with a masked key (buffer d holds tile nfull + d); the ring's first
        // tiles here too when there is none, else once those have landed (below).
        for (int d = 0; d < ntiles - nfull; ++d) {
            copy_k((nfull + d) * kBC, d);
            copy_v((nfull + d) * kBC, d);
        }
        if (ntiles == nfull) copy_ring_start();
    }

    // This lane's queries as the B operand of the score MFMA (zero past N).
    f16x8 qf[QB][KS];
    if (fold) {
        if constexpr (QB == 2) {
            // P^T[r][k] = P[k][fold_row(r)] (zero past m) in LDS; then per query block the
            // projection X~^T = P^T X^T on bf16 MFMA (k-steps in order, one RNE rounding of
            // the scaled result to fp16), as the preparation launch computes it.
            uint16_t* Pt = reinterpret_cast<uint16_t*>(lds + NBUF * BUF);
            if (pvecs) {
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const int v = tid + kThreads * i;
                    if (v >= fq.d * pvr) continue;
                    const int k = v / pvr, c8 = (v - k * pvr) * 8;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        Pt[fold_row(c8 + 2 * j) * PTP + k] = (uint16_t)(pvec[i][j] & 0xffffu);
                        Pt[fold_row(c8 + 2 * j + 1) * PTP + k] = (uint16_t)(pvec[i][j] >> 16);
                    }
                }
                for (int idx = tid; idx < (32 - fq.m) * fq.d; idx += kThreads) {
                    const int c = fq.m + idx / fq.d, k = idx % fq.d;
                    Pt[fold_row(c) * PTP + k] = 0;
                }
            } else {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int idx = tid + kThreads * i;
                    if (idx < 32 * fq.d) {
                        const int r = idx / fq.d, k = idx - r * fq.d;
                        Pt[r * PTP + k] = pel[i];
                    }
                }
            }
            __syncthreads();
#pragma unroll
            for (int b = 0; b < QB; ++b) {
                f32x16 a = f32x16_fill(0.0f);
#pragma unroll
                for (int ks = 0; ks < XK; ++ks) {
                    if (ks >= fks) break;
                    const u32x4 pa = *reinterpret_cast<const u32x4*>(Pt + col * PTP + ks * 16 + half * 8);
                    a = mfma32x32x16(__builtin_bit_cast(bf16x8, pa),
                                     __builtin_bit_cast(bf16x8, xq[b][ks]), a);
                }
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    u32x4 v;
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        v[j] = pack_f16x2(a[8 * ks + 2 * j] * fq.scale, a[8 * ks + 2 * j + 1] * fq.scale);
                    qf[b][ks] = __builtin_bit_cast(f16x8, v);
                }
            }
        }
    } else {
#pragma unroll
        for (int b = 0; b < QB; ++b)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                u32x4 v = {0u, 0u, 0u, 0u};
                if (myq[b] < N)
                    v = *reinterpret_cast<const u32x4*>(Qh + (size_t)myq[b] * MP + ks * 16 + half * 8);
                qf[b][ks] = __builtin_bit_cast(f16x8, v);
            }
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
    // VDIRECT operand reads: lane l of 16-lane group (half, gc) addresses key row
    // r = 4*half + (l & 15) / 4 and columns 16*gc + 4*(l & 3) .. +3 of V block db, i.e. row
    // bytes (64*db + 32*gc + 8*(l & 3)) ^ vxswz(r % 4) = vdir[db]; the step's rows (multiples
    // of 8, so r % 4 is the lane's) are added as immediates.
    int vdir[DB];
    {
        const int r = 4 * half + ((lane & 15) >> 2);
        const int cb = 32 * ((lane >> 4) & 1) + 8 * (lane & 3);
#pragma unroll
        for (int db = 0; db < DB; ++db) vdir[db] = r * VP + ((64 * db + cb) ^ vxswz(r & 3));
    }

    // ---- score bound: M = |q| * max |k| over the key blocks this workgroup reads -------
    {
        for (int b = lane + 64; b < kblocks; b += 64) kmx = fmaxf(kmx, kmax[(size_t)bh * nkb + b]);
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) kmx = fmaxf(kmx, __shfl_xor(kmx, o, 64));
    }
    float bound[QB];
#pragma unroll
    for (int b = 0; b < QB; ++b) {
        float qn2 = 0.0f;  // squared norm of the query as the MFMA sees it (fp16 values)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float v = (float)qf[b][ks][i];
                qn2 += v * v;
            }
        // The slack covers fp16 rounding of the keys and fp32 rounding of norms and sums.
        bound[b] = sqrtf(halves_sum(qn2)) * kmx * (1.0f + 0x1p-8f) + 0x1p-8f;
    }
    // QB = 2: a lane's two queries share one offset (the larger bound), so the pipelined
    // steps need one accumulator start value, not two. Any offset at least the row maximum
    // gives the same softmax; the exact fallback covers an offset that overshoots too far.
    if constexpr (QB == 2) bound[0] = bound[1] = fmaxf(bound[0], bound[1]);

    // ---- per-lane softmax state (queries myq[b]) ----------------------------------------
    f32x16 acc[QB][DB];
    float mu[QB];        // the exponent offset (base-2 units), identical in both half-waves
    float lsum[QB];      // partial normaliser over this half-wave's keys
    f32x16 cinit[QB];    // the score accumulator's start value, -mu
    // Matrix-core normaliser (kNormMfma): lacc[b] rows 0 and 1 of lanes 0-15 hold the sums
    // for queries 32b + lane and 32b + 16 + lane.
    typedef float f32x4_t __attribute__((ext_vector_type(4)));
    f32x4_t lacc[QB];
    bf16x8 lsel;
    {
        const int m = lane & 15, g = lane >> 4;
        const bool one = (m == 0 && (g & 1) == 0) || (m == 1 && (g & 1) == 1);
#pragma unroll
        for (int i = 0; i < 8; ++i) lsel[i] = one ? (__bf16)1.0f : (__bf16)0.0f;
    }

    // Scores^T of one key tile (64 keys x 32 queries per block), minus mu. Each key operand
    // read serves every query block.
    auto scores = [&](const char* Ks, f32x16 (&s)[QB][2]) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int b = 0; b < QB; ++b) s[b][kb] = cinit[b];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const f16x8 a = __builtin_bit_cast(
                    f16x8, *reinterpret_cast<const u32x4*>(Ks + kread[kb][ks]));
#pragma unroll
                for (int b = 0; b < QB; ++b) s[b][kb] = mfma32x32x16(a, qf[b][ks], s[b][kb]);
            }
        }
    };
    // Weights of query block b, k-step tt of key block kb, pair j (keys 2j, 2j+1 of the
    // lane's 8 slots): exp2, rounded to bf16, packed, and added to the normaliser. With a
    // mask, slot i of key block kb (key k0 + kb*32 + 8*(i/4) + 4*half + i%4) is dropped when
    // kb*32 + 8*(i/4) + i%4 > rel, rel being the lane's last admissible key minus
    // k0 + 4*half.
    auto weight_pair = [&](const f32x16 (&s)[QB][2], int b, int kb, int tt, int j, auto masked,
                           int rel) -> uint32_t {
        constexpr bool MASKED = decltype(masked)::value;
        float x0 = s[b][kb][8 * tt + 2 * j], x1 = s[b][kb][8 * tt + 2 * j + 1];
        if constexpr (MASKED) {
            const int i0 = 8 * tt + 2 * j;
            if (kb * 32 + 8 * (i0 >> 2) + (i0 & 3) > rel) x0 = -INFINITY;
            if (kb * 32 + 8 * (i0 >> 2) + (i0 & 3) + 1 > rel) x1 = -INFINITY;
        }
        const float p0 = __builtin_amdgcn_exp2f(x0);
        const float p1 = __builtin_amdgcn_exp2f(x1);
        const uint32_t w = pack_bf16x2(p0, p1);
        lsum[b] = add_bf16x2(w, lsum[b]);
        return w;
    };
    // The exps of one weight pair (as weight_pair), left unpacked.
    auto exp_pair = [&](const f32x16 (&s)[QB][2], int b, int kb, int tt, int j, auto masked,
                        int rel, float (&e)[2]) {
        constexpr bool MASKED = decltype(masked)::value;
        float x0 = s[b][kb][8 * tt + 2 * j], x1 = s[b][kb][8 * tt + 2 * j + 1];
        if constexpr (MASKED) {
            const int i0 = 8 * tt + 2 * j;
            if (kb * 32 + 8 * (i0 >> 2) + (i0 & 3) > rel) x0 = -INFINITY;
            if (kb * 32 + 8 * (i0 >> 2) + (i0 & 3) + 1 > rel) x1 = -INFINITY;
        }
        e[0] = __builtin_amdgcn_exp2f(x0);
        e[1] = __builtin_amdgcn_exp2f(x1);
    };
    // One PV step: O^T block db += V^T_tile(key block kb, k-step tt) . p^T for every query
    // block; the V operand is read once. Slot 8*half + j of k-step tt in key block kb holds
    // key kb*32 + 16*tt + 8*(j/4) + 4*half + j%4, in the score accumulator and in the V^T
    // tile alike.
    // The A operand of PV step (db, kb, tt): 8 keys (in the score accumulator's slot order)
    // of V column db*32 + col. VDIRECT: two transposing reads; in each, a 16-lane group
    // reads 4 key rows x 16 columns and lane i receives column i of the 4 rows.
    auto vop = [&](const char* Vs, int db, int kb, int tt) -> u32x4 {
        if constexpr (VDIRECT) {
            typedef short v4i16 __attribute__((ext_vector_type(4)));
            typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
            const char* base = Vs + vdir[db] + (kb * 32 + 16 * tt) * VP;
            const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_v4i16*)(__attribute__((address_space(3))) char*)(base));
            const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_v4i16*)(__attribute__((address_space(3))) char*)(base + 8 * VP));
            const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
            return u32x4{l2.x, l2.y, h2.x, h2.y};
        } else {
            return *reinterpret_cast<const u32x4*>(Vs + db * 32 * 128 + vread[kb][tt]);
        }
    };
    auto pv_step = [&](const char* Vs, const u32x4 (&p)[QB][2][2], int db, int kb, int tt) {
        const bf16x8 a = __builtin_bit_cast(bf16x8, vop(Vs, db, kb, tt));
#pragma unroll
        for (int b = 0; b < QB; ++b)
            acc[b][db] = mfma32x32x16(a, __builtin_bit_cast(bf16x8, p[b][kb][tt]), acc[b][db]);
    };
    auto pv = [&](const char* Vs, const u32x4 (&p)[QB][2][2]) {
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int tt = 0; tt < 2; ++tt) pv_step(Vs, p, db, kb, tt);
    };
    auto weights = [&](const f32x16 (&s)[QB][2], u32x4 (&p)[QB][2][2]) {
#pragma unroll
        for (int b = 0; b < QB; ++b)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        p[b][kb][tt][j] = weight_pair(s, b, kb, tt, j, std::false_type{}, 0);
    };
    // Order of the PV steps of a tile: V^T block db outermost with one query block (each
    // step's weights stay live to the end of the tile), key block kb outermost with two
    // (the weights of the first key block die halfway, and the next tile's take their
    // registers).
    auto pv_db = [](int v) { return QB == 1 ? v / 4 : v % DB; };
    auto pv_kb = [](int v) { return QB == 1 ? (v >> 1) & 1 : v / (2 * DB); };
    auto pv_tt = [](int v) { return QB == 1 ? v & 1 : (v / DB) & 1; };
    // One pipelined step: scores of the next tile (K tile Kn) and PV of this one (V^T tile
    // Vs, weights p), with the next tile's weights (out pn) computed while the PV MFMAs run.
    // The schedule is fixed explicitly (scheduling fences between slots), since the LDS
    // reads and the MFMA -> exp dependency each take about three MFMA issue slots to come
    // back: all K operands and the first PF V operands are read up front; the score MFMAs
    // follow; the V operand of PV step i + PF is read before PV step i; the weights start
    // WSTART PV MFMAs after the score MFMAs (their inputs are ready by then) and are spread
    // evenly over the remaining PV MFMAs, in the order the score MFMAs completed.
    constexpr int NPV = 4 * DB;      // PV steps (V operands) per tile
    constexpr int PF = QB == 1 ? 4 : 3;  // V operand prefetch distance, in PV steps
    // The score operands of the K tile at Kn, and the first PF V operands of the V^T tile
    // at Vs.
    auto load_ka = [&](const char* Kn, u32x4 (&ka)[2][KS]) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                ka[kb][ks] = *reinterpret_cast<const u32x4*>(Kn + kread[kb][ks]);
    };
    auto vload = [&](const char* Vs, u32x4 (&va)[NPV], int i) {
        va[i] = vop(Vs, pv_db(i), pv_kb(i), pv_tt(i));
    };
    auto load_va_prefix = [&](const char* Vs, u32x4 (&va)[NPV]) {
#pragma unroll
        for (int i = 0; i < PF; ++i) vload(Vs, va, i);
    };
    // The step with the next tile's score operands (ka) and this tile's first PF V operands
    // (va) already in registers.
    // With next_tag true (the ring), the step also reads the next step's operands (key tile
    // Kn, V tile Vn) into ka and va -- the key operands once its own second score block has
    // consumed them, the first V operands in its last PV slots -- so that their LDS latency
    // is hidden behind its MFMAs.
    auto step_core = [&](u32x4 (&ka)[2][KS], u32x4 (&va)[NPV], const char* Vs,
                         const u32x4 (&p)[QB][2][2], u32x4 (&pn)[QB][2][2], auto masked,
                         const int (&rel)[QB], auto next_tag, const char* Kn,
                         const char* Vn) {
        constexpr bool NEXT = decltype(next_tag)::value;
        constexpr int NM = NPV * QB;     // PV MFMAs per tile
        constexpr int WSTART = QB == 1 ? 3 : 2;  // first PV MFMA that weight work follows
        constexpr int NU = 16 * QB;      // weight pairs per tile
        // Weight pair u: key block u / (8 QB), query block (u / 8) % QB, k-step (u / 4) % 2,
        // pair u % 4 -- the order in which the score MFMAs finish. Slot i >= WSTART takes
        // pairs [ulo(i), ulo(i + 1)). With QB = 2 the score MFMAs of key block 1 are issued
        // halfway (SPLIT), once the exps of key block 0 have consumed theirs, so the two
        // blocks' scores share registers; each half then spreads its own pairs.
        constexpr bool SPLIT = QB != 1;
        auto ulo = [&](int i) {
            if constexpr (!SPLIT) {
                constexpr int NW = NM - WSTART;
                return i <= WSTART ? 0 : i >= NM ? NU : (i - WSTART) * NU / NW;
            } else {
                constexpr int H = NM / 2, NU2 = NU / 2, NW2 = H - WSTART;
                if (i >= NM) return NU;
                const int base = (i / H) * NU2, j = i % H;
                return j <= WSTART ? base : base + (j - WSTART) * NU2 / NW2;
            }
        };
        float ex[NU][2];
        f32x16 sn[QB][2];
        auto score_mfmas = [&](int kb) {
            if constexpr (QB == 1) {
                sn[0][kb] = cinit[0];
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    sn[0][kb] = mfma32x32x16(__builtin_bit_cast(f16x8, ka[kb][ks]), qf[0][ks],
                                             sn[0][kb]);
            } else {
                // VGPR-form MFMAs: the exps read these results; the first of them comes
                // at least WSTART PV MFMAs after the last score MFMA of its block.
#pragma unroll
                for (int b = 0; b < QB; ++b)
                    sn[b][kb] = mfma32x32x16_v(__builtin_bit_cast(f16x8, ka[kb][0]), qf[b][0],
                                               cinit[0]);
#pragma unroll
                for (int ks = 1; ks < KS; ++ks)
#pragma unroll
                    for (int b = 0; b < QB; ++b)
                        mfma32x32x16_v_acc(__builtin_bit_cast(f16x8, ka[kb][ks]), qf[b][ks],
                                           sn[b][kb]);
            }
        };
        score_mfmas(0);
        if constexpr (!SPLIT) score_mfmas(1);
        __builtin_amdgcn_sched_barrier(0);  // nothing below moves above the score MFMAs
#pragma unroll
        for (int i = 0; i < NM; ++i) {
            const int v = i / QB, b = i % QB;
            if (SPLIT && i == NM / 2) score_mfmas(1);
            if (b == 0 && v + PF < NPV) vload(Vs, va, v + PF);
            if constexpr (SPLIT && NEXT) {
                if (i == NM / 2 + 1) load_ka(Kn, ka);
                if (b == 0 && v >= NPV - PF) vload(Vn, va, v - (NPV - PF));
            }
            const int db = pv_db(v), kb = pv_kb(v), tt = pv_tt(v);
            acc[b][db] = mfma32x32x16(__builtin_bit_cast(bf16x8, va[v]),
                                      __builtin_bit_cast(bf16x8, p[b][kb][tt]), acc[b][db]);
            if constexpr (!kSkewWeights) {
                if (i >= WSTART) {
#pragma unroll
                    for (int u = ulo(i); u < ulo(i + 1); ++u) {
                        const int ukb = u / (8 * QB), ub = (u / 8) % QB, utt = (u >> 2) & 1,
                                  uj = u & 3;
                        pn[ub][ukb][utt][uj] =
                            weight_pair(sn, ub, ukb, utt, uj, masked, rel[ub]);
                    }
                }
            } else {
                // The weight pairs of this slot are exponentiated here, packed and summed
                // one slot later: with one wave per SIMD nothing else fills the latency of
                // exp -> pack -> sum, so each stage's input comes from the slot before.
                if (i > WSTART) {
#pragma unroll
                    for (int u = ulo(i - 1); u < ulo(i); ++u) {
                        const int ukb = u / (8 * QB), ub = (u / 8) % QB, utt = (u >> 2) & 1,
                                  uj = u & 3;
                        pn[ub][ukb][utt][uj] = pack_bf16x2(ex[u][0], ex[u][1]);
                    }
                }
                if (i >= WSTART) {
#pragma unroll
                    for (int u = ulo(i); u < ulo(i + 1); ++u) {
                        const int ukb = u / (8 * QB), ub = (u / 8) % QB, utt = (u >> 2) & 1,
                                  uj = u & 3;
                        exp_pair(sn, ub, ukb, utt, uj, masked, rel[ub], ex[u]);
                    }
                }
                if (i > WSTART) {
#pragma unroll
                    for (int u = ulo(i - 1); u < ulo(i); ++u) {
                        const int ukb = u / (8 * QB), ub = (u / 8) % QB, utt = (u >> 2) & 1,
                                  uj = u & 3;
                        if constexpr (!kNormMfma) lsum[ub] = add_bf16x2(pn[ub][ukb][utt][uj], lsum[ub]);
                    }
                }
            }
            // Slot fence: the compiler keeps this order (it would otherwise bunch the exps).
            __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (kSkewWeights) {
            // The last slot's pairs: pack and sum.
#pragma unroll
            for (int u = ulo(NM - 1); u < NU; ++u) {
                const int ukb = u / (8 * QB), ub = (u / 8) % QB, utt = (u >> 2) & 1, uj = u & 3;
                pn[ub][ukb][utt][uj] = pack_bf16x2(ex[u][0], ex[u][1]);
                if constexpr (!kNormMfma) lsum[ub] = add_bf16x2(pn[ub][ukb][utt][uj], lsum[ub]);
            }
        }
        // Keep the weights here, beside the MFMAs they overlap: the compiler may otherwise
        // sink the VALU work past a later branch, to their first use in the next step.
#pragma unroll
        for (int b = 0; b < QB; ++b) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int tt = 0; tt < 2; ++tt) asm volatile("" : "+v"(pn[b][kb][tt]));
            asm volatile("" : "+v"(lsum[b]));
        }
        if constexpr (kNormMfma) {
            // The normaliser of the new weights on the matrix core: one 16x16x32 MFMA per
            // 16 keys whose A operand selects, for output row 0 (1), the lanes holding
            // queries 0-15 (16-31) in both half-waves.
#pragma unroll
            for (int b = 0; b < QB; ++b)
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int tt = 0; tt < 2; ++tt)
                        lacc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            lsel, __builtin_bit_cast(bf16x8, pn[b][kb][tt]), lacc[b], 0, 0, 0);
        }
    };
    auto pipelined_step = [&](const char* Kn, const char* Vs, const u32x4 (&p)[QB][2][2],
                              u32x4 (&pn)[QB][2][2], auto masked, const int (&rel)[QB]) {
        u32x4 ka[2][KS], va[NPV];
        load_ka(Kn, ka);
        load_va_prefix(Vs, va);
        step_core(ka, va, Vs, p, pn, masked, rel, std::false_type{}, nullptr, nullptr);
    };
    auto init_state = [&](const float (&mu0)[QB]) {
#pragma unroll
        for (int b = 0; b < QB; ++b) {
#pragma unroll
            for (int db = 0; db < DB; ++db) acc[b][db] = f32x16_fill(0.0f);
            lsum[b] = 0.0f;
            lacc[b] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
            mu[b] = mu0[b];
            cinit[b] = f32x16_fill(-mu[b]);
        }
    };

    // Tiles [t0, ntiles), one at a time: the next tile's copy is issued first; keys past N
    // and after the query (causal) are masked; waves whose queries all precede a tile skip
    // it. The exact variant keeps a lazy running maximum per query.
    auto tile_loop = [&](auto exact_tag, int t0) {
        constexpr bool EXACT = decltype(exact_tag)::value;
#pragma unroll 1
        for (int t = t0; t < ntiles; ++t) {
            const int k0 = t * kBC;
            if (t + 1 < ntiles) {
                copy_k(k0 + kBC, (t + 1) & 1);
                copy_v(k0 + kBC, (t + 1) & 1);
            }
            const char* Ks = lds + TWO_BUF + (t & 1) * BUF;
            const char* Vs = Ks + K_BYTES;

            if (!CAUSAL || k0 <= qw0 + WQ - 1) {
                f32x16 s[QB][2];
                scores(Ks, s);
                const bool edge = (k0 + kBC > N) || (CAUSAL && k0 + kBC - 1 > qw0);
                if (edge) {
#pragma unroll
                    for (int b = 0; b < QB; ++b)
#pragma unroll
                        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                            for (int i = 0; i < 16; ++i) {
                                const int key = k0 + kb * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
                                if (key >= N || (CAUSAL && key > myq[b])) s[b][kb][i] = -INFINITY;
                            }
                }
                if constexpr (EXACT) {
#pragma unroll
                    for (int b = 0; b < QB; ++b) {
                        float tmax = -INFINITY;
#pragma unroll
                        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                            for (int i = 0; i < 16; ++i) tmax = fmaxf(tmax, s[b][kb][i]);
                        tmax = halves_max(tmax);
                        // The first tile sets mu to its maximum (key 0 is unmasked for every
                        // query, so that maximum is finite, and nothing has been accumulated
                        // yet); later tiles move mu only past the kTau slack, rescaling what
                        // was accumulated by 2^-delta <= 1.
                        if (t == 0 || __any(tmax > kTau)) {
                            const float delta = (t == 0) ? tmax : fmaxf(tmax, 0.0f);
                            if (t != 0) {
                                const float alpha = __builtin_amdgcn_exp2f(-delta);
                                lsum[b] *= alpha;
#pragma unroll
                                for (int db = 0; db < DB; ++db)
#pragma unroll
                                    for (int i = 0; i < 16; ++i) acc[b][db][i] *= alpha;
                            }
                            mu[b] += delta;
#pragma unroll
                            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                                for (int i = 0; i < 16; ++i) s[b][kb][i] -= delta;
                            cinit[b] = f32x16_fill(-mu[b]);
                        }
                    }
                }
                u32x4 p[QB][2][2];
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
    // immediate) and no branch around the MFMAs. The steps after it (the causal diagonal,
    // the ragged tail) mask the keys past N and past each query as the weights are formed,
    // and a wave skips the score or PV half of a step whose tile lies wholly after its
    // queries. Returns the number of tiles done (all, or none for the shapes that are not
    // pipelined). The copies of tile 0 (and of tile 1's keys) were issued at the top of the
    // kernel.
    auto fast_phase = [&]() -> int {
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if constexpr (!PIPELINED) {
            return 0;
        } else if constexpr (QB == 1) {
            // The lane's last admissible key per query block (ragged tail, causal diagonal).
            int klim[QB];
#pragma unroll
            for (int b = 0; b < QB; ++b) klim[b] = CAUSAL ? min(myq[b], N - 1) : N - 1;
            auto rel_of = [&](int k0, int (&rel)[QB]) {
#pragma unroll
                for (int b = 0; b < QB; ++b) rel[b] = klim[b] - k0 - 4 * half;
            };
            const int rel0[QB] = {};
            // Does this wave have an admissible key in tile t?
            auto wave_needs = [&](int t) { return !CAUSAL || t * kBC <= qw0 + WQ - 1; };
            u32x4 pa[QB][2][2], pb[QB][2][2];
            {
                f32x16 s[QB][2];
                scores(lds, s);
                if (nfull == 0) {
                    int rel[QB];
                    rel_of(0, rel);
#pragma unroll
                    for (int b = 0; b < QB; ++b)
#pragma unroll
                        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                            for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                                for (int j = 0; j < 4; ++j)
                                    pa[b][kb][tt][j] =
                                        weight_pair(s, b, kb, tt, j, std::true_type{}, rel[b]);
                } else {
                    weights(s, pa);
                }
            }
            __syncthreads();  // K[0] read by every wave before step 0 refills buffer 0
            // Step t of the unmasked loop, weights p of tile t in, pn of tile t+1 out.
            auto step = [&](auto parity, int t, const u32x4 (&p)[QB][2][2],
                            u32x4 (&pn)[QB][2][2]) {
                constexpr int PAR = decltype(parity)::value;
                copy_v((t + 1) * kBC, 1 - PAR);  // t + 1 < nfull <= ntiles
                if (t + 2 < ntiles) copy_k((t + 2) * kBC, PAR);
                pipelined_step(lds + (1 - PAR) * BUF, lds + PAR * BUF + K_BYTES, p, pn,
                               std::false_type{}, rel0);
                // The weights are plain register arithmetic, which the compiler may sink past
                // the barrier to their use in the next step; pin them here, beside the MFMAs
                // they are meant to overlap.
#pragma unroll
                for (int b = 0; b < QB; ++b) {
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                        for (int tt = 0; tt < 2; ++tt) asm volatile("" : "+v"(pn[b][kb][tt]));
                    asm volatile("" : "+v"(lsum[b]));
                }
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
            // The rest, t .. ntiles - 1 (t + 2 >= nfull; the causal diagonal adds at most
            // kBR / kBC tiles), with the buffer parity at run time and tile t's weights
            // always in pa.
#pragma unroll 1
            for (; t + 1 < ntiles; ++t) {
                const int par = t & 1;
                const char* Kn = lds + (1 - par) * BUF;
                const char* Vs = lds + par * BUF + K_BYTES;
                copy_v((t + 1) * kBC, 1 - par);
                if (t + 2 < ntiles) copy_k((t + 2) * kBC, par);
                if (wave_needs(t + 1)) {
                    if (t + 1 < nfull) {
                        pipelined_step(Kn, Vs, pa, pb, std::false_type{}, rel0);
                    } else {
                        int rel[QB];
                        rel_of((t + 1) * kBC, rel);
                        pipelined_step(Kn, Vs, pa, pb, std::true_type{}, rel);
                    }
                } else {
                    if (wave_needs(t)) pv(Vs, pa);
#pragma unroll
                    for (int b = 0; b < QB; ++b)
#pragma unroll
                        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                            for (int tt = 0; tt < 2; ++tt) pb[b][kb][tt] = u32x4{0u, 0u, 0u, 0u};
                }
#pragma unroll
                for (int b = 0; b < QB; ++b)
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                        for (int tt = 0; tt < 2; ++tt) pa[b][kb][tt] = pb[b][kb][tt];
                __builtin_amdgcn_s_waitcnt(0);
                __syncthreads();
            }
            if (wave_needs(t)) pv(lds + (t & 1) * BUF + K_BYTES, pa);
            return ntiles;
        } else {
            // One wave per SIMD: nothing else on the SIMD runs while this wave waits, so
            // every step starts with its operands in registers. Step t copies V[t+2] and
            // K[t+3] (the slots of tiles t-1 and t, both consumed before the last barrier),
            // issues tile t+1's score MFMAs from the key operands in ka and tile t's PV MFMAs
            // from its V^T slot (the first PF operands already in va), and before its closing
            // barrier reads the key operands of tile t+2 and the first V operands of tile
            // t+1 -- tiles whose copies were awaited before an earlier barrier.
            // Only the tiles [0, nfull) with no masked key for the whole workgroup run here (the
            // per-tile loop has done the rest); their first copies were issued at the top.
            const int nf = nfull;
            if (nf == 0) return 0;
            u32x4 pa[QB][2][2], pb[QB][2][2];
            u32x4 ka[2][KS], va[NPV];
            {
                f32x16 s[QB][2];
                scores(lds + kslot(0), s);
                weights(s, pa);
            }
            if (nf > 1) load_ka(lds + kslot(1), ka);
            load_va_prefix(lds + vslot(0), va);
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();  // K[0] read by every wave before step 0 refills its slot
            const int rel0[QB] = {};
            // Step t with ring slot S = t % 3 (a constant in the unrolled loop).
            auto ring_step = [&](int S, int t, const u32x4 (&p)[QB][2][2],
                                 u32x4 (&pn)[QB][2][2]) {
                const int S1 = S == 2 ? 0 : S + 1, S2 = S == 0 ? 2 : S - 1;
                if (t + 3 < nf) copy_k_to((t + 3) * kBC, kslot(S));
                if (t + 2 < nf) copy_v_to((t + 2) * kBC, vslot(S2));
                // (Past the last tile the next operands come from a slot no copy refills:
                // unused values.)
                step_core(ka, va, lds + vslot(S), p, pn, std::false_type{}, rel0,
                          std::true_type{}, lds + kslot(S2), lds + vslot(S1));
                __builtin_amdgcn_s_waitcnt(0);
                __syncthreads();
            };
            int t = 0;
            // Six steps per trip: constant ring slots, and the weights back in pa at the end.
#pragma unroll 1
            for (; t + 6 < nf; t += 6) {
                ring_step(0, t, pa, pb);
                ring_step(1, t + 1, pb, pa);
                ring_step(2, t + 2, pa, pb);
                ring_step(0, t + 3, pb, pa);
                ring_step(1, t + 4, pa, pb);
                ring_step(2, t + 5, pb, pa);
            }
            // The r < 6 steps left start, like every trip, at ring slot 0 with the weights in
            // pa: each keeps its constant slot and weight array; the last tile's PV follows.
            const int r = nf - 1 - t;
            if (r >= 1) ring_step(0, t, pa, pb);
            if (r >= 2) ring_step(1, t + 1, pb, pa);
            if (r >= 3) ring_step(2, t + 2, pa, pb);
            if (r >= 4) ring_step(0, t + 3, pb, pa);
            if (r >= 5) ring_step(1, t + 4, pa, pb);
            switch (r) {
                case 0: pv(lds + vslot(0), pa); break;
                case 1: pv(lds + vslot(1), pb); break;
                case 2: pv(lds + vslot(2), pa); break;
                case 3: pv(lds + vslot(0), pb); break;
                case 4: pv(lds + vslot(1), pa); break;
                default: pv(lds + vslot(2), pb); break;
            }
            return nf;
        }
    };

    init_state(bound);
    if constexpr (QB == 1) {
        tile_loop(std::false_type{}, fast_phase());
    } else {
        // The tiles with masked keys first (the causal diagonal, the ragged tail), one at a
        // time, while the ring's first copies land; then the pipelined ring over the rest.
        // The static offset makes the softmax independent of the tile order. (The queries
        // and key-norm bounds are loaded after the copies of the masked tiles, so waiting
        // for them waits for those copies too; the ring's are issued only now.)
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (ntiles != nfull) copy_ring_start();
        // Tiles are read only here, so no barrier between them: a wave with no admissible
        // key in a tile skips it.
        int klim[QB];
#pragma unroll
        for (int b = 0; b < QB; ++b) klim[b] = CAUSAL ? min(myq[b], N - 1) : N - 1;
#pragma unroll 1
        for (int d = 0; d < ntiles - nfull; ++d) {
            const int t = nfull + d;
            if (CAUSAL && t * kBC > qw0 + WQ - 1) continue;
            const char* Ks = lds + TWO_BUF + d * BUF;
            f32x16 s[QB][2];
            scores(Ks, s);
            u32x4 p[QB][2][2];
#pragma unroll
            for (int b = 0; b < QB; ++b) {
                const int rel = klim[b] - t * kBC - 4 * half;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            p[b][kb][tt][j] = weight_pair(s, b, kb, tt, j, std::true_type{}, rel);
            }
            pv(Ks + K_BYTES, p);
        }
        fast_phase();
    }
    float ltot[QB];
    bool low = false;
#pragma unroll
    for (int b = 0; b < QB; ++b) {
        ltot[b] = halves_sum(lsum[b]);
        if constexpr (kNormMfma) {
            const int src = col & 15;
            const float l0 = __shfl(lacc[b][0], src, 64), l1 = __shfl(lacc[b][1], src, 64);
            ltot[b] += col < 16 ? l0 : l1;
        }
        // A NaN normaliser takes the exact path too: the matrix-core sum multiplies the
        // weights of the query 16 rows away by zero, so a NaN score (from a NaN input) would
        // reach that query's normaliser as well; the exact path sums every row on its own.
        low = low || (myq[b] < N && !(ltot[b] >= 0x1p-64f));
    }
    if (__syncthreads_or(low)) {
        const float zero[QB] = {};
        init_state(zero);
        copy_k(0, 0);
        copy_v(0, 0);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        tile_loop(std::true_type{}, 0);
#pragma unroll
        for (int b = 0; b < QB; ++b) ltot[b] = halves_sum(lsum[b]);
    }

    // ---- epilogue: O = O_acc / l (both half-waves' key subsets summed) ------------------
#pragma unroll
    for (int b = 0; b < QB; ++b) {
        const float inv = 1.0f / ltot[b];
        if (myq[b] < N) {
            const size_t row = (size_t)bh * N + myq[b];
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                if (out_f32) {
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const int c0 = db * 32 + 8 * g + 4 * half;
                        float* dst = static_cast<float*>(O) + row * DV + c0;
                        *reinterpret_cast<float4*>(dst) = make_float4(
                            acc[b][db][4 * g] * inv, acc[b][db][4 * g + 1] * inv,
                            acc[b][db][4 * g + 2] * inv, acc[b][db][4 * g + 3] * inv);
                    }
                } else {
                    // 16-byte stores: of each pair of 8-column groups (g0, g1) the lower
                    // half-wave writes g0 and the upper g1, each taking the partner's four
                    // columns of it
#pragma unroll
                    for (int g0 = 0; g0 < 4; g0 += 2) {
                        u32x2 a, c;
                        a.x = pack_bf16x2(acc[b][db][4 * g0] * inv, acc[b][db][4 * g0 + 1] * inv);
                        a.y = pack_bf16x2(acc[b][db][4 * g0 + 2] * inv, acc[b][db][4 * g0 + 3] * inv);
                        c.x = pack_bf16x2(acc[b][db][4 * g0 + 4] * inv, acc[b][db][4 * g0 + 5] * inv);
                        c.y = pack_bf16x2(acc[b][db][4 * g0 + 6] * inv, acc[b][db][4 * g0 + 7] * inv);
                        const u32x2 send = half ? a : c;
                        u32x2 recv;
                        recv.x = __shfl_xor(send.x, 32, 64);
                        recv.y = __shfl_xor(send.y, 32, 64);
                        const u32x4 v = half ? u32x4{recv.x, recv.y, c.x, c.y}
                                             : u32x4{a.x, a.y, recv.x, recv.y};
                        bf16_t* dst = static_cast<bf16_t*>(O) + row * DV + db * 32 + 8 * (g0 + half);
                        *reinterpret_cast<u32x4*>(dst) = v;
                    }
                }
            }
            if (lse && half == 0) lse[row] = (mu[b] + __log2f(ltot[b])) * 0.69314718055994530942f;
        }
    }
}

// Query blocks per wave: two (one wave per SIMD, every LDS operand read and tile copy shared
// by 64 queries) where the register file holds them and the grid still has several
// workgroups per CU; one otherwise.
inline int pick_qb(int BH, int N, int mp, bool causal) {
    if (mp > 32) return 1;
    const long long wgs2 = (long long)BH * ((N + 255) / 256);
    return wgs2 >= 512 ? 2 : 1;
}

template <int MP, int DV, bool CAUSAL, int QB>
hipError_t launch(const void* Qt, const void* Kt, const void* Vt, const void* Vrow,
                  const float* kmax, void* O, float* lse, int BH, int N, bool out_f32,
                  const QueryFold& fq, hipStream_t stream) {
    constexpr int kBR = kWaves * 32 * QB;
    const int nqb = (N + kBR - 1) / kBR;
    attn_bf16_kernel<MP, DV, CAUSAL, QB><<<dim3(nqb * BH), kThreads, 0, stream>>>(
        static_cast<const uint16_t*>(Qt), static_cast<const uint16_t*>(Kt),
        static_cast<const bf16_t*>(Vt), static_cast<const bf16_t*>(Vrow), kmax, O, lse, N, nqb,
        out_f32 ? 1 : 0, fq);
    return hipGetLastError();
}

template <int MP, int DV>
hipError_t launch_c(const void* Qt, const void* Kt, const void* Vt, const void* Vrow,
                    const float* kmax, void* O, float* lse, int BH, int N, bool causal,
                    bool out_f32, int qb, const QueryFold& fq, hipStream_t stream) {
    if constexpr (MP <= 32) {
        if (qb == 2)
            return causal ? launch<MP, DV, true, 2>(Qt, Kt, Vt, Vrow, kmax, O, lse, BH, N, out_f32, fq, stream)
                          : launch<MP, DV, false, 2>(Qt, Kt, Vt, Vrow, kmax, O, lse, BH, N, out_f32, fq, stream);
    }
    return causal ? launch<MP, DV, true, 1>(Qt, Kt, Vt, Vrow, kmax, O, lse, BH, N, out_f32, fq, stream)
                  : launch<MP, DV, false, 1>(Qt, Kt, Vt, Vrow, kmax, O, lse, BH, N, out_f32, fq, stream);
}

template <int MP>
hipError_t launch_dv(const void* Qt, const void* Kt, const void* Vt, const void* Vrow,
                     const float* kmax, void* O, float* lse, int BH, int N, int dv, bool causal,
                     bool out_f32, int qb, const QueryFold& fq, hipStream_t stream) {
    switch (dv) {
        case 64: return launch_c<MP, 64>(Qt, Kt, Vt, Vrow, kmax, O, lse, BH, N, causal, out_f32, qb, fq, stream);
        case 128: return launch_c<MP, 128>(Qt, Kt, Vt, Vrow, kmax, O, lse, BH, N, causal, out_f32, qb, fq, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

bool attn_bf16_reads_v_rows(int BH, int N, int mp, int dv, bool causal) {
    return pick_qb(BH, N, mp, causal) == 2 && dv == 128;
}

bool attn_bf16_projects_queries(int BH, int N, int mp, int d, bool causal) {
    return pick_qb(BH, N, mp, causal) == 2 && (d == 64 || d == 128);
}

hipError_t launch_attn_bf16(const void* Qt, const void* Kt, const void* Vt, const void* Vrow,
                            const float* kmax, void* O, float* lse, int BH, int N, int mp,
                            int dv, bool causal, bool out_f32, hipStream_t stream, const void* Q,
                            const void* P, float qscale, int d, int H, int m) {
    const int qb = pick_qb(BH, N, mp, causal);
    const QueryFold fq{static_cast<const uint16_t*>(qb == 2 ? Q : nullptr),
                       static_cast<const uint16_t*>(P), qscale, d, H, m};
    switch (mp) {
        case 16: return launch_dv<16>(Qt, Kt, Vt, Vrow, kmax, O, lse, BH, N, dv, causal, out_f32, qb, fq, stream);
        case 32: return launch_dv<32>(Qt, Kt, Vt, Vrow, kmax, O, lse, BH, N, dv, causal, out_f32, qb, fq, stream);
        case 64: return launch_dv<64>(Qt, Kt, Vt, Vrow, kmax, O, lse, BH, N, dv, causal, out_f32, qb, fq, stream);
        case 128: return launch_dv<128>(Qt, Kt, Vt, Vrow, kmax, O, lse, BH, N, dv, causal, out_f32, qb, fq, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace spa
