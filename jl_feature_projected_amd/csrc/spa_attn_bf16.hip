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
// wave owns 32 of them. Key tiles of 64 are staged in LDS (projected keys as rows, V
// transposed), double buffered, with the next tile's global loads issued before the current
// tile's math. Per tile and wave:
//   scores^T (64 keys x 32 queries) = Kt_tile . Qt^T on 32x32x16 MFMA. The accumulator starts
//     at -mu (the running row maximum), so the MFMA output is already score - mu; a lane
//     owns one query and 16 keys per 32-key block, so row reductions are in-lane plus one
//     exchange with lane l xor 32.
//   lazy online softmax: mu only moves when a tile's maximum exceeds it by more than kTau
//     (base-2 units), which keeps every weight below 2^kTau; all else is exp2 on the VALU.
//   O^T (dv x 32 queries) += V^T_tile . p^T on 32x32x16 MFMA. The weights p go from the
//     score accumulator straight into the B operand: the k-order of the contraction is the
//     key order the score layout already has, and V^T is read from LDS in that same order.
// Queries arrive pre-scaled by scale*log2(e), so exp2 of the MFMA output is the softmax
// numerator. The projected queries and keys are fp16 (the score MFMA runs in fp16, whose
// 11-bit significand keeps the score error small); V and the weights are bf16. The
// normaliser is summed from the bf16-rounded weights, the same values the PV MFMA consumes.
#include "spa_device.h"
#include "spa_internal.h"

namespace spa {
namespace {

constexpr int kThreads = 256;
constexpr int kBR = 128;  // queries per workgroup (4 waves x 32)
constexpr int kBC = 64;   // keys per tile
constexpr float kTau = 8.0f;

template <int BYTES>
struct VecOf;
template <>
struct VecOf<16> {
    using T = u32x4;
};
template <>
struct VecOf<8> {
    using T = u32x2;
};

// Global -> register -> LDS staging of one key tile: 64 projected-key rows (fp16, LDS rows
// of MP + 8) and the matching 64 V rows, transposed to V^T (bf16, LDS rows of kVRow).
// Every thread moves the same number of bytes, so the loads need no branches: rows past N
// are clamped to row N-1 (their scores are masked, so their weights are exactly 0).
//
// V^T layout. A thread loads 4 consecutive keys (one key group) x VCOLS columns and writes
// VCOLS rows of V^T, 8 bytes each. Consecutive lanes take consecutive key groups, so the 16
// lanes of one LDS write cycle hit one row at 16 different 8-byte slots (no bank conflict).
// Inside a row, key group g is stored at slot kgslot(g), which swaps bits 0 and 1 of g: the
// two key groups one PV MFMA lane needs (g and g + 2, see the PV step) become adjacent, so
// the operand is a single 16-byte read; rows are 144 bytes apart, so 8 lanes reading 8
// consecutive rows cover the 32 banks once.
constexpr int kVRow = kBC + 8;  // V^T row pitch in bf16 elements (144 bytes)

__device__ __forceinline__ int kgslot(int g) { return (g & ~3) | ((g & 1) << 1) | ((g >> 1) & 1); }

template <int MP, int DV>
struct Stage {
    static constexpr int KROW = MP + 8;
    static constexpr int KBYTES = kBC * MP * 2 / kThreads;  // projected-key bytes per thread
    static constexpr int KVEC = KBYTES < 16 ? KBYTES : 16;  // bytes per load
    static constexpr int KLD = KBYTES / KVEC;               // loads per thread (1, 2 or 4)
    static constexpr int KPR = MP * 2 / KVEC;               // loads per key row
    static constexpr int VCOLS = DV / 16;                   // V columns per thread (x 4 keys)
    static constexpr int KG = kBC / 4;                      // key groups per tile (16)
    using KVec = typename VecOf<KVEC>::T;
    using VVec = typename VecOf<VCOLS * 2>::T;

    __device__ __forceinline__ static void load(KVec (&kreg)[KLD], VVec (&vreg)[4],
                                                const uint16_t* Kh, const bf16_t* Vh, int k0,
                                                int N, int tid, int vcg, int vkg) {
#pragma unroll
        for (int i = 0; i < KLD; ++i) {
            const int c = tid + i * kThreads;
            const int key = min(k0 + c / KPR, N - 1);
            kreg[i] = *reinterpret_cast<const KVec*>(Kh + (size_t)key * MP + (c % KPR) * (KVEC / 2));
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int key = min(k0 + vkg * 4 + r, N - 1);
            vreg[r] = *reinterpret_cast<const VVec*>(Vh + (size_t)key * DV + vcg * VCOLS);
        }
    }

    __device__ __forceinline__ static void store(const KVec (&kreg)[KLD], const VVec (&vreg)[4],
                                                 uint16_t* Ks, uint16_t* Vs, int tid, int vcg,
                                                 int vkg) {
#pragma unroll
        for (int i = 0; i < KLD; ++i) {
            const int c = tid + i * kThreads;
            *reinterpret_cast<KVec*>(Ks + (c / KPR) * KROW + (c % KPR) * (KVEC / 2)) = kreg[i];
        }
        // 4 keys x VCOLS columns -> VCOLS rows of V^T holding these 4 keys (8 bytes) each.
        uint16_t* dst = Vs + vcg * VCOLS * kVRow + kgslot(vkg) * 4;
#pragma unroll
        for (int a = 0; a < VCOLS / 2; ++a) {
            const uint32_t w0 = vreg[0][a], w1 = vreg[1][a], w2 = vreg[2][a], w3 = vreg[3][a];
            u32x2 lo, hi;
            lo.x = (w0 & 0xffffu) | (w1 << 16);
            lo.y = (w2 & 0xffffu) | (w3 << 16);
            hi.x = (w0 >> 16) | (w1 & 0xffff0000u);
            hi.y = (w2 >> 16) | (w3 & 0xffff0000u);
            *reinterpret_cast<u32x2*>(dst + (2 * a) * kVRow) = lo;
            *reinterpret_cast<u32x2*>(dst + (2 * a + 1) * kVRow) = hi;
        }
    }
};

template <int MP, int DV, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void attn_bf16_kernel(
    const uint16_t* __restrict__ Qt, const uint16_t* __restrict__ Kt, const bf16_t* __restrict__ V,
    void* __restrict__ O, float* __restrict__ lse, int N, int nqb, int out_f32) {
    constexpr int KS = MP / 16;          // score MFMA k-steps
    constexpr int KROW = MP + 8;         // LDS pitch of a projected-key row (fp16)
    constexpr int VROW = kVRow;          // LDS pitch of a V^T row (bf16)
    constexpr int K_ELEMS = kBC * KROW;  // one K tile
    constexpr int V_ELEMS = DV * VROW;   // one V^T tile
    constexpr int DB = DV / 32;          // 32-row blocks of V^T / O^T

    __shared__ __attribute__((aligned(16))) uint16_t lds[2 * (K_ELEMS + V_ELEMS)];

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
    const bf16_t* Vh = V + (size_t)bh * N * DV;

    // This lane's query as the B operand of the score MFMA (zero past N).
    f16x8 qf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        uint4 v = make_uint4(0, 0, 0, 0);
        if (myq < N) v = load16(Qh + (size_t)myq * MP + ks * 16 + half * 8);
        qf[ks] = as_f16x8(v);
    }

    const int kend = CAUSAL ? min(N, q0 + kBR) : N;
    const int ntiles = (kend + kBC - 1) / kBC;

    // ---- global -> register -> LDS staging --------------------------------------------
    using St = Stage<MP, DV>;
    typename St::KVec kreg[St::KLD];
    typename St::VVec vreg[4];
    const int vkg = tid % St::KG, vcg = tid / St::KG;  // key group, column group

    // ---- per-lane softmax state (query myq) --------------------------------------------
    f32x16 acc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[db] = f32x16_fill(0.0f);
    float mu = 0.0f;     // running maximum (base-2 units), identical in both half-waves
    float lsum = 0.0f;   // partial normaliser over this half-wave's keys
    f32x16 cinit = f32x16_fill(0.0f);  // -mu, the score accumulator's start value

    St::load(kreg, vreg, Kh, Vh, 0, N, tid, vcg, vkg);
    St::store(kreg, vreg, lds, lds + K_ELEMS, tid, vcg, vkg);
    __syncthreads();

#pragma unroll 1
    for (int t = 0; t < ntiles; ++t) {
        const int k0 = t * kBC;
        const bool more = t + 1 < ntiles;
        if (more) St::load(kreg, vreg, Kh, Vh, k0 + kBC, N, tid, vcg, vkg);

        const uint16_t* Ks = lds + (t & 1) * (K_ELEMS + V_ELEMS);
        const uint16_t* Vs = Ks + K_ELEMS;

        // Causal: a wave whose queries all precede the tile has nothing to do in it.
        if (!CAUSAL || k0 <= qw0 + 31) {
            f32x16 s[2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                s[kb] = cinit;
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const f16x8 a = as_f16x8(load16(Ks + (kb * 32 + col) * KROW + ks * 16 + half * 8));
                    s[kb] = mfma32x32x16(a, qf[ks], s[kb]);
                }
            }
            // Masks: keys past N, and keys after the query under the causal mask.
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
            float tmax = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i) tmax = fmaxf(tmax, s[kb][i]);
            tmax = halves_max(tmax);
            // The first tile sets mu to its maximum (key 0 is unmasked for every query, so
            // that maximum is finite, and nothing has been accumulated yet); later tiles move
            // mu only past the kTau slack, rescaling what was accumulated by 2^-delta <= 1.
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
            // Weights, their partial sum, and the bf16 B operands of the PV MFMA.
            bf16x8 pf[2][2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
                for (int tt = 0; tt < 2; ++tt) {
                    uint4 w;
                    uint32_t* wp = reinterpret_cast<uint32_t*>(&w);
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const float p0 = __builtin_amdgcn_exp2f(s[kb][8 * tt + 2 * j]);
                        const float p1 = __builtin_amdgcn_exp2f(s[kb][8 * tt + 2 * j + 1]);
                        wp[j] = pack_bf16x2(p0, p1);
                        lsum = add_bf16x2(wp[j], lsum);
                    }
                    pf[kb][tt] = as_bf16x8(w);
                }
            }
            // O^T += V^T . p^T. Slot 8*half + j of k-step tt in key block kb holds key
            // kb*32 + 16*tt + 8*(j/4) + 4*half + j%4, as in the score accumulator. The V^T
            // fragments of block db+1 are read while block db's MFMAs run.
            u32x4 vf[2][4];
            auto read_vfrags = [&](int db, u32x4* f) {
#pragma unroll
                for (int kt = 0; kt < 4; ++kt) {
                    // key groups g = 8*kb + 4*tt + half (slots 0-3) and g + 2 (slots 4-7)
                    const int g = 8 * (kt >> 1) + 4 * (kt & 1) + half;
                    f[kt] = *reinterpret_cast<const u32x4*>(Vs + (db * 32 + col) * VROW + kgslot(g) * 4);
                }
            };
            read_vfrags(0, vf[0]);
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                if (db + 1 < DB) read_vfrags(db + 1, vf[(db + 1) & 1]);
#pragma unroll
                for (int kt = 0; kt < 4; ++kt)
                    acc[db] = mfma32x32x16(__builtin_bit_cast(bf16x8, vf[db & 1][kt]), pf[kt >> 1][kt & 1], acc[db]);
            }
        }

        if (more) {
            uint16_t* Kn = lds + ((t + 1) & 1) * (K_ELEMS + V_ELEMS);
            St::store(kreg, vreg, Kn, Kn + K_ELEMS, tid, vcg, vkg);
        }
        __syncthreads();
    }

    // ---- epilogue: O = O_acc / l (both half-waves' key subsets summed) ------------------
    const float ltot = halves_sum(lsum);
    const float inv = 1.0f / ltot;
    if (myq < N) {
        const size_t row = (size_t)bh * N + myq;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int c0 = db * 32 + 8 * g + 4 * half;
                const float o0 = acc[db][4 * g + 0] * inv, o1 = acc[db][4 * g + 1] * inv;
                const float o2 = acc[db][4 * g + 2] * inv, o3 = acc[db][4 * g + 3] * inv;
                if (out_f32) {
                    float* dst = static_cast<float*>(O) + row * DV + c0;
                    *reinterpret_cast<float4*>(dst) = make_float4(o0, o1, o2, o3);
                } else {
                    bf16_t* dst = static_cast<bf16_t*>(O) + row * DV + c0;
                    uint2 w;
                    w.x = pack_bf16x2(o0, o1);
                    w.y = pack_bf16x2(o2, o3);
                    *reinterpret_cast<uint2*>(dst) = w;
                }
            }
        }
        if (lse && half == 0) lse[row] = (mu + __log2f(ltot)) * 0.69314718055994530942f;
    }
}

template <int MP, int DV, bool CAUSAL>
hipError_t launch(const void* Qt, const void* Kt, const void* V, void* O, float* lse, int BH,
                  int N, bool out_f32, hipStream_t stream) {
    const int nqb = (N + kBR - 1) / kBR;
    attn_bf16_kernel<MP, DV, CAUSAL><<<dim3(nqb * BH), kThreads, 0, stream>>>(
        static_cast<const uint16_t*>(Qt), static_cast<const uint16_t*>(Kt),
        static_cast<const bf16_t*>(V), O, lse, N, nqb, out_f32 ? 1 : 0);
    return hipGetLastError();
}

template <int MP, int DV>
hipError_t launch_c(const void* Qt, const void* Kt, const void* V, void* O, float* lse, int BH,
                    int N, bool causal, bool out_f32, hipStream_t stream) {
    return causal ? launch<MP, DV, true>(Qt, Kt, V, O, lse, BH, N, out_f32, stream)
                  : launch<MP, DV, false>(Qt, Kt, V, O, lse, BH, N, out_f32, stream);
}

template <int MP>
hipError_t launch_dv(const void* Qt, const void* Kt, const void* V, void* O, float* lse,
                     int BH, int N, int dv, bool causal, bool out_f32, hipStream_t stream) {
    switch (dv) {
        case 64: return launch_c<MP, 64>(Qt, Kt, V, O, lse, BH, N, causal, out_f32, stream);
        case 128: return launch_c<MP, 128>(Qt, Kt, V, O, lse, BH, N, causal, out_f32, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_attn_bf16(const void* Qt, const void* Kt, const void* V, void* O,
                            float* lse, int BH, int N, int mp, int dv, bool causal,
                            bool out_f32, hipStream_t stream) {
    switch (mp) {
        case 16: return launch_dv<16>(Qt, Kt, V, O, lse, BH, N, dv, causal, out_f32, stream);
        case 32: return launch_dv<32>(Qt, Kt, V, O, lse, BH, N, dv, causal, out_f32, stream);
        case 64: return launch_dv<64>(Qt, Kt, V, O, lse, BH, N, dv, causal, out_f32, stream);
        case 128: return launch_dv<128>(Qt, Kt, V, O, lse, BH, N, dv, causal, out_f32, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace spa
