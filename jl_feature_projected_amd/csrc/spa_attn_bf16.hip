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

template <int MP, int DV, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void attn_bf16_kernel(
    const uint16_t* __restrict__ Qt, const uint16_t* __restrict__ Kt, const bf16_t* __restrict__ V,
    void* __restrict__ O, float* __restrict__ lse, int N, int nqb, int out_f32) {
    constexpr int KS = MP / 16;          // score MFMA k-steps
    constexpr int KROW = MP + 8;         // LDS pitch of a projected-key row (fp16)
    constexpr int VROW = kBC + 4;        // LDS pitch of a V^T row (bf16)
    constexpr int K_ELEMS = kBC * KROW;  // one K tile
    constexpr int V_ELEMS = DV * VROW;   // one V^T tile
    constexpr int KCHUNKS = kBC * MP / 8;                  // 16-byte chunks per K tile
    constexpr int KPT = (KCHUNKS + kThreads - 1) / kThreads;
    constexpr int VSLOTS = (kBC / 4) * (DV / 8);           // 4 keys x 8 dv per slot
    constexpr int DB = DV / 32;                            // 32-row blocks of V^T / O^T

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
    uint4 kreg[KPT];
    uint4 vreg[4];
    auto load_tile = [&](int k0) {
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            const int c = tid + i * kThreads;
            kreg[i] = make_uint4(0, 0, 0, 0);
            if (c < KCHUNKS) {
                const int key = c / (MP / 8), cc = c % (MP / 8);
                if (k0 + key < N) kreg[i] = load16(Kh + (size_t)(k0 + key) * MP + cc * 8);
            }
        }
        if (tid < VSLOTS) {
            const int c8 = tid % (DV / 8), kg = tid / (DV / 8);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int key = k0 + kg * 4 + r;
                vreg[r] = key < N ? load16(Vh + (size_t)key * DV + c8 * 8) : make_uint4(0, 0, 0, 0);
            }
        }
    };
    auto store_tile = [&](int buf) {
        uint16_t* Ks = lds + buf * (K_ELEMS + V_ELEMS);
        uint16_t* Vs = Ks + K_ELEMS;
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            const int c = tid + i * kThreads;
            if (c < KCHUNKS) {
                const int key = c / (MP / 8), cc = c % (MP / 8);
                *reinterpret_cast<uint4*>(Ks + key * KROW + cc * 8) = kreg[i];
            }
        }
        if (tid < VSLOTS) {
            // 4 keys x 8 dv in registers -> 8 rows of V^T, 4 keys (8 bytes) each.
            const int c8 = tid % (DV / 8), kg = tid / (DV / 8);
            const uint32_t* w0 = reinterpret_cast<const uint32_t*>(&vreg[0]);
            const uint32_t* w1 = reinterpret_cast<const uint32_t*>(&vreg[1]);
            const uint32_t* w2 = reinterpret_cast<const uint32_t*>(&vreg[2]);
            const uint32_t* w3 = reinterpret_cast<const uint32_t*>(&vreg[3]);
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                uint2 lo, hi;
                lo.x = (w0[a] & 0xffffu) | (w1[a] << 16);
                lo.y = (w2[a] & 0xffffu) | (w3[a] << 16);
                hi.x = (w0[a] >> 16) | (w1[a] & 0xffff0000u);
                hi.y = (w2[a] >> 16) | (w3[a] & 0xffff0000u);
                *reinterpret_cast<uint2*>(Vs + (c8 * 8 + 2 * a) * VROW + kg * 4) = lo;
                *reinterpret_cast<uint2*>(Vs + (c8 * 8 + 2 * a + 1) * VROW + kg * 4) = hi;
            }
        }
    };

    // ---- per-lane softmax state (query myq) --------------------------------------------
    f32x16 acc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[db] = f32x16_fill(0.0f);
    float mu = 0.0f;     // running maximum (base-2 units), identical in both half-waves
    float lsum = 0.0f;   // partial normaliser over this half-wave's keys
    f32x16 cinit = f32x16_fill(0.0f);  // -mu, the score accumulator's start value

    load_tile(0);
    store_tile(0);
    __syncthreads();

#pragma unroll 1
    for (int t = 0; t < ntiles; ++t) {
        const int k0 = t * kBC;
        const bool more = t + 1 < ntiles;
        if (more) load_tile(k0 + kBC);

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
            tmax = fmaxf(tmax, swap_halves(tmax));
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
            // kb*32 + 16*tt + 8*(j/4) + 4*half + j%4, as in the score accumulator.
#pragma unroll
            for (int db = 0; db < DB; ++db) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
                    for (int tt = 0; tt < 2; ++tt) {
                        const uint16_t* vp = Vs + (db * 32 + col) * VROW + kb * 32 + tt * 16 + half * 4;
                        const uint2 lo = *reinterpret_cast<const uint2*>(vp);
                        const uint2 hi = *reinterpret_cast<const uint2*>(vp + 8);
                        const bf16x8 a = as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
                        acc[db] = mfma32x32x16(a, pf[kb][tt], acc[db]);
                    }
                }
            }
        }

        if (more) store_tile((t + 1) & 1);
        __syncthreads();
    }

    // ---- epilogue: O = O_acc / l (both half-waves' key subsets summed) ------------------
    const float ltot = lsum + swap_halves(lsum);
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
