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
// wave owns 32 of them. Key tiles of 64 are copied HBM -> LDS by buffer loads that write LDS
// directly (no registers, no VALU; rows past N read as zero), double buffered: the next
// tile's copy is issued before the current tile's math. Per tile and wave:
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
//     key order the score layout already has. The V tile stays row-major in LDS and the
//     A operand is read with ds_read_b64_tr_b16: within each 16-lane group, lane 4a+b
//     receives element b of the 8-byte rows that lanes a, a+4, a+8, a+12 address, so lane s
//     addressing V[r0 + s/4][c0 + 4(s%4)] gives lane i the keys r0..r0+3 of column c0 + i.
// LDS tiles are XOR-swizzled in 16-byte chunks (the copy picks, per lane, which global chunk
// lands in its LDS slot), so neither the score-operand reads nor the transposed reads hit
// a bank twice.
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

typedef short i16x4 __attribute__((ext_vector_type(4)));

// Buffer descriptor over [base, base + bytes): loads past the end return zero. Raw buffer
// (stride 0), 32-bit data format.
__device__ __forceinline__ u32x4 make_rsrc(const void* base, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    u32x4 r;
    r.x = (uint32_t)a;
    r.y = (uint32_t)(a >> 32) & 0xffffu;
    r.z = bytes;
    r.w = 0x00020000u;
    return r;
}

// 16 bytes per lane from buffer offset voff straight into LDS at dst + 16 * lane (dst is
// wave-uniform). Issued as inline assembly so the compiler does not track it: it cannot
// tell that the LDS it writes (the other buffer) is disjoint from the LDS the tile loop
// reads, and would otherwise wait for the copy before the first read. The copy's completion
// is awaited explicitly (vmcnt) before the barrier that hands the buffer over. Device pass
// only: the host pass does not parse AMDGPU assembly constraints.
__device__ __forceinline__ void copy16_to_lds(u32x4 rsrc, char* dst, uint32_t voff) {
#if defined(__HIP_DEVICE_COMPILE__)
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)dst);
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(m0), "v"(voff), "s"(rsrc)
                 : "m0");
#endif
}

// 16-byte chunk swizzles: LDS slot = global chunk ^ swizzle(row), a GF(2)-linear function of
// the row's low bits. The tables were chosen (by exhaustive search over such functions) so
// that every read pattern below touches each LDS bank once per service cycle, whether the
// LDS serves 128 bytes per cycle over 32 banks or 256 bytes over 64:
//   K tile (rows of MP*2 bytes), score operand: 8 or 16 consecutive rows, one chunk each;
//   V tile (rows of DV*2 bytes), transposed read: 4 rows x 2 or 4 chunks.
template <int MP>
__device__ __forceinline__ int kswz(int row) {
    constexpr int b0 = MP == 16 ? 0 : MP == 32 ? 0 : 1;
    constexpr int b1 = MP == 16 ? 0 : MP == 32 ? 1 : 2;
    constexpr int b2 = MP == 16 ? 1 : MP == 32 ? 2 : 4;
    constexpr int b3 = MP == 16 ? 1 : MP == 32 ? 1 : MP == 64 ? 1 : 8;
    return (row & 1 ? b0 : 0) ^ (row & 2 ? b1 : 0) ^ (row & 4 ? b2 : 0) ^ (row & 8 ? b3 : 0);
}
template <int DV>
__device__ __forceinline__ int vswz(int row) {
    constexpr int b0 = DV == 64 ? 2 : 4;
    constexpr int b1 = DV == 64 ? 4 : 10;
    return (row & 1 ? b0 : 0) ^ (row & 2 ? b1 : 0);
}

template <int MP, int DV, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void attn_bf16_kernel(
    const uint16_t* __restrict__ Qt, const uint16_t* __restrict__ Kt, const bf16_t* __restrict__ V,
    const float* __restrict__ kmax, void* __restrict__ O, float* __restrict__ lse, int N, int nqb,
    int out_f32) {
    constexpr int KS = MP / 16;              // score MFMA k-steps
    constexpr int KCH = MP / 8;              // 16-byte chunks per projected-key row
    constexpr int VCH = DV / 8;              // 16-byte chunks per V row
    constexpr int K_BYTES = kBC * MP * 2;    // one K tile
    constexpr int V_BYTES = kBC * DV * 2;    // one V tile
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
    const bf16_t* Vh = V + (size_t)bh * N * DV;

    // This lane's query as the B operand of the score MFMA (zero past N).
    f16x8 qf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        u32x4 v = {0u, 0u, 0u, 0u};
        if (myq < N) v = *reinterpret_cast<const u32x4*>(Qh + (size_t)myq * MP + ks * 16 + half * 8);
        qf[ks] = __builtin_bit_cast(f16x8, v);
    }

    const int kend = CAUSAL ? min(N, q0 + kBR) : N;
    const int ntiles = (kend + kBC - 1) / kBC;

    // ---- HBM -> LDS tile copy ---------------------------------------------------------
    // Copy j (64 lanes x 16 bytes) fills LDS chunks 64j .. 64j+63 of the tile; lane l writes
    // chunk c = 64j + l, which holds global chunk (c % CH) ^ swizzle(row) of row c / CH.
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
        const int row = c / VCH;
        voff[i] = row * DV * 2 + 16 * ((c % VCH) ^ vswz<DV>(row));
    }
    auto copy_tile = [&](int k0, int buf) {
        char* kdst = lds + buf * BUF;
        char* vdst = kdst + K_BYTES;
        const uint32_t rows_left = (uint32_t)(N - k0);
        const u32x4 kr = make_rsrc(Kh + (size_t)k0 * MP, rows_left * MP * 2);
        const u32x4 vr = make_rsrc(Vh + (size_t)k0 * DV, rows_left * DV * 2);
#pragma unroll
        for (int i = 0; i < KPW; ++i) {
            const int j = wave + kWaves * i;
            if (j < KINS) copy16_to_lds(kr, kdst + 1024 * j, koff[i]);
        }
#pragma unroll
        for (int i = 0; i < VPW; ++i)
            copy16_to_lds(vr, vdst + 1024 * (wave + kWaves * i), voff[i]);
    };

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
    // PV operand (transposed read): lane s of 16-lane group (half, gc) addresses key row
    // r0 + s/4 at column 32*db + 16*gc + 4*(s%4); r0 = kb*32 + 16*tt + 4*half, plus 8 for the
    // second half of the k-slots. Every such row has row % 4 == s/4, so the row's swizzle is
    // the same for all of this lane's reads: the swizzled chunk of each column block is
    // precomputed, and (kb, tt, lo/hi) only add a row offset.
    const int s16 = lane & 15, gc = (lane >> 4) & 1;
    const int vrow0 = 4 * half + (s16 >> 2);
    const int vbase = vrow0 * DV * 2 + 8 * (s16 & 1);  // + 2 * ((4*(s%4)) & 7)
    int vchunk[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
        vchunk[db] = vbase + 16 * ((4 * db + 2 * gc + ((s16 & 3) >> 1)) ^ vswz<DV>(vrow0));

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

    auto tile_loop = [&](auto exact_tag) {
        constexpr bool EXACT = decltype(exact_tag)::value;
#pragma unroll
        for (int db = 0; db < DB; ++db) acc[db] = f32x16_fill(0.0f);
        lsum = 0.0f;
        mu = EXACT ? 0.0f : bound;
        f32x16 cinit = f32x16_fill(-mu);  // the score accumulator's start value

        copy_tile(0, 0);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();

#pragma unroll 1
        for (int t = 0; t < ntiles; ++t) {
            const int k0 = t * kBC;
            if (t + 1 < ntiles) copy_tile(k0 + kBC, (t + 1) & 1);

            const char* Ks = lds + (t & 1) * BUF;
            const char* Vs = Ks + K_BYTES;

            // Causal: a wave whose queries all precede the tile has nothing to do in it.
            if (!CAUSAL || k0 <= qw0 + 31) {
                f32x16 s[2];
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
                // Weights, their partial sum, and the bf16 B operands of the PV MFMA.
                bf16x8 pf[2][2];
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
                    for (int tt = 0; tt < 2; ++tt) {
                        u32x4 w;
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const float p0 = __builtin_amdgcn_exp2f(s[kb][8 * tt + 2 * j]);
                            const float p1 = __builtin_amdgcn_exp2f(s[kb][8 * tt + 2 * j + 1]);
                            w[j] = pack_bf16x2(p0, p1);
                            lsum = add_bf16x2(w[j], lsum);
                        }
                        pf[kb][tt] = __builtin_bit_cast(bf16x8, w);
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
                            const char* vp = Vs + vchunk[db] + (kb * 32 + tt * 16) * DV * 2;
                            const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                (__attribute__((address_space(3))) i16x4*)(vp));
                            const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                (__attribute__((address_space(3))) i16x4*)(vp + 8 * DV * 2));
                            const bf16x8 a = __builtin_bit_cast(
                                bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                            acc[db] = mfma32x32x16(a, pf[kb][tt], acc[db]);
                        }
                    }
                }
            }

            // This wave's copies into the other buffer are done, and (barrier) everyone's
            // are, and everyone has finished reading this buffer.
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
        }
    };

    tile_loop(std::false_type{});
    float ltot = halves_sum(lsum);
    if (__syncthreads_or(myq < N && ltot < 0x1p-64f)) {
        tile_loop(std::true_type{});
        ltot = halves_sum(lsum);
    }

    // ---- epilogue: O = O_acc / l (both half-waves' key subsets summed) ------------------
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
                    u32x2 w;
                    w.x = pack_bf16x2(o0, o1);
                    w.y = pack_bf16x2(o2, o3);
                    *reinterpret_cast<u32x2*>(dst) = w;
                }
            }
        }
        if (lse && half == 0) lse[row] = (mu + __log2f(ltot)) * 0.69314718055994530942f;
    }
}

template <int MP, int DV, bool CAUSAL>
hipError_t launch(const void* Qt, const void* Kt, const void* V, const float* kmax, void* O,
                  float* lse, int BH, int N, bool out_f32, hipStream_t stream) {
    const int nqb = (N + kBR - 1) / kBR;
    attn_bf16_kernel<MP, DV, CAUSAL><<<dim3(nqb * BH), kThreads, 0, stream>>>(
        static_cast<const uint16_t*>(Qt), static_cast<const uint16_t*>(Kt),
        static_cast<const bf16_t*>(V), kmax, O, lse, N, nqb, out_f32 ? 1 : 0);
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
