// spa_project.hip -- the operand preparation launch of the bf16 path (gfx950): the projection
// X~ = X P of queries and keys on bf16 MFMA, and V transposed for the attention launch, as the
// roles of the workgroups of one launch.
//
// Projection: "Sparse Projection Attention" page, Sec. 3.1.2 and Algorithm 1 steps 2-3:
// queries and keys are mapped from d to m features by one shared matrix. "Projection-
// Decomposition Attention (PDA)", Algorithm 2.1 step 1, and Sec. 4.1 (cost O(L d m), small
// next to the O(L^2 m) scores): the launch is bound by HBM traffic.
//
// Each wave computes X~^T for 32 tokens: D[c][t] = sum_k P^T[c][k] X^T[k][t], with P^T
// staged once per workgroup in LDS as the A operand and 16-byte loads of X rows as the B
// operand. In the D layout a lane owns one token and 4 consecutive output columns per
// group, so every store is one 8-byte write of 4 values. The result is rounded once, to
// bf16 for the exported projection or to fp16 for the attention path's score operands.
// When asked (kmax != null), the launch also records, per (head, 256-token block) of the
// second tensor (the keys), the largest row norm of the projected values: the attention
// launch bounds every score of a row by the query norm times that maximum.
//
// V transpose (when Vt != null): the attention launch multiplies V^T (dv x keys) by the
// transposed weights on MFMA, whose A operand gives each lane 8 keys of one V column. With
// V row-major those 8 values are 8 rows apart, and reading them from LDS needs the
// transposing LDS read, which moves about a quarter of the bytes per clock of a plain
// 16-byte read. So this launch writes Vt[bh][c][k] = V[bh][k'][c] with the keys of every
// 16-key group stored in the order 0-3, 8-11, 4-7, 12-15 (the order in which the score
// accumulator holds them: a lane of half h holds keys 4h..4h+3 and 8+4h..8+4h+3 of each 16),
// rows zero-padded to a multiple of 64 keys. Every A operand is then one 16-byte read.
//
// Launch order: the roles of one (head, 256-token block) are adjacent, so the queries', keys'
// and values' traffic of a block run side by side.
//
// For the backward pass the same launch can also write the projections transposed, with
// the tokens of every 16-group in the V^T order (Yt0, Yt1), and transpose dO in place of V.
// The dO role can then also write, per query, -lse*log2(e) and -D with D = <dO, O> (the row
// term of the softmax gradient), reading O's rows beside dO's, and clear the rows of the
// projected-query gradient that the key-major backward kernel accumulates into.
#include "spa_device.h"
#include "spa_internal.h"

namespace spa {
namespace {

constexpr int kProjThreads = 256;
constexpr int kProjTokensPerWave = 32;
constexpr int kProjIters = 2;  // token blocks per wave: amortises the P^T staging
constexpr int kProjTokensPerBlock = kProjThreads / 64 * kProjTokensPerWave * kProjIters;
static_assert(kProjTokensPerBlock == kProjBlockTokens, "projection block size");

struct PrepArgs {
    const bf16_t* X0;
    const bf16_t* X1;
    const bf16_t* P;
    uint16_t* Y0;
    uint16_t* Y1;
    const uint16_t* V;  // V transpose role: input [BH, N, dv] ...
    uint16_t* Vt;       // ... and output [BH, dv, Np]; null: no such role
    uint16_t* Yt0;      // optional transposed projections [BH, out_cols, Np], tokens
    uint16_t* Yt1;      // permuted within 16-groups as in Vt
    float* kmax;
    PrepRowTerms rt;    // backward row terms (rt.LD null: none)
    int N, BH, H, m, out_stride, out_cols, nz, nroles, Np;
    int z0;  // first projection role (1: the first tensor is skipped)
    long long out_head_stride;  // elements between heads of Y0 / Y1
    float scale0, scale1;
};

// Round-to-nearest-even of two floats to the output type, packed into one dword.
template <bool F16>
__device__ __forceinline__ uint32_t pack_out(float lo, float hi) {
    return F16 ? pack_f16x2(lo, hi) : pack_bf16x2(lo, hi);
}

// Position p (0..15) of a 16-key group of V^T holds key vt_key(p).
__device__ __forceinline__ int vt_key(int p) {
    const int h = p >> 3, j = p & 7;
    return 8 * (j >> 2) + 4 * h + (j & 3);
}

// V^T for tokens [t0, t0 + 256) of head bh, in 64-key tiles through LDS (s: 64 x (DV+8)).
// The next tile's rows are loaded into registers while the current one is written out.
template <int DV>
__device__ void transpose_v(const PrepArgs& a, int bh, int t0, uint16_t* s) {
    constexpr int PITCH = DV + 8;  // LDS row pitch (elements): 16 bytes of padding
    constexpr int CH = DV / 8;     // 16-byte chunks per V row
    constexpr int LPT = kVtTileKeys * CH / kProjThreads;  // 16-byte loads per thread per tile
    static_assert(LPT * kProjThreads == kVtTileKeys * CH, "tile load split");
    const uint16_t* Vh = a.V + (size_t)bh * a.N * DV;
    uint16_t* Vth = a.Vt + (size_t)bh * DV * a.Np;
    const int kend = min(t0 + kProjTokensPerBlock, a.Np);
    const PrepRowTerms& rt = a.rt;
    const bool terms = rt.LD != nullptr;
    const uint16_t* Oh = terms ? static_cast<const uint16_t*>(rt.O) + (size_t)bh * a.N * DV : nullptr;
    u32x4 v[LPT], o[LPT];
    auto load = [&](int k0) {
#pragma unroll
        for (int i = 0; i < LPT; ++i) {
            const int c = threadIdx.x + i * kProjThreads;
            const int r = c / CH, ch = c - r * CH;
            v[i] = u32x4{0u, 0u, 0u, 0u};
            o[i] = u32x4{0u, 0u, 0u, 0u};
            if (k0 + r < a.N) {
                v[i] = *reinterpret_cast<const u32x4*>(Vh + (size_t)(k0 + r) * DV + ch * 8);
                if (terms) o[i] = *reinterpret_cast<const u32x4*>(Oh + (size_t)(k0 + r) * DV + ch * 8);
            }
        }
    };
    load(t0);
#pragma unroll 1
    for (int k0 = t0; k0 < kend; k0 += kVtTileKeys) {
        if (terms) {
            // D of each row: its CH chunks are held by CH adjacent lanes of one wave
#pragma unroll
            for (int i = 0; i < LPT; ++i) {
                const int c = threadIdx.x + i * kProjThreads;
                const int r = c / CH, ch = c - r * CH;
                const bf16x8 x = __builtin_bit_cast(bf16x8, v[i]);
                const bf16x8 y = __builtin_bit_cast(bf16x8, o[i]);
                float dot = 0.0f;
#pragma unroll
                for (int e = 0; e < 8; ++e) dot += (float)x[e] * (float)y[e];
#pragma unroll
                for (int off = 1; off < CH; off <<= 1) dot += __shfl_xor(dot, off, 64);
                const int row = k0 + r;
                if (ch == 0 && row < a.Np) {
                    float* dst = rt.LD + ((size_t)bh * a.Np + (row & ~31)) * 2 + (row & 31);
                    dst[0] = row < a.N ? -rt.lse[(size_t)bh * a.N + row] * rt.lse_scale : -INFINITY;
                    dst[32] = -dot;
                }
            }
            // the projected-query gradient rows of this tile start at zero
            const int cq = rt.dqt_cols / 4;
            for (int c = threadIdx.x; c < kVtTileKeys * cq; c += kProjThreads) {
                const int row = k0 + c / cq;
                if (row < a.N)
                    *reinterpret_cast<float4*>(rt.dQt + ((size_t)bh * a.N + row) * rt.dqt_cols + 4 * (c % cq)) =
                        make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            }
        }
#pragma unroll
        for (int i = 0; i < LPT; ++i) {
            const int c = threadIdx.x + i * kProjThreads;
            const int r = c / CH, ch = c - r * CH;
            *reinterpret_cast<u32x4*>(s + r * PITCH + ch * 8) = v[i];
        }
        __syncthreads();
        if (k0 + kVtTileKeys < kend) load(k0 + kVtTileKeys);
        for (int c = threadIdx.x; c < DV * (kVtTileKeys / 8); c += kProjThreads) {
            const int col = c >> 3, ch = c & 7;  // V column, 16-byte chunk of the 64-key row
            u32x4 w;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int p0 = 8 * (ch & 1) + 2 * i;  // position within the 16-key group
                const int kk = 16 * (ch >> 1);
                const uint32_t lo = s[(kk + vt_key(p0)) * PITCH + col];
                const uint32_t hi = s[(kk + vt_key(p0 + 1)) * PITCH + col];
                w[i] = lo | (hi << 16);
            }
            *reinterpret_cast<u32x4*>(Vth + (size_t)col * a.Np + k0 + ch * 8) = w;
        }
        __syncthreads();
    }
}

template <int D, int MB, bool F16, int DV>
__global__ __launch_bounds__(kProjThreads) void prep_bf16_kernel(PrepArgs a) {
    constexpr int PROW = D + 8;  // LDS row pitch in bf16: 16 bytes of padding per row
    constexpr int KS = D / 16;   // MFMA k-steps over the input features
    constexpr int PT_BYTES = MB * 32 * PROW * 2;
    constexpr int VT_BYTES = DV > 0 ? kVtTileKeys * (DV + 8) * 2 : 0;
    __shared__ __attribute__((aligned(16))) char smem[PT_BYTES > VT_BYTES ? PT_BYTES : VT_BYTES];
    __shared__ float wave_max[kProjThreads / 64];

    const int nblk = (a.N + kProjTokensPerBlock - 1) / kProjTokensPerBlock;
    const int role = a.z0 + blockIdx.x % a.nroles;
    const int rest = blockIdx.x / a.nroles;
    const int blk = rest % nblk;
    const int bh = rest / nblk;
    const int tid = threadIdx.x;

    if constexpr (DV > 0) {
        if (role == a.nz) {
            transpose_v<DV>(a, bh, blk * kProjTokensPerBlock, reinterpret_cast<uint16_t*>(smem));
            return;
        }
    }

    const int z = role;  // 0: X0 (queries), 1: X1 (keys)
    const bf16_t* X = z ? a.X1 : a.X0;
    uint16_t* Y = z ? a.Y1 : a.Y0;
    uint16_t* Yt = z ? a.Yt1 : a.Yt0;
    const float out_scale = z ? a.scale1 : a.scale0;
    const int h = bh % a.H;
    const int m = a.m;
    bf16_t* Pt = reinterpret_cast<bf16_t*>(smem);

    const int wave = tid / 64, lane = tid % 64, col = lane % 32, half = lane / 32;
    const bf16_t* Xh = X + (size_t)bh * a.N * D;
    // This lane's token of iteration it as the B operand (zero past N). The first
    // iteration's rows are requested before P^T is staged, the second's during the first.
    bf16x8 xf[kProjIters][KS];
    auto load_x = [&](int it) {
        const int tok = blk * kProjTokensPerBlock + (it * 4 + wave) * kProjTokensPerWave + col;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            u32x4 v = {0u, 0u, 0u, 0u};
            if (tok < a.N) v = *reinterpret_cast<const u32x4*>(Xh + (size_t)tok * D + ks * 16 + half * 8);
            xf[it][ks] = __builtin_bit_cast(bf16x8, v);
        }
    };
    load_x(0);

    // P^T[c][k] = P[h][k][c] for c < m; rows m .. 32*MB-1 are zero. Rows of P are read with
    // 16-byte loads when m allows it.
    const bf16_t* Ph = a.P + (size_t)h * D * m;
    if ((m & 7) == 0) {
        const int vpr = m >> 3;  // 16-byte vectors per row of P
        for (int v = tid; v < D * vpr; v += kProjThreads) {
            const int k = v / vpr, c8 = (v - k * vpr) * 8;
            const u32x4 x = *reinterpret_cast<const u32x4*>(Ph + (size_t)k * m + c8);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                Pt[(c8 + 2 * j) * PROW + k] = __builtin_bit_cast(bf16_t, (uint16_t)(x[j] & 0xffffu));
                Pt[(c8 + 2 * j + 1) * PROW + k] = __builtin_bit_cast(bf16_t, (uint16_t)(x[j] >> 16));
            }
        }
        for (int idx = tid; idx < (MB * 32 - m) * D; idx += kProjThreads) {
            const int c = m + idx / D, k = idx % D;
            Pt[c * PROW + k] = (bf16_t)0.0f;
        }
    } else {
        for (int idx = tid; idx < MB * 32 * D; idx += kProjThreads) {
            const int c = idx / D, k = idx % D;
            Pt[c * PROW + k] = c < m ? Ph[k * m + c] : (bf16_t)0.0f;
        }
    }
    __syncthreads();

    uint16_t* Yh = Y + (size_t)bh * a.out_head_stride;
    const bool vec_store = (a.out_stride % 4) == 0;
    const bool want_norm = a.kmax != nullptr && z == 1;
    float norm2_max = 0.0f;  // largest squared row norm among this lane's tokens

#pragma unroll
    for (int it = 0; it < kProjIters; ++it) {
        const int tok = blk * kProjTokensPerBlock + (it * 4 + wave) * kProjTokensPerWave + col;
        const bool valid = tok < a.N;
        if (it + 1 < kProjIters) load_x(it + 1);
        float norm2 = 0.0f;  // squared norm over this lane's half of the columns
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            f32x16 acc = f32x16_fill(0.0f);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const bf16x8 pa = __builtin_bit_cast(
                    bf16x8, *reinterpret_cast<const u32x4*>(Pt + (mb * 32 + col) * PROW + ks * 16 + half * 8));
                acc = mfma32x32x16(pa, xf[it][ks], acc);
            }
            if (want_norm) {
#pragma unroll
                for (int i = 0; i < 16; ++i) norm2 += acc[i] * acc[i];
            }
            if (Yt && tok < a.Np) {
                // X~^T in the V^T token order: lane = token, rows = 16 of this block's columns.
                const int pos = (tok & ~15) | vt_key(tok & 15);
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int c = mb * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
                    if (c < a.out_cols)
                        Yt[((size_t)bh * a.out_cols + c) * a.Np + pos] =
                            (uint16_t)(pack_out<F16>(acc[i] * out_scale, 0.0f) & 0xffffu);
                }
            }
            if (!valid) continue;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int c0 = mb * 32 + 8 * g + 4 * half;
                if (c0 >= a.out_cols) continue;
                uint16_t* dst = Yh + (size_t)tok * a.out_stride + c0;
                u32x2 w;
                w.x = pack_out<F16>(acc[4 * g + 0] * out_scale, acc[4 * g + 1] * out_scale);
                w.y = pack_out<F16>(acc[4 * g + 2] * out_scale, acc[4 * g + 3] * out_scale);
                if (vec_store && c0 + 4 <= a.out_cols) {
                    *reinterpret_cast<u32x2*>(dst) = w;
                } else {
                    const uint16_t v[4] = {(uint16_t)(w.x & 0xffffu), (uint16_t)(w.x >> 16),
                                           (uint16_t)(w.y & 0xffffu), (uint16_t)(w.y >> 16)};
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (c0 + r < a.out_cols) dst[r] = v[r];
                }
            }
        }
        if (want_norm) {
            // lanes l and l ^ 32 hold the two halves of one token's columns
            const float full = halves_sum(norm2) * out_scale * out_scale;
            if (valid) norm2_max = fmaxf(norm2_max, full);
        }
    }
    if (want_norm) {
        float v = norm2_max;
#pragma unroll
        for (int o = 16; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
        if (lane == 0) wave_max[wave] = v;
        __syncthreads();
        if (tid == 0) {
            float b = wave_max[0];
#pragma unroll
            for (int w = 1; w < kProjThreads / 64; ++w) b = fmaxf(b, wave_max[w]);
            a.kmax[(size_t)bh * nblk + blk] = sqrtf(b);
        }
    }
}

template <int D, int MB, bool F16, int DV>
hipError_t launch(const PrepArgs& a, hipStream_t stream) {
    const long long nblk = (a.N + kProjTokensPerBlock - 1) / kProjTokensPerBlock;
    const long long blocks = nblk * a.BH * a.nroles;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    prep_bf16_kernel<D, MB, F16, DV><<<dim3((unsigned)blocks), kProjThreads, 0, stream>>>(a);
    return hipGetLastError();
}

template <int D, int MB, bool F16>
hipError_t launch_v(const PrepArgs& a, int dv, hipStream_t stream) {
    if (!a.Vt) return launch<D, MB, F16, 0>(a, stream);
    switch (dv) {
        case 64: return launch<D, MB, F16, 64>(a, stream);
        case 128: return launch<D, MB, F16, 128>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

template <int D, bool F16>
hipError_t launch_mb(const PrepArgs& a, int dv, hipStream_t stream) {
    const int cols = a.out_cols > a.m ? a.out_cols : a.m;
    switch ((cols + 31) / 32) {
        case 1: return launch_v<D, 1, F16>(a, dv, stream);
        case 2: return launch_v<D, 2, F16>(a, dv, stream);
        case 3:
        case 4: return launch_v<D, 4, F16>(a, dv, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_project_bf16(const void* X0, const void* X1, const void* P, void* Y0,
                               void* Y1, int nz, int BH, int H, int N, int d, int m,
                               int out_stride, int out_cols, float out_scale0,
                               float out_scale1, bool out_f16, float* kmax, const void* V,
                               void* Vt, int dv, hipStream_t stream, void* Yt0, void* Yt1,
                               long long out_head_stride, const PrepRowTerms* row_terms) {
    PrepArgs a;
    a.rt = row_terms ? *row_terms : PrepRowTerms{};
    a.Yt0 = static_cast<uint16_t*>(Yt0);
    a.Yt1 = static_cast<uint16_t*>(Yt1);
    a.X0 = static_cast<const bf16_t*>(X0);
    a.X1 = static_cast<const bf16_t*>(X1);
    a.P = static_cast<const bf16_t*>(P);
    a.Y0 = static_cast<uint16_t*>(Y0);
    a.Y1 = static_cast<uint16_t*>(Y1);
    a.V = static_cast<const uint16_t*>(V);
    a.Vt = static_cast<uint16_t*>(Vt);
    a.kmax = kmax;
    a.N = N;
    a.BH = BH;
    a.H = H;
    a.m = m;
    a.out_stride = out_stride;
    a.out_cols = out_cols;
    a.out_head_stride = out_head_stride < 0 ? (long long)N * out_stride : out_head_stride;
    a.nz = nz;
    a.z0 = (X0 == nullptr && nz == 2) ? 1 : 0;
    a.nroles = nz - a.z0 + (Vt ? 1 : 0);
    a.Np = vt_padded_keys(N);
    a.scale0 = out_scale0;
    a.scale1 = out_scale1;
    switch (d) {
        case 64: return out_f16 ? launch_mb<64, true>(a, dv, stream) : launch_mb<64, false>(a, dv, stream);
        case 128: return out_f16 ? launch_mb<128, true>(a, dv, stream) : launch_mb<128, false>(a, dv, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace spa
