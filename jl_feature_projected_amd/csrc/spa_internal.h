// spa_internal.h -- launch functions shared between the ABI layer and the HIP kernels.
// Arguments reaching these functions have been validated by the ABI layer.
#pragma once

#include <hip/hip_runtime.h>

namespace spa {

// Padded projected width the bf16 attention kernel consumes: m rounded up to 16, 32, 64
// or 128 (the contraction depth of one 32x32x16 MFMA is 16).
inline int padded_m(int m) { return m <= 16 ? 16 : m <= 32 ? 32 : m <= 64 ? 64 : 128; }

// Tokens per projection workgroup, and the number of such blocks per head.
constexpr int kProjBlockTokens = 256;
__host__ __device__ inline int proj_blocks(int N) { return (N + kProjBlockTokens - 1) / kProjBlockTokens; }

// V^T layout for the attention launch: Vt[bh, c, k] (bf16, [BH, dv, vt_padded_keys(N)]) holds
// V[bh, k', c], keys permuted within each group of 16 (order 0-3, 8-11, 4-7, 12-15) and
// zero past N.
constexpr int kVtTileKeys = 64;
__host__ __device__ inline int vt_padded_keys(int N) { return (N + kVtTileKeys - 1) / kVtTileKeys * kVtTileKeys; }

// Operand preparation of bf16 inputs, one launch. Projection on bf16 MFMA:
// Y_z[bh, n, c] = out_scale_z * sum_k X_z[bh, n, k] P[h, k, c] for z < nz (nz = 1 or 2,
// e.g. queries and keys), accumulated in fp32 and rounded once to fp16 (out_f16) or bf16.
// P is [H, d, m]; columns m <= c < out_cols are written as zeros. Output rows are out_stride
// elements apart, heads out_head_stride (default N * out_stride). If kmax is not null, kmax[bh * proj_blocks(N) + b] receives the largest
// row norm (fp32, before rounding) of Y1 over tokens b*256 .. b*256+255 of head bh. If Vt is
// not null, the same launch writes V^T of V ([BH, N, dv] bf16) in the layout above. If Yt0
// (Yt1) is not null, Y0 (Y1) is also written transposed, [BH, out_cols, vt_padded_keys(N)],
// tokens in the same permuted order as V^T and zero past N.
// With X0 null and nz = 2 only the second tensor (X1 -> Y1, and kmax) is projected.
// Backward row terms written by the dO-transpose role (V = dO): per query -lse*lse_scale and
// -D, D = <dO, O> (O bf16 [BH, N, dv]), into LD [BH, Np/32, 2, 32] (-inf and 0 for the
// padding queries), and zeros over dQt [BH, N, dqt_cols] (dqt_cols a multiple of 4).
struct PrepRowTerms {
    const void* O = nullptr;
    const float* lse = nullptr;
    float* LD = nullptr;
    float* dQt = nullptr;
    int dqt_cols = 0;
    float lse_scale = 0.0f;
};
hipError_t launch_project_bf16(const void* X0, const void* X1, const void* P, void* Y0,
                               void* Y1, int nz, int BH, int H, int N, int d, int m,
                               int out_stride, int out_cols, float out_scale0,
                               float out_scale1, bool out_f16, float* kmax, const void* V,
                               void* Vt, int dv, hipStream_t stream, void* Yt0 = nullptr,
                               void* Yt1 = nullptr, long long out_head_stride = -1,
                               const PrepRowTerms* row_terms = nullptr);

// Attention over projected inputs. Qt and Kt are fp16 [BH, N, mp] with zero columns past m
// (score MFMA in fp16); Qt is pre-scaled by scale*log2(e) so the scores come out in base-2
// exponent units. The weights x V MFMA (bf16) reads V^T as written by launch_project_bf16
// (Vt) or, when attn_bf16_reads_v_rows(...) is true for these sizes, V itself ([BH, N, dv]
// bf16, Vrow); the other pointer may be null. O is [BH, N, dv] in fp32 (out_f32) or bf16;
// lse [BH, N] optional. kmax holds the per-block key norm maxima written by the projection
// launch.
// When attn_bf16_projects_queries(...) is true, the launch projects the queries itself from
// Q ([BH, N, d] bf16) and P ([H, d, m] bf16), scaled by qscale, and Qt is not read; otherwise
// (or with Q null) it reads the projected queries from Qt.
bool attn_bf16_reads_v_rows(int BH, int N, int mp, int dv, bool causal);
bool attn_bf16_projects_queries(int BH, int N, int mp, int d, bool causal);
hipError_t launch_attn_bf16(const void* Qt, const void* Kt, const void* Vt, const void* Vrow,
                            const float* kmax, void* O, float* lse, int BH, int N, int mp,
                            int dv, bool causal, bool out_f32, hipStream_t stream,
                            const void* Q = nullptr, const void* P = nullptr,
                            float qscale = 0.0f, int d = 0, int H = 1, int m = 0);

// Backward of the bf16 path. The preparation launch (launch_project_bf16 with the queries
// scaled by scale*log2(e), fp16 outputs, the transposed copies Qst and (not with fused_dq)
// Ktt, and dO transposed into dOt; with fused_dq also the row terms LD and the cleared dQt)
// runs first; this runs the rest: the query-major kernel (dQt and D = rowsum(dO * O); not
// with fused_dq), the key-major kernel (dV and dKt, with fused_dq also dQt), dQ = dQt P^T
// and dK = dKt P^T, and the projection gradient dP (fp32 partials per 256-row chunk in
// dPpart, then a fixed-order sum). mp is 16, 32, 64 or 128.
struct BwdArgs {
    const uint16_t* Q;    // bf16 [BH, N, d]
    const uint16_t* K;    // bf16 [BH, N, d]
    const uint16_t* P;    // bf16 [H, d, m]
    const uint16_t* Qs;   // fp16 [BH, N, mp], queries projected and scaled by scale*log2(e)
    const uint16_t* Kt;   // fp16 [BH, N, mp]
    const uint16_t* Qst;  // fp16 [BH, mp, Np], Qs transposed, tokens permuted as in V^T
    const uint16_t* Ktt;  // fp16 [BH, mp, Np] (read only by the query-major kernel)
    const uint16_t* V;    // bf16 [BH, N, dv]
    const uint16_t* O;    // bf16 [BH, N, dv] (the forward's output)
    const uint16_t* dO;   // bf16 [BH, N, dv]
    const uint16_t* dOt;  // bf16 [BH, dv, Np], dO transposed, tokens permuted
    const float* lse;     // [BH, N], natural log (the forward's)
    float* LD;            // [BH, Np/32, 2, 32]: per 32 queries, -lse*log2(e) then -D
    float* dQt;           // [BH, N, mp]
    float* dKt;           // [BH, N, mp]
    float* dPpart;        // [BH, ceil(N / 256), d, m]
    float* dP;            // [H, d, m]
    void* dQ;             // [BH, N, d], fp32 (g_f32) or bf16
    void* dK;
    void* dV;             // [BH, N, dv]
    int g_f32;
    int fused_dq;  // 1: the key-major kernel also accumulates dQt (bwd_fuses_dq)
    int BH, H, N, Np, d, m, mp, dv, causal;
    float scale;
};
hipError_t launch_attn_bwd_bf16(const BwdArgs& a, hipStream_t stream);
// True when the key-major kernel accumulates dQt itself (fp32 atomic adds into dQt, which
// the preparation launch clears, with LD from that launch too) and the query-major kernel is
// not run.
bool bwd_fuses_dq(int mp, int dv);

// fp32 projection: Y[bh, n, c] = out_scale * sum_k X[bh, n, k] P[h, k, c], fp32 FMAs; with
// X1 non-null the same launch also writes Y1 from X1.
hipError_t launch_project_f32(const float* X, const float* P, float* Y, int BH, int H, int N,
                              int d, int m, float out_scale, hipStream_t stream,
                              const float* X1 = nullptr, float* Y1 = nullptr);

// fp32 attention over projected inputs (natural-exponent online softmax, fp32 FMAs).
hipError_t launch_attn_f32(const float* Qt, const float* Kt, const float* V, float* O,
                           float* lse, int BH, int N, int m, int dv, bool causal, float scale,
                           hipStream_t stream);

// Backward of the fp32 path (all fp32, row-major): inputs as passed to spa_attn_fwd plus
// O, dO and the forward's natural-log lse; workspace Qt, Kt, dQt, dKt [B*H, N, m] and D
// [B*H, N]; outputs dQ, dK [B*H, N, d], dV [B*H, N, dv], dP [H, d, m].
struct BwdF32Args {
    const float *Q, *K, *V, *P, *O, *dO, *lse;
    float *Qt, *Kt, *D, *dQt, *dKt;
    float *dQ, *dK, *dV, *dP;
    int B, H, N, d, m, dv, causal;
    float scale;
};
hipError_t launch_attn_bwd_f32(const BwdF32Args& a, hipStream_t stream);

// Decode: Nq queries against a cache of Nk projected keys (fp16) and values (bf16) with
// `rows` rows per head; partial results per (query, key split) in fp32.
struct DecodeArgs {
    const uint16_t* Q;   // bf16 [BH, Nq, d]
    const uint16_t* Kc;  // fp16 [BH, rows, m]
    const uint16_t* Vc;  // bf16 [BH, rows, dv]
    const uint16_t* P;   // bf16 [H, d, m]
    void* O;             // [BH, Nq, dv], fp32 or bf16
    float* lse;          // [BH, Nq] or null
    float* partO;        // [BH, Nq, nsplit, dv]
    float* partML;       // [BH, Nq, nsplit, 2]: running max (base 2), sum
    float qscale;        // scale * log2(e)
    int causal, BH, H, Nq, Nk, rows, d, m, dv, o_f32, nsplit, chunk;
};
struct DecodeSplit {
    int nsplit, chunk;  // key splits per (head, query group) and keys per split
};
DecodeSplit decode_split(int BH, int Nq, int Nk);
hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t stream);

// Sparse feature attention operands: Topk_k of every row of Q and K (bf16 [BH, N, d],
// d in {64, 128}) into fp16 [BH, N, d] (queries times qscale), the largest selected key norm
// per 256-key block into kmax [BH, proj_blocks(N)].
hipError_t launch_sfa_topk(const void* Q, const void* K, void* Qt, void* Kt, float* kmax,
                           int BH, int N, int d, int k, float qscale, hipStream_t stream);

// Rate probes (spa_probe.hip): kind 0 the bf16 32x32x16 MFMA rate on random operands, kind 1
// the fp32 VALU FMA rate, in TFLOP/s, sustained over `launches` back-to-back launches, with
// the mean engine clock in GHz during the last one.
hipError_t run_probe(int kind, int launches, hipStream_t stream, double* tflops, double* ghz);

}  // namespace spa
