/*
 * spa.h -- C ABI of libspa: feature-axis projected softmax attention on MI355X (gfx950).
 *
 * The operation (per batch b and head h, with one projection P_h in R^{d x m} shared by
 * queries and keys):
 *
 *     Qt = Q P_h,  Kt = K P_h                                   (projection)
 *     O  = softmax_rows( scale * Qt Kt^T  [+ causal mask] ) V   (attention)
 *
 * Sources: "Sparse Projection Attention: A Computationally Efficient Framework for Long
 * Sequence Modeling", Sec. 3.1.2-3.1.3 and Algorithm 1 (project queries and keys with one
 * shared matrix, score in the projected space, softmax, multiply by V); "Projection-
 * Decomposition Attention (PDA)", Algorithm 2.1 steps 1-3 and 5 (Gaussian P with N(0, 1/m)
 * entries; the low-rank step 4 is not part of this library) and Sec. 4.2 (the score matrix
 * can be streamed and is never stored). The N x N score matrix is never written to memory.
 *
 * Conventions shared by every entry point:
 *   - Tensors are dense, contiguous and row-major. Q, K: [B,H,N,d]; V, O: [B,H,N,dv];
 *     P: [H,d,m] (one d x m matrix per head; a projection shared by all heads is passed as H
 *     identical copies); projected tensors: [B,H,N,m]; lse: [B,H,N].
 *   - Tensor pointers are DEVICE pointers. Base addresses must be 16-byte aligned (lse:
 *     4-byte aligned). The caller owns every buffer; the library keeps no pointer after a
 *     call returns.
 *   - `stream` is a hipStream_t (NULL = the default stream). Calls are asynchronous and
 *     stream-ordered: a returned SPA_OK means the work was enqueued, not that it finished.
 *   - Errors are reported only through the returned status; nothing aborts or throws.
 *     Arguments are validated on the host before any HIP call, so an invalid call touches
 *     neither the device nor the stream. spa_last_error() gives a readable reason.
 *   - Non-finite values in the tensors are not checked; they propagate to the outputs. In the
 *     forward, a NaN in a query row reaches that output row (and its lse) only, and a NaN in
 *     a key row only the rows whose scores include that key; every other row is unchanged.
 *     A non-finite value of V also reaches rows of its 64-key tile that the causal mask
 *     excludes (their zero weights meet it in the products).
 *   - The library is reentrant. Concurrent calls must use distinct outputs and workspaces.
 */
#ifndef SPA_H
#define SPA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum spa_status {
    SPA_OK = 0,
    SPA_ERR_INVALID_ARGUMENT = 1, /* null pointer, dim < 1, bad flag, non-finite scale,
                                     misaligned or overlapping buffers */
    SPA_ERR_UNSUPPORTED = 2,      /* a valid shape or dtype with no compiled kernel */
    SPA_ERR_WORKSPACE = 3,        /* workspace given but smaller than required */
    SPA_ERR_HIP = 4,              /* a HIP runtime call or kernel launch failed */
    /* Not statuses: these give the type the range of int, so that any int a caller passes
       (e.g. to spa_status_string) is a value C++ may load and compare. */
    SPA_STATUS_INT_MIN_ = -2147483647 - 1,
    SPA_STATUS_INT_MAX_ = 2147483647
} spa_status_t;

typedef enum spa_dtype {
    SPA_F32 = 0, /* IEEE binary32 */
    SPA_BF16 = 1, /* bfloat16 (8-bit exponent, 7-bit stored mantissa) */
    /* Not dtypes: these give the type the range of int, so that any int a caller passes is a
       value the library may load, compare and reject (SPA_ERR_INVALID_ARGUMENT). */
    SPA_DTYPE_INT_MIN_ = -2147483647 - 1,
    SPA_DTYPE_INT_MAX_ = 2147483647
} spa_dtype_t;

/* Library version, major*10000 + minor*100 + patch. */
int spa_version(void);

/* Readable name of a status code (static string). */
const char* spa_status_string(spa_status_t status);

/* Reason for the calling thread's last failed call ("" if none); valid until its next call. */
const char* spa_last_error(void);

/*
 * spa_project -- the projection step on its own: Xt[b,h,n,:] = X[b,h,n,:] P[h].
 * (SPA page Sec. 3.1.2 and Algorithm 1 steps 2-3; PDA page Algorithm 2.1 step 1.)
 *
 *   X  [B,H,N,d]  input rows, in `dtype`.
 *   P  [H,d,m]    projection, in `dtype`.
 *   Xt [B,H,N,m]  output, written in `dtype`; must not overlap X or P.
 *
 * Accumulation is fp32 (bf16 path: bf16 MFMA products with fp32 accumulation, the result
 * rounded to nearest-even bf16). Supported: SPA_BF16 with d in {64, 128} and 1 <= m <= 128;
 * SPA_F32 with 1 <= d <= 256 and 1 <= m <= 128.
 */
spa_status_t spa_project(const void* X, const void* P, void* Xt, int B, int H, int N, int d,
                         int m, spa_dtype_t dtype, void* stream);

/*
 * Workspace bytes spa_attn_fwd needs for these sizes. Returns 0 for arguments spa_attn_fwd
 * would reject. Contents (each region 256-byte aligned): the projected queries and keys
 * (bf16 path: fp16 at m rounded up to 16, 32, 64 or 128 columns; fp32 path: fp32 at m
 * columns) and, on the bf16 path only, one fp32 per (head, 256-key block) with that block's
 * largest projected key norm, and V transposed per head ([dv, N rounded up to 64] bf16).
 * The projected-query and V^T regions go unused where spa_attn_fwd_plan reports the
 * corresponding flag; the size does not depend on it.
 */
size_t spa_attn_fwd_workspace_bytes(int B, int H, int N, int d, int m, int dv,
                                    spa_dtype_t dtype);

/*
 * How spa_attn_fwd runs these sizes on the bf16 path (a host-side query; no GPU work, no
 * error recorded). Returns a set of flags, or -1 for arguments spa_attn_fwd would reject:
 *   SPA_PLAN_QUERIES_IN_ATTENTION: the attention launch projects the queries itself (the
 *     projection launch handles the keys only), so the projected queries never reach HBM;
 *   SPA_PLAN_V_ROW_MAJOR: the attention launch reads V as given (no transposed copy).
 * Neither changes the result beyond fp32 summation order; the fp32 path returns 0.
 */
#define SPA_PLAN_QUERIES_IN_ATTENTION 1
#define SPA_PLAN_V_ROW_MAJOR 2
int spa_attn_fwd_plan(int B, int H, int N, int d, int m, int dv, spa_dtype_t dtype,
                      int causal);

/*
 * spa_attn_fwd -- the projected attention forward:
 *
 *   O[b,h,i,:] = sum_j softmax_j( scale * <Q[b,h,i,:] P[h], K[b,h,j,:] P[h]> ) V[b,h,j,:]
 *
 * over j in 0..N-1, or j in 0..i when causal = 1 (square self-attention; the diagonal is
 * kept, so no row is ever empty). (SPA page Sec. 3.1.3 and Algorithm 1 steps 4-6; PDA page
 * Algorithm 2.1 steps 2, 3 and 5.) The scale is the caller's: the pages use 1/sqrt(m)
 * (SPA Sec. 3.1.3, PDA Algorithm 2.1) and 1/sqrt(d) (PDA revised proof Sec. 2.1, which keeps
 * projected scores on the exact-score scale).
 *
 *   Q, K  [B,H,N,d], V [B,H,N,dv], P [H,d,m]: inputs in `dtype`.
 *   scale finite float (any sign, zero allowed); causal 0 or 1.
 *   O     [B,H,N,dv] output in `o_dtype`: SPA_BF16 or SPA_F32 on the bf16 path, SPA_F32 on
 *         the fp32 path. Must not overlap any input, lse or the workspace.
 *   lse   optional [B,H,N] fp32 output (NULL to skip): the natural log of each row's
 *         softmax normaliser, log(sum_j exp(score_ij)).
 *   workspace / workspace_bytes: device scratch of at least
 *         spa_attn_fwd_workspace_bytes(...) bytes, 16-byte aligned (contents above). If
 *         workspace is NULL the library allocates and frees it stream-ordered
 *         (hipMallocAsync / hipFreeAsync) inside the call.
 *
 * The bf16 path runs two launches on `stream`: operand preparation (the projection of Q and
 * K on bf16 MFMA with fp32 accumulation, projected values rounded once to fp16, queries
 * pre-multiplied by scale*log2(e), the per-block key norm maxima, and V transposed) and
 * the attention launch (fp16 MFMA for the scores and bf16 MFMA for weights x V, both with
 * fp32 accumulation; the softmax weights are rounded to bf16 before they meet V and the
 * normaliser sums those rounded weights). Each row's exponent offset is the Cauchy-Schwarz
 * bound |q| * max |k| rather than a running maximum; rows for which that bound is so loose
 * that the normaliser would fall below 2^-64 are recomputed with an exact online maximum.
 * Accuracy of the bf16 path: rounding the two projected operands to fp16 moves a score
 * s_ij by at most 2^-10 * |scale| * sum_c |(QP)[i,c]| |(KP)[j,c]|, and an output row by at
 * most that times max_j |V[j,:] - O[i,:]| (first order); at the magnitudes of unit-norm
 * heads with m >= 8 the outputs stay within 2e-2 of the exact result for V entries of
 * order one, while very small m (large projected scores) loosens it by that bound.
 * Supported: d in {64, 128}, dv in {64, 128}, 1 <= m <= 128. Input range of the bf16
 * path: every projected key entry (K P)[j,c] and every scaled projected query entry
 * scale * log2(e) * (Q P)[i,c] must lie inside the fp16 range, |x| <= 65504 (bf16 inputs of
 * ordinary attention magnitudes are far inside it; entries beyond it become infinite and
 * the affected rows come out non-finite, or, where such a key's score is -infinity, with
 * that key's weight correctly zero -- never a finite value built on a clipped score). Use
 * the fp32 path for inputs outside that range. The fp32 path computes in fp32 throughout:
 * 1 <= d <= 256, 1 <= m <= 128, 1 <= dv <= 128. N may be any size from 1 to 2^22; tails are
 * masked.
 */
spa_status_t spa_attn_fwd(const void* Q, const void* K, const void* V, const void* P,
                          float scale, int causal, int B, int H, int N, int d, int m, int dv,
                          spa_dtype_t dtype, void* O, spa_dtype_t o_dtype, float* lse,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * spa_attn_fwd_noalloc -- spa_attn_fwd for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid allocation. Same
 * arguments and results as spa_attn_fwd without the workspace pair: the workspace is a
 * static device array inside the library, spa_attn_fwd_noalloc_max_workspace_bytes() bytes
 * (128 MiB) per GPU, which every GPU the library runs on holds until the process ends. The
 * call allocates nothing (no hipMalloc, no stream-ordered allocation). Sizes whose
 * spa_attn_fwd_workspace_bytes(...) exceeds that limit are rejected with
 * SPA_ERR_UNSUPPORTED before any HIP work; other errors as spa_attn_fwd. Every call on a GPU
 * shares that GPU's array, so calls that overlap on one GPU (on different streams, or from
 * several threads) race: serialize them. The array keeps the last call's contents; the
 * forward overwrites all of the workspace it reads, so nothing needs clearing.
 */
size_t spa_attn_fwd_noalloc_max_workspace_bytes(void);
spa_status_t spa_attn_fwd_noalloc(const void* Q, const void* K, const void* V, const void* P,
                                  float scale, int causal, int B, int H, int N, int d, int m,
                                  int dv, spa_dtype_t dtype, void* O, spa_dtype_t o_dtype,
                                  float* lse, void* stream);

/*
 * Workspace bytes spa_attn_bwd needs for these sizes (0 for arguments it would reject).
 * Contents (each region 256-byte aligned), bf16 path: the projected queries (scaled by
 * scale*log2(e)) and keys, fp16, row-major and transposed; dO transposed (bf16); the row
 * terms D_i = <dO_i, O_i> (fp32); the gradients of the projected queries and keys (fp32);
 * the projection gradient's per-256-row partial sums (fp32). fp32 path: the projected
 * queries and keys and their gradients (fp32 [B,H,N,m] each) and the row terms D (fp32).
 */
size_t spa_attn_bwd_workspace_bytes(int B, int H, int N, int d, int m, int dv,
                                    spa_dtype_t dtype);

/*
 * spa_attn_bwd -- gradients of a loss L through spa_attn_fwd, given dO = dL/dO: the chain
 * rule of the forward's definition (SPA page Sec. 3.1.3 and Algorithm 1; its Sec. 3.4.1
 * Gradient Flow writes the query term of the projection's gradient, and Algorithm 2 trains
 * the projection with it; the key term enters the same way). With A the forward's row
 * softmax:
 *
 *   D_i = <dO_i, O_i>,  dS_ij = A_ij (<dO_i, V_j> - D_i)
 *   dV_j = sum_i A_ij dO_i,  dQ = scale * (dS Kt) P^T,  dK = scale * (dS^T Qt) P^T
 *   dP_h = sum over batches of Q^T (scale dS Kt) + K^T (scale dS^T Qt)
 *
 *   Q, K, V, P, scale, causal, B, H, N, d, m, dv, dtype: as passed to spa_attn_fwd.
 *   O    [B,H,N,dv] the forward's output; dO [B,H,N,dv]; both in dtype.
 *   lse  [B,H,N] fp32, the forward's lse output (the weights are recomputed from it).
 *   dQ, dK [B,H,N,d] and dV [B,H,N,dv] in g_dtype (SPA_BF16 or SPA_F32; SPA_F32 only when
 *        dtype is SPA_F32); dP [H,d,m] fp32.
 *        No output may overlap an input, another output or the workspace.
 *   workspace / workspace_bytes: as for spa_attn_fwd, sized by
 *        spa_attn_bwd_workspace_bytes (NULL: allocated and freed stream-ordered).
 *
 * Supported: dtype SPA_BF16 with d in {64, 128}, dv in {64, 128}, 1 <= m <= 128; dtype
 * SPA_F32 with d <= 256, dv <= 128, m <= 128 (SPA_ERR_UNSUPPORTED otherwise). bf16: the
 * projected queries and keys are prepared exactly as in the forward (fp16), so the
 * recomputed scores match the forward's bit for bit; the weights meet dO in bf16 and dS
 * meets the projected operands in fp16, all on MFMA with fp32 accumulation; four launches
 * (five at m > 64). At m <= 64 the projected-query gradient is accumulated with fp32 atomic
 * adds, in an order that varies between runs: dQ and dP then agree run to run to rounding,
 * dK and dV bit for bit. fp32: every product and sum in fp32 on the VALU (the projections,
 * a query-major and a key-major pass, the gradients mapped back through P, and dP); seven
 * launches, deterministic. Both run on `stream`.
 */
spa_status_t spa_attn_bwd(const void* Q, const void* K, const void* V, const void* P,
                          const void* O, const void* dO, const float* lse, float scale,
                          int causal, int B, int H, int N, int d, int m, int dv,
                          spa_dtype_t dtype, void* dQ, void* dK, void* dV, float* dP,
                          spa_dtype_t g_dtype, void* workspace, size_t workspace_bytes,
                          void* stream);

/*
 * spa_sfa_fwd_workspace_bytes -- workspace bytes for spa_sfa_fwd (selected queries and keys,
 * fp16 [B,H,N,d] each; key-norm maxima; V^T), 0 if the shape is invalid or unsupported.
 */
size_t spa_sfa_fwd_workspace_bytes(int B, int H, int N, int d, int dv);

/*
 * spa_sfa_fwd -- sparse feature attention ("Scaling Attention via Feature Sparsity", key
 * designs 1 and 3): every row of Q and K keeps its topk features of largest magnitude
 * (ties: lower feature index first), the rest set to zero, and
 *
 *   O = softmax(scale * Topk(Q) Topk(K)^T [+ causal mask]) V       (exact)
 *
 *   Q, K   [B,H,N,d] bf16 (dtype SPA_BF16), d in {64, 128}; V [B,H,N,dv] bf16, dv in
 *          {64, 128}; 1 <= topk <= d.
 *   O, o_dtype, lse, workspace, workspace_bytes, stream: as for spa_attn_fwd (workspace
 *          sized by spa_sfa_fwd_workspace_bytes).
 *
 * Three launches: the Top-k selection (fp16 operands, queries times scale*log2 e), the V
 * transpose, and the streamed attention kernel of spa_attn_fwd with m = d. Errors as for
 * spa_attn_fwd; topk outside [1, d] is SPA_ERR_INVALID_ARGUMENT.
 */
spa_status_t spa_sfa_fwd(const void* Q, const void* K, const void* V, int topk, float scale,
                         int causal, int B, int H, int N, int d, int dv, spa_dtype_t dtype,
                         void* O, spa_dtype_t o_dtype, float* lse, void* workspace,
                         size_t workspace_bytes, void* stream);

/*
 * spa_kcache_append -- write projected keys into a key cache (SPA page Sec. 3.1.2: keys
 * enter the scores only through Kt = K P, so a cache of Kt serves every later query):
 *
 *   cache[b, h, row0 + n, :] = fp16(K[b, h, n, :] . P[h])   for 0 <= n < N
 *
 *   K      [B,H,N,d] bf16 (dtype SPA_BF16; d in {64, 128}), the new keys.
 *   P      [H,d,m] bf16, 1 <= m <= 128.
 *   cache  [B,H,rows,m] fp16 (device, caller-owned), rows per head >= row0 + N; rows outside
 *          [row0, row0 + N) are not touched. fp32 accumulation, one RNE rounding to fp16.
 *
 * 16-byte aligned bases; the cache may not overlap K or P. One launch on `stream`.
 */
spa_status_t spa_kcache_append(const void* K, const void* P, void* cache, int B, int H, int N,
                               int d, int m, int rows, int row0, spa_dtype_t dtype,
                               void* stream);

/*
 * spa_attn_decode_workspace_bytes -- bytes of scratch spa_attn_decode needs (per query and
 * key split dv + 2 floats: the split's unnormalised output, running maximum and sum), 0 if
 * the shape is invalid or unsupported.
 */
size_t spa_attn_decode_workspace_bytes(int B, int H, int Nq, int Nk, int dv);

/*
 * spa_attn_decode -- Nq queries against the first Nk rows of a projected-key cache and a
 * value cache: the forward of spa_attn_fwd (SPA page Sec. 3.1.3, Algorithm 1; PDA page
 * Algorithm 2.1 steps 1-3 and 5) with the keys given as Kt = K P:
 *
 *   O[b,h,i,:] = sum_j softmax_j(scale * (Q[b,h,i,:] P[h]) . cache[b,h,j,:]) Vc[b,h,j,:]
 *
 * over keys j < Nk; with causal = 1 the mask is aligned to the end of the cache: query i
 * sits at position Nk - Nq + i and sees keys j <= Nk - Nq + i (so Nq = Nk reproduces the
 * square causal forward, and Nq = 1 is one decode step).
 *
 *   Q      [B,H,Nq,d] bf16 (dtype SPA_BF16), d in {64, 128}; P [H,d,m] bf16, 1 <= m <= 128.
 *   cache  [B,H,rows,m] fp16, written by spa_kcache_append; Vc [B,H,rows,dv] bf16,
 *          dv in {64, 128}; 1 <= Nq <= Nk <= rows.
 *   O      [B,H,Nq,dv] in o_dtype (SPA_F32 or SPA_BF16); lse [B,H,Nq] fp32 (natural log of
 *          the softmax normaliser of the scaled scores) or NULL.
 *   workspace / workspace_bytes: spa_attn_decode_workspace_bytes(B, H, Nq, Nk, dv) bytes,
 *          or NULL (allocated and freed stream-ordered).
 *
 * Queries are projected in fp32. Up to four queries per head (or m not a multiple of 8):
 * scores, an exact online softmax and the weights x V in fp32 on the vector units. More
 * (m a multiple of 8): queries rounded to fp16 and weights to bf16 on the matrix cores,
 * fp32 accumulation and softmax state. Each cache byte is read once per head and group of
 * up to 16 queries.
 * Keys are split across workgroups and the splits merged in a fixed order: deterministic.
 * Errors: SPA_ERR_INVALID_ARGUMENT (nulls, dimensions, alignment, overlaps, Nq > Nk > rows),
 * SPA_ERR_UNSUPPORTED (dtype, d, m, dv), SPA_ERR_WORKSPACE, SPA_ERR_HIP. Two launches: the
 * attention over the key splits, then the merge of the splits.
 */
spa_status_t spa_attn_decode(const void* Q, const void* cache, const void* Vc, const void* P,
                             float scale, int causal, int B, int H, int Nq, int Nk, int rows,
                             int d, int m, int dv, spa_dtype_t dtype, void* O,
                             spa_dtype_t o_dtype, float* lse, void* workspace,
                             size_t workspace_bytes, void* stream);

/*
 * Per-launch timing for benchmarks. spa_profile_begin(max_calls) starts recording HIP
 * events around the projection and attention launches of the next max_calls spa_attn_fwd
 * calls (1 <= max_calls <= 65536; fails with SPA_ERR_INVALID_ARGUMENT if a recording is
 * already open). spa_profile_end() waits for the last recorded event and returns the summed
 * milliseconds of each launch and the number of calls recorded; any output pointer may be
 * NULL. Timing is process-wide state: do not record from several threads at once.
 */
spa_status_t spa_profile_begin(int max_calls);
spa_status_t spa_profile_end(double* project_ms, double* attn_ms, int* calls);

/*
 * Rate probes for the benchmark's roofline context (not part of the attention path): the
 * sustained rate of the bf16 matrix core (32x32x16 MFMAs on random operands, one wave per
 * SIMD, every CU) and of fp32 VALU FMAs (four waves per SIMD), in TFLOP/s, each over 100
 * back-to-back launches (the rate of the second half), with the mean engine clock in GHz
 * during the last launch (shader-clock counter against the 100 MHz counter). Runs
 * synchronously on `stream` (about 80 ms) and allocates a few KB of device memory for the
 * duration of the call. Every output pointer must be non-NULL (else SPA_ERR_INVALID_ARGUMENT);
 * SPA_ERR_HIP if a HIP call fails.
 */
spa_status_t spa_probe_rates(double* mfma_tflops, double* mfma_ghz, double* fma_tflops,
                             double* fma_ghz, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SPA_H */
