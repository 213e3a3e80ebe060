/*
 * spa_oracle.c -- plain, slow, double-precision CPU oracle for feature-axis projected
 * softmax attention.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test-suite, the package smoke check and the
 * benchmark's CPU-baseline leg load this library. It shares no code, header, table or helper
 * with the HIP path, and the HIP path never calls it.
 *
 * What it computes, for every batch b and head h, with the projection P_h in R^{d x m}:
 *
 *   Qt = Q P_h,  Kt = K P_h
 *       "Sparse Projection Attention" (SPA) page, Sec. 3.1.2 (projection layer) and
 *       Algorithm 1 steps 2-3; "Projection-Decomposition Attention" (PDA) page,
 *       Algorithm 2.1 step 1 (one P shared by queries and keys).
 *   St_ij = scale * <Qt_i, Kt_j>, and -infinity when causal and j > i
 *       SPA page Sec. 3.1.3 and Algorithm 1 step 4; PDA page Algorithm 2.1 step 2. The scale
 *       is a caller argument: the SPA page divides by sqrt(m), PDA's Algorithm 2.1 by
 *       sqrt(m), and PDA's revised proof (Sec. 2.1) keeps the exact-score scale 1/sqrt(d).
 *   A_i = softmax(St_i)   (row-wise; PDA revised proof Sec. 1.1 defines the row softmax)
 *       SPA Algorithm 1 step 5; PDA Algorithm 2.1 step 3.
 *   O = A V
 *       SPA Algorithm 1 step 6; PDA Algorithm 2.1 step 5 with step 4 (the SVD truncation)
 *       left out.
 *
 * The softmax is the plain two-pass form: the row maximum over the unmasked keys, then
 * exp(s - max), their sum, and the weights divided by the sum. Sums run over ascending
 * indices. Nothing is blocked, fused or reordered beyond that.
 *
 * All arrays are dense row-major double: Q, K [B,H,N,d]; V, O [B,H,N,dv]; P [H,d,m];
 * Qt, Kt [B,H,N,m]; S, A [B,H,N,N]; lse [B,H,N].
 * Every entry point returns 0 on success, -1 on a bad argument, -2 if memory runs out.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

static int threads_to_use(int nthreads) {
#ifdef _OPENMP
    return nthreads > 0 ? nthreads : omp_get_max_threads();
#else
    (void)nthreads;
    return 1;
#endif
}

/* Number of threads an entry point uses for a given request (0 = all). */
int spa_oracle_threads(int nthreads) { return threads_to_use(nthreads); }

/* x_row (length d) times P_h (d x m) -> out (length m). */
static void project_row(const double* x, const double* ph, int64_t d, int64_t m, double* out) {
    for (int64_t c = 0; c < m; ++c) {
        double acc = 0.0;
        for (int64_t k = 0; k < d; ++k) acc += x[k] * ph[k * m + c];
        out[c] = acc;
    }
}

/*
 * Xt[b,h,n,:] = X[b,h,n,:] P[h]  (SPA Sec. 3.1.2; PDA Algorithm 2.1 step 1).
 */
int spa_oracle_project(const double* X, const double* P, double* Xt, int64_t B, int64_t H,
                       int64_t N, int64_t d, int64_t m, int nthreads) {
    if (!X || !P || !Xt || B < 1 || H < 1 || N < 1 || d < 1 || m < 1) return -1;
    const int64_t rows = B * H * N;
#pragma omp parallel for schedule(static) num_threads(threads_to_use(nthreads))
    for (int64_t r = 0; r < rows; ++r) {
        const int64_t h = (r / N) % H;
        project_row(X + r * d, P + h * d * m, d, m, Xt + r * m);
    }
    return 0;
}

/* Unmasked keys of query i: 0..N-1, or 0..i when causal. */
static int64_t key_count(int64_t i, int64_t N, int causal) { return causal ? i + 1 : N; }

/*
 * One output row. qt: projected query (m); Kt: projected keys of the head (N x m);
 * V: values of the head (N x dv); w: scratch of length >= nkeys.
 * Writes o (dv) and, if lse != NULL, the log of the softmax normaliser, max + log(sum).
 */
static void attend_row(const double* qt, const double* Kt, const double* V, int64_t nkeys,
                       int64_t m, int64_t dv, double scale, double* w, double* o,
                       double* lse) {
    /* scores over the unmasked keys */
    for (int64_t j = 0; j < nkeys; ++j) {
        double acc = 0.0;
        for (int64_t c = 0; c < m; ++c) acc += qt[c] * Kt[j * m + c];
        w[j] = scale * acc;
    }
    /* pass 1: row maximum */
    double mx = -INFINITY;
    for (int64_t j = 0; j < nkeys; ++j)
        if (w[j] > mx) mx = w[j];
    /* pass 2: exponentials and their sum */
    double sum = 0.0;
    for (int64_t j = 0; j < nkeys; ++j) {
        w[j] = exp(w[j] - mx);
        sum += w[j];
    }
    /* weights times values */
    for (int64_t c = 0; c < dv; ++c) o[c] = 0.0;
    for (int64_t j = 0; j < nkeys; ++j) {
        const double a = w[j] / sum;
        const double* vj = V + j * dv;
        for (int64_t c = 0; c < dv; ++c) o[c] += a * vj[c];
    }
    if (lse) *lse = mx + log(sum);
}

static int check_attn_args(const void* Q, const void* K, const void* V, const void* P,
                           double scale, int causal, int64_t B, int64_t H, int64_t N,
                           int64_t d, int64_t m, int64_t dv) {
    if (!Q || !K || !V || !P) return -1;
    if (B < 1 || H < 1 || N < 1 || d < 1 || m < 1 || dv < 1) return -1;
    if (causal != 0 && causal != 1) return -1;
    if (!isfinite(scale)) return -1;
    return 0;
}

/*
 * Full forward: O[b,h,i,:] = sum_j softmax_j(scale <Qt_i, Kt_j> [causal: j <= i]) V[b,h,j,:].
 * lse may be NULL.
 */
int spa_oracle_attn_fwd(const double* Q, const double* K, const double* V, const double* P,
                        double scale, int causal, int64_t B, int64_t H, int64_t N, int64_t d,
                        int64_t m, int64_t dv, double* O, double* lse, int nthreads) {
    if (check_attn_args(Q, K, V, P, scale, causal, B, H, N, d, m, dv) || !O) return -1;
    const int nt = threads_to_use(nthreads);
    const int64_t BH = B * H;
    double* Qt = (double*)malloc(sizeof(double) * (size_t)(BH * N * m));
    double* Kt = (double*)malloc(sizeof(double) * (size_t)(BH * N * m));
    double* scratch = (double*)malloc(sizeof(double) * (size_t)N * (size_t)nt);
    if (!Qt || !Kt || !scratch) {
        free(Qt);
        free(Kt);
        free(scratch);
        return -2;
    }
    spa_oracle_project(Q, P, Qt, B, H, N, d, m, nt);
    spa_oracle_project(K, P, Kt, B, H, N, d, m, nt);
    const int64_t rows = BH * N;
#pragma omp parallel for schedule(dynamic, 16) num_threads(nt)
    for (int64_t r = 0; r < rows; ++r) {
        int tid = 0;
#ifdef _OPENMP
        tid = omp_get_thread_num();
#endif
        const int64_t bh = r / N, i = r % N;
        attend_row(Qt + r * m, Kt + bh * N * m, V + bh * N * dv, key_count(i, N, causal), m,
                   dv, scale, scratch + (size_t)tid * (size_t)N, O + r * dv,
                   lse ? lse + r : NULL);
    }
    free(Qt);
    free(Kt);
    free(scratch);
    return 0;
}

/*
 * The same forward on a sample of rows: row k of the output is query row_i[k] of flattened
 * head row_bh[k] (bh = b*H + h). O_rows [nrows, dv]; lse_rows [nrows] or NULL.
 * Only the heads that appear in the sample are projected.
 */
int spa_oracle_attn_rows(const double* Q, const double* K, const double* V, const double* P,
                         double scale, int causal, int64_t B, int64_t H, int64_t N, int64_t d,
                         int64_t m, int64_t dv, const int64_t* row_bh, const int64_t* row_i,
                         int64_t nrows, double* O_rows, double* lse_rows, int nthreads) {
    if (check_attn_args(Q, K, V, P, scale, causal, B, H, N, d, m, dv)) return -1;
    if (nrows < 0 || (nrows > 0 && (!row_bh || !row_i || !O_rows))) return -1;
    const int64_t BH = B * H;
    for (int64_t k = 0; k < nrows; ++k)
        if (row_bh[k] < 0 || row_bh[k] >= BH || row_i[k] < 0 || row_i[k] >= N) return -1;
    const int nt = threads_to_use(nthreads);
    /* map each needed head to a slot of projected keys */
    int64_t* slot = (int64_t*)malloc(sizeof(int64_t) * (size_t)BH);
    if (!slot) return -2;
    for (int64_t bh = 0; bh < BH; ++bh) slot[bh] = -1;
    int64_t nheads = 0;
    for (int64_t k = 0; k < nrows; ++k)
        if (slot[row_bh[k]] < 0) slot[row_bh[k]] = nheads++;
    int64_t* heads = (int64_t*)malloc(sizeof(int64_t) * (size_t)(nheads > 0 ? nheads : 1));
    double* Kt = (double*)malloc(sizeof(double) * (size_t)((nheads > 0 ? nheads : 1) * N * m));
    double* scratch = (double*)malloc(sizeof(double) * (size_t)(N + m) * (size_t)nt);
    if (!heads || !Kt || !scratch) {
        free(slot);
        free(heads);
        free(Kt);
        free(scratch);
        return -2;
    }
    for (int64_t bh = 0; bh < BH; ++bh)
        if (slot[bh] >= 0) heads[slot[bh]] = bh;
    const int64_t krows = nheads * N;
#pragma omp parallel for schedule(static) num_threads(nt)
    for (int64_t r = 0; r < krows; ++r) {
        const int64_t bh = heads[r / N], n = r % N;
        project_row(K + (bh * N + n) * d, P + (bh % H) * d * m, d, m, Kt + r * m);
    }
#pragma omp parallel for schedule(dynamic, 4) num_threads(nt)
    for (int64_t k = 0; k < nrows; ++k) {
        int tid = 0;
#ifdef _OPENMP
        tid = omp_get_thread_num();
#endif
        double* qt = scratch + (size_t)tid * (size_t)(N + m);
        double* w = qt + m;
        const int64_t bh = row_bh[k], i = row_i[k];
        project_row(Q + (bh * N + i) * d, P + (bh % H) * d * m, d, m, qt);
        attend_row(qt, Kt + slot[bh] * N * m, V + bh * N * dv, key_count(i, N, causal), m, dv,
                   scale, w, O_rows + k * dv, lse_rows ? lse_rows + k : NULL);
    }
    free(slot);
    free(heads);
    free(Kt);
    free(scratch);
    return 0;
}

/*
 * Projected score matrix S[b,h,i,j] = scale <Qt_i, Kt_j>, or -infinity where the causal
 * mask removes (i, j) (SPA Algorithm 1 step 4; PDA Algorithm 2.1 step 2).
 */
int spa_oracle_scores(const double* Q, const double* K, const double* P, double scale,
                      int causal, int64_t B, int64_t H, int64_t N, int64_t d, int64_t m,
                      double* S, int nthreads) {
    if (!Q || !K || !P || !S || B < 1 || H < 1 || N < 1 || d < 1 || m < 1) return -1;
    if ((causal != 0 && causal != 1) || !isfinite(scale)) return -1;
    const int nt = threads_to_use(nthreads);
    const int64_t BH = B * H;
    double* Qt = (double*)malloc(sizeof(double) * (size_t)(BH * N * m));
    double* Kt = (double*)malloc(sizeof(double) * (size_t)(BH * N * m));
    if (!Qt || !Kt) {
        free(Qt);
        free(Kt);
        return -2;
    }
    spa_oracle_project(Q, P, Qt, B, H, N, d, m, nt);
    spa_oracle_project(K, P, Kt, B, H, N, d, m, nt);
    const int64_t rows = BH * N;
#pragma omp parallel for schedule(static) num_threads(nt)
    for (int64_t r = 0; r < rows; ++r) {
        const int64_t bh = r / N, i = r % N;
        const double* qt = Qt + r * m;
        for (int64_t j = 0; j < N; ++j) {
            double v;
            if (causal && j > i) {
                v = -INFINITY;
            } else {
                double acc = 0.0;
                const double* kt = Kt + (bh * N + j) * m;
                for (int64_t c = 0; c < m; ++c) acc += qt[c] * kt[c];
                v = scale * acc;
            }
            S[r * N + j] = v;
        }
    }
    free(Qt);
    free(Kt);
    return 0;
}

/*
 * Attention weights A[b,h,i,:] = softmax(S[b,h,i,:]) with S as in spa_oracle_scores and the
 * same two-pass softmax as the forward (masked entries get weight 0).
 */
int spa_oracle_weights(const double* Q, const double* K, const double* P, double scale,
                       int causal, int64_t B, int64_t H, int64_t N, int64_t d, int64_t m,
                       double* A, int nthreads) {
    int rc = spa_oracle_scores(Q, K, P, scale, causal, B, H, N, d, m, A, nthreads);
    if (rc) return rc;
    const int64_t rows = B * H * N;
#pragma omp parallel for schedule(static) num_threads(threads_to_use(nthreads))
    for (int64_t r = 0; r < rows; ++r) {
        double* a = A + r * N;
        const int64_t nkeys = key_count(r % N, N, causal);
        double mx = -INFINITY;
        for (int64_t j = 0; j < nkeys; ++j)
            if (a[j] > mx) mx = a[j];
        double sum = 0.0;
        for (int64_t j = 0; j < nkeys; ++j) {
            a[j] = exp(a[j] - mx);
            sum += a[j];
        }
        for (int64_t j = 0; j < nkeys; ++j) a[j] /= sum;
        for (int64_t j = nkeys; j < N; ++j) a[j] = 0.0;
    }
    return 0;
}

/*
 * Backward of spa_oracle_attn_fwd for a loss L with dL/dO = dO: the chain rule of the
 * definition above. The "Sparse Projection Attention" page, Sec. 3.4.1 (Gradient Flow),
 * writes the query term of dL/dP, and its Algorithm 2 trains the projection with it; P
 * multiplies the keys too, so the key term enters the same way. Per (b, h), with A the row softmax and
 * O = A V as in the forward:
 *
 *   D_i    = sum_c dO_ic O_ic
 *   dA_ij  = sum_c dO_ic V_jc
 *   dS_ij  = A_ij (dA_ij - D_i)            (zero where the causal mask removes the key)
 *   dV_j   = sum_i A_ij dO_i
 *   dQt_i  = scale sum_j dS_ij Kt_j,       dKt_j = scale sum_i dS_ij Qt_i
 *   dQ     = dQt P_h^T,  dK = dKt P_h^T,   dP_h = sum_b (Q^T dQt + K^T dKt)
 *
 * Rows are visited in ascending order within a head, heads in parallel; dP is summed over
 * b in ascending order at the end. Arrays: dO, dV [B,H,N,dv]; dQ, dK [B,H,N,d]; dP [H,d,m].
 */
int spa_oracle_attn_bwd(const double* Q, const double* K, const double* V, const double* P,
                        const double* dO, double scale, int causal, int64_t B, int64_t H,
                        int64_t N, int64_t d, int64_t m, int64_t dv, double* dQ, double* dK,
                        double* dV, double* dP, int nthreads) {
    if (check_attn_args(Q, K, V, P, scale, causal, B, H, N, d, m, dv)) return -1;
    if (!dO || !dQ || !dK || !dV || !dP) return -1;
    const int nt = threads_to_use(nthreads);
    const int64_t BH = B * H;
    double* dPp = (double*)calloc((size_t)(BH * d * m), sizeof(double));
    if (!dPp) return -2;
    int failed = 0;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nt)
    for (int64_t bh = 0; bh < BH; ++bh) {
        const int64_t h = bh % H;
        const double* ph = P + h * d * m;
        const double* Qh = Q + bh * N * d;
        const double* Kh = K + bh * N * d;
        const double* Vh = V + bh * N * dv;
        const double* dOh = dO + bh * N * dv;
        double* dVh = dV + bh * N * dv;
        double* Qt = (double*)malloc(sizeof(double) * (size_t)(N * m));
        double* Kt = (double*)malloc(sizeof(double) * (size_t)(N * m));
        double* dQt = (double*)calloc((size_t)(N * m), sizeof(double));
        double* dKt = (double*)calloc((size_t)(N * m), sizeof(double));
        double* a = (double*)malloc(sizeof(double) * (size_t)N);
        double* o = (double*)malloc(sizeof(double) * (size_t)dv);
        if (!Qt || !Kt || !dQt || !dKt || !a || !o) {
#pragma omp atomic write
            failed = 1;
        } else {
            for (int64_t n = 0; n < N; ++n) {
                project_row(Qh + n * d, ph, d, m, Qt + n * m);
                project_row(Kh + n * d, ph, d, m, Kt + n * m);
            }
            for (int64_t j = 0; j < N * dv; ++j) dVh[j] = 0.0;
            for (int64_t i = 0; i < N; ++i) {
                const int64_t nk = key_count(i, N, causal);
                /* the forward's row: scores, two-pass softmax, output */
                for (int64_t j = 0; j < nk; ++j) {
                    double acc = 0.0;
                    for (int64_t c = 0; c < m; ++c) acc += Qt[i * m + c] * Kt[j * m + c];
                    a[j] = scale * acc;
                }
                double mx = -INFINITY;
                for (int64_t j = 0; j < nk; ++j)
                    if (a[j] > mx) mx = a[j];
                double sum = 0.0;
                for (int64_t j = 0; j < nk; ++j) {
                    a[j] = exp(a[j] - mx);
                    sum += a[j];
                }
                for (int64_t j = 0; j < nk; ++j) a[j] /= sum;
                for (int64_t c = 0; c < dv; ++c) o[c] = 0.0;
                for (int64_t j = 0; j < nk; ++j)
                    for (int64_t c = 0; c < dv; ++c) o[c] += a[j] * Vh[j * dv + c];
                /* D_i */
                double Di = 0.0;
                for (int64_t c = 0; c < dv; ++c) Di += dOh[i * dv + c] * o[c];
                /* per key: dA, dS, and the three accumulations */
                for (int64_t j = 0; j < nk; ++j) {
                    double dA = 0.0;
                    for (int64_t c = 0; c < dv; ++c) dA += dOh[i * dv + c] * Vh[j * dv + c];
                    const double dS = a[j] * (dA - Di);
                    for (int64_t c = 0; c < dv; ++c) dVh[j * dv + c] += a[j] * dOh[i * dv + c];
                    for (int64_t c = 0; c < m; ++c) {
                        dQt[i * m + c] += scale * dS * Kt[j * m + c];
                        dKt[j * m + c] += scale * dS * Qt[i * m + c];
                    }
                }
            }
            /* back through the projection */
            for (int64_t n = 0; n < N; ++n)
                for (int64_t k = 0; k < d; ++k) {
                    double gq = 0.0, gk = 0.0;
                    for (int64_t c = 0; c < m; ++c) {
                        gq += dQt[n * m + c] * ph[k * m + c];
                        gk += dKt[n * m + c] * ph[k * m + c];
                    }
                    dQ[(bh * N + n) * d + k] = gq;
                    dK[(bh * N + n) * d + k] = gk;
                }
            double* dPb = dPp + bh * d * m;
            for (int64_t n = 0; n < N; ++n)
                for (int64_t k = 0; k < d; ++k)
                    for (int64_t c = 0; c < m; ++c)
                        dPb[k * m + c] += Qh[n * d + k] * dQt[n * m + c] + Kh[n * d + k] * dKt[n * m + c];
        }
        free(Qt);
        free(Kt);
        free(dQt);
        free(dKt);
        free(a);
        free(o);
    }
    if (!failed) {
        for (int64_t h = 0; h < H; ++h)
            for (int64_t e = 0; e < d * m; ++e) {
                double acc = 0.0;
                for (int64_t b = 0; b < B; ++b) acc += dPp[(b * H + h) * d * m + e];
                dP[h * d * m + e] = acc;
            }
    }
    free(dPp);
    return failed ? -2 : 0;
}
