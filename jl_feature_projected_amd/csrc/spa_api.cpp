// spa_api.cpp -- the C ABI of libspa: argument validation, workspace handling, dispatch to
// the HIP kernels, status codes and per-launch timing.
//
// Every argument check runs on the host before the first HIP call, so a rejected call
// leaves the device and the stream untouched.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <vector>

#include "../../include/spa.h"
#include "spa_internal.h"

namespace {

constexpr int kMaxN = 1 << 22;
constexpr long long kMaxRows = 1LL << 31;  // B*H*N bound on every path

thread_local char g_err[512] = "";

spa_status_t fail(spa_status_t st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
spa_status_t fail(spa_status_t st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return st;
}

spa_status_t hip_fail(const char* where, hipError_t e) {
    return fail(SPA_ERR_HIP, "%s: %s (%d)", where, hipGetErrorString(e), (int)e);
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

struct Range {
    uintptr_t lo, hi;  // [lo, hi)
};
Range range(const void* p, size_t bytes) {
    const uintptr_t b = reinterpret_cast<uintptr_t>(p);
    return {b, b + bytes};
}
bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

size_t elem_size(spa_dtype_t t) { return t == SPA_BF16 ? 2 : 4; }

// Workspace layout: projected queries, projected keys, and (bf16 path) the per-block key
// norm maxima and V^T, each 256-byte aligned.
struct WorkspaceLayout {
    size_t tilde_bytes;  // one projected tensor
    size_t k_offset;
    size_t kmax_offset;
    size_t vt_offset;
    size_t total;
};
size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
WorkspaceLayout workspace_layout(int BH, int N, int m, int dv, spa_dtype_t dtype) {
    const long long rows = (long long)BH * N;
    const int cols = dtype == SPA_BF16 ? spa::padded_m(m) : m;
    WorkspaceLayout w;
    w.tilde_bytes = (size_t)rows * cols * elem_size(dtype);
    w.k_offset = align256(w.tilde_bytes);
    w.kmax_offset = align256(w.k_offset + w.tilde_bytes);
    if (dtype == SPA_BF16) {
        w.vt_offset = align256(w.kmax_offset + (size_t)BH * spa::proj_blocks(N) * sizeof(float));
        w.total = w.vt_offset + (size_t)BH * dv * spa::vt_padded_keys(N) * 2;
    } else {
        w.vt_offset = w.kmax_offset;
        w.total = w.kmax_offset;
    }
    return w;
}

// Backward workspace (bf16 path), each region 256-byte aligned: projected queries (scaled)
// and keys, fp16 [BH, N, mp] each; the same transposed, fp16 [BH, mp, Np] each; dO
// transposed, bf16 [BH, dv, Np]; per query -lse*log2(e) and -D (D = <dO, O>), fp32
// [BH, Np/32, 2, 32]; the projected gradients, fp32 [BH, N, mp]
// each; the projection gradient's partials, fp32 [BH, ceil(N / 256), d, m].
struct BwdLayout {
    size_t qs, kt, qst, ktt, dot, ld, dqt, dkt, part, total;
};
BwdLayout bwd_layout(int BH, int N, int d, int m, int dv) {
    const size_t mp = (size_t)spa::padded_m(m), np = (size_t)spa::vt_padded_keys(N);
    const size_t rows = (size_t)BH * N;
    BwdLayout w;
    size_t o = 0;
    auto take = [&](size_t bytes) {
        const size_t at = o;
        o = align256(o + bytes);
        return at;
    };
    w.qs = take(rows * mp * 2);
    w.kt = take(rows * mp * 2);
    w.qst = take((size_t)BH * mp * np * 2);
    w.ktt = take((size_t)BH * mp * np * 2);
    w.dot = take((size_t)BH * dv * np * 2);
    w.ld = take((size_t)BH * np * 2 * 4);
    w.dqt = take(rows * mp * 4);
    w.dkt = take(rows * mp * 4);
    w.part = take((size_t)BH * ((N + 255) / 256) * d * m * 4);
    w.total = o;
    return w;
}

// fp32 backward workspace: the projected queries and keys, their gradients (fp32 [B*H, N, m]
// each) and the row terms D (fp32 [B*H, N]), each region 256-byte aligned.
struct BwdF32Layout {
    size_t qt, kt, dqt, dkt, dd, total;
};
BwdF32Layout bwd_f32_layout(int BH, int N, int m) {
    const size_t rows = (size_t)BH * N;
    BwdF32Layout w;
    size_t o = 0;
    auto take = [&](size_t bytes) {
        const size_t at = o;
        o = align256(o + bytes);
        return at;
    };
    w.qt = take(rows * m * 4);
    w.kt = take(rows * m * 4);
    w.dqt = take(rows * m * 4);
    w.dkt = take(rows * m * 4);
    w.dd = take(rows * 4);
    w.total = o;
    return w;
}

spa_status_t check_dims(const char* fn, int B, int H, int N, int d, int m, int dv) {
    if (B < 1 || H < 1 || N < 1 || d < 1 || m < 1 || dv < 1)
        return fail(SPA_ERR_INVALID_ARGUMENT,
                    "%s: every dimension must be >= 1 (B=%d H=%d N=%d d=%d m=%d dv=%d)", fn, B,
                    H, N, d, m, dv);
    if (N > kMaxN) return fail(SPA_ERR_UNSUPPORTED, "%s: N=%d exceeds %d", fn, N, kMaxN);
    if ((long long)B * H * N >= kMaxRows)
        return fail(SPA_ERR_UNSUPPORTED, "%s: B*H*N=%lld exceeds 2^31", fn,
                    (long long)B * H * N);
    return SPA_OK;
}

spa_status_t check_shape_support(const char* fn, spa_dtype_t dtype, int d, int m, int dv) {
    if (dtype == SPA_BF16) {
        if (d != 64 && d != 128)
            return fail(SPA_ERR_UNSUPPORTED, "%s: bf16 path needs d in {64,128}, got %d", fn, d);
        if (m > 128)
            return fail(SPA_ERR_UNSUPPORTED, "%s: bf16 path needs m <= 128, got %d", fn, m);
        if (dv != 64 && dv != 128)
            return fail(SPA_ERR_UNSUPPORTED, "%s: bf16 path needs dv in {64,128}, got %d", fn,
                        dv);
        return SPA_OK;
    }
    if (dtype == SPA_F32) {
        if (d > 256 || m > 128 || dv > 128)
            return fail(SPA_ERR_UNSUPPORTED,
                        "%s: fp32 path needs d <= 256, m <= 128, dv <= 128 (d=%d m=%d dv=%d)",
                        fn, d, m, dv);
        return SPA_OK;
    }
    return fail(SPA_ERR_INVALID_ARGUMENT, "%s: unknown dtype %d", fn, (int)dtype);
}

// ---- launch timing ----------------------------------------------------------------------
struct Profile {
    std::mutex mu;
    bool on = false;
    int max_calls = 0;
    int calls = 0;
    std::vector<hipEvent_t> ev;  // 3 per call: before projection, between, after attention
} g_prof;

}  // namespace

extern "C" {

int spa_version(void) { return 100; }

const char* spa_status_string(spa_status_t s) {
    switch (s) {
        case SPA_OK: return "SPA_OK";
        case SPA_ERR_INVALID_ARGUMENT: return "SPA_ERR_INVALID_ARGUMENT";
        case SPA_ERR_UNSUPPORTED: return "SPA_ERR_UNSUPPORTED";
        case SPA_ERR_WORKSPACE: return "SPA_ERR_WORKSPACE";
        case SPA_ERR_HIP: return "SPA_ERR_HIP";
        default: break;
    }
    return "SPA_ERR_UNKNOWN";
}

const char* spa_last_error(void) { return g_err; }

spa_status_t spa_project(const void* X, const void* P, void* Xt, int B, int H, int N, int d,
                         int m, spa_dtype_t dtype, void* stream) {
    g_err[0] = '\0';
    const char* fn = "spa_project";
    if (!X || !P || !Xt) return fail(SPA_ERR_INVALID_ARGUMENT, "%s: null tensor pointer", fn);
    spa_status_t st = check_dims(fn, B, H, N, d, m, 1);
    if (st != SPA_OK) return st;
    if (dtype != SPA_BF16 && dtype != SPA_F32)
        return fail(SPA_ERR_INVALID_ARGUMENT, "%s: unknown dtype %d", fn, (int)dtype);
    if (dtype == SPA_BF16 ? (d != 64 && d != 128) || m > 128 : d > 256 || m > 128)
        return fail(SPA_ERR_UNSUPPORTED, "%s: unsupported d=%d m=%d for %s", fn, d, m,
                    dtype == SPA_BF16 ? "bf16" : "fp32");
    if (!aligned(X, 16) || !aligned(P, 16) || !aligned(Xt, 16))
        return fail(SPA_ERR_INVALID_ARGUMENT, "%s: tensor base not 16-byte aligned", fn);
    const size_t es = elem_size(dtype);
    const long long rows = (long long)B * H * N;
    const Range rx = range(X, rows * d * es), rp = range(P, (size_t)H * d * m * es),
                ry = range(Xt, rows * m * es);
    if (overlap(ry, rx) || overlap(ry, rp))
        return fail(SPA_ERR_INVALID_ARGUMENT, "%s: output overlaps an input", fn);

    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    if (dtype == SPA_BF16)
        e = spa::launch_project_bf16(X, nullptr, P, Xt, nullptr, 1, B * H, H, N, d, m, m, m,
                                     1.0f, 1.0f, /*out_f16=*/false, nullptr, nullptr, nullptr,
                                     0, s);
    else
        e = spa::launch_project_f32(static_cast<const float*>(X), static_cast<const float*>(P),
                                    static_cast<float*>(Xt), B * H, H, N, d, m, 1.0f, s);
    if (e != hipSuccess) return hip_fail(fn, e);
    return SPA_OK;
}

size_t spa_attn_fwd_workspace_bytes(int B, int H, int N, int d, int m, int dv,
                                    spa_dtype_t dtype) {
    char saved[sizeof(g_err)];
    memcpy(saved, g_err, sizeof(g_err));
    size_t out = 0;
    if (check_dims("spa_attn_fwd_workspace_bytes", B, H, N, d, m, dv) == SPA_OK &&
        check_shape_support("spa_attn_fwd_workspace_bytes", dtype, d, m, dv) == SPA_OK)
        out = workspace_layout(B * H, N, m, dv, dtype).total;
    memcpy(g_err, saved, sizeof(g_err));
    return out;
}

int spa_attn_fwd_plan(int B, int H, int N, int d, int m, int dv, spa_dtype_t dtype,
                      int causal) {
    char saved[sizeof(g_err)];
    memcpy(saved, g_err, sizeof(g_err));
    int out = -1;
    if (check_dims("spa_attn_fwd_plan", B, H, N, d, m, dv) == SPA_OK &&
        check_shape_support("spa_attn_fwd_plan", dtype, d, m, dv) == SPA_OK &&
        (causal == 0 || causal == 1)) {
        out = 0;
        if (dtype == SPA_BF16) {
            const int mp = spa::padded_m(m);
            if (spa::attn_bf16_projects_queries(B * H, N, mp, d, causal == 1))
                out |= SPA_PLAN_QUERIES_IN_ATTENTION;
            if (spa::attn_bf16_reads_v_rows(B * H, N, mp, dv, causal == 1))
                out |= SPA_PLAN_V_ROW_MAJOR;
        }
    }
    memcpy(g_err, saved, sizeof(g_err));
    return out;
}

}  // extern "C"

namespace {

// The forward behind spa_attn_fwd and spa_attn_fwd_noalloc. A null workspace is allocated
// stream-ordered (spa_attn_fwd only: the allocation-free entry point always passes one);
// `timed` lets the launch timing of spa_profile_begin record events.
spa_status_t attn_fwd_impl(const char* fn, const void* Q, const void* K, const void* V,
                           const void* P, float scale, int causal, int B, int H, int N, int d,
                           int m, int dv, spa_dtype_t dtype, void* O, spa_dtype_t o_dtype,
                           float* lse, void* workspace, size_t workspace_bytes, void* stream,
                           bool timed) {
    if (!Q || !K || !V || !P || !O)
        return fail(SPA_ERR_INVALID_ARGUMENT, "%s: null tensor pointer", fn);
    spa_status_t st = check_dims(fn, B, H, N, d, m, dv);
    if (st != SPA_OK) return st;
    if (causal != 0 && causal != 1)
        return fail(SPA_ERR_INVALID_ARGUMENT, "%s: causal must be 0 or 1, got %d", fn, causal);
    if (!std::isfinite(scale))
        return fail(SPA_ERR_INVALID_ARGUMENT, "%s: scale must be finite", fn);
    st = check_shape_support(fn, dtype, d, m, dv);
    if (st != SPA_OK) return st;
    if (o_dtype != SPA_F32 && o_dtype != SPA_BF16)
        return fail(SPA_ERR_INVALID_ARGUMENT, "%s: unknown o_dtype %d", fn, (int)o_dtype);
    if (dtype == SPA_F32 && o_dtype != SPA_F32)
        return fail(SPA_ERR_UNSUPPORTED, "%s: the fp32 path writes fp32 outputs only", fn);
    if (!aligned(Q, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(P, 16) ||
        !aligned(O, 16))
        return fail(SPA_ERR_INVALID_ARGUMENT, "%s: tensor base not 16-byte aligned", fn);
    if (lse && !aligned(lse, 4))
        return fail(SPA_ERR_INVALID_ARGUMENT, "%s: lse not 4-byte aligned", fn);
    if (workspace && !aligned(workspace, 16))
        return fail(SPA_ERR_INVALID_ARGUMENT, "%s: workspace not 16-byte aligned", fn);

    const long long rows = (long long)B * H * N;
    const size_t es = elem_size(dtype);
    const WorkspaceLayout wl = workspace_layout(B * H, N, m, dv, dtype);
    if (workspace && workspace_bytes < wl.total)
        return fail(SPA_ERR_WORKSPACE, "%s: workspace of %zu bytes, %zu needed", fn,
                    workspace_bytes, wl.total);
    const Range ro = range(O, rows * dv * elem_size(o_dtype));
    const Range ins[4] = {range(Q, rows * d * es), range(K, rows * d * es),
                          range(V, rows * dv * es), range(P, (size_t)H * d * m * es)};
    for (const Range& r : ins)
        if (overlap(ro, r)) return fail(SPA_ERR_INVALID_ARGUMENT, "%s: O overlaps an input", fn);
    if (lse) {
        const Range rl = range(lse, rows * sizeof(float));
        if (overlap(rl, ro)) return fail(SPA_ERR_INVALID_ARGUMENT, "%s: lse overlaps O", fn);
        for (const Range& r : ins)
            if (overlap(rl, r))
                return fail(SPA_ERR_INVALID_ARGUMENT, "%s: lse overlaps an input", fn);
    }
    if (workspace) {
        const Range rw = range(workspace, wl.total);
        if (overlap(rw, ro) || (lse && overlap(rw, range(lse, rows * sizeof(float)))))
            return fail(SPA_ERR_INVALID_ARGUMENT, "%s: workspace overlaps an output", fn);
        for (const Range& r : ins)
            if (overlap(rw, r))
                return fail(SPA_ERR_INVALID_ARGUMENT, "%s: workspace overlaps an input", fn);
    }

    // ---- validated: HIP work starts here ------------------------------------------------
    hipStream_t s = static_cast<hipStream_t>(stream);
    void* ws = workspace;
    if (!ws) {
        hipError_t e = hipMallocAsync(&ws, wl.total, s);
        if (e != hipSuccess) return hip_fail("spa_attn_fwd: hipMallocAsync", e);
    }
    char* wsb = static_cast<char*>(ws);
    void* Qt = wsb;
    void* Kt = wsb + wl.k_offset;
    float* kmax = reinterpret_cast<float*>(wsb + wl.kmax_offset);
    void* Vt = wsb + wl.vt_offset;

    hipEvent_t ev[3] = {nullptr, nullptr, nullptr};
    if (timed) {
        std::lock_guard<std::mutex> lock(g_prof.mu);
        if (g_prof.on && g_prof.calls < g_prof.max_calls) {
            for (int i = 0; i < 3; ++i) ev[i] = g_prof.ev[3 * g_prof.calls + i];
            ++g_prof.calls;
        }
    }
    hipError_t e = hipSuccess;
    if (ev[0]) e = hipEventRecord(ev[0], s);
    if (e == hipSuccess) {
        if (dtype == SPA_BF16) {
            const int mp = spa::padded_m(m);
            // Queries carry scale*log2(e) so that scores come out in base-2 exponent units.
            // The projected operands of the score MFMA are kept in fp16: its 11-bit
            // significand holds the score error well inside the bf16 path's tolerance where
            // bf16 operands (8 bits) do not, at the same MFMA rate.
            const float qscale = scale * 1.44269504088896340736f;
            // V^T is written only for the attention variant that reads it, and the queries
            // are projected here only for the variant that does not project them itself.
            const bool vrows = spa::attn_bf16_reads_v_rows(B * H, N, mp, dv, causal == 1);
            const bool qfold = spa::attn_bf16_projects_queries(B * H, N, mp, d, causal == 1);
            e = spa::launch_project_bf16(qfold ? nullptr : Q, K, P, Qt, Kt, 2, B * H, H, N, d, m,
                                         mp, mp, qscale, 1.0f, /*out_f16=*/true, kmax,
                                         vrows ? nullptr : V, vrows ? nullptr : Vt, dv, s);
            if (e == hipSuccess && ev[1]) e = hipEventRecord(ev[1], s);
            if (e == hipSuccess)
                e = spa::launch_attn_bf16(Qt, Kt, vrows ? nullptr : Vt, vrows ? V : nullptr,
                                          kmax, O, lse, B * H, N, mp, dv, causal == 1,
                                          o_dtype == SPA_F32, s, qfold ? Q : nullptr, P,
                                          qscale, d, H, m);
        } else {
            e = spa::launch_project_f32(static_cast<const float*>(Q),
                                        static_cast<const float*>(P), static_cast<float*>(Qt),
                                        B * H, H, N, d, m, 1.0f, s,
                                        static_cast<const float*>(K), static_cast<float*>(Kt));
            if (e == hipSuccess && ev[1]) e = hipEventRecord(ev[1], s);
            if (e == hipSuccess)
                e = spa::launch_attn_f32(static_cast<const float*>(Qt),
                                         static_cast<const float*>(Kt),
                                         static_cast<const float*>(V), static_cast<float*>(O),
                                         lse, B * H, N, m, dv, causal == 1, scale, s);
        }
    }
    if (e == hipSuccess && ev[2]) e = hipEventRecord(ev[2], s);
    if (!workspace) {
        hipError_t e2 = hipFreeAsync(ws, s);
        if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return hip_fail(fn, e);
    return SPA_OK;
}

// Workspace of the allocation-free forward: one array per GPU the library runs on, held
// until the process ends. kScratchBytes covers the forward's workspace up to, e.g.,
// B*H = 32 heads of N = 8192 at d = m = dv = 128 on the bf16 path (96 MiB).
constexpr size_t kScratchBytes = size_t(128) << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// This device's address of `scratch` (looked up once per device, with that device current;
// the host-side name of the array is not a device address).
spa_status_t scratch_for_current_device(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail("spa_attn_fwd_noalloc: hipGetDevice", e);
    if (dev < 0 || dev >= kMaxDevices)
        return fail(SPA_ERR_UNSUPPORTED, "spa_attn_fwd_noalloc: device %d beyond %d", dev,
                    kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail("spa_attn_fwd_noalloc: hipGetSymbolAddress", e);
        if (!ptr) return fail(SPA_ERR_HIP, "spa_attn_fwd_noalloc: null scratch address");
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return SPA_OK;
}

}  // namespace

extern "C" {

spa_status_t spa_attn_fwd(const void* Q, const void* K, const void* V, const void* P,
                          float scale, int causal, int B, int H, int N, int d, int m, int dv,
                          spa_dtype_t dtype, void* O, spa_dtype_t o_dtype, float* lse,
                          void* workspace, size_t workspace_bytes, void* stream) {
    g_err[0] = '\0';
    return attn_fwd_impl("spa_attn_fwd", Q, K, V, P, scale, causal, B, H, N, d, m, dv, dtype,
                         O, o_dtype, lse, workspace, workspace_bytes, stream, true);
}

size_t spa_attn_fwd_noalloc_max_workspace_bytes(void) { return kScratchBytes; }

spa_status_t spa_attn_fwd_noalloc(const void* Q, const void* K, const void* V, const void* P,
                                  float scale, int causal, int B, int H, int N, int d, int m,
                                  int dv, spa_dtype_t dtype, void* O, spa_dtype_t o_dtype,
                                  float* lse, void* stream) {
    g_err[0] = '\0';
    const char* fn = "spa_attn_fwd_noalloc";
    // The size check needs only the dimensions; everything else is validated by the
    // forward before any HIP work.
    spa_status_t st = check_dims(fn, B, H, N, d, m, dv);
    if (st != SPA_OK) return st;
    st = check_shape_support(fn, dtype, d, m, dv);
    if (st != SPA_OK) return st;
    const size_t need = workspace_layout(B * H, N, m, dv, dtype).total;
    if (need > kScratchBytes)
        return fail(SPA_ERR_UNSUPPORTED,
                    "%s: these sizes need %zu bytes of workspace, more than the %zu of the "
                    "library's static scratch; use spa_attn_fwd with a workspace",
                    fn, need, kScratchBytes);
    void* ws = nullptr;
    st = scratch_for_current_device(&ws);
    if (st != SPA_OK) return st;
    return attn_fwd_impl(fn, Q, K, V, P, scale, causal, B, H, N, d, m, dv, dtype, O, o_dtype,
                         lse, ws, kScratchBytes, stream, false);
}

spa_status_t spa_kcache_append(const void* K, const void* P, void* cache, int B, int H, int N,
                               int d, int m, int rows, int row0, spa_dtype_t dtype,
                               void* stream) {
    g_err[0] = '\0';
    const char* fn = "spa_kcache_append";
    if (!K || !P || !cache) return fail(SPA_ERR_INVALID_ARGUMENT, "%s: null tensor pointer", fn);
    spa_status_t st = check_dims(fn, B, H, N, d, m, 1);
    if (st != SPA_OK) return st;
    if (row0 < 0 || rows < 1 || (long long)row0 + N > rows || rows > kMaxN)
        return fail(SPA_ERR_INVALID_ARGUMENT, "%s: rows %d .. %lld outside a cache of %d rows",
                    fn, row0, (long long)row0 + N, rows);
    if ((long long)B * H * rows >= kMaxRows)
        return fail(SPA_ERR_UNSUPPORTED, "%s: B*H*rows exceeds 2^31", fn);
    if (dtype != SPA_BF16)
        return fail(SPA_ERR_UNSUPPORTED, "%s: the key cache takes bf16 keys", fn);
    if ((d != 64 && d != 128) || m > 128)
        return fail(SPA_ERR_UNSUPPORTED, "%s: needs d in {64,128} and m <= 128 (d=%d m=%d)", fn,
                    d, m);
    if (!aligned(K, 16) || !aligned(P, 16) || !aligned(cache, 16))
        return fail(SPA_ERR_INVALID_ARGUMENT, "%s: tensor base not 16-byte aligned", fn);
    const Range rk = range(K, (size_t)B * H * N * d * 2), rp = range(P, (size_t)H * d * m * 2),
                rc = range(cache, (size_t)B * H * rows * m * 2);
    if (overlap(rc, rk) || overlap(rc, rp))
        return fail(SPA_ERR_INVALID_ARGUMENT, "%s: the cache overlaps an input", fn);
    char* first = static_cast<char*>(cache) + (size_t)row0 * m * 2;
    hipError_t e = spa::launch_project_bf16(K, nullptr, P, first, nullptr, 1, B * H, H, N, d, m,
                                            m, m, 1.0f, 1.0f, /*out_f16=*/true, nullptr,
                                            nullptr, nullptr, 0,
                                            static_cast<hipStream_t>(stream), nullptr, nullptr,
                                            (long long)rows * m);
    if (e != hipSuccess) return hip_fail(fn, e);
    return SPA_OK;
}

size_t spa_attn_decode_workspace_bytes(int B, int H, int Nq, int Nk, int dv) {
    if (B < 1 || H < 1 || Nq < 1 || Nk < Nq || Nk > kMaxN || dv < 1 ||
        (long long)B * H * Nk >= kMaxRows)
        return 0;
    const spa::DecodeSplit sp = spa::decode_split(B * H, Nq, Nk);
    return (size_t)B * H * Nq * sp.nsplit * ((size_t)dv + 2) * sizeof(float);
}

spa_status_t spa_attn_decode(const void* Q, const void* cache, const void* Vc, const void* P,
                             float scale, int causal, int B, int H, int Nq, int Nk, int rows,
                             int d, int m, int dv, spa_dtype_t dtype, void* O,
                             spa_dtype_t o_dtype, float* lse, void* workspace,
                             size_t workspace_bytes, void* stream) {
    g_err[0] = '\0';
    const char* fn = "spa_attn_decode";
    if (!Q || !cache || !Vc || !P || !O)
        return fail(SPA_ERR_INVALID_ARGUMENT, "%s: null tensor pointer", fn);
    spa_status_t st = check_dims(fn, B, H, Nq, d, m, dv);
    if (st != SPA_OK) return st;
    if (Nk < Nq || rows < Nk || rows > kMaxN)
        return fail(SPA_ERR_INVALID_ARGUMENT, "%s: needs 1 <= Nq <= Nk <= rows (Nq=%d Nk=%d rows=%d)",
                    fn, Nq, Nk, rows);
    if ((long long)B * H * rows >= kMaxRows)
        return fail(SPA_ERR_UNSUPPORTED, "%s: B*H*rows exceeds 2^31", fn);
    if (causal != 0 && causal != 1)
        return fail(SPA_ERR_INVALID_ARGUMENT, "%s: causal must be 0 or 1, got %d", fn, causal);
    if (!std::isfinite(scale))
        return fail(SPA_ERR_INVALID_ARGUMENT, "%s: scale must be finite", fn);
    if (dtype != SPA_BF16)
        return fail(SPA_ERR_UNSUPPORTED, "%s: the decode path takes bf16 queries and values", fn);
    if ((d != 64 && d != 128) || m > 128 || (dv != 64 && dv != 128))
        return fail(SPA_ERR_UNSUPPORTED, "%s: needs d, dv in {64,128} and m <= 128 (d=%d m=%d dv=%d)",
                    fn, d, m, dv);
    if (o_dtype != SPA_F32 && o_dtype != SPA_BF16)
        return fail(SPA_ERR_INVALID_ARGUMENT, "%s: unknown o_dtype %d", fn, (int)o_dtype);
    if (!aligned(Q, 16) || !aligned(cache, 16) || !aligned(Vc, 16) || !aligned(P, 16) ||
        !aligned(O, 16))
        return fail(SPA_ERR_INVALID_ARGUMENT, "%s: tensor base not 16-byte aligned", fn);
    if (lse && !aligned(lse, 4))
        return fail(SPA_ERR_INVALID_ARGUMENT, "%s: lse not 4-byte aligned", fn);
    if (workspace && !aligned(workspace, 16))
        return fail(SPA_ERR_INVALID_ARGUMENT, "%s: workspace not 16-byte aligned", fn);
    const size_t need = spa_attn_decode_workspace_bytes(B, H, Nq, Nk, dv);
    if (workspace && workspace_bytes < need)
        return fail(SPA_ERR_WORKSPACE, "%s: workspace of %zu bytes, %zu needed", fn,
                    workspace_bytes, need);
    const long long bh = (long long)B * H;
    const Range ro = range(O, (size_t)bh * Nq * dv * elem_size(o_dtype));
    const Range ins[4] = {range(Q, (size_t)bh * Nq * d * 2), range(cache, (size_t)bh * rows * m * 2),
                          range(Vc, (size_t)bh * rows * dv * 2), range(P, (size_t)H * d * m * 2)};
    const Range rl = lse ? range(lse, (size_t)bh * Nq * sizeof(float)) : Range{0, 0};
    for (const Range& r : ins) {
        if (overlap(ro, r)) return fail(SPA_ERR_INVALID_ARGUMENT, "%s: O overlaps an input", fn);
        if (lse && overlap(rl, r))
            return fail(SPA_ERR_INVALID_ARGUMENT, "%s: lse overlaps an input", fn);
    }
    if (lse && overlap(rl, ro)) return fail(SPA_ERR_INVALID_ARGUMENT, "%s: lse overlaps O", fn);
    if (workspace) {
        const Range rw = range(workspace, need);
        if (overlap(rw, ro) || (lse && overlap(rw, rl)))
            return fail(SPA_ERR_INVALID_ARGUMENT, "%s: workspace overlaps an output", fn);
        for (const Range& r : ins)
            if (overlap(rw, r))
                return fail(SPA_ERR_INVALID_ARGUMENT, "%s: workspace overlaps an input", fn);
    }

    hipStream_t s = static_cast<hipStream_t>(stream);
    void* ws = workspace;
    if (!ws) {
        hipError_t e = hipMallocAsync(&ws, need, s);
        if (e != hipSuccess) return hip_fail("spa_attn_decode: hipMallocAsync", e);
    }
    const spa::DecodeSplit sp = spa::decode_split(B * H, Nq, Nk);
    spa::DecodeArgs a;
    a.Q = static_cast<const uint16_t*>(Q);
    a.Kc = static_cast<const uint16_t*>(cache);
    a.Vc = static_cast<const uint16_t*>(Vc);
    a.P = static_cast<const uint16_t*>(P);
    a.O = O;
    a.lse = lse;
    a.partO = static_cast<float*>(ws);
    a.partML = static_cast<float*>(ws) + (size_t)bh * Nq * sp.nsplit * dv;
    a.qscale = scale * 1.44269504088896340736f;
    a.causal = causal;
    a.BH = B * H;
    a.H = H;
    a.Nq = Nq;
    a.Nk = Nk;
    a.rows = rows;
    a.d = d;
    a.m = m;
    a.dv = dv;
    a.o_f32 = o_dtype == SPA_F32;
    a.nsplit = sp.nsplit;
    a.chunk = sp.chunk;
    hipError_t e = spa::launch_decode_bf16(a, s);
    if (!workspace) {
        hipError_t e2 = hipFreeAsync(ws, s);
        if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return hip_fail(fn, e);
    return SPA_OK;
}

size_t spa_sfa_fwd_workspace_bytes(int B, int H, int N, int d, int dv) {
    if (check_dims("spa_sfa_fwd_workspace_bytes", B, H, N, d, d, dv) != SPA_OK ||
        (d != 64 && d != 128) || (dv != 64 && dv != 128)) {
        g_err[0] = '\0';
        return 0;
    }
    return workspace_layout(B * H, N, d, dv, SPA_BF16).total;
}

spa_status_t spa_sfa_fwd(const void* Q, const void* K, const void* V, int topk, float scale,
                         int causal, int B, int H, int N, int d, int dv, spa_dtype_t dtype,
                         void* O, spa_dtype_t o_dtype, float* lse, void* workspace,
                         size_t workspace_bytes, void* stream) {
    g_err[0] = '\0';
    const char* fn = "spa_sfa_fwd";
    if (!Q || !K || !V || !O) return fail(SPA_ERR_INVALID_ARGUMENT, "%s: null tensor pointer", fn);
    spa_status_t st = check_dims(fn, B, H, N, d, d, dv);
    if (st != SPA_OK) return st;
    if (topk < 1 || topk > d)
        return fail(SPA_ERR_INVALID_ARGUMENT, "%s: topk must be in [1, d], got %d", fn, topk);
    if (causal != 0 && causal != 1)
        return fail(SPA_ERR_INVALID_ARGUMENT, "%s: causal must be 0 or 1, got %d", fn, causal);
    if (!std::isfinite(scale))
        return fail(SPA_ERR_INVALID_ARGUMENT, "%s: scale must be finite", fn);
    if (dtype != SPA_BF16)
        return fail(SPA_ERR_UNSUPPORTED, "%s: sparse feature attention takes bf16 inputs", fn);
    if ((d != 64 && d != 128) || (dv != 64 && dv != 128))
        return fail(SPA_ERR_UNSUPPORTED, "%s: needs d, dv in {64,128} (d=%d dv=%d)", fn, d, dv);
    if (o_dtype != SPA_F32 && o_dtype != SPA_BF16)
        return fail(SPA_ERR_INVALID_ARGUMENT, "%s: unknown o_dtype %d", fn, (int)o_dtype);
    if (!aligned(Q, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(O, 16))
        return fail(SPA_ERR_INVALID_ARGUMENT, "%s: tensor base not 16-byte aligned", fn);
    if (lse && !aligned(lse, 4))
        return fail(SPA_ERR_INVALID_ARGUMENT, "%s: lse not 4-byte aligned", fn);
    if (workspace && !aligned(workspace, 16))
        return fail(SPA_ERR_INVALID_ARGUMENT, "%s: workspace not 16-byte aligned", fn);
    const WorkspaceLayout wl = workspace_layout(B * H, N, d, dv, SPA_BF16);
    if (workspace && workspace_bytes < wl.total)
        return fail(SPA_ERR_WORKSPACE, "%s: workspace of %zu bytes, %zu needed", fn,
                    workspace_bytes, wl.total);
    const long long rows = (long long)B * H * N;
    const Range ro = range(O, rows * dv * elem_size(o_dtype));
    const Range ins[3] = {range(Q, rows * d * 2), range(K, rows * d * 2), range(V, rows * dv * 2)};
    const Range rl = lse ? range(lse, rows * sizeof(float)) : Range{0, 0};
    for (const Range& r : ins) {
        if (overlap(ro, r)) return fail(SPA_ERR_INVALID_ARGUMENT, "%s: O overlaps an input", fn);
        if (lse && overlap(rl, r))
            return fail(SPA_ERR_INVALID_ARGUMENT, "%s: lse overlaps an input", fn);
    }
    if (lse && overlap(rl, ro)) return fail(SPA_ERR_INVALID_ARGUMENT, "%s: lse overlaps O", fn);
    if (workspace) {
        const Range rw = range(workspace, wl.total);
        if (overlap(rw, ro) || (lse && overlap(rw, rl)))
            return fail(SPA_ERR_INVALID_ARGUMENT, "%s: workspace overlaps an output", fn);
        for (const Range& r : ins)
            if (overlap(rw, r))
                return fail(SPA_ERR_INVALID_ARGUMENT, "%s: workspace overlaps an input", fn);
    }

    hipStream_t s = static_cast<hipStream_t>(stream);
    void* ws = workspace;
    if (!ws) {
        hipError_t e = hipMallocAsync(&ws, wl.total, s);
        if (e != hipSuccess) return hip_fail("spa_sfa_fwd: hipMallocAsync", e);
    }
    char* wsb = static_cast<char*>(ws);
    void* Qt = wsb;
    void* Kt = wsb + wl.k_offset;
    float* kmax = reinterpret_cast<float*>(wsb + wl.kmax_offset);
    void* Vt = wsb + wl.vt_offset;
    hipError_t e = spa::launch_sfa_topk(Q, K, Qt, Kt, kmax, B * H, N, d, topk,
                                        scale * 1.44269504088896340736f, s);
    // V^T through the preparation kernel's transpose role alone (no projection roles)
    if (e == hipSuccess)
        e = spa::launch_project_bf16(nullptr, nullptr, nullptr, nullptr, nullptr, 0, B * H, H,
                                     N, d, 1, 1, 1, 1.0f, 1.0f, true, nullptr, V, Vt, dv, s);
    if (e == hipSuccess)
        e = spa::launch_attn_bf16(Qt, Kt, Vt, nullptr, kmax, O, lse, B * H, N, d, dv, causal == 1,
                                  o_dtype == SPA_F32, s);
    if (!workspace) {
        hipError_t e2 = hipFreeAsync(ws, s);
        if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return hip_fail(fn, e);
    return SPA_OK;
}

size_t spa_attn_bwd_workspace_bytes(int B, int H, int N, int d, int m, int dv,
                                    spa_dtype_t dtype) {
    if (B < 1 || H < 1 || N < 1 || N > kMaxN || (long long)B * H * N >= kMaxRows) return 0;
    if (dtype == SPA_F32) {
        if (d < 1 || d > 256 || m < 1 || m > 128 || dv < 1 || dv > 128) return 0;
        return bwd_f32_layout(B * H, N, m).total;
    }
    if (dtype != SPA_BF16 || (d != 64 && d != 128) || m < 1 || m > 128 || (dv != 64 && dv != 128))
        return 0;
    return bwd_layout(B * H, N, d, m, dv).total;
}

spa_status_t spa_attn_bwd(const void* Q, const void* K, const void* V, const void* P,
                          const void* O, const void* dO, const float* lse, float scale,
                          int causal, int B, int H, int N, int d, int m, int dv,
                          spa_dtype_t dtype, void* dQ, void* dK, void* dV, float* dP,
                          spa_dtype_t g_dtype, void* workspace, size_t workspace_bytes,
                          void* stream) {
    g_err[0] = '\0';
    const char* fn = "spa_attn_bwd";
    if (!Q || !K || !V || !P || !O || !dO || !lse || !dQ || !dK || !dV || !dP)
        return fail(SPA_ERR_INVALID_ARGUMENT, "%s: null pointer", fn);
    spa_status_t st = check_dims(fn, B, H, N, d, m, dv);
    if (st != SPA_OK) return st;
    if (causal != 0 && causal != 1)
        return fail(SPA_ERR_INVALID_ARGUMENT, "%s: causal must be 0 or 1, got %d", fn, causal);
    if (!std::isfinite(scale))
        return fail(SPA_ERR_INVALID_ARGUMENT, "%s: scale must be finite", fn);
    if (dtype != SPA_BF16 && dtype != SPA_F32)
        return fail(SPA_ERR_INVALID_ARGUMENT, "%s: unknown dtype %d", fn, (int)dtype);
    if (g_dtype != SPA_BF16 && g_dtype != SPA_F32)
        return fail(SPA_ERR_INVALID_ARGUMENT, "%s: unknown g_dtype %d", fn, (int)g_dtype);
    if (dtype == SPA_F32) {
        if (d > 256 || m > 128 || dv > 128)
            return fail(SPA_ERR_UNSUPPORTED,
                        "%s: fp32 backward needs d <= 256, m <= 128, dv <= 128 (d=%d m=%d dv=%d)",
                        fn, d, m, dv);
        if (g_dtype != SPA_F32)
            return fail(SPA_ERR_UNSUPPORTED, "%s: the fp32 path writes fp32 gradients only", fn);
    } else if ((d != 64 && d != 128) || m > 128 || (dv != 64 && dv != 128)) {
        return fail(SPA_ERR_UNSUPPORTED,
                    "%s: backward needs d in {64,128}, m <= 128, dv in {64,128} (d=%d m=%d dv=%d)",
                    fn, d, m, dv);
    }
    const void* al16[] = {Q, K, V, P, O, dO, dQ, dK, dV};
    for (const void* p : al16)
        if (!aligned(p, 16))
            return fail(SPA_ERR_INVALID_ARGUMENT, "%s: tensor base not 16-byte aligned", fn);
    if (!aligned(lse, 4) || !aligned(dP, 4))
        return fail(SPA_ERR_INVALID_ARGUMENT, "%s: lse or dP not 4-byte aligned", fn);
    if (workspace && !aligned(workspace, 16))
        return fail(SPA_ERR_INVALID_ARGUMENT, "%s: workspace not 16-byte aligned", fn);
    const long long rows = (long long)B * H * N;
    const bool f32 = dtype == SPA_F32;
    const BwdLayout wl = bwd_layout(B * H, N, d, m, dv);
    const BwdF32Layout wl32 = bwd_f32_layout(B * H, N, m);
    const size_t need = f32 ? wl32.total : wl.total;
    if (workspace && workspace_bytes < need)
        return fail(SPA_ERR_WORKSPACE, "%s: workspace of %zu bytes, %zu needed", fn,
                    workspace_bytes, need);
    const size_t ge = g_dtype == SPA_F32 ? 4 : 2;
    const size_t ie = f32 ? 4 : 2;
    const Range ins[8] = {range(Q, rows * d * ie),  range(K, rows * d * ie),
                          range(V, rows * dv * ie), range(P, (size_t)H * d * m * ie),
                          range(O, rows * dv * ie), range(dO, rows * dv * ie),
                          range(lse, rows * 4),     range(workspace, workspace ? need : 0)};
    const Range outs[4] = {range(dQ, rows * d * ge), range(dK, rows * d * ge),
                           range(dV, rows * dv * ge), range(dP, (size_t)H * d * m * 4)};
    for (int i = 0; i < 4; ++i) {
        for (const Range& r : ins)
            if (overlap(outs[i], r))
                return fail(SPA_ERR_INVALID_ARGUMENT, "%s: an output overlaps an input or the workspace", fn);
        for (int j = 0; j < i; ++j)
            if (overlap(outs[i], outs[j]))
                return fail(SPA_ERR_INVALID_ARGUMENT, "%s: outputs overlap", fn);
    }
    if (workspace)
        for (int i = 0; i < 7; ++i)
            if (overlap(ins[7], ins[i]))
                return fail(SPA_ERR_INVALID_ARGUMENT, "%s: workspace overlaps an input", fn);

    // ---- validated: HIP work starts here ------------------------------------------------
    hipStream_t s = static_cast<hipStream_t>(stream);
    void* ws = workspace;
    if (!ws) {
        hipError_t e = hipMallocAsync(&ws, need, s);
        if (e != hipSuccess) return hip_fail("spa_attn_bwd: hipMallocAsync", e);
    }
    char* w = static_cast<char*>(ws);
    if (f32) {
        spa::BwdF32Args a;
        a.Q = static_cast<const float*>(Q);
        a.K = static_cast<const float*>(K);
        a.V = static_cast<const float*>(V);
        a.P = static_cast<const float*>(P);
        a.O = static_cast<const float*>(O);
        a.dO = static_cast<const float*>(dO);
        a.lse = lse;
        a.Qt = reinterpret_cast<float*>(w + wl32.qt);
        a.Kt = reinterpret_cast<float*>(w + wl32.kt);
        a.dQt = reinterpret_cast<float*>(w + wl32.dqt);
        a.dKt = reinterpret_cast<float*>(w + wl32.dkt);
        a.D = reinterpret_cast<float*>(w + wl32.dd);
        a.dQ = static_cast<float*>(dQ);
        a.dK = static_cast<float*>(dK);
        a.dV = static_cast<float*>(dV);
        a.dP = dP;
        a.B = B;
        a.H = H;
        a.N = N;
        a.d = d;
        a.m = m;
        a.dv = dv;
        a.causal = causal;
        a.scale = scale;
        hipError_t e = spa::launch_attn_bwd_f32(a, s);
        if (!workspace) {
            hipError_t e2 = hipFreeAsync(ws, s);
            if (e == hipSuccess) e = e2;
        }
        if (e != hipSuccess) return hip_fail(fn, e);
        return SPA_OK;
    }
    const int mp = spa::padded_m(m);
    const float log2e = 1.44269504088896340736f;
    const float qscale = scale * log2e;
    const bool fused = spa::bwd_fuses_dq(mp, dv);
    spa::PrepRowTerms rt;
    if (fused) {
        rt.O = O;
        rt.lse = lse;
        rt.LD = reinterpret_cast<float*>(w + wl.ld);
        rt.dQt = reinterpret_cast<float*>(w + wl.dqt);
        rt.dqt_cols = mp;
        rt.lse_scale = log2e;
    }
    // K~^T is read only by the query-major kernel, which the fused form does not run.
    hipError_t e = spa::launch_project_bf16(Q, K, P, w + wl.qs, w + wl.kt, 2, B * H, H, N, d, m,
                                            mp, mp, qscale, 1.0f, /*out_f16=*/true, nullptr, dO,
                                            w + wl.dot, dv, s, w + wl.qst,
                                            fused ? nullptr : w + wl.ktt, -1,
                                            fused ? &rt : nullptr);
    if (e == hipSuccess) {
        spa::BwdArgs a;
        a.Q = static_cast<const uint16_t*>(Q);
        a.K = static_cast<const uint16_t*>(K);
        a.P = static_cast<const uint16_t*>(P);
        a.Qs = reinterpret_cast<const uint16_t*>(w + wl.qs);
        a.Kt = reinterpret_cast<const uint16_t*>(w + wl.kt);
        a.Qst = reinterpret_cast<const uint16_t*>(w + wl.qst);
        a.Ktt = reinterpret_cast<const uint16_t*>(w + wl.ktt);
        a.V = static_cast<const uint16_t*>(V);
        a.O = static_cast<const uint16_t*>(O);
        a.dO = static_cast<const uint16_t*>(dO);
        a.dOt = reinterpret_cast<const uint16_t*>(w + wl.dot);
        a.lse = lse;
        a.LD = reinterpret_cast<float*>(w + wl.ld);
        a.dQt = reinterpret_cast<float*>(w + wl.dqt);
        a.dKt = reinterpret_cast<float*>(w + wl.dkt);
        a.dPpart = reinterpret_cast<float*>(w + wl.part);
        a.dP = dP;
        a.dQ = dQ;
        a.dK = dK;
        a.dV = dV;
        a.g_f32 = g_dtype == SPA_F32 ? 1 : 0;
        a.fused_dq = fused ? 1 : 0;
        a.BH = B * H;
        a.H = H;
        a.N = N;
        a.Np = spa::vt_padded_keys(N);
        a.d = d;
        a.m = m;
        a.mp = mp;
        a.dv = dv;
        a.causal = causal;
        a.scale = scale;
        e = spa::launch_attn_bwd_bf16(a, s);
    }
    if (!workspace) {
        hipError_t e2 = hipFreeAsync(ws, s);
        if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return hip_fail(fn, e);
    return SPA_OK;
}

spa_status_t spa_probe_rates(double* mfma_tflops, double* mfma_ghz, double* fma_tflops,
                             double* fma_ghz, void* stream) {
    g_err[0] = '\0';
    if (!mfma_tflops || !mfma_ghz || !fma_tflops || !fma_ghz)
        return fail(SPA_ERR_INVALID_ARGUMENT, "spa_probe_rates: null output pointer");
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = spa::run_probe(0, 100, s, mfma_tflops, mfma_ghz);
    if (e == hipSuccess) e = spa::run_probe(1, 100, s, fma_tflops, fma_ghz);
    if (e != hipSuccess) return hip_fail("spa_probe_rates", e);
    return SPA_OK;
}

spa_status_t spa_profile_begin(int max_calls) {
    g_err[0] = '\0';
    if (max_calls < 1 || max_calls > 65536)
        return fail(SPA_ERR_INVALID_ARGUMENT, "spa_profile_begin: max_calls=%d", max_calls);
    std::lock_guard<std::mutex> lock(g_prof.mu);
    if (g_prof.on) return fail(SPA_ERR_INVALID_ARGUMENT, "spa_profile_begin: already recording");
    g_prof.ev.assign(3 * (size_t)max_calls, nullptr);
    for (auto& e : g_prof.ev) {
        hipError_t r = hipEventCreate(&e);
        if (r != hipSuccess) {
            for (auto& x : g_prof.ev)
                if (x) (void)hipEventDestroy(x);
            g_prof.ev.clear();
            return hip_fail("spa_profile_begin: hipEventCreate", r);
        }
    }
    g_prof.max_calls = max_calls;
    g_prof.calls = 0;
    g_prof.on = true;
    return SPA_OK;
}

spa_status_t spa_profile_end(double* project_ms, double* attn_ms, int* calls) {
    g_err[0] = '\0';
    std::lock_guard<std::mutex> lock(g_prof.mu);
    if (!g_prof.on) return fail(SPA_ERR_INVALID_ARGUMENT, "spa_profile_end: not recording");
    double pt = 0.0, at = 0.0;
    hipError_t err = hipSuccess;
    if (g_prof.calls > 0) err = hipEventSynchronize(g_prof.ev[3 * g_prof.calls - 1]);
    for (int c = 0; c < g_prof.calls && err == hipSuccess; ++c) {
        float a = 0.0f, b = 0.0f;
        err = hipEventElapsedTime(&a, g_prof.ev[3 * c], g_prof.ev[3 * c + 1]);
        if (err == hipSuccess) err = hipEventElapsedTime(&b, g_prof.ev[3 * c + 1], g_prof.ev[3 * c + 2]);
        pt += a;
        at += b;
    }
    const int n = g_prof.calls;
    for (auto& e : g_prof.ev) (void)hipEventDestroy(e);
    g_prof.ev.clear();
    g_prof.on = false;
    g_prof.calls = 0;
    if (err != hipSuccess) return hip_fail("spa_profile_end", err);
    if (project_ms) *project_ms = pt;
    if (attn_ms) *attn_ms = at;
    if (calls) *calls = n;
    return SPA_OK;
}

}  // extern "C"
