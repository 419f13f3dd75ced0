// C-ABI entry points of liblrc: argument validation, then dispatch to the per-op launchers.
// Nothing is launched when validation fails.
#include <atomic>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <unordered_map>
#include <string>
#include <vector>

#include "lrc_internal.h"
#include "cov_mfma.h"

namespace lrc {

static thread_local std::string g_last_error;

lrc_status fail(lrc_status s, const std::string &msg) {
    g_last_error = msg;
    return s;
}

lrc_status hip_fail(hipError_t e, const char *what) {
    char buf[512];
    snprintf(buf, sizeof(buf), "%s failed: %s (%d)", what, hipGetErrorString(e), int(e));
    g_last_error = buf;
    return LRC_ERR_HIP;
}

static bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// ---------------------------------------------------------------------------------------------
// kernel timing records
// ---------------------------------------------------------------------------------------------
struct TimingRec {
    std::string kernel;
    hipEvent_t start, stop;
    double flops;
};
static std::mutex g_tmu;
static std::atomic<bool> g_timing{false};  // read without the lock on every launch
static int g_stride = 1;                                    // record every g_stride-th launch
static std::unordered_map<std::string, int64_t> g_counts;  // launches seen per kernel
static std::unordered_map<std::string, int> g_kstride;     // per-kernel strides (override g_stride)
static std::vector<TimingRec> g_recs;
static std::vector<hipEvent_t> g_free;  // events of discarded records, reused (creation is slow)

static bool take_event(hipEvent_t *e) {
    if (!g_free.empty()) {
        *e = g_free.back();
        g_free.pop_back();
        return true;
    }
    return hipEventCreate(e) == hipSuccess;
}

bool timing_sample(const char *kernel, double work, hipEvent_t *start, hipEvent_t *stop) {
    if (!g_timing.load(std::memory_order_relaxed)) return false;
    std::lock_guard<std::mutex> lk(g_tmu);
    if (!g_timing) return false;
    const auto ks = g_kstride.find(kernel);
    const int stride = ks == g_kstride.end() ? g_stride : ks->second;
    if (g_counts[kernel]++ % stride != 0) return false;
    TimingRec r;
    r.kernel = kernel;
    r.flops = work;
    if (!take_event(&r.start)) return false;
    if (!take_event(&r.stop)) {
        g_free.push_back(r.start);
        return false;
    }
    g_recs.push_back(r);
    *start = r.start;
    *stop = r.stop;
    return true;
}

}  // namespace lrc

using namespace lrc;

#define REQUIRE(cond, code, msg) \
    do {                         \
        if (!(cond)) return fail(code, msg); \
    } while (0)

extern "C" {

int lrc_abi_version(void) { return LRC_ABI_VERSION; }

const char *lrc_status_string(lrc_status s) {
    switch (s) {
        case LRC_OK: return "ok";
        case LRC_ERR_ARG: return "invalid argument";
        case LRC_ERR_DTYPE: return "unsupported dtype";
        case LRC_ERR_WORKSPACE: return "workspace missing or too small";
        case LRC_ERR_HIP: return "HIP runtime error";
        case LRC_ERR_UNIMPLEMENTED: return "not implemented";
    }
    return "unknown status";
}

const char *lrc_last_error(void) { return g_last_error.c_str(); }

lrc_status lrc_timing_enable(int stride) {
    REQUIRE(stride >= 0, LRC_ERR_ARG, "stride must be >= 0");
    std::lock_guard<std::mutex> lk(g_tmu);
    g_timing = stride != 0;
    if (stride > 0) g_stride = stride;
    g_counts.clear();
    return LRC_OK;
}

lrc_status lrc_timing_set_stride(const char *kernel, int stride) {
    REQUIRE(kernel && stride >= 1, LRC_ERR_ARG, "kernel must be non-NULL and stride >= 1");
    std::lock_guard<std::mutex> lk(g_tmu);
    g_kstride[kernel] = stride;
    return LRC_OK;
}

lrc_status lrc_timing_read(const char *kernel, int64_t *launches, double *total_ms, double *total_work, int reset) {
    REQUIRE(kernel && launches && total_ms && total_work, LRC_ERR_ARG, "null argument");
    std::lock_guard<std::mutex> lk(g_tmu);
    int64_t n = 0;
    double ms = 0.0, fl = 0.0;
    for (auto &r : g_recs) {
        if (r.kernel != kernel) continue;
        hipError_t e = hipEventSynchronize(r.stop);
        if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize");
        float t = 0.f;
        e = hipEventElapsedTime(&t, r.start, r.stop);
        if (e != hipSuccess) return hip_fail(e, "hipEventElapsedTime");
        ms += double(t);
        fl += r.flops;
        ++n;
    }
    *launches = n;
    *total_ms = ms;
    *total_work = fl;
    if (reset) {
        for (auto &r : g_recs) {
            (void)hipEventSynchronize(r.stop);
            g_free.push_back(r.start);
            g_free.push_back(r.stop);
        }
        g_recs.clear();
    }
    return LRC_OK;
}

// ---------------------------------------------------------------------------------------------
size_t lrc_cov_accumulate_workspace(lrc_dtype x_t, int64_t n_tok, int64_t d_in, int has_w, int64_t d_out,
                                    int32_t n_blocks) {
    if (n_tok <= 0 || d_in <= 0 || d_out <= 0 || n_blocks <= 0) return 0;
    return cov_workspace(x_t, n_tok, d_in, has_w, d_out, n_blocks);
}

lrc_status lrc_cov_accumulate(const void *X, lrc_dtype x_t, int64_t n_tok, int64_t d_in, int64_t ldx,
                              const void *W, lrc_dtype w_t, int64_t d_out, int64_t ldw, int32_t n_blocks,
                              float *C, int64_t ldc, void *ws, size_t ws_bytes, int32_t *info, void *stream) {
    REQUIRE(X && C && info, LRC_ERR_ARG, "X, C and info must be non-NULL");
    REQUIRE(n_tok > 0 && d_in > 0 && d_out > 0, LRC_ERR_ARG, "n_tok, d_in, d_out must be positive");
    REQUIRE(ldx >= d_in, LRC_ERR_ARG, "ldx < d_in");
    REQUIRE(n_blocks >= 1 && d_out % n_blocks == 0, LRC_ERR_ARG, "n_blocks must divide d_out");
    REQUIRE(x_t == LRC_BF16 || x_t == LRC_F32, LRC_ERR_DTYPE, "x_t must be LRC_BF16 or LRC_F32");
    if (W) {
        REQUIRE(w_t == x_t, LRC_ERR_DTYPE, "w_t must equal x_t");
        REQUIRE(ldw >= d_out, LRC_ERR_ARG, "ldw < d_out");
    } else {
        REQUIRE(d_out == d_in, LRC_ERR_ARG, "W == NULL (identity) needs d_out == d_in");
    }
    const int64_t hd = d_out / n_blocks;
    REQUIRE(ldc >= hd && (n_blocks > 1 || ldc >= d_out), LRC_ERR_ARG, "ldc too small");
    size_t need = cov_workspace(x_t, n_tok, d_in, W != nullptr, d_out, n_blocks);
    REQUIRE(ws_bytes >= need && (need == 0 || (ws && aligned(ws, 256))), LRC_ERR_WORKSPACE,
            "workspace smaller than lrc_cov_accumulate_workspace() or not 256-byte aligned");
    CovArgs a{X, x_t, n_tok, d_in, ldx, W, d_out, ldw, n_blocks, C, ldc, info};
    return cov_run(a, ws, ws_bytes, static_cast<hipStream_t>(stream));
}

// ---------------------------------------------------------------------------------------------
size_t lrc_range_factor_workspace(int64_t d_in, int64_t n) {
    if (d_in <= 0 || n <= 0) return 0;
    Counter c;
    c.carve<double>(size_t(d_in) * size_t(n));
    c.carve<char>(cholesky_workspace(d_in));
    return c.off;
}

lrc_status lrc_range_factor(const void *W, lrc_dtype w_t, int64_t d_in, int64_t n, int64_t ldw, double *L,
                            int64_t ldl, void *ws, size_t ws_bytes, int32_t *info, void *stream) {
    REQUIRE(W && L && info, LRC_ERR_ARG, "W, L and info must be non-NULL");
    REQUIRE(d_in > 0 && n >= d_in, LRC_ERR_ARG, "need 0 < d_in <= n");
    REQUIRE(ldw >= n && ldl >= d_in, LRC_ERR_ARG, "ldw < n or ldl < d_in");
    REQUIRE(w_t == LRC_BF16 || w_t == LRC_F32 || w_t == LRC_F64, LRC_ERR_DTYPE, "w_t must be LRC_BF16, LRC_F32 or LRC_F64");
    const size_t need = lrc_range_factor_workspace(d_in, n);
    REQUIRE(ws_bytes >= need && ws && aligned(ws, 256), LRC_ERR_WORKSPACE,
            "workspace smaller than lrc_range_factor_workspace() or not 256-byte aligned");
    Carver cv(ws, ws_bytes);
    double *Wf = cv.carve<double>(size_t(d_in) * size_t(n));
    void *chol = cv.carve<char>(cholesky_workspace(d_in));
    return range_factor_enqueue(W, w_t, d_in, n, ldw, Wf, L, ldl, chol, info, static_cast<hipStream_t>(stream));
}

size_t lrc_cov_accumulate_range_workspace(int64_t n_tok, int64_t d_in) {
    if (n_tok <= 0 || d_in <= 0) return 0;
    return cov_range_workspace(n_tok, d_in);
}

lrc_status lrc_cov_accumulate_range(const void *X, lrc_dtype x_t, int64_t n_tok, int64_t d_in, int64_t ldx,
                                    const double *L, int64_t ldl, float *B, int64_t ldb, void *ws, size_t ws_bytes,
                                    int32_t *info, void *stream) {
    REQUIRE(X && L && B && info, LRC_ERR_ARG, "X, L, B and info must be non-NULL");
    REQUIRE(n_tok > 0 && d_in > 0, LRC_ERR_ARG, "n_tok and d_in must be positive");
    REQUIRE(x_t == LRC_BF16, LRC_ERR_DTYPE, "x_t must be LRC_BF16");
    REQUIRE(d_in % 32 == 0, LRC_ERR_ARG, "d_in must be a multiple of 32");
    REQUIRE(ldx >= d_in && ldl >= d_in && ldb >= d_in, LRC_ERR_ARG, "ldx, ldl or ldb < d_in");
    REQUIRE(cov_mfma_supported(x_t, X, ldx, nullptr, 0, d_in, d_in, 1), LRC_ERR_ARG,
            "X must be 16-byte aligned with ldx a multiple of 8 (and below 2^21)");
    const size_t need = cov_range_workspace(n_tok, d_in);
    REQUIRE(ws_bytes >= need && ws && aligned(ws, 256), LRC_ERR_WORKSPACE,
            "workspace smaller than lrc_cov_accumulate_range_workspace() or not 256-byte aligned");
    CovArgs a{X, x_t, n_tok, d_in, ldx, nullptr, d_in, 0, 1, B, ldb, info, L, ldl};
    return cov_run(a, ws, ws_bytes, static_cast<hipStream_t>(stream));
}

// ---------------------------------------------------------------------------------------------
size_t lrc_eigh_workspace(int64_t n, int64_t batch, int64_t n_vec, lrc_dtype prec) {
    if (n <= 0 || batch <= 0 || n_vec < 0 || n_vec > n) return 0;
    return eigh_workspace(n, batch, n_vec, prec);
}

// nc: the order of the stored matrices (n, or d_in for a projected group)
static lrc_status check_eigh(const float *C, int64_t n, int64_t ldc, int64_t batch, int64_t stride_c,
                             const double *lambda, const float *V, int64_t ldv, int64_t n_vec, int64_t stride_v,
                             const int32_t *info, int64_t nc = -1) {
    if (nc < 0) nc = n;
    REQUIRE(C && lambda && info, LRC_ERR_ARG, "C, lambda and info must be non-NULL");
    REQUIRE(n > 0 && batch > 0, LRC_ERR_ARG, "n and batch must be positive");
    REQUIRE(n <= (int64_t(1) << 20), LRC_ERR_ARG, "n too large");
    REQUIRE(ldc >= nc, LRC_ERR_ARG, "ldc < n (d_in for a projected group)");
    REQUIRE(batch == 1 || stride_c >= nc * ldc - (ldc - nc), LRC_ERR_ARG, "stride_c overlaps matrices");
    REQUIRE(n_vec >= 0 && n_vec <= n, LRC_ERR_ARG, "n_vec must be in [0, n]");
    REQUIRE(n_vec == 0 || (V && ldv >= n_vec), LRC_ERR_ARG, "V NULL or ldv < n_vec");
    REQUIRE(n_vec == 0 || batch == 1 || stride_v >= n * ldv - (ldv - n_vec), LRC_ERR_ARG,
            "stride_v overlaps matrices");
    return LRC_OK;
}

lrc_status lrc_eigh(const float *C, int64_t n, int64_t ldc, int64_t batch, int64_t stride_c, lrc_dtype prec,
                    double *lambda, float *V, int64_t ldv, int64_t n_vec, int64_t stride_v, void *ws,
                    size_t ws_bytes, int32_t *info, void *stream) {
    lrc_status st = check_eigh(C, n, ldc, batch, stride_c, lambda, V, ldv, n_vec, stride_v, info);
    if (st != LRC_OK) return st;
    REQUIRE(prec == LRC_F32 || prec == LRC_F64, LRC_ERR_DTYPE, "prec must be LRC_F32 or LRC_F64");
    size_t need = eigh_workspace(n, batch, n_vec, prec);
    REQUIRE(ws_bytes >= need && (need == 0 || (ws && aligned(ws, 256))), LRC_ERR_WORKSPACE,
            "workspace smaller than lrc_eigh_workspace() or not 256-byte aligned");
    EighArgs a{C, n, ldc, batch, stride_c, prec, lambda, V, ldv, n_vec, stride_v, info};
    return eigh_run(a, ws, ws_bytes, static_cast<hipStream_t>(stream));
}

static std::vector<EighArgs> eigh_groups(const lrc_eigh_group *g, int32_t count, lrc_dtype prec) {
    std::vector<EighArgs> v;
    v.reserve(size_t(count));
    for (int32_t i = 0; i < count; ++i)
        v.push_back(EighArgs{g[i].C, g[i].n, g[i].ldc, g[i].batch, g[i].stride_c, prec, g[i].lambda, g[i].V,
                             g[i].ldv, g[i].n_vec, g[i].stride_v, g[i].info, g[i].W, g[i].w_t, g[i].d_in,
                             g[i].ldw, g[i].stride_w, g[i].projected, g[i].L, g[i].ldl, g[i].stride_l, g[i].A,
                             g[i].lda, g[i].stride_a});
    return v;
}

size_t lrc_eigh_multi_workspace(const lrc_eigh_group *groups, int32_t count, lrc_dtype prec) {
    if (!groups || count <= 0) return 0;
    for (int32_t i = 0; i < count; ++i)
        if (groups[i].n <= 0 || groups[i].batch <= 0 || groups[i].n_vec < 0 || groups[i].n_vec > groups[i].n) return 0;
    std::vector<EighArgs> v = eigh_groups(groups, count, prec);
    return eigh_multi_workspace(v.data(), count, prec);
}

lrc_status lrc_eigh_multi(const lrc_eigh_group *groups, int32_t count, lrc_dtype prec, void *ws, size_t ws_bytes,
                          void *stream) {
    REQUIRE(groups && count > 0, LRC_ERR_ARG, "groups must be non-NULL and count positive");
    for (int32_t i = 0; i < count; ++i) {
        const lrc_eigh_group &g = groups[i];
        REQUIRE(g.projected == 0 || g.projected == 1, LRC_ERR_ARG, "projected must be 0 or 1");
        if (g.projected)
            REQUIRE(g.W && g.d_in > 128 && g.d_in < g.n && g.n_vec <= g.d_in, LRC_ERR_ARG,
                    "a projected group needs its range basis W with 128 < d_in < n and n_vec <= d_in");
        if (g.L)
            REQUIRE(g.W && g.ldl >= g.d_in && (g.batch == 1 || g.stride_l >= g.d_in * g.ldl - (g.ldl - g.d_in)),
                    LRC_ERR_ARG, "L needs the range basis W, ldl >= d_in and stride_l between members");
        if (g.A)
            REQUIRE(g.projected && g.n_vec > 0 && g.lda >= g.n_vec &&
                        (g.batch == 1 || g.stride_a >= g.d_in * g.lda - (g.lda - g.n_vec)),
                    LRC_ERR_ARG, "A needs a projected group, n_vec > 0, lda >= n_vec and stride_a between members");
        lrc_status st = check_eigh(g.C, g.n, g.ldc, g.batch, g.stride_c, g.lambda, g.V, g.ldv, g.n_vec, g.stride_v,
                                   g.info, g.projected ? g.d_in : g.n);
        if (st != LRC_OK) return st;
        if (g.W) {
            REQUIRE(g.w_t == LRC_BF16 || g.w_t == LRC_F32 || g.w_t == LRC_F64, LRC_ERR_DTYPE,
                    "w_t must be LRC_BF16, LRC_F32 or LRC_F64");
            REQUIRE(g.d_in > 0 && g.ldw >= g.n, LRC_ERR_ARG, "range basis: d_in must be positive and ldw >= n");
            REQUIRE(g.batch == 1 || g.stride_w >= g.d_in * g.ldw - (g.ldw - g.n), LRC_ERR_ARG,
                    "stride_w overlaps range bases");
        }
    }
    REQUIRE(prec == LRC_F32 || prec == LRC_F64, LRC_ERR_DTYPE, "prec must be LRC_F32 or LRC_F64");
    std::vector<EighArgs> v = eigh_groups(groups, count, prec);
    size_t need = eigh_multi_workspace(v.data(), count, prec);
    REQUIRE(ws_bytes >= need && (need == 0 || (ws && aligned(ws, 256))), LRC_ERR_WORKSPACE,
            "workspace smaller than lrc_eigh_multi_workspace() or not 256-byte aligned");
    return eigh_multi_run(v.data(), count, prec, ws, ws_bytes, static_cast<hipStream_t>(stream));
}

// ---------------------------------------------------------------------------------------------
lrc_status lrc_error_curve(const double *lambda, int64_t n, int64_t batch, double *eps, void *stream) {
    REQUIRE(lambda && eps, LRC_ERR_ARG, "lambda and eps must be non-NULL");
    REQUIRE(n > 0 && batch > 0, LRC_ERR_ARG, "n and batch must be positive");
    return error_curve_run(lambda, n, batch, eps, static_cast<hipStream_t>(stream));
}

// ---------------------------------------------------------------------------------------------
lrc_status lrc_factorize(const void *W, lrc_dtype w_t, int32_t trans_w, int64_t d_in, int64_t d_out, int64_t ldw,
                         const float *V, int64_t ldv, int64_t k, int64_t batch, int64_t stride_w,
                         int64_t stride_v, float *A, int64_t lda, int64_t stride_a, float *B, int64_t ldb,
                         int64_t stride_b, void *stream) {
    REQUIRE(W && V && (A || B), LRC_ERR_ARG, "W and V must be non-NULL, and A or B");
    REQUIRE(trans_w == 0 || trans_w == 1, LRC_ERR_ARG, "trans_w must be 0 or 1");
    REQUIRE(d_in > 0 && d_out > 0 && k > 0 && batch > 0, LRC_ERR_ARG, "sizes must be positive");
    REQUIRE(ldw >= d_out, LRC_ERR_ARG, "ldw < d_out");
    REQUIRE(ldv >= k && (!A || lda >= k), LRC_ERR_ARG, "ldv or lda < k");
    const int64_t vrows = trans_w ? d_in : d_out;
    REQUIRE(k <= vrows, LRC_ERR_ARG, "k larger than the rows of V");
    REQUIRE(!B || ldb >= vrows, LRC_ERR_ARG, "ldb < rows of V");
    REQUIRE(batch == 1 || (stride_w >= 0 && stride_v >= 0 && (!A || stride_a > 0) && (!B || stride_b > 0)),
            LRC_ERR_ARG, "bad batch strides");
    REQUIRE(w_t == LRC_BF16 || w_t == LRC_F32 || w_t == LRC_F64, LRC_ERR_DTYPE, "w_t must be bf16, f32 or f64");
    FactorizeArgs a{W, w_t, trans_w, d_in, d_out, ldw, V, ldv, k, batch, stride_w, stride_v,
                    A, lda, stride_a, B, ldb, stride_b};
    return factorize_run(a, static_cast<hipStream_t>(stream));
}

// ---------------------------------------------------------------------------------------------
size_t lrc_fisher_scores_workspace(int32_t n_mats, const int64_t *numel) {
    if (n_mats <= 0 || !numel) return 0;
    for (int i = 0; i < n_mats; ++i)
        if (numel[i] < 0) return 0;
    return fisher_workspace(n_mats, numel);
}

lrc_status lrc_fisher_scores(int32_t n_mats, const void *const *G, const void *const *W, const int64_t *numel,
                             lrc_dtype t, double *alpha, void *ws, size_t ws_bytes, int32_t *info, void *stream) {
    REQUIRE(n_mats > 0 && G && W && numel && alpha && info, LRC_ERR_ARG, "null argument or n_mats <= 0");
    REQUIRE(t == LRC_BF16 || t == LRC_F32, LRC_ERR_DTYPE, "t must be LRC_BF16 or LRC_F32");
    for (int i = 0; i < n_mats; ++i) {
        REQUIRE(numel[i] >= 0, LRC_ERR_ARG, "negative numel");
        REQUIRE(numel[i] == 0 || (G[i] && W[i]), LRC_ERR_ARG, "null G[m] or W[m]");
    }
    size_t need = fisher_workspace(n_mats, numel);
    REQUIRE(ws_bytes >= need && (need == 0 || (ws && aligned(ws, 256))), LRC_ERR_WORKSPACE,
            "workspace smaller than lrc_fisher_scores_workspace() or not 256-byte aligned");
    return fisher_run(n_mats, G, W, numel, t, alpha, ws, ws_bytes, info, static_cast<hipStream_t>(stream));
}

lrc_status lrc_fisher_scores_noalloc(int32_t n_mats, const void *const *G, const void *const *W,
                                     const int64_t *numel, lrc_dtype t, double *alpha, int32_t *info, void *stream) {
    REQUIRE(n_mats > 0 && G && W && numel && alpha && info, LRC_ERR_ARG, "null argument or n_mats <= 0");
    REQUIRE(t == LRC_BF16 || t == LRC_F32, LRC_ERR_DTYPE, "t must be LRC_BF16 or LRC_F32");
    for (int i = 0; i < n_mats; ++i) {
        REQUIRE(numel[i] >= 0, LRC_ERR_ARG, "negative numel");
        REQUIRE(numel[i] == 0 || (G[i] && W[i]), LRC_ERR_ARG, "null G[m] or W[m]");
    }
    return fisher_run_noalloc(n_mats, G, W, numel, t, alpha, info, static_cast<hipStream_t>(stream));
}

// ---------------------------------------------------------------------------------------------
size_t lrc_allocate_ranks_workspace(int32_t n_mats, int64_t n_items) {
    if (n_mats <= 0 || n_items < 0) return 0;
    return alloc_workspace(n_mats, n_items);
}

lrc_status lrc_allocate_ranks(int32_t n_mats, const double *alpha, const double *lambda_packed,
                              const int64_t *offsets, int64_t n_items, const double *eps0, const int64_t *cost,
                              const int32_t *k_min, int64_t budget_params, int32_t *k_out, void *ws,
                              size_t ws_bytes, int32_t *info, void *stream) {
    REQUIRE(n_mats > 0 && alpha && offsets && eps0 && cost && k_out && info, LRC_ERR_ARG,
            "null argument or n_mats <= 0");
    REQUIRE(n_items >= 0 && (n_items == 0 || lambda_packed), LRC_ERR_ARG, "bad n_items or lambda_packed");
    REQUIRE(n_items < (int64_t(1) << 31), LRC_ERR_ARG, "n_items too large");
    REQUIRE(budget_params >= 0, LRC_ERR_ARG, "negative budget");
    size_t need = alloc_workspace(n_mats, n_items);
    REQUIRE(ws_bytes >= need && (need == 0 || (ws && aligned(ws, 256))), LRC_ERR_WORKSPACE,
            "workspace smaller than lrc_allocate_ranks_workspace() or not 256-byte aligned");
    AllocArgs a{n_mats, alpha, lambda_packed, offsets, n_items, eps0, cost, k_min, budget_params, k_out, info};
    return alloc_run(a, ws, ws_bytes, static_cast<hipStream_t>(stream));
}

lrc_status lrc_allocate_proportional(int32_t n_mats, const double *alpha, int32_t n_budgets, const int64_t *budgets,
                                     int64_t *r_out, int32_t *info, void *stream) {
    REQUIRE(alpha && budgets && r_out && info, LRC_ERR_ARG, "null argument");
    REQUIRE(n_mats > 0 && n_mats <= PROP_MAX, LRC_ERR_ARG, "n_mats must be in 1 .. 1024");
    REQUIRE(n_budgets > 0, LRC_ERR_ARG, "n_budgets must be positive");
    return alloc_prop_run(n_mats, alpha, n_budgets, budgets, r_out, info, static_cast<hipStream_t>(stream));
}

lrc_status lrc_allocate_swift(int32_t n_mats, const double *beta, const double *eps_kbar, const int64_t *kbar,
                              const int64_t *cost, const int64_t *k_cap, double delta, int32_t n_alpha,
                              const double *alpha_grid, int64_t budget_params, double *scores, int32_t *k_out,
                              int32_t *info, void *stream) {
    REQUIRE(beta && eps_kbar && kbar && cost && k_cap && alpha_grid && scores && k_out && info, LRC_ERR_ARG,
            "null argument");
    REQUIRE(n_mats > 0 && n_mats <= 1024, LRC_ERR_ARG, "n_mats must be in 1 .. 1024");
    REQUIRE(n_alpha > 0 && n_alpha <= 65535, LRC_ERR_ARG, "n_alpha must be in 1 .. 65535");
    REQUIRE(budget_params >= 0, LRC_ERR_ARG, "negative budget");
    return alloc_swift_run(n_mats, beta, eps_kbar, kbar, cost, k_cap, delta, n_alpha, alpha_grid, budget_params,
                           scores, k_out, info, static_cast<hipStream_t>(stream));
}

size_t lrc_component_fisher_workspace(int64_t d_in, int64_t k, int64_t batch) {
    return (d_in > 0 && k > 0 && batch > 0) ? comp_fisher_workspace(d_in, k, batch) : 0;
}

lrc_status lrc_component_fisher(const void *W, const void *G, lrc_dtype t, int64_t d_in, int64_t d_out, int64_t ldw,
                                int64_t ldg, const float *V, int64_t ldv, int64_t k, int64_t batch, int64_t stride_w,
                                int64_t stride_g, int64_t stride_v, double *score, int64_t stride_s, void *ws,
                                size_t ws_bytes, void *stream) {
    REQUIRE(W && G && V && score, LRC_ERR_ARG, "null argument");
    REQUIRE(t == LRC_BF16 || t == LRC_F32, LRC_ERR_DTYPE, "W and G must be bf16 or fp32");
    REQUIRE(d_in > 0 && d_out > 0 && k > 0 && k <= d_out && batch > 0, LRC_ERR_ARG, "bad sizes");
    REQUIRE(ldw >= d_out && ldg >= d_out && ldv >= k, LRC_ERR_ARG, "bad leading dims");
    REQUIRE(batch == 1 || (stride_w >= 0 && stride_g >= 0 && stride_v >= 0 && stride_s >= k), LRC_ERR_ARG,
            "bad batch strides");
    const size_t need = comp_fisher_workspace(d_in, k, batch);
    REQUIRE(ws && ws_bytes >= need && aligned(ws, 256), LRC_ERR_WORKSPACE,
            "workspace smaller than lrc_component_fisher_workspace() or not 256-byte aligned");
    CompFisherArgs a{W, G, t, d_in, d_out, ldw, ldg, V, ldv, k, batch, stride_w, stride_g, stride_v, score,
                     batch == 1 ? k : stride_s};
    return comp_fisher_run(a, ws, ws_bytes, static_cast<hipStream_t>(stream));
}

size_t lrc_allocate_components_workspace(int32_t n_mats, int64_t n_items) {
    if (n_mats <= 0 || n_items < 0) return 0;
    return alloc_workspace(n_mats, n_items);
}

lrc_status lrc_allocate_components(int32_t n_mats, const double *score_packed, const int64_t *offsets,
                                   int64_t n_items, const int64_t *cost, const int32_t *k_min, int64_t budget_params,
                                   int32_t *k_out, uint8_t *selected, void *ws, size_t ws_bytes, int32_t *info,
                                   void *stream) {
    REQUIRE(n_mats > 0 && offsets && cost && k_out && info, LRC_ERR_ARG, "null argument or n_mats <= 0");
    REQUIRE(n_items >= 0 && (n_items == 0 || score_packed), LRC_ERR_ARG, "bad n_items or score_packed");
    REQUIRE(n_items < (int64_t(1) << 31), LRC_ERR_ARG, "n_items too large");
    REQUIRE(budget_params >= 0, LRC_ERR_ARG, "negative budget");
    size_t need = alloc_workspace(n_mats, n_items);
    REQUIRE(ws_bytes >= need && (need == 0 || (ws && aligned(ws, 256))), LRC_ERR_WORKSPACE,
            "workspace smaller than lrc_allocate_components_workspace() or not 256-byte aligned");
    AllocArgs a{n_mats, nullptr, score_packed, offsets, n_items, nullptr, cost, k_min, budget_params, k_out, info};
    a.per_component = 1;
    a.selected = selected;
    return alloc_run(a, ws, ws_bytes, static_cast<hipStream_t>(stream));
}

// ---------------------------------------------------------------------------------------------
size_t lrc_cholesky_workspace(int64_t n) { return n > 0 ? cholesky_workspace(n) : 0; }

lrc_status lrc_cholesky(double *A, int64_t n, int64_t lda, void *ws, size_t ws_bytes, int32_t *info, void *stream) {
    REQUIRE(A && info, LRC_ERR_ARG, "A and info must be non-NULL");
    REQUIRE(n > 0 && lda >= n, LRC_ERR_ARG, "bad n or lda");
    size_t need = cholesky_workspace(n);
    REQUIRE(ws_bytes >= need && (need == 0 || (ws && aligned(ws, 256))), LRC_ERR_WORKSPACE,
            "workspace smaller than lrc_cholesky_workspace() or not 256-byte aligned");
    return cholesky_run(A, n, lda, ws, ws_bytes, info, static_cast<hipStream_t>(stream));
}

size_t lrc_trmm_workspace(int64_t m, int64_t n) { return (m > 0 && n > 0) ? trmm_workspace(m, n) : 0; }

lrc_status lrc_trmm(int32_t side, int32_t trans, int64_t m, int64_t n, const double *L, int64_t ldl, double *B,
                    int64_t ldb, void *ws, size_t ws_bytes, void *stream) {
    REQUIRE(L && B, LRC_ERR_ARG, "L and B must be non-NULL");
    REQUIRE((side == 0 || side == 1) && (trans == 0 || trans == 1), LRC_ERR_ARG, "side/trans must be 0 or 1");
    REQUIRE(m > 0 && n > 0 && ldb >= n && ldl >= (side ? n : m), LRC_ERR_ARG, "bad sizes or leading dims");
    size_t need = trmm_workspace(m, n);
    REQUIRE(ws_bytes >= need && ws && aligned(ws, 256), LRC_ERR_WORKSPACE,
            "workspace smaller than lrc_trmm_workspace() or not 256-byte aligned");
    return trmm_run(side, trans, m, n, L, ldl, B, ldb, ws, static_cast<hipStream_t>(stream));
}

size_t lrc_trsm_workspace(int32_t side, int64_t m, int64_t n) {
    return (m > 0 && n > 0 && (side == 0 || side == 1)) ? trsm_workspace(side, m, n) : 0;
}

lrc_status lrc_trsm(int32_t side, int32_t trans, int64_t m, int64_t n, const double *L, int64_t ldl, double *B,
                    int64_t ldb, void *ws, size_t ws_bytes, void *stream) {
    REQUIRE(L && B, LRC_ERR_ARG, "L and B must be non-NULL");
    REQUIRE((side == 0 || side == 1) && (trans == 0 || trans == 1), LRC_ERR_ARG, "side/trans must be 0 or 1");
    REQUIRE(m > 0 && n > 0 && ldb >= n && ldl >= (side ? n : m), LRC_ERR_ARG, "bad sizes or leading dims");
    size_t need = trsm_workspace(side, m, n);
    REQUIRE(ws_bytes >= need && ws && aligned(ws, 256), LRC_ERR_WORKSPACE,
            "workspace smaller than lrc_trsm_workspace() or not 256-byte aligned");
    return trsm_run(side, trans, m, n, L, ldl, B, ldb, ws, static_cast<hipStream_t>(stream));
}

lrc_status lrc_sym_to_f64(const float *C, int64_t n, int64_t ldc, double scale, double *A, int64_t lda,
                          void *stream) {
    REQUIRE(C && A, LRC_ERR_ARG, "C and A must be non-NULL");
    REQUIRE(n > 0 && ldc >= n && lda >= n, LRC_ERR_ARG, "bad n or leading dims");
    return sym_to_f64_run(C, n, ldc, scale, A, lda, static_cast<hipStream_t>(stream));
}

lrc_status lrc_to_f64(const void *X, lrc_dtype t, int64_t rows, int64_t cols, int64_t ldx, double scale, double *Y,
                      int64_t ldy, void *stream) {
    REQUIRE(X && Y, LRC_ERR_ARG, "X and Y must be non-NULL");
    REQUIRE(t == LRC_BF16 || t == LRC_F32 || t == LRC_F64, LRC_ERR_DTYPE, "X must be bf16, fp32 or fp64");
    REQUIRE(rows > 0 && cols > 0 && ldx >= cols && ldy >= cols, LRC_ERR_ARG, "bad sizes or leading dims");
    return to_f64_run(X, t, rows, cols, ldx, scale, Y, ldy, static_cast<hipStream_t>(stream));
}

// C = W^T H W from the input covariance H = X^T X (SAES-SVD page, section 1 of the method (CEALC):
// the closed form works from the layer's input covariance H); the same C as the covariance of
// Y = X W by associativity.  fp64 workspace: H widened to both triangles, W widened, T = H W.
static size_t cov_from_input_layout(int64_t d_in, int64_t d_out, size_t *offs) {
    const size_t sz[3] = {size_t(d_in) * size_t(d_in), size_t(d_in) * size_t(d_out), size_t(d_in) * size_t(d_out)};
    size_t off = 0;
    for (int i = 0; i < 3; ++i) {
        if (offs) offs[i] = off;
        off += (sz[i] * sizeof(double) + 255) / 256 * 256;
    }
    return off;
}

size_t lrc_cov_from_input_workspace(int64_t d_in, int64_t d_out) {
    return (d_in > 0 && d_out > 0) ? cov_from_input_layout(d_in, d_out, nullptr) : 0;
}

lrc_status lrc_cov_from_input(const float *H, int64_t d_in, int64_t ldh, const void *W, lrc_dtype w_t, int64_t d_out,
                              int64_t ldw, float *C, int64_t ldc, void *ws, size_t ws_bytes, void *stream) {
    REQUIRE(H && W && C, LRC_ERR_ARG, "H, W and C must be non-NULL");
    REQUIRE(w_t == LRC_BF16 || w_t == LRC_F32 || w_t == LRC_F64, LRC_ERR_DTYPE, "W must be bf16, fp32 or fp64");
    REQUIRE(d_in > 0 && d_out > 0 && ldh >= d_in && ldw >= d_out && ldc >= d_out, LRC_ERR_ARG,
            "bad sizes or leading dims");
    size_t offs[3];
    const size_t need = cov_from_input_layout(d_in, d_out, offs);
    REQUIRE(ws && ws_bytes >= need && reinterpret_cast<uintptr_t>(ws) % 256 == 0, LRC_ERR_WORKSPACE,
            "workspace smaller than lrc_cov_from_input_workspace() or not 256-byte aligned");
    const hipStream_t s = static_cast<hipStream_t>(stream);
    char *base = static_cast<char *>(ws);
    double *H64 = reinterpret_cast<double *>(base + offs[0]);
    double *W64 = reinterpret_cast<double *>(base + offs[1]);
    double *T = reinterpret_cast<double *>(base + offs[2]);
    lrc_status st = sym_to_f64_run(H, d_in, ldh, 1.0, H64, d_in, s);
    if (st == LRC_OK) st = to_f64_run(W, w_t, d_in, d_out, ldw, 1.0, W64, d_out, s);
    // T = H W (d_in x d_out), then C[upper] = W^T T rounded once to fp32
    if (st == LRC_OK) st = dgemm_run(0, 0, d_in, d_out, d_in, H64, d_in, W64, d_out, T, d_out, 0, nullptr, s);
    if (st == LRC_OK) st = dgemm_run(1, 0, d_out, d_out, d_in, W64, d_out, T, d_out, nullptr, ldc, 2, C, s);
    return st;
}

lrc_status lrc_gram_f64(const double *B, int64_t m, int64_t n, int64_t ldb, float *G, int64_t ldg, void *stream) {
    REQUIRE(B && G, LRC_ERR_ARG, "B and G must be non-NULL");
    REQUIRE(m > 0 && n > 0 && ldb >= n && ldg >= m, LRC_ERR_ARG, "bad sizes or leading dims");
    return gram_f64_run(B, m, n, ldb, G, ldg, static_cast<hipStream_t>(stream));
}

}  // extern "C"
