// Internal declarations of liblrc (not installed, not part of the C ABI).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <string>

#include "../../include/lrc.h"

namespace lrc {

// ---------------------------------------------------------------------------------------------
// host-side error plumbing
// ---------------------------------------------------------------------------------------------
lrc_status fail(lrc_status s, const std::string &msg);
lrc_status hip_fail(hipError_t e, const char *what);

#define LRC_HIP(call)                                        \
    do {                                                     \
        hipError_t e_ = (call);                              \
        if (e_ != hipSuccess) return ::lrc::hip_fail(e_, #call); \
    } while (0)

#define LRC_LAUNCH_CHECK(what)                                    \
    do {                                                          \
        hipError_t e_ = hipGetLastError();                        \
        if (e_ != hipSuccess) return ::lrc::hip_fail(e_, what);   \
    } while (0)

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Bump allocator over a caller-provided workspace.  carve() returns nullptr when the
// workspace is exhausted; callers size the workspace with the matching *_workspace query,
// so a nullptr here is an internal error.
struct Carver {
    char *base;
    size_t size;
    size_t off = 0;
    Carver(void *b, size_t s) : base(static_cast<char *>(b)), size(s) {}
    template <class T>
    T *carve(size_t count) {
        size_t bytes = align256(count * sizeof(T));
        if (off + bytes > size) return nullptr;
        T *p = reinterpret_cast<T *>(base + off);
        off += bytes;
        return p;
    }
};
// The same layout, only counting bytes (for the *_workspace queries).
struct Counter {
    size_t off = 0;
    template <class T>
    void carve(size_t count) { off += align256(count * sizeof(T)); }
};

inline int cdiv(int64_t a, int64_t b) { return static_cast<int>((a + b - 1) / b); }

// Kernel timing (api.hip).  timing_sample returns true when this launch of `kernel` is one of the
// sampled ones; the caller then launches with hipExtLaunchKernelGGL and the two events, which the
// dispatch itself records at the kernel's start and end (so the duration excludes queueing).
bool timing_sample(const char *kernel, double work, hipEvent_t *start, hipEvent_t *stop);

#define LRC_TIMED_LAUNCH(name, work, kern, grid, block, shmem, stream, ...)                          \
    do {                                                                                            \
        hipEvent_t ts_, te_;                                                                        \
        if (::lrc::timing_sample(name, work, &ts_, &te_))                                           \
            hipExtLaunchKernelGGL(kern, grid, block, shmem, stream, ts_, te_, 0, __VA_ARGS__);      \
        else                                                                                        \
            hipLaunchKernelGGL(kern, grid, block, shmem, stream, __VA_ARGS__);                      \
    } while (0)

// ---------------------------------------------------------------------------------------------
// device helpers
// ---------------------------------------------------------------------------------------------
typedef uint16_t bf16_t;  // raw bf16 bit pattern

__device__ __forceinline__ float bf16_to_f32(bf16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// Round fp32 to bf16, nearest-even (finite inputs; NaN stays NaN).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return bf16_t((u >> 16) | 0x40);
    u += 0x7fffu + ((u >> 16) & 1u);
    return bf16_t(u >> 16);
}

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(4 * sizeof(double)))) double f64x4_t;
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------------------------
// per-op launchers (arguments already validated by api.hip)
// ---------------------------------------------------------------------------------------------
struct CovArgs {
    const void *X;
    lrc_dtype x_t;
    int64_t n_tok, d_in, ldx;
    const void *W;
    int64_t d_out, ldw;
    int32_t n_blocks;
    float *C;
    int64_t ldc;
    int32_t *info;
    // range-projected covariance (lrc_cov_accumulate_range): W is NULL and C += (X L)^T (X L) with
    // L (d_in x d_in, fp64, lower triangle read, leading dim ldl); d_out == d_in
    const double *L = nullptr;
    int64_t ldl = 0;
};
size_t cov_range_workspace(int64_t n_tok, int64_t d);
size_t cov_workspace(lrc_dtype x_t, int64_t n_tok, int64_t d_in, int has_w, int64_t d_out, int32_t n_blocks);
lrc_status cov_run(const CovArgs &a, void *ws, size_t ws_bytes, hipStream_t s);

struct EighArgs {
    const float *C;
    int64_t n, ldc, batch, stride_c;
    lrc_dtype prec;
    double *lambda;
    float *V;
    int64_t ldv, n_vec, stride_v;
    int32_t *info;
    // optional range basis (lrc_eigh_group): C = (X W)^T (X W) with W d_in x n
    const void *W = nullptr;
    lrc_dtype w_t = LRC_BF16;
    int64_t d_in = 0, ldw = 0, stride_w = 0;
    // C holds B = Q^T C Q (d_in x d_in), the covariance of lrc_cov_accumulate_range
    int32_t projected = 0;
    // optional factor of W W^T from lrc_range_factor (lower, d_in x d_in, member b at L + b stride_l)
    const double *L = nullptr;
    int64_t ldl = 0, stride_l = 0;
    // optional, projected members: A = W V[:, :n_vec] (d_in x n_vec fp32) formed as L U
    float *A = nullptr;
    int64_t lda = 0, stride_a = 0;
};
lrc_status range_factor_enqueue(const void *W, lrc_dtype w_t, int64_t r, int64_t n, int64_t ldw, double *Wf,
                                double *L, int64_t ldl, void *chol_ws, int32_t *info, hipStream_t s);
size_t eigh_workspace(int64_t n, int64_t batch, int64_t n_vec, lrc_dtype prec);
lrc_status eigh_run(const EighArgs &a, void *ws, size_t ws_bytes, hipStream_t s);
// several groups in one call (prec overrides each group's own)
size_t eigh_multi_workspace(const EighArgs *g, int count, lrc_dtype prec);
lrc_status eigh_multi_run(const EighArgs *g, int count, lrc_dtype prec, void *ws, size_t ws_bytes, hipStream_t s);
// small-n batched Jacobi (n <= 128)
size_t jacobi_workspace(int64_t n, int64_t batch, lrc_dtype prec);
lrc_status jacobi_run(const EighArgs &a, void *ws, size_t ws_bytes, hipStream_t s);

lrc_status error_curve_run(const double *lambda, int64_t n, int64_t batch, double *eps, hipStream_t s);

struct FactorizeArgs {
    const void *W;
    lrc_dtype w_t;
    int trans_w;
    int64_t d_in, d_out, ldw;
    const float *V;
    int64_t ldv, k, batch, stride_w, stride_v;
    float *A;
    int64_t lda, stride_a;
    float *B;
    int64_t ldb, stride_b;
};
lrc_status factorize_run(const FactorizeArgs &a, hipStream_t s);

size_t fisher_workspace(int32_t n_mats, const int64_t *numel);
lrc_status fisher_run(int32_t n_mats, const void *const *G, const void *const *W, const int64_t *numel,
                      lrc_dtype t, double *alpha, void *ws, size_t ws_bytes, int32_t *info, hipStream_t s);
// the same with the partials in the library's file-scope device array (no workspace, no allocation)
lrc_status fisher_run_noalloc(int32_t n_mats, const void *const *G, const void *const *W, const int64_t *numel,
                              lrc_dtype t, double *alpha, int32_t *info, hipStream_t s);
int64_t fisher_scratch_partials();

struct AllocArgs {
    int32_t n_mats;
    const double *alpha, *lambda_packed;
    const int64_t *offsets;
    int64_t n_items;
    const double *eps0;
    const int64_t *cost;
    const int32_t *k_min;
    int64_t budget;
    int32_t *k_out;
    int32_t *info;
    int per_component = 0;       // 1: lambda_packed holds per-component scores, p = s / cost
    uint8_t *selected = nullptr;  // optional mask of kept components, one byte per item
};
size_t alloc_workspace(int32_t n_mats, int64_t n_items);
lrc_status alloc_run(const AllocArgs &a, void *ws, size_t ws_bytes, hipStream_t s);

size_t cholesky_workspace(int64_t n);
lrc_status cholesky_run(double *A, int64_t n, int64_t lda, void *ws, size_t ws_bytes, int32_t *info,
                        hipStream_t s);
size_t trmm_workspace(int64_t m, int64_t n);
lrc_status trmm_run(int side, int trans, int64_t m, int64_t n, const double *L, int64_t ldl, double *B,
                    int64_t ldb, void *ws, hipStream_t s);
size_t trsm_workspace(int side, int64_t m, int64_t n);
lrc_status trsm_run(int side, int trans, int64_t m, int64_t n, const double *L, int64_t ldl, double *B,
                    int64_t ldb, void *ws, hipStream_t s);
lrc_status sym_to_f64_run(const float *C, int64_t n, int64_t ldc, double scale, double *A, int64_t lda,
                          hipStream_t s);
lrc_status to_f64_run(const void *X, lrc_dtype t, int64_t rows, int64_t cols, int64_t ldx, double scale,
                      double *Y, int64_t ldy, hipStream_t s);
// C = op(A) op(B) in fp64 (ta, tb: 0 plain, 1 transposed; tiles 0 all, 1 lower, 2 upper); with Cf the
// product goes to Cf as fp32 instead
// Swift-SVD allocation candidates (one per alpha of a grid)
lrc_status alloc_swift_run(int32_t n, const double *beta, const double *eps_kbar, const int64_t *kbar,
                           const int64_t *cost, const int64_t *k_cap, double delta, int32_t n_alpha,
                           const double *alpha_grid, int64_t budget, double *scores, int32_t *k_out, int32_t *info,
                           hipStream_t s);
// per-component empirical-Fisher scores s_i = ((W v_i) . (G v_i))^2
struct CompFisherArgs {
    const void *W, *G;
    lrc_dtype t;
    int64_t d_in, d_out, ldw, ldg;
    const float *V;
    int64_t ldv, k, batch, stride_w, stride_g, stride_v;
    double *score;
    int64_t stride_s;
};
size_t comp_fisher_workspace(int64_t d_in, int64_t k, int64_t batch);
lrc_status comp_fisher_run(const CompFisherArgs &a, void *ws, size_t ws_bytes, hipStream_t s);
constexpr int PROP_MAX = 1024;  // matrices per proportional allocation
lrc_status alloc_prop_run(int32_t n, const double *alpha, int32_t nb, const int64_t *budgets, int64_t *r_out,
                          int32_t *info, hipStream_t s);
lrc_status dgemm_run(int ta, int tb, int64_t M, int64_t N, int64_t K, const double *A, int64_t lda, const double *B,
                     int64_t ldb, double *C, int64_t ldc, int tiles, float *Cf, hipStream_t s);
lrc_status gram_f64_run(const double *B, int64_t m, int64_t n, int64_t ldb, float *G, int64_t ldg,
                        hipStream_t s);
// C (m x n) = L B with L lower triangular (m x m, its strict upper triangle not read), fp64
lrc_status lower_product_run(int64_t m, int64_t n, const double *L, int64_t ldl, const double *B, int64_t ldb,
                             double *C, int64_t ldc, hipStream_t s);

}  // namespace lrc
