// Covariance accumulation C[upper] += (X W)^T (X W).
//
// Swift-SVD page, section 2-ga: the covariance of the layer output Y = XW is aggregated over
// the calibration tokens (incrementally), before one eigendecomposition.  Per-head diagonal
// blocks: WSVD page, methodology 1 (per-head SVD of W_K).
//
// Two phases per chunk of tokens, both on the GPU:
//   1. Y^T (d_out x T) = W^T X^T for the chunk, stored token-contiguous in the workspace.
//   2. upper-triangle rank-T update of C from Y^T (only tiles I <= J; only diagonal blocks
//      in the per-head case).
// Storing Y^T token-contiguous makes both operands of phase 2 contiguous along the
// contraction (token) axis.
//
// Paths:
//   * generic: any dtype/alignment, fp32 arithmetic, LDS-tiled FMA (used for fp32 inputs).
//   * mfma (cov_mfma.hip): bf16 inputs with 16-byte aligned rows; bf16 MFMA for Y, each output
//     scaled by a power of two and split into fp16 hi + lo, C += 2^-(e_i + e_j) (hi^T hi + hi^T lo +
//     lo^T hi) with fp16 MFMA and fp32 accumulation, plus the diagonal's sum of lo^2 on its own.
#include "lrc_internal.h"
#include "cov_mfma.h"

namespace lrc {

constexpr int GT = 64;   // generic tile
constexpr int GK = 16;   // generic k step
constexpr int64_t GEN_CHUNK = 4096;  // tokens per generic chunk

template <class XT>
__device__ __forceinline__ float ld_as_f32(const XT *p, int64_t i);
template <>
__device__ __forceinline__ float ld_as_f32<bf16_t>(const bf16_t *p, int64_t i) { return bf16_to_f32(p[i]); }
template <>
__device__ __forceinline__ float ld_as_f32<float>(const float *p, int64_t i) { return p[i]; }

// Y^T[i][t] = sum_k X[t0+t][k] W[k][i]  (W == nullptr: Y^T[i][t] = X[t0+t][i])
template <class XT>
__global__ void __launch_bounds__(256) k_gemm_y_generic(const XT *__restrict__ X, int64_t ldx, const XT *__restrict__ W,
                                                        int64_t ldw, int64_t d_in, int64_t d_out, int64_t t0, int64_t tc,
                                                        float *__restrict__ Yt, int64_t ldy) {
    __shared__ float As[GK][GT + 1];  // W tile: k x i
    __shared__ float Bs[GK][GT + 1];  // X tile: k x t
    const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
    const int64_t i0 = int64_t(blockIdx.x) * GT, tt0 = int64_t(blockIdx.y) * GT;
    if (!W) {
        for (int e = threadIdx.x; e < GT * GT; e += 256) {
            const int ii = e / GT, tt = e % GT;
            const int64_t i = i0 + ii, t = tt0 + tt;
            if (i < d_out && t < tc) Yt[i * ldy + t] = ld_as_f32(X, (t0 + t) * ldx + i);
        }
        return;
    }
    float acc[4][4] = {};
    for (int64_t k0 = 0; k0 < d_in; k0 += GK) {
        for (int e = threadIdx.x; e < GK * GT; e += 256) {
            const int kk = e / GT, c = e % GT;
            const int64_t k = k0 + kk;
            As[kk][c] = (k < d_in && i0 + c < d_out) ? ld_as_f32(W, k * ldw + i0 + c) : 0.f;
            const int tt = e / GK, kk2 = e % GK;
            const int64_t k2 = k0 + kk2;
            Bs[kk2][tt] = (k2 < d_in && tt0 + tt < tc) ? ld_as_f32(X, (t0 + tt0 + tt) * ldx + k2) : 0.f;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < GK; ++kk) {
            float a[4], b[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                a[q] = As[kk][ty * 4 + q];
                b[q] = Bs[kk][tx * 4 + q];
            }
#pragma unroll
            for (int p = 0; p < 4; ++p)
#pragma unroll
                for (int q = 0; q < 4; ++q) acc[p][q] = fmaf(a[p], b[q], acc[p][q]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int p = 0; p < 4; ++p)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int64_t i = i0 + ty * 4 + p, t = tt0 + tx * 4 + q;
            if (i < d_out && t < tc) Yt[i * ldy + t] = acc[p][q];
        }
}

// C_h[r][c] += sum_t Y^T[h hd + r][t] Y^T[h hd + c][t] for r <= c (upper, incl. diagonal)
__global__ void __launch_bounds__(256) k_syrk_generic(const float *__restrict__ Yt, int64_t ldy, int64_t tc,
                                                      float *__restrict__ C, int64_t ldc, int64_t hd) {
    const int I = blockIdx.x, J = blockIdx.y, h = blockIdx.z;
    if (I > J) return;
    __shared__ float As[GK][GT + 1];
    __shared__ float Bs[GK][GT + 1];
    const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
    const int64_t r0 = int64_t(I) * GT, c0 = int64_t(J) * GT;
    const float *Yh = Yt + int64_t(h) * hd * ldy;
    float acc[4][4] = {};
    for (int64_t t0 = 0; t0 < tc; t0 += GK) {
        for (int e = threadIdx.x; e < GK * GT; e += 256) {
            const int rr = e / GK, kk = e % GK;
            const int64_t t = t0 + kk;
            As[kk][rr] = (t < tc && r0 + rr < hd) ? Yh[(r0 + rr) * ldy + t] : 0.f;
            Bs[kk][rr] = (t < tc && c0 + rr < hd) ? Yh[(c0 + rr) * ldy + t] : 0.f;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < GK; ++kk) {
            float a[4], b[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                a[q] = As[kk][ty * 4 + q];
                b[q] = Bs[kk][tx * 4 + q];
            }
#pragma unroll
            for (int p = 0; p < 4; ++p)
#pragma unroll
                for (int q = 0; q < 4; ++q) acc[p][q] = fmaf(a[p], b[q], acc[p][q]);
        }
        __syncthreads();
    }
    float *Ch = C + int64_t(h) * hd * ldc;
#pragma unroll
    for (int p = 0; p < 4; ++p)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int64_t r = r0 + ty * 4 + p, c = c0 + tx * 4 + q;
            if (r < hd && c < hd && r <= c) Ch[r * ldc + c] += acc[p][q];
        }
}

// info = 1 when a diagonal entry of the updated C is not finite
__global__ void k_cov_check(const float *__restrict__ C, int64_t ldc, int64_t hd, int32_t n_blocks, int32_t *info) {
    __shared__ int bad;
    if (threadIdx.x == 0) bad = 0;
    __syncthreads();
    const int64_t n = int64_t(hd) * n_blocks;
    for (int64_t i = threadIdx.x; i < n; i += blockDim.x) {
        const int64_t h = i / hd, r = i % hd;
        if (!isfinite(C[h * hd * ldc + r * ldc + r])) atomicOr(&bad, 1);
    }
    __syncthreads();
    if (threadIdx.x == 0) *info = bad ? LRC_INFO_NONFINITE : LRC_INFO_OK;
}

static bool use_mfma(const CovArgs &a) {
    return cov_mfma_supported(a.x_t, a.X, a.ldx, a.W, a.ldw, a.d_in, a.d_out, a.n_blocks);
}

size_t cov_workspace(lrc_dtype x_t, int64_t n_tok, int64_t d_in, int has_w, int64_t d_out, int32_t n_blocks) {
    if (x_t == LRC_BF16 && cov_mfma_shape_ok(d_in, d_out, n_blocks))
        return cov_mfma_workspace(n_tok, d_in, has_w, d_out, n_blocks);
    Counter c;
    const int64_t tc = std::min<int64_t>(GEN_CHUNK, n_tok);
    c.carve<float>(size_t(d_out) * size_t(tc));
    return c.off;
}

lrc_status cov_run(const CovArgs &a, void *ws, size_t ws_bytes, hipStream_t s) {
    const int64_t hd = a.d_out / a.n_blocks;
    if (use_mfma(a)) {
        lrc_status st = cov_mfma_run(a, ws, ws_bytes, s);
        if (st != LRC_OK) return st;
    } else {
        Carver cv(ws, ws_bytes);
        const int64_t tcmax = std::min<int64_t>(GEN_CHUNK, a.n_tok);
        float *Yt = cv.carve<float>(size_t(a.d_out) * size_t(tcmax));
        if (!Yt) return fail(LRC_ERR_WORKSPACE, "covariance workspace too small");
        const int64_t ldy = tcmax;
        for (int64_t t0 = 0; t0 < a.n_tok; t0 += tcmax) {
            const int64_t tc = std::min(tcmax, a.n_tok - t0);
            dim3 g1(cdiv(a.d_out, GT), cdiv(tc, GT));
            if (a.x_t == LRC_BF16)
                hipLaunchKernelGGL(k_gemm_y_generic<bf16_t>, g1, dim3(256), 0, s, static_cast<const bf16_t *>(a.X), a.ldx,
                                   static_cast<const bf16_t *>(a.W), a.ldw, a.d_in, a.d_out, t0, tc, Yt, ldy);
            else
                hipLaunchKernelGGL(k_gemm_y_generic<float>, g1, dim3(256), 0, s, static_cast<const float *>(a.X), a.ldx,
                                   static_cast<const float *>(a.W), a.ldw, a.d_in, a.d_out, t0, tc, Yt, ldy);
            LRC_LAUNCH_CHECK("k_gemm_y_generic");
            dim3 g2(cdiv(hd, GT), cdiv(hd, GT), a.n_blocks);
            hipLaunchKernelGGL(k_syrk_generic, g2, dim3(256), 0, s, Yt, ldy, tc, a.C, a.ldc, hd);
            LRC_LAUNCH_CHECK("k_syrk_generic");
        }
    }
    hipLaunchKernelGGL(k_cov_check, dim3(1), dim3(256), 0, s, a.C, a.ldc, hd, a.n_blocks, a.info);
    LRC_LAUNCH_CHECK("k_cov_check");
    return LRC_OK;
}

}  // namespace lrc
