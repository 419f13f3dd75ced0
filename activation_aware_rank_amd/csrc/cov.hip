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
//   * fp32: any dtype/alignment, fp32 arithmetic on the 32x32x2 fp32 MFMA (used for fp32 inputs).
//   * mfma (cov_mfma.hip): bf16 inputs with 16-byte aligned rows; bf16 MFMA for Y, each output
//     scaled by a power of two and split into fp16 hi + lo, C += 2^-(e_i + e_j) (hi^T hi + hi^T lo +
//     lo^T hi) with fp16 MFMA and fp32 accumulation, plus the diagonal's sum of lo^2 on its own.
//   * range-projected (cov_mfma.hip, lrc_cov_accumulate_range): C += (X L)^T (X L) for the factor L of
//     W W^T, L^T as three bf16 pieces in the same GEMM, then the same split SYRK.
#include "lrc_internal.h"
#include "cov_mfma.h"

namespace lrc {

constexpr int64_t GEN_CHUNK = 4096;  // tokens per chunk of the fp32 path

template <class XT>
__device__ __forceinline__ float ld_as_f32(const XT *p, int64_t i);
template <>
__device__ __forceinline__ float ld_as_f32<bf16_t>(const bf16_t *p, int64_t i) { return bf16_to_f32(p[i]); }
template <>
__device__ __forceinline__ float ld_as_f32<float>(const float *p, int64_t i) { return p[i]; }

// fp32 MFMA path (fp32 inputs, and bf16 inputs the bf16 MFMA path cannot take): 128 x 128 block
// tiles on 4 waves of 64 x 64, each 2 x 2 tiles of the 32x32x2 fp32 MFMA (one product per lane and
// k slice, fp32 accumulation, so the same arithmetic as an fp32 FMA chain), k steps of FK staged
// k-major in two LDS buffers; the next step's values are loaded into registers while the current
// step's MFMAs run.
constexpr int FT = 128;      // block tile
constexpr int FK = 16;       // k step
constexpr int FLD = FT + 1;  // padded LDS row
constexpr int FPT = FT * FK / 256;  // values per thread and operand per step

// Element (k, m) of an operand tile: KC operands are contiguous along k (X and Y^T rows: 16 threads
// read 16 consecutive k of one row), the others along m (W rows).  Values past `rows` or `klen` are 0.
template <class ET, bool KC>
struct F32Operand {
    const ET *p;
    int64_t ld;
    int rows;
    __device__ __forceinline__ void load(int64_t k0, int64_t klen, float (&r)[FPT]) const {
#pragma unroll
        for (int u = 0; u < FPT; ++u) {
            const int idx = int(threadIdx.x) + 256 * u;
            const int k = KC ? idx % FK : idx / FT, m = KC ? idx / FK : idx % FT;
            const int64_t kk = k0 + k;
            r[u] = (m < rows && kk < klen) ? ld_as_f32(p, KC ? int64_t(m) * ld + kk : kk * ld + m) : 0.f;
        }
    }
    __device__ __forceinline__ void store(const float (&r)[FPT], float (*s)[FLD]) const {
#pragma unroll
        for (int u = 0; u < FPT; ++u) {
            const int idx = int(threadIdx.x) + 256 * u;
            const int k = KC ? idx % FK : idx / FT, m = KC ? idx / FK : idx % FT;
            s[k][m] = r[u];
        }
    }
};

// acc[x][y] = sum over k < klen of A(k, m) B(k, n) for the wave's 64 x 64 tile
template <class OA, class OB>
__device__ __forceinline__ void f32_mainloop(const OA &A, const OB &B, int64_t klen, f32x16_t (&acc)[2][2]) {
    __shared__ float sa[2][FK][FLD], sb[2][FK][FLD];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int y = 0; y < 2; ++y) acc[x][y] = f32x16_t{};
    const int64_t nk = (klen + FK - 1) / FK;
    if (nk <= 0) return;
    float ra[FPT], rb[FPT];
    A.load(0, klen, ra);
    B.load(0, klen, rb);
    A.store(ra, sa[0]);
    B.store(rb, sb[0]);
    __syncthreads();
    for (int64_t kt = 0; kt < nk; ++kt) {
        const int cur = int(kt & 1);
        if (kt + 1 < nk) {
            A.load((kt + 1) * FK, klen, ra);
            B.load((kt + 1) * FK, klen, rb);
        }
#pragma unroll
        for (int kk = 0; kk < FK; kk += 2) {
            const int k = kk + (lane >> 5);
            const float a0 = sa[cur][k][wm + (lane & 31)], a1 = sa[cur][k][wm + 32 + (lane & 31)];
            const float b0 = sb[cur][k][wn + (lane & 31)], b1 = sb[cur][k][wn + 32 + (lane & 31)];
            acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, b0, acc[0][0], 0, 0, 0);
            acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, b1, acc[0][1], 0, 0, 0);
            acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, b0, acc[1][0], 0, 0, 0);
            acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, b1, acc[1][1], 0, 0, 0);
        }
        if (kt + 1 < nk) {  // the other buffer was last read before the previous barrier
            A.store(ra, sa[cur ^ 1]);
            B.store(rb, sb[cur ^ 1]);
        }
        __syncthreads();
    }
}

// row and column of accumulator element r of lane `lane` in the wave's tile (x, y)
__device__ __forceinline__ int f32_row(int x, int r, int lane) { return x * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3); }
__device__ __forceinline__ int f32_col(int y, int lane) { return y * 32 + (lane & 31); }

// Y^T[i][t] = sum_k X[t0+t][k] W[k][i] for the chunk's tokens; block (i tile, t tile)
template <class XT>
__global__ void __launch_bounds__(256) k_gemm_y_f32(const XT *__restrict__ X, int64_t ldx, const XT *__restrict__ W,
                                                    int64_t ldw, int64_t d_in, int64_t d_out, int64_t t0, int64_t tc,
                                                    float *__restrict__ Yt, int64_t ldy) {
    const int64_t i0 = int64_t(blockIdx.x) * FT, tt0 = int64_t(blockIdx.y) * FT;
    const F32Operand<XT, false> A{W + i0, ldw, int(std::min<int64_t>(FT, d_out - i0))};
    const F32Operand<XT, true> B{X + (t0 + tt0) * ldx, ldx, int(std::min<int64_t>(FT, tc - tt0))};
    f32x16_t acc[2][2];
    f32_mainloop(A, B, d_in, acc);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int y = 0; y < 2; ++y) {
            const int64_t t = tt0 + wn + f32_col(y, lane);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t i = i0 + wm + f32_row(x, r, lane);
                if (i < d_out && t < tc) Yt[i * ldy + t] = acc[x][y][r];
            }
        }
}

// Y^T[i][t] = X[t0+t][i] (no W: the covariance of X itself)
template <class XT>
__global__ void __launch_bounds__(256) k_copy_xt(const XT *__restrict__ X, int64_t ldx, int64_t d_out, int64_t t0,
                                                 int64_t tc, float *__restrict__ Yt, int64_t ldy) {
    __shared__ float tile[64][65];
    const int64_t i0 = int64_t(blockIdx.x) * 64, tt0 = int64_t(blockIdx.y) * 64;
    for (int e = threadIdx.x; e < 64 * 64; e += 256) {  // read along i (X rows), write along t
        const int tt = e / 64, ii = e % 64;
        tile[tt][ii] = (i0 + ii < d_out && tt0 + tt < tc) ? ld_as_f32(X, (t0 + tt0 + tt) * ldx + i0 + ii) : 0.f;
    }
    __syncthreads();
    for (int e = threadIdx.x; e < 64 * 64; e += 256) {
        const int ii = e / 64, tt = e % 64;
        if (i0 + ii < d_out && tt0 + tt < tc) Yt[(i0 + ii) * ldy + tt0 + tt] = tile[tt][ii];
    }
}

// C_h[r][c] += sum_t Y^T[h hd + r][t] Y^T[h hd + c][t] for r <= c (upper, incl. diagonal); block
// (I, J, h) with I <= J
__global__ void __launch_bounds__(256) k_syrk_f32(const float *__restrict__ Yt, int64_t ldy, int64_t tc,
                                                  float *__restrict__ C, int64_t ldc, int64_t hd) {
    const int I = blockIdx.x, J = blockIdx.y, h = blockIdx.z;
    if (I > J) return;
    const int64_t r0 = int64_t(I) * FT, c0 = int64_t(J) * FT;
    const float *Yh = Yt + int64_t(h) * hd * ldy;
    const F32Operand<float, true> A{Yh + r0 * ldy, ldy, int(std::min<int64_t>(FT, hd - r0))};
    const F32Operand<float, true> B{Yh + c0 * ldy, ldy, int(std::min<int64_t>(FT, hd - c0))};
    f32x16_t acc[2][2];
    f32_mainloop(A, B, tc, acc);
    float *Ch = C + int64_t(h) * hd * ldc;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int y = 0; y < 2; ++y) {
            const int64_t c = c0 + wn + f32_col(y, lane);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t rr = r0 + wm + f32_row(x, r, lane);
                if (rr < hd && c < hd && rr <= c) Ch[rr * ldc + c] += acc[x][y][r];
            }
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
    if (a.L || use_mfma(a)) {  // the range-projected product has only the MFMA path
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
            if (!a.W) {
                dim3 g0(cdiv(a.d_out, 64), cdiv(tc, 64));
                if (a.x_t == LRC_BF16)
                    hipLaunchKernelGGL(k_copy_xt<bf16_t>, g0, dim3(256), 0, s, static_cast<const bf16_t *>(a.X), a.ldx,
                                       a.d_out, t0, tc, Yt, ldy);
                else
                    hipLaunchKernelGGL(k_copy_xt<float>, g0, dim3(256), 0, s, static_cast<const float *>(a.X), a.ldx,
                                       a.d_out, t0, tc, Yt, ldy);
                LRC_LAUNCH_CHECK("k_copy_xt");
            } else {
                dim3 g1(cdiv(a.d_out, FT), cdiv(tc, FT));
                if (a.x_t == LRC_BF16)
                    hipLaunchKernelGGL(k_gemm_y_f32<bf16_t>, g1, dim3(256), 0, s, static_cast<const bf16_t *>(a.X),
                                       a.ldx, static_cast<const bf16_t *>(a.W), a.ldw, a.d_in, a.d_out, t0, tc, Yt, ldy);
                else
                    hipLaunchKernelGGL(k_gemm_y_f32<float>, g1, dim3(256), 0, s, static_cast<const float *>(a.X), a.ldx,
                                       static_cast<const float *>(a.W), a.ldw, a.d_in, a.d_out, t0, tc, Yt, ldy);
                LRC_LAUNCH_CHECK("k_gemm_y_f32");
            }
            dim3 g2(cdiv(hd, FT), cdiv(hd, FT), a.n_blocks);
            hipLaunchKernelGGL(k_syrk_f32, g2, dim3(256), 0, s, Yt, ldy, tc, a.C, a.ldc, hd);
            LRC_LAUNCH_CHECK("k_syrk_f32");
        }
    }
    hipLaunchKernelGGL(k_cov_check, dim3(1), dim3(256), 0, s, a.C, a.ldc, hd, a.n_blocks, a.info);
    LRC_LAUNCH_CHECK("k_cov_check");
    return LRC_OK;
}

}  // namespace lrc
