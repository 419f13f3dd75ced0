// Factor projection of the closed-form truncation (Swift-SVD page, section 2-ga:
// W_k = (W V_k) V_k^T): A = W V[:, :k] (or W^T V[:, :k]) and B = V[:, :k]^T.
// Products and sums in fp64 (inputs widened exactly), A rounded once to fp32.
#include "lrc_internal.h"

namespace lrc {

constexpr int FT = 64;        // output tile (4 waves of 32 x 32)
constexpr int FK = 16;        // contraction step
constexpr int FLD = FT + 16;  // padded LDS row (doubles)

template <class WT>
__device__ __forceinline__ double wload(const WT *p, int64_t i);
template <>
__device__ __forceinline__ double wload<bf16_t>(const bf16_t *p, int64_t i) { return double(bf16_to_f32(p[i])); }
template <>
__device__ __forceinline__ double wload<float>(const float *p, int64_t i) { return double(p[i]); }
template <>
__device__ __forceinline__ double wload<double>(const double *p, int64_t i) { return p[i]; }

// A[i][j] = sum_r Wop[i][r] V[r][j]; Wop = W (TRANS 0: i < d_in, r < d_out) or W^T (TRANS 1).
// Both operands are widened exactly to fp64 while staged in LDS (k-major), the next step's values
// are loaded while the current one is multiplied, and the products run on 16x16x4 fp64 MFMA.
template <class WT, int TRANS>
__global__ void __launch_bounds__(256) k_factor_gemm(const WT *__restrict__ W, int64_t ldw, int64_t d_in, int64_t d_out,
                                                     const float *__restrict__ V, int64_t ldv, int64_t k,
                                                     float *__restrict__ A, int64_t lda, int64_t stride_w,
                                                     int64_t stride_v, int64_t stride_a) {
    __shared__ double Ws[FK][FLD];
    __shared__ double Vs[FK][FLD];
    const int64_t b = blockIdx.z;
    W += b * stride_w;
    V += b * stride_v;
    A += b * stride_a;
    const int64_t M = TRANS ? d_out : d_in;  // rows of A
    const int64_t R = TRANS ? d_in : d_out;  // contraction length
    const int64_t i0 = int64_t(blockIdx.y) * FT, j0 = int64_t(blockIdx.x) * FT;
    const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
    const int wr = (wv >> 1) * 32, wc = (wv & 1) * 32;
    // each thread stages 4 values of each operand per step: W along its contiguous axis, V along j
    double ra[4], rb[4];
    auto gload = [&](int64_t r0) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            if (TRANS) {  // W[r][i], contiguous in i
                const int rr = t >> 4, ii = (t & 15) * 4 + u;
                const int64_t r = r0 + rr, i = i0 + ii;
                ra[u] = (r < R && i < M) ? wload(W, r * ldw + i) : 0.0;
            } else {      // W[i][r], contiguous in r
                const int ii = t >> 2, rr = (t & 3) * 4 + u;
                const int64_t r = r0 + rr, i = i0 + ii;
                ra[u] = (r < R && i < M) ? wload(W, i * ldw + r) : 0.0;
            }
            const int vr = t >> 4, vj = (t & 15) * 4 + u;
            const int64_t rv = r0 + vr, jj = j0 + vj;
            rb[u] = (rv < R && jj < k) ? double(V[rv * ldv + jj]) : 0.0;
        }
    };
    auto sstore = [&]() {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            if (TRANS) Ws[t >> 4][(t & 15) * 4 + u] = ra[u];
            else Ws[(t & 3) * 4 + u][t >> 2] = ra[u];
            Vs[t >> 4][(t & 15) * 4 + u] = rb[u];
        }
    };
    f64x4_t acc[2][2];
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int y = 0; y < 2; ++y) acc[x][y] = f64x4_t{0.0, 0.0, 0.0, 0.0};
    gload(0);
    for (int64_t r0 = 0; r0 < R; r0 += FK) {
        sstore();
        __syncthreads();
        if (r0 + FK < R) gload(r0 + FK);
#pragma unroll
        for (int ks = 0; ks < FK / 4; ++ks) {
            // 16x16x4 f64 MFMA operands: lane i + 16 kq holds row (or column) i of k-slice kq
            const int kk = ks * 4 + (lane >> 4);
            const double a0 = Ws[kk][wr + (lane & 15)];
            const double a1 = Ws[kk][wr + 16 + (lane & 15)];
            const double b0 = Vs[kk][wc + (lane & 15)];
            const double b1 = Vs[kk][wc + 16 + (lane & 15)];
            acc[0][0] = __builtin_amdgcn_mfma_f64_16x16x4f64(a0, b0, acc[0][0], 0, 0, 0);
            acc[0][1] = __builtin_amdgcn_mfma_f64_16x16x4f64(a0, b1, acc[0][1], 0, 0, 0);
            acc[1][0] = __builtin_amdgcn_mfma_f64_16x16x4f64(a1, b0, acc[1][0], 0, 0, 0);
            acc[1][1] = __builtin_amdgcn_mfma_f64_16x16x4f64(a1, b1, acc[1][1], 0, 0, 0);
        }
        __syncthreads();
    }
    // accumulator r of a lane holds row 4 r + lane / 16, column lane % 16 of its 16x16 tile
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int y = 0; y < 2; ++y)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t i = i0 + wr + x * 16 + r * 4 + (lane >> 4);
                const int64_t j = j0 + wc + y * 16 + (lane & 15);
                if (i < M && j < k) A[i * lda + j] = float(acc[x][y][r]);
            }
}

// B[q][r] = V[r][q], q < k, r < rows
__global__ void __launch_bounds__(256) k_factor_bt(const float *__restrict__ V, int64_t ldv, int64_t rows, int64_t k,
                                                   float *__restrict__ B, int64_t ldb, int64_t stride_v, int64_t stride_b) {
    __shared__ float tile[64][65];
    const int64_t b = blockIdx.z;
    V += b * stride_v;
    B += b * stride_b;
    const int64_t r0 = int64_t(blockIdx.y) * 64, q0 = int64_t(blockIdx.x) * 64;
    for (int e = threadIdx.x; e < 64 * 64; e += 256) {
        const int rr = e / 64, qq = e % 64;
        if (r0 + rr < rows && q0 + qq < k) tile[rr][qq] = V[(r0 + rr) * ldv + q0 + qq];
    }
    __syncthreads();
    for (int e = threadIdx.x; e < 64 * 64; e += 256) {
        const int qq = e / 64, rr = e % 64;
        if (r0 + rr < rows && q0 + qq < k) B[(q0 + qq) * ldb + r0 + rr] = tile[rr][qq];
    }
}

template <class WT>
static void launch_gemm(const FactorizeArgs &a, hipStream_t s) {
    const int64_t M = a.trans_w ? a.d_out : a.d_in;
    dim3 g(cdiv(a.k, FT), cdiv(M, FT), unsigned(a.batch));
    const WT *W = static_cast<const WT *>(a.W);
    if (a.trans_w)
        hipLaunchKernelGGL((k_factor_gemm<WT, 1>), g, dim3(256), 0, s, W, a.ldw, a.d_in, a.d_out, a.V, a.ldv, a.k, a.A,
                           a.lda, a.stride_w, a.stride_v, a.stride_a);
    else
        hipLaunchKernelGGL((k_factor_gemm<WT, 0>), g, dim3(256), 0, s, W, a.ldw, a.d_in, a.d_out, a.V, a.ldv, a.k, a.A,
                           a.lda, a.stride_w, a.stride_v, a.stride_a);
}

lrc_status factorize_run(const FactorizeArgs &a, hipStream_t s) {
    if (a.batch > 65535) return fail(LRC_ERR_ARG, "batch too large");
    if (a.A) {
        switch (a.w_t) {
            case LRC_BF16: launch_gemm<bf16_t>(a, s); break;
            case LRC_F32: launch_gemm<float>(a, s); break;
            case LRC_F64: launch_gemm<double>(a, s); break;
        }
        LRC_LAUNCH_CHECK("k_factor_gemm");
    }
    if (a.B) {
        const int64_t rows = a.trans_w ? a.d_in : a.d_out;
        dim3 g(cdiv(a.k, 64), cdiv(rows, 64), unsigned(a.batch));
        hipLaunchKernelGGL(k_factor_bt, g, dim3(256), 0, s, a.V, a.ldv, rows, a.k, a.B, a.ldb, a.stride_v, a.stride_b);
        LRC_LAUNCH_CHECK("k_factor_bt");
    }
    return LRC_OK;
}

}  // namespace lrc
