// Factor projection of the closed-form truncation (Swift-SVD page, section 2-ga:
// W_k = (W V_k) V_k^T): A = W V[:, :k] (or W^T V[:, :k]) and B = V[:, :k]^T.
// Products and sums in fp64 (inputs widened exactly), A rounded once to fp32.
#include "lrc_internal.h"

namespace lrc {

constexpr int FK = 16;  // contraction step

template <class WT>
__device__ __forceinline__ double wload(const WT *p, int64_t i);
template <>
__device__ __forceinline__ double wload<bf16_t>(const bf16_t *p, int64_t i) { return double(bf16_to_f32(p[i])); }
template <>
__device__ __forceinline__ double wload<float>(const float *p, int64_t i) { return double(p[i]); }
template <>
__device__ __forceinline__ double wload<double>(const double *p, int64_t i) { return p[i]; }

// Four consecutive elements from a 4-element-aligned address, widened exactly to fp64.
template <class WT>
__device__ __forceinline__ void wload4(const WT *p, double (&o)[4]);
template <>
__device__ __forceinline__ void wload4<bf16_t>(const bf16_t *p, double (&o)[4]) {
    const uint2 v = *reinterpret_cast<const uint2 *>(p);
    o[0] = double(__uint_as_float(v.x << 16));
    o[1] = double(__uint_as_float(v.x & 0xffff0000u));
    o[2] = double(__uint_as_float(v.y << 16));
    o[3] = double(__uint_as_float(v.y & 0xffff0000u));
}
template <>
__device__ __forceinline__ void wload4<float>(const float *p, double (&o)[4]) {
    const float4 v = *reinterpret_cast<const float4 *>(p);
    o[0] = double(v.x);
    o[1] = double(v.y);
    o[2] = double(v.z);
    o[3] = double(v.w);
}
template <>
__device__ __forceinline__ void wload4<double>(const double *p, double (&o)[4]) {
    const double2 a = *reinterpret_cast<const double2 *>(p), b = *reinterpret_cast<const double2 *>(p + 2);
    o[0] = a.x;
    o[1] = a.y;
    o[2] = b.x;
    o[3] = b.y;
}

// A[i][j] = sum_r Wop[i][r] V[r][j]; Wop = W (TRANS 0: i < d_in, r < d_out) or W^T (TRANS 1).
// Both operands are widened exactly to fp64 while staged in LDS (k-major), the next step's values
// are loaded while the current one is multiplied, and the products run on 16x16x4 fp64 MFMA.
// BT: output tile edge, 64 (4 waves of 32 x 32) or 128 (4 waves of 64 x 64, two workgroups to a CU:
// half the operand traffic per flop, for products with enough tiles to fill the GPU).  VEC: every
// row of W and V starts 4-element aligned, so each thread's four consecutive values of an operand
// come in one vector load where all four are in range.
template <class WT, int TRANS, int BT, bool VEC>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(BT == 128 ? 2 : 1)))
k_factor_gemm(const WT *__restrict__ W, int64_t ldw, int64_t d_in, int64_t d_out, const float *__restrict__ V,
              int64_t ldv, int64_t k, float *__restrict__ A, int64_t lda, int64_t stride_w, int64_t stride_v,
              int64_t stride_a) {
    constexpr int NF = BT / 32;  // MFMA tiles per wave and dimension
    constexpr int NU = BT / 64;  // 64-row passes of the operand loads
    constexpr int LD = BT + 16;  // padded LDS row (doubles)
    __shared__ double Ws[FK][LD];
    __shared__ double Vs[FK][LD];
    const int64_t b = blockIdx.z;
    W += b * stride_w;
    V += b * stride_v;
    A += b * stride_a;
    const int64_t M = TRANS ? d_out : d_in;  // rows of A
    const int64_t R = TRANS ? d_in : d_out;  // contraction length
    const int64_t i0 = int64_t(blockIdx.y) * BT, j0 = int64_t(blockIdx.x) * BT;
    const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
    const int wr = (wv >> 1) * (BT / 2), wc = (wv & 1) * (BT / 2);
    // each thread stages 4 NU values of each operand per step: W along its contiguous axis, V along j
    double ra[4 * NU], rb[4 * NU];
    auto gload = [&](int64_t r0) {
        if (VEC) {
#pragma unroll
            for (int q = 0; q < NU; ++q) {
                double w4[4], v4[4];
                if (TRANS) {  // W[r][i .. i+3]
                    const int64_t r = r0 + (t >> 4), i = i0 + (t & 15) * 4 + 64 * q;
                    if (r < R && i + 3 < M) {
                        wload4(W + r * ldw + i, w4);
                    } else {
#pragma unroll
                        for (int u = 0; u < 4; ++u) w4[u] = (r < R && i + u < M) ? wload(W, r * ldw + i + u) : 0.0;
                    }
                } else {      // W[i][r .. r+3]
                    const int64_t i = i0 + (t >> 2) + 64 * q, r = r0 + (t & 3) * 4;
                    if (i < M && r + 3 < R) {
                        wload4(W + i * ldw + r, w4);
                    } else {
#pragma unroll
                        for (int u = 0; u < 4; ++u) w4[u] = (i < M && r + u < R) ? wload(W, i * ldw + r + u) : 0.0;
                    }
                }
                const int64_t rv = r0 + (t >> 4), jj = j0 + (t & 15) * 4 + 64 * q;
                if (rv < R && jj + 3 < k) {
                    wload4(V + rv * ldv + jj, v4);
                } else {
#pragma unroll
                    for (int u = 0; u < 4; ++u) v4[u] = (rv < R && jj + u < k) ? double(V[rv * ldv + jj + u]) : 0.0;
                }
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    ra[4 * q + u] = w4[u];
                    rb[4 * q + u] = v4[u];
                }
            }
            return;
        }
#pragma unroll
        for (int q = 0; q < NU; ++q)
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                if (TRANS) {  // W[r][i], contiguous in i
                    const int rr = t >> 4, ii = (t & 15) * 4 + 64 * q + u;
                    const int64_t r = r0 + rr, i = i0 + ii;
                    ra[4 * q + u] = (r < R && i < M) ? wload(W, r * ldw + i) : 0.0;
                } else {      // W[i][r], contiguous in r
                    const int ii = (t >> 2) + 64 * q, rr = (t & 3) * 4 + u;
                    const int64_t r = r0 + rr, i = i0 + ii;
                    ra[4 * q + u] = (r < R && i < M) ? wload(W, i * ldw + r) : 0.0;
                }
                const int vr = t >> 4, vj = (t & 15) * 4 + 64 * q + u;
                const int64_t rv = r0 + vr, jj = j0 + vj;
                rb[4 * q + u] = (rv < R && jj < k) ? double(V[rv * ldv + jj]) : 0.0;
            }
    };
    auto sstore = [&]() {
#pragma unroll
        for (int q = 0; q < NU; ++q)
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                if (TRANS) Ws[t >> 4][(t & 15) * 4 + 64 * q + u] = ra[4 * q + u];
                else Ws[(t & 3) * 4 + u][(t >> 2) + 64 * q] = ra[4 * q + u];
                Vs[t >> 4][(t & 15) * 4 + 64 * q + u] = rb[4 * q + u];
            }
    };
    f64x4_t acc[NF][NF];
#pragma unroll
    for (int x = 0; x < NF; ++x)
#pragma unroll
        for (int y = 0; y < NF; ++y) acc[x][y] = f64x4_t{0.0, 0.0, 0.0, 0.0};
    gload(0);
    for (int64_t r0 = 0; r0 < R; r0 += FK) {
        sstore();
        __syncthreads();
        if (r0 + FK < R) gload(r0 + FK);
#pragma unroll
        for (int ks = 0; ks < FK / 4; ++ks) {
            // 16x16x4 f64 MFMA operands: lane i + 16 kq holds row (or column) i of k-slice kq
            const int kk = ks * 4 + (lane >> 4);
            double av[NF], bv[NF];
#pragma unroll
            for (int x = 0; x < NF; ++x) {
                av[x] = Ws[kk][wr + x * 16 + (lane & 15)];
                bv[x] = Vs[kk][wc + x * 16 + (lane & 15)];
            }
#pragma unroll
            for (int x = 0; x < NF; ++x)
#pragma unroll
                for (int y = 0; y < NF; ++y)
                    acc[x][y] = __builtin_amdgcn_mfma_f64_16x16x4f64(av[x], bv[y], acc[x][y], 0, 0, 0);
        }
        __syncthreads();
    }
    // accumulator r of a lane holds row 4 r + lane / 16, column lane % 16 of its 16x16 tile
#pragma unroll
    for (int x = 0; x < NF; ++x)
#pragma unroll
        for (int y = 0; y < NF; ++y)
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

// every row (and batch member) of a matrix starts on a multiple of `bytes`
static bool aligned_rows(const void *p, size_t bytes, int64_t ld, int64_t stride) {
    const size_t el = bytes / 4;  // element size: the alignment is four elements
    return reinterpret_cast<uintptr_t>(p) % bytes == 0 && (size_t(ld) * el) % bytes == 0 &&
           (size_t(stride) * el) % bytes == 0;
}

template <class WT, int TRANS, int BT>
static void launch_tiles(const FactorizeArgs &a, int64_t M, hipStream_t s) {
    const dim3 g(cdiv(a.k, BT), cdiv(M, BT), unsigned(a.batch));
    const double flops = 2.0 * double(M) * double(a.k) * double(a.trans_w ? a.d_in : a.d_out) * double(a.batch);
    const bool vec = aligned_rows(a.W, 4 * sizeof(WT), a.ldw, a.stride_w) &&
                     aligned_rows(a.V, 4 * sizeof(float), a.ldv, a.stride_v);
    if (vec)
        LRC_TIMED_LAUNCH("k_factor_gemm", flops, (k_factor_gemm<WT, TRANS, BT, true>), g, dim3(256), 0, s,
                         static_cast<const WT *>(a.W), a.ldw, a.d_in, a.d_out, a.V, a.ldv, a.k, a.A, a.lda, a.stride_w,
                         a.stride_v, a.stride_a);
    else
        LRC_TIMED_LAUNCH("k_factor_gemm", flops, (k_factor_gemm<WT, TRANS, BT, false>), g, dim3(256), 0, s,
                         static_cast<const WT *>(a.W), a.ldw, a.d_in, a.d_out, a.V, a.ldv, a.k, a.A, a.lda, a.stride_w,
                         a.stride_v, a.stride_a);
}

// 128 x 128 tiles when there are at least 512 of them (two workgroups on every CU) and the
// contraction is long, else 64 x 64
template <class WT>
static void launch_gemm(const FactorizeArgs &a, hipStream_t s) {
    const int64_t M = a.trans_w ? a.d_out : a.d_in, R = a.trans_w ? a.d_in : a.d_out;
    const bool big = int64_t(cdiv(a.k, 128)) * cdiv(M, 128) * a.batch >= 512 && R >= 512;
    if (a.trans_w) {
        if (big) launch_tiles<WT, 1, 128>(a, M, s);
        else launch_tiles<WT, 1, 64>(a, M, s);
    } else {
        if (big) launch_tiles<WT, 0, 128>(a, M, s);
        else launch_tiles<WT, 0, 64>(a, M, s);
    }
}

lrc_status factorize_run(const FactorizeArgs &a, hipStream_t s) {
    if (a.batch > 65535) return fail(LRC_ERR_ARG, "batch too large");
    if (cdiv(a.trans_w ? a.d_out : a.d_in, 64) > 65535) return fail(LRC_ERR_ARG, "A has too many rows");
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
