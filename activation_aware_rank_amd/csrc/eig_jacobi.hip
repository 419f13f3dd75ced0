// Batched eigendecomposition of small symmetric positive semi-definite matrices (n <= 128),
// one matrix per workgroup, held in LDS in fp64.
//
// Swift-SVD page, section 2-ga: V and Sigma^2 of Y from one eigendecomposition of Y^T Y; the
// per-head case (WSVD page, methodology 1) has one 128 x 128 covariance per attention head.
//
// Method: one-sided (Hestenes) Jacobi on G <- C.  Column pairs (p, q) are rotated so that
// g_p^T g_q = 0; the disjoint pairs of a round (round-robin ordering, n/2 pairs per round,
// n-1 rounds per sweep) are independent.  When every pair of a sweep satisfies
// |g_p^T g_q| <= tol ||g_p|| ||g_q||, G = C V has orthogonal columns, so for PSD C
// G = V diag(lambda): lambda_i = ||g_i|| and v_i = g_i / ||g_i||, and the rotations never need
// to be accumulated into a second matrix.  (For a PSD input the computed lambda_i = ||g_i|| are
// non-negative; eigenvalues at rounding level below zero come out as their magnitude.)
//
// Work layout: a group of 16 lanes owns one pair of a round (64 groups in the 1024 threads, so
// a round of n = 128 is one pass); lane l of a group holds elements l, l + 16, ... of both
// columns in registers, forms its share of the three dot products and the group sums them with
// four DPP steps inside the lane's row of 16 (quad permutes, then the half-row and row mirrors),
// which cost a few cycles each where a wave-wide shuffle through the LDS crossbar waits for every
// step.
#include <cfloat>

#include "lrc_internal.h"

namespace lrc {

constexpr int JAC_THREADS = 1024;
constexpr int JAC_MAX_N = 128;
constexpr int JAC_MAX_SWEEPS = 40;
constexpr int JAC_GROUP = 16;                 // lanes per pair
constexpr int JAC_EL = JAC_MAX_N / JAC_GROUP;  // elements per lane and column

// v moved across the lanes of its row of 16 by the DPP control `ctrl` (both 32-bit halves)
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
    const int lo = __builtin_amdgcn_mov_dpp(__double2loint(v), CTRL, 0xf, 0xf, false);
    const int hi = __builtin_amdgcn_mov_dpp(__double2hiint(v), CTRL, 0xf, 0xf, false);
    return __hiloint2double(hi, lo);
}
// Sum over the 16 lanes of a row.  Every step adds values of lanes paired both ways (a with b and
// b with a), so each step's sum is the same in both lanes and all 16 lanes end with the bit-identical
// total (the group's lanes must agree exactly: each applies the rotation to its own elements).
__device__ __forceinline__ double row16_sum(double v) {
    v += dpp_f64<0xB1>(v);   // quad_perm [1, 0, 3, 2]: lane i with i ^ 1
    v += dpp_f64<0x4E>(v);   // quad_perm [2, 3, 0, 1]: lane i with i ^ 2
    v += dpp_f64<0x141>(v);  // row_half_mirror: quad 0 with quad 1, quad 2 with quad 3
    v += dpp_f64<0x140>(v);  // row_mirror: the two halves of the row
    return v;
}

template <class T>
__device__ __forceinline__ T wave_sum(T v) {
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

template <class T>
__global__ void __launch_bounds__(JAC_THREADS) k_jacobi(const float *__restrict__ C, int n, int64_t ldc, int64_t stride_c,
                                                        double *__restrict__ lambda, float *__restrict__ V, int64_t ldv,
                                                        int n_vec, int64_t stride_v, int32_t *__restrict__ info) {
    extern __shared__ __attribute__((aligned(16))) char smem[];
    T *G = reinterpret_cast<T *>(smem);            // column-major: column p at G + p * n
    T *nrm = G + n * n;                            // column norms
    int *rank = reinterpret_cast<int *>(nrm + n);  // output position of column i
    __shared__ int s_flag, s_bad;
    const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nwaves = JAC_THREADS / 64;
    const float *Cb = C + int64_t(b) * stride_c;
    if (tid == 0) s_bad = 0;
    __syncthreads();
    for (int e = tid; e < n * n; e += JAC_THREADS) {
        const int p = e / n, i = e % n;  // G[p][i] = C(i, p), upper triangle read
        const float v = i <= p ? Cb[int64_t(i) * ldc + p] : Cb[int64_t(p) * ldc + i];
        if (!isfinite(v)) s_bad = 1;
        G[e] = T(v);
    }
    __syncthreads();
    const bool bad = s_bad != 0;
    const int m = n + (n & 1), np = m / 2;
    const T tol = T(n) * DBL_EPSILON, tol2 = tol * tol;
    const int grp = tid / JAC_GROUP, gl = tid % JAC_GROUP;
    const int ngrp = JAC_THREADS / JAC_GROUP;
    int converged = bad ? 1 : 0;
    for (int sweep = 0; sweep < JAC_MAX_SWEEPS && !converged; ++sweep) {
        if (tid == 0) s_flag = 0;
        __syncthreads();
        for (int r = 0; r < m - 1; ++r) {
            for (int pi = grp; pi < np; pi += ngrp) {
                int p, q;
                if (pi == 0) { p = r; q = m - 1; }
                else { p = (r + pi) % (m - 1); q = (r - pi + (m - 1)) % (m - 1); }
                if (p > q) { const int t = p; p = q; q = t; }
                if (q >= n) continue;  // dummy player (odd n): the whole group skips together
                T *gp = G + p * n, *gq = G + q * n;
                T x[JAC_EL], y[JAC_EL];
                T al = T(0), be = T(0), ga = T(0);
#pragma unroll
                for (int e = 0; e < JAC_EL; ++e) {
                    const int i = gl + JAC_GROUP * e;
                    x[e] = i < n ? gp[i] : T(0);
                    y[e] = i < n ? gq[i] : T(0);
                    al += x[e] * x[e];
                    be += y[e] * y[e];
                    ga += x[e] * y[e];
                }
                al = row16_sum(al);
                be = row16_sum(be);
                ga = row16_sum(ga);
                // |ga| > tol ||g_p|| ||g_q||, squared (no square roots on the test that decides
                // most pairs of the late sweeps; the squares stay far inside the fp64 range)
                if (ga != T(0) && ga * ga > tol2 * (al * be)) {
                    const T zeta = (be - al) / (T(2) * ga);
                    const T sg = zeta >= T(0) ? T(1) : T(-1);
                    const T t = sg / (fabs(zeta) + sqrt(T(1) + zeta * zeta));
                    const T c = T(1) / sqrt(T(1) + t * t), sn = c * t;
#pragma unroll
                    for (int e = 0; e < JAC_EL; ++e) {
                        const int i = gl + JAC_GROUP * e;
                        if (i < n) {
                            gp[i] = c * x[e] - sn * y[e];
                            gq[i] = sn * x[e] + c * y[e];
                        }
                    }
                    if (gl == 0) s_flag = 1;
                }
            }
            __syncthreads();
        }
        converged = s_flag == 0;
        __syncthreads();
    }
    // norms, ranks (descending, ties by index), outputs
    for (int i = wave; i < n; i += nwaves) {
        const T x0 = lane < n ? G[i * n + lane] : T(0), x1 = lane + 64 < n ? G[i * n + lane + 64] : T(0);
        const T s2 = wave_sum(x0 * x0 + x1 * x1);
        if (lane == 0) nrm[i] = sqrt(s2);
    }
    __syncthreads();
    for (int i = tid; i < n; i += JAC_THREADS) {
        const T ni = nrm[i];
        int rk = 0;
        for (int j = 0; j < n; ++j) rk += (nrm[j] > ni) || (nrm[j] == ni && j < i);
        rank[i] = rk;
        lambda[int64_t(b) * n + rk] = bad ? double(NAN) : double(ni);
    }
    __syncthreads();
    for (int i = wave; i < n; i += nwaves) {
        const int j = rank[i];
        if (j >= n_vec) continue;
        const T ni = nrm[i];
        const T inv = ni > T(0) ? T(1) / ni : T(0);
        // sign: entry of largest magnitude positive, first index on ties
        T best = T(-1);
        int bi = n;
        for (int k = lane; k < n; k += 64) {
            const T a = fabs(G[i * n + k]);
            if (a > best) { best = a; bi = k; }
        }
        for (int o = 32; o > 0; o >>= 1) {
            const T ob = __shfl_xor(best, o);
            const int oi = __shfl_xor(bi, o);
            if (ob > best || (ob == best && oi < bi)) { best = ob; bi = oi; }
        }
        const T sgn = (bi < n && G[i * n + bi] < T(0)) ? T(-1) : T(1);
        float *Vb = V + int64_t(b) * stride_v;
        for (int k = lane; k < n; k += 64) {
            T v = ni > T(0) ? G[i * n + k] * inv * sgn : (k == i ? T(1) : T(0));
            Vb[int64_t(k) * ldv + j] = float(v);
        }
    }
    if (tid == 0) info[b] = bad ? LRC_INFO_NONFINITE : (converged ? LRC_INFO_OK : LRC_INFO_NO_CONVERGENCE);
}

template <class T>
static size_t jac_smem(int64_t n) {
    return size_t(n) * size_t(n) * sizeof(T) + size_t(n) * sizeof(T) + size_t(n) * sizeof(int) + 16;
}

size_t jacobi_workspace(int64_t, int64_t, lrc_dtype) { return 0; }

lrc_status jacobi_run(const EighArgs &a, void *, size_t, hipStream_t s) {
    if (a.n > JAC_MAX_N) return fail(LRC_ERR_ARG, "jacobi path needs n <= 128");
    if (a.batch > 65535 * 64) return fail(LRC_ERR_ARG, "batch too large");
    // Always fp64, whatever the requested working precision: a 128 x 128 fp64 matrix (128 KiB)
    // fits in LDS, and fp32 sweeps stop at a pair tolerance (n FLT_EPSILON) that leaves retained
    // subspaces of the per-head matrices only a few times inside 1e-3 rad.
    const size_t sm = jac_smem<double>(a.n);
    LRC_HIP(hipFuncSetAttribute(reinterpret_cast<const void *>(k_jacobi<double>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, int(sm)));
    hipLaunchKernelGGL(k_jacobi<double>, dim3(unsigned(a.batch)), dim3(JAC_THREADS), sm, s, a.C, int(a.n), a.ldc,
                       a.stride_c, a.lambda, a.V, a.ldv, int(a.n_vec), a.stride_v, a.info);
    LRC_LAUNCH_CHECK("k_jacobi");
    return LRC_OK;
}

}  // namespace lrc
