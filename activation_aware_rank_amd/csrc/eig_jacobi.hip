// Batched eigendecomposition of small symmetric positive semi-definite matrices (n <= 128),
// one matrix per workgroup, held in LDS.
//
// Swift-SVD page, section 2-ga: V and Sigma^2 of Y from one eigendecomposition of Y^T Y; the
// per-head case (WSVD page, methodology 1) has one 128 x 128 covariance per attention head.
//
// Method: one-sided (Hestenes) Jacobi on G <- C.  Column pairs (p, q) are rotated so that
// g_p^T g_q = 0; the disjoint pairs of a round (round-robin ordering, n/2 pairs per round,
// n-1 rounds per sweep) are independent and run on different wavefronts, each dot product a
// wave64 shuffle reduction.  When every pair of a sweep satisfies
// |g_p^T g_q| <= tol ||g_p|| ||g_q||, G = C V has orthogonal columns, so for PSD C
// G = V diag(lambda): lambda_i = ||g_i|| and v_i = g_i / ||g_i||, and the rotations never need
// to be accumulated into a second matrix.  (For a PSD input the computed lambda_i = ||g_i|| are
// non-negative; eigenvalues at rounding level below zero come out as their magnitude.)
#include <cfloat>

#include "lrc_internal.h"

namespace lrc {

constexpr int JAC_THREADS = 512;
constexpr int JAC_MAX_N = 128;
constexpr int JAC_MAX_SWEEPS = 40;

template <class T>
__device__ __forceinline__ T wave_sum(T v) {
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

template <class T>
__device__ __forceinline__ T eps_of();
template <>
__device__ __forceinline__ double eps_of<double>() { return DBL_EPSILON; }

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
    const T tol = T(n) * eps_of<T>();
    int converged = bad ? 1 : 0;
    for (int sweep = 0; sweep < JAC_MAX_SWEEPS && !converged; ++sweep) {
        if (tid == 0) s_flag = 0;
        __syncthreads();
        for (int r = 0; r < m - 1; ++r) {
            for (int pi = wave; pi < np; pi += nwaves) {
                int p, q;
                if (pi == 0) { p = r; q = m - 1; }
                else { p = (r + pi) % (m - 1); q = (r - pi + (m - 1)) % (m - 1); }
                if (p > q) { const int t = p; p = q; q = t; }
                if (q >= n) continue;  // dummy player (odd n)
                T *gp = G + p * n, *gq = G + q * n;
                const T x0 = lane < n ? gp[lane] : T(0), y0 = lane < n ? gq[lane] : T(0);
                const T x1 = lane + 64 < n ? gp[lane + 64] : T(0), y1 = lane + 64 < n ? gq[lane + 64] : T(0);
                const T al = wave_sum(x0 * x0 + x1 * x1);
                const T be = wave_sum(y0 * y0 + y1 * y1);
                const T ga = wave_sum(x0 * y0 + x1 * y1);
                if (ga != T(0) && fabs(ga) > tol * sqrt(al) * sqrt(be)) {
                    const T zeta = (be - al) / (T(2) * ga);
                    const T sg = zeta >= T(0) ? T(1) : T(-1);
                    const T t = sg / (fabs(zeta) + sqrt(T(1) + zeta * zeta));
                    const T c = T(1) / sqrt(T(1) + t * t), s = c * t;
                    if (lane < n) { gp[lane] = c * x0 - s * y0; gq[lane] = s * x0 + c * y0; }
                    if (lane + 64 < n) { gp[lane + 64] = c * x1 - s * y1; gq[lane + 64] = s * x1 + c * y1; }
                    if (lane == 0) s_flag = 1;
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
