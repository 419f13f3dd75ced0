// Symmetric eigendecomposition for n > 128 (Swift-SVD page, section 2-ga: one eigendecomposition
// of Y^T Y yields V and Sigma^2 of Y).
//
// Stages, all on the GPU:
//  1. Householder tridiagonalisation Q^T C Q = T, blocked (panel of NB columns, then a rank-2NB
//     update of the trailing matrix), working precision T_ (fp32 or fp64).  The matrix is kept
//     in full (both triangles) so the symmetric matrix-vector product of each column is a plain
//     row-wise product with coalesced rows.
//  2. All n eigenvalues of T by bisection on Sturm counts, fp64, one thread per eigenvalue.
//  3. Eigenvectors of T for the n_vec largest eigenvalues by inverse iteration, fp64, one thread
//     per vector (LU with partial pivoting of T - lambda I, recomputed each iteration); vectors of
//     eigenvalues closer than a cluster tolerance are re-orthogonalised by modified Gram-Schmidt.
//  4. Back-transformation V = Q Z with the reflectors grouped in blocks of NBT,
//     Q_b = I - V_b T_b V_b^T (compact WY), applied from the last block to the first, in fp64.
//  5. Each column's entry of largest magnitude made positive.
// Reflector c is H_c = I - tau_c v_c v_c^T with v_c[c+1] = 1 and v_c[r] = 0 for r <= c.
#include <cfloat>
#include <cmath>

#include "lrc_internal.h"

namespace lrc {

constexpr int NB = 32;    // tridiagonalisation panel width
constexpr int NBT = 32;   // back-transformation block of reflectors
constexpr int RCH = 512;  // rows per partial in the back-transformation reductions
constexpr int SYMV_ROWS = 16;  // rows per block in the symmetric product

// ---------------------------------------------------------------------------------------------
// 1. tridiagonalisation
// ---------------------------------------------------------------------------------------------
template <class T>
__global__ void k_fill_full(const float *__restrict__ C, int64_t ldc, int64_t n, T *__restrict__ A, int64_t lda,
                            int *__restrict__ bad) {
    const int64_t total = n * n;
    for (int64_t e = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; e < total; e += int64_t(gridDim.x) * blockDim.x) {
        const int64_t i = e / n, j = e % n;
        const float v = i <= j ? C[i * ldc + j] : C[j * ldc + i];
        if (!isfinite(v)) atomicOr(bad, 1);
        A[i * lda + j] = T(v);
    }
}

template <class T>
__global__ void k_fill_zero(T *__restrict__ p, int64_t n) {
    for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += int64_t(gridDim.x) * blockDim.x)
        p[i] = T(0);
}

template <class T>
__device__ __forceinline__ T block_sum(T v, T *sh) {
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    __syncthreads();
    if (lane == 0) sh[wid] = v;
    __syncthreads();
    T r = T(0);
    for (int i = 0; i < int(blockDim.x >> 6); ++i) r += sh[i];
    __syncthreads();
    return r;  // every thread
}

// A[r][c] -= sum_{q<j} V[r][q] W[c][q] + W[r][q] V[c][q] for r in [c, n); partial sum of squares of
// rows r >= c+2 (the part of the column below the reflector's leading entry)
template <class T>
__global__ void __launch_bounds__(256) k_col_update(T *__restrict__ A, int64_t lda, int64_t n, int64_t c, int j,
                                                    const T *__restrict__ Vp, const T *__restrict__ Wp,
                                                    T *__restrict__ part) {
    __shared__ T sh[4];
    __shared__ T vc[NB], wc[NB];
    if (threadIdx.x < j) {
        vc[threadIdx.x] = Vp[c * NB + threadIdx.x];
        wc[threadIdx.x] = Wp[c * NB + threadIdx.x];
    }
    __syncthreads();
    const int64_t r = c + int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    T ss = T(0);
    if (r < n) {
        T a = A[r * lda + c];
        for (int q = 0; q < j; ++q) a -= Vp[r * NB + q] * wc[q] + Wp[r * NB + q] * vc[q];
        A[r * lda + c] = a;
        if (r >= c + 2) ss = a * a;
    }
    ss = block_sum(ss, sh);
    if (threadIdx.x == 0) part[blockIdx.x] = ss;
}

// One block: the reflector of column c from the updated column, and its vector v (v[c+1] = 1).
template <class T>
__global__ void __launch_bounds__(1024) k_householder(T *__restrict__ A, int64_t lda, int64_t n, int64_t c,
                                                      const T *__restrict__ part, int npart, T *__restrict__ vbuf,
                                                      T *__restrict__ Rt, int64_t ldr, T *__restrict__ tau,
                                                      double *__restrict__ d, double *__restrict__ e, T *__restrict__ scal) {
    __shared__ T sh[16];
    __shared__ T s_scale;
    T acc = T(0);
    if (threadIdx.x == 0)
        for (int i = 0; i < npart; ++i) acc += part[i];  // fixed order
    if (threadIdx.x == 0) {
        const T sigma2 = acc;
        const T alpha = A[(c + 1) * lda + c];
        T beta, tv, scale;
        if (sigma2 == T(0)) {
            tv = T(0);
            beta = alpha;
            scale = T(0);
        } else {
            const T nrm = sqrt(alpha * alpha + sigma2);
            beta = alpha >= T(0) ? -nrm : nrm;
            tv = (beta - alpha) / beta;
            scale = T(1) / (alpha - beta);
        }
        d[c] = double(A[c * lda + c]);
        e[c] = double(beta);
        tau[c] = tv;
        scal[0] = tv;
        s_scale = scale;
    }
    __syncthreads();
    const T scale = s_scale;
    for (int64_t r = threadIdx.x; r < n; r += blockDim.x) {
        T v;
        if (r <= c) v = T(0);
        else if (r == c + 1) v = T(1);
        else v = A[r * lda + c] * scale;
        if (r > c) vbuf[r] = v;
        Rt[c * ldr + r] = v;
    }
}

// w_raw[r] = sum_{k > c} A[r][k] v[k] for rows r in [c+1, n), SYMV_ROWS rows per block (one wave
// per row at a time); block partials of q1 = W^T v and q2 = V^T v over the block's rows.
template <class T>
__global__ void __launch_bounds__(256) k_symv(const T *__restrict__ A, int64_t lda, int64_t n, int64_t c,
                                              const T *__restrict__ vbuf, T *__restrict__ wbuf, const T *__restrict__ Vp,
                                              const T *__restrict__ Wp, int j, T *__restrict__ qpart) {
    extern __shared__ __attribute__((aligned(16))) char smem_raw[];
    T *vs = reinterpret_cast<T *>(smem_raw);  // v[c+1 .. n)
    const int64_t m = n - c - 1;
    for (int64_t k = threadIdx.x; k < m; k += blockDim.x) vs[k] = vbuf[c + 1 + k];
    __syncthreads();
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t rbase = c + 1 + int64_t(blockIdx.x) * SYMV_ROWS;
    for (int rr = wave; rr < SYMV_ROWS; rr += 4) {
        const int64_t r = rbase + rr;
        if (r >= n) break;
        const T *row = A + r * lda + c + 1;
        T acc = T(0);
        for (int64_t k = lane; k < m; k += 64) acc += row[k] * vs[k];
        for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
        if (lane == 0) wbuf[r] = acc;
    }
    // q partials: thread q (< 2j) sums over the block's rows
    const int t = threadIdx.x;
    if (t < 2 * j) {
        const int q = t % j;
        const T *src = t < j ? Wp : Vp;
        T acc = T(0);
        for (int rr = 0; rr < SYMV_ROWS; ++rr) {
            const int64_t r = rbase + rr;
            if (r >= n) break;
            acc += src[r * NB + q] * vs[r - c - 1];
        }
        qpart[int64_t(blockIdx.x) * 2 * NB + t] = acc;
    }
}

// q[t] = sum over blocks of qpart (fixed order); one block
template <class T>
__global__ void k_qreduce(const T *__restrict__ qpart, int nblk, int j, T *__restrict__ q) {
    const int t = threadIdx.x;
    if (t >= 2 * j) return;
    T acc = T(0);
    for (int b = 0; b < nblk; ++b) acc += qpart[int64_t(b) * 2 * NB + t];
    q[t] = acc;
}

// w[r] = tau (w_raw[r] - V[r] q1 - W[r] q2); partial dots w.v
template <class T>
__global__ void __launch_bounds__(256) k_wfinal1(int64_t n, int64_t c, const T *__restrict__ vbuf, T *__restrict__ wbuf,
                                                 const T *__restrict__ Vp, const T *__restrict__ Wp, int j,
                                                 const T *__restrict__ q, const T *__restrict__ scal, T *__restrict__ dpart) {
    __shared__ T sh[4];
    __shared__ T qs[2 * NB];
    if (threadIdx.x < 2 * j) qs[threadIdx.x] = q[threadIdx.x];
    __syncthreads();
    const T tv = scal[0];
    const int64_t r = c + 1 + int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    T dot = T(0);
    if (r < n) {
        T w = wbuf[r];
        for (int k = 0; k < j; ++k) w -= Vp[r * NB + k] * qs[k] + Wp[r * NB + k] * qs[j + k];
        w *= tv;
        wbuf[r] = w;
        dot = w * vbuf[r];
    }
    dot = block_sum(dot, sh);
    if (threadIdx.x == 0) dpart[blockIdx.x] = dot;
}

// w -= (tau/2)(w.v) v; store V[:, j] = v, W[:, j] = w for rows r > c
template <class T>
__global__ void __launch_bounds__(256) k_wfinal2(int64_t n, int64_t c, const T *__restrict__ vbuf, const T *__restrict__ wbuf,
                                                 T *__restrict__ Vp, T *__restrict__ Wp, int j, const T *__restrict__ scal,
                                                 const T *__restrict__ dpart, int ndp) {
    __shared__ T s_g;
    if (threadIdx.x == 0) {
        T g = T(0);
        for (int i = 0; i < ndp; ++i) g += dpart[i];
        s_g = g;
    }
    __syncthreads();
    const T half = T(0.5) * scal[0] * s_g;
    const int64_t r = c + 1 + int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (r < n) {
        const T v = vbuf[r];
        Vp[r * NB + j] = v;
        Wp[r * NB + j] = wbuf[r] - half * v;
    }
}

// A[r][s] -= sum_q V[r][q] W[s][q] + W[r][q] V[s][q]   for r, s in [p, n)   (64 x 64 tiles)
template <class T>
__global__ void __launch_bounds__(256) k_trailing(T *__restrict__ A, int64_t lda, int64_t n, int64_t p, int jn,
                                                  const T *__restrict__ Vp, const T *__restrict__ Wp) {
    __shared__ T vr[64][NB + 1], wr[64][NB + 1], vs_[64][NB + 1], ws_[64][NB + 1];
    const int64_t r0 = p + int64_t(blockIdx.y) * 64, s0 = p + int64_t(blockIdx.x) * 64;
    for (int e = threadIdx.x; e < 64 * NB; e += 256) {
        const int rr = e / NB, q = e % NB;
        const bool okr = r0 + rr < n && q < jn, oks = s0 + rr < n && q < jn;
        vr[rr][q] = okr ? Vp[(r0 + rr) * NB + q] : T(0);
        wr[rr][q] = okr ? Wp[(r0 + rr) * NB + q] : T(0);
        vs_[rr][q] = oks ? Vp[(s0 + rr) * NB + q] : T(0);
        ws_[rr][q] = oks ? Wp[(s0 + rr) * NB + q] : T(0);
    }
    __syncthreads();
    const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
    T acc[4][4] = {};
    for (int q = 0; q < jn; ++q) {
        T a1[4], a2[4], b1[4], b2[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            a1[u] = vr[ty * 4 + u][q];
            a2[u] = wr[ty * 4 + u][q];
            b1[u] = ws_[tx * 4 + u][q];
            b2[u] = vs_[tx * 4 + u][q];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int w = 0; w < 4; ++w) acc[u][w] += a1[u] * b1[w] + a2[u] * b2[w];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const int64_t r = r0 + ty * 4 + u, s = s0 + tx * 4 + w;
            if (r < n && s < n) A[r * lda + s] -= acc[u][w];
        }
}

template <class T>
__global__ void k_last_diag(const T *__restrict__ A, int64_t lda, int64_t n, double *__restrict__ d) {
    if (threadIdx.x == 0 && blockIdx.x == 0) d[n - 1] = double(A[(n - 1) * lda + (n - 1)]);
}

// ---------------------------------------------------------------------------------------------
// 2. bisection (fp64)
// ---------------------------------------------------------------------------------------------
// number of eigenvalues of T strictly less than x (Sturm sequence of the LDL^T of T - x I)
__device__ __forceinline__ int sturm_count(const double *__restrict__ d, const double *__restrict__ e2, int64_t n,
                                           double x, double pivmin) {
    int cnt = 0;
    double q = d[0] - x;
    if (fabs(q) < pivmin) q = -pivmin;
    if (q < 0.0) ++cnt;
    for (int64_t i = 1; i < n; ++i) {
        q = d[i] - x - e2[i - 1] / q;
        if (fabs(q) < pivmin) q = -pivmin;
        if (q < 0.0) ++cnt;
    }
    return cnt;
}

__global__ void k_tri_prep(const double *__restrict__ d, const double *__restrict__ e, int64_t n, double *__restrict__ e2,
                           double *__restrict__ bounds) {
    // one block: e2, Gershgorin bounds, pivmin, norm
    __shared__ double smin[256], smax[256], se2[256];
    double lo = DBL_MAX, hi = -DBL_MAX, mx = 0.0;
    for (int64_t i = threadIdx.x; i < n; i += blockDim.x) {
        const double el = i > 0 ? fabs(e[i - 1]) : 0.0, er = i < n - 1 ? fabs(e[i]) : 0.0;
        lo = fmin(lo, d[i] - el - er);
        hi = fmax(hi, d[i] + el + er);
        if (i < n - 1) {
            e2[i] = e[i] * e[i];
            mx = fmax(mx, e2[i]);
        }
    }
    smin[threadIdx.x] = lo;
    smax[threadIdx.x] = hi;
    se2[threadIdx.x] = mx;
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int i = 1; i < blockDim.x; ++i) {
            lo = fmin(lo, smin[i]);
            hi = fmax(hi, smax[i]);
            mx = fmax(mx, se2[i]);
        }
        const double tnorm = fmax(fabs(lo), fabs(hi));
        const double pad = 2.0 * DBL_EPSILON * tnorm * double(n) + DBL_MIN;
        bounds[0] = lo - pad;
        bounds[1] = hi + pad;
        bounds[2] = DBL_MIN * fmax(1.0, mx);  // pivmin
        bounds[3] = tnorm;
    }
}

// lam_asc[i] = i-th smallest eigenvalue of T
__global__ void __launch_bounds__(64) k_bisect(const double *__restrict__ d, const double *__restrict__ e2, int64_t n,
                                               const double *__restrict__ bounds, double *__restrict__ lam_asc) {
    const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= n) return;
    double lo = bounds[0], hi = bounds[1];
    const double pivmin = bounds[2];
    const double atol = DBL_EPSILON * bounds[3];  // absolute accuracy eps ||T||
    for (int it = 0; it < 128; ++it) {
        const double mid = 0.5 * (lo + hi);
        if (mid <= lo || mid >= hi) break;
        if (hi - lo <= 2.0 * DBL_EPSILON * fmax(fabs(lo), fabs(hi)) + atol) break;
        if (sturm_count(d, e2, n, mid, pivmin) > i) hi = mid; else lo = mid;
    }
    lam_asc[i] = 0.5 * (lo + hi);
}

// lambda (descending) from lam_asc
__global__ void k_lambda_desc(const double *__restrict__ lam_asc, int64_t n, double *__restrict__ lambda, const int *bad) {
    const int64_t j = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (j < n) lambda[j] = *bad ? double(NAN) : lam_asc[n - 1 - j];
}

// ---------------------------------------------------------------------------------------------
// 3. inverse iteration (fp64), one thread per eigenvector; arrays laid out [row][vector] so the
// threads of a wavefront touch consecutive addresses.
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ double hash_unit(uint64_t x) {
    x ^= x >> 33;
    x *= 0xff51afd7ed558ccdULL;
    x ^= x >> 33;
    x *= 0xc4ceb9fe1a85ec53ULL;
    x ^= x >> 33;
    return double(x >> 11) * (1.0 / 9007199254740992.0) * 2.0 - 1.0;  // [-1, 1)
}

__global__ void __launch_bounds__(64) k_invit(const double *__restrict__ d, const double *__restrict__ e, int64_t n,
                                              const double *__restrict__ lam_asc, const double *__restrict__ bounds,
                                              int64_t nv, double *__restrict__ Z, double *__restrict__ U0,
                                              double *__restrict__ U1, double *__restrict__ U2) {
    const int64_t j = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (j >= nv) return;
    const double lam = lam_asc[n - 1 - j];
    const double tnorm = bounds[3];
    const double tiny = DBL_EPSILON * fmax(tnorm, DBL_MIN);
    // start vector
    for (int64_t r = 0; r < n; ++r) Z[r * nv + j] = hash_unit(uint64_t(r) * 0x9E3779B97F4A7C15ULL + uint64_t(j) + 1);
    for (int iter = 0; iter < 4; ++iter) {
        // forward elimination with partial pivoting on T - lam I, applied to b = Z[:, j]
        double u0 = d[0] - lam, u1 = n > 1 ? e[0] : 0.0, u2 = 0.0;  // current pivot-row candidates
        double bcur = Z[j];
        for (int64_t k = 0; k < n - 1; ++k) {
            const double l = e[k], dd = d[k + 1] - lam, ee = k + 1 < n - 1 ? e[k + 1] : 0.0;
            const double bnext = Z[(k + 1) * nv + j];
            double p0, p1, p2, bp, n1, n2, bn;
            if (fabs(l) > fabs(u0)) {  // swap rows k, k+1
                const double mlt = u0 / l;
                p0 = l; p1 = dd; p2 = ee; bp = bnext;
                n1 = u1 - mlt * dd; n2 = u2 - mlt * ee; bn = bcur - mlt * bnext;
            } else {
                if (u0 == 0.0) u0 = tiny;
                const double mlt = l / u0;
                p0 = u0; p1 = u1; p2 = u2; bp = bcur;
                n1 = dd - mlt * u1; n2 = ee - mlt * u2; bn = bnext - mlt * bcur;
            }
            U0[k * nv + j] = p0;
            U1[k * nv + j] = p1;
            U2[k * nv + j] = p2;
            Z[k * nv + j] = bp;
            u0 = n1; u1 = n2; u2 = 0.0; bcur = bn;
        }
        if (u0 == 0.0) u0 = tiny;
        // back substitution
        double y2 = 0.0, y1 = bcur / u0, ymax = fabs(y1);
        Z[(n - 1) * nv + j] = y1;
        for (int64_t k = n - 2; k >= 0; --k) {
            const double y = (Z[k * nv + j] - U1[k * nv + j] * y1 - U2[k * nv + j] * y2) / U0[k * nv + j];
            Z[k * nv + j] = y;
            ymax = fmax(ymax, fabs(y));
            y2 = y1;
            y1 = y;
        }
        const double inv = ymax > 0.0 ? 1.0 / ymax : 1.0;
        for (int64_t r = 0; r < n; ++r) Z[r * nv + j] *= inv;
    }
    double s = 0.0;
    for (int64_t r = 0; r < n; ++r) s += Z[r * nv + j] * Z[r * nv + j];
    const double inv = s > 0.0 ? 1.0 / sqrt(s) : 0.0;
    for (int64_t r = 0; r < n; ++r) Z[r * nv + j] *= inv;
}

// Re-orthogonalise clusters: vector j starts a cluster when lam_{j-1} - lam_j > ctol; the leader's
// block runs modified Gram-Schmidt over its cluster members in order.
__global__ void __launch_bounds__(256) k_cluster_mgs(const double *__restrict__ lam_asc, int64_t n, int64_t nv,
                                                     const double *__restrict__ bounds, double *__restrict__ Z) {
    __shared__ double sh[4];
    const int64_t j0 = blockIdx.x;
    const double ctol = 1e-10 * bounds[3];
    auto lamd = [&](int64_t j) { return lam_asc[n - 1 - j]; };
    if (j0 > 0 && lamd(j0 - 1) - lamd(j0) <= ctol) return;  // not a leader
    int64_t j1 = j0 + 1;
    while (j1 < nv && lamd(j1 - 1) - lamd(j1) <= ctol) ++j1;
    if (j1 - j0 < 2) return;
    for (int64_t j = j0 + 1; j < j1; ++j) {
        for (int64_t k = j0; k < j; ++k) {
            double dot = 0.0;
            for (int64_t r = threadIdx.x; r < n; r += blockDim.x) dot += Z[r * nv + k] * Z[r * nv + j];
            dot = block_sum(dot, sh);
            for (int64_t r = threadIdx.x; r < n; r += blockDim.x) Z[r * nv + j] -= dot * Z[r * nv + k];
            __syncthreads();
        }
        double s = 0.0;
        for (int64_t r = threadIdx.x; r < n; r += blockDim.x) s += Z[r * nv + j] * Z[r * nv + j];
        s = block_sum(s, sh);
        const double inv = s > 0.0 ? 1.0 / sqrt(s) : 0.0;
        for (int64_t r = threadIdx.x; r < n; r += blockDim.x) Z[r * nv + j] *= inv;
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------------------------
// 4. back-transformation
// ---------------------------------------------------------------------------------------------
// partial Gram S[a][b] = sum_{r in chunk} Rt[c0+a][r] Rt[c0+b][r]
template <class T>
__global__ void __launch_bounds__(256) k_bt_gram(const T *__restrict__ Rt, int64_t ldr, int64_t n, int64_t c0, int nb,
                                                 double *__restrict__ Sp) {
    __shared__ double vs[NBT][RCH / 8 + 1];
    const int64_t r0 = int64_t(blockIdx.x) * RCH;
    double acc[4] = {0, 0, 0, 0};
    const int ab = threadIdx.x;  // pairs ab + 256 u, u < 4: a = pair / NBT, b = pair % NBT
    for (int64_t rs = 0; rs < RCH; rs += RCH / 8) {
        for (int e = threadIdx.x; e < NBT * (RCH / 8); e += 256) {
            const int q = e / (RCH / 8), rr = e % (RCH / 8);
            const int64_t r = r0 + rs + rr;
            vs[q][rr] = (q < nb && r < n) ? double(Rt[(c0 + q) * ldr + r]) : 0.0;
        }
        __syncthreads();
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int pidx = ab + 256 * u;
            const int pa = pidx / NBT, pb = pidx % NBT;
            double s = 0.0;
            for (int rr = 0; rr < RCH / 8; ++rr) s += vs[pa][rr] * vs[pb][rr];
            acc[u] += s;
        }
        __syncthreads();
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) Sp[int64_t(blockIdx.x) * NBT * NBT + ab + 256 * u] = acc[u];
}

// one block: S = sum of partials; T factor of the block (forward, columnwise)
template <class T>
__global__ void __launch_bounds__(256) k_bt_tfactor(const double *__restrict__ Sp, int nchunk, const T *__restrict__ tau,
                                                    int64_t c0, int nb, double *__restrict__ Tf) {
    __shared__ double S[NBT][NBT], Tm[NBT][NBT];
    for (int e = threadIdx.x; e < NBT * NBT; e += 256) {
        double s = 0.0;
        for (int k = 0; k < nchunk; ++k) s += Sp[int64_t(k) * NBT * NBT + e];
        S[e / NBT][e % NBT] = s;
        Tm[e / NBT][e % NBT] = 0.0;
    }
    __syncthreads();
    for (int i = 0; i < nb; ++i) {
        const double ti = double(tau[c0 + i]);
        // T[0:i, i] = -tau_i T[0:i, 0:i] S[0:i, i]
        double v = 0.0;
        const int a = threadIdx.x;
        if (a < i) {
            for (int k = a; k < i; ++k) v += Tm[a][k] * S[k][i];
        }
        __syncthreads();
        if (a < i) Tm[a][i] = -ti * v;
        if (a == 0) Tm[i][i] = ti;
        __syncthreads();
    }
    for (int e = threadIdx.x; e < NBT * NBT; e += 256) Tf[e] = Tm[e / NBT][e % NBT];
}

// partial G[q][col] = sum_{r in chunk} Rt[c0+q][r] Z[r][col]; grid (col tiles of 64, row chunks)
template <class T>
__global__ void __launch_bounds__(256) k_bt_g(const T *__restrict__ Rt, int64_t ldr, int64_t n, int64_t c0, int nb,
                                              const double *__restrict__ Z, int64_t nv, double *__restrict__ Gp) {
    __shared__ double vs[NBT][65];
    __shared__ double zs[64][65];
    const int64_t col0 = int64_t(blockIdx.x) * 64, r0 = int64_t(blockIdx.y) * RCH;
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;  // 4 rows of q per thread group
    double acc[NBT / 4];
#pragma unroll
    for (int u = 0; u < NBT / 4; ++u) acc[u] = 0.0;
    for (int64_t rs = 0; rs < RCH; rs += 64) {
        for (int e = threadIdx.x; e < NBT * 64; e += 256) {
            const int q = e / 64, rr = e % 64;
            const int64_t r = r0 + rs + rr;
            vs[q][rr] = (q < nb && r < n) ? double(Rt[(c0 + q) * ldr + r]) : 0.0;
        }
        for (int e = threadIdx.x; e < 64 * 64; e += 256) {
            const int rr = e / 64, cc = e % 64;
            const int64_t r = r0 + rs + rr, col = col0 + cc;
            zs[rr][cc] = (r < n && col < nv) ? Z[r * nv + col] : 0.0;
        }
        __syncthreads();
        for (int rr = 0; rr < 64; ++rr) {
            const double z = zs[rr][tx];
#pragma unroll
            for (int u = 0; u < NBT / 4; ++u) acc[u] += vs[ty + 4 * u][rr] * z;
        }
        __syncthreads();
    }
    const int64_t col = col0 + tx;
    if (col < nv)
#pragma unroll
        for (int u = 0; u < NBT / 4; ++u) Gp[(int64_t(blockIdx.y) * NBT + ty + 4 * u) * nv + col] = acc[u];
}

// G = T (sum of partials)
__global__ void __launch_bounds__(256) k_bt_greduce(const double *__restrict__ Gp, int nchunk, int64_t nv,
                                                    const double *__restrict__ Tf, double *__restrict__ G) {
    __shared__ double Tm[NBT][NBT];
    for (int e = threadIdx.x; e < NBT * NBT; e += 256) Tm[e / NBT][e % NBT] = Tf[e];
    __syncthreads();
    const int64_t col = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (col >= nv) return;
    double g[NBT];
#pragma unroll
    for (int q = 0; q < NBT; ++q) {
        double s = 0.0;
        for (int k = 0; k < nchunk; ++k) s += Gp[(int64_t(k) * NBT + q) * nv + col];
        g[q] = s;
    }
#pragma unroll
    for (int a = 0; a < NBT; ++a) {
        double s = 0.0;
#pragma unroll
        for (int q = 0; q < NBT; ++q) s += Tm[a][q] * g[q];
        G[int64_t(a) * nv + col] = s;
    }
}

// Z[r][col] -= sum_q Rt[c0+q][r] G[q][col] for r > c0
template <class T>
__global__ void __launch_bounds__(256) k_bt_update(const T *__restrict__ Rt, int64_t ldr, int64_t n, int64_t c0, int nb,
                                                   const double *__restrict__ G, double *__restrict__ Z, int64_t nv) {
    __shared__ double vs[64][NBT + 1];
    __shared__ double gs[NBT][65];
    const int64_t col0 = int64_t(blockIdx.x) * 64, r0 = c0 + 1 + int64_t(blockIdx.y) * 64;
    for (int e = threadIdx.x; e < NBT * 64; e += 256) {
        const int q = e / 64, rr = e % 64;
        const int64_t r = r0 + rr, col = col0 + rr;
        vs[rr][q] = (q < nb && r < n) ? double(Rt[(c0 + q) * ldr + r]) : 0.0;
        gs[q][rr] = (q < nb && col < nv) ? G[int64_t(q) * nv + col] : 0.0;
    }
    __syncthreads();
    const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
    double acc[4][4] = {};
    for (int q = 0; q < nb; ++q) {
        double a[4], b[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            a[u] = vs[ty * 4 + u][q];
            b[u] = gs[q][tx * 4 + u];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int w = 0; w < 4; ++w) acc[u][w] += a[u] * b[w];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const int64_t r = r0 + ty * 4 + u, col = col0 + tx * 4 + w;
            if (r < n && col < nv) Z[r * nv + col] -= acc[u][w];
        }
}

// ---------------------------------------------------------------------------------------------
// 5. signs and output
// ---------------------------------------------------------------------------------------------
__global__ void __launch_bounds__(256) k_sign_out(const double *__restrict__ Z, int64_t n, int64_t nv,
                                                  float *__restrict__ V, int64_t ldv, const int *bad) {
    __shared__ double sb[256];
    __shared__ int si[256];
    const int64_t j = blockIdx.x;
    double best = -1.0;
    int64_t bi = n;
    for (int64_t r = threadIdx.x; r < n; r += blockDim.x) {
        const double a = fabs(Z[r * nv + j]);
        if (a > best) { best = a; bi = r; }
    }
    sb[threadIdx.x] = best;
    si[threadIdx.x] = int(bi);
    __syncthreads();
    for (int o = 128; o > 0; o >>= 1) {
        if (threadIdx.x < o) {
            const double ob = sb[threadIdx.x + o];
            const int oi = si[threadIdx.x + o];
            if (ob > sb[threadIdx.x] || (ob == sb[threadIdx.x] && oi < si[threadIdx.x])) {
                sb[threadIdx.x] = ob;
                si[threadIdx.x] = oi;
            }
        }
        __syncthreads();
    }
    const double sgn = (si[0] < n && Z[int64_t(si[0]) * nv + j] < 0.0) ? -1.0 : 1.0;
    const bool isbad = *bad != 0;
    for (int64_t r = threadIdx.x; r < n; r += blockDim.x)
        V[r * ldv + j] = isbad ? NAN : float(sgn * Z[r * nv + j]);
}

__global__ void k_set_info(int32_t *info, const int *bad) {
    if (threadIdx.x == 0) *info = *bad ? LRC_INFO_NONFINITE : LRC_INFO_OK;
}

// ---------------------------------------------------------------------------------------------
// host
// ---------------------------------------------------------------------------------------------
template <class T>
struct LargeWs {
    T *A, *Rt, *Vp, *Wp, *tau, *vbuf, *wbuf, *part, *qpart, *q, *dpart, *scal;
    double *d, *e, *e2, *bounds, *lam, *Z, *U0, *U1, *U2, *Sp, *Tf, *Gp, *G;
    int *bad;
    int64_t lda;
};

static int64_t nsymv_blocks(int64_t n) { return (n + SYMV_ROWS - 1) / SYMV_ROWS; }

template <class C_, class T>
static void layout(C_ &cv, LargeWs<T> &w, int64_t n, int64_t nv, bool count_only) {
    (void)count_only;
    w.lda = n;
    const int64_t nv1 = nv > 0 ? nv : 1;
    const int64_t nch = (n + RCH - 1) / RCH;
    w.A = cv.template carve<T>(size_t(n) * size_t(n));
    w.Rt = cv.template carve<T>(size_t(n) * size_t(n));
    w.Vp = cv.template carve<T>(size_t(n) * NB);
    w.Wp = cv.template carve<T>(size_t(n) * NB);
    w.tau = cv.template carve<T>(size_t(n));
    w.vbuf = cv.template carve<T>(size_t(n));
    w.wbuf = cv.template carve<T>(size_t(n));
    w.part = cv.template carve<T>(size_t((n + 255) / 256 + 1));
    w.qpart = cv.template carve<T>(size_t(nsymv_blocks(n)) * 2 * NB);
    w.q = cv.template carve<T>(2 * NB);
    w.dpart = cv.template carve<T>(size_t((n + 255) / 256 + 1));
    w.scal = cv.template carve<T>(4);
    w.d = cv.template carve<double>(size_t(n));
    w.e = cv.template carve<double>(size_t(n));
    w.e2 = cv.template carve<double>(size_t(n));
    w.bounds = cv.template carve<double>(4);
    w.lam = cv.template carve<double>(size_t(n));
    w.Z = cv.template carve<double>(size_t(n) * size_t(nv1));
    w.U0 = cv.template carve<double>(size_t(n) * size_t(nv1));
    w.U1 = cv.template carve<double>(size_t(n) * size_t(nv1));
    w.U2 = cv.template carve<double>(size_t(n) * size_t(nv1));
    w.Sp = cv.template carve<double>(size_t(nch) * NBT * NBT);
    w.Tf = cv.template carve<double>(NBT * NBT);
    w.Gp = cv.template carve<double>(size_t(nch) * NBT * size_t(nv1));
    w.G = cv.template carve<double>(NBT * size_t(nv1));
    w.bad = cv.template carve<int>(1);
}

struct CountCarver {
    Counter c;
    template <class T>
    T *carve(size_t count) {
        c.carve<T>(count);
        return nullptr;
    }
};

template <class T>
static size_t large_ws(int64_t n, int64_t nv) {
    CountCarver cc;
    LargeWs<T> w;
    layout(cc, w, n, nv, true);
    return cc.c.off;
}

template <class T>
static lrc_status large_run_one(const float *C, int64_t ldc, int64_t n, double *lambda, float *V, int64_t ldv,
                                int64_t nv, int32_t *info, LargeWs<T> &w, hipStream_t s) {
    const int64_t lda = w.lda;
    hipLaunchKernelGGL(k_fill_zero<int>, dim3(1), dim3(64), 0, s, w.bad, int64_t(1));
    hipLaunchKernelGGL(k_fill_full<T>, dim3(2048), dim3(256), 0, s, C, ldc, n, w.A, lda, w.bad);
    LRC_LAUNCH_CHECK("k_fill_full");
    const size_t symv_smem = size_t(n) * sizeof(T);
    LRC_HIP(hipFuncSetAttribute(reinterpret_cast<const void *>(k_symv<T>), hipFuncAttributeMaxDynamicSharedMemorySize,
                                int(symv_smem)));
    // 1. tridiagonalisation, panels over reflector columns 0 .. n-2
    for (int64_t p0 = 0; p0 < n - 1; p0 += NB) {
        const int64_t p1 = std::min<int64_t>(p0 + NB, n - 1);
        hipLaunchKernelGGL(k_fill_zero<T>, dim3(64), dim3(256), 0, s, w.Vp, int64_t(n) * NB);
        hipLaunchKernelGGL(k_fill_zero<T>, dim3(64), dim3(256), 0, s, w.Wp, int64_t(n) * NB);
        for (int64_t c = p0; c < p1; ++c) {
            const int j = int(c - p0);
            const int nbu = cdiv(n - c, 256);
            hipLaunchKernelGGL(k_col_update<T>, dim3(nbu), dim3(256), 0, s, w.A, lda, n, c, j, w.Vp, w.Wp, w.part);
            hipLaunchKernelGGL(k_householder<T>, dim3(1), dim3(1024), 0, s, w.A, lda, n, c, w.part, nbu, w.vbuf, w.Rt, n,
                               w.tau, w.d, w.e, w.scal);
            const int64_t m = n - c - 1;
            const int nsb = cdiv(m, SYMV_ROWS);
            hipLaunchKernelGGL(k_symv<T>, dim3(nsb), dim3(256), size_t(m) * sizeof(T), s, w.A, lda, n, c, w.vbuf, w.wbuf,
                               w.Vp, w.Wp, j, w.qpart);
            hipLaunchKernelGGL(k_qreduce<T>, dim3(1), dim3(64), 0, s, w.qpart, nsb, j, w.q);
            const int nwb = cdiv(m, 256);
            hipLaunchKernelGGL(k_wfinal1<T>, dim3(nwb), dim3(256), 0, s, n, c, w.vbuf, w.wbuf, w.Vp, w.Wp, j, w.q, w.scal,
                               w.dpart);
            hipLaunchKernelGGL(k_wfinal2<T>, dim3(nwb), dim3(256), 0, s, n, c, w.vbuf, w.wbuf, w.Vp, w.Wp, j, w.scal,
                               w.dpart, nwb);
        }
        LRC_LAUNCH_CHECK("tridiagonal panel");
        const int jn = int(p1 - p0);
        if (p1 < n - 1) {
            const int64_t m = n - p1;
            dim3 g(cdiv(m, 64), cdiv(m, 64));
            hipLaunchKernelGGL(k_trailing<T>, g, dim3(256), 0, s, w.A, lda, n, p1, jn, w.Vp, w.Wp);
            LRC_LAUNCH_CHECK("k_trailing");
        } else {
            hipLaunchKernelGGL(k_col_update<T>, dim3(1), dim3(256), 0, s, w.A, lda, n, n - 1, jn, w.Vp, w.Wp, w.part);
            LRC_LAUNCH_CHECK("k_col_update");
        }
    }
    hipLaunchKernelGGL(k_last_diag<T>, dim3(1), dim3(64), 0, s, w.A, lda, n, w.d);
    // 2. eigenvalues
    hipLaunchKernelGGL(k_tri_prep, dim3(1), dim3(256), 0, s, w.d, w.e, n, w.e2, w.bounds);
    hipLaunchKernelGGL(k_bisect, dim3(cdiv(n, 64)), dim3(64), 0, s, w.d, w.e2, n, w.bounds, w.lam);
    hipLaunchKernelGGL(k_lambda_desc, dim3(cdiv(n, 256)), dim3(256), 0, s, w.lam, n, lambda, w.bad);
    LRC_LAUNCH_CHECK("bisection");
    if (nv > 0) {
        // 3. eigenvectors of T
        hipLaunchKernelGGL(k_invit, dim3(cdiv(nv, 64)), dim3(64), 0, s, w.d, w.e, n, w.lam, w.bounds, nv, w.Z, w.U0, w.U1,
                           w.U2);
        hipLaunchKernelGGL(k_cluster_mgs, dim3(unsigned(nv)), dim3(256), 0, s, w.lam, n, nv, w.bounds, w.Z);
        LRC_LAUNCH_CHECK("inverse iteration");
        // 4. back-transformation, last block of reflectors first
        const int64_t nrefl = n - 1;
        const int nch = cdiv(n, RCH);
        for (int64_t c0 = ((nrefl - 1) / NBT) * NBT; c0 >= 0; c0 -= NBT) {
            const int nb = int(std::min<int64_t>(NBT, nrefl - c0));
            hipLaunchKernelGGL(k_bt_gram<T>, dim3(nch), dim3(256), 0, s, w.Rt, n, n, c0, nb, w.Sp);
            hipLaunchKernelGGL(k_bt_tfactor<T>, dim3(1), dim3(256), 0, s, w.Sp, nch, w.tau, c0, nb, w.Tf);
            hipLaunchKernelGGL(k_bt_g<T>, dim3(cdiv(nv, 64), nch), dim3(256), 0, s, w.Rt, n, n, c0, nb, w.Z, nv, w.Gp);
            hipLaunchKernelGGL(k_bt_greduce, dim3(cdiv(nv, 256)), dim3(256), 0, s, w.Gp, nch, nv, w.Tf, w.G);
            const int64_t mrows = n - c0 - 1;
            hipLaunchKernelGGL(k_bt_update<T>, dim3(cdiv(nv, 64), cdiv(mrows, 64)), dim3(256), 0, s, w.Rt, n, n, c0, nb,
                               w.G, w.Z, nv);
        }
        LRC_LAUNCH_CHECK("back-transformation");
        hipLaunchKernelGGL(k_sign_out, dim3(unsigned(nv)), dim3(256), 0, s, w.Z, n, nv, V, ldv, w.bad);
        LRC_LAUNCH_CHECK("k_sign_out");
    }
    hipLaunchKernelGGL(k_set_info, dim3(1), dim3(64), 0, s, info, w.bad);
    LRC_LAUNCH_CHECK("k_set_info");
    return LRC_OK;
}

size_t eigh_workspace(int64_t n, int64_t batch, int64_t n_vec, lrc_dtype prec) {
    (void)batch;
    if (n <= 128) return jacobi_workspace(n, batch, prec);
    return prec == LRC_F64 ? large_ws<double>(n, n_vec) : large_ws<float>(n, n_vec);
}

template <class T>
static lrc_status large_run(const EighArgs &a, void *ws, size_t ws_bytes, hipStream_t s) {
    Carver cv(ws, ws_bytes);
    LargeWs<T> w;
    layout(cv, w, a.n, a.n_vec, false);
    if (!w.bad) return fail(LRC_ERR_WORKSPACE, "eigh workspace too small");
    for (int64_t b = 0; b < a.batch; ++b) {
        lrc_status st = large_run_one<T>(a.C + b * a.stride_c, a.ldc, a.n, a.lambda + b * a.n,
                                         a.V ? a.V + b * a.stride_v : nullptr, a.ldv, a.n_vec, a.info + b, w, s);
        if (st != LRC_OK) return st;
    }
    return LRC_OK;
}

lrc_status eigh_run(const EighArgs &a, void *ws, size_t ws_bytes, hipStream_t s) {
    if (a.n <= 128) return jacobi_run(a, ws, ws_bytes, s);
    if (int64_t(a.n) * int64_t(sizeof(double)) > 160 * 1024 && a.prec == LRC_F64)
        return fail(LRC_ERR_UNIMPLEMENTED, "fp64 working precision supports n <= 20480");
    if (int64_t(a.n) * int64_t(sizeof(float)) > 160 * 1024) return fail(LRC_ERR_UNIMPLEMENTED, "n > 40960");
    return a.prec == LRC_F64 ? large_run<double>(a, ws, ws_bytes, s) : large_run<float>(a, ws, ws_bytes, s);
}

}  // namespace lrc
