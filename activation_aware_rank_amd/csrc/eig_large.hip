// Symmetric eigendecomposition for n > 128 (Swift-SVD page, section 2-ga: one eigendecomposition
// of Y^T Y yields V and Sigma^2 of Y).
//
// Stages, all on the GPU:
//  1. Householder tridiagonalisation Q^T C Q = T, blocked (panel of NB columns, then a rank-2NB
//     update of the trailing matrix), working precision T_ (fp32 or fp64).  The matrix is kept
//     in full (both triangles) so the symmetric matrix-vector product of each column is a plain
//     row-wise product with coalesced rows; three launches per column.
//  2. All n eigenvalues of T by multisection on Sturm counts, fp64, 16 lanes per eigenvalue.
//  3. Eigenvectors of T for the n_vec largest eigenvalues by inverse iteration, fp64, one thread
//     per vector (LU with partial pivoting of T - lambda I once, then three solves); vectors of
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
constexpr int SYMV_BLOCKS = 128;  // blocks of 16 waves in the symmetric product (rows strided over them)

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

// Each column of a panel takes three launches; each global reduction is done by the next launch,
// redundantly in every block that needs it and always in the same fixed order, so all blocks see
// bit-identical values (no atomics, no device-wide fences):
//   k_trd_col : finish W[:, j-1] (reduces the previous column's w1.v partials), update column c,
//               partials of ||x||^2
//   k_trd_symv: reflector of column c (reduces the ||x||^2 partials; block 0 stores d[c], e[c],
//               tau[c]); v into V[:, j] and Rt[c]; w_raw = A v over the trailing rows; partials of
//               W^T v and V^T v
//   k_trd_w1  : w1 = tau (w_raw - V q1 - W q2) (reduces the q partials); partials of w1.v
// W[:, j] = w1 - (tau/2)(w1.v) v is formed by the next k_trd_col (or k_trd_wlast at panel end).

// fixed-order sum of p[0..np) by one block: strided per-thread sums, then a tree (every thread)
template <class T>
__device__ __forceinline__ T block_sum_array(const T *__restrict__ p, int np, T *red) {
    T acc = T(0);
    for (int i = threadIdx.x; i < np; i += blockDim.x) acc += p[i];
    return block_sum(acc, red);
}

template <class T>
__global__ void __launch_bounds__(256) k_trd_col(T *__restrict__ A, int64_t lda, int64_t n, int64_t c, int j,
                                                 T *__restrict__ Vp, T *__restrict__ Wp, const T *__restrict__ w1buf,
                                                 T *__restrict__ colbuf, T *__restrict__ part, const T *__restrict__ dpart,
                                                 int ndp, const T *__restrict__ tau, double *__restrict__ d) {
    __shared__ T sh[4];
    __shared__ T vc[NB], wc[NB];
    T half = T(0);
    if (j > 0) half = T(0.5) * tau[c - 1] * block_sum_array(dpart, ndp, sh);
    if (threadIdx.x < NB) {
        const int q = threadIdx.x;
        vc[q] = q < j ? Vp[c * NB + q] : T(0);
        T wv = q < j ? Wp[c * NB + q] : T(0);
        if (q == j - 1) wv = w1buf[c] - half * Vp[c * NB + q];  // row c of the column being finished
        wc[q] = wv;
    }
    __syncthreads();
    const int64_t r = c + int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    T ss = T(0);
    if (r < n) {
        T wl = T(0);
        if (j > 0) {  // finish W[r][j-1] for this row
            wl = w1buf[r] - half * Vp[r * NB + j - 1];
            Wp[r * NB + j - 1] = wl;
        }
        T a = A[r * lda + c];
        for (int q = 0; q < j; ++q) {
            const T wr = (q == j - 1) ? wl : Wp[r * NB + q];
            a -= Vp[r * NB + q] * wc[q] + wr * vc[q];
        }
        A[r * lda + c] = a;
        colbuf[r] = a;
        if (r >= c + 2) ss = a * a;
        if (r == c) d[c] = double(a);
    }
    ss = block_sum(ss, sh);
    if (threadIdx.x == 0) part[blockIdx.x] = ss;
}

// w_raw[r] = sum_{k > c} A[r][k] v[k] for rows r in [c+1, n), one row per wave at a time (rows
// strided over the grid), read with 16-byte loads from the aligned column kb <= c+1 (v[k] = 0 for
// k <= c).  Also stores v in V[:, j] and Rt[c], and the block partials of W^T v and V^T v.
constexpr int SYMV_WAVES = 16;
template <class T>
__global__ void __launch_bounds__(SYMV_WAVES * 64) k_trd_symv(const T *__restrict__ A, int64_t lda, int64_t n, int64_t c,
                                                              int j, const T *__restrict__ colbuf,
                                                              const T *__restrict__ part, int npart,
                                                              T *__restrict__ Vp, const T *__restrict__ Wp,
                                                              T *__restrict__ Rt, T *__restrict__ wbuf,
                                                              T *__restrict__ qpart, T *__restrict__ tau,
                                                              double *__restrict__ e) {
    constexpr int VEC = 16 / sizeof(T);
    constexpr int NW = SYMV_WAVES;
    typedef T vec_t __attribute__((ext_vector_type(VEC)));
    extern __shared__ __attribute__((aligned(16))) char smem_raw[];
    T *vs = reinterpret_cast<T *>(smem_raw);  // v[kb .. n)
    __shared__ T sh[NW];
    // the reflector of column c: alpha = x[0], sigma2 = ||x[1:]||^2; tau = (beta - alpha)/beta,
    // v = [1, x[1:] / (alpha - beta)], beta = -sign(alpha) ||x||; tau = 0 when x[1:] = 0
    const T sigma2 = block_sum_array(part, npart, sh);
    const T alpha = colbuf[c + 1];
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
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        e[c] = double(beta);
        tau[c] = tv;
    }
    const int64_t kb = (c + 1) / VEC * VEC;
    const int64_t m = n - kb;
    const int64_t mv = m / VEC;
    for (int64_t k = threadIdx.x; k < m; k += blockDim.x) {
        const int64_t kk = kb + k;
        vs[k] = kk <= c ? T(0) : (kk == c + 1 ? T(1) : colbuf[kk] * scale);
    }
    if (blockIdx.x == 0)  // the reflector's zeros above row c+1
        for (int64_t k = threadIdx.x; k <= c; k += blockDim.x) Rt[c * n + k] = T(0);
    __syncthreads();
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t nrows = n - c - 1;
    const int64_t wstride = int64_t(gridDim.x) * NW;
    T qw = T(0), qv = T(0);
    const vec_t *vs4 = reinterpret_cast<const vec_t *>(vs);
    for (int64_t rr = int64_t(blockIdx.x) * NW + wave; rr < nrows; rr += wstride) {
        const int64_t r = c + 1 + rr;
        const T *row = A + r * lda + kb;
        const vec_t *row4 = reinterpret_cast<const vec_t *>(row);
        T acc0 = T(0), acc1 = T(0), acc2 = T(0), acc3 = T(0);
        int64_t kv = lane;
        for (; kv + 192 < mv; kv += 256) {
            const vec_t a0 = __builtin_nontemporal_load(row4 + kv), a1 = __builtin_nontemporal_load(row4 + kv + 64);
            const vec_t a2 = __builtin_nontemporal_load(row4 + kv + 128), a3 = __builtin_nontemporal_load(row4 + kv + 192);
            const vec_t b0 = vs4[kv], b1 = vs4[kv + 64], b2 = vs4[kv + 128], b3 = vs4[kv + 192];
#pragma unroll
            for (int q = 0; q < VEC; ++q) {
                acc0 += a0[q] * b0[q];
                acc1 += a1[q] * b1[q];
                acc2 += a2[q] * b2[q];
                acc3 += a3[q] * b3[q];
            }
        }
        for (; kv < mv; kv += 64) {
            const vec_t a0 = row4[kv], b0 = vs4[kv];
#pragma unroll
            for (int q = 0; q < VEC; ++q) acc0 += a0[q] * b0[q];
        }
        for (int64_t k = mv * VEC + lane; k < m; k += 64) acc0 += row[k] * vs[k];
        T acc = (acc0 + acc1) + (acc2 + acc3);
        for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
        const T vr = vs[r - kb];
        if (lane == 0) {
            wbuf[r] = acc;
            Rt[c * n + r] = vr;
            Vp[r * NB + j] = vr;
        }
        if (lane < j) {
            qw += Wp[r * NB + lane] * vr;
            qv += Vp[r * NB + lane] * vr;
        }
    }
    __shared__ T qs[NW][2 * NB];
    if (lane < NB) {
        qs[wave][lane] = lane < j ? qw : T(0);
        qs[wave][NB + lane] = lane < j ? qv : T(0);
    }
    __syncthreads();
    const int t = threadIdx.x;
    if (t < 2 * NB) {
        T sum = T(0);
        for (int w = 0; w < NW; ++w) sum += qs[w][t];
        qpart[int64_t(blockIdx.x) * 2 * NB + t] = sum;
    }
}

// w1[r] = tau (w_raw[r] - V[r][:j] q1 - W[r][:j] q2) for r in [c+1, n); partials of w1.v
template <class T>
__global__ void __launch_bounds__(256) k_trd_w1(int64_t n, int64_t c, int j, const T *__restrict__ Vp,
                                                const T *__restrict__ Wp, const T *__restrict__ wbuf,
                                                const T *__restrict__ qpart, int nqp, const T *__restrict__ tau,
                                                T *__restrict__ w1buf, T *__restrict__ dpart) {
    __shared__ T sh[4];
    __shared__ T red[4][2 * NB];
    __shared__ T qs[2 * NB];
    {  // q[v] = sum over the symv blocks, fixed order: 4 strided sums per value, then in order
        const int v = threadIdx.x % (2 * NB), sidx = threadIdx.x / (2 * NB);
        T acc = T(0);
        for (int b = sidx; b < nqp; b += 4) acc += qpart[int64_t(b) * 2 * NB + v];
        red[sidx][v] = acc;
        __syncthreads();
        if (sidx == 0) qs[v] = (red[0][v] + red[1][v]) + (red[2][v] + red[3][v]);
        __syncthreads();
    }
    const T tv = tau[c];
    const int64_t r = c + 1 + int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    T dot = T(0);
    if (r < n) {
        T w = wbuf[r];
        for (int k = 0; k < j; ++k) w -= Vp[r * NB + k] * qs[k] + Wp[r * NB + k] * qs[NB + k];
        w *= tv;
        w1buf[r] = w;
        dot = w * Vp[r * NB + j];
    }
    dot = block_sum(dot, sh);
    if (threadIdx.x == 0) dpart[blockIdx.x] = dot;
}

// W[r][j] = w1[r] - (tau/2)(w1.v) v[r] for the panel's last column (rows r > c)
template <class T>
__global__ void __launch_bounds__(256) k_trd_wlast(int64_t n, int64_t c, int j, const T *__restrict__ Vp,
                                                   T *__restrict__ Wp, const T *__restrict__ w1buf,
                                                   const T *__restrict__ dpart, int ndp, const T *__restrict__ tau) {
    __shared__ T sh[4];
    const T half = T(0.5) * tau[c] * block_sum_array(dpart, ndp, sh);
    const int64_t r = c + 1 + int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (r < n) Wp[r * NB + j] = w1buf[r] - half * Vp[r * NB + j];
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

// lam_asc[i] = i-th smallest eigenvalue of T, by 16-way multisection: a group of 16 lanes owns one
// eigenvalue; each pass the lanes count at 15 interior points of [lo, hi] and the group keeps the
// sixteenth that holds eigenvalue i (about 14 passes to full fp64 accuracy).
constexpr int MSEC = 16;
__global__ void __launch_bounds__(256) k_bisect(const double *__restrict__ d, const double *__restrict__ e2, int64_t n,
                                                const double *__restrict__ bounds, double *__restrict__ lam_asc) {
    const int64_t gid = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t i = gid / MSEC;
    const int sub = int(gid % MSEC);
    if (i >= n) return;  // whole groups leave together (n * MSEC threads rounded to blocks)
    double lo = bounds[0], hi = bounds[1];
    const double pivmin = bounds[2];
    const double atol = DBL_EPSILON * bounds[3];  // absolute accuracy eps ||T||
    for (int it = 0; it < 24; ++it) {
        if (hi - lo <= 2.0 * DBL_EPSILON * fmax(fabs(lo), fabs(hi)) + atol) break;
        const double x = sub < MSEC - 1 ? lo + (hi - lo) * double(sub + 1) / double(MSEC) : hi;
        const bool at_or_below = sub < MSEC - 1 && x > lo && x < hi && sturm_count(d, e2, n, x, pivmin) <= i;
        const bool above = sub < MSEC - 1 && x > lo && x < hi && !at_or_below;
        double nlo = at_or_below ? x : lo, nhi = above ? x : hi;
        for (int o = MSEC / 2; o > 0; o >>= 1) {
            nlo = fmax(nlo, __shfl_xor(nlo, o));
            nhi = fmin(nhi, __shfl_xor(nhi, o));
        }
        if (nlo == lo && nhi == hi) break;  // no representable point strictly inside
        lo = nlo;
        hi = nhi;
    }
    if (sub == 0) lam_asc[i] = 0.5 * (lo + hi);
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
                                              double *__restrict__ U1, double *__restrict__ U2, double *__restrict__ ML,
                                              uint8_t *__restrict__ SW) {
    const int64_t j = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (j >= nv) return;
    const double lam = lam_asc[n - 1 - j];
    const double tnorm = bounds[3];
    const double tiny = DBL_EPSILON * fmax(tnorm, DBL_MIN);
    // LU with partial pivoting of T - lam I, once: rows k of U in (U0 = 1/pivot, U1, U2), the
    // multiplier of step k in ML and whether rows k, k+1 were swapped in SW; the start vector is
    // eliminated on the way
    double u0 = d[0] - lam, u1 = n > 1 ? e[0] : 0.0, u2 = 0.0;
    double bcur = hash_unit(uint64_t(j) + 1);
    for (int64_t k = 0; k < n - 1; ++k) {
        const double l = e[k], dd = d[k + 1] - lam, ee = k + 1 < n - 1 ? e[k + 1] : 0.0;
        const double bnext = hash_unit(uint64_t(k + 1) * 0x9E3779B97F4A7C15ULL + uint64_t(j) + 1);
        double p0, p1, p2, bp, mlt;
        uint8_t sw;
        if (fabs(l) > fabs(u0)) {
            mlt = u0 / l;
            sw = 1;
            p0 = l; p1 = dd; p2 = ee; bp = bnext;
            u0 = u1 - mlt * dd; u1 = u2 - mlt * ee; bcur = bcur - mlt * bnext;
        } else {
            if (u0 == 0.0) u0 = tiny;
            mlt = l / u0;
            sw = 0;
            p0 = u0; p1 = u1; p2 = u2; bp = bcur;
            u0 = dd - mlt * u1; u1 = ee - mlt * u2; bcur = bnext - mlt * bcur;
        }
        u2 = 0.0;
        U0[k * nv + j] = 1.0 / p0;
        U1[k * nv + j] = p1;
        U2[k * nv + j] = p2;
        ML[k * nv + j] = mlt;
        SW[k * nv + j] = sw;
        Z[k * nv + j] = bp;
    }
    if (u0 == 0.0) u0 = tiny;
    U0[(n - 1) * nv + j] = 1.0 / u0;
    Z[(n - 1) * nv + j] = bcur;
    for (int iter = 0; iter < 3; ++iter) {
        if (iter > 0) {  // apply the stored elimination to the new right-hand side
            double bc = Z[j];
            for (int64_t k = 0; k < n - 1; ++k) {
                const double bn = Z[(k + 1) * nv + j], mlt = ML[k * nv + j];
                if (SW[k * nv + j]) {
                    Z[k * nv + j] = bn;
                    bc = bc - mlt * bn;
                } else {
                    Z[k * nv + j] = bc;
                    bc = bn - mlt * bc;
                }
            }
            Z[(n - 1) * nv + j] = bc;
        }
        // back substitution with U, then scale by the largest entry
        double y2 = 0.0, y1 = Z[(n - 1) * nv + j] * U0[(n - 1) * nv + j], ymax = fabs(y1);
        Z[(n - 1) * nv + j] = y1;
        for (int64_t k = n - 2; k >= 0; --k) {
            const double y = (Z[k * nv + j] - U1[k * nv + j] * y1 - U2[k * nv + j] * y2) * U0[k * nv + j];
            Z[k * nv + j] = y;
            ymax = fmax(ymax, fabs(y));
            y2 = y1;
            y1 = y;
        }
        const double inv = ymax > 0.0 ? 1.0 / ymax : 1.0;
        for (int64_t r = 0; r < n; ++r) Z[r * nv + j] *= inv;
    }
    double s2 = 0.0;
    for (int64_t r = 0; r < n; ++r) s2 += Z[r * nv + j] * Z[r * nv + j];
    const double inv = s2 > 0.0 ? 1.0 / sqrt(s2) : 0.0;
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

// G = T (sum of partials): thread (q, col) adds the partials of G[q][col] in chunk order, then
// thread (a, col) forms sum_q T[a][q] G[q][col] from LDS.  Blocks of 8 columns x NBT.
constexpr int GR_COLS = 256 / NBT;
__global__ void __launch_bounds__(256) k_bt_greduce(const double *__restrict__ Gp, int nchunk, int64_t nv,
                                                    const double *__restrict__ Tf, double *__restrict__ G) {
    __shared__ double Tm[NBT][NBT + 1];
    __shared__ double g[NBT][GR_COLS];
    for (int e = threadIdx.x; e < NBT * NBT; e += 256) Tm[e / NBT][e % NBT] = Tf[e];
    const int q = threadIdx.x / GR_COLS, cl = threadIdx.x % GR_COLS;
    const int64_t col = int64_t(blockIdx.x) * GR_COLS + cl;
    double acc = 0.0;
    if (col < nv)
        for (int k = 0; k < nchunk; ++k) acc += Gp[(int64_t(k) * NBT + q) * nv + col];
    g[q][cl] = acc;
    __syncthreads();
    double r = 0.0;
#pragma unroll 8
    for (int qq = 0; qq < NBT; ++qq) r += Tm[q][qq] * g[qq][cl];
    if (col < nv) G[int64_t(q) * nv + col] = r;
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
    T *A, *Rt, *Vp, *Wp, *tau, *colbuf, *wbuf, *w1buf, *part, *qpart, *dpart;
    double *d, *e, *e2, *bounds, *lam, *Z, *U0, *U1, *U2, *ML, *Sp, *Tf, *Gp, *G;
    uint8_t *SW;
    int *bad;
    int64_t lda;
};

static int64_t nsymv_blocks(int64_t) { return SYMV_BLOCKS; }

template <class C_, class T>
static void layout(C_ &cv, LargeWs<T> &w, int64_t n, int64_t nv, bool count_only) {
    (void)count_only;
    w.lda = (n + 63) / 64 * 64;
    const int64_t nv1 = nv > 0 ? nv : 1;
    const int64_t nch = (n + RCH - 1) / RCH;
    w.A = cv.template carve<T>(size_t(n) * size_t(w.lda));
    w.Rt = cv.template carve<T>(size_t(n) * size_t(n));
    w.Vp = cv.template carve<T>(size_t(n) * NB);
    w.Wp = cv.template carve<T>(size_t(n) * NB);
    w.tau = cv.template carve<T>(size_t(n));
    w.colbuf = cv.template carve<T>(size_t(n));
    w.w1buf = cv.template carve<T>(size_t(n));
    w.wbuf = cv.template carve<T>(size_t(n));
    w.part = cv.template carve<T>(size_t((n + 255) / 256 + 1));
    w.qpart = cv.template carve<T>(size_t(nsymv_blocks(n)) * 2 * NB);
    w.dpart = cv.template carve<T>(size_t((n + 255) / 256 + 1));
    w.d = cv.template carve<double>(size_t(n));
    w.e = cv.template carve<double>(size_t(n));
    w.e2 = cv.template carve<double>(size_t(n));
    w.bounds = cv.template carve<double>(4);
    w.lam = cv.template carve<double>(size_t(n));
    w.Z = cv.template carve<double>(size_t(n) * size_t(nv1));
    w.U0 = cv.template carve<double>(size_t(n) * size_t(nv1));
    w.U1 = cv.template carve<double>(size_t(n) * size_t(nv1));
    w.U2 = cv.template carve<double>(size_t(n) * size_t(nv1));
    w.ML = cv.template carve<double>(size_t(n) * size_t(nv1));
    w.SW = cv.template carve<uint8_t>(size_t(n) * size_t(nv1));
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
    LRC_HIP(hipFuncSetAttribute(reinterpret_cast<const void *>(k_trd_symv<T>), hipFuncAttributeMaxDynamicSharedMemorySize,
                                int(symv_smem)));
    // 1. tridiagonalisation, panels over reflector columns 0 .. n-2 (three launches per column)
    int ndp = 0;  // number of w1.v partials of the previous column
    for (int64_t p0 = 0; p0 < n - 1; p0 += NB) {
        const int64_t p1 = std::min<int64_t>(p0 + NB, n - 1);
        hipLaunchKernelGGL(k_fill_zero<T>, dim3(256), dim3(256), 0, s, w.Vp, int64_t(n) * NB);
        hipLaunchKernelGGL(k_fill_zero<T>, dim3(256), dim3(256), 0, s, w.Wp, int64_t(n) * NB);
        for (int64_t c = p0; c < p1; ++c) {
            const int j = int(c - p0);
            const int nbu = cdiv(n - c, 256);
            hipLaunchKernelGGL(k_trd_col<T>, dim3(nbu), dim3(256), 0, s, w.A, lda, n, c, j, w.Vp, w.Wp, w.w1buf,
                               w.colbuf, w.part, w.dpart, ndp, w.tau, w.d);
            const int64_t m = n - c - 1;
            const int nsb = int(std::min<int64_t>(SYMV_BLOCKS, (m + SYMV_WAVES - 1) / SYMV_WAVES));
            const int64_t kb = (c + 1) / (16 / int(sizeof(T))) * (16 / int(sizeof(T)));
            hipLaunchKernelGGL(k_trd_symv<T>, dim3(nsb), dim3(SYMV_WAVES * 64), size_t(n - kb) * sizeof(T), s, w.A, lda,
                               n, c, j, w.colbuf, w.part, nbu, w.Vp, w.Wp, w.Rt, w.wbuf, w.qpart, w.tau, w.e);
            ndp = cdiv(m, 256);
            hipLaunchKernelGGL(k_trd_w1<T>, dim3(ndp), dim3(256), 0, s, n, c, j, w.Vp, w.Wp, w.wbuf, w.qpart, nsb, w.tau,
                               w.w1buf, w.dpart);
        }
        LRC_LAUNCH_CHECK("tridiagonal panel");
        const int jn = int(p1 - p0);
        if (p1 < n - 1) {
            hipLaunchKernelGGL(k_trd_wlast<T>, dim3(cdiv(n - p1, 256)), dim3(256), 0, s, n, p1 - 1, jn - 1, w.Vp, w.Wp,
                               w.w1buf, w.dpart, ndp, w.tau);
            const int64_t m = n - p1;
            dim3 g(cdiv(m, 64), cdiv(m, 64));
            hipLaunchKernelGGL(k_trailing<T>, g, dim3(256), 0, s, w.A, lda, n, p1, jn, w.Vp, w.Wp);
            LRC_LAUNCH_CHECK("k_trailing");
        } else {  // last column: finish W[:, jn-1], update it, d[n-1]
            hipLaunchKernelGGL(k_trd_col<T>, dim3(1), dim3(256), 0, s, w.A, lda, n, n - 1, jn, w.Vp, w.Wp, w.w1buf,
                               w.colbuf, w.part, w.dpart, ndp, w.tau, w.d);
            LRC_LAUNCH_CHECK("k_trd_col");
        }
    }
    // 2. eigenvalues
    hipLaunchKernelGGL(k_tri_prep, dim3(1), dim3(256), 0, s, w.d, w.e, n, w.e2, w.bounds);
    hipLaunchKernelGGL(k_bisect, dim3(cdiv(n * MSEC, 256)), dim3(256), 0, s, w.d, w.e2, n, w.bounds, w.lam);
    hipLaunchKernelGGL(k_lambda_desc, dim3(cdiv(n, 256)), dim3(256), 0, s, w.lam, n, lambda, w.bad);
    LRC_LAUNCH_CHECK("bisection");
    if (nv > 0) {
        // 3. eigenvectors of T
        hipLaunchKernelGGL(k_invit, dim3(cdiv(nv, 64)), dim3(64), 0, s, w.d, w.e, n, w.lam, w.bounds, nv, w.Z, w.U0, w.U1,
                           w.U2, w.ML, w.SW);
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
            hipLaunchKernelGGL(k_bt_greduce, dim3(cdiv(nv, GR_COLS)), dim3(256), 0, s, w.Gp, nch, nv, w.Tf, w.G);
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
