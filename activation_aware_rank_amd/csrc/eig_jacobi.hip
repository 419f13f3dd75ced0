// Batched eigendecomposition of small symmetric positive semi-definite matrices (n <= 128),
// one matrix per workgroup, held in LDS in fp64.
//
// Swift-SVD page, section 2-ga: V and Sigma^2 of Y from one eigendecomposition of Y^T Y; the
// per-head case (WSVD page, methodology 1) has one 128 x 128 covariance per attention head.
//
// Method: one-sided (Hestenes) Jacobi on G <- C.  Column pairs (p, q) are rotated so that
// g_p^T g_q = 0.  When every pair of a sweep satisfies |g_p^T g_q| <= tol ||g_p|| ||g_q||, G = C V
// has orthogonal columns, so for PSD C G = V diag(lambda): lambda_i = ||g_i|| and
// v_i = g_i / ||g_i||, and the rotations never need to be accumulated into a second matrix.  (For
// a PSD input the computed lambda_i = ||g_i|| are non-negative; eigenvalues at rounding level below
// zero come out as their magnitude.)
//
// Ordering (block cyclic): the 128 columns (zero-padded when n < 128) form 16 blocks of 8.  A sweep
// is, first, the 28 pairs inside every block (pairs x, x ^ s for s = 1 .. 7, seven rounds), then
// 15 block rounds of the round-robin tournament of the 16 blocks; in a block round wave w takes one
// block pair (A, B) and meets every column of A with every column of B in eight inner rounds,
// column A_i with B_(i ^ s) for s in Gray-code order 0, 1, 3, 2, 6, 7, 5, 4.  Each of the 8128
// pairs comes once per sweep, and the inner rounds of a block pair need nothing from other waves:
// a sweep has 16 workgroup barriers instead of one per round (127).
//
// Work layout: 512 threads, 8 waves; a group of 8 lanes owns one pair, lane l holding elements
// 2l + 16e and 2l + 16e + 1 (e < 8) of both columns in registers (16-byte LDS accesses).  During a
// block round group i keeps column A_i and receives the next B column from the group whose index
// differs in the bit that the Gray code flips: 8 lanes away by a DPP row rotation, 16 or 32 lanes
// away by a lane permute, so LDS is read and written once per block round, not once per round.
// The dot product of a pair is summed over the group's lanes by three DPP steps (quad permutes,
// then the half-row mirror); every step adds a lane pair both ways, so the 8 lanes hold the
// bit-identical sum and rotate consistently.
//
// Rotation (block rounds): the squared column norms are formed once per block round and then
// updated with each rotation (||g_p'||^2 = ||g_p||^2 - t g_p^T g_q, ||g_q'||^2 = ||g_q||^2 +
// t g_p^T g_q), so only g_p^T g_q is summed per round.  The columns are kept as d_p x_p with a scale
// per column: the rotation [c, s; -s, c] with s = c t becomes x_p <- x_p - (t d_q / d_p) x_q,
// x_q <- x_q + (t d_p / d_q) x_p (one fused multiply-add per element) and d <- c d, and the scales are
// multiplied back in before the columns return to LDS (|t| <= 1, so a column grows at most by
// 2^(1/2) per rotation and by 16 over a block round).  t and c come from the hardware reciprocal and
// reciprocal square root estimates refined by two Newton steps each: rotation parameters a few
// units in the last place off still give a rotation orthogonal to rounding (c^2 (1 + t^2) = 1), and
// a pair left a little off orthogonal is met again in the next sweep.
#include <cfloat>

#include "lrc_internal.h"

namespace lrc {

constexpr int JAC_THREADS = 512;
constexpr int JAC_N = 128;                   // matrices are zero-padded to this order
constexpr int JAC_LD = JAC_N + 8;            // LDS column stride (doubles): 8 block columns start on 4 bank offsets
constexpr int JAC_MAX_SWEEPS = 40;
constexpr int JAC_GROUP = 8;                 // lanes per pair
constexpr int JAC_EL = JAC_N / JAC_GROUP;    // elements per lane and column
constexpr int JAC_BS = 8;                    // columns per block
constexpr int JAC_NBK = JAC_N / JAC_BS;      // blocks

// v moved across the lanes of its row of 16 by the DPP control `ctrl` (both 32-bit halves)
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
    const int lo = __builtin_amdgcn_mov_dpp(__double2loint(v), CTRL, 0xf, 0xf, false);
    const int hi = __builtin_amdgcn_mov_dpp(__double2hiint(v), CTRL, 0xf, 0xf, false);
    return __hiloint2double(hi, lo);
}
// Sum over the 8 lanes of a group (lanes 8k .. 8k + 7); every lane ends with the bit-identical total.
__device__ __forceinline__ double group8_sum(double v) {
    v += dpp_f64<0xB1>(v);   // quad_perm [1, 0, 3, 2]: lane i with i ^ 1
    v += dpp_f64<0x4E>(v);   // quad_perm [2, 3, 0, 1]: lane i with i ^ 2
    v += dpp_f64<0x141>(v);  // row_half_mirror: the two quads of each half-row
    return v;
}
// the value of lane (l ^ dist), dist in {8, 16, 32}
__device__ __forceinline__ double lane_xor(double v, int dist) {
    if (dist == 8) return dpp_f64<0x128>(v);  // row_ror:8 within a row of 16 is l ^ 8
    return __shfl_xor(v, dist);
}
// 1/x and 1/sqrt(x) from the hardware estimates and two Newton steps each
__device__ __forceinline__ double rcp_nr(double x) {
    double r = __builtin_amdgcn_rcp(x);
    double e = fma(-x, r, 1.0);
    r = fma(r, e, r);
    e = fma(-x, r, 1.0);
    return fma(r, e, r);
}
__device__ __forceinline__ double rsq_nr(double x) {
    double r = __builtin_amdgcn_rsq(x);
    double h = 0.5 * x * r;
    r = fma(r, fma(-h, r, 0.5), r);
    h = 0.5 * x * r;
    return fma(r, fma(-h, r, 0.5), r);
}

template <class T>
__device__ __forceinline__ T wave_sum(T v) {
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

__global__ void __launch_bounds__(JAC_THREADS) k_jacobi(const float *__restrict__ C, int n, int64_t ldc, int64_t stride_c,
                                                        double *__restrict__ lambda, float *__restrict__ V, int64_t ldv,
                                                        int n_vec, int64_t stride_v, int32_t *__restrict__ info) {
    extern __shared__ __attribute__((aligned(16))) char smem[];
    double *G = reinterpret_cast<double *>(smem);  // column-major: column p at G + p * JAC_LD
    double *nrm = G + JAC_N * JAC_LD;              // column norms
    int *rank = reinterpret_cast<int *>(nrm + JAC_N);  // output position of column i
    __shared__ int s_flag[2], s_bad;
    const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int grp = lane / JAC_GROUP, gl = lane % JAC_GROUP;
    constexpr int nwaves = JAC_THREADS / 64;
    const float *Cb = C + int64_t(b) * stride_c;
    if (tid == 0) s_bad = 0;
    if (tid < 2) s_flag[tid] = 0;
    __syncthreads();
    for (int e = tid; e < JAC_N * JAC_N; e += JAC_THREADS) {
        const int p = e / JAC_N, i = e % JAC_N;  // G[p][i] = C(i, p), upper triangle read
        float v = 0.f;
        if (p < n && i < n) {
            v = i <= p ? Cb[int64_t(i) * ldc + p] : Cb[int64_t(p) * ldc + i];
            if (!isfinite(v)) s_bad = 1;
        }
        G[p * JAC_LD + i] = double(v);
    }
    __syncthreads();
    const bool bad = s_bad != 0;
    const double tol = double(n) * DBL_EPSILON, tol2 = tol * tol;
    auto load = [&](int col, double (&x)[JAC_EL]) {
        const double *base = G + col * JAC_LD + 2 * gl;
#pragma unroll
        for (int e = 0; e < JAC_EL / 2; ++e) {
            const double2 v = *reinterpret_cast<const double2 *>(base + 2 * JAC_GROUP * e);
            x[2 * e] = v.x;
            x[2 * e + 1] = v.y;
        }
    };
    auto store = [&](int col, const double (&x)[JAC_EL]) {
        double *base = G + col * JAC_LD + 2 * gl;
#pragma unroll
        for (int e = 0; e < JAC_EL / 2; ++e) {
            double2 v;
            v.x = x[2 * e];
            v.y = x[2 * e + 1];
            *reinterpret_cast<double2 *>(base + 2 * JAC_GROUP * e) = v;
        }
    };
    auto dot = [&](const double (&x)[JAC_EL], const double (&y)[JAC_EL]) {
        double s0 = 0.0, s1 = 0.0, s2 = 0.0, s3 = 0.0;
#pragma unroll
        for (int e = 0; e < JAC_EL; e += 4) {
            s0 = fma(x[e], y[e], s0);
            s1 = fma(x[e + 1], y[e + 1], s1);
            s2 = fma(x[e + 2], y[e + 2], s2);
            s3 = fma(x[e + 3], y[e + 3], s3);
        }
        return group8_sum((s0 + s1) + (s2 + s3));
    };
    // whether the pair with squared norms al, be and product ga is rotated
    auto needs = [&](double al, double be, double ga) { return ga != 0.0 && ga * ga > tol2 * (al * be); };
    // t = tan(theta) of the rotation zeroing the pair's product (the root of t^2 + 2 zeta t = 1 of
    // smaller magnitude, zeta = (be - al) / (2 ga)), 0 when the pair is not rotated
    auto tangent = [&](bool rot, double al, double be, double ga) {
        const double zeta = (be - al) * rcp_nr(2.0 * (rot ? ga : 1.0));
        const double y = fma(zeta, zeta, 1.0);
        return rot ? copysign(rcp_nr(fabs(zeta) + y * rsq_nr(y)), zeta) : 0.0;
    };
    int converged = bad ? 1 : 0;
    for (int sweep = 0; sweep < JAC_MAX_SWEEPS && !converged; ++sweep) {
        bool rotated = false;
        // s_flag[sweep & 1] was last read two sweeps ago, before at least 16 barriers
        if (tid == 0) s_flag[sweep & 1] = 0;
        // pairs inside the blocks 2 wave and 2 wave + 1: (x, x ^ s) for x without the top bit of s;
        // rounds of one wave only, through LDS
        for (int s = 1; s < JAC_BS; ++s) {
            const int hb = 31 - __builtin_clz(s);
            const int lo = grp & (JAC_BS / 2 - 1);
            const int x = ((lo >> hb) << (hb + 1)) | (lo & ((1 << hb) - 1));
            const int blk = 2 * wave + grp / (JAC_BS / 2);
            const int p = blk * JAC_BS + x, q = blk * JAC_BS + (x ^ s);
            double gp[JAC_EL], gq[JAC_EL];
            load(p, gp);
            load(q, gq);
            const double al = dot(gp, gp), be = dot(gq, gq), ga = dot(gp, gq);
            if (needs(al, be, ga)) {
                rotated = true;
                const double t = tangent(true, al, be, ga);
                const double c = rsq_nr(fma(t, t, 1.0)), sn = c * t;
#pragma unroll
                for (int e = 0; e < JAC_EL; ++e) {
                    const double xe = gp[e], ye = gq[e];
                    gp[e] = c * xe - sn * ye;
                    gq[e] = sn * xe + c * ye;
                }
                store(p, gp);
                store(q, gq);
            }
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
            __builtin_amdgcn_wave_barrier();
        }
        __syncthreads();
        for (int R = 0; R < JAC_NBK - 1; ++R) {
            int A, B;  // block pair of this wave in round R of the tournament
            if (wave == 0) {
                A = R;
                B = JAC_NBK - 1;
            } else {
                A = (R + wave) % (JAC_NBK - 1);
                B = (R - wave + JAC_NBK - 1) % (JAC_NBK - 1);
            }
            double xa[JAC_EL], xb[JAC_EL];
            load(A * JAC_BS + grp, xa);
            load(B * JAC_BS + grp, xb);
            double al = dot(xa, xa), be = dot(xb, xb);
            double da = 1.0, ida = 1.0, db = 1.0, idb = 1.0;  // scales and their inverses
#pragma unroll
            for (int k = 0; k < JAC_BS; ++k) {
                // every group computes a rotation; t = 0 (c = 1) leaves the pair exactly as it is
                const double ga = da * db * dot(xa, xb);
                const bool rot = needs(al, be, ga);
                rotated |= rot;
                const double t = tangent(rot, al, be, ga);
                const double u = fma(t, t, 1.0);
                const double c = rsq_nr(u);
                const double ta = t * db * ida, tb = t * da * idb;
#pragma unroll
                for (int e = 0; e < JAC_EL; ++e) {
                    const double xe = xa[e], ye = xb[e];
                    xa[e] = fma(-ta, ye, xe);
                    xb[e] = fma(tb, xe, ye);
                }
                const double ic = u * c;  // 1 / c
                da *= c;
                db *= c;
                ida *= ic;
                idb *= ic;
                al = fma(-t, ga, al);
                be = fma(t, ga, be);
                if (k < JAC_BS - 1) {  // the B column of the next inner round, with its state
                    const int dist = JAC_GROUP * ((k ^ (k >> 1)) ^ ((k + 1) ^ ((k + 1) >> 1)));
#pragma unroll
                    for (int e = 0; e < JAC_EL; ++e) xb[e] = lane_xor(xb[e], dist);
                    be = lane_xor(be, dist);
                    db = lane_xor(db, dist);
                    idb = lane_xor(idb, dist);
                }
            }
            constexpr int LAST = (JAC_BS - 1) ^ ((JAC_BS - 1) >> 1);  // group i ends with B_(i ^ LAST)
#pragma unroll
            for (int e = 0; e < JAC_EL; ++e) {
                xa[e] *= da;
                xb[e] *= db;
            }
            store(A * JAC_BS + grp, xa);
            store(B * JAC_BS + (grp ^ LAST), xb);
            if (R == JAC_NBK - 2 && rotated && gl == 0) s_flag[sweep & 1] = 1;
            __syncthreads();
        }
        converged = s_flag[sweep & 1] == 0;
    }
    // norms, ranks (descending, ties by index), outputs; columns n .. 127 are zero
    for (int i = wave; i < n; i += nwaves) {
        const double x0 = G[i * JAC_LD + lane], x1 = G[i * JAC_LD + lane + 64];
        const double s2 = wave_sum(x0 * x0 + x1 * x1);
        if (lane == 0) nrm[i] = sqrt(s2);
    }
    __syncthreads();
    for (int i = tid; i < n; i += JAC_THREADS) {
        const double ni = nrm[i];
        int rk = 0;
        for (int j = 0; j < n; ++j) rk += (nrm[j] > ni) || (nrm[j] == ni && j < i);
        rank[i] = rk;
        lambda[int64_t(b) * n + rk] = bad ? double(NAN) : ni;
    }
    __syncthreads();
    for (int i = wave; i < n; i += nwaves) {
        const int j = rank[i];
        if (j >= n_vec) continue;
        const double ni = nrm[i];
        const double inv = ni > 0.0 ? 1.0 / ni : 0.0;
        // sign: entry of largest magnitude positive, first index on ties
        double best = -1.0;
        int bi = n;
        for (int k = lane; k < n; k += 64) {
            const double a = fabs(G[i * JAC_LD + k]);
            if (a > best) {
                best = a;
                bi = k;
            }
        }
        for (int o = 32; o > 0; o >>= 1) {
            const double ob = __shfl_xor(best, o);
            const int oi = __shfl_xor(bi, o);
            if (ob > best || (ob == best && oi < bi)) {
                best = ob;
                bi = oi;
            }
        }
        const double sgn = (bi < n && G[i * JAC_LD + bi] < 0.0) ? -1.0 : 1.0;
        float *Vb = V + int64_t(b) * stride_v;
        for (int k = lane; k < n; k += 64) {
            const double v = ni > 0.0 ? G[i * JAC_LD + k] * inv * sgn : (k == i ? 1.0 : 0.0);
            Vb[int64_t(k) * ldv + j] = float(v);
        }
    }
    if (tid == 0) info[b] = bad ? LRC_INFO_NONFINITE : (converged ? LRC_INFO_OK : LRC_INFO_NO_CONVERGENCE);
}

static size_t jac_smem() {
    return size_t(JAC_N) * JAC_LD * sizeof(double) + JAC_N * sizeof(double) + JAC_N * sizeof(int) + 16;
}

size_t jacobi_workspace(int64_t, int64_t, lrc_dtype) { return 0; }

lrc_status jacobi_run(const EighArgs &a, void *, size_t, hipStream_t s) {
    if (a.n > JAC_N) return fail(LRC_ERR_ARG, "jacobi path needs n <= 128");
    if (a.batch > 65535 * 64) return fail(LRC_ERR_ARG, "batch too large");
    // Always fp64, whatever the requested working precision: a 128 x 128 fp64 matrix (136 KiB with
    // the padded columns) fits in LDS, and fp32 sweeps stop at a pair tolerance (n FLT_EPSILON) that
    // leaves retained subspaces of the per-head matrices only a few times inside 1e-3 rad.
    const size_t sm = jac_smem();
    LRC_HIP(hipFuncSetAttribute(reinterpret_cast<const void *>(k_jacobi), hipFuncAttributeMaxDynamicSharedMemorySize,
                                int(sm)));
    hipLaunchKernelGGL(k_jacobi, dim3(unsigned(a.batch)), dim3(JAC_THREADS), sm, s, a.C, int(a.n), a.ldc, a.stride_c,
                       a.lambda, a.V, a.ldv, int(a.n_vec), a.stride_v, a.info);
    LRC_LAUNCH_CHECK("k_jacobi");
    return LRC_OK;
}

}  // namespace lrc
