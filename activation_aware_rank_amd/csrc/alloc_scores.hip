// Two more ways to turn per-layer or per-component scores into ranks.
//
//  * Swift-SVD page, section 2-na (dynamic rank allocation), steps 1-2: the score of matrix i is
//    s_i = beta_i^alpha * log(e + eps_{kbar,i})^(1 - alpha), from its importance beta_i and its
//    closed-form error at the uniform rank kbar_i; every matrix keeps at least floor(kbar_i delta);
//    one candidate allocation per alpha of a grid.  The rule that turns scores into ranks is not
//    printed; here the parameters left after the minima are split in proportion to the scores,
//    floor(share / cost_i) ranks each, capped at k_cap_i, a capped matrix's excess split again
//    among the others (water filling).
//  * LASER page, method 2 (empirical-Fisher importance score): the score of component i of a
//    matrix is <G, W v_i v_i^T>^2 = ((W v_i) . (G v_i))^2, the empirical-Fisher loss of removing
//    it; two fp64 MFMA products W V_k and G V_k with the column dot products in the epilogue.  The
//    greedy scan over these scores is k_allocate<1> (small_ops.hip).
#include <cmath>

#include "lrc_internal.h"

#pragma clang fp contract(off)

namespace lrc {

// ---------------------------------------------------------------------------------------------
// Swift-SVD candidates: one workgroup per alpha, one thread per matrix.  Sums of scores are taken
// in index order by one thread and every rank decision uses the same fp64 operations as a
// sequential evaluation, so the result is bit-exact given the same scores.
// ---------------------------------------------------------------------------------------------
constexpr int SWF_MAX = 1024;

__global__ void __launch_bounds__(SWF_MAX) k_alloc_swift(int32_t n, const double *__restrict__ beta,
                                                         const double *__restrict__ eps_kbar,
                                                         const int64_t *__restrict__ kbar, const int64_t *__restrict__ cost,
                                                         const int64_t *__restrict__ k_cap, double delta,
                                                         const double *__restrict__ alpha_grid, int64_t budget,
                                                         double *__restrict__ scores, int32_t *__restrict__ k_out,
                                                         int32_t *__restrict__ info) {
    __shared__ double s_sh[SWF_MAX];
    __shared__ long long kmin_sh[SWF_MAX], x_sh[SWF_MAX], cost_sh[SWF_MAX], cap_sh[SWF_MAX];
    __shared__ int open_sh[SWF_MAX], capped_sh[SWF_MAX];
    __shared__ int bad_sh, any_capped;
    __shared__ double S_sh;
    __shared__ long long mand_sh, committed_sh;
    const int m = threadIdx.x, a = blockIdx.x;
    const double alpha = alpha_grid[a];
    if (m == 0) bad_sh = (alpha >= 0.0 && alpha <= 1.0 && delta >= 0.0 && delta <= 1.0) ? 0 : 1;
    __syncthreads();
    if (m < n) {
        const double b = beta[m], e = eps_kbar[m];
        const int64_t kb = kbar[m], c = cost[m], cap = k_cap[m];
        const double L = log(M_E + (isnan(e) ? e : e > 0.0 ? e : 0.0));  // a NaN error makes the score NaN
        // the grid's end points exactly: x^1 = x and x^0 = 1 (the device pow may round x^1)
        const double pb = alpha == 1.0 ? b : alpha == 0.0 ? 1.0 : pow(b, alpha);
        const double pl = alpha == 0.0 ? L : alpha == 1.0 ? 1.0 : pow(L, 1.0 - alpha);
        const double sc = pb * pl;
        if (!(sc >= 0.0 && sc <= 1.7976931348623157e308) || c <= 0 || kb < 0 || kb > cap) atomicOr(&bad_sh, 1);
        s_sh[m] = sc;
        scores[int64_t(a) * n + m] = sc;
        kmin_sh[m] = (long long)floor(double(kb) * delta);
        x_sh[m] = 0;
        cost_sh[m] = c;
        cap_sh[m] = cap;
        open_sh[m] = kmin_sh[m] < cap ? 1 : 0;
    }
    __syncthreads();
    int32_t *ko = k_out + int64_t(a) * n;
    if (bad_sh) {
        if (m < n) ko[m] = 0;
        if (m == 0) info[a] = LRC_INFO_BAD_SCORE;
        return;
    }
    if (m == 0) {
        long long mand = 0;
        for (int i = 0; i < n; ++i) mand += kmin_sh[i] * cost_sh[i];
        mand_sh = mand;
        committed_sh = 0;
    }
    __syncthreads();
    if (mand_sh > budget) {
        if (m < n) ko[m] = int32_t(kmin_sh[m]);
        if (m == 0) info[a] = LRC_INFO_BUDGET;
        return;
    }
    const long long E = budget - mand_sh;
    for (int round = 0; round <= n; ++round) {  // every round but the last closes at least one matrix
        if (m == 0) {
            double S = 0.0;
            for (int i = 0; i < n; ++i)
                if (open_sh[i]) S = S + s_sh[i];
            S_sh = S;
            any_capped = 0;
        }
        __syncthreads();
        const double S = S_sh;
        if (!(S > 0.0)) break;  // nothing open, or only zero scores: no more ranks
        const double R = double(E - committed_sh);
        long long q = 0;
        if (m < n && open_sh[m]) {
            q = (long long)floor(((s_sh[m] * R) / S) / double(cost_sh[m]));
            capped_sh[m] = kmin_sh[m] + q >= cap_sh[m] ? 1 : 0;
            if (capped_sh[m]) any_capped = 1;
        } else if (m < n) {
            capped_sh[m] = 0;
        }
        __syncthreads();
        if (!any_capped) {
            if (m < n && open_sh[m]) x_sh[m] = q;
            __syncthreads();
            break;
        }
        if (m < n && capped_sh[m]) {
            x_sh[m] = cap_sh[m] - kmin_sh[m];
            open_sh[m] = 0;
        }
        __syncthreads();
        if (m == 0) {
            long long c = 0;
            for (int i = 0; i < n; ++i)
                if (capped_sh[i]) c += x_sh[i] * cost_sh[i];
            committed_sh += c;
        }
        __syncthreads();
    }
    if (m == 0) {  // rounding can in principle overshoot by a rank: the last open matrices give back
        long long tot = 0;
        for (int i = 0; i < n; ++i) tot += (kmin_sh[i] + x_sh[i]) * cost_sh[i];
        for (int i = n - 1; i >= 0 && tot > budget;) {
            if (open_sh[i] && x_sh[i] > 0) {
                --x_sh[i];
                tot -= cost_sh[i];
            } else {
                --i;
            }
        }
    }
    __syncthreads();
    if (m < n) ko[m] = int32_t(kmin_sh[m] + x_sh[m]);
    if (m == 0) info[a] = LRC_INFO_OK;
}

lrc_status alloc_swift_run(int32_t n, const double *beta, const double *eps_kbar, const int64_t *kbar,
                           const int64_t *cost, const int64_t *k_cap, double delta, int32_t n_alpha,
                           const double *alpha_grid, int64_t budget, double *scores, int32_t *k_out, int32_t *info,
                           hipStream_t s) {
    hipLaunchKernelGGL(k_alloc_swift, dim3(unsigned(n_alpha)), dim3(SWF_MAX), 0, s, n, beta, eps_kbar, kbar, cost,
                       k_cap, delta, alpha_grid, budget, scores, k_out, info);
    LRC_LAUNCH_CHECK("k_alloc_swift");
    return LRC_OK;
}

// ---------------------------------------------------------------------------------------------
// Per-component empirical-Fisher scores.  A workgroup takes 64 rows of W and G and 64 components:
// P = W_rows V and Q = G_rows V on 16x16x4 fp64 MFMA (inputs widened exactly, staged k-major in
// LDS, next step loaded during the current one), then sum_rows P .* Q per component, reduced in a
// fixed order (in-lane rows, then lanes, then the two row halves) to one fp64 partial per row tile.
// A second kernel adds a component's partials in row-tile order and squares the sum.
// ---------------------------------------------------------------------------------------------
constexpr int CF_T = 64;
constexpr int CF_K = 16;
constexpr int CF_LD = CF_T + 16;

template <class T>
__device__ __forceinline__ double cf_load(const T *p, int64_t i);
template <>
__device__ __forceinline__ double cf_load<bf16_t>(const bf16_t *p, int64_t i) { return double(bf16_to_f32(p[i])); }
template <>
__device__ __forceinline__ double cf_load<float>(const float *p, int64_t i) { return double(p[i]); }

template <class T>
__global__ void __launch_bounds__(256) k_comp_fisher(const T *__restrict__ W, const T *__restrict__ G, int64_t ldw,
                                                     int64_t ldg, int64_t d_in, int64_t d_out,
                                                     const float *__restrict__ V, int64_t ldv, int64_t k,
                                                     int64_t stride_w, int64_t stride_g, int64_t stride_v,
                                                     double *__restrict__ partials) {
    __shared__ double Ws[CF_K][CF_LD];
    __shared__ double Gs[CF_K][CF_LD];
    __shared__ double Vs[CF_K][CF_LD];
    __shared__ double half_sh[2][CF_T];
    const int64_t b = blockIdx.z;
    W += b * stride_w;
    G += b * stride_g;
    V += b * stride_v;
    const int64_t i0 = int64_t(blockIdx.y) * CF_T, j0 = int64_t(blockIdx.x) * CF_T;
    const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
    const int wr = (wv >> 1) * 32, wc = (wv & 1) * 32;
    double rw[4], rg[4], rv[4];
    auto gload = [&](int64_t r0) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int ii = t >> 2, rr = (t & 3) * 4 + u;  // W[i][r], contiguous in r
            const int64_t r = r0 + rr, i = i0 + ii;
            const bool in = r < d_out && i < d_in;
            rw[u] = in ? cf_load(W, i * ldw + r) : 0.0;
            rg[u] = in ? cf_load(G, i * ldg + r) : 0.0;
            const int vr = t >> 4, vj = (t & 15) * 4 + u;
            const int64_t rvv = r0 + vr, jj = j0 + vj;
            rv[u] = (rvv < d_out && jj < k) ? double(V[rvv * ldv + jj]) : 0.0;
        }
    };
    auto sstore = [&]() {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            Ws[(t & 3) * 4 + u][t >> 2] = rw[u];
            Gs[(t & 3) * 4 + u][t >> 2] = rg[u];
            Vs[t >> 4][(t & 15) * 4 + u] = rv[u];
        }
    };
    f64x4_t aw[2][2], ag[2][2];
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int y = 0; y < 2; ++y) {
            aw[x][y] = f64x4_t{0.0, 0.0, 0.0, 0.0};
            ag[x][y] = f64x4_t{0.0, 0.0, 0.0, 0.0};
        }
    gload(0);
    for (int64_t r0 = 0; r0 < d_out; r0 += CF_K) {
        sstore();
        __syncthreads();
        if (r0 + CF_K < d_out) gload(r0 + CF_K);
#pragma unroll
        for (int ks = 0; ks < CF_K / 4; ++ks) {
            const int kk = ks * 4 + (lane >> 4);
            const double w0 = Ws[kk][wr + (lane & 15)], w1 = Ws[kk][wr + 16 + (lane & 15)];
            const double g0 = Gs[kk][wr + (lane & 15)], g1 = Gs[kk][wr + 16 + (lane & 15)];
            const double v0 = Vs[kk][wc + (lane & 15)], v1 = Vs[kk][wc + 16 + (lane & 15)];
            aw[0][0] = __builtin_amdgcn_mfma_f64_16x16x4f64(w0, v0, aw[0][0], 0, 0, 0);
            aw[0][1] = __builtin_amdgcn_mfma_f64_16x16x4f64(w0, v1, aw[0][1], 0, 0, 0);
            aw[1][0] = __builtin_amdgcn_mfma_f64_16x16x4f64(w1, v0, aw[1][0], 0, 0, 0);
            aw[1][1] = __builtin_amdgcn_mfma_f64_16x16x4f64(w1, v1, aw[1][1], 0, 0, 0);
            ag[0][0] = __builtin_amdgcn_mfma_f64_16x16x4f64(g0, v0, ag[0][0], 0, 0, 0);
            ag[0][1] = __builtin_amdgcn_mfma_f64_16x16x4f64(g0, v1, ag[0][1], 0, 0, 0);
            ag[1][0] = __builtin_amdgcn_mfma_f64_16x16x4f64(g1, v0, ag[1][0], 0, 0, 0);
            ag[1][1] = __builtin_amdgcn_mfma_f64_16x16x4f64(g1, v1, ag[1][1], 0, 0, 0);
        }
        __syncthreads();
    }
    // accumulator r of a lane holds row 4 r + lane / 16, column lane % 16 of its 16x16 tile; rows
    // past d_in and columns past k hold zeros (their operands were zero)
#pragma unroll
    for (int y = 0; y < 2; ++y) {
        double d = 0.0;
#pragma unroll
        for (int x = 0; x < 2; ++x)
#pragma unroll
            for (int r = 0; r < 4; ++r) d = d + aw[x][y][r] * ag[x][y][r];
        d = d + __shfl_xor(d, 16);
        d = d + __shfl_xor(d, 32);
        if (lane < 16) half_sh[wr / 32][wc + y * 16 + lane] = d;
    }
    __syncthreads();
    if (t < CF_T) {
        const int64_t j = j0 + t;
        if (j < k) partials[(b * gridDim.y + blockIdx.y) * k + j] = half_sh[0][t] + half_sh[1][t];
    }
}

__global__ void k_comp_fisher_final(const double *__restrict__ partials, int64_t n_tiles, int64_t k, int64_t batch,
                                    double *__restrict__ score, int64_t stride_s) {
    const int64_t e = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (e >= batch * k) return;
    const int64_t b = e / k, j = e % k;
    double acc = 0.0;
    for (int64_t tile = 0; tile < n_tiles; ++tile) acc = acc + partials[(b * n_tiles + tile) * k + j];
    score[b * stride_s + j] = acc * acc;
}

size_t comp_fisher_workspace(int64_t d_in, int64_t k, int64_t batch) {
    Counter c;
    c.carve<double>(size_t(cdiv(d_in, CF_T)) * size_t(k) * size_t(batch));
    return c.off;
}

lrc_status comp_fisher_run(const CompFisherArgs &a, void *ws, size_t ws_bytes, hipStream_t s) {
    if (a.batch > 65535) return fail(LRC_ERR_ARG, "batch too large");
    const int64_t n_tiles = cdiv(a.d_in, CF_T);
    if (n_tiles > 65535) return fail(LRC_ERR_ARG, "d_in too large");
    Carver cv(ws, ws_bytes);
    double *partials = cv.carve<double>(size_t(n_tiles) * size_t(a.k) * size_t(a.batch));
    if (!partials) return fail(LRC_ERR_WORKSPACE, "component score workspace too small");
    dim3 g(cdiv(a.k, CF_T), unsigned(n_tiles), unsigned(a.batch));
    if (a.t == LRC_BF16)
        hipLaunchKernelGGL(k_comp_fisher<bf16_t>, g, dim3(256), 0, s, static_cast<const bf16_t *>(a.W),
                           static_cast<const bf16_t *>(a.G), a.ldw, a.ldg, a.d_in, a.d_out, a.V, a.ldv, a.k,
                           a.stride_w, a.stride_g, a.stride_v, partials);
    else
        hipLaunchKernelGGL(k_comp_fisher<float>, g, dim3(256), 0, s, static_cast<const float *>(a.W),
                           static_cast<const float *>(a.G), a.ldw, a.ldg, a.d_in, a.d_out, a.V, a.ldv, a.k,
                           a.stride_w, a.stride_g, a.stride_v, partials);
    LRC_LAUNCH_CHECK("k_comp_fisher");
    const int64_t total = a.batch * a.k;
    hipLaunchKernelGGL(k_comp_fisher_final, dim3(cdiv(total, 256)), dim3(256), 0, s, partials, n_tiles, a.k, a.batch,
                       a.score, a.stride_s);
    LRC_LAUNCH_CHECK("k_comp_fisher_final");
    return LRC_OK;
}

}  // namespace lrc
