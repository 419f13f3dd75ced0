// Error curve, Fisher importance and greedy rank allocation.
//
//  * error curve: Swift-SVD page, section 2-ga (closed-form minimal error eps*_k = sum of the
//    eigenvalues beyond k).
//  * Fisher importance: FLRC page, method 1 (alpha_{l,p} = sum_i (G[i] W[i])^2).
//  * greedy allocation: LASER page, method 2 (take components of highest importance per
//    parameter until the budget is reached), Swift-SVD page, section 2-na (minimum rank); the
//    same scan over per-component empirical-Fisher scores (LASER page, method 2).
#include <cmath>
#include <algorithm>
#include <cstring>
#include <mutex>

#include "lrc_internal.h"

#pragma clang fp contract(off)

namespace lrc {

// ---------------------------------------------------------------------------------------------
// error curve: one thread per matrix, summed from the smallest eigenvalue (fixed order).  The
// values come in blocks of ECB, the next block's loads issued before the current block's adds, so the
// chain of dependent adds does not wait for memory at every step.
// ---------------------------------------------------------------------------------------------
constexpr int ECB = 32;
__global__ void k_error_curve(const double *__restrict__ lam, int64_t n, int64_t batch, double *__restrict__ eps) {
    int64_t b = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (b >= batch) return;
    const double *l = lam + b * n;
    double *e = eps + b * (n + 1);
    double acc = 0.0;
    e[n] = 0.0;
    // block q holds l[k] for k = n - 1 - q ECB - i, i = 0 .. ECB - 1 (those >= 0)
    double cur[ECB], nxt[ECB];
#pragma unroll
    for (int i = 0; i < ECB; ++i) cur[i] = n - 1 - i >= 0 ? l[n - 1 - i] : 0.0;
    for (int64_t k0 = n - 1; k0 >= 0; k0 -= ECB) {
        const int64_t k1 = k0 - ECB;  // first index of the next block
#pragma unroll
        for (int i = 0; i < ECB; ++i) nxt[i] = k1 - i >= 0 ? l[k1 - i] : 0.0;
#pragma unroll
        for (int i = 0; i < ECB; ++i) {
            if (k0 - i >= 0) {
                acc = acc + cur[i];
                e[k0 - i] = acc;
            }
        }
#pragma unroll
        for (int i = 0; i < ECB; ++i) cur[i] = nxt[i];
    }
}

lrc_status error_curve_run(const double *lambda, int64_t n, int64_t batch, double *eps, hipStream_t s) {
    hipLaunchKernelGGL(k_error_curve, dim3(cdiv(batch, 64)), dim3(64), 0, s, lambda, n, batch, eps);
    LRC_LAUNCH_CHECK("k_error_curve");
    return LRC_OK;
}

// ---------------------------------------------------------------------------------------------
// Fisher scores: HBM-bound streaming reduction.  Each block reduces FSH_PER_BLOCK contiguous
// elements of one matrix to an fp64 partial; a second kernel adds each matrix's partials in
// index order.  Products are formed in fp64 (exact for bf16 and fp32 inputs), squared in fp64.
// ---------------------------------------------------------------------------------------------
constexpr int FSH_THREADS = 256;
constexpr int FSH_VEC = 8;     // elements per 16-byte bf16 load
constexpr int FSH_ITERS = 16;  // vector loads per thread per block
constexpr int64_t FSH_PER_BLOCK = int64_t(FSH_THREADS) * FSH_VEC * FSH_ITERS;  // 32768
constexpr int FSH_GROUP = 64;  // matrices per launch (kernel arguments by value)

struct FisherGroup {
    const void *g[FSH_GROUP];
    const void *w[FSH_GROUP];
    int64_t numel[FSH_GROUP];
    int64_t block_start[FSH_GROUP + 1];  // first block of each matrix (relative to group)
    int64_t partial_base;                // index of the group's first partial
    int32_t n;
    int32_t vec_ok[FSH_GROUP];  // 16-byte aligned (bf16) / 16-byte aligned (f32)
};

__device__ __forceinline__ double block_sum_f64(double v, double *sh) {
    // fixed-order reduction: wave shuffle tree, then the waves' results in order
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    __syncthreads();
    if (lane == 0) sh[wid] = v;
    __syncthreads();
    double r = 0.0;
    if (threadIdx.x == 0)
        for (int i = 0; i < int(blockDim.x >> 6); ++i) r += sh[i];
    return r;  // valid in thread 0
}

template <bool BF16>
__global__ void __launch_bounds__(FSH_THREADS) k_fisher_partial(FisherGroup grp, double *__restrict__ partials) {
    __shared__ double sh[FSH_THREADS / 64];
    const int64_t blk = blockIdx.x;
    int m = 0;
    while (m + 1 < grp.n && grp.block_start[m + 1] <= blk) ++m;
    const int64_t e0 = (blk - grp.block_start[m]) * FSH_PER_BLOCK;
    const int64_t e1 = min(e0 + FSH_PER_BLOCK, grp.numel[m]);
    double acc = 0.0;
    if (BF16) {
        const bf16_t *G = static_cast<const bf16_t *>(grp.g[m]);
        const bf16_t *W = static_cast<const bf16_t *>(grp.w[m]);
        if (grp.vec_ok[m] && e1 - e0 == FSH_PER_BLOCK) {
            const u32x4_t *G4 = reinterpret_cast<const u32x4_t *>(G + e0);
            const u32x4_t *W4 = reinterpret_cast<const u32x4_t *>(W + e0);
            u32x4_t gv[FSH_ITERS], wv[FSH_ITERS];
#pragma unroll
            for (int it = 0; it < FSH_ITERS; ++it) {
                gv[it] = __builtin_nontemporal_load(G4 + it * FSH_THREADS + threadIdx.x);
                wv[it] = __builtin_nontemporal_load(W4 + it * FSH_THREADS + threadIdx.x);
            }
#pragma unroll
            for (int it = 0; it < FSH_ITERS; ++it) {
                const uint32_t ga[4] = {gv[it].x, gv[it].y, gv[it].z, gv[it].w};
                const uint32_t wa[4] = {wv[it].x, wv[it].y, wv[it].z, wv[it].w};
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    double p0 = double(__uint_as_float(ga[q] << 16)) * double(__uint_as_float(wa[q] << 16));
                    double p1 = double(__uint_as_float(ga[q] & 0xffff0000u)) *
                                double(__uint_as_float(wa[q] & 0xffff0000u));
                    acc = acc + p0 * p0;
                    acc = acc + p1 * p1;
                }
            }
        } else {
            for (int64_t e = e0 + threadIdx.x; e < e1; e += FSH_THREADS) {
                double p = double(bf16_to_f32(G[e])) * double(bf16_to_f32(W[e]));
                acc = acc + p * p;
            }
        }
    } else {
        const float *G = static_cast<const float *>(grp.g[m]);
        const float *W = static_cast<const float *>(grp.w[m]);
        for (int64_t e = e0 + threadIdx.x; e < e1; e += FSH_THREADS) {
            double p = double(G[e]) * double(W[e]);
            acc = acc + p * p;
        }
    }
    double tot = block_sum_f64(acc, sh);
    if (threadIdx.x == 0) partials[grp.partial_base + blk] = tot;
}

// one block per matrix of a group: add its partials in index order (strided per thread, then a
// fixed tree)
struct FisherFinal {
    int64_t pstart[FSH_GROUP + 1];  // absolute partial index range of each matrix
    int32_t m0, n;
};

__global__ void __launch_bounds__(256) k_fisher_final(const double *__restrict__ partials, FisherFinal f,
                                                      double *__restrict__ alpha, int32_t *__restrict__ info) {
    __shared__ double sh[4];
    const int i = blockIdx.x;
    if (i >= f.n) return;
    const int64_t p0 = f.pstart[i], p1 = f.pstart[i + 1];
    double acc = 0.0;
    for (int64_t q = p0 + threadIdx.x; q < p1; q += 256) acc = acc + partials[q];
    double tot = block_sum_f64(acc, sh);
    if (threadIdx.x == 0) {
        alpha[f.m0 + i] = tot;
        info[f.m0 + i] = isfinite(tot) ? LRC_INFO_OK : LRC_INFO_NONFINITE;
    }
}

static int64_t fisher_blocks(int64_t numel) { return (numel + FSH_PER_BLOCK - 1) / FSH_PER_BLOCK; }

size_t fisher_workspace(int32_t n_mats, const int64_t *numel) {
    int64_t nb = 0;
    for (int i = 0; i < n_mats; ++i) nb += fisher_blocks(numel[i]);
    Counter c;
    c.carve<double>(size_t(nb > 0 ? nb : 1));
    return c.off;
}

lrc_status fisher_run(int32_t n_mats, const void *const *G, const void *const *W, const int64_t *numel,
                      lrc_dtype t, double *alpha, void *ws, size_t ws_bytes, int32_t *info, hipStream_t s) {
    int64_t nb_total = 0;
    for (int i = 0; i < n_mats; ++i) nb_total += fisher_blocks(numel[i]);
    Carver cv(ws, ws_bytes);
    double *partials = cv.carve<double>(size_t(nb_total > 0 ? nb_total : 1));
    if (!partials) return fail(LRC_ERR_WORKSPACE, "fisher workspace too small");
    int64_t base = 0;
    for (int g0 = 0; g0 < n_mats; g0 += FSH_GROUP) {
        FisherGroup grp;
        FisherFinal fin;
        memset(&grp, 0, sizeof(grp));
        memset(&fin, 0, sizeof(fin));
        grp.n = std::min(FSH_GROUP, n_mats - g0);
        grp.partial_base = base;
        fin.m0 = g0;
        fin.n = grp.n;
        int64_t nb = 0;
        for (int i = 0; i < grp.n; ++i) {
            grp.g[i] = G[g0 + i];
            grp.w[i] = W[g0 + i];
            grp.numel[i] = numel[g0 + i];
            grp.block_start[i] = nb;
            fin.pstart[i] = base + nb;
            grp.vec_ok[i] = (reinterpret_cast<uintptr_t>(G[g0 + i]) % 16 == 0) &&
                            (reinterpret_cast<uintptr_t>(W[g0 + i]) % 16 == 0);
            nb += fisher_blocks(numel[g0 + i]);
        }
        grp.block_start[grp.n] = nb;
        fin.pstart[grp.n] = base + nb;
        if (nb > 0) {
            if (t == LRC_BF16)
                hipLaunchKernelGGL(k_fisher_partial<true>, dim3(unsigned(nb)), dim3(FSH_THREADS), 0, s, grp, partials);
            else
                hipLaunchKernelGGL(k_fisher_partial<false>, dim3(unsigned(nb)), dim3(FSH_THREADS), 0, s, grp,
                                   partials);
            LRC_LAUNCH_CHECK("k_fisher_partial");
        }
        hipLaunchKernelGGL(k_fisher_final, dim3(grp.n), dim3(256), 0, s, partials, fin, alpha, info);
        LRC_LAUNCH_CHECK("k_fisher_final");
        base += nb;
    }
    return LRC_OK;
}

// ---------------------------------------------------------------------------------------------
// Fisher scores without a caller workspace: the partials go to a file-scope device array of fixed
// size (one copy per GPU, held until the process ends).  Host code never passes the array's name
// to a kernel -- on the host that name is only a stand-in -- but the device address that
// hipGetSymbolAddress returns for it, looked up once per device with that device current.  Every
// partial is written before it is read in the same call, so the array needs no clearing; calls that
// overlap on one GPU share it and race.
// ---------------------------------------------------------------------------------------------
constexpr int64_t FSH_SCRATCH_PARTIALS = int64_t(1) << 19;  // 4 MiB: up to 2^34 elements in one call
static __device__ __align__(256) double scratch[FSH_SCRATCH_PARTIALS];

constexpr int SCR_MAX_DEVICES = 64;
static std::mutex g_scr_mu;
static double *g_scr_ptr[SCR_MAX_DEVICES] = {};

static lrc_status scratch_ptr(double **out) {
    int dev = -1;
    LRC_HIP(hipGetDevice(&dev));
    if (dev < 0 || dev >= SCR_MAX_DEVICES) return fail(LRC_ERR_ARG, "device index beyond the scratch table");
    std::lock_guard<std::mutex> lk(g_scr_mu);
    if (!g_scr_ptr[dev]) {
        void *p = nullptr;
        LRC_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
        if (!p) return fail(LRC_ERR_HIP, "hipGetSymbolAddress returned no address for the scratch array");
        g_scr_ptr[dev] = static_cast<double *>(p);
    }
    *out = g_scr_ptr[dev];
    return LRC_OK;
}

int64_t fisher_scratch_partials() { return FSH_SCRATCH_PARTIALS; }

lrc_status fisher_run_noalloc(int32_t n_mats, const void *const *G, const void *const *W, const int64_t *numel,
                              lrc_dtype t, double *alpha, int32_t *info, hipStream_t s) {
    int64_t nb_total = 0;
    for (int i = 0; i < n_mats; ++i) nb_total += fisher_blocks(numel[i]);
    if (nb_total > FSH_SCRATCH_PARTIALS)
        return fail(LRC_ERR_ARG, "input larger than the scratch maximum (2^34 elements per call)");
    double *ptr = nullptr;
    const lrc_status st = scratch_ptr(&ptr);
    if (st != LRC_OK) return st;
    return fisher_run(n_mats, G, W, numel, t, alpha, ptr, size_t(FSH_SCRATCH_PARTIALS) * sizeof(double), info, s);
}

// ---------------------------------------------------------------------------------------------
// Greedy allocation.  Instead of sorting the candidates, find the priority t* of the item at
// which the ordered scan stops: t* is the smallest fp64 value t >= 0 with
// cost(items with p > t) <= budget left, found by bisection over the bit patterns of
// non-negative doubles (their integer order is their value order).  Every item with p > t*
// is taken; the items with p == t* are taken in (m asc, k asc) order while they fit, and the
// first that does not fit ends the scan.  Same result as sorting by (p desc, m asc, k asc)
// and scanning, with exact integer costs and the same fp64 priorities.
// ---------------------------------------------------------------------------------------------
constexpr int ALC_THREADS = 1024;

__device__ __forceinline__ int64_t block_sum_i64(int64_t v, int64_t *sh) {
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    __syncthreads();
    if (lane == 0) sh[wid] = v;
    __syncthreads();
    int64_t r = 0;
    for (int i = 0; i < int(blockDim.x >> 6); ++i) r += sh[i];
    __syncthreads();
    return r;  // valid in every thread
}

// Marks the kept items of each matrix (one thread per matrix, its items in k order): the first
// k_min always; with how == 1 every candidate; with how == 2 the candidates with p > t* and the first
// take[m] of those with p == t*.
__device__ void alloc_mark(int32_t n_mats, const int64_t *offsets, const int32_t *k_min, const double *p, int how,
                           double tstar, const int32_t *take, uint8_t *selected) {
    for (int m = threadIdx.x; m < n_mats; m += blockDim.x) {
        const int64_t j0 = offsets[m], j1 = offsets[m + 1];
        const int32_t km = k_min ? k_min[m] : 0;
        int32_t ties = how == 2 ? __hip_atomic_load(&take[m], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0;
        for (int64_t j = j0; j < j1; ++j) {
            bool keep = j - j0 < km;
            if (!keep && how == 1) keep = true;
            if (!keep && how == 2) {
                const double pj = p[j];
                if (pj > tstar) keep = true;
                else if (pj == tstar && ties > 0) { keep = true; --ties; }
            }
            selected[j] = keep ? 1 : 0;
        }
    }
}

// MODE 0: p = w_m max(lambda, 0) with w_m = alpha_m / (eps0_m cost_m) (Fisher-weighted eigenvalues).
// MODE 1: p = s / cost_m with s = lam[j] a per-component score (alpha and eps0 unused); a negative or
//         NaN score is a bad score.
// selected (optional): one byte per item, 1 for the kept components.
template <int MODE>
__global__ void __launch_bounds__(ALC_THREADS) k_allocate(int32_t n_mats, const double *__restrict__ alpha,
                                                          const double *__restrict__ lam, const int64_t *__restrict__ offsets,
                                                          int64_t n_items, const double *__restrict__ eps0,
                                                          const int64_t *__restrict__ cost, const int32_t *__restrict__ k_min,
                                                          int64_t budget, int32_t *__restrict__ k_out, int32_t *__restrict__ info,
                                                          double *__restrict__ wm, double *__restrict__ p,
                                                          int32_t *__restrict__ item_m, int32_t *__restrict__ cnt_above,
                                                          int32_t *__restrict__ cnt_tie, uint8_t *__restrict__ selected) {
    __shared__ int64_t sh[ALC_THREADS / 64];
    __shared__ int bad;
    const int tid = threadIdx.x;
    if (tid == 0) bad = 0;
    __syncthreads();
    // 1. weights, validity, mandatory ranks
    int64_t mand = 0;
    for (int m = tid; m < n_mats; m += ALC_THREADS) {
        const int64_t c = cost[m];
        double w = 0.0;
        if (MODE == 0) {
            const double a = alpha[m], e0 = eps0[m];
            if (!(a >= 0.0) || !(e0 >= 0.0) || c <= 0) {
                atomicOr(&bad, 1);
            } else if (e0 != 0.0) {
                const double t = e0 * double(c);
                w = a / t;
                if (!isfinite(w)) atomicOr(&bad, 1);
            }
        } else if (c <= 0) {
            atomicOr(&bad, 1);
        }
        wm[m] = w;
        const int32_t km = k_min ? k_min[m] : 0;
        const int64_t K = offsets[m + 1] - offsets[m];
        if (km < 0 || km > K) atomicOr(&bad, 1);
        mand += int64_t(km) * c;
        cnt_above[m] = 0;
        cnt_tie[m] = 0;
    }
    mand = block_sum_i64(mand, sh);
    __syncthreads();
    // 2. priorities (-1 marks a non-candidate: rank at or below k_min)
    for (int64_t j = tid; j < n_items; j += ALC_THREADS) {
        int lo = 0, hi = n_mats - 1;  // last m with offsets[m] <= j
        while (lo < hi) {
            int mid = (lo + hi + 1) >> 1;
            if (offsets[mid] <= j) lo = mid; else hi = mid - 1;
        }
        const int m = lo;
        const int64_t k = j - offsets[m] + 1;
        const int32_t km = k_min ? k_min[m] : 0;
        const double l = lam[j];
        item_m[j] = m;
        if (MODE == 0) {
            if (isnan(l)) atomicOr(&bad, 1);
            p[j] = (k > km) ? wm[m] * (l > 0.0 ? l : 0.0) : -1.0;
        } else {
            if (!(l >= 0.0)) atomicOr(&bad, 1);
            p[j] = (k > km) ? l / double(cost[m]) : -1.0;
        }
    }
    __syncthreads();
    if (bad || mand > budget) {
        for (int m = tid; m < n_mats; m += ALC_THREADS) k_out[m] = k_min ? k_min[m] : 0;
        if (selected) alloc_mark(n_mats, offsets, k_min, p, 0, 0.0, cnt_tie, selected);
        if (tid == 0) *info = bad ? LRC_INFO_BAD_SCORE : LRC_INFO_BUDGET;
        return;
    }
    const int64_t rem = budget - mand;
    // 3. total cost of all candidates
    int64_t tot = 0;
    for (int64_t j = tid; j < n_items; j += ALC_THREADS)
        if (p[j] >= 0.0) tot += cost[item_m[j]];
    tot = block_sum_i64(tot, sh);
    if (tot <= rem) {
        for (int m = tid; m < n_mats; m += ALC_THREADS)
            k_out[m] = int32_t(offsets[m + 1] - offsets[m]);
        if (selected) alloc_mark(n_mats, offsets, k_min, p, 1, 0.0, cnt_tie, selected);
        if (tid == 0) *info = LRC_INFO_OK;
        return;
    }
    // 4. bisection over bit patterns: lo = "below zero" (everything), hi = +inf (nothing)
    int64_t lo = -1, hi = 0x7ff0000000000000LL;
    while (hi - lo > 1) {
        const int64_t mid = lo + (hi - lo) / 2;
        const double t = __longlong_as_double(mid);
        int64_t sabove = 0;
        for (int64_t j = tid; j < n_items; j += ALC_THREADS)
            if (p[j] > t) sabove += cost[item_m[j]];
        sabove = block_sum_i64(sabove, sh);
        if (sabove <= rem) hi = mid; else lo = mid;
    }
    const double tstar = __longlong_as_double(hi);
    // 5. counts above t* and in the tie group, per matrix (integer atomics: order-free)
    int64_t cabove = 0;
    for (int64_t j = tid; j < n_items; j += ALC_THREADS) {
        const double pj = p[j];
        if (pj > tstar) {
            atomicAdd(&cnt_above[item_m[j]], 1);
            cabove += cost[item_m[j]];
        } else if (pj == tstar) {
            atomicAdd(&cnt_tie[item_m[j]], 1);
        }
    }
    cabove = block_sum_i64(cabove, sh);
    __threadfence();
    __syncthreads();
    // 6. the tie group in (m asc, k asc) order, stopping at the first item that does not fit
    if (tid == 0) {
        int64_t r = rem - cabove;
        bool stopped = false;
        for (int m = 0; m < n_mats; ++m) {
            const int64_t c = cost[m];
            const int64_t ct = __hip_atomic_load(&cnt_tie[m], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            int64_t take = 0;
            if (!stopped && ct > 0) {
                if (ct * c <= r) {
                    take = ct;
                } else {
                    take = r / c;
                    stopped = true;
                }
                r -= take * c;
            }
            __hip_atomic_store(&cnt_tie[m], int32_t(take), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    __threadfence();
    __syncthreads();
    for (int m = tid; m < n_mats; m += ALC_THREADS)
        k_out[m] = (k_min ? k_min[m] : 0) +
                   __hip_atomic_load(&cnt_above[m], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) +
                   __hip_atomic_load(&cnt_tie[m], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (selected) alloc_mark(n_mats, offsets, k_min, p, 2, tstar, cnt_tie, selected);
    if (tid == 0) *info = LRC_INFO_OK;
}

size_t alloc_workspace(int32_t n_mats, int64_t n_items) {
    Counter c;
    c.carve<double>(size_t(n_mats));
    c.carve<double>(size_t(n_items > 0 ? n_items : 1));
    c.carve<int32_t>(size_t(n_items > 0 ? n_items : 1));
    c.carve<int32_t>(size_t(n_mats));
    c.carve<int32_t>(size_t(n_mats));
    return c.off;
}

// Proportional ranks (FLRC page, method 1: r_m = round(alpha_m / S * R); method 2: the same rule for
// each budget R(t) of a non-increasing schedule), one workgroup per budget, one thread per matrix.
// Rounding half away from zero, then the sum brought to R by largest remainders: the d matrices
// first in (q_m - r_m descending, m ascending) order gain one when the sum is short by d; when it is
// over by d, the d matrices with r_m > 0 first in (q_m - r_m ascending, m ascending) order lose one
// (one unit per matrix suffices: every rounding moved q_m by at most one half).  q_m = (alpha_m R) / S
// in fp64 with S summed in index order by one thread, so the decisions match a sequential
// evaluation bit for bit.
__global__ void __launch_bounds__(PROP_MAX) k_alloc_prop(int32_t n, const double *__restrict__ alpha, int32_t nb,
                                                         const int64_t *__restrict__ budgets, int64_t *__restrict__ r_out,
                                                         int32_t *__restrict__ info) {
    __shared__ double S_sh;
    __shared__ int bad_sh;
    __shared__ double rem[PROP_MAX];
    __shared__ long long rr[PROP_MAX];
    __shared__ long long sum_sh;
    const int m = threadIdx.x, t = blockIdx.x;
    if (m == 0) {
        double S = 0.0;
        int bad = 0;
        for (int i = 0; i < n; ++i) {
            const double v = alpha[i];
            if (!(v >= 0.0)) bad = 1;
            S = S + v;
        }
        if (!(S > 0.0 && S <= 1.7976931348623157e308)) bad = 1;
        for (int i = 0; i < nb; ++i)
            if (budgets[i] < 0) bad = 1;
        S_sh = S;
        bad_sh = bad;
    }
    __syncthreads();
    if (bad_sh) {
        if (m < n) r_out[int64_t(t) * n + m] = 0;
        if (t == 0 && m == 0) *info = 5;
        return;
    }
    const int64_t R = budgets[t];
    double q = 0.0;
    long long r = 0;
    if (m < n) {
        q = (alpha[m] * double(R)) / S_sh;
        r = (long long)floor(q + 0.5);
        rem[m] = q - double(r);
        rr[m] = r;
    }
    __syncthreads();
    if (m == 0) {
        long long sm = 0;
        for (int i = 0; i < n; ++i) sm += rr[i];
        sum_sh = sm;
    }
    __syncthreads();
    const long long d = (long long)R - sum_sh;
    if (m < n) {
        if (d > 0) {
            long long rank = 0;
            for (int i = 0; i < n; ++i) rank += (rem[i] > rem[m] || (rem[i] == rem[m] && i < m)) ? 1 : 0;
            if (rank < d) r += 1;
        } else if (d < 0 && rr[m] > 0) {
            long long rank = 0;
            for (int i = 0; i < n; ++i)
                rank += (rr[i] > 0 && (rem[i] < rem[m] || (rem[i] == rem[m] && i < m))) ? 1 : 0;
            if (rank < -d) r -= 1;
        }
        r_out[int64_t(t) * n + m] = r;
    }
    if (t == 0 && m == 0) *info = 0;
}

lrc_status alloc_prop_run(int32_t n, const double *alpha, int32_t nb, const int64_t *budgets, int64_t *r_out,
                          int32_t *info, hipStream_t s) {
    hipLaunchKernelGGL(k_alloc_prop, dim3(unsigned(nb)), dim3(PROP_MAX), 0, s, n, alpha, nb, budgets, r_out, info);
    LRC_LAUNCH_CHECK("k_alloc_prop");
    return LRC_OK;
}

lrc_status alloc_run(const AllocArgs &a, void *ws, size_t ws_bytes, hipStream_t s) {
    Carver cv(ws, ws_bytes);
    double *wm = cv.carve<double>(size_t(a.n_mats));
    double *p = cv.carve<double>(size_t(a.n_items > 0 ? a.n_items : 1));
    int32_t *im = cv.carve<int32_t>(size_t(a.n_items > 0 ? a.n_items : 1));
    int32_t *ca = cv.carve<int32_t>(size_t(a.n_mats));
    int32_t *ct = cv.carve<int32_t>(size_t(a.n_mats));
    if (!ct) return fail(LRC_ERR_WORKSPACE, "allocation workspace too small");
    if (a.per_component)
        hipLaunchKernelGGL(k_allocate<1>, dim3(1), dim3(ALC_THREADS), 0, s, a.n_mats, a.alpha, a.lambda_packed,
                           a.offsets, a.n_items, a.eps0, a.cost, a.k_min, a.budget, a.k_out, a.info, wm, p, im, ca, ct,
                           a.selected);
    else
        hipLaunchKernelGGL(k_allocate<0>, dim3(1), dim3(ALC_THREADS), 0, s, a.n_mats, a.alpha, a.lambda_packed,
                           a.offsets, a.n_items, a.eps0, a.cost, a.k_min, a.budget, a.k_out, a.info, wm, p, im, ca, ct,
                           a.selected);
    LRC_LAUNCH_CHECK("k_allocate");
    return LRC_OK;
}

}  // namespace lrc
