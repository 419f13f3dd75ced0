// Symmetric eigendecomposition for n > 128 (Swift-SVD page, section 2-ga: one eigendecomposition
// of Y^T Y yields V and Sigma^2 of Y).
//
// Stages, all on the GPU:
//  1. Householder tridiagonalisation Q^T C Q = T, blocked (panel of NB columns, then a rank-2NB
//     update of the trailing matrix), working precision T_ (fp32 or fp64).  Only the upper
//     triangle is kept current; the symmetric product of each column reads every upper tile once
//     and forms both its row and its column contribution.  Two launches per column (the product,
//     then the column's W and the next column), one for all members of a lockstep group.  Once the
//     trailing block fits in LDS (order <= 256 in fp32, <= 176 in fp64; from the start for such
//     orders), one workgroup reduces the rest of it (k_trd_small).
//  2. All n eigenvalues of T by multisection on Sturm counts, fp64, 16 lanes per eigenvalue.
//  3. Eigenvectors of T for the n_vec largest eigenvalues by inverse iteration, fp64, one thread
//     per vector (LU with partial pivoting of T - lambda I once, then three solves); vectors of
//     eigenvalues closer than a cluster tolerance are re-orthogonalised by modified Gram-Schmidt.
//  4. Back-transformation V = Q Z with the reflectors grouped in blocks of NBT,
//     Q_b = I - V_b T_b V_b^T (compact WY), applied from the last block to the first, in fp64.
//  5. Each column's entry of largest magnitude made positive.
// Reflector c is H_c = I - tau_c v_c v_c^T with v_c[c+1] = 1 and v_c[r] = 0 for r <= c.
#include <algorithm>
#include <atomic>
#include <cfloat>
#include <cmath>
#include <cstdlib>
#include <map>
#include <memory>
#include <mutex>
#include <string>
#include <thread>
#include <vector>

#include "lrc_internal.h"

namespace lrc {

constexpr int NB = 32;    // tridiagonalisation panel width
constexpr int NBT = 64;   // back-transformation block of reflectors
constexpr int RCH = 256;  // rows per partial in the back-transformation reductions

// ---------------------------------------------------------------------------------------------
// 1. tridiagonalisation
// ---------------------------------------------------------------------------------------------
// Storage: A is n x lda (lda a multiple of 64), row-major; only the upper triangle (r <= s) is kept
// current, and the padding columns [n, lda) hold zeros.  Column c below the diagonal is read as
// row c right of it, so every access to it is contiguous.  The panel factors V and W (NB columns
// of length n) are column-major, V[q][r] at Vp[q * n + r], so that per-row loops over a panel
// column read consecutive addresses.
template <class T>
__global__ void k_fill_full(const float *__restrict__ C, int64_t ldc, int64_t n, T *__restrict__ A, int64_t lda,
                            int *__restrict__ bad) {
    const int64_t total = n * lda;
    for (int64_t e = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; e < total; e += int64_t(gridDim.x) * blockDim.x) {
        const int64_t i = e / lda, j = e % lda;
        if (j >= n) {
            A[e] = T(0);
            continue;
        }
        const float v = i <= j ? C[i * ldc + j] : C[j * ldc + i];
        if (!isfinite(v)) atomicOr(bad, 1);
        A[e] = T(v);
    }
}

// Several matrices of one order decomposed in lockstep: the tridiagonalisation kernels take the
// pointers of the first matrix's workspace region and the byte stride zs between regions (every
// region has the same layout), and workgroup z works on matrix z.  zs = 0 with one z: one matrix.
template <class P>
__device__ __forceinline__ P zoff(P p, int64_t zs) {
    return reinterpret_cast<P>(reinterpret_cast<uintptr_t>(p) + uintptr_t(int64_t(blockIdx.z) * zs));
}

template <class T>
__global__ void k_fill_zero(T *__restrict__ p, int64_t n, int64_t zs) {
    p = zoff(p, zs);
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

// Kernel arguments are read from memory by scalar loads, which the compiler issues where each
// value is first needed, every group followed by a wait for it; in a short kernel these round
// trips line up one after another before the first global load can start.  Naming all the
// arguments in one empty asm statement at entry makes it load them in one batch.
#define LRC_ARGS_AT_ENTRY(...) asm volatile("" ::__VA_ARGS__)

// Sum of at(i) for i = i0, i0 + step, ... < i1 with eight loads in flight (eight running sums,
// combined in a fixed order); a loop of dependent load-add steps would wait for every load.  The
// last (partial) group of eight is loaded under a mask, also in one batch.
template <class T, class F>
__device__ __forceinline__ T sum_strided8(F at, int i0, int i1, int step) {
    T a[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) a[u] = T(0);
    int i = i0;
    for (; i + 7 * step < i1; i += 8 * step) {
        T v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = at(i + u * step);
#pragma unroll
        for (int u = 0; u < 8; ++u) a[u] += v[u];
    }
    if (i < i1) {
        T v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = i + u * step < i1 ? at(i + u * step) : T(0);
#pragma unroll
        for (int u = 0; u < 8; ++u) a[u] += v[u];
    }
    return ((a[0] + a[1]) + (a[2] + a[3])) + ((a[4] + a[5]) + (a[6] + a[7]));
}

// The same sum in two steps, so that the loads of several sums are in flight together: first()
// loads the first eight terms under a mask in straight-line code, rest() adds them and any
// further terms (eight loads at a time).  Terms are summed in the order sum_strided8 uses.
template <class T>
struct StridedSum {
    T v[8];
    int i0, i1, step;
    template <class F>
    __device__ __forceinline__ void first(F at, int a0, int a1, int st) {
        i0 = a0;
        i1 = a1;
        step = st;
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = i0 + u * step < i1 ? at(i0 + u * step) : T(0);
    }
    template <class F>
    __device__ __forceinline__ T rest(F at) {
        for (int i = i0 + 8 * step; i < i1; i += 8 * step) {
            T w[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) w[u] = i + u * step < i1 ? at(i + u * step) : T(0);
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] += w[u];
        }
        return ((v[0] + v[1]) + (v[2] + v[3])) + ((v[4] + v[5]) + (v[6] + v[7]));
    }
};

// Each column of a panel takes two launches; each global reduction is done by the next launch,
// redundantly in every block that needs it and always in the same fixed order, so all blocks see
// bit-identical values (no atomics, no device-wide fences):
//   k_trd_symv : reflector of column c (reduces the ||x||^2 partials; block 0 also reduces the
//                W^T x, V^T x partials into q and stores e[c], tau[c]); y = A v over the upper
//                tiles of the trailing matrix as fixed-order partials, with scalar partials of
//                v^T y; v into V[:, j] and Rt[c]
//   k_trd_w1col: W[:, j] from y, q and v^T y; then row c+1 with the panel's corrections (the
//                next column), its ||x||^2 and W^T x, V^T x partials
// The first column of a panel takes k_trd_col0 instead of a previous k_trd_w1col.

// fixed-order sum of p[0..np) by one block: strided per-thread sums, then a tree (every thread)
// One reduce-scatter step over lane bit MBIT: lanes with the bit set keep values HALF .. 2 HALF - 1
// (moved to 0 .. HALF - 1), the others 0 .. HALF - 1, each summed with the partner's copy.
template <int HALF, int MBIT, int N, class T>
__device__ __forceinline__ void rs_step(T (&p)[N], int lane) {
    static_assert(2 * HALF <= N, "reduce-scatter step");
    const bool up = (lane & MBIT) != 0;
#pragma unroll
    for (int k = 0; k < HALF; ++k) {
        const T send = up ? p[k] : p[k + HALF];
        const T keep = up ? p[k + HALF] : p[k];
        p[k] = keep + __shfl_xor(send, MBIT);
    }
}

// First column c of a panel (no panel corrections yet): x = row c right of the diagonal,
// d[c], partials of ||x[2:]||^2 over 256-row blocks.
template <class T>
__global__ void __launch_bounds__(256) k_trd_col0(const T *__restrict__ A, int64_t lda, int64_t n, int64_t c,
                                                  T *__restrict__ colbuf, T *__restrict__ part,
                                                  double *__restrict__ d, int64_t zs) {
    __shared__ T sh[4];
    A = zoff(A, zs);
    colbuf = zoff(colbuf, zs);
    part = zoff(part, zs);
    d = zoff(d, zs);
    const int64_t r = c + int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    T ss = T(0);
    if (r < n) {
        const T a = A[c * lda + r];  // = A[r][c] (upper storage)
        colbuf[r] = a;
        if (r >= c + 2) ss = a * a;
        if (r == c) d[c] = double(a);
    }
    ss = block_sum(ss, sh);
    if (threadIdx.x == 0) part[blockIdx.x] = ss;
}

// Symmetric product y = A v over the upper tiles of the trailing matrix.  Tiles are TS x TS,
// aligned to multiples of TS (TS = 64 for fp32, 32 for fp64: 256-byte tile rows of 16 chunks of
// 16 bytes).  Work item (block row i, chunk ch) covers tiles J = i + ch*CH ... of that block row;
// the items are numbered by L = NT - i (the number of upper tiles in block row i), L = 1 first.
// Each wave takes one tile at a time: it stages the tile in LDS with the 16-byte chunks of row r
// XOR-permuted by (r mod 16), then lane rr forms the row part sum_k A[rr][k] v_J[k] (reading
// 16-byte chunks along its row) and lane cc the column part sum_r A[r][cc] v_I[r] (scalar reads
// down its column); both patterns are free of bank conflicts.  Row parts accumulate over the
// chunk's tiles and are written once per item; column parts go to colpart[i][J] (J > i) or, for
// the diagonal tile, into the row part (strict upper entries only; the lower half of a diagonal
// tile is never read).
template <class T>
struct SymvTile {
    static constexpr int TS = sizeof(T) == 4 ? 64 : 32;
    static constexpr int EPC = 16 / int(sizeof(T));  // elements per 16-byte chunk
    static constexpr int H = 64 / TS;                 // lanes per tile row
};

// number of work items of block rows with L = 1 .. m tiles, chunks of ch tiles
__host__ __device__ __forceinline__ int64_t symv_items(int64_t m, int64_t ch) {
    const int64_t q = m / ch, r = m % ch;
    return ch * q * (q + 1) / 2 + r * (q + 1);
}

// Tiles per wave of a symmetric-product work item (1 or 2), and waves per SIMD.  One tile per wave
// keeps a wave under 128 registers, so four workgroups share a CU: while one forms its products
// from registers the others' loads are in flight (two tiles per wave, two workgroups per CU
// keep the memory system busy for a smaller share of the time).
#ifndef SYMV_TPW
#define SYMV_TPW 1
#endif
#ifndef SYMV_WPE
#define SYMV_WPE (SYMV_TPW == 1 ? 4 : 2)
#endif
#ifndef SYMV_MIN_ITEMS
#define SYMV_MIN_ITEMS 256
#endif

template <class T>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(SYMV_WPE, SYMV_WPE))) k_trd_symv(const T *__restrict__ A, int64_t lda, int64_t n, int64_t c, int j,
                                                  const T *__restrict__ colbuf, const T *__restrict__ part,
                                                  int npart, T *__restrict__ Vp, const T *__restrict__ Wp,
                                                  T *__restrict__ Rt, T *__restrict__ rowpart,
                                                  T *__restrict__ colpart, const T *__restrict__ qcol,
                                                  T *__restrict__ qvec, T *__restrict__ spart, T *__restrict__ tau,
                                                  double *__restrict__ e, int NT, int CHK, int64_t zs) {
    LRC_ARGS_AT_ENTRY("s"(A), "s"(lda), "s"(n), "s"(c), "s"(j), "s"(colbuf), "s"(part), "s"(npart), "s"(Vp), "s"(Wp),
                      "s"(Rt), "s"(rowpart), "s"(colpart), "s"(qcol), "s"(qvec), "s"(spart), "s"(tau), "s"(e),
                      "s"(NT), "s"(CHK), "s"(zs));
    A = zoff(A, zs);
    colbuf = zoff(colbuf, zs);
    part = zoff(part, zs);
    Vp = zoff(Vp, zs);
    Wp = zoff(Wp, zs);
    Rt = zoff(Rt, zs);
    rowpart = zoff(rowpart, zs);
    colpart = zoff(colpart, zs);
    qcol = zoff(qcol, zs);
    qvec = zoff(qvec, zs);
    spart = zoff(spart, zs);
    tau = zoff(tau, zs);
    e = zoff(e, zs);
    constexpr int TS = SymvTile<T>::TS, EPC = SymvTile<T>::EPC, H = SymvTile<T>::H;
    static_assert(16 * EPC == TS, "tile geometry");
    typedef T vec_t __attribute__((ext_vector_type(EPC)));
    __shared__ __attribute__((aligned(16))) T vI[TS];
    constexpr int NVJ = 4 * SYMV_TPW * TS;            // v values of an item's column tiles
    constexpr int XJ = NVJ >= 256 ? NVJ / 256 : 1;     // ... per thread
    __shared__ __attribute__((aligned(16))) T vJ[NVJ];
    __shared__ T rowacc[4][TS];
    __shared__ T dcol[4][TS];
    __shared__ T qr[256];
    __shared__ T sh[4];
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    // work item: L with items(L - 1) <= g < items(L)
    const int64_t g = blockIdx.x;
    const int T0 = int((c + 1) / TS);
    int lo = 1, hi = NT - T0;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (symv_items(mid, CHK) > g) hi = mid; else lo = mid + 1;
    }
    const int L = lo;
    const int i = NT - L;
    const int ch = int(g - symv_items(L - 1, CHK));
    const int J0 = i + ch * CHK, J1 = min(J0 + CHK, NT);
    const int rows_i = int(min<int64_t>(TS, n - int64_t(i) * TS));
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<T *>(A + int64_t(i) * TS * lda), short(0), int(int64_t(rows_i) * lda * int64_t(sizeof(T))),
        0x00020000);
    // Every load that does not depend on the reflector is issued first: this wave's tiles, the raw
    // column values behind v, the ||x||^2 partials, and (block 0) the W^T x, V^T x partials.  A work
    // item has at most 4 SYMV_TPW tiles, so wave w has at most SYMV_TPW of them (J0 + w, and
    // J0 + w + 4 when SYMV_TPW = 2), each loaded into a register set of its own.
    u32x4_t pre[SYMV_TPW][TS / 4];
    auto tile_load = [&](int J, u32x4_t (&dst)[TS / 4]) {
#pragma unroll
        for (int u = 0; u < TS / 4; ++u) {  // TS rows x 16 chunks, 64 lanes
            const int idx = lane + 64 * u;
            const int r = idx >> 4, q = idx & 15;
            dst[u] = __builtin_amdgcn_raw_buffer_load_b128(
                rs, int((int64_t(r) * lda + int64_t(J) * TS) * int64_t(sizeof(T))) + q * 16, 0, 0);
        }
    };
    const int Jf = J0 + wave;
    if (Jf < J1) tile_load(Jf, pre[0]);
    if (SYMV_TPW == 2 && Jf + 4 < J1) tile_load(Jf + 4, pre[SYMV_TPW - 1]);
    auto xraw = [&](int64_t x) -> T { return (x <= c + 1 || x >= n) ? T(0) : colbuf[x]; };
    const T xI = t < TS ? xraw(int64_t(i) * TS + t) : T(0);
    T xJ[XJ];
#pragma unroll
    for (int u = 0; u < XJ; ++u) {
        const int x = t + 256 * u;
        xJ[u] = x < (J1 - J0) * TS ? xraw(int64_t(J0) * TS + x) : T(0);
    }
    const T sacc = sum_strided8<T>([&](int b2) { return part[b2]; }, t, npart, 256);
    const T alpha = colbuf[c + 1];
    T qacc = T(0);  // block 0: W^T x, V^T x, value t % 64, every fourth partial from t / 64
    if (blockIdx.x == 0)
        qacc = sum_strided8<T>([&](int b2) { return qcol[int64_t(b2) * 2 * NB + (t & 63)]; }, t >> 6, npart, 4);
    // the reflector of column c: alpha = x[0], sigma2 = ||x[1:]||^2; tau = (beta - alpha)/beta,
    // v = [1, x[1:] / (alpha - beta)], beta = -sign(alpha) ||x||; tau = 0 when x[1:] = 0
    const T sigma2 = block_sum(sacc, sh);
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
    if (blockIdx.x == 0 && t == 0) {
        e[c] = double(beta);
        tau[c] = tv;
    }
    auto vof = [&](int64_t x, T raw) -> T { return x == c + 1 ? T(1) : raw * scale; };
    if (t < TS) vI[t] = vof(int64_t(i) * TS + t, xI);
#pragma unroll
    for (int u = 0; u < XJ; ++u) {
        const int x = t + 256 * u;
        if (x < (J1 - J0) * TS) vJ[x] = vof(int64_t(J0) * TS + x, xJ[u]);
    }
    __syncthreads();

    // Each lane holds, of every tile it loaded, rows gq + 4u (u < RPL) and the EPC columns of
    // chunk q.  Both parts are formed from these registers: the row part accumulates over the
    // wave's tiles and is reduced once across the 16 lanes that share rows (each lane keeps one
    // row); the column part of each tile is reduced across the 4 lanes that share columns (each
    // keeps one column).  No LDS copy of the tile: staging it and reading it back (a scalar read
    // per column element) took 40 % of the kernel's time at the largest trailing sizes.
    constexpr int RPL = TS / 4;  // rows per lane (16 fp32, 8 fp64)
    const int gq = lane >> 4, q = lane & 15;
    const int xsel = EPC == 4 ? ((lane >> 4) & 3) : ((lane >> 5) & 1);  // column kept after the reduction
    const int csel = q * EPC + xsel;
    const int rsel = gq + 4 * (RPL == 16 ? (lane & 15) : ((lane & 14) >> 1));  // row kept after the reduction
    const bool cwriter = EPC == 4 || (lane & 16) == 0;  // one lane per column (fp64: two hold it)
    T vIr[RPL];
#pragma unroll
    for (int u = 0; u < RPL; ++u) vIr[u] = vI[gq + 4 * u];
    T rp[RPL];
#pragma unroll
    for (int u = 0; u < RPL; ++u) rp[u] = T(0);
    T sdot = T(0);  // this lane's share of v^T y from the column parts
    T dcs = T(0);   // diagonal tile: this lane's column sum, added to the row of the same index
    bool had_diag = false;
#pragma unroll
    for (int tt = 0; tt < SYMV_TPW; ++tt) {
        const int J = Jf + 4 * tt;
        if (J >= J1) break;
        const bool diag = (J == i);
        const vec_t bj = *reinterpret_cast<const vec_t *>(vJ + (J - J0) * TS + q * EPC);
        T cp[EPC];
#pragma unroll
        for (int x = 0; x < EPC; ++x) cp[x] = T(0);
#pragma unroll
        for (int u = 0; u < RPL; ++u) {
            const vec_t a = __builtin_bit_cast(vec_t, pre[tt][u]);
            const int r = gq + 4 * u;
#pragma unroll
            for (int x = 0; x < EPC; ++x) {
                const int cc = q * EPC + x;
                // the diagonal tile holds the upper triangle only: the row part takes cc >= r and
                // the column part r < cc
                const T ar = (diag && cc < r) ? T(0) : a[x];
                const T ac = (diag && r >= cc) ? T(0) : a[x];
                rp[u] += ar * bj[x];
                cp[x] += ac * vIr[u];
            }
        }
        if constexpr (EPC == 4) {
            rs_step<2, 32>(cp, lane);
            rs_step<1, 16>(cp, lane);
        } else {
            rs_step<1, 32>(cp, lane);
            cp[0] += __shfl_xor(cp[0], 16);
        }
        if (diag) {
            had_diag = true;
            dcs = cp[0];
        } else if (cwriter) {
            colpart[(int64_t(i) * NT + J) * TS + csel] = cp[0];
            sdot += cp[0] * bj[xsel];
        }
    }
    if constexpr (RPL == 16) {
        rs_step<8, 8>(rp, lane);
        rs_step<4, 4>(rp, lane);
        rs_step<2, 2>(rp, lane);
        rs_step<1, 1>(rp, lane);
    } else {
        rs_step<4, 8>(rp, lane);
        rs_step<2, 4>(rp, lane);
        rs_step<1, 2>(rp, lane);
        rp[0] += __shfl_xor(rp[0], 1);
    }
    T yrow = rp[0];
    if (had_diag) {  // wave-uniform
        dcol[wave][csel] = dcs;
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier();
        yrow += dcol[wave][rsel];
    }
    rowacc[wave][rsel] = yrow;
    __syncthreads();
    if (t < TS) {
        const T yr = (rowacc[0][t] + rowacc[1][t]) + (rowacc[2][t] + rowacc[3][t]);
        rowpart[(int64_t(i) * NT + ch) * TS + t] = yr;
        sdot += yr * vI[t];
    }
    sdot = block_sum(sdot, sh);
    if (t == 0) spart[g] = sdot;
    if (blockIdx.x == 0)  // the reflector's zeros before the first block row
        for (int64_t r = t; r < int64_t(T0) * TS; r += 256) Rt[c * n + r] = T(0);
    if (ch == 0 && t < TS) {  // v into Rt[c] and V[:, j] for block row i
        const int64_t r = int64_t(i) * TS + t;
        if (r < n) {
            Rt[c * n + r] = vI[t];
            if (r > c) Vp[int64_t(j) * n + r] = vI[t];
        }
    }
    if (blockIdx.x == 0) {
        // q = (W^T v, V^T v) over the panel's first j columns from the column kernel's partials of
        // W^T x, V^T x over rows c+2 .. n-1 (fixed order): v = scale x there and v[c+1] = 1
        __syncthreads();
        qr[t] = qacc;
        __syncthreads();
        if (t < 2 * NB) {
            const int q = t % NB;
            const T acc = (qr[t] + qr[64 + t]) + (qr[128 + t] + qr[192 + t]);
            T qv = T(0);
            if (q < j) qv = scale * acc + (t < NB ? Wp[int64_t(q) * n + c + 1] : Vp[int64_t(q) * n + c + 1]);
            qvec[t] = qv;
        }
    }
}

// Second launch of column c (rows r in [c+1, n), 64 per block; the block's four waves share every
// row: wave sub reduces a quarter of the symv partials of y[r] and holds panel columns
// q = 8 sub .. 8 sub + 7 of the row):
//   w1[r]   = tau (y[r] - V[r][:j] q1 - W[r][:j] q2)       (q1 = W^T v, q2 = V^T v)
//   W[r][j] = w1[r] - (tau/2)(w1.v) v[r],  w1.v = tau (v^T y - 2 q1.q2)  (v^T y from the symv's
//             scalar partials, so no further reduction is needed)
// and, unless the panel ends here, the first launch of column c+1 for the same rows: row c+1 of the
// current matrix (the column below the diagonal) with the panel's corrections, ||x||^2 partials and
// the W^T x, V^T x partials.  Each block forms W[c+1][j] itself from a redundant reduction of y[c+1].
// Sums over q are formed per wave and added in wave order; every load of the kernel is issued
// before the first wait (a wave has at most about 50 in flight).
template <class T>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
k_trd_w1col(T *__restrict__ A, int64_t lda, int64_t n, int64_t c, int j, int next, T *__restrict__ Vp,
            T *__restrict__ Wp, const T *__restrict__ rowpart, const T *__restrict__ colpart,
            const T *__restrict__ qvec, const T *__restrict__ spart, int nsp, int NT, int CHK,
            const T *__restrict__ tau, T *__restrict__ colbuf, T *__restrict__ part, T *__restrict__ qcol,
            double *__restrict__ d, int64_t zs) {
    constexpr int QW = NB / 4;  // panel columns per wave
    __shared__ T sh[8];
    __shared__ T qs[2 * NB];
    __shared__ T ys[4][64], pw[4][64], pa[4][64];
    __shared__ T vc[NB], wc[NB];
    __shared__ T v1s[NB], w1s[NB];
    LRC_ARGS_AT_ENTRY("s"(A), "s"(lda), "s"(n), "s"(c), "s"(j), "s"(next), "s"(Vp), "s"(Wp), "s"(rowpart),
                      "s"(colpart), "s"(qvec), "s"(spart), "s"(nsp), "s"(NT), "s"(CHK), "s"(tau), "s"(colbuf),
                      "s"(part), "s"(qcol), "s"(d), "s"(zs));
    A = zoff(A, zs);
    Vp = zoff(Vp, zs);
    Wp = zoff(Wp, zs);
    rowpart = zoff(rowpart, zs);
    colpart = zoff(colpart, zs);
    qvec = zoff(qvec, zs);
    spart = zoff(spart, zs);
    tau = zoff(tau, zs);
    colbuf = zoff(colbuf, zs);
    part = zoff(part, zs);
    qcol = zoff(qcol, zs);
    d = zoff(d, zs);
    const int T0 = int((c + 1) / SymvTile<T>::TS);
    const int t = threadIdx.x;
    const int rl = t & 63, sub = t >> 6;
    const int64_t r = c + 1 + int64_t(blockIdx.x) * 64 + rl;
    const bool live = r < n;
    // every independent load first: q, row c+1 of V and W, the v^T y partials, the partials of
    // y[c+1] and y[r], the row's panel values in this wave's columns, V[r][j] and A[c+1][r]
    const T qv = t < 2 * NB ? qvec[t] : T(0);
    T w1row = T(0), v1row = T(0);
    if (t < NB) {
        w1row = Wp[int64_t(t) * n + c + 1];
        v1row = Vp[int64_t(t) * n + c + 1];
    }
    // y[x] = sum of the row parts of block row I = x / TS (chunks ch) and the column parts of the
    // tiles above it (block rows T0 .. I-1), each sum split over the threads given to it
    constexpr int TS = SymvTile<T>::TS;
    auto rowp = [&](int64_t x) { return [=](int ch) { return rowpart[(x / TS * NT + ch) * TS + x % TS]; }; };
    auto colp = [&](int64_t x) { return [=](int ib) { return colpart[(int64_t(ib) * NT + x / TS) * TS + x % TS]; }; };
    auto nchunks = [&](int64_t x) { return int((NT - x / TS + CHK - 1) / CHK); };
    StridedSum<T> s_sp, s_cr, s_rr, s_rc;
    s_sp.first([&](int b2) { return spart[b2]; }, t, nsp, 256);
    s_cr.first(rowp(c + 1), t, next ? nchunks(c + 1) : 0, 256);  // y[c+1]: no tiles above (I = T0)
    const int Ir = int(r / TS);
    s_rr.first(rowp(r), sub, live ? nchunks(r) : 0, 4);
    s_rc.first(colp(r), T0 + sub, live ? Ir : 0, 4);
    T vr[QW], wr[QW];
#pragma unroll
    for (int u = 0; u < QW; ++u) {
        const int q = QW * sub + u;
        vr[u] = (live && q <= j) ? Vp[int64_t(q) * n + r] : T(0);
        wr[u] = (live && q < j) ? Wp[int64_t(q) * n + r] : T(0);
    }
    const T vj = live ? Vp[int64_t(j) * n + r] : T(0);
    const T aold = (live && next) ? A[(c + 1) * lda + r] : T(0);
    const T tv = tau[c];
    const T sp = s_sp.rest([&](int b2) { return spart[b2]; });
    const T ycp = s_cr.rest(rowp(c + 1));
    const T yr = s_rr.rest(rowp(r)) + s_rc.rest(colp(r));
    if (t < 2 * NB) qs[t] = qv;
    if (t < NB) {  // row c+1 of the panel, for the thread that forms W[c+1][j]
        w1s[t] = w1row;
        v1s[t] = v1row;
    }
    ys[sub][rl] = yr;
    // v^T y and y[c+1] in one block reduction
    T vty = sp, yc = ycp;
    for (int o = 32; o > 0; o >>= 1) {
        vty += __shfl_xor(vty, o);
        yc += __shfl_xor(yc, o);
    }
    __syncthreads();
    if (rl == 0) {
        sh[sub] = vty;
        sh[4 + sub] = yc;
    }
    // this wave's share of V[r][:j] q1 + W[r][:j] q2
    T pwv = T(0);
#pragma unroll
    for (int u = 0; u < QW; ++u) pwv += vr[u] * qs[QW * sub + u] + wr[u] * qs[NB + QW * sub + u];
    pw[sub][rl] = pwv;
    __syncthreads();
    vty = (sh[0] + sh[1]) + (sh[2] + sh[3]);
    yc = (sh[4] + sh[5]) + (sh[6] + sh[7]);
    T q12 = T(0);
    for (int k = 0; k < j; ++k) q12 += qs[k] * qs[NB + k];
    const T half = T(0.5) * tv * (tv * (vty - T(2) * q12));
    if (next && t < NB) {  // row c+1 of the panel, with W[c+1][j] from y[c+1]
        const int q = t;
        T wv = q < j ? w1row : T(0);
        if (q == j) {
            T w = yc;
            for (int k = 0; k < j; ++k) w -= v1s[k] * qs[k] + w1s[k] * qs[NB + k];
            wv = tv * w - half * v1row;
        }
        wc[q] = wv;
        vc[q] = q <= j ? v1row : T(0);
    }
    const T w = ((ys[0][rl] + ys[1][rl]) + (ys[2][rl] + ys[3][rl])) -
                ((pw[0][rl] + pw[1][rl]) + (pw[2][rl] + pw[3][rl]));
    const T wj = tv * w - half * vj;
    if (sub == 0 && live) Wp[int64_t(j) * n + r] = wj;
    if (!next) return;
    __syncthreads();
    // row c+1 of the current matrix, corrected by the panel's first j+1 columns (W[r][j] = wj)
#pragma unroll
    for (int u = 0; u < QW; ++u)
        if (QW * sub + u == j) wr[u] = wj;
    T pav = T(0);
#pragma unroll
    for (int u = 0; u < QW; ++u) pav += vr[u] * wc[QW * sub + u] + wr[u] * vc[QW * sub + u];
    pa[sub][rl] = pav;
    __syncthreads();
    const T a = aold - ((pa[0][rl] + pa[1][rl]) + (pa[2][rl] + pa[3][rl]));
    if (sub == 0 && live) {
        A[(c + 1) * lda + r] = a;
        colbuf[r] = a;
        if (r == c + 1) d[c + 1] = double(a);
    }
    const bool tailrow = live && r >= c + 3;  // rows of x[2:]
    T ss = (sub == 0 && tailrow) ? a * a : T(0);
    // W^T x and V^T x over the block's rows: this wave's 2 QW values summed over its 64 lanes by a
    // reduce-scatter over lane bits 5 .. 2 and a sum over bits 1, 0; lane l ends with value
    // (l >> 2) & 15: W part for values 0 .. QW-1, V part for QW .. 2 QW - 1
    static_assert(QW == 8, "reduce-scatter layout");
    T pq[2 * QW];
#pragma unroll
    for (int u = 0; u < QW; ++u) {
        pq[u] = tailrow ? wr[u] * a : T(0);
        pq[QW + u] = tailrow ? vr[u] * a : T(0);
    }
    rs_step<8, 32>(pq, rl);
    rs_step<4, 16>(pq, rl);
    rs_step<2, 8>(pq, rl);
    rs_step<1, 4>(pq, rl);
    T qsum = pq[0];
    qsum += __shfl_xor(qsum, 2);
    qsum += __shfl_xor(qsum, 1);
    ss = block_sum(ss, sh);
    if (t == 0) part[blockIdx.x] = ss;
    if ((rl & 3) == 0) {
        const int v = (rl >> 2) & 15;
        const int idx = v < QW ? QW * sub + v : NB + QW * sub + (v - QW);
        qcol[int64_t(blockIdx.x) * 2 * NB + idx] = qsum;
    }
}

// The last m = n - p0 columns of the tridiagonalisation by one workgroup (the whole matrix when
// p0 = 0), with the trailing block's upper triangle packed in LDS: row i of the block holds A(i, j),
// j >= i, at rb(i) + j, rb(i) = i (2m - i - 1) / 2.  Same reflectors as the column chain above
// (H_c = I - tau v v^T, v[c+1] = 1), unblocked.  Per column c = p0 + k, with L = m - k - 1, the
// trailing indices a, b < L and x the block's row k right of the diagonal:
//   beta, tau, v from x: every wave forms ||x[1:]||^2 itself (the same sum in the same order) and
//     every lane takes v[a] = x[a] / (alpha - beta) from LDS where it needs it, so no barrier;
//   wave w loads its rows b = w, w + 16, ... (entries a >= b, lane l holding a = l + 64 u) into
//     registers, all at once; from them, p = tau A_t v as row parts sum_{a>=b} A(b, a) v[a] (summed
//     over each 16-lane row by DPP, four sums per row to LDS) and column parts sum_{b<a} A(b, a) v[b]
//     (accumulated per lane over the wave's rows, one vector per wave to LDS); barrier; the parts
//     added in a fixed order, four lanes per entry; barrier;
//   w = p - (tau/2)(p^T v) v (p^T v formed by every wave), A_t -= v w^T + w v^T from the rows still in
//     registers; barrier.
// Each stored entry is read once per column, a wave's accesses to the triangle are to consecutive
// entries, and its loads are all in flight together.  Three barriers per column instead of two
// launches.
template <class T>
struct TrdSmall {
    static constexpr int NMAX = sizeof(T) == 4 ? 256 : 176;  // triangle + partial sums within 160 KiB
    static constexpr int RPW = (NMAX + 15) / 16;             // rows per wave
    static constexpr int CH = (NMAX + 63) / 64;              // 64-entry chunks of a row
    static size_t smem(int m) { return (size_t(m) * size_t(m + 1) / 2 + 21 * size_t(m)) * sizeof(T); }
};
constexpr int TRS_THREADS = 1024;

template <int CTRL>
__device__ __forceinline__ float trs_dpp(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, false));
}
template <int CTRL>
__device__ __forceinline__ double trs_dpp(double v) {
    const int lo = __builtin_amdgcn_mov_dpp(__double2loint(v), CTRL, 0xf, 0xf, false);
    const int hi = __builtin_amdgcn_mov_dpp(__double2hiint(v), CTRL, 0xf, 0xf, false);
    return __hiloint2double(hi, lo);
}
__device__ __forceinline__ float trs_lane(float v, int l) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l)); }
__device__ __forceinline__ double trs_lane(double v, int l) {
    return __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(v), l), __builtin_amdgcn_readlane(__double2loint(v), l));
}
// sums over the four lanes of a quad and over each row of 16 lanes, the same value in each lane
// (every step adds a lane pair both ways)
template <class T>
__device__ __forceinline__ T trs_quad_sum(T v) {
    v += trs_dpp<0xB1>(v);        // quad_perm [1, 0, 3, 2]
    return v + trs_dpp<0x4E>(v);  // quad_perm [2, 3, 0, 1]
}
template <class T>
__device__ __forceinline__ T trs_row16_sum(T v) {
    v = trs_quad_sum(v);
    v += trs_dpp<0x141>(v);        // row_half_mirror
    return v + trs_dpp<0x140>(v);  // row_mirror
}
// sum over the 64 lanes, the same value in each: the four row sums added in a fixed order
template <class T>
__device__ __forceinline__ T trs_wave_sum(T v) {
    v = trs_row16_sum(v);
    return (trs_lane(v, 0) + trs_lane(v, 16)) + (trs_lane(v, 32) + trs_lane(v, 48));
}

template <class T>
__global__ void __launch_bounds__(TRS_THREADS) k_trd_small(const T *__restrict__ A, int64_t lda, int64_t n, int64_t p0,
                                                         T *__restrict__ Rt, T *__restrict__ tau,
                                                         double *__restrict__ d, double *__restrict__ e, int64_t zs) {
    using S = TrdSmall<T>;
    A = zoff(A, zs);
    Rt = zoff(Rt, zs);
    tau = zoff(tau, zs);
    d = zoff(d, zs);
    e = zoff(e, zs);
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int m = int(n - p0);
    constexpr int NW = TRS_THREADS / 64;
    T *P = reinterpret_cast<T *>(smem);
    T *cpw = P + m * (m + 1) / 2;  // column parts, one vector of m per wave
    T *rp4 = cpw + NW * m;         // row parts, four per entry
    T *pp = rp4 + 4 * m;           // p
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    auto rb = [m](int i) { return i * (2 * m - i - 1) / 2; };
    for (int i = wave; i < m; i += NW) {
        const T *src = A + (p0 + i) * lda + p0;
        T *dst = P + rb(i);
        for (int j = i + lane; j < m; j += 64) dst[j] = src[j];
    }
    __syncthreads();
    for (int k = 0; k < m - 1; ++k) {
        const int64_t c = p0 + k;
        const int L = m - k - 1, k1 = k + 1;
        const T *x = P + rb(k) + k1;  // x[a] = A(k, k + 1 + a), a < L
        T s2 = T(0);
        for (int a = 1 + lane; a < L; a += 64) s2 += x[a] * x[a];
        s2 = trs_wave_sum(s2);
        const T alpha = x[0];
        T beta, tv, scale;
        if (s2 == T(0)) {
            tv = T(0);
            beta = alpha;
            scale = T(0);
        } else {
            const T nrm = sqrt(alpha * alpha + s2);
            beta = alpha >= T(0) ? -nrm : nrm;
            tv = (beta - alpha) / beta;
            scale = T(1) / (alpha - beta);
        }
        auto v = [&](int a) -> T { return a == 0 ? T(1) : x[a] * scale; };
        if (tid == 0) {
            d[c] = double(P[rb(k) + k]);
            e[c] = double(beta);
            tau[c] = tv;
        }
        for (int64_t r = tid; r < n; r += TRS_THREADS) Rt[c * n + r] = r <= c ? T(0) : v(int(r - c - 1));
        T vj[S::CH];  // v of this lane's entries a = lane + 64 u
#pragma unroll
        for (int u = 0; u < S::CH; ++u) vj[u] = lane + 64 * u < L ? v(lane + 64 * u) : T(0);
        // this wave's rows, entries a >= b of row b, all loaded before any is used
        T el[S::RPW][S::CH];
#pragma unroll
        for (int t = 0; t < S::RPW; ++t) {
            const int b = wave + NW * t;
            const T *row = P + rb(k1 + (b < L ? b : 0)) + k1;
#pragma unroll
            for (int u = 0; u < S::CH; ++u) {
                const int a = lane + 64 * u;
                el[t][u] = (b < L && a >= b && a < L) ? row[a] : T(0);
            }
        }
        T cacc[S::CH];
#pragma unroll
        for (int u = 0; u < S::CH; ++u) cacc[u] = T(0);
#pragma unroll
        for (int t = 0; t < S::RPW; ++t) {
            const int b = wave + NW * t;
            if (b >= L) break;  // wave-uniform
            T rs = T(0);
#pragma unroll
            for (int u = 0; u < S::CH; ++u) rs += el[t][u] * vj[u];
            rs = trs_row16_sum(rs);
            if ((lane & 15) == 0) rp4[b * 4 + (lane >> 4)] = rs;
            const T vb = v(b);
#pragma unroll
            for (int u = 0; u < S::CH; ++u)
                if (lane + 64 * u > b) cacc[u] += el[t][u] * vb;
        }
#pragma unroll
        for (int u = 0; u < S::CH; ++u)
            if (lane + 64 * u < m) cpw[wave * m + lane + 64 * u] = cacc[u];
        __syncthreads();
        {  // p[a] = tau (row part + column parts of the 16 waves), lane g of a's four adding four waves
            const int a = tid >> 2, g = tid & 3;
            T sp = T(0);
            if (a < L) {
                sp = rp4[a * 4 + g];
#pragma unroll
                for (int w = 0; w < 4; ++w) sp += cpw[(4 * g + w) * m + a];
            }
            sp = trs_quad_sum(sp);
            if (g == 0 && a < L) pp[a] = tv * sp;
        }
        __syncthreads();
        T pv = T(0);
#pragma unroll
        for (int u = 0; u < S::CH; ++u)
            if (lane + 64 * u < L) pv += pp[lane + 64 * u] * vj[u];
        pv = trs_wave_sum(pv);
        const T K = T(0.5) * tv * pv;
        T wj[S::CH];
#pragma unroll
        for (int u = 0; u < S::CH; ++u) wj[u] = lane + 64 * u < L ? pp[lane + 64 * u] - K * vj[u] : T(0);
#pragma unroll
        for (int t = 0; t < S::RPW; ++t) {
            const int b = wave + NW * t;
            if (b >= L) break;
            const T vb = v(b), wb = pp[b] - K * vb;
            T *row = P + rb(k1 + b) + k1;
#pragma unroll
            for (int u = 0; u < S::CH; ++u) {
                const int a = lane + 64 * u;
                if (a >= b && a < L) row[a] = el[t][u] - (vb * wj[u] + wb * vj[u]);
            }
        }
        __syncthreads();
    }
    if (tid == 0) d[n - 1] = double(P[rb(m - 1) + m - 1]);
}

// Rank-2 jn update of the trailing matrix, A[r][s] -= sum_q V[r][q] W[s][q] + W[r][q] V[s][q] for
// p <= r, s < n, over the 64 x 64 tiles (I, J) with I <= J (block u: column J, row I, numbered
// column by column).  A tile is the product [V_I W_I] [W_J V_J]^T, a contraction of length 2 NB
// (panel columns q >= jn are zero), staged k-major in LDS and formed on MFMA by 4 waves of
// 32 x 32: fp32 32x32x2 (one product per lane and k slice), fp64 16x16x4 (2 x 2 products).
// The lower half of a diagonal tile is updated too and never read; the padding columns [n, lda)
// are left alone.
template <class T>
struct TrailMfma;
template <>
struct TrailMfma<float> {
    typedef f32x16_t acc_t[1][1];
    static __device__ __forceinline__ void zero(acc_t &c) { c[0][0] = f32x16_t{}; }
    template <int LD>
    static __device__ __forceinline__ void run(const float (*ar)[LD], const float (*bs)[LD], int wr, int wc, int lane,
                                               acc_t &c) {
#pragma unroll 8
        for (int k = 0; k < 2 * NB; k += 2) {
            const float a = ar[k + (lane >> 5)][wr + (lane & 31)];
            const float b = bs[k + (lane >> 5)][wc + (lane & 31)];
            c[0][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c[0][0], 0, 0, 0);
        }
    }
    // element r of the lane: row and column within the wave's 32 x 32 tile
    static __device__ __forceinline__ int row(int x, int r, int lane) { return (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3); }
    static __device__ __forceinline__ int col(int y, int lane) { return lane & 31; }
    static __device__ __forceinline__ float get(const acc_t &c, int x, int y, int r) { return c[0][0][r]; }
    static constexpr int NX = 1, NR = 16;
};
template <>
struct TrailMfma<double> {
    typedef f64x4_t acc_t[2][2];
    static __device__ __forceinline__ void zero(acc_t &c) {
#pragma unroll
        for (int x = 0; x < 2; ++x)
#pragma unroll
            for (int y = 0; y < 2; ++y) c[x][y] = f64x4_t{0.0, 0.0, 0.0, 0.0};
    }
    template <int LD>
    static __device__ __forceinline__ void run(const double (*ar)[LD], const double (*bs)[LD], int wr, int wc, int lane,
                                               acc_t &c) {
#pragma unroll 4
        for (int k = 0; k < 2 * NB; k += 4) {
            const int kk = k + (lane >> 4);
            const double a0 = ar[kk][wr + (lane & 15)], a1 = ar[kk][wr + 16 + (lane & 15)];
            const double b0 = bs[kk][wc + (lane & 15)], b1 = bs[kk][wc + 16 + (lane & 15)];
            c[0][0] = __builtin_amdgcn_mfma_f64_16x16x4f64(a0, b0, c[0][0], 0, 0, 0);
            c[0][1] = __builtin_amdgcn_mfma_f64_16x16x4f64(a0, b1, c[0][1], 0, 0, 0);
            c[1][0] = __builtin_amdgcn_mfma_f64_16x16x4f64(a1, b0, c[1][0], 0, 0, 0);
            c[1][1] = __builtin_amdgcn_mfma_f64_16x16x4f64(a1, b1, c[1][1], 0, 0, 0);
        }
    }
    static __device__ __forceinline__ int row(int x, int r, int lane) { return x * 16 + r * 4 + (lane >> 4); }
    static __device__ __forceinline__ int col(int y, int lane) { return y * 16 + (lane & 15); }
    static __device__ __forceinline__ double get(const acc_t &c, int x, int y, int r) { return c[x][y][r]; }
    static constexpr int NX = 2, NR = 4;
};

template <class T>
__global__ void __launch_bounds__(256) k_trailing(T *__restrict__ A, int64_t lda, int64_t n, int64_t p, int jn,
                                                  const T *__restrict__ Vp, const T *__restrict__ Wp, int64_t zs) {
    using M = TrailMfma<T>;
    A = zoff(A, zs);
    Vp = zoff(Vp, zs);
    Wp = zoff(Wp, zs);
    constexpr int LD = 64 + 4;
    __shared__ T ar[2 * NB][LD], bs[2 * NB][LD];
    const int u = blockIdx.x;
    int J = int((sqrtf(8.f * float(u) + 1.f) - 1.f) * 0.5f);
    while (J * (J + 1) / 2 > u) --J;
    while ((J + 1) * (J + 2) / 2 <= u) ++J;
    const int I = u - J * (J + 1) / 2;
    const int64_t r0 = p + int64_t(I) * 64, s0 = p + int64_t(J) * 64;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int wr = (wv >> 1) * 32, wc = (wv & 1) * 32;
    // every load first (one round trip): the operands, k-major (ar[k][i] = V[r0+i][k] for k < NB,
    // W[r0+i][k-NB] above; bs[k][j] = W[s0+j][k], V[s0+j][k-NB]), and this lane's entries of A
    constexpr int PER = 2 * NB * 64 / 256;
    T va[PER], vb[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) {
        const int e = threadIdx.x + 256 * u;
        const int k = e >> 6, i = e & 63, q = k % NB;
        const bool hiq = k >= NB;
        const bool okr = r0 + i < n && q < jn, oks = s0 + i < n && q < jn;
        va[u] = okr ? (hiq ? Wp : Vp)[int64_t(q) * n + r0 + i] : T(0);
        vb[u] = oks ? (hiq ? Vp : Wp)[int64_t(q) * n + s0 + i] : T(0);
    }
    T aold[M::NX][M::NX][M::NR];
#pragma unroll
    for (int x = 0; x < M::NX; ++x)
#pragma unroll
        for (int y = 0; y < M::NX; ++y) {
            const int64_t sc = s0 + wc + M::col(y, lane);
#pragma unroll
            for (int r = 0; r < M::NR; ++r) {
                const int64_t rr = r0 + wr + M::row(x, r, lane);
                aold[x][y][r] = (rr < n && sc < n) ? A[rr * lda + sc] : T(0);
            }
        }
#pragma unroll
    for (int u = 0; u < PER; ++u) {
        const int e = threadIdx.x + 256 * u;
        ar[e >> 6][e & 63] = va[u];
        bs[e >> 6][e & 63] = vb[u];
    }
    __syncthreads();
    typename M::acc_t acc;
    M::zero(acc);
    M::template run<LD>(ar, bs, wr, wc, lane, acc);
#pragma unroll
    for (int x = 0; x < M::NX; ++x)
#pragma unroll
        for (int y = 0; y < M::NX; ++y) {
            const int64_t sc = s0 + wc + M::col(y, lane);
#pragma unroll
            for (int r = 0; r < M::NR; ++r) {
                const int64_t rr = r0 + wr + M::row(x, r, lane);
                if (rr < n && sc < n) A[rr * lda + sc] = aold[x][y][r] - M::get(acc, x, y, r);
            }
        }
}

// ---------------------------------------------------------------------------------------------
// 2. bisection (fp64)
// ---------------------------------------------------------------------------------------------
// 1/q from the hardware estimate and one Newton step, r1 = r0 (2 - q r0) (the estimate's relative
// error squared, so within a few units in the last place); a correctly rounded division is a
// chain about three times as long, and the Sturm recurrence is one such step after another.
__device__ __forceinline__ double recip_nr(double q) {
    const double r0 = __builtin_amdgcn_rcp(q);
    return fma(r0, fma(-q, r0, 1.0), r0);
}

// number of eigenvalues of T strictly less than x (Sturm sequence of the LDL^T of T - x I); the
// pivots stay away from zero (|q| >= pivmin), so 1/q is finite
__device__ __forceinline__ int sturm_count(const double *__restrict__ d, const double *__restrict__ e2, int64_t n,
                                           double x, double pivmin) {
    int cnt = 0;
    double q = d[0] - x;
    if (fabs(q) < pivmin) q = -pivmin;
    if (q < 0.0) ++cnt;
    int64_t i = 1;
    // 8 steps at a time with their loads issued first (they do not depend on the recurrence)
    for (; i + 8 <= n; i += 8) {
        double dd[8], ee[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            dd[u] = d[i + u];
            ee[u] = e2[i + u - 1];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            q = (dd[u] - x) - ee[u] * recip_nr(q);
            if (fabs(q) < pivmin) q = -pivmin;
            if (q < 0.0) ++cnt;
        }
    }
    for (; i < n; ++i) {
        q = (d[i] - x) - e2[i - 1] * recip_nr(q);
        if (fabs(q) < pivmin) q = -pivmin;
        if (q < 0.0) ++cnt;
    }
    return cnt;
}

__global__ void k_tri_prep(const double *__restrict__ d, const double *__restrict__ e, int64_t n, double *__restrict__ e2,
                           double *__restrict__ bounds, int64_t zs) {
    d = zoff(d, zs);
    e = zoff(e, zs);
    e2 = zoff(e2, zs);
    bounds = zoff(bounds, zs);
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
                                                const double *__restrict__ bounds, double *__restrict__ lam_asc,
                                                int64_t zs) {
    d = zoff(d, zs);
    e2 = zoff(e2, zs);
    bounds = zoff(bounds, zs);
    lam_asc = zoff(lam_asc, zs);
    const int64_t gid = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t i = gid / MSEC;
    const int sub = int(gid % MSEC);
    if (i >= n) return;  // whole groups leave together (n * MSEC threads rounded to blocks)
    double lo = bounds[0], hi = bounds[1];
    const double pivmin = bounds[2];
    // stop at a width of 1e-13 relative plus 1e-13 ||T|| absolute: about 11 passes from the
    // Gershgorin interval, far below the working precision of the matrix the eigenvalues come from
    const double atol = 1e-13 * bounds[3];
    for (int it = 0; it < 24; ++it) {
        if (hi - lo <= 1e-13 * fmax(fabs(lo), fabs(hi)) + atol) break;
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

// Rows of a sweep in batches of IB, the next batch's loads in flight while the current one is
// processed.  The loads use clamped (always valid) row indices, so they are unconditional; the
// processing step skips rows outside the sweep.
constexpr int IB = 8;
template <class Buf, class Load, class Proc>
__device__ __forceinline__ void sweep_pipelined(int64_t nbatch, const Load &load, const Proc &proc) {
    Buf s0, s1;
    load(int64_t(0), s0);
    int64_t b = 0;
    for (; b + 1 < nbatch; b += 2) {
        load(b + 1, s1);
        proc(b, s0);
        load(b + 2, s0);
        proc(b + 1, s1);
    }
    if (b < nbatch) proc(b, s0);
}

__global__ void __launch_bounds__(64) k_invit(const double *__restrict__ d, const double *__restrict__ e, int64_t n,
                                              const double *__restrict__ lam_asc, const double *__restrict__ bounds,
                                              int64_t nv, double *__restrict__ Z, double2 *__restrict__ PU,
                                              double2 *__restrict__ PD, uint8_t *__restrict__ SW, int64_t zs) {
    d = zoff(d, zs);
    e = zoff(e, zs);
    lam_asc = zoff(lam_asc, zs);
    bounds = zoff(bounds, zs);
    Z = zoff(Z, zs);
    PU = zoff(PU, zs);
    PD = zoff(PD, zs);
    SW = zoff(SW, zs);
    const int64_t j = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (j >= nv) return;
    const double lam = lam_asc[n - 1 - j];
    const double tnorm = bounds[3];
    const double tiny = DBL_EPSILON * fmax(tnorm, DBL_MIN);
    auto at = [&](int64_t k) { return k * nv + j; };
    // LU with partial pivoting of T - lam I, once: row k of U in PU[k] = (U1, U2) and PD[k].x = 1/U0,
    // the multiplier of step k in PD[k].y and whether rows k, k+1 were swapped in SW[k]; the start
    // vector is eliminated on the way.  The entries of T for IB steps are loaded first.
    double u0 = d[0] - lam, u1 = n > 1 ? e[0] : 0.0, u2 = 0.0;
    double bcur = hash_unit(uint64_t(j) + 1);
    for (int64_t k0 = 0; k0 < n - 1; k0 += IB) {
        double ev[IB + 1], dv[IB];
#pragma unroll
        for (int u = 0; u <= IB; ++u) ev[u] = k0 + u < n - 1 ? e[k0 + u] : 0.0;
#pragma unroll
        for (int u = 0; u < IB; ++u) dv[u] = k0 + u + 1 < n ? d[k0 + u + 1] : 0.0;
#pragma unroll
        for (int u = 0; u < IB; ++u) {
            const int64_t k = k0 + u;
            if (k >= n - 1) break;
            const double l = ev[u], dd = dv[u] - lam, ee = ev[u + 1];  // ev[u + 1] = e[k + 1], 0 past the end
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
            PU[at(k)] = double2{p1, p2};
            PD[at(k)] = double2{1.0 / p0, mlt};
            SW[at(k)] = sw;
            Z[at(k)] = bp;
        }
    }
    if (u0 == 0.0) u0 = tiny;
    PD[at(n - 1)] = double2{1.0 / u0, 0.0};
    Z[at(n - 1)] = bcur;
    // three steps of inverse iteration; each back substitution's result is scaled by 1/max when
    // it is read by the next sweep (the elimination of the next step, or the final normalisation)
    struct EBuf {
        double bn[IB];
        double2 pd[IB];
        uint8_t sw[IB];
    };
    struct BBuf {
        double z[IB];
        double2 pu[IB], pd[IB];
    };
    double scl = 1.0;
    const int64_t nb = (n - 1 + IB - 1) / IB;  // batches over rows 0 .. n-2
    for (int iter = 0; iter < 3; ++iter) {
        if (iter > 0) {  // apply the stored elimination to the new right-hand side, rows 0 .. n-2
            double bc = Z[at(0)] * scl;
            sweep_pipelined<EBuf>(
                nb,
                [&](int64_t bt, EBuf &B) {
#pragma unroll
                    for (int u = 0; u < IB; ++u) {
                        const int64_t k = min(bt * IB + u, n - 2);
                        B.bn[u] = Z[at(k + 1)];
                        B.pd[u] = PD[at(k)];
                        B.sw[u] = SW[at(k)];
                    }
                },
                [&](int64_t bt, const EBuf &B) {
#pragma unroll
                    for (int u = 0; u < IB; ++u) {
                        const int64_t k = bt * IB + u;
                        if (k >= n - 1) break;
                        const double bn = B.bn[u] * scl, mlt = B.pd[u].y;
                        if (B.sw[u]) {
                            Z[at(k)] = bn;
                            bc = bc - mlt * bn;
                        } else {
                            Z[at(k)] = bc;
                            bc = bn - mlt * bc;
                        }
                    }
                });
            Z[at(n - 1)] = bc;
        }
        // back substitution with U, rows n-2 .. 0; the largest entry sets the next scale
        double y2 = 0.0, y1 = Z[at(n - 1)] * PD[at(n - 1)].x, ymax = fabs(y1);
        Z[at(n - 1)] = y1;
        sweep_pipelined<BBuf>(
            nb,
            [&](int64_t bt, BBuf &B) {
#pragma unroll
                for (int u = 0; u < IB; ++u) {
                    const int64_t k = max(n - 2 - (bt * IB + u), int64_t(0));
                    B.z[u] = Z[at(k)];
                    B.pu[u] = PU[at(k)];
                    B.pd[u] = PD[at(k)];
                }
            },
            [&](int64_t bt, const BBuf &B) {
#pragma unroll
                for (int u = 0; u < IB; ++u) {
                    const int64_t k = n - 2 - (bt * IB + u);
                    if (k < 0) break;
                    const double y = (B.z[u] - B.pu[u].x * y1 - B.pu[u].y * y2) * B.pd[u].x;
                    Z[at(k)] = y;
                    ymax = fmax(ymax, fabs(y));
                    y2 = y1;
                    y1 = y;
                }
            });
        scl = ymax > 0.0 ? 1.0 / ymax : 1.0;
    }
    // normalise: sum of squares (eight running sums, 32 loads at a time), then the scaled vector
    constexpr int NQ = 32;
    double s8[8] = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0};
    for (int64_t r0 = 0; r0 < n; r0 += NQ) {
        double z[NQ];
#pragma unroll
        for (int u = 0; u < NQ; ++u) z[u] = Z[at(min(r0 + u, n - 1))] * scl;
#pragma unroll
        for (int u = 0; u < NQ; ++u)
            if (r0 + u < n) s8[u % 8] += z[u] * z[u];
    }
    const double s2 = ((s8[0] + s8[1]) + (s8[2] + s8[3])) + ((s8[4] + s8[5]) + (s8[6] + s8[7]));
    const double inv = s2 > 0.0 ? scl / sqrt(s2) : 0.0;
    for (int64_t r0 = 0; r0 < n; r0 += NQ) {
        double z[NQ];
#pragma unroll
        for (int u = 0; u < NQ; ++u) z[u] = Z[at(min(r0 + u, n - 1))];
#pragma unroll
        for (int u = 0; u < NQ; ++u)
            if (r0 + u < n) Z[at(r0 + u)] = z[u] * inv;
    }
}

// Re-orthogonalise clusters: vector j starts a cluster when lam_{j-1} - lam_j > ctol; the leader's
// block runs modified Gram-Schmidt over its cluster members in order.
__global__ void __launch_bounds__(256) k_cluster_mgs(const double *__restrict__ lam_asc, int64_t n, int64_t nv,
                                                     const double *__restrict__ bounds, double *__restrict__ Z,
                                                     int64_t zs) {
    lam_asc = zoff(lam_asc, zs);
    bounds = zoff(bounds, zs);
    Z = zoff(Z, zs);
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
// T factor of every block of NBT reflectors in one launch (block b = blockIdx.x, reflectors
// c0 = b NBT ...): S = V_b^T V_b over the block's rows (fixed order: per-thread strided sums, then a
// fixed tree), then T forward, column by column: T[0:i, i] = -tau_i T[0:i, 0:i] S[0:i, i], T[i][i] =
// tau_i.  V_b is rows c0 .. c0+nb-1 of Rt, nonzero from column c0+1 on.
template <class T>
__global__ void __launch_bounds__(256) k_bt_tall(const T *__restrict__ Rt, int64_t ldr, int64_t n, int64_t nrefl,
                                                 const T *__restrict__ tau, double *__restrict__ Tall, int64_t zs) {
    Rt = zoff(Rt, zs);
    tau = zoff(tau, zs);
    Tall = zoff(Tall, zs);
    __shared__ double vs[NBT][65];
    __shared__ double S[NBT][NBT + 1], Tm[NBT][NBT + 1];
    const int64_t c0 = int64_t(blockIdx.x) * NBT;
    const int nb = int(min<int64_t>(NBT, nrefl - c0));
    const int t = threadIdx.x;
    constexpr int PU = NBT * NBT / 256;  // pairs per thread
    double acc[PU];                      // pairs t + 256 u: a = pair / NBT, b = pair % NBT
#pragma unroll
    for (int u = 0; u < PU; ++u) acc[u] = 0.0;
    for (int64_t r0 = c0 + 1; r0 < n; r0 += 64) {
        for (int e = t; e < NBT * 64; e += 256) {
            const int q = e / 64, rr = e % 64;
            const int64_t r = r0 + rr;
            vs[q][rr] = (q < nb && r < n) ? double(Rt[(c0 + q) * ldr + r]) : 0.0;
        }
        __syncthreads();
#pragma unroll
        for (int u = 0; u < PU; ++u) {
            const int pidx = t + 256 * u;
            const int pa = pidx / NBT, pb = pidx % NBT;
            double sacc = 0.0;
            for (int rr = 0; rr < 64; ++rr) sacc += vs[pa][rr] * vs[pb][rr];
            acc[u] += sacc;
        }
        __syncthreads();
    }
#pragma unroll
    for (int u = 0; u < PU; ++u) {
        const int pidx = t + 256 * u;
        S[pidx / NBT][pidx % NBT] = acc[u];
        Tm[pidx / NBT][pidx % NBT] = 0.0;
    }
    __syncthreads();
    for (int i = 0; i < nb; ++i) {
        const double ti = double(tau[c0 + i]);
        double v = 0.0;
        if (t < i)
            for (int k = t; k < i; ++k) v += Tm[t][k] * S[k][i];
        __syncthreads();
        if (t < i) Tm[t][i] = -ti * v;
        if (t == 0) Tm[i][i] = ti;
        __syncthreads();
    }
    double *out = Tall + int64_t(blockIdx.x) * NBT * NBT;
    for (int e = t; e < NBT * NBT; e += 256) out[e] = Tm[e / NBT][e % NBT];
}

// fp64 MFMA tiles of the back-transformation: a workgroup of 4 waves forms a 64 x 64 tile, wave wv
// the 32 x 32 quarter (wr, wc), as 2 x 2 products of 16x16x4 fp64 MFMA.
constexpr int BK = 16;         // contraction step staged in LDS
constexpr int BLD = 64 + 16;   // padded LDS row (doubles)

// acc += sum_{k0 <= k < k1} A(i, k) B(k, j) over the tile.  la(i, k) and lb(k, j) return an operand
// value (0 outside the operand); each thread reads 4 consecutive values of each operand per step,
// along k for A when AK = 1 (A contiguous in k), else along i, and along j for B.  Both operands are
// staged k-major in LDS, and the next step's values are loaded while the current one is multiplied.
template <int AK, class LA, class LB>
__device__ __forceinline__ void bt_mfma(const LA &la, const LB &lb, int64_t k0, int64_t k1, f64x4_t (&acc)[2][2],
                                        double (&As)[BK][BLD], double (&Bs)[BK][BLD]) {
    const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
    const int wr = (wv >> 1) * 32, wc = (wv & 1) * 32;
    double ra[4], rb[4];
    auto gload = [&](int64_t kb) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            if (AK) ra[u] = la(t >> 2, kb + (t & 3) * 4 + u);
            else ra[u] = la((t & 15) * 4 + u, kb + (t >> 4));
            rb[u] = lb(kb + (t >> 4), (t & 15) * 4 + u);
        }
    };
    gload(k0);
    for (int64_t kb = k0; kb < k1; kb += BK) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            if (AK) As[(t & 3) * 4 + u][t >> 2] = ra[u];
            else As[t >> 4][(t & 15) * 4 + u] = ra[u];
            Bs[t >> 4][(t & 15) * 4 + u] = rb[u];
        }
        __syncthreads();
        if (kb + BK < k1) gload(kb + BK);
#pragma unroll
        for (int ks = 0; ks < BK / 4; ++ks) {
            // operands: lane i + 16 kq holds row (or column) i of k-slice kq
            const int kk = ks * 4 + (lane >> 4);
            const double a0 = As[kk][wr + (lane & 15)], a1 = As[kk][wr + 16 + (lane & 15)];
            const double b0 = Bs[kk][wc + (lane & 15)], b1 = Bs[kk][wc + 16 + (lane & 15)];
            acc[0][0] = __builtin_amdgcn_mfma_f64_16x16x4f64(a0, b0, acc[0][0], 0, 0, 0);
            acc[0][1] = __builtin_amdgcn_mfma_f64_16x16x4f64(a0, b1, acc[0][1], 0, 0, 0);
            acc[1][0] = __builtin_amdgcn_mfma_f64_16x16x4f64(a1, b0, acc[1][0], 0, 0, 0);
            acc[1][1] = __builtin_amdgcn_mfma_f64_16x16x4f64(a1, b1, acc[1][1], 0, 0, 0);
        }
        __syncthreads();
    }
}

// accumulator r of a lane holds row 4 r + lane / 16, column lane % 16 of its 16 x 16 product
__device__ __forceinline__ int bt_row(int x, int r) { return ((threadIdx.x >> 7) * 32) + x * 16 + r * 4 + ((threadIdx.x & 63) >> 4); }
__device__ __forceinline__ int bt_col(int y) { return (((threadIdx.x >> 6) & 1) * 32) + y * 16 + (threadIdx.x & 15); }

// partial G[q][col] = sum of Rt[c0+q][r] Z[r][col] over rows r of chunk y, rows c0+1 + y rch ..
// (the block's reflectors vanish on rows <= c0); grid (column tiles of 64, chunks)
template <class T>
__global__ void __launch_bounds__(256) k_bt_g(const T *__restrict__ Rt, int64_t ldr, int64_t n, int64_t c0, int nb,
                                              const double *__restrict__ Z, int64_t nv, double *__restrict__ Gp,
                                              int rch, int64_t zs) {
    Rt = zoff(Rt, zs);
    Z = zoff(Z, zs);
    Gp = zoff(Gp, zs);
    __shared__ double As[BK][BLD], Bs[BK][BLD];
    const int64_t j0 = int64_t(blockIdx.x) * 64;
    const int64_t r0 = c0 + 1 + int64_t(blockIdx.y) * rch, r1 = min(r0 + rch, n);
    const T *V = Rt + c0 * ldr;
    f64x4_t acc[2][2];
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int y = 0; y < 2; ++y) acc[x][y] = f64x4_t{0.0, 0.0, 0.0, 0.0};
    bt_mfma<1>([&](int q, int64_t r) { return (q < nb && r < r1) ? double(V[q * ldr + r]) : 0.0; },
               [&](int64_t r, int j) { return (r < r1 && j0 + j < nv) ? Z[r * nv + j0 + j] : 0.0; }, r0, r1, acc, As,
               Bs);
    double *out = Gp + int64_t(blockIdx.y) * NBT * nv;
#pragma unroll
    for (int y = 0; y < 2; ++y) {
        const int64_t col = j0 + bt_col(y);
        if (col < nv)
#pragma unroll
            for (int x = 0; x < 2; ++x)
#pragma unroll
                for (int r = 0; r < 4; ++r) out[int64_t(bt_row(x, r)) * nv + col] = acc[x][y][r];
    }
}

// G = T (sum of the partials): thread (column cl, rows 4 qg .. 4 qg + 3) adds the nchunk partials of
// its 4 values in chunk order, then forms its 4 rows of T G from LDS (T is upper triangular).
// Blocks of 16 columns.
constexpr int GR_COLS = 16;
__global__ void __launch_bounds__(256) k_bt_greduce(const double *__restrict__ Gp, int nchunk, int64_t nv,
                                                    const double *__restrict__ Tf, double *__restrict__ G, int64_t zs) {
    Gp = zoff(Gp, zs);
    Tf = zoff(Tf, zs);
    G = zoff(G, zs);
    __shared__ double Tm[NBT][NBT + 1];
    __shared__ double g[NBT][GR_COLS + 1];
    const int t = threadIdx.x, cl = t % GR_COLS, qg = t / GR_COLS;
    for (int e = t; e < NBT * NBT; e += 256) Tm[e / NBT][e % NBT] = Tf[e];
    const int64_t col = int64_t(blockIdx.x) * GR_COLS + cl;
    double a[4] = {0.0, 0.0, 0.0, 0.0};
    if (col < nv)
        for (int k = 0; k < nchunk; ++k)
#pragma unroll
            for (int u = 0; u < 4; ++u) a[u] += Gp[(int64_t(k) * NBT + 4 * qg + u) * nv + col];
#pragma unroll
    for (int u = 0; u < 4; ++u) g[4 * qg + u][cl] = a[u];
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int q = 4 * qg + u;
        double r = 0.0;
        for (int qq = q; qq < NBT; ++qq) r += Tm[q][qq] * g[qq][cl];
        if (col < nv) G[int64_t(q) * nv + col] = r;
    }
}

// Z[r][col] -= sum_q Rt[c0+q][r] G[q][col] for rows r > c0: 64 x 64 tiles of Z, the contraction over
// the block's nb reflectors on MFMA; grid (column tiles, row tiles from row c0 + 1)
template <class T>
__global__ void __launch_bounds__(256) k_bt_update(const T *__restrict__ Rt, int64_t ldr, int64_t n, int64_t c0, int nb,
                                                   const double *__restrict__ G, double *__restrict__ Z, int64_t nv,
                                                   int64_t zs) {
    Rt = zoff(Rt, zs);
    G = zoff(G, zs);
    Z = zoff(Z, zs);
    __shared__ double As[BK][BLD], Bs[BK][BLD];
    const int64_t j0 = int64_t(blockIdx.x) * 64, i0 = c0 + 1 + int64_t(blockIdx.y) * 64;
    const T *V = Rt + c0 * ldr + i0;
    f64x4_t acc[2][2];
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int y = 0; y < 2; ++y) acc[x][y] = f64x4_t{0.0, 0.0, 0.0, 0.0};
    bt_mfma<0>([&](int i, int64_t q) { return (q < nb && i0 + i < n) ? double(V[q * ldr + i]) : 0.0; },
               [&](int64_t q, int j) { return (q < nb && j0 + j < nv) ? G[q * nv + j0 + j] : 0.0; }, 0, nb, acc, As,
               Bs);
#pragma unroll
    for (int y = 0; y < 2; ++y) {
        const int64_t col = j0 + bt_col(y);
        if (col < nv)
#pragma unroll
            for (int x = 0; x < 2; ++x)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int64_t row = i0 + bt_row(x, r);
                    if (row < n) Z[row * nv + col] -= acc[x][y][r];
                }
    }
}

// ---------------------------------------------------------------------------------------------
// 5. signs and output
// ---------------------------------------------------------------------------------------------
// Sign rule and fp32 output: column j of V (from Z, n x nv fp64) is scaled by the sign of its entry
// of largest magnitude (the first such row on ties; NaN entries never win), and with Z2 != NULL
// column j of A (from Z2, n2 x nv) takes the same sign.  A workgroup takes 16 columns, its 64 row
// groups stride down them, so every row's 16 values come in one 128-byte run; the per-group
// maxima are combined in a fixed tree with the same tie rule.  NaN everywhere when *bad is set.
constexpr int SG_COLS = 16, SG_ROWS = 64;
__global__ void __launch_bounds__(SG_COLS * SG_ROWS) k_sign_cols(const double *__restrict__ Z, int64_t n, int64_t nv,
                                                               float *__restrict__ V, int64_t ldv,
                                                               const double *__restrict__ Z2, int64_t n2,
                                                               float *__restrict__ A, int64_t lda, const int *bad) {
    __shared__ double sb[SG_ROWS][SG_COLS];
    __shared__ int si[SG_ROWS][SG_COLS];
    __shared__ double sg[SG_COLS];
    const int t = threadIdx.x, jc = t % SG_COLS, rg = t / SG_COLS;
    const int64_t j = int64_t(blockIdx.x) * SG_COLS + jc;
    const bool live = j < nv;
    double best = -1.0;
    int64_t bi = n;
    if (live) {
#pragma unroll 8
        for (int64_t r = rg; r < n; r += SG_ROWS) {
            const double a = fabs(Z[r * nv + j]);
            if (a > best) {
                best = a;
                bi = r;
            }
        }
    }
    sb[rg][jc] = best;
    si[rg][jc] = int(bi);
    __syncthreads();
    for (int o = SG_ROWS / 2; o > 0; o >>= 1) {
        if (rg < o) {
            const double ob = sb[rg + o][jc];
            const int oi = si[rg + o][jc];
            if (ob > sb[rg][jc] || (ob == sb[rg][jc] && oi < si[rg][jc])) {
                sb[rg][jc] = ob;
                si[rg][jc] = oi;
            }
        }
        __syncthreads();
    }
    if (rg == 0) sg[jc] = (live && si[0][jc] < n && Z[int64_t(si[0][jc]) * nv + j] < 0.0) ? -1.0 : 1.0;
    __syncthreads();
    if (!live) return;
    const double sgn = sg[jc];
    const bool isbad = *bad != 0;
    for (int64_t r = rg; r < n; r += SG_ROWS) V[r * ldv + j] = isbad ? NAN : float(sgn * Z[r * nv + j]);
    if (Z2)
        for (int64_t r = rg; r < n2; r += SG_ROWS) A[r * lda + j] = isbad ? NAN : float(sgn * Z2[r * nv + j]);
}

static void sign_out(const double *Z, int64_t n, int64_t nv, float *V, int64_t ldv, const int *bad, hipStream_t s,
                     const double *Z2 = nullptr, int64_t n2 = 0, float *A = nullptr, int64_t lda = 0) {
    hipLaunchKernelGGL(k_sign_cols, dim3(unsigned(cdiv(nv, SG_COLS))), dim3(SG_COLS * SG_ROWS), 0, s, Z, n, nv, V, ldv,
                       Z2, n2, A, lda, bad);
}

__global__ void k_set_info(int32_t *info, const int *bad) {
    if (threadIdx.x == 0) *info = *bad ? LRC_INFO_NONFINITE : LRC_INFO_OK;
}

__global__ void k_zero_i32(int32_t *p) {
    if (threadIdx.x == 0) *p = 0;
}

// ---------------------------------------------------------------------------------------------
// host
// ---------------------------------------------------------------------------------------------
template <class T>
struct LargeWs {
    T *A, *Rt, *Vp, *Wp, *tau, *colbuf, *part, *qcol, *qvec, *spart, *rowpart, *colpart;
    double *d, *e, *e2, *bounds, *lam, *Z, *Tf, *Gp, *G;
    double2 *PU, *PD;  // inverse iteration's LU rows: (U1, U2) and (1/U0, multiplier)
    uint8_t *SW;
    int *bad;
    int64_t lda;
};

template <class T>
static int64_t symv_tiles(int64_t n) { return (n + SymvTile<T>::TS - 1) / SymvTile<T>::TS; }

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
    const int64_t nt = symv_tiles<T>(n);
    w.part = cv.template carve<T>(size_t((n + 63) / 64 + 1));
    w.qcol = cv.template carve<T>(size_t((n + 63) / 64 + 1) * 2 * NB);
    w.qvec = cv.template carve<T>(2 * NB);
    w.spart = cv.template carve<T>(size_t(symv_items(nt, 1)));
    w.rowpart = cv.template carve<T>(size_t(nt) * size_t(nt) * SymvTile<T>::TS);
    w.colpart = cv.template carve<T>(size_t(nt) * size_t(nt) * SymvTile<T>::TS);
    w.d = cv.template carve<double>(size_t(n));
    w.e = cv.template carve<double>(size_t(n));
    w.e2 = cv.template carve<double>(size_t(n));
    w.bounds = cv.template carve<double>(4);
    w.lam = cv.template carve<double>(size_t(n));
    w.Z = cv.template carve<double>(size_t(n) * size_t(nv1));
    w.PU = cv.template carve<double2>(size_t(n) * size_t(nv1));
    w.PD = cv.template carve<double2>(size_t(n) * size_t(nv1));
    w.SW = cv.template carve<uint8_t>(size_t(n) * size_t(nv1));
    w.Tf = cv.template carve<double>(size_t((n + NBT - 1) / NBT) * NBT * NBT);
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

// One matrix's decomposition as a resumable sequence of launches: advance() enqueues the next
// few columns of the tridiagonalisation (or the next blocks of the back-transformation) on the
// job's stream and returns, so that the host can feed several matrices' streams in turn instead
// of blocking on one stream's full queue while the others sit idle.
template <class T>
struct EigJob {
    const float *C = nullptr;
    int64_t ldc = 0, n = 0, ldv = 0, nv = 0;
    double *lambda = nullptr;
    float *V = nullptr;
    int32_t *info = nullptr;
    LargeWs<T> *w = nullptr;
    hipStream_t s = nullptr;
    int stage = 0;  // 0 start, 1 tridiagonalisation, 2 eigenvalues and vectors of T, 3 back-transformation, 4 done
    bool keep_z = false;  // leave the fp64 eigenvectors in w->Z (no sign rule, no fp32 output)
    // lockstep: the tridiagonalisation of nbatch matrices of order n whose workspace regions start
    // zs bytes apart (w is the first one's); such a job stops after stage 1
    unsigned nbatch = 1;
    int64_t zs = 0;
    int NT = 0, npart = 0;
    int64_t p0 = 0, p1 = 0, c = 0, c0 = 0;

    // the last columns by one workgroup in LDS (p0 = 0: the whole matrix), then on to stage 2
    lrc_status small_tail() {
        const size_t sm = TrdSmall<T>::smem(int(n - p0));
        LRC_HIP(hipFuncSetAttribute(reinterpret_cast<const void *>(k_trd_small<T>),
                                    hipFuncAttributeMaxDynamicSharedMemorySize, int(sm)));
        hipLaunchKernelGGL(k_trd_small<T>, dim3(1, 1, nbatch), dim3(TRS_THREADS), sm, s, w->A, w->lda, n, p0, w->Rt,
                           w->tau, w->d, w->e, zs);
        LRC_LAUNCH_CHECK("k_trd_small");
        stage = 2;
        return LRC_OK;
    }
    // stage 1 from column 0 (or the whole tridiagonalisation in LDS for a small order)
    lrc_status begin_tridiagonal() {
        p0 = 0;
        if (n <= TrdSmall<T>::NMAX) return small_tail();
        start_panel();
        stage = 1;
        return LRC_OK;
    }

    void start_panel() {
        p1 = std::min<int64_t>(p0 + NB, n - 1);
        hipLaunchKernelGGL(k_fill_zero<T>, dim3(256, 1, nbatch), dim3(256), 0, s, w->Vp, int64_t(n) * NB, zs);
        hipLaunchKernelGGL(k_fill_zero<T>, dim3(256, 1, nbatch), dim3(256), 0, s, w->Wp, int64_t(n) * NB, zs);
        npart = cdiv(n - p0, 256);
        hipLaunchKernelGGL(k_trd_col0<T>, dim3(npart, 1, nbatch), dim3(256), 0, s, w->A, w->lda, n, p0, w->colbuf,
                           w->part, w->d, zs);
        c = p0;
    }

    // stage 0 up to the tridiagonalisation: the info flag cleared, C copied into A (both
    // triangles' storage, padding zero)
    lrc_status prepare() {
        hipLaunchKernelGGL(k_fill_zero<int>, dim3(1), dim3(64), 0, s, w->bad, int64_t(1), int64_t(0));
        hipLaunchKernelGGL(k_fill_full<T>, dim3(2048), dim3(256), 0, s, C, ldc, n, w->A, w->lda, w->bad);
        LRC_LAUNCH_CHECK("k_fill_full");
        NT = int(symv_tiles<T>(n));
        return LRC_OK;
    }

    void column() {
        const int64_t lda = w->lda;
        const int j = int(c - p0);
        // tiles per symv work item: the largest power of two up to 4 SYMV_TPW that still gives
        // >= SYMV_MIN_ITEMS items (more, smaller items only add dispatch time: workgroups start at
        // about 100 per microsecond)
        const int mt = NT - int((c + 1) / SymvTile<T>::TS);
        int chk = 4 * SYMV_TPW;
        while (chk > 1 && symv_items(mt, chk) < SYMV_MIN_ITEMS) chk >>= 1;
        const int nitems = int(symv_items(mt, chk));
        // algorithmic bytes: the upper triangle of the trailing matrix, read once
        const double m1 = double(n - c - 1);
        LRC_TIMED_LAUNCH("k_trd_symv", m1 * (m1 + 1.0) * 0.5 * double(sizeof(T)) * double(nbatch), k_trd_symv<T>,
                         dim3(nitems, 1, nbatch), dim3(256), 0, s, w->A, lda, n, c, j, w->colbuf, w->part, npart, w->Vp,
                         w->Wp, w->Rt, w->rowpart, w->colpart, w->qcol, w->qvec, w->spart, w->tau, w->e, NT, chk, zs);
        // the next column is handled here unless a trailing update comes first (the last column
        // n-1 has no reflector, only d[n-1])
        const int next = (c + 1 < p1 || p1 == n - 1) ? 1 : 0;
        const int nw = cdiv(n - c - 1, 64);
        hipLaunchKernelGGL(k_trd_w1col<T>, dim3(nw, 1, nbatch), dim3(256), 0, s, w->A, lda, n, c, j, next, w->Vp,
                           w->Wp, w->rowpart, w->colpart, w->qvec, w->spart, nitems, NT, chk, w->tau, w->colbuf,
                           w->part, w->qcol, w->d, zs);
        npart = nw;
    }

    // Enqueues about `cols` columns' worth of launches; returns LRC_OK or a launch error.
    lrc_status advance(int cols) {
        if (stage == 0) {
            const lrc_status st = prepare();
            if (st != LRC_OK) return st;
            return begin_tridiagonal();
        }
        if (stage == 1) {  // 1. tridiagonalisation, panels over reflector columns 0 .. n-2
            for (int q = 0; q < cols; ++q) {
                column();
                if (++c < p1) continue;
                LRC_LAUNCH_CHECK("tridiagonal panel");
                if (p1 < n - 1) {
                    const int64_t nt = cdiv(n - p1, 64);  // tile rows of the trailing matrix
                    hipLaunchKernelGGL(k_trailing<T>, dim3(unsigned(nt * (nt + 1) / 2), 1, nbatch), dim3(256), 0, s,
                                       w->A, w->lda, n, p1, int(p1 - p0), w->Vp, w->Wp, zs);
                    LRC_LAUNCH_CHECK("k_trailing");
                }
                p0 += NB;
                if (p0 >= n - 1) {
                    stage = 2;
                    return LRC_OK;
                }
                if (n - p0 <= TrdSmall<T>::NMAX) return small_tail();
                start_panel();
            }
            return LRC_OK;
        }
        if (stage == 2) {
            // 2. eigenvalues
            hipLaunchKernelGGL(k_tri_prep, dim3(1, 1, nbatch), dim3(256), 0, s, w->d, w->e, n, w->e2, w->bounds, zs);
            hipLaunchKernelGGL(k_bisect, dim3(cdiv(n * MSEC, 256), 1, nbatch), dim3(256), 0, s, w->d, w->e2, n,
                               w->bounds, w->lam, zs);
            if (nbatch == 1)  // a batch's per-matrix outputs are written by its caller
                hipLaunchKernelGGL(k_lambda_desc, dim3(cdiv(n, 256)), dim3(256), 0, s, w->lam, n, lambda, w->bad);
            LRC_LAUNCH_CHECK("bisection");
            if (nv > 0) {
                // 3. eigenvectors of T
                hipLaunchKernelGGL(k_invit, dim3(cdiv(nv, 64), 1, nbatch), dim3(64), 0, s, w->d, w->e, n, w->lam,
                                   w->bounds, nv, w->Z, w->PU, w->PD, w->SW, zs);
                hipLaunchKernelGGL(k_cluster_mgs, dim3(unsigned(nv), 1, nbatch), dim3(256), 0, s, w->lam, n, nv,
                                   w->bounds, w->Z, zs);
                LRC_LAUNCH_CHECK("inverse iteration");
                // all T factors of the back-transformation first, in one launch
                hipLaunchKernelGGL(k_bt_tall<T>, dim3(cdiv(n - 1, NBT), 1, nbatch), dim3(256), 0, s, w->Rt, n, n, n - 1,
                                   w->tau, w->Tf, zs);
                c0 = ((n - 2) / NBT) * NBT;
                stage = 3;
                return LRC_OK;
            }
            stage = 4;
        }
        if (stage == 3) {  // 4. back-transformation, last block of reflectors first
            const int64_t nrefl = n - 1;
            for (int q = 0; q < cols && c0 >= 0; ++q, c0 -= NBT) {
                const int nb = int(std::min<int64_t>(NBT, nrefl - c0));
                const int64_t mrows = n - c0 - 1;  // rows the block's reflectors touch
                const int nch = cdiv(mrows, RCH);
                hipLaunchKernelGGL(k_bt_g<T>, dim3(cdiv(nv, 64), nch, nbatch), dim3(256), 0, s, w->Rt, n, n, c0, nb,
                                   w->Z, nv, w->Gp, RCH, zs);
                hipLaunchKernelGGL(k_bt_greduce, dim3(cdiv(nv, GR_COLS), 1, nbatch), dim3(256), 0, s, w->Gp, nch, nv,
                                   w->Tf + (c0 / NBT) * NBT * NBT, w->G, zs);
                hipLaunchKernelGGL(k_bt_update<T>, dim3(cdiv(nv, 64), cdiv(mrows, 64), nbatch), dim3(256), 0, s,
                                   w->Rt, n, n, c0, nb, w->G, w->Z, nv, zs);
            }
            LRC_LAUNCH_CHECK("back-transformation");
            if (c0 >= 0) return LRC_OK;
            if (!keep_z && nbatch == 1) {
                sign_out(w->Z, n, nv, V, ldv, w->bad, s);
                LRC_LAUNCH_CHECK("k_sign_cols");
            }
            stage = 4;
        }
        if (nbatch == 1) {
            hipLaunchKernelGGL(k_set_info, dim3(1), dim3(64), 0, s, info, w->bad);
            LRC_LAUNCH_CHECK("k_set_info");
        }
        stage = 5;
        return LRC_OK;
    }
    bool done() const { return stage == 5; }
};

// ---------------------------------------------------------------------------------------------
// 6. range-restricted decomposition (C = (X W)^T (X W), W d_in x n with d_in < n)
// ---------------------------------------------------------------------------------------------
// The range of C lies in that of W^T, so with Q (n x d_in) an orthonormal basis of it the
// eigenpairs of C are those of B = Q^T C Q (d_in x d_in), V = Q U, plus n - d_in zero eigenvalues.
// Q comes from the Cholesky factor of W W^T = L L^T: Q^T = L^{-1} W (fp64; its departure from
// orthogonality is about kappa(W)^2 times the fp64 unit roundoff).

// lambda (n, descending) from the d_in eigenvalues of B (descending) and n - d_in zeros: the p
// non-negative ones, the zeros, then the negative ones; info 3 when W W^T was not positive
// definite, 1 for non-finite input, 6 when fewer than n_vec eigenvalues of B are non-negative (the
// vectors of the zero eigenvalues are not formed), else 0.
__global__ void k_range_finish(const double *__restrict__ lamB, int64_t r, int64_t n, double *__restrict__ lam,
                               const int *__restrict__ bad, const int32_t *__restrict__ chol_info, int64_t nv,
                               int32_t *__restrict__ info) {
    const bool nan = *bad != 0;
    int64_t lo = 0, hi = r;  // p = first index with lamB < 0 (lamB descending)
    while (lo < hi) {
        const int64_t mid = (lo + hi) >> 1;
        if (lamB[mid] >= 0.0) lo = mid + 1; else hi = mid;
    }
    const int64_t p = lo, z = n - r;
    for (int64_t j = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; j < n; j += int64_t(gridDim.x) * blockDim.x)
        lam[j] = nan ? double(NAN) : (j < p ? lamB[j] : (j < p + z ? 0.0 : lamB[j - z]));
    if (blockIdx.x == 0 && threadIdx.x == 0)
        *info = *chol_info != 0 ? 3 : (nan ? 1 : (nv > p ? 6 : 0));
}

// The factor L of W W^T = L L^T has the singular values of W, so max/min of its diagonal bounds
// kappa(W) from below; the basis Q^T = L^{-1} W loses orthogonality like kappa(W)^2 times the
// fp64 unit roundoff.  A ratio above 1e5 (or a non-finite diagonal) marks the basis as unusable
// (chol_info 3), as a failed Cholesky does.  One workgroup, fixed-order reduction.
__global__ void __launch_bounds__(256) k_range_check(const double *__restrict__ L, int64_t r, int64_t ldl,
                                                     int32_t *chol_info) {
    __shared__ double smin[256], smax[256];
    double mn = DBL_MAX, mx = 0.0;
    for (int64_t i = threadIdx.x; i < r; i += 256) {
        const double v = L[i * ldl + i];
        mn = fmin(mn, isfinite(v) ? fabs(v) : 0.0);
        mx = fmax(mx, isfinite(v) ? fabs(v) : DBL_MAX);
    }
    smin[threadIdx.x] = mn;
    smax[threadIdx.x] = mx;
    __syncthreads();
    for (int o = 128; o > 0; o >>= 1) {
        if (threadIdx.x < o) {
            smin[threadIdx.x] = fmin(smin[threadIdx.x], smin[threadIdx.x + o]);
            smax[threadIdx.x] = fmax(smax[threadIdx.x], smax[threadIdx.x + o]);
        }
        __syncthreads();
    }
    if (threadIdx.x == 0 && *chol_info == 0 && !(smin[0] > 1e-5 * smax[0] && smax[0] < DBL_MAX)) *chol_info = 3;
}

struct RangeWs {
    double *Qt, *C64, *T, *G, *lamB, *A64;
    void *chol, *trsm;
    float *B;
    int32_t *iw;
};

// The decomposition's own arrays come first, at the offsets a member without a basis of order r has,
// so that members of both kinds can be tridiagonalised in lockstep.  A projected member (its matrix
// is B = Q^T C Q already) needs neither the fp64 copy of C nor B.
template <class C_, class T>
static void range_layout(C_ &cv, RangeWs &rw, LargeWs<T> &w, int64_t n, int64_t r, int64_t nv, bool proj) {
    layout(cv, w, r, nv, false);
    rw.Qt = cv.template carve<double>(size_t(r) * size_t(n));
    rw.C64 = proj ? nullptr : cv.template carve<double>(size_t(n) * size_t(n));
    rw.T = cv.template carve<double>(size_t(r) * size_t(n));  // later the n x n_vec vectors Q Z
    rw.G = cv.template carve<double>(size_t(r) * size_t(r));
    rw.lamB = cv.template carve<double>(size_t(r));
    rw.chol = cv.template carve<char>(cholesky_workspace(r));
    rw.trsm = cv.template carve<char>(trsm_workspace(0, r, n));
    rw.B = proj ? nullptr : cv.template carve<float>(size_t(r) * size_t(r));
    rw.iw = cv.template carve<int32_t>(2);
    rw.A64 = proj ? cv.template carve<double>(size_t(r) * size_t(nv)) : nullptr;  // L U, for the factor A
}

template <class T>
static size_t range_ws(int64_t n, int64_t r, int64_t nv, bool proj) {
    CountCarver cc;
    RangeWs rw;
    LargeWs<T> w;
    range_layout(cc, rw, w, n, r, nv, proj);
    return cc.c.off;
}

// the range path applies when 128 < d_in < n and n_vec <= d_in
static bool use_range(const EighArgs &a) { return a.W && a.d_in > 128 && a.d_in < a.n && a.n_vec <= a.d_in; }

// The factor L of W W^T = L L^T (W: r x n of dtype w_t, ldw): Wf = W in fp64 (r x n, leading dim n),
// the lower triangle of W W^T into L (ldl), its Cholesky factorisation in place, and the check of
// L's diagonal; info 3 when W W^T is not positive definite or the diagonal spans more than 1e5.
// Used by the range path of the eigendecomposition and by lrc_range_factor, with the same kernels,
// so both give the same L bit for bit.
lrc_status range_factor_enqueue(const void *W, lrc_dtype w_t, int64_t r, int64_t n, int64_t ldw, double *Wf,
                                double *L, int64_t ldl, void *chol_ws, int32_t *info, hipStream_t s) {
    lrc_status st = to_f64_run(W, w_t, r, n, ldw, 1.0, Wf, n, s);
    if (st == LRC_OK) st = dgemm_run(0, 1, r, r, n, Wf, n, Wf, n, L, ldl, 1, nullptr, s);  // W W^T, lower
    if (st == LRC_OK) st = cholesky_run(L, r, ldl, chol_ws, cholesky_workspace(r), info, s);
    if (st == LRC_OK) {
        hipLaunchKernelGGL(k_range_check, dim3(1), dim3(256), 0, s, L, r, ldl, info);
        LRC_LAUNCH_CHECK("k_range_check");
    }
    return st;
}

// Batch members are independent: up to EIG_LANES of them run at once, each on a helper stream
// of its own with its own workspace, so the per-column launch chains of several matrices
// overlap (one chain alone leaves most of the GPU idle once the trailing matrix is small).  Each
// lane is fed by a host thread of its own: a chain is two or three small launches per column, and
// one thread enqueueing for all lanes would both cap the launch rate and stall every lane while
// one lane's queue is full.  The helper streams (default priority) and their events are created
// per device on first use and kept; the caller's stream waits for all of them, so a call stays
// asynchronous (it returns once every launch is enqueued).  Eight lanes: with the GPU's default
// four hardware queues per process, the seven decompositions of a transformer block all at once
// took 297 ms against 358 ms four at a time (six at a time: 356 ms).
constexpr int EIG_LANES = 8;

// Calls may run at once from several host threads (for instance one per group of matrices whose
// covariances are ready): each call takes its lanes from a rotating base, so calls that together
// have at most EIG_LANES members use different streams, and its own events from a pool.
struct EigLanes {
    hipStream_t st[EIG_LANES];
    std::atomic<unsigned> base{0};  // first lane of the next call
    std::mutex pool_mu;
    std::vector<hipEvent_t> pool;  // events not in use by a call (never destroyed)
    bool ok = false;
};

static lrc_status take_events(EigLanes *L, int n, hipEvent_t *out) {
    std::lock_guard<std::mutex> lk(L->pool_mu);
    for (int i = 0; i < n; ++i) {
        if (L->pool.empty()) {
            hipEvent_t e;
            LRC_HIP(hipEventCreateWithFlags(&e, hipEventDisableTiming));
            L->pool.push_back(e);
        }
        out[i] = L->pool.back();
        L->pool.pop_back();
    }
    return LRC_OK;
}

// events go back once the waits on them are enqueued: a later record does not affect them
static void give_events(EigLanes *L, int n, const hipEvent_t *ev) {
    std::lock_guard<std::mutex> lk(L->pool_mu);
    for (int i = 0; i < n; ++i) L->pool.push_back(ev[i]);
}

static lrc_status eig_lanes(EigLanes **out) {
    static std::mutex mu;
    static std::map<int, EigLanes> lanes;
    int devid = 0;
    LRC_HIP(hipGetDevice(&devid));
    std::lock_guard<std::mutex> lk(mu);
    EigLanes &L = lanes[devid];
    if (!L.ok) {
        for (int i = 0; i < EIG_LANES; ++i) LRC_HIP(hipStreamCreateWithFlags(&L.st[i], hipStreamNonBlocking));
        L.ok = true;
    }
    *out = &L;
    return LRC_OK;
}

// Workspace of a multi-group call: one region for the Jacobi groups (run one after another on the
// caller's stream) followed by one region per lane, each sized for the largest n and n_vec among
// the n > 128 groups (every field of the layout grows with n and n_vec).
struct MultiPlan {
    size_t jac = 0, per = 0;
    int lanes = 0;
    int64_t maxn = 0, maxnv = 0, members = 0;
};

static MultiPlan multi_plan(const EighArgs *g, int count, lrc_dtype prec) {
    MultiPlan p;
    size_t per_range = 0;
    for (int i = 0; i < count; ++i) {
        if (g[i].n <= 128) {
            p.jac = std::max(p.jac, jacobi_workspace(g[i].n, g[i].batch, prec));
        } else {
            p.members += g[i].batch;
            if (use_range(g[i])) {
                const bool pj = g[i].projected != 0;
                per_range = std::max(per_range, prec == LRC_F64 ? range_ws<double>(g[i].n, g[i].d_in, g[i].n_vec, pj)
                                                                : range_ws<float>(g[i].n, g[i].d_in, g[i].n_vec, pj));
            } else {
                p.maxn = std::max(p.maxn, g[i].n);
                p.maxnv = std::max(p.maxnv, g[i].n_vec);
            }
        }
    }
    p.jac = align256(p.jac);
    if (p.members > 0) {
        p.lanes = int(std::min<int64_t>(p.members, EIG_LANES));
        if (p.maxn > 0)
            p.per = prec == LRC_F64 ? large_ws<double>(p.maxn, p.maxnv) : large_ws<float>(p.maxn, p.maxnv);
        p.per = std::max(p.per, per_range);
    }
    return p;
}

size_t eigh_multi_workspace(const EighArgs *g, int count, lrc_dtype prec) {
    const MultiPlan p = multi_plan(g, count, prec);
    return p.jac + size_t(p.lanes) * p.per;
}

size_t eigh_workspace(int64_t n, int64_t batch, int64_t n_vec, lrc_dtype prec) {
    EighArgs a{nullptr, n, n, batch, 0, prec, nullptr, nullptr, n_vec, n_vec, 0, nullptr};
    return eigh_multi_workspace(&a, 1, prec);
}

struct EigMember {
    const float *C;
    int64_t ldc, n;
    double *lambda;
    float *V;
    int64_t ldv, nv;
    int32_t *info;
    const void *W;  // range basis (W d_in x n), or nullptr
    lrc_dtype w_t;
    int64_t d_in, ldw;
    bool proj;  // C holds B = Q^T C Q (d_in x d_in, ldc) instead of C
    const double *L;  // the factor of W W^T given by the caller (lower, ldl), or nullptr
    int64_t ldl;
    float *A;  // a projected member's factor W V = L U (d_in x nv, lda), or nullptr
    int64_t lda;
};

// One member's decomposition: its layout on a workspace region and its job; for a member with a
// range basis also the basis Q and B = Q^T C Q (the job decomposes B) and, once the job is done,
// V = Q Z and the eigenvalues with the n - d_in zeros.
template <class T>
struct MemberRun {
    EigMember m{};
    LargeWs<T> w;
    RangeWs rw{};
    EigJob<T> j;
    const double *L = nullptr;  // the factor of W W^T in use (the caller's or rw.G)
    int64_t ldl = 0;
};

// Lays out the region and sets up the job; a range member's basis and B are enqueued on s.
template <class T>
static lrc_status member_begin(MemberRun<T> &R, const MultiPlan &p, char *lws, hipStream_t s) {
    const EigMember &m = R.m;
    Carver cv(lws, p.per);
    R.w = LargeWs<T>();
    EigJob<T> &j = R.j;
    j = EigJob<T>();
    j.w = &R.w;
    j.s = s;
    if (!m.W) {
        layout(cv, R.w, m.n, m.nv, false);
        if (!R.w.bad) return fail(LRC_ERR_WORKSPACE, "eigh workspace too small");
        j.C = m.C;
        j.ldc = m.ldc;
        j.n = m.n;
        j.lambda = m.lambda;
        j.V = m.V;
        j.ldv = m.ldv;
        j.nv = m.nv;
        j.info = m.info;
        return LRC_OK;
    }
    const int64_t n = m.n, r = m.d_in, nv = m.nv;
    RangeWs &rw = R.rw;
    range_layout(cv, rw, R.w, n, r, nv, m.proj);
    if (!R.w.bad) return fail(LRC_ERR_WORKSPACE, "eigh workspace too small");
    // rw.Qt first holds W in fp64; a projected member keeps it so (V = W^T (L^{-T} Z) at the end,
    // a triangular solve on the d_in x n_vec block instead of on the d_in x n basis)
    lrc_status st = LRC_OK;
    if (m.L) {  // the caller's factor (from lrc_range_factor, the same kernels)
        R.L = m.L;
        R.ldl = m.ldl;
        st = to_f64_run(m.W, m.w_t, r, n, m.ldw, 1.0, rw.Qt, n, s);
        hipLaunchKernelGGL(k_zero_i32, dim3(1), dim3(64), 0, s, rw.iw);
        LRC_LAUNCH_CHECK("k_zero_i32");
    } else {
        R.L = rw.G;
        R.ldl = r;
        st = range_factor_enqueue(m.W, m.w_t, r, n, m.ldw, rw.Qt, rw.G, r, rw.chol, rw.iw, s);
    }
    if (!m.proj) {
        if (st == LRC_OK) st = trsm_run(0, 0, r, n, R.L, R.ldl, rw.Qt, n, rw.trsm, s);  // Q^T = L^{-1} W
        if (st == LRC_OK) st = sym_to_f64_run(m.C, n, m.ldc, 1.0, rw.C64, n, s);
        if (st == LRC_OK) st = dgemm_run(0, 0, r, n, n, rw.Qt, n, rw.C64, n, rw.T, n, 0, nullptr, s);  // Q^T C
        if (st == LRC_OK) st = dgemm_run(0, 1, r, r, n, rw.T, n, rw.Qt, n, nullptr, r, 2, rw.B, s);  // B, upper
    }
    if (st != LRC_OK) return st;
    j.C = m.proj ? m.C : rw.B;
    j.ldc = m.proj ? m.ldc : r;
    j.n = r;
    j.lambda = rw.lamB;
    j.V = nullptr;
    j.ldv = nv;
    j.nv = nv;
    j.info = rw.iw + 1;
    j.keep_z = true;
    return LRC_OK;
}

// After the job: a range member's V = Q Z (sign rule) and lambda with the zeros, on s.
template <class T>
static lrc_status member_end(MemberRun<T> &R, hipStream_t s) {
    const EigMember &m = R.m;
    if (!m.W) return LRC_OK;
    const int64_t n = m.n, r = m.d_in, nv = m.nv;
    RangeWs &rw = R.rw;
    if (nv > 0) {
        lrc_status st = LRC_OK;
        if (m.proj) {  // Q Z = W^T L^{-T} Z: Z <- L^{-T} Z, then W^T Z (first L Z for the factor A)
            if (m.A) st = lower_product_run(r, nv, R.L, R.ldl, R.w.Z, nv, rw.A64, nv, s);
            if (st == LRC_OK) st = trsm_run(0, 1, r, nv, R.L, R.ldl, R.w.Z, nv, rw.trsm, s);
            if (st == LRC_OK) st = dgemm_run(1, 0, n, nv, r, rw.Qt, n, R.w.Z, nv, rw.T, nv, 0, nullptr, s);
        } else {
            st = dgemm_run(1, 0, n, nv, r, rw.Qt, n, R.w.Z, nv, rw.T, nv, 0, nullptr, s);  // Q Z
        }
        if (st != LRC_OK) return st;
        if (m.proj && m.A)
            sign_out(rw.T, n, nv, m.V, m.ldv, R.w.bad, s, rw.A64, r, m.A, m.lda);
        else
            sign_out(rw.T, n, nv, m.V, m.ldv, R.w.bad, s);
        LRC_LAUNCH_CHECK("k_sign_cols");
    }
    hipLaunchKernelGGL(k_range_finish, dim3(cdiv(n, 256)), dim3(256), 0, s, rw.lamB, r, n, m.lambda, R.w.bad, rw.iw, nv,
                       m.info);
    LRC_LAUNCH_CHECK("k_range_finish");
    return LRC_OK;
}

// All members with n > 128 over up to EIG_LANES helper streams, largest n first: each lane's
// thread takes the next member once its own is enqueued (its stream runs in order, so the lane's
// workspace is free by then).  Which lane runs a member does not change its results: the
// computation depends only on the member, and every lane's workspace has the same layout.
template <class T>
static lrc_status run_member(const EigMember &m, const MultiPlan &p, char *lws, hipStream_t s, MemberRun<T> &R) {
    R.m = m;
    lrc_status st = member_begin(R, p, lws, s);
    while (st == LRC_OK && !R.j.done()) st = R.j.advance(64);
    if (st == LRC_OK) st = member_end(R, s);
    return st;
}

// Members whose matrices have one order (n, or d_in with a range basis) and fit a workspace region
// each are tridiagonalised in lockstep: every launch of the column chain works on all of them (one
// z slice per matrix), so a chain of two small launches per column serves the whole group instead
// of each matrix paying its own launch and latency cost on a stream of its own.  The eigenvalues, the
// vectors of T and the back-transformation are batched the same way for the members that share n_vec
// (one launch per step for all of them): on the call's stream when all do, else one class of equal
// n_vec per helper stream.  A range member's V = Q Z follows (two or more range members each on a
// helper stream, concurrently).  Every member's arithmetic is the same as alone, so its results are
// bit-identical to a call on it alone.
// LRC_EIGH_LOCKSTEP=0 turns this off (each member on a lane of its own throughout, as for members
// of different orders).
static int64_t trd_order(const EigMember &m) { return m.W ? m.d_in : m.n; }

static bool lockstep_ok(const std::vector<EigMember> &mem, int lanes) {
    if (mem.size() < 2 || mem.size() > size_t(lanes)) return false;
    const char *e = std::getenv("LRC_EIGH_LOCKSTEP");
    if (e && e[0] == '0' && e[1] == 0) return false;
    for (const EigMember &m : mem)
        if (trd_order(m) != trd_order(mem[0])) return false;
    return true;
}

template <class T>
static lrc_status large_lockstep(std::vector<EigMember> &mem, const MultiPlan &p, char *ws, hipStream_t s,
                                 MemberRun<T> *R) {
    const int nb = int(mem.size());
    // members of one n_vec next to each other (regions in this order), so that each such class can
    // run the stages after the tridiagonalisation batched; a member's results do not depend on its place
    std::stable_sort(mem.begin(), mem.end(), [](const EigMember &x, const EigMember &y) { return x.nv > y.nv; });
    // 1. each member's setup (a range member's basis and B) and its matrix copied into A, on s
    for (int i = 0; i < nb; ++i) {
        R[i].m = mem[i];
        lrc_status st = member_begin(R[i], p, ws + p.per * size_t(i), s);
        if (st == LRC_OK) st = R[i].j.prepare();
        if (st != LRC_OK) return st;
    }
    // 2. the tridiagonalisations in lockstep, on s (regions p.per bytes apart, identical layouts up to
    // the arrays that depend on n_vec, which the tridiagonalisation does not touch)
    EigJob<T> bj = R[0].j;
    bj.nbatch = unsigned(nb);
    bj.zs = int64_t(p.per);
    {
        const lrc_status st = bj.begin_tridiagonal();
        if (st != LRC_OK) return st;
    }
    while (bj.stage == 1) {
        const lrc_status st = bj.advance(64);
        if (st != LRC_OK) return st;
    }
    bool same_nv = true;
    for (int i = 1; i < nb; ++i) same_nv = same_nv && R[i].j.nv == R[0].j.nv;
    if (same_nv) {
        // 3. with one n_vec the regions agree up to their last array, so the eigenvalues, the vectors
        // of T and the back-transformation run batched as well (workgroup z on member z), on s;
        // then each member's outputs and a range member's V = Q Z and lambda with the zeros
        while (!bj.done()) {
            const lrc_status st = bj.advance(64);
            if (st != LRC_OK) return st;
        }
        std::vector<int> rg;  // members with a range basis: V = Q Z and lambda with the zeros to follow
        for (int i = 0; i < nb; ++i) {
            const EigJob<T> &j = R[i].j;
            LargeWs<T> &w = R[i].w;
            hipLaunchKernelGGL(k_lambda_desc, dim3(cdiv(j.n, 256)), dim3(256), 0, s, w.lam, j.n, j.lambda, w.bad);
            if (j.nv > 0 && !j.keep_z)
                sign_out(w.Z, j.n, j.nv, j.V, j.ldv, w.bad, s);
            hipLaunchKernelGGL(k_set_info, dim3(1), dim3(64), 0, s, j.info, w.bad);
            LRC_LAUNCH_CHECK("lockstep outputs");
            if (R[i].m.W) rg.push_back(i);
        }
        if (rg.size() < 2) {
            for (int i : rg) {
                const lrc_status st = member_end(R[i], s);
                if (st != LRC_OK) return st;
            }
            return LRC_OK;
        }
        // two or more range members: each one's V = Q Z (a triangular solve of many small launches for
        // a projected member, then an fp64 product) on a helper stream of its own, so that the solves
        // overlap; the call's stream waits for all of them
        const int nr = int(rg.size());
        EigLanes *L = nullptr;
        lrc_status st0 = eig_lanes(&L);
        if (st0 != LRC_OK) return st0;
        hipEvent_t ev[EIG_LANES + 1];
        st0 = take_events(L, nr + 1, ev);
        if (st0 != LRC_OK) return st0;
        const unsigned base = L->base.fetch_add(unsigned(nr));
        auto fan = [&]() -> lrc_status {
            LRC_HIP(hipEventRecord(ev[0], s));
            for (int q = 0; q < nr; ++q) {
                hipStream_t lq = L->st[(base + unsigned(q)) % EIG_LANES];
                LRC_HIP(hipStreamWaitEvent(lq, ev[0], 0));
                const lrc_status st = member_end(R[rg[q]], lq);
                if (st != LRC_OK) return st;
                LRC_HIP(hipEventRecord(ev[1 + q], lq));
                LRC_HIP(hipStreamWaitEvent(s, ev[1 + q], 0));
            }
            return LRC_OK;
        };
        const lrc_status st = fan();
        give_events(L, nr + 1, ev);
        return st;
    }
    // 3. otherwise the members fall into classes of consecutive members with one n_vec (the order is
    // the callers', stable under the sort by n); each class runs the stages after the tridiagonal-
    // isation batched, as above, on a helper stream of its own (a class of one as a single job)
    std::vector<std::pair<int, int>> cls;  // [first, last + 1)
    for (int i = 0; i < nb;) {
        int k = i + 1;
        while (k < nb && R[k].j.nv == R[i].j.nv) ++k;
        cls.push_back({i, k});
        i = k;
    }
    const int ncl = int(cls.size());
    EigLanes *L = nullptr;
    lrc_status st0 = eig_lanes(&L);
    if (st0 != LRC_OK) return st0;
    hipEvent_t ev[EIG_LANES + 1];
    st0 = take_events(L, ncl + 1, ev);
    if (st0 != LRC_OK) return st0;
    const unsigned base = L->base.fetch_add(unsigned(ncl));
    hipStream_t ls[EIG_LANES];
    for (int q = 0; q < ncl; ++q) ls[q] = L->st[(base + unsigned(q)) % EIG_LANES];
    auto fan = [&]() -> lrc_status {
        LRC_HIP(hipEventRecord(ev[0], s));
        for (int q = 0; q < ncl; ++q) LRC_HIP(hipStreamWaitEvent(ls[q], ev[0], 0));
        for (int q = 0; q < ncl; ++q) {
            const int i0 = cls[q].first, i1 = cls[q].second;
            EigJob<T> cj = R[i0].j;  // member i0's region; the class's regions follow p.per apart
            cj.s = ls[q];
            cj.stage = 2;
            cj.nbatch = unsigned(i1 - i0);
            cj.zs = int64_t(p.per);
            while (!cj.done()) {
                const lrc_status st = cj.advance(64);
                if (st != LRC_OK) return st;
            }
            for (int i = i0; i < i1; ++i) {
                if (i1 - i0 > 1) {  // a batch's per-matrix outputs
                    const EigJob<T> &j = R[i].j;
                    LargeWs<T> &w = R[i].w;
                    hipLaunchKernelGGL(k_lambda_desc, dim3(cdiv(j.n, 256)), dim3(256), 0, ls[q], w.lam, j.n, j.lambda,
                                       w.bad);
                    if (j.nv > 0 && !j.keep_z)
                        sign_out(w.Z, j.n, j.nv, j.V, j.ldv, w.bad, ls[q]);
                    hipLaunchKernelGGL(k_set_info, dim3(1), dim3(64), 0, ls[q], j.info, w.bad);
                    LRC_LAUNCH_CHECK("lockstep class outputs");
                }
                const lrc_status st = member_end(R[i], ls[q]);
                if (st != LRC_OK) return st;
            }
        }
        for (int q = 0; q < ncl; ++q) {
            LRC_HIP(hipEventRecord(ev[1 + q], ls[q]));
            LRC_HIP(hipStreamWaitEvent(s, ev[1 + q], 0));
        }
        return LRC_OK;
    };
    const lrc_status st = fan();
    give_events(L, ncl + 1, ev);
    return st;
}

template <class T>
static lrc_status large_sched(std::vector<EigMember> &mem, const MultiPlan &p, char *ws, hipStream_t s) {
    std::stable_sort(mem.begin(), mem.end(), [](const EigMember &x, const EigMember &y) { return x.n > y.n; });
    const int lanes = p.lanes;
    std::unique_ptr<MemberRun<T>[]> R(new MemberRun<T>[EIG_LANES]);
    if (lanes <= 1) {
        for (const EigMember &m : mem) {
            const lrc_status st = run_member<T>(m, p, ws, s, R[0]);
            if (st != LRC_OK) return st;
        }
        return LRC_OK;
    }
    if (lockstep_ok(mem, lanes)) return large_lockstep<T>(mem, p, ws, s, R.get());
    EigLanes *L = nullptr;
    lrc_status st0 = eig_lanes(&L);
    if (st0 != LRC_OK) return st0;
    int dev = 0;
    LRC_HIP(hipGetDevice(&dev));
    hipEvent_t ev[EIG_LANES + 1];  // ev[0]: start on s; ev[1 + l]: lane l done
    st0 = take_events(L, lanes + 1, ev);
    if (st0 != LRC_OK) return st0;
    const unsigned base = L->base.fetch_add(unsigned(lanes));
    hipStream_t ls[EIG_LANES];
    for (int l = 0; l < lanes; ++l) ls[l] = L->st[(base + unsigned(l)) % EIG_LANES];
    auto enqueue_start = [&]() -> lrc_status {
        LRC_HIP(hipEventRecord(ev[0], s));
        for (int l = 0; l < lanes; ++l) LRC_HIP(hipStreamWaitEvent(ls[l], ev[0], 0));
        return LRC_OK;
    };
    st0 = enqueue_start();
    if (st0 != LRC_OK) {
        give_events(L, lanes + 1, ev);
        return st0;
    }
    std::atomic<size_t> next{0};
    std::atomic<bool> stop{false};
    lrc_status st[EIG_LANES];
    std::string msg[EIG_LANES];
    auto lane = [&](int l) {
        st[l] = LRC_OK;
        const hipError_t e = hipSetDevice(dev);  // the current device is per thread
        if (e != hipSuccess) st[l] = hip_fail(e, "hipSetDevice");
        while (st[l] == LRC_OK && !stop.load()) {
            const size_t i = next.fetch_add(1);
            if (i >= mem.size()) break;
            char *lws = ws + p.per * size_t(l);
            st[l] = run_member<T>(mem[i], p, lws, ls[l], R[l]);
        }
        if (st[l] != LRC_OK) {
            msg[l] = lrc_last_error();
            stop.store(true);
        }
    };
    // LRC_EIGH_HOST_THREADS=0: the calling thread enqueues all the work itself, on lane 0 (for
    // tools that cannot follow launches from several host threads, such as counter collection,
    // which serialises the kernels anyway)
    const char *ht = std::getenv("LRC_EIGH_HOST_THREADS");
    const bool threaded = !(ht && ht[0] == '0' && ht[1] == 0);
    std::vector<std::thread> th;
    if (threaded) {
        try {
            for (int l = 1; l < lanes; ++l) th.emplace_back(lane, l);
        } catch (...) {
            stop.store(true);
            for (auto &t : th) t.join();
            give_events(L, lanes + 1, ev);
            return fail(LRC_ERR_HIP, "could not start the eigh lane threads");
        }
    }
    lane(0);
    for (auto &t : th) t.join();
    for (int l = threaded ? lanes : 1; l < lanes; ++l) st[l] = LRC_OK;
    auto enqueue_done = [&]() -> lrc_status {
        for (int l = 0; l < lanes; ++l) {
            LRC_HIP(hipEventRecord(ev[1 + l], ls[l]));
            LRC_HIP(hipStreamWaitEvent(s, ev[1 + l], 0));
        }
        return LRC_OK;
    };
    const lrc_status sd = enqueue_done();
    give_events(L, lanes + 1, ev);
    if (sd != LRC_OK) return sd;
    for (int l = 0; l < lanes; ++l)
        if (st[l] != LRC_OK) return fail(st[l], msg[l]);
    return LRC_OK;
}

lrc_status eigh_multi_run(const EighArgs *g, int count, lrc_dtype prec, void *ws, size_t ws_bytes, hipStream_t s) {
    for (int i = 0; i < count; ++i) {
        if (g[i].n <= 128) continue;
        if (g[i].n * int64_t(sizeof(double)) > 160 * 1024 && prec == LRC_F64)
            return fail(LRC_ERR_UNIMPLEMENTED, "fp64 working precision supports n <= 20480");
        if (g[i].n * int64_t(sizeof(float)) > 160 * 1024) return fail(LRC_ERR_UNIMPLEMENTED, "n > 40960");
    }
    const MultiPlan p = multi_plan(g, count, prec);
    if (ws_bytes < p.jac + size_t(p.lanes) * p.per) return fail(LRC_ERR_WORKSPACE, "eigh workspace too small");
    for (int i = 0; i < count; ++i) {
        if (g[i].n > 128) continue;
        EighArgs a = g[i];
        a.prec = prec;
        lrc_status st = jacobi_run(a, ws, p.jac, s);
        if (st != LRC_OK) return st;
    }
    if (p.members == 0) return LRC_OK;
    std::vector<EigMember> mem;
    mem.reserve(size_t(p.members));
    for (int i = 0; i < count; ++i) {
        const EighArgs &a = g[i];
        if (a.n <= 128) continue;
        const bool rng = use_range(a);
        const size_t esz = a.w_t == LRC_BF16 ? 2 : (a.w_t == LRC_F32 ? 4 : 8);
        for (int64_t b = 0; b < a.batch; ++b)
            mem.push_back(EigMember{a.C + b * a.stride_c, a.ldc, a.n, a.lambda + b * a.n,
                                    a.V ? a.V + b * a.stride_v : nullptr, a.ldv, a.n_vec, a.info + b,
                                    rng ? static_cast<const char *>(a.W) + size_t(b * a.stride_w) * esz : nullptr,
                                    a.w_t, a.d_in, a.ldw, rng && a.projected != 0,
                                    rng && a.L ? a.L + b * a.stride_l : nullptr, a.ldl,
                                    rng && a.projected && a.A ? a.A + b * a.stride_a : nullptr, a.lda});
    }
    char *lw = static_cast<char *>(ws) + p.jac;
    return prec == LRC_F64 ? large_sched<double>(mem, p, lw, s) : large_sched<float>(mem, p, lw, s);
}

lrc_status eigh_run(const EighArgs &a, void *ws, size_t ws_bytes, hipStream_t s) {
    return eigh_multi_run(&a, 1, a.prec, ws, ws_bytes, s);
}

}  // namespace lrc
