// MFMA path of the covariance accumulation.
//
// Per call, before the chunks: e_i = 14 - q_i, where 2^(q_i - 1) <= max_t ||x_t|| ||W^T_i|| < 2^q_i.
// By Cauchy-Schwarz |y_i(t)| 2^e_i < 2^14 for every token, a quarter of the fp16 range.
// Per chunk of tokens (Swift-SVD page, section 2-ga: C is aggregated over the calibration
// tokens, one chunk at a time):
//   1. GEMM  Y^T[i][t] = sum_k W^T[i][k] X[t][k]        (bf16 MFMA, fp32 accumulation)
//      epilogue: s = y 2^e_i (exact), hi = fp16(s), lo = fp16(s - hi), so hi + lo carries 22 bits
//      of y; stored in blocks of MK tokens: Y^T[i][t] at ((t / MK) * D + i) * MK + t % MK
//      (D = d_out), so that the MK-token slice of consecutive rows that one k step of the SYRK
//      reads is one contiguous run.
//   2. SYRK  C[I,J] += 2^-(e_I + e_J) (hi_I hi_J^T + hi_I lo_J^T + lo_I hi_J^T), fp16 MFMA
//      products with fp32 accumulation, for tiles I <= J.  The power-of-two scales cost no
//      rounding.
//   3. C_ii += 2^-2e_i sum_t lo_i(t)^2, summed on its own.  The lo lo^T terms are about 2^-24 of
//      the hi hi^T ones.  Off the diagonal they are as often positive as negative and are left
//      out.  On the diagonal they all have one sign (left out, every quadratic form v^T C v would
//      lose ||Ylo v||^2), and inside the MFMA chain they would not survive either: a 16-token
//      sum of lo^2 is below half a unit in the last place of the running fp32 chain, so round to
//      nearest drops it every time.
// With W == NULL (C += X^T X) the chunk is transposed exactly (bf16) and one bf16 product
// suffices.
//
// Both phases are one "NT" kernel: D = A B^T with A and B row-major along the contraction
// axis, which is exactly the layout the 32x32x16 bf16 MFMA operands want (each lane holds 8
// contiguous k-values of one row).  The GEMM's block tile is 256 x 256 on 8 waves (2 x 4) of
// 128 x 64, two waves to a SIMD (10 % faster than 4 waves of 128 x 128 at d_in 4096: a wave's
// accumulators and operands fit its registers without spills, and one wave's MFMAs run while the
// other waits; with the operands loaded straight into LDS the 4-wave tile is still 5-10 % slower);
// the SYRK's is 128 x 128 on 4 waves; k step 32, LDS stages with an XOR swizzle of the 16-byte
// chunks (no padding, no bank conflicts on 16-byte reads), both operands loaded by 16-byte buffer
// loads with an LDS destination (GEMM: three stages, 4-5 % faster than staging the loads through
// registers, which remains for a contraction length that is not a multiple of 32), one barrier
// per k step, placed between the step's two k slices: the LDS reads of the next step's first
// slice go out right after it and land while the current step's second slice is multiplied,
// instead of stalling the next step's first MFMAs (GEMM 3-4 %, SYRK up to 4 % faster).  A
// scheduling barrier at each step boundary keeps the compiler from moving a step's MFMAs past
// the next step's wait for its loads (SYRK 3-4 % faster).
//
// Load balance of the SYRK: the upper triangle may have fewer tiles than the GPU has CUs, so
// the token range of a chunk is split S ways; split s > 0 accumulates into its own fp32
// buffer and the buffers are added to C in split order at the end of the call (fixed order,
// deterministic).
#include <cmath>
#include <cstdlib>
#include <type_traits>

#include "cov_mfma.h"

namespace lrc {

constexpr int MK = 32;                   // k step, bf16 elements (4 chunks of 16 bytes)
constexpr int64_t MFMA_CHUNK = 32768;    // tokens per internal chunk
// Tokens per internal chunk for d_out outputs: twice MFMA_CHUNK up to d_out 8192 (fewer, longer
// SYRK launches: at d_out 4096 the 7 token splits of a launch then each run 2x as many k steps,
// 5 % faster), MFMA_CHUNK above (at 11008 the larger chunk was 3 % slower).  2 MFMA_CHUNK x 8193
// rows of Y^T stay below the 2^31-byte reach of a buffer resource.
static int64_t chunk_tokens(int64_t d_out) { return d_out <= 8192 ? 2 * MFMA_CHUNK : MFMA_CHUNK; }

// 16-byte chunk c of row r: XOR with bits 1..3 of r so that 16 consecutive rows reading one chunk
// column hit 16 distinct 16-byte bank groups (and 8 consecutive rows 8 distinct groups)
__device__ __forceinline__ int swz(int r, int c) { return r * MK + ((c ^ (((r >> 1) ^ (r >> 3)) & 3)) << 3); }

// Block tile BM x BN (BM rows of the A operands, BN rows of the B operands), THREADS/64 waves
// arranged WGM x WGN, wave tile (BM/WGM) x (BN/WGN).
template <int BM, int BN, int THREADS, int WGM>
struct MfmaCfg {
    static constexpr int WAVES = THREADS / 64;
    static constexpr int WGN = WAVES / WGM;
    static constexpr int WM = BM / WGM, WN = BN / WGN;  // wave tile
    static constexpr int TM = WM / 32, TN = WN / 32;    // 32x32 MFMA tiles per wave
    static constexpr int UA = BM * (MK / 8) / THREADS;  // 16-byte chunks per thread of an A operand
    static constexpr int UB = BN * (MK / 8) / THREADS;  // ... of a B operand
    static_assert(UA * THREADS == BM * (MK / 8) && UB * THREADS == BN * (MK / 8), "operand tile / threads");
};

// GEMM main loop (one bf16 product, operands A = W^T rows and B = X rows, both contiguous along k)
// with the LDS reads of each step's first k slice issued before the previous step ends.  Global
// loads run two steps ahead through two register sets; per step kt:
//   loads of step kt+2; LDS reads of slice 2 of kt; MFMAs of slice 1 (its fragments were read at
//   the end of step kt-1); LDS stores of step kt+1 into the other buffer; every wave's LDS reads
//   and stores done, barrier; LDS reads of slice 1 of kt+1; MFMAs of slice 2 of kt.
// so the reads after the barrier are in flight while slice 2's MFMAs run instead of stalling the
// first MFMAs of the next step.  A buffer is stored only after the barrier that follows the last
// reads of it (slice 2 of its previous step, waited for before that barrier).
template <int BM, int THREADS, int WGM, bool KCHECK>
__device__ __forceinline__ void gemm_mainloop(const bf16_t *const *base, const int64_t *ld, const int *rows,
                                              int64_t klen,
                                              f32x16_t (&acc)[MfmaCfg<BM, BM, THREADS, WGM>::TM][MfmaCfg<BM, BM, THREADS, WGM>::TN],
                                              bf16_t *lds) {
    using T = MfmaCfg<BM, BM, THREADS, WGM>;
    constexpr int TM = T::TM, TN = T::TN, U = T::UA;
    static_assert(T::UA == T::UB, "square block tile");
    constexpr int BUFSZ = 2 * BM * MK;  // one buffer: A then B, BM rows of MK elements each
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / T::WGN, wn = wave % T::WGN;
    const int nk = int((klen + MK - 1) / MK);
    if (nk <= 0) return;
    __amdgpu_buffer_rsrc_t rs[2];
#pragma unroll
    for (int o = 0; o < 2; ++o)
        rs[o] = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<bf16_t *>(base[o]), short(0),
            int(rows[o] > 0 ? ((int64_t(rows[o]) - 1) * ld[o] + klen) * 2 : int64_t(0)), 0x00020000);
    u32x4_t regs[2][2][U];
    auto gload = [&](int kt, auto set) {
        constexpr int S = decltype(set)::value;
        const int k0 = kt * MK;
#pragma unroll
        for (int o = 0; o < 2; ++o)
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int q = tid + THREADS * u;
                const int r = q >> 2, c = q & 3;
                const int k = k0 + c * 8;
                u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(rs[o], (r * int(ld[o]) + k) * 2, 0, 0);
                if (KCHECK && k >= klen) v = u32x4_t{0u, 0u, 0u, 0u};
                regs[S][o][u] = v;
            }
    };
    auto sstore = [&](int buf, auto set) {
        constexpr int S = decltype(set)::value;
#pragma unroll
        for (int o = 0; o < 2; ++o)
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int q = tid + THREADS * u;
                const int r = q >> 2, c = q & 3;
                *reinterpret_cast<u32x4_t *>(lds + buf * BUFSZ + o * BM * MK + swz(r, c)) = regs[S][o][u];
            }
    };
    bf16x8_t f1a[TM], f1b[TN], f2a[TM], f2b[TN];  // fragments of slices 1 and 2
    auto fread = [&](int buf, int ks, bf16x8_t (&fa)[TM], bf16x8_t (&fb)[TN]) {
        const bf16_t *sb = lds + buf * BUFSZ;
        const int c = ks * 2 + (lane >> 5);
#pragma unroll
        for (int t = 0; t < TM; ++t)
            fa[t] = *reinterpret_cast<const bf16x8_t *>(sb + swz(wm * T::WM + t * 32 + (lane & 31), c));
#pragma unroll
        for (int t = 0; t < TN; ++t)
            fb[t] = *reinterpret_cast<const bf16x8_t *>(sb + BM * MK + swz(wn * T::WN + t * 32 + (lane & 31), c));
    };
    auto mfmas = [&](const bf16x8_t (&fa)[TM], const bf16x8_t (&fb)[TN]) {
#pragma unroll
        for (int tm = 0; tm < TM; ++tm)
#pragma unroll
            for (int tn = 0; tn < TN; ++tn)
                acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[tm], fb[tn], acc[tm][tn], 0, 0, 0);
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    gload(0, I0{});
    sstore(0, I0{});
    gload(1, I1{});
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    fread(0, 0, f1a, f1b);
    // step kt: data in buffer kt & 1; its slice-1 fragments already in f1; the loads of step kt+1
    // are in register set (kt+1) & 1 and those of kt+2 go to set kt & 1 (stored at step kt-1).
    // Every load, store and read is issued in every step (past the end the loads return zero and
    // the stores and reads touch buffers no later step uses), so the compiler counts the loads in
    // flight exactly.
    auto step = [&](int kt, auto lset, auto sset) {
        const int cur = kt & 1;
        __builtin_amdgcn_sched_barrier(0);
        gload(kt + 2, lset);
        fread(cur, 1, f2a, f2b);
        mfmas(f1a, f1b);
        sstore(cur ^ 1, sset);
        // 256 x 256 tile on 8 waves of 128 x 64: the 4 global loads and the 6 slice-2 reads among
        // the first 4 MFMAs, the 4 LDS stores among the last 4
        if constexpr (TM == 4 && TN == 2 && U == 2) {
            __builtin_amdgcn_sched_group_barrier(0x020, 4, 0);  // global loads
            __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);  // LDS reads of slice 2
            __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);  // MFMA
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
                __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);  // LDS store
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        fread(cur ^ 1, 0, f1a, f1b);
        mfmas(f2a, f2b);
        if constexpr (TM == 4 && TN == 2) {
            __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);  // LDS reads of the next slice 1
            __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);  // MFMAs of slice 2
        }
    };
    int kt = 0;
    for (; kt + 1 < nk; kt += 2) {
        step(kt, I0{}, I1{});
        step(kt + 1, I1{}, I0{});
    }
    if (kt < nk) step(kt, I0{}, I1{});
    __builtin_amdgcn_sched_barrier(0);
}

// SYRK main loop with the operands loaded straight into LDS (16-byte buffer loads with an LDS
// destination) from the MK-token block layout of Y^T.  Three LDS stages, each its own array: the
// loads of step kt + 2 are issued right after the barrier of step kt, into the stage that step
// kt - 1 read.  Before the barrier of step kt each wave waits only for its own loads of step kt
// (those of step kt + 1 stay in flight); the barrier is a plain s_barrier, since the compiler
// would otherwise wait for every load into LDS before each barrier.  No registers stage the
// operands and no LDS stores are issued.
// A wave's 16-byte load of row r lands at lds + r * 64 + 16 * (lane & 3) (linear in the lane), so
// the XOR swizzle of swz() is applied to the global side: that lane loads chunk (lane & 3) ^ f(r).
// Rows past rows[o] read zero through an offset of 2^31, past every operand's resource.
// The MFMA chains restart from zero every 64 tokens (two steps) and their sums are added to acc
// with one round-to-nearest fp32 add, so a running sum over many tokens carries the error of one
// fp32 addition per 64 tokens instead of a long chain of MFMA accumulations.
// NST 2: two stages and loads one step ahead, for kernels that share a CU two at a time (the other
// workgroup's MFMAs run while one waits), with each step's first LDS reads issued before the
// previous step ends (step2 below).
typedef __attribute__((address_space(3))) void lds_void_t;
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
__device__ __forceinline__ void lds_barrier() { asm volatile("s_barrier" ::: "memory"); }
// s_waitcnt with vmcnt = n (0..63) and no wait on the other counters (gfx9 encoding)
#define LRC_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (7 << 4) | (15 << 8) | (((n) >> 4) << 14))

// GEMM main loop with the operands loaded straight into LDS (k a multiple of the k step).  Three LDS
// stages; per step kt: loads of step kt+2 into the stage step kt-1 read; LDS reads of slice 2 of
// kt; MFMAs of slice 1 (its fragments read at the end of step kt-1); this wave's loads of step kt+1
// and its LDS reads done, barrier; LDS reads of slice 1 of kt+1; MFMAs of slice 2 of kt.  A lane's
// 16-byte load of row r lands at st + r * MK + 8 (lane & 3) (linear in the lane), so the swizzle of
// swz() is applied on the global side; rows past rows[o] read zero through an offset of 2^31.
//
// NP > 1 (the range-projected product): the A rows hold NP pieces of klen values each, side by
// side (A row length NP klen), all multiplied by the same B row, and only k steps kt0 .. klen/MK - 1
// of each piece are taken (A is zero left of them): step j of the loop is step kt0 + j % span of
// piece j / span, span = klen/MK - kt0.
template <int BM, int THREADS, int WGM, int NP = 1>
__device__ __forceinline__ void gemm_dma_mainloop(const bf16_t *const *base, const int64_t *ld, const int *rows,
                                                  int64_t klen,
                                                  f32x16_t (&acc)[MfmaCfg<BM, BM, THREADS, WGM>::TM][MfmaCfg<BM, BM, THREADS, WGM>::TN],
                                                  bf16_t *lds0, bf16_t *lds1, bf16_t *lds2, int kt0 = 0) {
    using T = MfmaCfg<BM, BM, THREADS, WGM>;
    constexpr int TM = T::TM, TN = T::TN, U = T::UA;
    static_assert(T::UA == T::UB, "square block tile");
    constexpr int RPU = 16 * (THREADS / 64);  // rows covered by one load per thread
    constexpr int LPS = 2 * U;                // loads per thread per step
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / T::WGN, wn = wave % T::WGN;
    const int nkx = int(klen / MK);
    const int span = NP == 1 ? nkx : nkx - kt0;
    const int nk = NP * span;
    if (nk <= 0) return;
    __amdgpu_buffer_rsrc_t rs[2];
    uint32_t roff[2][U];
#pragma unroll
    for (int o = 0; o < 2; ++o) {
        const int64_t kl = o == 0 ? NP * klen : klen;  // row length of the operand
        rs[o] = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<bf16_t *>(base[o]), short(0),
            int(rows[o] > 0 ? ((int64_t(rows[o]) - 1) * ld[o] + kl) * 2 : int64_t(0)), 0x00020000);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int r = 16 * wave + (lane >> 2) + RPU * u;
            const int c = (lane & 3) ^ (((r >> 1) ^ (r >> 3)) & 3);
            roff[o][u] = r < rows[o] ? uint32_t((int64_t(r) * ld[o] + c * 8) * 2) : 0x80000000u;
        }
    }
    auto issue = [&](int kt, bf16_t *st) {
        int ks[2] = {kt, kt};  // k step of A and of B
        if constexpr (NP > 1) {
            // steps past the last one (loaded, never read) stay inside the operands' resources
            static_assert(NP <= 3, "at most three pieces");
            const int p = int(kt >= span) + int(NP > 2 && kt >= 2 * span);
            ks[1] = kt0 + kt - p * span;
            ks[0] = p * nkx + ks[1];
        }
#pragma unroll
        for (int o = 0; o < 2; ++o)
#pragma unroll
            for (int u = 0; u < U; ++u)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rs[o], (lds_void_t *)(st + o * BM * MK + (16 * wave + RPU * u) * MK),
                                                         16, int(roff[o][u] + uint32_t(ks[o]) * uint32_t(MK * 2)), 0, 0, 0);
    };
    bf16x8_t f1a[TM], f1b[TN], f2a[TM], f2b[TN];
    auto fread = [&](const bf16_t *st, int ks, bf16x8_t (&fa)[TM], bf16x8_t (&fb)[TN]) {
        const int c = ks * 2 + (lane >> 5);
#pragma unroll
        for (int t = 0; t < TM; ++t)
            fa[t] = *reinterpret_cast<const bf16x8_t *>(st + swz(wm * T::WM + t * 32 + (lane & 31), c));
#pragma unroll
        for (int t = 0; t < TN; ++t)
            fb[t] = *reinterpret_cast<const bf16x8_t *>(st + BM * MK + swz(wn * T::WN + t * 32 + (lane & 31), c));
    };
    auto mfmas = [&](const bf16x8_t (&fa)[TM], const bf16x8_t (&fb)[TN]) {
#pragma unroll
        for (int tm = 0; tm < TM; ++tm)
#pragma unroll
            for (int tn = 0; tn < TN; ++tn)
                acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[tm], fb[tn], acc[tm][tn], 0, 0, 0);
    };
    auto step = [&](int kt, const bf16_t *cur, const bf16_t *nxt, bf16_t *fre) {
        __builtin_amdgcn_sched_barrier(0);
        issue(kt + 2, fre);
        fread(cur, 1, f2a, f2b);
        mfmas(f1a, f1b);
        if constexpr (TM == 4 && TN == 2 && LPS == 4) {
#pragma unroll
            for (int i = 0; i < 3; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // load into LDS
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // LDS reads of slice 2
                __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // MFMA
            }
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        LRC_WAIT_VMCNT(LPS);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        lds_barrier();
        __builtin_amdgcn_sched_barrier(0);
        fread(nxt, 0, f1a, f1b);
        mfmas(f2a, f2b);
        if constexpr (TM == 4 && TN == 2) {
#pragma unroll
            for (int i = 0; i < 3; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // LDS reads of the next slice 1
                __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // MFMA
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        }
    };
    issue(0, lds0);
    issue(1, lds1);
    LRC_WAIT_VMCNT(LPS);
    lds_barrier();
    fread(lds0, 0, f1a, f1b);
    int kt = 0;
    for (; kt + 2 < nk; kt += 3) {
        step(kt, lds0, lds1, lds2);
        step(kt + 1, lds1, lds2, lds0);
        step(kt + 2, lds2, lds0, lds1);
    }
    if (kt < nk) step(kt, lds0, lds1, lds2);
    if (kt + 1 < nk) step(kt + 1, lds1, lds2, lds0);
    // the loads issued past the last step still write LDS: let them land before the epilogue
    __builtin_amdgcn_sched_barrier(0);
    LRC_WAIT_VMCNT(0);
    lds_barrier();
}

template <int BM, int BN, int NOPS, int NPROD, int NST, int THREADS, int WGM>
__device__ __forceinline__ void syrk_dma_mainloop(const bf16_t *const *base, const int64_t D, const int *rows,
                                                  int64_t klen, const int64_t *nrec,
                                                  f32x16_t (&acc)[MfmaCfg<BM, BN, THREADS, WGM>::TM][MfmaCfg<BM, BN, THREADS, WGM>::TN],
                                                  bf16_t *lds0, bf16_t *lds1, bf16_t *lds2) {
    using T = MfmaCfg<BM, BN, THREADS, WGM>;
    constexpr int RPU = 16 * (THREADS / 64);  // rows of an operand covered by one load per thread
    constexpr int TM = T::TM, TN = T::TN, UA = T::UA, UB = T::UB;
    constexpr int U = UA > UB ? UA : UB;
    constexpr int NSIDE = NOPS / 2;
    // NPROD 1: one bf16 operand per side; 3: fp16 hi and lo per side, hi hi + hi lo + lo hi
    constexpr int NA = (NPROD == 3) ? 2 : 1;
    static_assert(NSIDE == NA, "hi/lo operands per side");
    static_assert(NPROD == 1 || NPROD == 3, "products");
    using OpT = typename std::conditional<NPROD == 1, bf16x8_t, f16x8_t>::type;
    auto mfma = [](OpT x, OpT y, f32x16_t c) {
        if constexpr (NPROD == 1)
            return __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, y, c, 0, 0, 0);
        else
            return __builtin_amdgcn_mfma_f32_32x32x16_f16(x, y, c, 0, 0, 0);
    };
    constexpr int LPS = NSIDE * (UA + UB);  // loads per thread per step
    auto opoff = [](int o) { return o < NSIDE ? o * BM * MK : NSIDE * BM * MK + (o - NSIDE) * BN * MK; };
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / T::WGN, wn = wave % T::WGN;
    const int nk = int(klen / MK);
    if (nk <= 0) return;
    __amdgpu_buffer_rsrc_t rs[NOPS];
    uint32_t roff[NOPS][U];
#pragma unroll
    for (int o = 0; o < NOPS; ++o) {
        rs[o] = __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t *>(base[o]), short(0), int(nrec[o]), 0x00020000);
#pragma unroll
        for (int u = 0; u < (o < NSIDE ? UA : UB); ++u) {
            const int r = 16 * wave + (lane >> 2) + RPU * u;  // row of this lane's 16 bytes
            const int c = (lane & 3) ^ (((r >> 1) ^ (r >> 3)) & 3);
            roff[o][u] = r < rows[o] ? uint32_t((r * MK + c * 8) * 2) : 0x80000000u;
        }
    }
    const uint32_t kstride = uint32_t(D * MK * 2);
    // loads of step kt into a stage: for operand o and chunk u, wave w fills rows 16 w + 64 u ..
    auto issue = [&](int kt, bf16_t *st) {
#pragma unroll
        for (int o = 0; o < NOPS; ++o)
#pragma unroll
            for (int u = 0; u < (o < NSIDE ? UA : UB); ++u)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rs[o], (lds_void_t *)(st + opoff(o) + (16 * wave + RPU * u) * MK), 16,
                    int(roff[o][u] + uint32_t(kt) * kstride), 0, 0, 0);
    };
    f32x16_t p[TM][TN];
#pragma unroll
    for (int tm = 0; tm < TM; ++tm)
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) p[tm][tn] = f32x16_t{};
    auto flush = [&]() {
#pragma unroll
        for (int tm = 0; tm < TM; ++tm)
#pragma unroll
            for (int tn = 0; tn < TN; ++tn)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[tm][tn][r] = __fadd_rn(acc[tm][tn][r], p[tm][tn][r]);
    };
    // one step: publish stage `cur` (this wave's loads of step kt done, then the barrier), issue the
    // loads of step kt + 2 into `nxt`, then the MFMAs from `cur`; PAR: position in the flush group
    auto step = [&](int kt, const bf16_t *cur, bf16_t *nxt, auto par) {
        constexpr int PAR = decltype(par)::value;
        // nothing moves across a step boundary: the wait below is for loads issued a step earlier,
        // and MFMAs of the previous step scheduled after it would wait for them too
        __builtin_amdgcn_sched_barrier(0);
        LRC_WAIT_VMCNT(LPS);
        lds_barrier();
        issue(kt + 2, nxt);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const int c = ks * 2 + (lane >> 5);
            OpT af[NA][TM], bfr[NA][TN];
#pragma unroll
            for (int a = 0; a < NA; ++a) {
#pragma unroll
                for (int t = 0; t < TM; ++t)
                    af[a][t] = *reinterpret_cast<const OpT *>(cur + opoff(a) + swz(wm * T::WM + t * 32 + (lane & 31), c));
#pragma unroll
                for (int t = 0; t < TN; ++t)
                    bfr[a][t] =
                        *reinterpret_cast<const OpT *>(cur + opoff(NSIDE + a) + swz(wn * T::WN + t * 32 + (lane & 31), c));
            }
#pragma unroll
            for (int tm = 0; tm < TM; ++tm)
#pragma unroll
                for (int tn = 0; tn < TN; ++tn) {
                    // a flush group's first slice starts the chain from a literal zero
                    const bool fresh = PAR == 0 && ks == 0;
                    f32x16_t q = mfma(af[0][tm], bfr[0][tn], fresh ? f32x16_t{} : p[tm][tn]);
                    if (NPROD == 3) {
                        q = mfma(af[0][tm], bfr[1][tn], q);
                        q = mfma(af[1][tm], bfr[0][tn], q);
                    }
                    p[tm][tn] = q;
                }
        }
        if (PAR == 1) flush();
        if constexpr (NST == 3 && NPROD == 3 && LPS == 12 && NA * (TM + TN) == 12 && TM * TN * NPROD == 24) {
            // 256 x 128 split tile: spread the step's 12 loads over the first slice's 24 MFMAs, with
            // the second slice's 12 LDS reads between them, instead of issuing the loads in one
            // burst after the barrier (7 % faster at d_out 11008, 3 % at 4096)
            __builtin_amdgcn_sched_group_barrier(0x100, 12, 0);  // LDS reads of the first slice
#pragma unroll
            for (int i = 0; i < 12; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // MFMA
                __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // load into LDS
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read of the second slice
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 24, 0);  // MFMAs of the second slice
        }
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    // Two stages, with the LDS reads of each step's first slice issued before the previous step
    // ends.  Step kt (its slice-1 fragments read at the end of step kt-1): slice-2 reads of kt and
    // slice-1 MFMAs; this wave's loads of step kt+1 and its LDS reads done, barrier; loads of step
    // kt+2 into the stage of kt (read completely before the barrier); slice-1 reads of kt+1; slice-2
    // MFMAs of kt.  The loads of a step have one step of MFMAs to land, and the reads after the
    // barrier are in flight while the slice-2 MFMAs run instead of stalling the next step's first.
    OpT f1a[NA][TM], f1b[NA][TN], f2a[NA][TM], f2b[NA][TN];
    auto fread = [&](const bf16_t *st, int ks, OpT (&fa)[NA][TM], OpT (&fb)[NA][TN]) {
        const int c = ks * 2 + (lane >> 5);
#pragma unroll
        for (int a = 0; a < NA; ++a) {
#pragma unroll
            for (int t = 0; t < TM; ++t)
                fa[a][t] = *reinterpret_cast<const OpT *>(st + opoff(a) + swz(wm * T::WM + t * 32 + (lane & 31), c));
#pragma unroll
            for (int t = 0; t < TN; ++t)
                fb[a][t] = *reinterpret_cast<const OpT *>(st + opoff(NSIDE + a) + swz(wn * T::WN + t * 32 + (lane & 31), c));
        }
    };
    auto mfmas = [&](const OpT (&fa)[NA][TM], const OpT (&fb)[NA][TN], bool fresh) {
#pragma unroll
        for (int tm = 0; tm < TM; ++tm)
#pragma unroll
            for (int tn = 0; tn < TN; ++tn) {
                f32x16_t q = mfma(fa[0][tm], fb[0][tn], fresh ? f32x16_t{} : p[tm][tn]);
                if (NPROD == 3) {
                    q = mfma(fa[0][tm], fb[1][tn], q);
                    q = mfma(fa[1][tm], fb[0][tn], q);
                }
                p[tm][tn] = q;
            }
    };
    auto step2 = [&](int kt, bf16_t *cur, const bf16_t *nxt, auto par) {
        constexpr int PAR = decltype(par)::value;
        __builtin_amdgcn_sched_barrier(0);
        fread(cur, 1, f2a, f2b);
        mfmas(f1a, f1b, PAR == 0);  // a flush group's first slice starts its chains from zero
        if constexpr (NPROD == 3 && NA * (TM + TN) == 8 && TM * TN == 4) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // LDS reads of slice 2
                __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);  // MFMA
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        LRC_WAIT_VMCNT(0);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        lds_barrier();
        __builtin_amdgcn_sched_barrier(0);
        issue(kt + 2, cur);
        fread(nxt, 0, f1a, f1b);
        mfmas(f2a, f2b, false);
        if constexpr (NPROD == 3 && NA * (TM + TN) == 8 && TM * TN == 4 && LPS == 8) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);  // loads into LDS
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // LDS reads of the next slice 1
                __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);  // MFMA
            }
        }
        if (PAR == 1) flush();
    };
    if constexpr (NST == 2) {
        // stages 0 1 0 1 ..., flush-group positions 0 1 0 1 ...
        issue(0, lds0);
        LRC_WAIT_VMCNT(0);
        lds_barrier();
        issue(1, lds1);
        fread(lds0, 0, f1a, f1b);
        int kt = 0;
        for (; kt + 1 < nk; kt += 2) {
            step2(kt, lds0, lds1, I0{});
            step2(kt + 1, lds1, lds0, I1{});
        }
        if (kt < nk) {
            step2(kt, lds0, lds1, I0{});
            flush();  // the last flush group had only its first step
        }
        // the loads issued past the last step still write LDS: let them land before the epilogue
        LRC_WAIT_VMCNT(0);
        lds_barrier();
        return;
    }
    issue(0, lds0);
    issue(1, lds1);
    // six steps per iteration: stages 0 1 2 0 1 2, flush-group positions 0 1 0 1 0 1
    int kt = 0;
    for (; kt + 5 < nk; kt += 6) {
        step(kt, lds0, lds2, I0{});
        step(kt + 1, lds1, lds0, I1{});
        step(kt + 2, lds2, lds1, I0{});
        step(kt + 3, lds0, lds2, I1{});
        step(kt + 4, lds1, lds0, I0{});
        step(kt + 5, lds2, lds1, I1{});
    }
    const int r = nk - kt;
    if (r > 0) step(kt, lds0, lds2, I0{});
    if (r > 1) step(kt + 1, lds1, lds0, I1{});
    if (r > 2) step(kt + 2, lds2, lds1, I0{});
    if (r > 3) step(kt + 3, lds0, lds2, I1{});
    if (r > 4) step(kt + 4, lds1, lds0, I0{});
    if (r & 1) flush();  // the last flush group had only its first step
    // the loads issued past the last step still write LDS: let them land before the epilogue
    LRC_WAIT_VMCNT(0);
    lds_barrier();
}

// Output position of accumulator element r of lane `lane` in a 32x32 MFMA tile.
__device__ __forceinline__ int acc_row(int lane, int r) { return (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3); }
__device__ __forceinline__ int acc_col(int lane) { return lane & 31; }

// Y^T[ib + row][t] for the 16 values of one lane, in the MK-token block layout: s = y 2^ex[i]
// (exact), hi = fp16(s), lo = fp16(s - hi) (s - hi is exact in fp32), stored as fp16 bit patterns
__device__ __forceinline__ void store_split_tile(const f32x16_t a, int64_t ib, int64_t t, int lane, int64_t d_out,
                                                 const int32_t *__restrict__ ex, bf16_t *__restrict__ Yhi,
                                                 bf16_t *__restrict__ Ylo) {
    const int64_t tb = (t / MK) * d_out * MK + t % MK;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int64_t i = ib + acc_row(lane, r);
        if (i < d_out) {
            const float y = ldexpf(a[r], ex[i]);
            const _Float16 hi = _Float16(y);
            const _Float16 lo = _Float16(y - float(hi));
            Yhi[tb + i * MK] = __builtin_bit_cast(bf16_t, hi);
            Ylo[tb + i * MK] = __builtin_bit_cast(bf16_t, lo);
        }
    }
}

// dst[rb + row][cc] += value for the upper triangle (row <= col) inside the hd x hd block; with
// ex (exponents of the block's rows), value = a 2^-(ex[row] + ex[col]), exact up to fp32 range
__device__ __forceinline__ void add_upper_tile(const f32x16_t a, int64_t rb, int64_t cc, int lane, int64_t hd,
                                               const int32_t *__restrict__ ex, float *__restrict__ dst, int64_t ldd) {
    const int ec = (ex && cc < hd) ? ex[cc] : 0;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int64_t rr = rb + acc_row(lane, r);
        if (rr < hd && cc < hd && rr <= cc) dst[rr * ldd + cc] += ex ? ldexpf(a[r], -(ex[rr] + ec)) : a[r];
    }
}

// Phase 1: Y^T tile (rows = output features i, cols = tokens t), split into hi/lo.
constexpr int G_BM = 256, G_THREADS = 512, G_WGM = 2;
constexpr int G_GT = 8;  // token tiles per group of the launch order

// Tile (i, t) of block b in a 1-D launch of gi x gt tiles.  Workgroups go to the 8 XCDs in turn
// (b mod 8), and each XCD has an L2 of its own: XCD x gets a contiguous share of the tiles, taken
// in groups of G_GT token tiles by all gi feature tiles, feature tile after feature tile, so the
// ~32 workgroups an XCD runs at once share 4 tiles of W^T and 8 of X.  In the order of a 2-D grid
// the workgroups sharing a tile of X sat on different XCDs: a 4096 x 11008 chunk fetched 18.6 GB
// from HBM against 5.0 GB in this order (the kernel is bound by its MFMA loop, not by this traffic:
// 1.5 % faster).
__device__ __forceinline__ void gemm_tile_of(int64_t b, int64_t gi, int64_t gt, int64_t &i, int64_t &t) {
    const int64_t N = gi * gt, per = N / 8, extra = N % 8;
    const int64_t x = b % 8, slot = b / 8;
    const int64_t L = x * per + (x < extra ? x : extra) + slot;
    const int64_t g = L / (G_GT * gi);
    const int64_t t0 = g * G_GT, gte = gt - t0 < G_GT ? gt - t0 : G_GT;
    const int64_t r = L - g * G_GT * gi;
    i = r / gte;
    t = t0 + r % gte;
}
// NP == 3: the range-projected product Y~ = X L.  Wt then holds A = L^T (d_out = d_in rows) as
// three bf16 pieces side by side (row length 3 d_in, see k_range_pieces); A is upper triangular,
// so block row i0 takes only the k steps from i0 / MK on, in each piece.
template <int BM, bool KCHECK, int NP = 1>
__global__ void __launch_bounds__(G_THREADS) __attribute__((amdgpu_waves_per_eu(2, 2)))
k_cov_gemm_y(const bf16_t *__restrict__ Wt, int64_t d_in, int64_t d_out, const bf16_t *__restrict__ X, int64_t ldx,
             int64_t tc, const int32_t *__restrict__ ex, bf16_t *__restrict__ Yhi, bf16_t *__restrict__ Ylo) {
    static_assert(NP == 1 || !KCHECK, "pieces need a contraction length that is a multiple of the k step");
    using Cfg = MfmaCfg<BM, BM, G_THREADS, G_WGM>;
    __shared__ __attribute__((aligned(16))) bf16_t lds[(KCHECK ? 2 : 3) * 2 * BM * MK];
    int64_t ti, tt;
    gemm_tile_of(blockIdx.x, (d_out + BM - 1) / BM, (tc + BM - 1) / BM, ti, tt);
    const int64_t i0 = ti * BM, t0 = tt * BM;
    const bf16_t *base[2] = {Wt + i0 * d_in * NP, X + t0 * ldx};
    const int64_t ld[2] = {d_in * NP, ldx};
    const int rows[2] = {int(std::min<int64_t>(BM, d_out - i0)), int(std::max<int64_t>(0, std::min<int64_t>(BM, tc - t0)))};
    f32x16_t acc[Cfg::TM][Cfg::TN];
#pragma unroll
    for (int a = 0; a < Cfg::TM; ++a)
#pragma unroll
        for (int b = 0; b < Cfg::TN; ++b) acc[a][b] = f32x16_t{};
    if constexpr (KCHECK)
        gemm_mainloop<BM, G_THREADS, G_WGM, KCHECK>(base, ld, rows, d_in, acc, lds);
    else
        gemm_dma_mainloop<BM, G_THREADS, G_WGM, NP>(base, ld, rows, d_in, acc, lds, lds + 2 * BM * MK, lds + 4 * BM * MK,
                                                    NP > 1 ? int(i0 / MK) : 0);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, wm = wave / Cfg::WGN, wn = wave % Cfg::WGN;
#pragma unroll
    for (int tm = 0; tm < Cfg::TM; ++tm)
#pragma unroll
        for (int tn = 0; tn < Cfg::TN; ++tn) {
            const int64_t ib = i0 + wm * Cfg::WM + tm * 32;
            const int64_t t = t0 + wn * Cfg::WN + tn * 32 + acc_col(lane);
            store_split_tile(acc[tm][tn], ib, t, lane, d_out, ex, Yhi, Ylo);
        }
}

// Per-head covariance in one kernel (WSVD page, methodology 1: the covariance of each head's slice of
// the output): workgroup (h, s) takes head h's 128 outputs over token range s.  Per 128-token tile the
// GEMM main loop above forms Y_h^T (128 outputs x 128 tokens) = W_h^T X_tile^T; the epilogue scales y
// by 2^e_i and splits it into fp16 hi and lo straight into LDS (over the GEMM's stages, free by then);
// C_h's upper 64 x 64 blocks then take hi hi^T + hi lo^T + lo hi^T from LDS (three of the four waves;
// each 64-token MFMA chain starts from zero and is added to the running block with a round-to-nearest
// fp32 add, as in k_cov_syrk), and every output's sum of lo^2 is formed from LDS too, so Y never goes
// to memory.  The range's C_h (scaled back by 2^-(e_i + e_j)) and sums of lo^2 (by 2^-2e_i) go to
// P[s][h] and PD[s][h]; k_head_reduce adds them into C in range order.  Workgroup b = h S + s runs on
// XCD b mod 8, so with S a multiple of 8 every head of one token range runs on one XCD and its L2 holds
// the range's rows of X for all of them.
constexpr int HF = 128;  // head width, and tokens per tile
constexpr int HF_THREADS = 512;
constexpr int HF_WGM = 4;  // 8 waves, 4 x 2, of 32 x 64
// element (i, t) of a 128 x 128 fp16 tile, row i contiguous along t, 16-byte chunks XOR-swizzled by i so
// that the 16 rows a quarter-wave reads at one chunk column land in 16 different bank groups
__device__ __forceinline__ int hf_sw(int i, int t) { return i * HF + (((t >> 3) ^ (i & 15)) << 3) + (t & 7); }

__global__ void __launch_bounds__(HF_THREADS) __attribute__((amdgpu_waves_per_eu(2, 2)))
k_cov_head_fused(const bf16_t *__restrict__ Wt, int64_t d_in, const bf16_t *__restrict__ X, int64_t ldx,
                 int64_t n_tok, int64_t tpr, int S, const int32_t *__restrict__ ex, float *__restrict__ P,
                 float *__restrict__ PD) {
    using Cfg = MfmaCfg<HF, HF, HF_THREADS, HF_WGM>;
    static_assert(Cfg::TM == 1 && Cfg::TN == 2 && Cfg::WM == 32 && Cfg::WN == 64, "wave tile");
    // three GEMM stages (2 x 128 x 32 bf16 each) or the Y tile (hi and lo, 2 x 128 x 128 fp16)
    __shared__ __attribute__((aligned(16))) bf16_t lds[2 * HF * HF];
    const int H = int(gridDim.x) / S;
    const int h = int(blockIdx.x) / S, s = int(blockIdx.x) % S;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / Cfg::WGN, wn = wave % Cfg::WGN;
    const int64_t tbeg = int64_t(s) * tpr, tend = std::min<int64_t>(n_tok, tbeg + tpr);
    const int32_t *exh = ex + int64_t(h) * HF;
    bf16_t *yhi = lds, *ylo = lds + HF * HF;
    // this wave's block of C_h: rows 32 wm .. + 31, columns 64 wn .. + 63; the six blocks that meet the
    // upper triangle are formed (waves (2, 0) and (3, 0) lie below it)
    const bool cwave = wm <= 2 * wn + 1;
    f32x16_t cacc[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) cacc[b] = f32x16_t{};
    float sq = 0.f;  // sum of lo^2 of output tid / 4 over tokens (tid & 3) 32 .. + 31 of each tile
    for (int64_t t0 = tbeg; t0 < tend; t0 += HF) {
        f32x16_t acc[1][2] = {{f32x16_t{}, f32x16_t{}}};
        const bf16_t *base[2] = {Wt + int64_t(h) * HF * d_in, X + t0 * ldx};
        const int64_t ld[2] = {d_in, ldx};
        const int rows[2] = {HF, int(std::min<int64_t>(HF, tend - t0))};
        // ends with its loads landed and a barrier: the stages are free afterwards
        gemm_dma_mainloop<HF, HF_THREADS, HF_WGM>(base, ld, rows, d_in, acc, lds, lds + 2 * HF * MK,
                                                  lds + 4 * HF * MK);
#pragma unroll
        for (int tn = 0; tn < 2; ++tn)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int i = wm * 32 + acc_row(lane, r);
                const int t = wn * 64 + tn * 32 + acc_col(lane);
                const float y = ldexpf(acc[0][tn][r], exh[i]);
                const _Float16 hi = _Float16(y);
                const _Float16 lo = _Float16(y - float(hi));
                yhi[hf_sw(i, t)] = __builtin_bit_cast(bf16_t, hi);
                ylo[hf_sw(i, t)] = __builtin_bit_cast(bf16_t, lo);
            }
        __syncthreads();
        {
            const int i = tid >> 2, tb = (tid & 3) * 32;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const f16x8_t v = *reinterpret_cast<const f16x8_t *>(ylo + hf_sw(i, tb + c * 8));
#pragma unroll
                for (int u = 0; u < 8; ++u) sq = fmaf(float(v[u]), float(v[u]), sq);
            }
        }
        if (cwave) {
#pragma unroll
            for (int ch = 0; ch < 2; ++ch) {  // two 64-token chains
                f32x16_t p[2];
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {  // 16 tokens per slice
                    const int tok = ch * 64 + ks * 16 + (lane >> 5) * 8;
                    const int ia = wm * 32 + (lane & 31);
                    const f16x8_t ah = *reinterpret_cast<const f16x8_t *>(yhi + hf_sw(ia, tok));
                    const f16x8_t al = *reinterpret_cast<const f16x8_t *>(ylo + hf_sw(ia, tok));
                    f16x8_t bh[2], bl[2];
#pragma unroll
                    for (int q = 0; q < 2; ++q) {
                        const int ib = wn * 64 + q * 32 + (lane & 31);
                        bh[q] = *reinterpret_cast<const f16x8_t *>(yhi + hf_sw(ib, tok));
                        bl[q] = *reinterpret_cast<const f16x8_t *>(ylo + hf_sw(ib, tok));
                    }
#pragma unroll
                    for (int tn = 0; tn < 2; ++tn) {
                        f32x16_t q = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah, bh[tn], ks == 0 ? f32x16_t{} : p[tn],
                                                                            0, 0, 0);
                        q = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah, bl[tn], q, 0, 0, 0);
                        q = __builtin_amdgcn_mfma_f32_32x32x16_f16(al, bh[tn], q, 0, 0, 0);
                        p[tn] = q;
                    }
                }
#pragma unroll
                for (int tn = 0; tn < 2; ++tn)
#pragma unroll
                    for (int r = 0; r < 16; ++r) cacc[tn][r] = __fadd_rn(cacc[tn][r], p[tn][r]);
            }
        }
        __syncthreads();  // the next tile's loads overwrite the Y tile
    }
    float *dst = P + (int64_t(s) * H + h) * HF * HF;
    if (cwave) {
#pragma unroll
        for (int tn = 0; tn < 2; ++tn)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int i = wm * 32 + acc_row(lane, r);
                const int j = wn * 64 + tn * 32 + acc_col(lane);
                if (i <= j) dst[i * HF + j] = ldexpf(cacc[tn][r], -(exh[i] + exh[j]));
            }
    }
    sq += __shfl_xor(sq, 1);
    sq += __shfl_xor(sq, 2);
    if ((tid & 3) == 0) PD[(int64_t(s) * H + h) * HF + (tid >> 2)] = ldexpf(sq, -2 * exh[tid >> 2]);
}

// C_h[i][j] (i <= j) += sum_s P[s][h][i][j] (+ sum_s PD[s][h][i] on the diagonal), s in order; head h's
// block at C + h * HF * ldc
__global__ void __launch_bounds__(256) k_head_reduce(float *__restrict__ C, int64_t ldc, const float *__restrict__ P,
                                                     const float *__restrict__ PD, int S, int H) {
    const int64_t per = int64_t(HF) * HF, total = per * H;
    for (int64_t e = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; e < total; e += int64_t(gridDim.x) * blockDim.x) {
        const int h = int(e / per), i = int((e % per) / HF), j = int(e % HF);
        if (i > j) continue;
        float acc = C[int64_t(h) * HF * ldc + int64_t(i) * ldc + j];
        for (int s = 0; s < S; ++s) acc += P[(int64_t(s) * H + h) * per + int64_t(i) * HF + j];
        if (i == j)
            for (int s = 0; s < S; ++s) acc += PD[(int64_t(s) * H + h) * HF + i];
        C[int64_t(h) * HF * ldc + int64_t(i) * ldc + j] = acc;
    }
}

// Phase 2: block tiles of each head block that meet its upper triangle, split s of the token
// range.  A tile is BM rows (block row I) by BN columns (block column J); it meets the upper
// triangle when its last column is at or right of its first row.  Tiles are numbered column
// by column: column J holds syrk_col_tiles(J) tiles, I = 0, 1, ...
template <int BM, int BN>
__host__ __device__ __forceinline__ int syrk_col_tiles(int J, int nI) {
    return min(nI, (BN * J + BN - 1) / BM + 1);
}
template <int BM, int BN>
__host__ __device__ __forceinline__ int syrk_tiles(int hd) {
    const int nI = (hd + BM - 1) / BM, nJ = (hd + BN - 1) / BN;
    int n = 0;
    for (int J = 0; J < nJ; ++J) n += syrk_col_tiles<BM, BN>(J, nI);
    return n;
}
template <int BM, int BN, int THREADS>
struct SyrkCfg {  // 4 waves of (BM/2) x (BN/2), or 8 waves of (BM/4) x (BN/2)
    static constexpr int WGM = THREADS == 512 ? 4 : 2;
};
// SPLIT: Y^T as fp16 hi/lo with the row exponents ex, three products (the diagonal's sum of lo^2
// is added by k_lo_sq_add); else Y^T = X^T in bf16, one product.
// NST: LDS stages of the main loop; 2 lets two workgroups share a CU (65536 bytes of LDS each).
template <int BM, int BN, bool SPLIT, int NST, int THREADS = 256>
__global__ void __launch_bounds__(THREADS)
__attribute__((amdgpu_waves_per_eu(NST == 2 || THREADS == 512 ? 2 : 1, NST == 2 || THREADS == 512 ? 2 : 1)))
k_cov_syrk(const bf16_t *__restrict__ Yhi, const bf16_t *__restrict__ Ylo, const int32_t *__restrict__ ex,
           int64_t ldy, int64_t ktot, int64_t kchunk, int64_t hd, float *__restrict__ C, int64_t ldc,
           float *__restrict__ P, int32_t n_blocks, int32_t xcd_order) {
    constexpr int WGM = SyrkCfg<BM, BN, THREADS>::WGM;
    static_assert(THREADS == 256 || THREADS == 512, "launch bounds");
    using Cfg = MfmaCfg<BM, BN, THREADS, WGM>;
    constexpr int NOPS = SPLIT ? 4 : 2;
    constexpr int STAGE = (NOPS / 2) * (BM + BN) * MK;  // elements of one LDS stage
    __shared__ __attribute__((aligned(16))) bf16_t lds0[STAGE];
    __shared__ __attribute__((aligned(16))) bf16_t lds1[STAGE];
    __shared__ __attribute__((aligned(16))) bf16_t lds2[NST == 3 ? STAGE : 8];
    int u = blockIdx.x, h = blockIdx.y, s = blockIdx.z;
    int I, J;
    if (BM == BN && xcd_order) {
        // Workgroups go to the 8 XCDs in turn (linear id mod 8), each with an L2 of its own: XCD x
        // takes a contiguous share of the (tile, head block, split) order, and tiles are ordered in
        // super-tiles of 8 x 8, so the ~64 workgroups an XCD runs at once share 16 panels of Y^T
        // (d_out 11008: 12.55 -> 11.96 ms per chunk; at 4096, 528 tiles in 7 token splits, 4 %
        // slower, so the host asks for it only with many tiles per split).
        const int64_t G = int64_t(gridDim.x) * gridDim.y * gridDim.z;
        const int64_t g = blockIdx.x + int64_t(gridDim.x) * (blockIdx.y + int64_t(gridDim.y) * blockIdx.z);
        const int64_t x = g % 8, slot = g / 8, per = G / 8, extra = G % 8;
        const int64_t L = x * per + (x < extra ? x : extra) + slot;
        u = int(L % gridDim.x);
        h = int((L / gridDim.x) % gridDim.y);
        s = int(L / (int64_t(gridDim.x) * gridDim.y));
        // tile u: super-tile column block jb (columns 8 jb ..), super-tile row block ib, then column
        // by column inside the super-tile; column j holds min(nI, j + 1) tiles
        const int nI = int((hd + BM - 1) / BM), nJ = nI;
        constexpr int SI = 8, SJ = 8;
        int rem = u, jb = 0;
        for (;; ++jb) {
            int cnt = 0;
            for (int j = jb * SJ; j < min(nJ, jb * SJ + SJ); ++j) cnt += min(nI, j + 1);
            if (rem < cnt || jb * SJ + SJ >= nJ) break;
            rem -= cnt;
        }
        int ib = 0;
        for (;; ++ib) {
            int cnt = 0;
            for (int j = jb * SJ; j < min(nJ, jb * SJ + SJ); ++j) cnt += max(0, min(min(nI, j + 1), ib * SI + SI) - ib * SI);
            if (rem < cnt || ib * SI + SI >= nI) break;
            rem -= cnt;
        }
        J = jb * SJ;
        I = ib * SI;
        for (int j = jb * SJ; j < min(nJ, jb * SJ + SJ); ++j) {
            const int nj = max(0, min(min(nI, j + 1), ib * SI + SI) - ib * SI);
            if (rem < nj) {
                J = j;
                I = ib * SI + rem;
                break;
            }
            rem -= nj;
        }
    } else if constexpr (BM == BN) {  // column J holds J + 1 tiles: closed form
        J = int((sqrtf(8.f * float(u) + 1.f) - 1.f) * 0.5f);
        while (J * (J + 1) / 2 > u) --J;
        while ((J + 1) * (J + 2) / 2 <= u) ++J;
        I = u - J * (J + 1) / 2;
    } else {
        const int nI = int((hd + BM - 1) / BM);
        int rem = u;
        J = 0;
        while (rem >= syrk_col_tiles<BM, BN>(J, nI)) rem -= syrk_col_tiles<BM, BN>(J++, nI);
        I = rem;
    }
    const int64_t kb = int64_t(s) * kchunk;
    const int64_t klen = std::min(kchunk, ktot - kb);
    if (klen <= 0) return;
    const int64_t r0 = int64_t(h) * hd + int64_t(I) * BM, c0 = int64_t(h) * hd + int64_t(J) * BN;
    const int rowsI = int(std::min<int64_t>(BM, hd - int64_t(I) * BM));
    const int rowsJ = int(std::min<int64_t>(BN, hd - int64_t(J) * BN));
    // operands in the MK-token block layout (D rows per block); each buffer resource runs from
    // the operand's first element to the end of the chunk (D * ldy elements)
    const int64_t D = hd * n_blocks;
    const int64_t offI = (kb / MK) * D * MK + r0 * MK, offJ = (kb / MK) * D * MK + c0 * MK;
    const bf16_t *base[4];
    int64_t ld[4];
    int rows[4];
    if (SPLIT) {
        base[0] = Yhi + offI; base[1] = Ylo + offI;
        base[2] = Yhi + offJ; base[3] = Ylo + offJ;
        rows[0] = rows[1] = rowsI; rows[2] = rows[3] = rowsJ;
    } else {
        base[0] = Yhi + offI; base[1] = Yhi + offJ;
        rows[0] = rowsI; rows[1] = rowsJ;
    }
    int64_t nrec[4];  // bytes from each operand's base to the end of its buffer
    for (int o = 0; o < 4; ++o) ld[o] = D;
    if (SPLIT) {
        nrec[0] = nrec[1] = (D * ldy - offI) * 2;
        nrec[2] = nrec[3] = (D * ldy - offJ) * 2;
    } else {
        nrec[0] = (D * ldy - offI) * 2;
        nrec[1] = (D * ldy - offJ) * 2;
    }
    f32x16_t acc[Cfg::TM][Cfg::TN];
#pragma unroll
    for (int a = 0; a < Cfg::TM; ++a)
#pragma unroll
        for (int b = 0; b < Cfg::TN; ++b) acc[a][b] = f32x16_t{};
    // klen is a multiple of MK here, so no k check is needed
    syrk_dma_mainloop<BM, BN, NOPS, SPLIT ? 3 : 1, NST, THREADS, WGM>(base, D, rows, klen, nrec, acc, lds0, lds1, lds2);
    float *dst;
    int64_t ldd;
    if (s == 0) {
        dst = C + int64_t(h) * hd * ldc;
        ldd = ldc;
    } else {
        dst = P + (int64_t(s - 1) * n_blocks + h) * hd * hd;
        ldd = hd;
    }
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, wm = wave / Cfg::WGN, wn = wave % Cfg::WGN;
#pragma unroll
    for (int tm = 0; tm < Cfg::TM; ++tm)
#pragma unroll
        for (int tn = 0; tn < Cfg::TN; ++tn) {
            const int64_t rb = int64_t(I) * BM + wm * Cfg::WM + tm * 32;
            const int64_t cc = int64_t(J) * BN + wn * Cfg::WN + tn * 32 + acc_col(lane);
            add_upper_tile(acc[tm][tn], rb, cc, lane, hd, SPLIT ? ex + int64_t(h) * hd : nullptr, dst, ldd);
        }
}

// W^T (d_out x d_in) from W (d_in x d_out, ldw)
__global__ void __launch_bounds__(256) k_transpose_bf16(const bf16_t *__restrict__ W, int64_t ldw, int64_t rows,
                                                        int64_t cols, bf16_t *__restrict__ Wt, int64_t ldt) {
    __shared__ bf16_t tile[64][65];
    const int64_t r0 = int64_t(blockIdx.y) * 64, c0 = int64_t(blockIdx.x) * 64;
    for (int e = threadIdx.x; e < 64 * 64; e += 256) {
        const int rr = e / 64, cc = e % 64;
        if (r0 + rr < rows && c0 + cc < cols) tile[rr][cc] = W[(r0 + rr) * ldw + c0 + cc];
    }
    __syncthreads();
    for (int e = threadIdx.x; e < 64 * 64; e += 256) {
        const int cc = e / 64, rr = e % 64;
        if (r0 + rr < rows && c0 + cc < cols) Wt[(c0 + cc) * ldt + r0 + rr] = tile[rr][cc];
    }
}

// Y^T = X^T for a chunk of tc tokens, in the MK-token block layout; tokens tc .. ldy-1 are zero.
__global__ void __launch_bounds__(256) k_chunk_transpose(const bf16_t *__restrict__ X, int64_t ldx, int64_t tc,
                                                         int64_t d, bf16_t *__restrict__ Yt, int64_t ldy) {
    __shared__ bf16_t tile[64][65];
    const int64_t t0 = int64_t(blockIdx.y) * 64, c0 = int64_t(blockIdx.x) * 64;
    for (int e = threadIdx.x; e < 64 * 64; e += 256) {
        const int rr = e / 64, cc = e % 64;
        tile[rr][cc] = (t0 + rr < tc && c0 + cc < d) ? X[(t0 + rr) * ldx + c0 + cc] : bf16_t(0);
    }
    __syncthreads();
    for (int e = threadIdx.x; e < 64 * 64; e += 256) {
        const int cc = e / 64, rr = e % 64;
        const int64_t t = t0 + rr;
        if (c0 + cc < d && t < ldy) Yt[((t / MK) * d + c0 + cc) * MK + t % MK] = tile[rr][cc];
    }
}

// Sum of squares of one row of d bf16 values (16-byte aligned, d a multiple of 8), wave-wide:
// 16-byte loads, then a butterfly, so every lane returns the same value.
__device__ __forceinline__ float wave_row_sq(const bf16_t *__restrict__ row, int64_t d, int lane) {
    float acc = 0.f;
    for (int64_t k = int64_t(lane) * 8; k < d; k += 512) {
        const u32x4_t v = *reinterpret_cast<const u32x4_t *>(row + k);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float lo = __uint_as_float(v[q] << 16), hi = __uint_as_float(v[q] & 0xffff0000u);
            acc = fmaf(lo, lo, acc);
            acc = fmaf(hi, hi, acc);
        }
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) acc += __shfl_xor(acc, m);
    return acc;
}

constexpr int XNORM_BLOCKS = 1024;
// part[b] = max over the rows t of block b's share of ||x_t||^2 (0 for none)
__global__ void __launch_bounds__(256) k_xnorm_partial(const bf16_t *__restrict__ X, int64_t ldx, int64_t n_tok,
                                                       int64_t d, float *__restrict__ part) {
    __shared__ float sh[4];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    float m = 0.f;
    for (int64_t t = int64_t(blockIdx.x) * 4 + wave; t < n_tok; t += int64_t(gridDim.x) * 4)
        m = fmaxf(m, wave_row_sq(X + t * ldx, d, lane));
    if (lane == 0) sh[wave] = m;
    __syncthreads();
    if (threadIdx.x == 0) part[blockIdx.x] = fmaxf(fmaxf(sh[0], sh[1]), fmaxf(sh[2], sh[3]));
}

// ex[i] = 14 - q with 2^(q-1) <= b < 2^q, b = max_t ||x_t|| ||W^T_i||: |y_i(t)| 2^ex[i] < 2^14.
// 0 when b is zero or not finite (a NaN or infinity then reaches C as before).  One wave per row.
__global__ void __launch_bounds__(256) k_split_exp(const float *__restrict__ part, int npart,
                                                   const bf16_t *__restrict__ Wt, int64_t d_in, int64_t d_out,
                                                   int32_t *__restrict__ ex) {
    const int lane = threadIdx.x & 63;
    const int64_t i = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
    if (i >= d_out) return;
    float xm = 0.f;
    for (int b = lane; b < npart; b += 64) xm = fmaxf(xm, part[b]);
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) xm = fmaxf(xm, __shfl_xor(xm, m));
    const float w2 = wave_row_sq(Wt + i * d_in, d_in, lane);
    const double b = sqrt(double(xm) * double(w2));
    int e = 0;
    if (b > 0.0 && b <= 1.7e308) {
        int q;
        (void)frexp(b, &q);
        e = min(126, max(-126, 14 - q));
    }
    if (lane == 0) ex[i] = e;
}

constexpr int LOSQ_SEG = 16;  // token-block segments of k_lo_sq
// part[seg][i] = sum of lo_i(t)^2 (fp16 values, fp32 sums) over the MK-token blocks
// b = seg, seg + LOSQ_SEG, ... < nb of the chunk's Y^T lo.  A workgroup covers 64 rows, whose
// MK-token slices are one 4 KB run per block: thread t reads 16 bytes of row t / 4.
__global__ void __launch_bounds__(256) k_lo_sq(const bf16_t *__restrict__ Ylo, int64_t D, int64_t nb,
                                               float *__restrict__ part) {
    const int64_t i = int64_t(blockIdx.x) * 64 + (threadIdx.x >> 2);
    const int qd = threadIdx.x & 3;
    float acc = 0.f;
    if (i < D) {
        for (int64_t b = blockIdx.y; b < nb; b += LOSQ_SEG) {
            const u32x4_t v = *reinterpret_cast<const u32x4_t *>(Ylo + (b * D + i) * MK + qd * 8);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float lo = float(__builtin_bit_cast(_Float16, uint16_t(v[q] & 0xffffu)));
                const float hi = float(__builtin_bit_cast(_Float16, uint16_t(v[q] >> 16)));
                acc = fmaf(lo, lo, acc);
                acc = fmaf(hi, hi, acc);
            }
        }
    }
    acc += __shfl_xor(acc, 1);
    acc += __shfl_xor(acc, 2);
    if (i < D && qd == 0) part[int64_t(blockIdx.y) * D + i] = acc;
}

// C_jj += 2^-2ex[j] sum_seg part[seg][j] in segment order; the diagonal of head block h = j / hd
// is at C[j * ldc + j % hd]
__global__ void __launch_bounds__(256) k_lo_sq_add(const float *__restrict__ part, int64_t D, int64_t hd,
                                                   const int32_t *__restrict__ ex, float *__restrict__ C, int64_t ldc) {
    const int64_t j = int64_t(blockIdx.x) * 256 + threadIdx.x;
    if (j >= D) return;
    float s = 0.f;
#pragma unroll
    for (int g = 0; g < LOSQ_SEG; ++g) s += part[int64_t(g) * D + j];
    C[j * ldc + j % hd] += ldexpf(s, -2 * ex[j]);
}

// A = L^T in three bf16 pieces from the lower triangle of L (d x d fp64, ldl): row i of A is
// [hi | mid | lo] of column i of L, A[i][p d + k] = piece p of L[k][i] for k >= i and 0 for k < i
// (the strict upper triangle of L is not read).  hi = bf16(v), mid = bf16(v - hi), lo =
// bf16(v - hi - mid), each difference exact in fp64, so hi + mid + lo equals v to about 2^-26 |v|.
// 64 x 64 tiles of L transposed through LDS.
__global__ void __launch_bounds__(256) k_range_pieces(const double *__restrict__ L, int64_t ldl, int64_t d,
                                                      bf16_t *__restrict__ A) {
    __shared__ double tile[64][65];
    const int64_t k0 = int64_t(blockIdx.y) * 64, i0 = int64_t(blockIdx.x) * 64;
    for (int e = threadIdx.x; e < 64 * 64; e += 256) {
        const int kk = e / 64, ii = e % 64;
        const int64_t k = k0 + kk, i = i0 + ii;
        tile[kk][ii] = (k < d && i < d && k >= i) ? L[k * ldl + i] : 0.0;
    }
    __syncthreads();
    for (int e = threadIdx.x; e < 64 * 64; e += 256) {
        const int ii = e / 64, kk = e % 64;
        const int64_t k = k0 + kk, i = i0 + ii;
        if (k >= d || i >= d) continue;
        const double v = tile[kk][ii];
        const bf16_t hi = f32_to_bf16(float(v));
        const double r1 = v - double(bf16_to_f32(hi));
        const bf16_t mid = f32_to_bf16(float(r1));
        const double r2 = r1 - double(bf16_to_f32(mid));
        const bf16_t lo = f32_to_bf16(float(r2));
        bf16_t *row = A + i * 3 * d;
        row[k] = hi;
        row[d + k] = mid;
        row[2 * d + k] = lo;
    }
}

__global__ void k_fill_f32(float *__restrict__ p, int64_t n) {
    for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += int64_t(gridDim.x) * blockDim.x)
        p[i] = 0.f;
}

// C[upper] += P_1 + ... + P_{S-1} in split order
__global__ void k_add_partials(float *__restrict__ C, int64_t ldc, const float *__restrict__ P, int nsplit,
                               int64_t hd, int32_t n_blocks) {
    const int64_t per = hd * hd;
    const int64_t total = per * n_blocks;
    for (int64_t e = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; e < total; e += int64_t(gridDim.x) * blockDim.x) {
        const int64_t h = e / per, rr = (e % per) / hd, cc = e % hd;
        if (rr > cc) continue;
        float acc = C[h * hd * ldc + rr * ldc + cc];
        for (int s = 0; s < nsplit - 1; ++s) acc += P[int64_t(s) * total + e];
        C[h * hd * ldc + rr * ldc + cc] = acc;
    }
}

// ---------------------------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------------------------
struct MfmaPlan {
    bool wide;      // SYRK block tile 256 x 128 (4 waves of 128 x 64); else 128 x 128 (64 x 64)
    bool pair;      // SYRK with two LDS stages, two workgroups per CU (the split path's 128 x 128)
    int64_t tcmax;  // tokens per chunk
    int64_t ldy;    // leading dim of Y^T (multiple of 256)
    int nsplit;     // token splits of the SYRK
    int64_t n_upper;  // SYRK tiles per head block
};

static MfmaPlan plan(int64_t n_tok, int64_t d_out, int32_t n_blocks, bool has_w) {
    MfmaPlan p;
    const int64_t hd = d_out / n_blocks;
    // The split path (fp16 hi and lo, three products) runs 128 x 128 tiles with two LDS stages, two
    // workgroups to a CU: 21 % faster than one 256 x 128 workgroup with three stages at d_out
    // 4096, 1-4 % at 11008.  The one-product path keeps the wide tile, which moves a quarter less
    // LDS and L2 data per MFMA (below 256 rows it would be half empty).
    p.pair = has_w;
    p.wide = !has_w && hd >= 256;
    p.tcmax = std::min<int64_t>(chunk_tokens(d_out), n_tok);
    p.ldy = (p.tcmax + 255) / 256 * 256;
    p.n_upper = p.wide ? syrk_tiles<256, 128>(int(hd)) : syrk_tiles<128, 128>(int(hd));
    const int64_t tiles = p.n_upper * n_blocks;
    // smallest split count that fills >= 90% of the last wave of 256 CUs x the resident blocks
    // per CU, while keeping at least 8 k-steps per split
    const int64_t ksteps = p.ldy / MK;
    const int64_t slots = 256 * (p.pair ? 2 : 1);
    p.nsplit = 1;
    for (int s = 1; s <= 16; ++s) {
        if (s > 1 && ksteps / s < 8) break;
        const int64_t blocks = tiles * s;
        const int64_t waves = (blocks + slots - 1) / slots;
        p.nsplit = s;
        if (double(blocks) / double(waves * slots) >= 0.9) break;
    }
    return p;
}

bool cov_mfma_shape_ok(int64_t d_in, int64_t d_out, int32_t n_blocks) {
    return d_in % 8 == 0 && d_out > 0 && n_blocks > 0;
}

bool cov_mfma_supported(lrc_dtype x_t, const void *X, int64_t ldx, const void *W, int64_t ldw, int64_t d_in,
                        int64_t d_out, int32_t n_blocks) {
    (void)W;
    (void)ldw;
    // buffer-load byte offsets are 32-bit: a 256-row operand tile of X and W, and the Y^T chunk
    // (d_out x MFMA_CHUNK bf16 read through one resource, plus the two k steps loaded past its
    // end), must stay below 2^31 bytes
    return x_t == LRC_BF16 && cov_mfma_shape_ok(d_in, d_out, n_blocks) && ldx % 8 == 0 &&
           (reinterpret_cast<uintptr_t>(X) % 16) == 0 && ldx < (int64_t(1) << 21) && d_in < (int64_t(1) << 21) &&
           (d_out + 1) * (MFMA_CHUNK + 4 * MK) * 2 < (int64_t(1) << 31);
}

// The fused per-head kernel, taken with the environment variable LRC_HEAD_FUSED=1 for head blocks of
// width HF with a weight and d_in a multiple of the k step.  It is not the default: on the per-head keys
// (32768 tokens, 32 heads of 128) it took 2.21 ms against 1.42 ms for the GEMM and the SYRK through
// memory, whose 256 x 256 GEMM tiles give each wave twice the MFMAs per barrier, while Y's round trip
// through HBM costs about 0.1 ms there.
static bool head_fused(int has_w, int64_t d_in, int64_t d_out, int32_t n_blocks, int np) {
    const char *e = std::getenv("LRC_HEAD_FUSED");
    if (!(e && e[0] == '1' && e[1] == 0)) return false;
    return has_w && np == 1 && n_blocks > 1 && d_out / n_blocks == HF && d_in % MK == 0;
}
// token ranges of the fused per-head kernel: about 256 workgroups in all (one per CU), at most one per
// 128-token tile
static int head_ranges_max(int32_t n_blocks) { return std::max(1, (256 + n_blocks - 1) / n_blocks); }

// np: 1, or 3 for the range-projected product (A = L^T in three pieces)
static size_t mfma_workspace(int64_t n_tok, int64_t d_in, int has_w, int64_t d_out, int32_t n_blocks, int np) {
    const MfmaPlan p = plan(n_tok, d_out, n_blocks, has_w != 0);
    const int64_t hd = d_out / n_blocks;
    Counter c;
    if (has_w) c.carve<bf16_t>(size_t(np) * size_t(d_out) * size_t(d_in));
    c.carve<bf16_t>(size_t(d_out) * size_t(p.ldy));
    if (has_w) c.carve<bf16_t>(size_t(d_out) * size_t(p.ldy));
    c.carve<float>(size_t(p.nsplit - 1) * size_t(n_blocks) * size_t(hd) * size_t(hd) + 1);
    if (has_w) {
        c.carve<float>(XNORM_BLOCKS);
        c.carve<int32_t>(size_t(d_out));
        c.carve<float>(size_t(LOSQ_SEG) * size_t(d_out));
    }
    if (head_fused(has_w, d_in, d_out, n_blocks, np)) {
        const size_t hs = size_t(n_blocks) * size_t(head_ranges_max(n_blocks));
        c.carve<float>(hs * HF * HF);
        c.carve<float>(hs * HF);
    }
    // the generic path's buffer, used when the call's pointers are not aligned
    if (np == 1) c.carve<float>(size_t(d_out) * size_t(std::min<int64_t>(4096, n_tok)));
    return c.off;
}

size_t cov_mfma_workspace(int64_t n_tok, int64_t d_in, int has_w, int64_t d_out, int32_t n_blocks) {
    return mfma_workspace(n_tok, d_in, has_w, d_out, n_blocks, 1);
}

size_t cov_range_workspace(int64_t n_tok, int64_t d) { return mfma_workspace(n_tok, d, 1, d, 1, 3); }

lrc_status cov_mfma_run(const CovArgs &a, void *ws, size_t ws_bytes, hipStream_t s) {
    const bool rng = a.L != nullptr;  // range-projected: A = L^T in three pieces
    const bool has_w = a.W != nullptr || rng;
    const int np = rng ? 3 : 1;
    const MfmaPlan p = plan(a.n_tok, a.d_out, a.n_blocks, has_w);
    const int64_t hd = a.d_out / a.n_blocks;
    Carver cv(ws, ws_bytes);
    bf16_t *Wt = has_w ? cv.carve<bf16_t>(size_t(np) * size_t(a.d_out) * size_t(a.d_in)) : nullptr;
    bf16_t *Yhi = cv.carve<bf16_t>(size_t(a.d_out) * size_t(p.ldy));
    bf16_t *Ylo = has_w ? cv.carve<bf16_t>(size_t(a.d_out) * size_t(p.ldy)) : nullptr;
    const size_t pn = size_t(p.nsplit - 1) * size_t(a.n_blocks) * size_t(hd) * size_t(hd);
    float *P = cv.carve<float>(pn + 1);
    float *part = has_w ? cv.carve<float>(XNORM_BLOCKS) : nullptr;
    int32_t *ex = has_w ? cv.carve<int32_t>(size_t(a.d_out)) : nullptr;
    float *lpart = has_w ? cv.carve<float>(size_t(LOSQ_SEG) * size_t(a.d_out)) : nullptr;
    const bool hf = head_fused(has_w, a.d_in, a.d_out, a.n_blocks, np);
    const size_t hs = size_t(a.n_blocks) * size_t(head_ranges_max(a.n_blocks));
    float *HP = hf ? cv.carve<float>(hs * HF * HF) : nullptr;
    float *HPD = hf ? cv.carve<float>(hs * HF) : nullptr;
    if (!P || !Yhi || (has_w && (!Wt || !Ylo || !part || !ex || !lpart)) || (hf && (!HP || !HPD)))
        return fail(LRC_ERR_WORKSPACE, "covariance workspace too small");
    const bf16_t *X = static_cast<const bf16_t *>(a.X);
    if (rng) {
        dim3 g(cdiv(a.d_in, 64), cdiv(a.d_in, 64));
        hipLaunchKernelGGL(k_range_pieces, g, dim3(256), 0, s, a.L, a.ldl, a.d_in, Wt);
        LRC_LAUNCH_CHECK("k_range_pieces");
    } else if (has_w) {
        dim3 g(cdiv(a.d_out, 64), cdiv(a.d_in, 64));
        hipLaunchKernelGGL(k_transpose_bf16, g, dim3(256), 0, s, static_cast<const bf16_t *>(a.W), a.ldw, a.d_in,
                           a.d_out, Wt, a.d_in);
        LRC_LAUNCH_CHECK("k_transpose_bf16");
    }
    if (has_w) {
        // the row exponents of the fp16 split, from all tokens of the call (with pieces the row norm
        // of hi, mid and lo together, within 2^-8 of that of L's column)
        hipLaunchKernelGGL(k_xnorm_partial, dim3(XNORM_BLOCKS), dim3(256), 0, s, X, a.ldx, a.n_tok, a.d_in, part);
        LRC_LAUNCH_CHECK("k_xnorm_partial");
        hipLaunchKernelGGL(k_split_exp, dim3(unsigned(cdiv(a.d_out, 4))), dim3(256), 0, s, part, XNORM_BLOCKS, Wt,
                           np * a.d_in, a.d_out, ex);
        LRC_LAUNCH_CHECK("k_split_exp");
    }
    if (hf) {  // per-head blocks of 128: GEMM, split and SYRK in one kernel, then the range sums
        const int H = a.n_blocks;
        const int64_t tiles = (a.n_tok + HF - 1) / HF;
        const int S = int(std::min<int64_t>(tiles, head_ranges_max(H)));
        const int64_t tpr = (tiles + S - 1) / S * HF;
        const double fl = double(a.n_tok) * (2.0 * double(a.d_in) * double(a.d_out) + double(H) * HF * (HF + 1));
        LRC_TIMED_LAUNCH("k_cov_head_fused", fl, k_cov_head_fused, dim3(unsigned(H * S)), dim3(HF_THREADS), 0, s, Wt,
                         a.d_in, X, a.ldx, a.n_tok, tpr, S, ex, HP, HPD);
        LRC_LAUNCH_CHECK("k_cov_head_fused");
        hipLaunchKernelGGL(k_head_reduce, dim3(1024), dim3(256), 0, s, a.C, a.ldc, HP, HPD, S, H);
        LRC_LAUNCH_CHECK("k_head_reduce");
        return LRC_OK;
    }
    if (pn) {
        hipLaunchKernelGGL(k_fill_f32, dim3(1024), dim3(256), 0, s, P, int64_t(pn));
        LRC_LAUNCH_CHECK("k_fill_f32");
    }
    for (int64_t t0 = 0; t0 < a.n_tok; t0 += p.tcmax) {
        const int64_t tc = std::min(p.tcmax, a.n_tok - t0);
        const int64_t ktot = (tc + MK - 1) / MK * MK;
        if (rng) {
            dim3 g(unsigned(cdiv(a.d_out, G_BM)) * unsigned(cdiv(tc, G_BM)));
            // algorithmic flops of the triangular product X L: d (d + 1) per token
            const double fl = double(tc) * double(a.d_in) * double(a.d_in + 1);
            LRC_TIMED_LAUNCH("k_cov_gemm_l", fl, (k_cov_gemm_y<G_BM, false, 3>), g, dim3(G_THREADS), 0, s, Wt, a.d_in,
                             a.d_out, X + t0 * a.ldx, a.ldx, tc, ex, Yhi, Ylo);
            LRC_LAUNCH_CHECK("k_cov_gemm_l");
        } else if (has_w) {
            dim3 g(unsigned(cdiv(a.d_out, G_BM)) * unsigned(cdiv(tc, G_BM)));
            const double fl = 2.0 * double(tc) * double(a.d_in) * double(a.d_out);
            // d_in a multiple of the k step: no partial last step, no k check in the loads
            if (a.d_in % MK == 0)
                LRC_TIMED_LAUNCH("k_cov_gemm_y", fl, (k_cov_gemm_y<G_BM, false>), g, dim3(G_THREADS), 0, s, Wt,
                                 a.d_in, a.d_out, X + t0 * a.ldx, a.ldx, tc, ex, Yhi, Ylo);
            else
                LRC_TIMED_LAUNCH("k_cov_gemm_y", fl, (k_cov_gemm_y<G_BM, true>), g, dim3(G_THREADS), 0, s, Wt,
                                 a.d_in, a.d_out, X + t0 * a.ldx, a.ldx, tc, ex, Yhi, Ylo);
            LRC_LAUNCH_CHECK("k_cov_gemm_y");
        } else {
            dim3 g(cdiv(a.d_out, 64), cdiv(ktot, 64));
            hipLaunchKernelGGL(k_chunk_transpose, g, dim3(256), 0, s, X + t0 * a.ldx, a.ldx, tc, a.d_out, Yhi, p.ldy);
            LRC_LAUNCH_CHECK("k_chunk_transpose");
        }
        const int64_t kchunk = ((ktot + p.nsplit - 1) / p.nsplit + MK - 1) / MK * MK;
        dim3 g(unsigned(p.n_upper), unsigned(a.n_blocks), unsigned(p.nsplit));
        // algorithmic flops of the launch: the upper triangle (incl. diagonal) of each head block
        const double fl = double(tc) * double(hd) * double(hd + 1) * double(a.n_blocks);
        // the per-XCD order with at least 2048 tiles per token split (d_out 11008: 3741; 4096: 528)
        const int32_t xo = p.pair && p.n_upper * a.n_blocks >= 2048 ? 1 : 0;
        if (p.pair)
            LRC_TIMED_LAUNCH("k_cov_syrk", fl, (k_cov_syrk<128, 128, true, 2>), g, dim3(256), 0, s, Yhi, Ylo, ex, p.ldy,
                             ktot, kchunk, hd, a.C, a.ldc, P, a.n_blocks, xo);
        else if (p.wide)
            LRC_TIMED_LAUNCH("k_cov_syrk", fl, (k_cov_syrk<256, 128, false, 3>), g, dim3(256), 0, s, Yhi, Ylo, ex, p.ldy,
                             ktot, kchunk, hd, a.C, a.ldc, P, a.n_blocks, 0);
        else
            LRC_TIMED_LAUNCH("k_cov_syrk", fl, (k_cov_syrk<128, 128, false, 3>), g, dim3(256), 0, s, Yhi, Ylo, ex, p.ldy,
                             ktot, kchunk, hd, a.C, a.ldc, P, a.n_blocks, 0);
        LRC_LAUNCH_CHECK("k_cov_syrk");
        if (has_w) {
            hipLaunchKernelGGL(k_lo_sq, dim3(unsigned(cdiv(a.d_out, 64)), LOSQ_SEG), dim3(256), 0, s, Ylo, a.d_out,
                               ktot / MK, lpart);
            LRC_LAUNCH_CHECK("k_lo_sq");
            hipLaunchKernelGGL(k_lo_sq_add, dim3(unsigned(cdiv(a.d_out, 256))), dim3(256), 0, s, lpart, a.d_out, hd, ex,
                               a.C, a.ldc);
            LRC_LAUNCH_CHECK("k_lo_sq_add");
        }
    }
    if (p.nsplit > 1) {
        hipLaunchKernelGGL(k_add_partials, dim3(2048), dim3(256), 0, s, a.C, a.ldc, P, p.nsplit, hd, a.n_blocks);
        LRC_LAUNCH_CHECK("k_add_partials");
    }
    return LRC_OK;
}

}  // namespace lrc
