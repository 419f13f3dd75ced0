"""fp64 CPU oracle for activation-aware truncated SVD and Fisher-weighted rank allocation.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU
baseline leg of ``bench.py`` may import this package.  It shares no code with the GPU
library (``activation_aware_rank_amd``): it neither imports it nor is imported by it.
It takes stored inputs (fp32 arrays, or bf16 as raw uint16 bit patterns), widens them
exactly to fp64 with its own conversion, and computes every quantity in fp64 from its
plain definition:

O1 ``covariance``     C = sum_t y_t^T y_t for Y = X W (Swift-SVD page, section 2-ga: the
                      output covariance of Y = XW, aggregated over calibration tokens);
                      per-head diagonal blocks (WSVD page, methodology 1, per-head SVD).
O2 ``eigh``           one symmetric eigendecomposition C = V diag(lam) V^T (Swift-SVD page,
                      section 2-ga: V and Sigma^2 of Y from one eig of Y^T Y), solved by the
                      cyclic two-sided Jacobi method in ``lrco.c``; ``eigh_large`` runs the
                      same sweeps from a nearly diagonalising start basis (orders ~4096).
O3 ``truncate``       W_k = (W V_k) V_k^T with factors A = W V_k, B = V_k^T (Swift-SVD page,
                      section 2-ga, the closed-form optimum W*_k).
O4 ``error_curve``    eps_k = sum_{i>k} lam_i, k = 0..n (the closed-form minimal error eps*_k
                      of the same section), summed from the smallest term.
O5 ``direct_error``   ||X W - X W_k||_F^2, straight from its definition.
O6 ``fisher``         alpha = sum_i (G[i] W[i])^2 (FLRC page, method 1, importance alpha_{l,p}).
O7 ``allocate_ranks`` greedy global allocation by importance per parameter (LASER page,
                      method 2, "global optimisation"), with per-matrix Fisher weights;
                      ``allocate_proportional`` (FLRC page, methods 1-2), ``swift_scores`` /
                      ``swift_allocate`` (Swift-SVD page, section 2-na), ``component_fisher`` /
                      ``allocate_components`` (LASER page, method 2, per-component score).
O8 ``kfac_*``         LASER page, method 1: covariances of activations and gradients,
                      Cholesky factors, whitened W~ = L_x^T W L_g, its SVD from the eig of
                      W~ W~^T, factors mapped back; ``cholesky``, ``tri_product`` and
                      ``tri_solve`` are its dense steps on their own.

Readings of points the pages leave open (each one stated where it is used):
* C is unnormalised (a sum over tokens), so eps_k = ||XW - XW_k||_F^2 exactly.
* Eigenvalues descending, ties stable by position; each eigenvector's entry of largest
  magnitude is positive (first index on ties).
* Allocation priority p_{m,k} = w_m * max(lam_{m,k}, 0), w_m = alpha_m / (eps_{m,0} * cost_m)
  with cost_m = d_in + d_out; total order (p desc, m asc, k asc); candidates k_min+1..K_m;
  scan in order and stop at the first item that does not fit the budget.

parity pinned: every function here is checked in ``tests/test_oracle_*.py`` against closed
forms, invariants, brute force on tiny inputs or LAPACK, none of which share its code.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "liblrco.so")
_SRC = os.path.join(_HERE, "lrco.c")
_lib = None


def build(force: bool = False) -> str:
    """Compile lrco.c with gcc (OpenMP, no FMA contraction) into liblrco.so."""
    if force or not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
        tmp = _SO + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-shared", "-fPIC",
                               _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _SO)
    return _SO


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_SO)
        dp = ctypes.POINTER(ctypes.c_double)
        lib.lrco_jacobi_eigh.argtypes = [ctypes.c_int, dp, dp, dp, ctypes.c_int, ctypes.POINTER(ctypes.c_int)]
        lib.lrco_jacobi_eigh.restype = ctypes.c_int
        lib.lrco_cholesky.argtypes = [ctypes.c_int, dp]
        lib.lrco_cholesky.restype = ctypes.c_int
        _lib = lib
    return _lib


def _dp(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


class OracleError(RuntimeError):
    pass


# ----------------------------------------------------------------------------------------------
# exact widening of stored inputs (the oracle's own conversion)
# ----------------------------------------------------------------------------------------------

def widen(a: np.ndarray, dtype: str) -> np.ndarray:
    """Stored array -> fp64.  'bf16' arrays are uint16 bit patterns: value = bits << 16 as fp32."""
    if dtype == "bf16":
        u = np.asarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return u.view(np.float32).astype(np.float64)
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    if dtype == "f64":
        return np.asarray(a, dtype=np.float64)
    raise ValueError(dtype)


# ----------------------------------------------------------------------------------------------
# O1 covariance
# ----------------------------------------------------------------------------------------------

def covariance(X: np.ndarray, x_dtype: str, W: np.ndarray | None = None, w_dtype: str = "f64",
               n_blocks: int = 1, chunk_rows: int = 8192) -> np.ndarray:
    """C = sum_t y_t^T y_t with y_t = x_t W, in fp64 (W None: W = I).

    Swift-SVD page, section 2-ga: the covariance of Y = XW is aggregated over the calibration
    tokens, then eigendecomposed once.  Unnormalised sum (a reading: the pages do not say).
    Streams over row chunks; the sum is order-insensitive to fp64 rounding level.
    n_blocks > 1: only the n_blocks diagonal blocks of width d_out/n_blocks (per-head case,
    WSVD page, methodology 1) are returned, as an array (n_blocks, hd, hd).
    """
    n_tok = X.shape[0]
    W64 = None if W is None else widen(W, w_dtype)
    d_out = X.shape[1] if W64 is None else W64.shape[1]
    if d_out % n_blocks:
        raise ValueError("d_out not divisible by n_blocks")
    hd = d_out // n_blocks
    C = np.zeros((n_blocks, hd, hd)) if n_blocks > 1 else np.zeros((d_out, d_out))
    for r0 in range(0, n_tok, chunk_rows):
        Xc = widen(X[r0:r0 + chunk_rows], x_dtype)
        Y = Xc if W64 is None else Xc @ W64
        if n_blocks == 1:
            C += Y.T @ Y
        else:
            for h in range(n_blocks):
                Yh = Y[:, h * hd:(h + 1) * hd]
                C[h] += Yh.T @ Yh
    return C


def covariance_entries(X: np.ndarray, x_dtype: str, W: np.ndarray, w_dtype: str, rows, cols,
                       chunk_rows: int = 8192) -> np.ndarray:
    """Selected entries C[rows[i], cols[i]] = sum_t y_ti y_tj, each from its own columns of Y.

    Used at full size, where the whole C is too costly on the CPU.
    """
    rows = np.asarray(rows)
    cols = np.asarray(cols)
    need = np.unique(np.concatenate([rows, cols]))
    pos = {int(c): i for i, c in enumerate(need)}
    W64 = widen(W, w_dtype)[:, need]
    acc = np.zeros(len(rows))
    ri = np.array([pos[int(r)] for r in rows])
    ci = np.array([pos[int(c)] for c in cols])
    for r0 in range(0, X.shape[0], chunk_rows):
        Y = widen(X[r0:r0 + chunk_rows], x_dtype) @ W64
        acc += np.einsum("ti,ti->i", Y[:, ri], Y[:, ci])
    return acc


# ----------------------------------------------------------------------------------------------
# O2 eigendecomposition
# ----------------------------------------------------------------------------------------------

def eigh(C: np.ndarray, max_sweeps: int = 60) -> tuple[np.ndarray, np.ndarray]:
    """Eigenpairs of a symmetric matrix by cyclic Jacobi (lrco.c), descending, signs fixed.

    Swift-SVD page, section 2-ga: V (right singular vectors of Y) and Sigma^2 from one
    eigendecomposition of Y^T Y.
    """
    C = np.asarray(C, dtype=np.float64)
    n = C.shape[0]
    if C.shape != (n, n):
        raise ValueError("square matrix expected")
    A = np.ascontiguousarray((C + C.T) * 0.5) if not np.array_equal(C, C.T) else np.array(C, order="C")
    lam = np.empty(n)
    V = np.empty((n, n))
    sweeps = ctypes.c_int(0)
    rc = _load().lrco_jacobi_eigh(n, _dp(A), _dp(lam), _dp(V), max_sweeps, ctypes.byref(sweeps))
    if rc != 0:
        raise OracleError("Jacobi did not converge in %d sweeps" % max_sweeps)
    return lam, V


def eigh_from_basis(C: np.ndarray, Q: np.ndarray, max_sweeps: int = 60) -> tuple[np.ndarray, np.ndarray]:
    """Eigenpairs of C by the same cyclic Jacobi, started from an orthogonal basis Q.

    The sweeps run on B = Q^T C Q (formed in fp64) and stop under the same relative threshold
    as ``eigh``; then C = (Q V_B) diag(lam) (Q V_B)^T.  Q only changes how many sweeps are
    needed: whatever basis it is, the result is certified by the sweeps, which leave every
    off-diagonal entry of the rotated B below 2^-52 of its diagonal scale.  Q must be
    orthogonal to fp64 rounding.  Descending order and signs as in ``eigh``.
    """
    C = np.ascontiguousarray(C, dtype=np.float64)
    Q = np.ascontiguousarray(Q, dtype=np.float64)  # strided views would leave the BLAS path
    n = C.shape[0]
    if C.shape != (n, n) or Q.shape != (n, n):
        raise ValueError("square matrices of one order expected")
    Cs = (C + C.T) * 0.5
    B = Q.T @ Cs @ Q
    B = np.ascontiguousarray((B + B.T) * 0.5)
    lam = np.empty(n)
    VB = np.empty((n, n))
    sweeps = ctypes.c_int(0)
    rc = _load().lrco_jacobi_eigh(n, _dp(B), _dp(lam), _dp(VB), max_sweeps, ctypes.byref(sweeps))
    if rc != 0:
        raise OracleError("Jacobi did not converge in %d sweeps" % max_sweeps)
    V = Q @ VB
    # the sign rule of eigh, applied after the change of basis
    idx = np.argmax(np.abs(V), axis=0)
    V *= np.where(V[idx, np.arange(n)] < 0, -1.0, 1.0)[None, :]
    return lam, V


def eigh_large(C: np.ndarray, max_sweeps: int = 60) -> tuple[np.ndarray, np.ndarray]:
    """``eigh`` for orders in the thousands, where sweeps from the identity take minutes on a host.

    The cyclic Jacobi starts from the eigenvectors that LAPACK's symmetric eigensolver
    (numpy.linalg.eigh, a test-only library step) gives for C, so that one sweep does the
    remaining rotations and the next one confirms convergence (``eigh_from_basis``).  The answer
    rests on the Jacobi sweeps' stopping rule, not on the library's accuracy.
    """
    C = np.asarray(C, dtype=np.float64)
    _, Q = np.linalg.eigh((C + C.T) * 0.5)
    return eigh_from_basis(C, Q[:, ::-1], max_sweeps)


def eigh_upper(C_upper: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """eigh of the symmetric matrix whose upper triangle (incl. diagonal) is given."""
    U = np.triu(np.asarray(C_upper, dtype=np.float64))
    return eigh(U + np.triu(U, 1).T)


# ----------------------------------------------------------------------------------------------
# O3-O5 truncation and error
# ----------------------------------------------------------------------------------------------

def truncate(W64: np.ndarray, V: np.ndarray, k: int) -> tuple[np.ndarray, np.ndarray]:
    """Factors of the closed-form optimum W_k = (W V_k) V_k^T: A = W V_k, B = V_k^T.

    Swift-SVD page, section 2-ga (the closed-form W*_k).
    """
    Vk = V[:, :k]
    return W64 @ Vk, Vk.T.copy()


def error_curve(lam: np.ndarray) -> np.ndarray:
    """eps_k = sum_{i>k} lam_i for k = 0..n (eps_n = 0), summed from the smallest term.

    Swift-SVD page, section 2-ga (the closed-form minimal error eps*_k).
    """
    lam = np.asarray(lam, dtype=np.float64)
    n = lam.shape[-1]
    eps = np.zeros(lam.shape[:-1] + (n + 1,))
    for k in range(n - 1, -1, -1):
        eps[..., k] = eps[..., k + 1] + lam[..., k]
    return eps


def direct_error(X: np.ndarray, x_dtype: str, W64: np.ndarray, Wk64: np.ndarray,
                 chunk_rows: int = 8192) -> float:
    """||X W - X W_k||_F^2 in fp64, from its definition."""
    D = W64 - Wk64
    tot = 0.0
    for r0 in range(0, X.shape[0], chunk_rows):
        R = widen(X[r0:r0 + chunk_rows], x_dtype) @ D
        tot += float(np.sum(R * R))
    return tot


# ----------------------------------------------------------------------------------------------
# O6 Fisher importance
# ----------------------------------------------------------------------------------------------

def fisher(G: np.ndarray, W: np.ndarray, dtype: str = "bf16") -> float:
    """alpha = sum_i (G[i] * W[i])^2 in fp64 (FLRC page, method 1, importance alpha_{l,p})."""
    g = widen(G, dtype).ravel()
    w = widen(W, dtype).ravel()
    prod = g * w
    return float(np.sum(prod * prod))


# ----------------------------------------------------------------------------------------------
# O7 greedy allocation
# ----------------------------------------------------------------------------------------------

def allocation_priorities(alpha, lams, eps0, cost, k_min):
    """Candidate list: (p, m, k) for k = k_min_m+1 .. K_m, K_m = len(lams[m]).

    p_{m,k} = w_m * max(lam_{m,k}, 0) with w_m = alpha_m / (eps0_m * cost_m), w_m = 0 when
    eps0_m == 0; each operation a single IEEE fp64 multiply or divide.
    """
    M = len(lams)
    p_all, m_all, k_all = [], [], []
    for m in range(M):
        t = np.float64(eps0[m]) * np.float64(cost[m])
        w = np.float64(alpha[m]) / t if eps0[m] != 0 else np.float64(0.0)
        lam = np.asarray(lams[m], dtype=np.float64)
        ks = np.arange(int(k_min[m]) + 1, lam.shape[0] + 1)
        p = w * np.maximum(lam[ks - 1], 0.0)
        p_all.append(p)
        m_all.append(np.full(ks.shape, m, dtype=np.int64))
        k_all.append(ks.astype(np.int64))
    return np.concatenate(p_all), np.concatenate(m_all), np.concatenate(k_all)


def allocate_proportional(alpha, budgets) -> tuple[np.ndarray, int]:
    """Ranks in proportion to the Fisher importance, for one or several rank budgets.

    FLRC page, method 1: r_m = round(alpha_m / S * R) with S the sum of the alpha_m and R the total
    rank budget; method 2 evaluates the same rule for a non-increasing budget R(t) per decoding
    step.  Readings (the page fixes neither): round half away from zero, then the sum is brought to
    exactly R by largest remainders -- while it is short, the matrix with the largest q_m - r_m
    (ties: smaller m) gains one; while it is over, the matrix with r_m > 0 and the smallest
    q_m - r_m (ties: smaller m) loses one -- with q_m = (alpha_m * R) / S in fp64 and S summed in
    index order.  Returns (r, info): r has one row per budget; info 5 when an alpha is negative or
    NaN or S is not positive and finite, or a budget is negative (r is then all zero).
    """
    a = np.asarray(alpha, dtype=np.float64)
    B = [int(b) for b in budgets]
    r = np.zeros((len(B), len(a)), dtype=np.int64)
    S = 0.0
    for v in a:  # index order
        S = S + float(v)
    if np.any(~(a >= 0)) or not (0 < S < np.inf) or any(b < 0 for b in B):
        return r, 5
    for t, R in enumerate(B):
        q = [(float(a[m]) * float(R)) / S for m in range(len(a))]
        rt = [int(np.floor(x + 0.5)) for x in q]  # half away from zero (q >= 0)
        d = R - sum(rt)
        while d > 0:
            m = max(range(len(a)), key=lambda i: (q[i] - rt[i], -i))
            rt[m] += 1
            d -= 1
        while d < 0:
            cand = [i for i in range(len(a)) if rt[i] > 0]
            m = min(cand, key=lambda i: (q[i] - rt[i], i))
            rt[m] -= 1
            d += 1
        r[t] = rt
    return r, 0


def allocate_ranks(alpha, lams, eps0, cost, budget: int, k_min=None) -> tuple[np.ndarray, int]:
    """Greedy global rank allocation under a parameter budget.

    LASER page, method 2 ("global optimisation"): pick the singular components with the
    highest importance per parameter cost until the parameter budget is reached; FLRC page,
    method 1: per-projection Fisher importance alpha.  The Swift-SVD page, section 2-na,
    guarantees a minimum rank per layer (k_min here).

    Sort the candidates by (p desc, m asc, k asc), subtract the mandatory sum k_min_m cost_m
    from the budget, take items in order while they fit and stop at the first that does not.
    Returns (k per matrix, info) with info 4 when the mandatory ranks exceed the budget and
    5 when an alpha or eps0 is negative or NaN, a weight is not finite, a cost is not positive,
    an eigenvalue is NaN or a minimum rank is outside [0, K_m].
    """
    M = len(lams)
    k_min = np.zeros(M, dtype=np.int64) if k_min is None else np.asarray(k_min, dtype=np.int64)
    cost = np.asarray(cost, dtype=np.int64)
    alpha = np.asarray(alpha, dtype=np.float64)
    eps0 = np.asarray(eps0, dtype=np.float64)
    # a score that is not a non-negative number makes the order undefined: info 5
    with np.errstate(all="ignore"):
        w = np.where(eps0 != 0, alpha / (eps0 * cost.astype(np.float64)), 0.0)
    bad = (np.any(~(alpha >= 0)) or np.any(~(eps0 >= 0)) or np.any(cost <= 0) or np.any(~np.isfinite(w))
           or any(np.any(np.isnan(np.asarray(l, dtype=np.float64))) for l in lams)
           or np.any(k_min < 0) or any(int(k_min[m]) > len(lams[m]) for m in range(M)))
    if bad:
        return k_min.copy(), 5
    mandatory = int(np.sum(k_min * cost))
    if mandatory > budget:
        return k_min.copy(), 4
    p, m, k = allocation_priorities(alpha, lams, eps0, cost, k_min)
    order = np.lexsort((k, m, -p))
    rem = int(budget) - mandatory
    kout = k_min.copy()
    for idx in order:
        c = int(cost[m[idx]])
        if c > rem:
            break
        rem -= c
        kout[m[idx]] += 1
    return kout, 0


def swift_scores(beta, eps_kbar, alpha: float) -> np.ndarray:
    """Allocation scores of the Swift-SVD page, section 2-na (strategy, step 1).

    s_i = beta_i^alpha * log(e + eps_{kbar,i})^(1 - alpha): beta_i the importance of matrix i and
    eps_{kbar,i} its closed-form error at the uniform rank kbar_i.  Readings: beta is the Fisher
    importance of the FLRC page (the only importance this path computes; any non-negative
    importance can be passed), eps is the absolute closed-form error eps*_k (negative rounding
    residue counts as 0).  log(e + eps) >= 1, so s_i > 0 whenever beta_i > 0.  fp64 with the host
    C library's pow and log.
    """
    b = np.asarray(beta, dtype=np.float64)
    e = np.asarray(eps_kbar, dtype=np.float64)
    out = np.empty(b.shape[0])
    for i in range(b.shape[0]):
        x = float(e[i])
        L = math.log(math.e + (x if (math.isnan(x) or x > 0.0) else 0.0))  # NaN stays NaN
        out[i] = math.pow(float(b[i]), alpha) * math.pow(L, 1.0 - alpha)
    return out


def swift_allocate(scores, kbar, cost, k_cap, delta: float, budget: int) -> tuple[np.ndarray, int]:
    """Ranks from Swift-SVD scores under a parameter budget (Swift-SVD page, section 2-na, steps 1-2).

    Step 2 guarantees every matrix the minimum rank floor(kbar_i * delta) (the retained ratio delta of
    the uniform rank kbar_i).  Reading of step 1 (the page gives the score, not the rule that turns it
    into ranks): the parameters left after the minima, E = budget - sum kmin_i cost_i, go to the
    matrices in proportion to their scores, rank = floor(share / cost_i), no rank above k_cap_i; a
    matrix that reaches k_cap_i keeps it and the rest is split again among the others (water
    filling).  Each split takes S = sum of the scores of the matrices still open (index order) and
    R = the parameters not yet committed, and gives matrix i floor(((s_i * R) / S) / cost_i) more
    ranks (fp64, one operation at a time).  Should rounding ever overshoot the budget, the open
    matrix of highest index with an extra rank gives one back, until the total fits.
    Returns (k, info): info 4 when the minima exceed the budget (k = minima), 5 for a negative,
    NaN or infinite score, a kbar outside [0, k_cap], a cost <= 0 or delta outside [0, 1] (k = zeros).
    """
    s = [float(x) for x in scores]
    kbar = [int(x) for x in kbar]
    cost = [int(x) for x in cost]
    k_cap = [int(x) for x in k_cap]
    M = len(s)
    if (not (0.0 <= delta <= 1.0) or any(not (0.0 <= x < math.inf) for x in s) or any(c <= 0 for c in cost)
            or any(kbar[i] < 0 or kbar[i] > k_cap[i] for i in range(M))):
        return np.zeros(M, dtype=np.int64), 5
    kmin = [int(math.floor(float(kbar[i]) * delta)) for i in range(M)]
    mand = sum(kmin[i] * cost[i] for i in range(M))
    if mand > budget:
        return np.array(kmin, dtype=np.int64), 4
    E = int(budget) - mand
    x = [0] * M
    open_ = [i for i in range(M) if kmin[i] < k_cap[i]]
    committed = 0
    while open_:
        S = 0.0
        for i in open_:
            S = S + s[i]
        if not S > 0.0:
            break
        R = float(E - committed)
        q = {i: int(math.floor(((s[i] * R) / S) / float(cost[i]))) for i in open_}
        capped = [i for i in open_ if kmin[i] + q[i] >= k_cap[i]]
        if not capped:
            for i in open_:
                x[i] = q[i]
            break
        for i in capped:
            x[i] = k_cap[i] - kmin[i]
            committed += x[i] * cost[i]
        open_ = [i for i in open_ if i not in capped]
    total = sum((kmin[i] + x[i]) * cost[i] for i in range(M))
    while total > budget:
        i = max(j for j in open_ if x[j] > 0)
        x[i] -= 1
        total -= cost[i]
    return np.array([kmin[i] + x[i] for i in range(M)], dtype=np.int64), 0


def component_fisher(W64: np.ndarray, G64: np.ndarray, V: np.ndarray, k: int) -> np.ndarray:
    """Empirical-Fisher importance of each retained component (LASER page, method 2).

    Removing component i of the truncation changes W by dW_i = W v_i v_i^T.  Reading (the page
    describes the score, it does not print it): with the calibration gradient G of the same shape
    as W, the empirical-Fisher quadratic loss of that change is <G, dW_i>^2 = (v_i^T W^T G v_i)^2,
    which grows with the component's magnitude W v_i and its alignment with the gradient.  Computed
    as the diagonal of V_k^T (W^T G) V_k in fp64.
    """
    Vk = np.asarray(V, dtype=np.float64)[:, :k]
    M = W64.T @ G64
    d = np.einsum("ri,ri->i", Vk, M @ Vk)
    return d * d


def allocate_components(scores, cost, budget: int, k_min=None) -> tuple[np.ndarray, list, int]:
    """Greedy selection of single components by importance per parameter (LASER page, method 2).

    Candidates are the components i = k_min_m+1 .. K_m of every matrix m (K_m = len(scores[m]));
    the first k_min_m components of m (largest eigenvalues) are kept and charged first.  Priority
    p = s_{m,i} / cost_m (one IEEE fp64 division); candidates are taken in (p desc, m asc, i asc)
    order while they fit and the first that does not ends the scan.  The taken components of a
    matrix need not be its leading ones: the result is k_m and, per matrix, the mask of kept
    components.  Returns (k, masks, info): info 4 when the minima exceed the budget, 5 for a
    negative or NaN score, a cost <= 0 or a k_min outside [0, K_m].
    """
    M = len(scores)
    sc = [np.asarray(x, dtype=np.float64) for x in scores]
    k_min = [0] * M if k_min is None else [int(v) for v in k_min]
    cost = [int(c) for c in cost]
    masks = [np.zeros(len(x), dtype=bool) for x in sc]
    if (any(np.any(~(x >= 0.0)) for x in sc) or any(c <= 0 for c in cost)
            or any(k_min[m] < 0 or k_min[m] > len(sc[m]) for m in range(M))):
        return np.array(k_min, dtype=np.int64), masks, 5
    for m in range(M):
        masks[m][:k_min[m]] = True
    rem = int(budget) - sum(k_min[m] * cost[m] for m in range(M))
    if rem < 0:
        return np.array(k_min, dtype=np.int64), masks, 4
    p, mm, ii = [], [], []
    for m in range(M):
        idx = np.arange(k_min[m], len(sc[m]))
        p.append(sc[m][idx] / np.float64(cost[m]))
        mm.append(np.full(idx.shape, m, dtype=np.int64))
        ii.append(idx.astype(np.int64))
    p, mm, ii = np.concatenate(p), np.concatenate(mm), np.concatenate(ii)
    order = np.lexsort((ii, mm, -p))
    k = list(k_min)
    for j in order:
        c = cost[mm[j]]
        if c > rem:
            break
        rem -= c
        k[mm[j]] += 1
        masks[mm[j]][ii[j]] = True
    return np.array(k, dtype=np.int64), masks, 0


# ----------------------------------------------------------------------------------------------
# O8 curvature-weighted (K-FAC) variant
# ----------------------------------------------------------------------------------------------

def cholesky(S: np.ndarray) -> np.ndarray:
    """Lower Cholesky factor L, S = L L^T (lrco.c, column by column)."""
    A = np.array(S, dtype=np.float64, order="C")
    rc = _load().lrco_cholesky(A.shape[0], _dp(A))
    if rc != 0:
        raise OracleError("matrix not positive definite (pivot %d)" % rc)
    return A


def solve_lower(L: np.ndarray, B: np.ndarray) -> np.ndarray:
    """L^{-1} B by forward substitution, row by row."""
    n = L.shape[0]
    X = np.array(B, dtype=np.float64)
    for i in range(n):
        if i:
            X[i] -= L[i, :i] @ X[:i]
        X[i] /= L[i, i]
    return X


def solve_lower_t(L: np.ndarray, B: np.ndarray) -> np.ndarray:
    """L^{-T} B by back substitution, row by row."""
    n = L.shape[0]
    X = np.array(B, dtype=np.float64)
    for i in range(n - 1, -1, -1):
        if i < n - 1:
            X[i] -= L[i + 1:, i] @ X[i + 1:]
        X[i] /= L[i, i]
    return X


def tri_product(side: int, trans: int, L: np.ndarray, B: np.ndarray) -> np.ndarray:
    """op(L) B (side 0) or B op(L) (side 1), op(L) = L or L^T with L's lower triangle only
    (the products of the curvature transform W~ = L_x^T W L_g, LASER page, method 1)."""
    Lt = np.tril(np.asarray(L, dtype=np.float64))
    op = Lt.T if trans else Lt
    B = np.asarray(B, dtype=np.float64)
    return op @ B if side == 0 else B @ op


def tri_solve(side: int, trans: int, L: np.ndarray, B: np.ndarray) -> np.ndarray:
    """op(L)^{-1} B (side 0) or B op(L)^{-1} (side 1) by substitution with L's lower triangle
    (the map back A = L_x^{-T} U_k of LASER page, method 1).  Side 1 goes through the
    transpose: B L^{-1} = (L^{-T} B^T)^T and B L^{-T} = (L^{-1} B^T)^T."""
    B = np.asarray(B, dtype=np.float64)
    if side == 0:
        return solve_lower_t(L, B) if trans else solve_lower(L, B)
    return (solve_lower(L, B.T) if trans else solve_lower_t(L, B.T)).T


def kfac_compress(Sx: np.ndarray, Sg: np.ndarray, W64: np.ndarray, k: int) -> dict:
    """Curvature-weighted truncation (LASER page, method 1).

    Loss increase ~ 1/2 vec(dW)^T (G (x) X) vec(dW) with X, G the activation and gradient
    covariances.  Reading of the transform: lower Cholesky Sx = Lx Lx^T, Sg = Lg Lg^T and
    W~ = Lx^T W Lg, so ||Lx^T dW Lg||_F^2 = vec(dW)^T (Sg (x) Sx) vec(dW) for Y = XW.
    SVD of W~ through the eig of M = W~ W~^T (d_in x d_in): W~ = U S V^T.  Mapped back:
    A = Lx^{-T} U_k S_k,  B = V_k^T Lg^{-1} = S_k^{-1} U_k^T Lx^T W, so W_k = A B.
    """
    Lx = cholesky(Sx)
    Lg = cholesky(Sg)
    Wt = Lx.T @ W64 @ Lg
    lam, U = eigh(Wt @ Wt.T)
    sig = np.sqrt(np.maximum(lam, 0.0))
    Uk = U[:, :k]
    sk = sig[:k]
    A = solve_lower_t(Lx, Uk * sk)
    B = (Uk.T @ (Lx.T @ W64)) / sk[:, None]
    return {"Lx": Lx, "Lg": Lg, "Wt": Wt, "lam": lam, "U": U, "A": A, "B": B}
