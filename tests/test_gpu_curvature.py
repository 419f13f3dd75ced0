"""Parity of the curvature-weighted chain (LASER page, method 1) on the GPU against the fp64 oracle:
the fp64 Cholesky factor, the triangular products and solves, the conversions and the Gram
matrix on their own, then the whole chain X, G, W -> Sigma_x, Sigma_g -> L_x, L_g -> W~ -> eig of
W~ W~^T -> A, B on one seeded cfg-5-shaped layer at reduced size.

Tolerances, from the arithmetic:
* Cholesky (backward stable): |L - L_o|_ij <= 1e-11 sqrt(S_ii) on matrices whose correlation part
  has condition number about 34 (rows scaled by lognormal channel scales).
* Triangular product: |X - X_o| <= dim 2^-52 (|L| |B|) elementwise (fp64 dot products).
* Triangular solve: max |X - X_o| <= 1e-12 max |X_o| for well-conditioned factors; Frobenius
  1e-10 with lognormal row scales (the blocked solve multiplies by inverted 64x64 blocks).
* Conversions: bit-exact.  Gram: fp64 sums rounded once to fp32, so within one fp32 rounding.
* Chain: eigenvalues of W~ W~^T within 1e-5 lambda_max, retained subspace within 1e-3 rad, the
  closed form ||L_x^T (W - W_k) L_g||_F^2 = sum of the discarded eigenvalues within 1e-4 of the
  tail (GPU quantities only); W_k within 1e-4 relative (Frobenius) as a diagnostic.
"""
import numpy as np
import pytest
import torch

import oracle
from activation_aware_rank_amd import inputs
from parity_utils import check_lambda, dev, gap, host, sin_theta_max

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lrc():
    from activation_aware_rank_amd import lrc as m
    return m


def _say(msg):
    print("\n[case] " + msg, flush=True)


def _spd(n, seed, scaled=True):
    """Input recipe: S = Z^T Z / m, Z m x n Gaussian (m = 2n + 8), optionally D S D with lognormal
    channel scales D -- the shape of an activation covariance."""
    m = 2 * n + 8
    Z = inputs.as_f64(inputs.gaussian(m, n, 1.0, "f32", inputs.CFG_KFAC, 1, seed, inputs.S_ACT), "f32")
    S = Z.T @ Z / m
    if scaled:
        d = inputs.channel_scales_lognormal(n, inputs.CFG_KFAC, 1, seed)
        S = S * d[:, None] * d[None, :]
    return S


def _gauss64(rows, cols, seed):
    return inputs.as_f64(inputs.gaussian(rows, cols, 1.0, "f32", inputs.CFG_KFAC, 2, seed, inputs.S_ACT), "f32")


# ---------------------------------------------------------------------------------------------
# Cholesky
# ---------------------------------------------------------------------------------------------

@pytest.mark.parametrize("n", [1, 63, 64, 65, 200, 333])
def test_cholesky_parity(lrc, n):
    _say("cholesky n=%d lda=n+5, strict upper NaN" % n)
    S = _spd(n, 10 + n)
    A = np.full((n, n + 5), np.nan)
    A[:, :n] = np.where(np.tri(n, dtype=bool), S, np.nan)
    Ad = dev(A, "f64")
    _, info = lrc.lrc_cholesky(Ad[:, :n])
    L = host(Ad)
    assert int(host(info)[0]) == 0
    assert np.all(np.isnan(L[:, n:])), "columns beyond n were written"
    L = L[:, :n]
    assert np.all(L[np.triu_indices(n, 1)] == 0.0)
    Lo = oracle.cholesky(S)
    err = np.max(np.abs(L - Lo) / np.sqrt(np.diag(S))[:, None])
    assert err <= 1e-11, "Cholesky error %.3e" % err


def test_cholesky_not_positive_definite(lrc):
    _say("cholesky info codes")
    S = _spd(150, 7, scaled=False)
    S[100, 100] = -1.0
    _, info = lrc.lrc_cholesky(dev(S, "f64"))
    assert int(host(info)[0]) == 3
    S = _spd(90, 8, scaled=False)
    S[0, 0] = np.nan
    _, info = lrc.lrc_cholesky(dev(S, "f64"))
    assert int(host(info)[0]) == 1
    # a good call after a failed one reports 0 again
    _, info = lrc.lrc_cholesky(dev(_spd(90, 8, scaled=False), "f64"), info=info)
    assert int(host(info)[0]) == 0


# ---------------------------------------------------------------------------------------------
# triangular product and solve
# ---------------------------------------------------------------------------------------------

def _lower_with_nan_upper(n, seed, scaled):
    L = oracle.cholesky(_spd(n, seed, scaled))
    Lg = L.copy()
    Lg[np.triu_indices(n, 1)] = np.nan
    return L, Lg


@pytest.mark.parametrize("side,trans", [(0, 0), (0, 1), (1, 0), (1, 1)])
def test_trmm_parity(lrc, side, trans):
    m, n = 130, 77
    dim = m if side == 0 else n
    _say("trmm side=%d trans=%d m=%d n=%d" % (side, trans, m, n))
    L, Lnan = _lower_with_nan_upper(dim, 20 + dim, True)
    B = _gauss64(m, n, 30 + 2 * side + trans)
    Bd = dev(B, "f64")
    lrc.lrc_trmm(side, trans, dev(Lnan, "f64"), Bd)
    X = host(Bd)
    Xo = oracle.tri_product(side, trans, L, B)
    bound = dim * 2.0 ** -52 * oracle.tri_product(side, trans, np.abs(L), np.abs(B))
    assert np.all(np.abs(X - Xo) <= bound + 1e-300), "trmm max excess %.3e" % np.max(np.abs(X - Xo) - bound)


@pytest.mark.parametrize("side,trans", [(0, 0), (0, 1), (1, 0), (1, 1)])
@pytest.mark.parametrize("scaled", [False, True])
def test_trsm_parity(lrc, side, trans, scaled):
    m, n = (200, 70) if side == 0 else (70, 200)
    dim = m if side == 0 else n
    _say("trsm side=%d trans=%d m=%d n=%d scaled=%d" % (side, trans, m, n, scaled))
    L, Lnan = _lower_with_nan_upper(dim, 40 + dim, scaled)
    B = _gauss64(m, n, 50 + 2 * side + trans)
    Bd = dev(B, "f64")
    lrc.lrc_trsm(side, trans, dev(Lnan, "f64"), Bd)
    X = host(Bd)
    Xo = oracle.tri_solve(side, trans, L, B)
    if scaled:
        err = np.linalg.norm(X - Xo) / np.linalg.norm(Xo)
        assert err <= 1e-10, "trsm Frobenius error %.3e" % err
    else:
        err = np.max(np.abs(X - Xo)) / np.max(np.abs(Xo))
        assert err <= 1e-12, "trsm error %.3e" % err


@pytest.mark.parametrize("side,trans", [(0, 0), (0, 1), (1, 0), (1, 1)])
def test_trsm_wide_parity(lrc, side, trans):
    """B with at least 128 tiles of 64 across one block (8200 wide): the solve takes the
    left-looking order (one product per block with every block solved before it, its k range split
    in up to 4 parts here, 1088 deep at the last block)."""
    m, n = (1100, 8200) if side == 0 else (8200, 1100)
    dim = m if side == 0 else n
    _say("trsm wide side=%d trans=%d m=%d n=%d" % (side, trans, m, n))
    L, Lnan = _lower_with_nan_upper(dim, 70 + 2 * side + trans, False)
    B = _gauss64(m, n, 80 + 2 * side + trans)
    Bd = dev(B, "f64")
    lrc.lrc_trsm(side, trans, dev(Lnan, "f64"), Bd)
    X = host(Bd)
    Xo = oracle.tri_solve(side, trans, L, B)
    err = np.max(np.abs(X - Xo)) / np.max(np.abs(Xo))
    assert err <= 1e-12, "trsm error %.3e" % err


def test_trsm_strided_and_single_row(lrc):
    _say("trsm ldb > n, m = 1; trmm on a column slice")
    L, Lnan = _lower_with_nan_upper(1, 61, False)
    B = np.full((1, 9), 3.0)
    Bd = dev(B, "f64")
    lrc.lrc_trsm(0, 0, dev(Lnan, "f64"), Bd)
    assert np.allclose(host(Bd), 3.0 / L[0, 0], rtol=1e-15)
    L, Lnan = _lower_with_nan_upper(96, 62, False)
    big = np.full((96, 50), np.nan)
    B = _gauss64(96, 40, 63)
    big[:, 5:45] = B
    Bd = dev(big, "f64")
    lrc.lrc_trsm(0, 1, dev(Lnan, "f64"), Bd[:, 5:45])
    out = host(Bd)
    assert np.all(np.isnan(out[:, :5])) and np.all(np.isnan(out[:, 45:]))
    Xo = oracle.tri_solve(0, 1, L, B)
    assert np.max(np.abs(out[:, 5:45] - Xo)) <= 1e-12 * np.max(np.abs(Xo))


# ---------------------------------------------------------------------------------------------
# conversions and the Gram matrix
# ---------------------------------------------------------------------------------------------

def test_sym_to_f64_bit_exact(lrc):
    _say("sym_to_f64 n=150 ldc=160")
    n = 150
    C = np.full((n, 160), np.nan, dtype=np.float32)
    C[:, :n] = np.where(np.tri(n, dtype=bool).T, _gauss64(n, n, 70).astype(np.float32), np.nan)
    scale = 1.0 / 3.0
    A = host(lrc.lrc_sym_to_f64(dev(C, "f32")[:, :n], scale))
    U = np.triu(C[:, :n].astype(np.float64) * scale)
    ref = U + np.triu(U, 1).T
    assert np.array_equal(A, ref)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_to_f64_bit_exact(lrc, dt):
    _say("to_f64 %s 77x130" % dt)
    X = inputs.gaussian(77, 130, 0.5, dt, inputs.CFG_KFAC, 3, 0, inputs.S_ACT)
    Y = host(lrc.lrc_to_f64(dev(X, dt), 0.25))
    assert np.array_equal(Y, oracle.widen(X, dt) * 0.25)


def test_gram_f64(lrc):
    _say("gram_f64 150x333")
    m, n = 150, 333
    B = _gauss64(m, n, 80) * np.exp(_gauss64(m, 1, 81))
    G = torch.full((m, m), float("nan"), dtype=torch.float32, device="cuda")
    lrc.lrc_gram_f64(dev(B, "f64"), G)
    G = host(G).astype(np.float64)
    Go = oracle.covariance(B.T, "f64")
    up = np.triu(np.ones((m, m), dtype=bool))
    assert np.all(np.isnan(G[~up])), "strict lower triangle was written"
    d = np.sqrt(np.diag(Go))
    bound = 2.0 ** -24 * np.abs(Go) * 1.0001 + n * 2.0 ** -52 * d[:, None] * d[None, :]
    assert np.all(np.abs(G - Go)[up] <= bound[up])


# ---------------------------------------------------------------------------------------------
# the chain
# ---------------------------------------------------------------------------------------------

@pytest.mark.parametrize("prec", [1, 2])
def test_curvature_chain_parity(lrc, prec):
    from activation_aware_rank_amd.curvature import curvature_truncation
    n_tok, d_in, d_out, k = 4096, 200, 330, 48
    _say("curvature chain N=%d %dx%d k=%d prec=%d" % (n_tok, d_in, d_out, k, prec))
    d = inputs.curvature_layer(n_tok, d_in, d_out)
    out = curvature_truncation(dev(d["X"], "bf16"), dev(d["G"], "bf16"), dev(d["W"], "bf16"), k, prec)
    info = host(out["info"])
    assert np.all(info == 0), info
    lam, U = host(out["lam"]), host(out["U"])
    A, Bt = host(out["A"]), host(out["Bt"]).astype(np.float64)
    Lx, Lg = host(out["Lx"]), host(out["Lg"])

    W64 = oracle.widen(d["W"], "bf16")
    Sx = oracle.covariance(d["X"], "bf16") / n_tok
    Sg = oracle.covariance(d["G"], "bf16") / n_tok
    ref = oracle.kfac_compress(Sx, Sg, W64, k)
    check_lambda(lam, ref["lam"])
    assert gap(ref["lam"], k) > 1e-4
    s = sin_theta_max(U, ref["U"], k)
    assert s <= 1e-3, "retained subspace sin theta %.3e" % s
    Wk = A @ Bt.T
    Wk_o = ref["A"] @ ref["B"]
    e = np.linalg.norm(Wk - Wk_o) / np.linalg.norm(Wk_o)
    assert e <= 1e-4, "W_k relative error %.3e" % e
    print("W_k relative error %.3e, sin theta %.3e" % (e, s))
    # closed form in the curvature metric, from GPU quantities alone
    R = Lx.T @ (W64 - Wk) @ Lg
    tail = np.sum(np.maximum(lam[k:], 0.0))
    assert abs(np.sum(R * R) - tail) <= 1e-4 * tail


def test_curvature_chain_full_size_properties(lrc):
    """13B-shaped FFN matrix at full size (131072 tokens, 5120 x 13824, k = 1024), inputs drawn on
    the GPU; checked through properties that hold at any size (fp64 torch products as the checker):
    Cholesky backward error on sampled rows, the whitening products on sampled columns, eigen-
    residual and orthogonality of U_k, L_x^T A = U_k, and the closed-form weighted error."""
    from activation_aware_rank_amd.curvature import curvature_truncation
    n_tok, d_in, d_out, k = 131072, 5120, 13824, 1024
    _say("curvature chain full size N=%d %dx%d k=%d prec=2" % (n_tok, d_in, d_out, k))
    d = inputs.curvature_layer_gpu(n_tok, d_in, d_out, 20261203, torch.device("cuda"))
    out = curvature_truncation(d["X"], d["G"], d["W"], k, prec=2)
    assert np.all(host(out["info"]) == 0), host(out["info"])
    f64 = torch.float64
    gen = torch.Generator().manual_seed(5)

    # Cholesky: |L L^T - Sigma|_ij <= 2 (n + 1) 2^-53 sqrt(Sigma_ii Sigma_jj), Sigma recomputed by
    # the same deterministic entry points
    for name, X, n in (("Lx", d["X"], d_in), ("Lg", d["G"], d_out)):
        C = torch.zeros(n, n, dtype=torch.float32, device="cuda")
        lrc.lrc_cov_accumulate(X, None, C)
        S = lrc.lrc_sym_to_f64(C, 1.0 / n_tok)
        del C
        L = out[name]
        rows = torch.randint(0, n, (48,), generator=gen).cuda()
        R = L[rows] @ L.T
        dS = torch.sqrt(torch.diagonal(S))
        bound = 2 * (n + 1) * 2.0 ** -53 * dS[rows][:, None] * dS[None, :]
        excess = float(((R - S[rows]).abs() - bound).max())
        assert excess <= 0.0, "%s backward error exceeds the bound by %.3e" % (name, excess)
        del S, R
    Lx, Lg = out["Lx"], out["Lg"]
    W64 = d["W"].to(f64)
    # whitening: W~[:, cols] = L_x^T (W L_g[:, cols])
    cols = torch.randint(0, d_out, (32,), generator=gen).cuda()
    ref = Lx.T @ (W64 @ Lg[:, cols])
    e = float((out["Wt"][:, cols] - ref).abs().max() / ref.abs().max())
    assert e <= 1e-12, "whitening error %.3e" % e
    # eigenpairs of M = W~ W~^T (fp32 storage): residual and orthogonality of U_k
    lam = out["lam"]
    U = out["U"].to(f64)
    Wt = out["Wt"]
    MU = Wt @ (Wt.T @ U)
    res = float(torch.linalg.vector_norm(MU - U * lam[:k], dim=0).max() / lam[0])
    orth = float((U.T @ U - torch.eye(k, dtype=f64, device="cuda")).abs().max())
    assert res <= 1e-5 and orth <= 1e-5, "eig residual %.3e, orthogonality %.3e" % (res, orth)
    # A solves L_x^T A = U_k
    e = float((Lx.T @ out["A"] - U).abs().max())
    assert e <= 1e-10, "triangular solve residual %.3e" % e
    # closed form: ||L_x^T (W - A B) L_g||_F^2 = sum of the discarded eigenvalues
    D = W64 - out["A"] @ out["Bt"].to(f64).T
    R = (Lx.T @ D) @ Lg
    tail = float(lam[k:].clamp(min=0).sum())
    got = float((R * R).sum())
    print("closed form: %.6e vs tail %.6e, eig residual %.2e, orth %.2e" % (got, tail, res, orth))
    assert abs(got - tail) <= 1e-4 * tail
