"""Parity of the HIP path (through the C ABI) against the fp64 oracle on the same seeded inputs,
at sizes the oracle finishes in seconds that still span several tiles and have ragged tails.

Tolerances (the contract): eigenvalues within 1e-5 lambda_max; eps_k within 1e-4 relative where
eps_k >= 1e-4 eps_0 and below that within 2^-23 eps_0 (fp32 eigensolver) or 2^-24 eps_0 (fp64 eigensolver
and the n <= 128 Jacobi path); largest principal angle of the retained subspace below 1e-3 rad; allocation bit-exact on identical inputs; error curve bit-exact on
identical eigenvalues (same summation order).  Diagnostics: covariance entries within 1e-5
lambda_max, Fisher scores within 1e-12 relative, factors within 1e-6 relative (Frobenius).
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from activation_aware_rank_amd import inputs
from parity_utils import check_eps, check_lambda, dev, gap, host, sin_theta_max

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module")
def lrc():
    from activation_aware_rank_amd import lrc as m
    return m


def _say(msg):
    print("\n[case] " + msg, flush=True)


# ---------------------------------------------------------------------------------------------
# covariance
# ---------------------------------------------------------------------------------------------

def _cov_gpu(lrc, X, xdt, W, n_blocks=1, C=None):
    Xd = dev(X, xdt)
    Wd = dev(W, xdt) if W is not None else None
    d_out = X.shape[1] if W is None else W.shape[1]
    hd = d_out // n_blocks
    if C is None:
        C = torch.zeros((n_blocks, hd, hd) if n_blocks > 1 else (d_out, d_out), dtype=torch.float32, device="cuda")
    info = lrc.lrc_cov_accumulate(Xd, Wd, C, n_blocks=n_blocks)
    assert int(host(info)[0]) == 0
    return C


def _upper_err(C_hat, C_ref):
    U = np.triu(np.ones(C_ref.shape[-2:], dtype=bool))
    return np.max(np.abs(np.where(U, C_hat - C_ref, 0.0)))


@pytest.mark.parametrize("n_tok,d_in,heads", [(1000, 256, 8), (300, 512, 3), (5000, 4096, 2)])
def test_cov_per_head_fused_vs_oracle(lrc, n_tok, d_in, heads):
    """Heads of 128 with LRC_HEAD_FUSED=1 take the fused kernel (GEMM, fp16 split and SYRK of each head's
    128-token tiles in LDS, partial sums per token range added in range order): every head block against
    the oracle's per-head covariance (1e-5 of sqrt(C_ii C_jj)), and the default two-kernel path through
    memory to the same bar; ragged token counts, the fused path over two accumulating calls."""
    _say("cov per-head fused %d x %d, %d heads of 128" % (n_tok, d_in, heads))
    X = inputs.per_head(n_tok=n_tok, d_model=d_in, head_dim=128)["X"]
    W = inputs.weight(d_in, heads * 128, "bf16", inputs.CFG_HEADS, 0, 7)
    os.environ["LRC_HEAD_FUSED"] = "1"
    try:
        C = _cov_gpu(lrc, X[:n_tok // 3], "bf16", W, n_blocks=heads)
        _cov_gpu(lrc, X[n_tok // 3:], "bf16", W, n_blocks=heads, C=C)
    finally:
        del os.environ["LRC_HEAD_FUSED"]
    C = host(C).astype(np.float64)
    C2 = host(_cov_gpu(lrc, X, "bf16", W, n_blocks=heads)).astype(np.float64)
    Cr = oracle.covariance(X, "bf16", W, "bf16", n_blocks=heads)
    U = np.triu(np.ones((128, 128), dtype=bool))
    for hh in range(heads):
        dg = np.sqrt(np.outer(np.diag(Cr[hh]), np.diag(Cr[hh])))
        e1 = np.max(np.abs(C[hh] - Cr[hh])[U] / dg[U])
        e2 = np.max(np.abs(C2[hh] - Cr[hh])[U] / dg[U])
        print("head %d: fused %.2e, through memory %.2e of sqrt(C_ii C_jj)" % (hh, e1, e2))
        assert e1 <= 1e-5 and e2 <= 1e-5
        assert np.all(np.tril(C[hh], -1) == 0)


def test_cov_single_layer_fp32(lrc):
    _say("cov fp32 2048x256 -> 256 (full single-layer size)")
    d = inputs.single_layer()
    C = host(_cov_gpu(lrc, d["X"], "f32", d["W"]))
    Cr = oracle.covariance(d["X"], "f32", d["W"], "f32")
    lam1 = np.linalg.eigvalsh(Cr)[-1]
    assert _upper_err(C, Cr) <= 1e-5 * lam1
    assert np.all(np.tril(C, -1) == 0)  # lower triangle never written


@pytest.mark.parametrize("n_tok,d_in,d_out", [(5000, 512, 1376), (40000, 256, 600), (777, 136, 200)])
def test_cov_bf16_mfma_ragged(lrc, n_tok, d_in, d_out):
    _say("cov bf16 %dx%d -> %d" % (n_tok, d_in, d_out))
    X = inputs.block_activations(d_in, n_tok)
    W = inputs.weight(d_in, d_out, "bf16", inputs.CFG_BLOCK, 0, 1)
    C = host(_cov_gpu(lrc, X, "bf16", W))
    Cr = oracle.covariance(X, "bf16", W, "bf16")
    lam1 = np.linalg.eigvalsh(Cr)[-1]
    err = _upper_err(C, Cr) / lam1
    print("max |dC| / lambda_max = %.3e" % err)
    assert err <= 1e-5
    assert np.all(np.tril(C, -1) == 0)


def _bf16_pow2(a, e):
    """bf16 bit patterns times 2^e (e broadcast against a), exact for the normal range used here."""
    f = (a.astype(np.uint32) << 16).view(np.float32) * np.exp2(np.asarray(e, dtype=np.float32))
    return (np.ascontiguousarray(f, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


@pytest.mark.parametrize("sx,sw", [(10, 7), (-14, -10)])
def test_cov_split_scaled_columns(lrc, sx, sw):
    """Per-output power-of-two scales of the fp16 hi/lo split: output magnitudes spread over 2^-9 ..
    2^9 around 2^(sx + sw) (far outside the fp16 range at either end without the scales), two
    outputs identically zero.  Every upper entry is checked against sqrt(C_ii C_jj), so a column
    that lost bits to fp16 underflow or overflow fails even when it is small next to lambda_max."""
    _say("cov split scales 2^%d x 2^%d, 6000 x 256 -> 520" % (sx, sw))
    n_tok, d_in, d_out = 6000, 256, 520
    X = _bf16_pow2(inputs.block_activations(d_in, n_tok), sx)
    e = sw + (np.arange(d_out) % 7) * 3 - 9
    W = _bf16_pow2(inputs.weight(d_in, d_out, "bf16", inputs.CFG_BLOCK, 0, 2), e[None, :])
    W[:, [5, 17]] = 0
    C = host(_cov_gpu(lrc, X, "bf16", W))
    Cr = oracle.covariance(X, "bf16", W, "bf16")
    dg = np.diag(Cr)
    scale = np.sqrt(np.outer(dg, dg))
    U = np.triu(np.ones((d_out, d_out), dtype=bool)) & (scale > 0)
    rel = np.max(np.abs(C - Cr)[U] / scale[U])
    rel_diag = np.max(np.abs(np.diag(C) - dg)[dg > 0] / dg[dg > 0])
    print("max |dC_ij| / sqrt(C_ii C_jj) = %.3e, diagonal %.3e" % (rel, rel_diag))
    assert rel <= 1e-5 and rel_diag <= 1e-5
    for j in (5, 17):  # a zero output gives an exactly zero row and column
        assert np.all(C[j, j:] == 0) and np.all(C[:j, j] == 0)


def test_cov_many_tiles_xcd_order(lrc):
    """d_out 8320: 65 block rows of 128, 2145 upper tiles per token split, enough for the per-XCD
    super-tile order (a ragged last super-tile row and column: 65 = 8 x 8 + 1)."""
    _say("cov bf16 300 x 136 -> 8320")
    X = inputs.block_activations(136, 300)
    W = inputs.weight(136, 8320, "bf16", inputs.CFG_BLOCK, 0, 3)
    C = host(_cov_gpu(lrc, X, "bf16", W))
    Cr = oracle.covariance(X, "bf16", W, "bf16")
    dg = np.diag(Cr)
    scale = np.sqrt(np.outer(dg, dg))
    U = np.triu(np.ones(Cr.shape, dtype=bool))
    rel = np.max(np.abs(C - Cr)[U] / scale[U])
    print("max |dC_ij| / sqrt(C_ii C_jj) = %.3e" % rel)
    assert rel <= 1e-5
    assert np.all(np.tril(C, -1) == 0)


@pytest.mark.parametrize("d_out", [640, 384])
def test_cov_from_input_vs_oracle(lrc, d_out):
    """C = W^T H W from the GPU's input covariance H = X^T X (one bf16 product, fp32 sums) against the
    oracle's direct covariance of Y = X W: every upper entry relative to sqrt(C_ii C_jj), then the
    eigenvalues and the error curve of the factored C to the pipeline's tolerances."""
    _say("cov from input covariance, 5000 x 512 -> %d" % d_out)
    X = inputs.block_activations(512, 5000)
    W = inputs.weight(512, d_out, "bf16", inputs.CFG_BLOCK, 0, 4)
    H = _cov_gpu(lrc, X, "bf16", None)
    C = lrc.lrc_cov_from_input(H, dev(W, "bf16"))
    Cr = oracle.covariance(X, "bf16", W, "bf16")
    Ch = host(C).astype(np.float64)
    dg = np.sqrt(np.outer(np.diag(Cr), np.diag(Cr)))
    U = np.triu(np.ones(Cr.shape, dtype=bool))
    rel = np.max(np.abs(Ch - Cr)[U] / dg[U])
    print("max |dC_ij| / sqrt(C_ii C_jj) = %.3e" % rel)
    assert rel <= 1e-5
    assert np.all(np.tril(Ch, -1) == 0)
    lam, V, info = lrc.lrc_eigh(C, n_vec=64, prec=2)
    assert int(info.item()) == 0
    eps = host(lrc.lrc_error_curve(lam[None]))[0]
    lam_r, V_r = oracle.eigh(Cr)
    check_lambda(host(lam), lam_r)
    check_eps(eps, oracle.error_curve(lam_r), prec=2)


def test_cov_identity_weight(lrc):
    _say("cov bf16 W = I, 3000 x 264")
    X = inputs.block_activations(264, 3000)
    C = host(_cov_gpu(lrc, X, "bf16", None))
    Cr = oracle.covariance(X, "bf16")
    lam1 = np.linalg.eigvalsh(Cr)[-1]
    assert _upper_err(C, Cr) <= 2e-6 * lam1


def test_cov_per_head_blocks(lrc):
    _say("cov per-head bf16 4096 x 512, 4 heads of 128")
    d = inputs.per_head(n_tok=4096, d_model=512, head_dim=128)
    C = host(_cov_gpu(lrc, d["X"], "bf16", d["W"], n_blocks=4))
    Cr = oracle.covariance(d["X"], "bf16", d["W"], "bf16", n_blocks=4)
    for h in range(4):
        lam1 = np.linalg.eigvalsh(Cr[h])[-1]
        assert _upper_err(C[h], Cr[h]) <= 1e-5 * lam1, h


def test_cov_accumulates_and_is_deterministic(lrc):
    _say("cov chunked calls and repeatability")
    X = inputs.block_activations(256, 6000)
    W = inputs.weight(256, 384, "bf16", inputs.CFG_BLOCK, 0, 2)
    C1 = host(_cov_gpu(lrc, X, "bf16", W))
    C1b = host(_cov_gpu(lrc, X, "bf16", W))
    assert np.array_equal(C1, C1b)  # bitwise repeatable
    C = torch.zeros(384, 384, dtype=torch.float32, device="cuda")
    _cov_gpu(lrc, X[:2500], "bf16", W, C=C)
    _cov_gpu(lrc, X[2500:], "bf16", W, C=C)
    C2 = host(C)
    lam1 = np.linalg.eigvalsh(np.triu(C1) + np.triu(C1, 1).T)[-1]
    assert np.max(np.abs(C2 - C1)) <= 1e-6 * lam1


def test_cov_nonfinite_input_sets_info(lrc):
    _say("cov with a NaN input")
    X = inputs.single_layer(n_tok=64, d_in=16, d_out=16)["X"].copy()
    X[3, 5] = np.nan
    Xd, Wd = dev(X, "f32"), dev(np.eye(16, dtype=np.float32), "f32")
    C = torch.zeros(16, 16, dtype=torch.float32, device="cuda")
    info = lrc.lrc_cov_accumulate(Xd, Wd, C)
    assert int(host(info)[0]) == 1


def test_cov_rejects_empty(lrc):
    X = torch.zeros(0, 8, dtype=torch.float32, device="cuda")
    C = torch.zeros(8, 8, dtype=torch.float32, device="cuda")
    with pytest.raises(lrc.LrcError):
        lrc.lrc_cov_accumulate(X, None, C)


# ---------------------------------------------------------------------------------------------
# eigendecomposition
# ---------------------------------------------------------------------------------------------

def _oracle_cov32(X, xdt, W, n_blocks=1):
    """Oracle covariance rounded to fp32 (the GPU eig's input) and the same values in fp64."""
    C = oracle.covariance(X, xdt, W, xdt, n_blocks=n_blocks)
    C32 = C.astype(np.float32)
    return C32, C32.astype(np.float64)


@pytest.mark.parametrize("prec", [1, 2])
@pytest.mark.parametrize("case", ["single256", "block300", "gate_like", "order129", "order193"])
def test_eigh_large_vs_oracle(lrc, case, prec):
    """Orders above 128: 256 (fp32: the whole tridiagonalisation by one workgroup in LDS), 300 and 430
    (the column chain, then the last block in LDS), 129 (the smallest order of this path) and 193 (fp64:
    one column panel before the block)."""
    _say("eigh large %s prec %d" % (case, prec))
    if case == "single256":
        d = inputs.single_layer()
        C32, C64 = _oracle_cov32(d["X"], "f32", d["W"])
        k = 64
    elif case in ("order129", "order193"):
        n = 129 if case == "order129" else 193
        d = inputs.single_layer(n_tok=1024, d_in=n, d_out=n)
        C32, C64 = _oracle_cov32(d["X"], "f32", d["W"])
        k = n // 4
    elif case == "block300":
        X = inputs.block_activations(320, 4096)
        W = inputs.weight(320, 300, "bf16", inputs.CFG_BLOCK, 0, 3)
        C32, C64 = _oracle_cov32(X, "bf16", W)
        k = inputs.rank_at_ratio(320, 300, 0.6)
    else:  # 160 -> 430: rank-deficient covariance, like gate/up
        X = inputs.block_activations(160, 4096)
        W = inputs.weight(160, 430, "bf16", inputs.CFG_BLOCK, 0, 4)
        C32, C64 = _oracle_cov32(X, "bf16", W)
        k = inputs.rank_at_ratio(160, 430, 0.6)
    n = C32.shape[0]
    lam_r, V_r = oracle.eigh(C64)
    Cu = np.triu(C32) + np.tril(np.full((n, n), np.nan, np.float32), -1)  # lower triangle must not be read
    lam, V, info = lrc.lrc_eigh(dev(Cu, "f32"), n_vec=n, prec=prec)
    lam, V = host(lam), host(V)
    assert int(host(info)[0]) == 0
    e = check_lambda(lam, lam_r)
    s = sin_theta_max(V, V_r, k)
    print("lambda err %.2e, sin theta(k=%d) %.2e, gap %.2e" % (e, k, s, gap(lam_r, k)))
    assert s <= 1e-3
    V64 = V.astype(np.float64)
    assert np.max(np.abs(V64.T @ V64 - np.eye(n))) <= 1e-5
    assert np.linalg.norm(C64 @ V64 - V64 * lam) <= 1e-5 * np.linalg.norm(C64)
    idx = np.argmax(np.abs(V), axis=0)
    assert np.all(V[idx, np.arange(n)] > 0)
    assert np.all(np.diff(lam) <= 0)


@pytest.mark.parametrize("prec", [1, 2])
@pytest.mark.parametrize("n,batch", [(128, 4), (17, 3), (64, 2)])
def test_eigh_jacobi_vs_oracle(lrc, n, batch, prec):
    _say("eigh jacobi n=%d batch=%d prec %d" % (n, batch, prec))
    d = inputs.per_head(n_tok=4096, d_model=n * batch, head_dim=n)
    C = oracle.covariance(d["X"], "bf16", d["W"], "bf16", n_blocks=batch) if batch > 1 else None
    C32 = C.astype(np.float32)
    lam, V, info = lrc.lrc_eigh(dev(C32, "f32"), n_vec=n, prec=prec)
    lam, V, info = host(lam), host(V), host(info)
    k = max(1, n // 4)
    for b in range(batch):
        assert info[b] == 0
        lam_r, V_r = oracle.eigh(C32[b].astype(np.float64))
        el = check_lambda(lam[b], lam_r)
        s = sin_theta_max(V[b], V_r, k)
        print("matrix %d: lambda err %.2e lambda_max, sin theta(k=%d) %.2e, gap %.2e" % (b, el, k, s, gap(lam_r, k)))
        assert s <= 1e-3, (b, s, gap(lam_r, k))


def test_eigh_jacobi_degenerate(lrc):
    """The n <= 128 path on degenerate inputs: a rank-deficient per-head covariance (40 tokens,
    n = 128: 88 eigenvalues at rounding level), a permuted diagonal with repeated eigenvalues
    (n = 96), the zero matrix and the orders 1 and 2."""
    _say("eigh jacobi degenerate inputs")
    d = inputs.per_head(n_tok=40, d_model=128, head_dim=128)
    C = oracle.covariance(d["X"], "bf16", d["W"], "bf16").astype(np.float32)
    lam, V, info = lrc.lrc_eigh(dev(C, "f32"), n_vec=128, prec=2)
    lam, V = host(lam), host(V).astype(np.float64)
    assert int(host(info)[0]) == 0
    lam_r, V_r = oracle.eigh(C.astype(np.float64))
    assert np.max(np.abs(lam - lam_r)) <= 1e-5 * lam_r[0]
    assert np.all(np.abs(lam[40:]) <= 1e-5 * lam_r[0])
    assert sin_theta_max(V, V_r, 32) <= 1e-3
    assert np.max(np.abs(V.T @ V - np.eye(128))) <= 1e-5
    dvals = np.array([3.0] * 30 + [1.5] * 50 + [0.25] * 16, dtype=np.float32)
    perm = np.random.default_rng(4).permutation(96)
    lam, V, info = lrc.lrc_eigh(dev(np.diag(dvals[perm]), "f32"), n_vec=96, prec=2)
    lam, V = host(lam), host(V).astype(np.float64)
    assert int(host(info)[0]) == 0
    assert np.allclose(lam, np.sort(dvals)[::-1], rtol=0, atol=1e-12)
    assert np.max(np.abs(V.T @ V - np.eye(96))) <= 1e-12
    P = V[:, :30] @ V[:, :30].T
    assert np.allclose(P, np.diag((dvals[perm] == 3).astype(float)), atol=1e-12)
    lam, V, info = lrc.lrc_eigh(torch.zeros(128, 128, dtype=torch.float32, device="cuda"), n_vec=128, prec=2)
    assert int(host(info)[0]) == 0 and np.all(host(lam) == 0)
    assert np.array_equal(host(V), np.eye(128, dtype=np.float32))
    for Cs in (np.array([[2.5]]), np.array([[2.0, 1.0], [1.0, 2.0]])):
        lam, V, info = lrc.lrc_eigh(dev(Cs.astype(np.float32), "f32"), n_vec=len(Cs), prec=2)
        lam_r, V_r = oracle.eigh(Cs)
        assert int(host(info)[0]) == 0
        assert np.allclose(host(lam), lam_r, rtol=1e-14, atol=0)
        assert np.allclose(np.abs(host(V)), np.abs(V_r), atol=1e-7)


@pytest.mark.parametrize("prec", [1, 2])
def test_eigh_large_batch_matches_single_calls(lrc, prec):
    """Members of a batch (n > 128) run concurrently on helper streams, several at a time, each
    with a workspace of its own; every member must equal the same matrix decomposed alone, bit for
    bit, and a non-finite member flags only itself."""
    _say("eigh large batch of 10 (n = 300, more members than helper streams) prec %d" % prec)
    n, batch, nv = 300, 10, 40
    X = inputs.block_activations(320, 4096)
    Cs = []
    for b in range(batch):
        W = inputs.weight(320, n, "bf16", inputs.CFG_BLOCK, 0, 10 + b)
        Cs.append(oracle.covariance(X, "bf16", W, "bf16").astype(np.float32))
    Cs[4][2, 9] = np.nan
    Cb = dev(np.stack(Cs), "f32")
    lam, V, info = lrc.lrc_eigh(Cb, n_vec=nv, prec=prec)
    lam, V, info = host(lam), host(V), host(info)
    assert list(info) == [0, 0, 0, 0, 1, 0, 0, 0, 0, 0]
    for b in (0, 1, 2, 3, 5):
        l1, V1, i1 = lrc.lrc_eigh(dev(Cs[b], "f32"), n_vec=nv, prec=prec)
        assert int(host(i1)[0]) == 0
        assert np.array_equal(lam[b], host(l1)), b
        assert np.array_equal(V[b], host(V1)), b
    lam_r, V_r = oracle.eigh(Cs[5].astype(np.float64))
    check_lambda(lam[5], lam_r)
    assert sin_theta_max(V[5], V_r, 20) <= 1e-3


@pytest.mark.parametrize("prec", [1, 2])
def test_eigh_multi_matches_single_calls(lrc, prec):
    """Groups of different n in one call: the n > 128 members share the helper streams (here more
    members than streams, so a stream goes on from a larger matrix to a smaller one in the same
    workspace region) and the Jacobi group runs on the caller's stream; every member must equal
    lrc_eigh on that member alone, bit for bit."""
    _say("eigh multi: 1 x 513, 2 x 300, 3 x 200 and a Jacobi group 2 x 64, prec %d" % prec)
    X = inputs.block_activations(320, 4096)
    spec = [(300, 2, 40), (200, 3, 64), (64, 2, 16), (513, 1, 10)]
    groups, mats = [], []
    for gi, (n, b, nv) in enumerate(spec):
        Cs = []
        for m in range(b):
            W = inputs.weight(320, n, "bf16", inputs.CFG_BLOCK, 0, 20 + 4 * gi + m)
            Cs.append(oracle.covariance(X, "bf16", W, "bf16").astype(np.float32))
        mats.append(Cs)
        groups.append((dev(np.stack(Cs), "f32"), nv))
    out = lrc.lrc_eigh_multi(groups, prec=prec)
    for (n, b, nv), Cs, (lam, V, info) in zip(spec, mats, out):
        lam, V, info = host(lam), host(V), host(info)
        assert np.all(info == 0)
        for m in range(b):
            l1, V1, i1 = lrc.lrc_eigh(dev(Cs[m], "f32"), n_vec=nv, prec=prec)
            assert int(host(i1)[0]) == 0
            assert np.array_equal(lam[m], host(l1)), (n, m)
            assert np.array_equal(V[m], host(V1)), (n, m)
    lam_r, V_r = oracle.eigh(mats[3][0].astype(np.float64))
    check_lambda(host(out[3][0])[0], lam_r)
    assert sin_theta_max(host(out[3][1])[0], V_r, 10) <= 1e-3
    # the calling thread enqueueing every member itself (one helper stream): the same bits
    import os
    os.environ["LRC_EIGH_HOST_THREADS"] = "0"
    try:
        out1 = lrc.lrc_eigh_multi(groups, prec=prec)
    finally:
        del os.environ["LRC_EIGH_HOST_THREADS"]
    for (lam, V, info), (lam1, V1, info1) in zip(out, out1):
        assert np.array_equal(host(info1), host(info))
        assert np.array_equal(host(lam1), host(lam))
        assert np.array_equal(host(V1), host(V))


def test_eigh_multi_concurrent_calls(lrc):
    """Three lrc_eigh_multi calls at once from three host threads, each on its own stream with its own
    workspace (the calls take different helper streams: 3 + 2 + 1 members fit the eight): every member
    must equal the same matrix decomposed alone, bit for bit."""
    import threading
    _say("eigh multi: three concurrent calls (3 x 300, 2 x 260, 1 x 513)")
    X = inputs.block_activations(320, 4096)
    spec = [(300, 3, 40), (260, 2, 24), (513, 1, 10)]
    mats, Cd = [], []
    for gi, (n, b, nv) in enumerate(spec):
        Cs = [oracle.covariance(X, "bf16", inputs.weight(320, n, "bf16", inputs.CFG_BLOCK, 0, 60 + 4 * gi + m),
                                "bf16").astype(np.float32) for m in range(b)]
        mats.append(Cs)
        Cd.append(dev(np.stack(Cs), "f32"))
    streams = [torch.cuda.Stream() for _ in spec]
    wss = [torch.empty(lrc.lrc_eigh_multi_workspace([(n, b, nv)], 1), dtype=torch.uint8, device="cuda")
           for n, b, nv in spec]
    # outputs allocated (and info zeroed) here, before the threads, so no call orders against another stream
    outs = [(torch.empty(b, n, dtype=torch.float64, device="cuda"), torch.empty(b, n, nv, dtype=torch.float32,
             device="cuda"), torch.zeros(b, dtype=torch.int32, device="cuda")) for n, b, nv in spec]
    torch.cuda.synchronize()
    out, errs = [None] * len(spec), []

    def run(i):
        try:
            n, b, nv = spec[i]
            lrc.lrc_eigh_multi([(Cd[i], nv) + outs[i]], prec=1, ws=wss[i], stream=streams[i])
            out[i] = outs[i]
        except Exception as e:  # reported after the join
            errs.append(e)

    th = [threading.Thread(target=run, args=(i,)) for i in range(len(spec))]
    for t in th:
        t.start()
    for t in th:
        t.join()
    assert not errs, errs
    torch.cuda.synchronize()
    for (n, b, nv), Cs, (lam, V, info) in zip(spec, mats, out):
        lam, V, info = host(lam), host(V), host(info)
        assert np.all(info == 0)
        for m in range(b):
            l1, V1, i1 = lrc.lrc_eigh(dev(Cs[m], "f32"), n_vec=nv, prec=1)
            assert np.array_equal(lam[m], host(l1)), (n, m)
            assert np.array_equal(V[m], host(V1)), (n, m)


@pytest.mark.parametrize("prec", [1, 2])
def test_eigh_range_basis_vs_oracle(lrc, prec):
    """A covariance of Y = X W with d_in < d_out decomposed through B = Q^T C Q, Q a basis of range(W^T):
    the oracle's full eigendecomposition (its n - d_in trailing eigenvalues are zero to rounding), the
    closed form through the factors, and a batch with a stride between the bases equal to single
    calls; the lower triangle of C is never read."""
    _say("eigh with a range basis: 200 -> 520, 2048 tokens, prec %d" % prec)
    d_in, n, k = 200, 520, 48
    X = inputs.block_activations(d_in, 2048)
    Ws = [inputs.weight(d_in, n, "bf16", inputs.CFG_BLOCK, 0, 30 + i) for i in range(2)]
    Cs = [_oracle_cov32(X, "bf16", W)[0] for W in Ws]
    Cu = np.stack([np.triu(C) + np.tril(np.full((n, n), np.nan, np.float32), -1) for C in Cs])
    Wd = torch.stack([dev(W, "bf16") for W in Ws])
    out = lrc.lrc_eigh_multi([(dev(Cu, "f32"), k, None, None, None, Wd)], prec=prec)
    lam_b, V_b, info_b = (host(x) for x in out[0])
    assert np.all(info_b == 0), info_b
    X64 = oracle.widen(X, "bf16")
    for m in range(2):
        lam, V = lam_b[m], V_b[m]
        C64 = Cs[m].astype(np.float64)
        lam_r, V_r = oracle.eigh(C64)
        e = check_lambda(lam, lam_r)
        assert np.all(np.diff(lam) <= 0)
        assert np.count_nonzero(lam == 0.0) >= n - d_in  # the complement of range(W^T)
        s = sin_theta_max(V, V_r, k)
        V64 = V.astype(np.float64)
        orth = np.max(np.abs(V64.T @ V64 - np.eye(k)))
        res = np.linalg.norm(C64 @ V64 - V64 * lam[:k], axis=0).max() / lam_r[0]
        print("member %d: lambda err %.2e, sin theta %.2e (gap %.2e), orthogonality %.2e, residual %.2e"
              % (m, e, s, gap(lam_r, k), orth, res))
        assert s <= 1e-3 and orth <= 1e-5 and res <= 1e-5
        idx = np.argmax(np.abs(V), axis=0)
        assert np.all(V[idx, np.arange(k)] > 0)
        # closed form: ||X W - X W V_k V_k^T||^2 = sum of the eigenvalues past k
        W64 = oracle.widen(Ws[m], "bf16")
        R = X64 @ (W64 - (W64 @ V64) @ V64.T)
        eps = oracle.error_curve(lam_r)
        assert abs(np.sum(R * R) - eps[k]) <= 1e-4 * eps[k] + 1e-6 * eps[0]
        # the member alone: the same bits
        l1, V1, i1 = lrc.lrc_eigh_multi([(dev(Cu[m], "f32"), k, None, None, None, Wd[m])], prec=prec)[0]
        assert int(host(i1)[0]) == 0
        assert np.array_equal(host(l1), lam) and np.array_equal(host(V1), V)


def test_eigh_padded_vector_rows(lrc):
    """V with a leading dimension larger than n_vec (rows padded to 16 bytes, as bench.py allocates it):
    a lockstep pair of order 300 and a member through a 300-row range basis of order 520, n_vec = 37,
    equal the contiguous outputs bit for bit, and the padding columns are left as they were."""
    _say("eigh with padded V rows: 2 x 300 and 520 via a 300-row basis, n_vec 37 in rows of 40")
    X = inputs.block_activations(300, 1024)
    Cf = np.stack([oracle.covariance(X, "bf16", inputs.weight(300, 300, "bf16", inputs.CFG_BLOCK, 0, 80 + m),
                                     "bf16").astype(np.float32) for m in range(2)])
    Wr = inputs.weight(300, 520, "bf16", inputs.CFG_BLOCK, 0, 82)
    Cr = _oracle_cov32(X, "bf16", Wr)[0]
    nv = 37
    ref = lrc.lrc_eigh_multi([(dev(Cf, "f32"), nv), (dev(Cr, "f32"), nv, None, None, None, dev(Wr, "bf16"))], prec=1)
    Vp1 = torch.full((2, 300, 40), float("nan"), dtype=torch.float32, device="cuda")
    Vp2 = torch.full((520, 40), float("nan"), dtype=torch.float32, device="cuda")
    out = lrc.lrc_eigh_multi([(dev(Cf, "f32"), nv, None, Vp1[:, :, :nv], None),
                              (dev(Cr, "f32"), nv, None, Vp2[:, :nv], None, dev(Wr, "bf16"))], prec=1)
    for (l0, V0, i0), (l1, V1, i1) in zip(ref, out):
        assert np.all(host(i1) == 0)
        assert torch.equal(l0, l1) and torch.equal(V0, V1)
    assert bool(torch.isnan(Vp1[:, :, nv:]).all()) and bool(torch.isnan(Vp2[:, nv:]).all())


@pytest.mark.parametrize("prec,same_nv", [(1, False), (2, False), (1, True), (2, True)])
def test_eigh_lockstep_mixed_members(lrc, prec, same_nv):
    """Members of one tridiagonal order in one call are tridiagonalised in lockstep (one launch per
    column for all of them): two full decompositions of order 300 (one with a NaN entry), one of order
    520 through a 300-row range basis, and a third full one in a group of its own.  With one n_vec for
    all, the eigenvalues, vectors of T and back-transformation are batched too; with different n_vec
    they run per member.  Every member must equal the same call with lockstep off and the member
    decomposed alone, bit for bit; the NaN member reports info 1 without touching the others."""
    _say("eigh lockstep: 2 x 300 (one NaN) + 520 via a 300-row basis + 1 x 300, prec %d, same n_vec %s"
         % (prec, same_nv))
    nvs = (24, 24, 24) if same_nv else (24, 40, 16)
    X = inputs.block_activations(300, 1024)
    Cf = [oracle.covariance(X, "bf16", inputs.weight(300, 300, "bf16", inputs.CFG_BLOCK, 0, 70 + m),
                            "bf16").astype(np.float32) for m in range(3)]
    Cf[1][2, 9] = np.nan
    Wr = inputs.weight(300, 520, "bf16", inputs.CFG_BLOCK, 0, 74)
    Cr = _oracle_cov32(X, "bf16", Wr)[0]
    groups = [(dev(np.stack(Cf[:2]), "f32"), nvs[0]), (dev(Cr, "f32"), nvs[1], None, None, None, dev(Wr, "bf16")),
              (dev(Cf[2], "f32"), nvs[2])]
    out = lrc.lrc_eigh_multi(groups, prec=prec)
    os.environ["LRC_EIGH_LOCKSTEP"] = "0"
    try:
        off = lrc.lrc_eigh_multi(groups, prec=prec)
    finally:
        del os.environ["LRC_EIGH_LOCKSTEP"]
    for (lam, V, info), (lam0, V0, info0) in zip(out, off):
        assert np.array_equal(host(info), host(info0))
        assert np.array_equal(host(lam), host(lam0), equal_nan=True)
        assert np.array_equal(host(V), host(V0), equal_nan=True)
    assert list(host(out[0][2])) == [0, 1] and int(host(out[1][2])[0]) == 0 and int(host(out[2][2])[0]) == 0
    # a 2-D C gives lambda (n,), V (n, n_vec), info (1,)
    singles = [((dev(Cf[0], "f32"), nvs[0]), out[0][0][0], out[0][1][0]),
               ((dev(Cr, "f32"), nvs[1], None, None, None, dev(Wr, "bf16")), out[1][0], out[1][1]),
               ((dev(Cf[2], "f32"), nvs[2]), out[2][0], out[2][1])]
    for grp, lam, V in singles:
        l1, V1, i1 = lrc.lrc_eigh_multi([grp], prec=prec)[0]
        assert int(host(i1)[0]) == 0
        assert np.array_equal(host(l1), host(lam)) and np.array_equal(host(V1), host(V))
    lam_r, V_r = oracle.eigh(Cr.astype(np.float64))
    check_lambda(host(out[1][0]), lam_r)
    assert sin_theta_max(host(out[1][1]), V_r, nvs[1]) <= 1e-3


@pytest.mark.parametrize("prec", [1, 2])
@pytest.mark.parametrize("d_in,n,n_tok", [(320, 640, 3000), (256, 416, 1000)])
def test_cov_range_projected_vs_oracle(lrc, prec, d_in, n, n_tok):
    """The widening layer's covariance through its range basis without forming C: L from
    lrc_range_factor (W W^T = L L^T), B = (X L)^T (X L) from lrc_cov_accumulate_range in two calls (a
    ragged split of the tokens), B's eigendecomposition with projected = 1.  Against the oracle's
    direct covariance C = (X W)^T (X W) of the same bytes and its cyclic-Jacobi eigendecomposition:
    all n eigenvalues (the n - d_in past d_in are zero), eps_k, the retained subspace at k and the
    sign rule.  Diagnostics: L against numpy's Cholesky of W W^T, B against (X L)^T (X L) in fp64.
    320 spans two 256-row block tiles of the product (the second starting at its diagonal) and three
    128-wide SYRK tiles, ragged."""
    _say("cov range-projected %d x %d -> %d, prec %d" % (n_tok, d_in, n, prec))
    k = 64
    X = inputs.block_activations(d_in, n_tok)
    W = inputs.weight(d_in, n, "bf16", inputs.CFG_BLOCK, 0, 90)
    Xd, Wd = dev(X, "bf16"), dev(W, "bf16")
    L, info = lrc.lrc_range_factor(Wd)
    assert int(host(info)[0]) == 0
    B = torch.zeros(d_in, d_in, dtype=torch.float32, device="cuda")
    t1 = n_tok // 3 + 5
    for a, b in ((0, t1), (t1, n_tok)):
        i2 = lrc.lrc_cov_accumulate_range(Xd[a:b], L, B)
        assert int(host(i2)[0]) == 0
    X64, W64 = oracle.widen(X, "bf16"), oracle.widen(W, "bf16")
    L_np = np.linalg.cholesky(W64 @ W64.T)
    L_h = np.tril(host(L))
    errL = np.max(np.abs(L_h - L_np)) / np.max(np.abs(L_np))
    Y = X64 @ L_np
    B_ref = Y.T @ Y
    B_h = host(B).astype(np.float64)
    dg = np.sqrt(np.outer(np.diag(B_ref), np.diag(B_ref)))
    U = np.triu(np.ones((d_in, d_in), dtype=bool))
    errB = np.max(np.abs(B_h - B_ref)[U] / dg[U])
    assert np.all(np.tril(B_h, -1) == 0)
    out = lrc.lrc_eigh_multi([(B, k, None, None, None, Wd, True)], prec=prec)
    lam, V, info3 = (host(x) for x in out[0])
    assert int(info3[0]) == 0
    # the caller's factor in place of the library's own: the same values, so the same bits; and the
    # full covariance route with that factor equals the route without it
    outL = lrc.lrc_eigh_multi([(B, k, None, None, None, Wd, True, L)], prec=prec)
    assert int(host(outL[0][2])[0]) == 0
    assert np.array_equal(host(outL[0][0]), lam) and np.array_equal(host(outL[0][1]), V)
    eps = host(lrc.lrc_error_curve(torch.from_numpy(lam).cuda()))
    C = oracle.covariance(X, "bf16", W, "bf16")
    lam_r, V_r = oracle.eigh(C)
    e = check_lambda(lam, lam_r)
    assert np.all(np.diff(lam) <= 0) and np.count_nonzero(lam == 0.0) >= n - d_in
    eb, es = check_eps(eps, oracle.error_curve(lam_r), prec=prec)
    s = sin_theta_max(V, V_r, k)
    V64 = V.astype(np.float64)
    orth = np.max(np.abs(V64.T @ V64 - np.eye(k)))
    print("L err %.2e, B err %.2e (of sqrt(B_ii B_jj)), lambda err %.2e, eps err %.2e / tail %.2e, "
          "sin theta %.2e (gap %.2e), orthogonality %.2e" % (errL, errB, e, eb, es, s, gap(lam_r, k), orth))
    assert errL <= 1e-12 and errB <= 1e-5
    assert s <= 1e-3 and orth <= 1e-5
    idx = np.argmax(np.abs(V), axis=0)
    assert np.all(V[idx, np.arange(k)] > 0)


def test_cov_range_batched_members_and_dtypes(lrc):
    """Two projected members stacked in one group (B, W and L with strides) equal the members decomposed
    one by one, bit for bit; lrc_range_factor gives the same L from the bf16 weight and from its exact
    fp32 and fp64 widenings."""
    _say("projected members in one group: 2 x (2048 x 256 -> 448)")
    d_in, n, k = 256, 448, 40
    X = inputs.block_activations(d_in, 2048)
    Ws = [inputs.weight(d_in, n, "bf16", inputs.CFG_BLOCK, 0, 92 + i) for i in range(2)]
    Wd = torch.stack([dev(W, "bf16") for W in Ws])
    Xd = dev(X, "bf16")
    Ls, Bs = [], []
    for i in range(2):
        L, info = lrc.lrc_range_factor(Wd[i])
        assert int(host(info)[0]) == 0
        B = torch.zeros(d_in, d_in, dtype=torch.float32, device="cuda")
        assert int(host(lrc.lrc_cov_accumulate_range(Xd, L, B))[0]) == 0
        Ls.append(L)
        Bs.append(B)
        W64 = oracle.widen(Ws[i], "bf16")
        for w in (torch.from_numpy(W64.astype(np.float32)).cuda(), torch.from_numpy(W64).cuda()):
            L2, info2 = lrc.lrc_range_factor(w)
            assert int(host(info2)[0]) == 0
            assert torch.equal(torch.tril(L2), torch.tril(L))
    Bst, Lst = torch.stack(Bs), torch.stack(Ls)
    for prec in (1, 2):
        Ast = torch.empty(2, d_in, k, dtype=torch.float32, device="cuda")
        lam, V, info = lrc.lrc_eigh_multi([(Bst, k, None, None, None, Wd, True, Lst, Ast)], prec=prec)[0]
        assert np.all(host(info) == 0)
        for i in range(2):
            A1 = torch.empty(d_in, k, dtype=torch.float32, device="cuda")
            l1, V1, i1 = lrc.lrc_eigh_multi([(Bs[i], k, None, None, None, Wd[i], True, Ls[i], A1)], prec=prec)[0]
            assert int(host(i1)[0]) == 0
            assert torch.equal(l1, lam[i]) and torch.equal(V1, V[i]) and torch.equal(A1, Ast[i])
            # the factor A = W V = L U against the fp64 product of W and the returned V, and against
            # lrc_factorize's own A; B alone from lrc_factorize (A = NULL)
            W64 = oracle.widen(Ws[i], "bf16")
            Ar = W64 @ host(V[i]).astype(np.float64)
            Ah = host(Ast[i]).astype(np.float64)
            err = np.linalg.norm(Ah - Ar) / np.linalg.norm(Ar)
            A2 = torch.empty(d_in, k, dtype=torch.float32, device="cuda")
            lrc.lrc_factorize(Wd[i], V[i], k, A2, None)
            Bt2 = torch.empty(k, n, dtype=torch.float32, device="cuda")
            lrc.lrc_factorize(Wd[i], V[i], k, None, Bt2)
            err2 = np.linalg.norm(Ah - host(A2).astype(np.float64)) / np.linalg.norm(Ar)
            print("member %d prec %d: A from the decomposition vs W V %.2e, vs lrc_factorize %.2e" % (i, prec, err, err2))
            assert err <= 1e-6 and err2 <= 1e-6
            assert torch.equal(Bt2, V[i].T.contiguous())


@pytest.mark.parametrize("n_tok", [1, 37])
def test_cov_range_tiny_and_nonfinite(lrc, n_tok):
    """d_in = 160 (one partly filled 256-row block of the product, two 128-wide SYRK tiles) and 1 or 37
    tokens: B against (X L)^T (X L) in fp64; a NaN in X sets info 1."""
    d_in, n = 160, 300
    X = inputs.block_activations(d_in, 64)[:n_tok].copy()
    W = inputs.weight(d_in, n, "bf16", inputs.CFG_BLOCK, 0, 93)
    Wd = dev(W, "bf16")
    L, info = lrc.lrc_range_factor(Wd)
    assert int(host(info)[0]) == 0
    B = torch.zeros(d_in, d_in, dtype=torch.float32, device="cuda")
    assert int(host(lrc.lrc_cov_accumulate_range(dev(X, "bf16"), L, B))[0]) == 0
    Y = oracle.widen(X, "bf16") @ np.tril(host(L))
    B_ref = Y.T @ Y
    dg = np.sqrt(np.outer(np.diag(B_ref), np.diag(B_ref)))
    U = np.triu(np.ones((d_in, d_in), dtype=bool))
    err = np.max(np.abs(host(B).astype(np.float64) - B_ref)[U] / dg[U])
    assert err <= 1e-5, err
    Xn = X.copy()
    Xn[0, 5] = 0x7FC0  # bf16 NaN
    B2 = torch.zeros(d_in, d_in, dtype=torch.float32, device="cuda")
    assert int(host(lrc.lrc_cov_accumulate_range(dev(Xn, "bf16"), L, B2))[0]) == 1


def test_cov_range_rank_deficient_basis(lrc):
    """A weight whose rows are not independent: lrc_range_factor reports info 3."""
    W = inputs.weight(160, 400, "bf16", inputs.CFG_BLOCK, 0, 91)
    W[9] = W[4]
    L, info = lrc.lrc_range_factor(dev(W, "bf16"))
    assert int(host(info)[0]) == 3


def test_eigh_range_basis_fallbacks(lrc):
    """d_in >= n, or n_vec > d_in: the basis is ignored (the full decomposition, bit for bit); a basis
    without full row rank: info 3."""
    X = inputs.block_activations(200, 1024)
    W = inputs.weight(200, 180, "bf16", inputs.CFG_BLOCK, 0, 40)
    C = _oracle_cov32(X, "bf16", W)[0]
    l0, V0, _ = lrc.lrc_eigh(dev(C, "f32"), n_vec=20)
    l1, V1, i1 = lrc.lrc_eigh_multi([(dev(C, "f32"), 20, None, None, None, dev(W, "bf16"))])[0]
    assert int(host(i1)[0]) == 0
    assert np.array_equal(host(l0), host(l1)) and np.array_equal(host(V0), host(V1))
    W2 = inputs.weight(150, 300, "bf16", inputs.CFG_BLOCK, 0, 41)
    X2 = inputs.block_activations(150, 1024)
    C2 = _oracle_cov32(X2, "bf16", W2)[0]
    l0, V0, _ = lrc.lrc_eigh(dev(C2, "f32"), n_vec=160)
    l1, V1, i1 = lrc.lrc_eigh_multi([(dev(C2, "f32"), 160, None, None, None, dev(W2, "bf16"))])[0]
    assert np.array_equal(host(l0), host(l1)) and np.array_equal(host(V0), host(V1))
    W3 = W2.copy()
    W3[7] = W3[3]  # two equal rows: W W^T singular
    l3, V3, i3 = lrc.lrc_eigh_multi([(dev(C2, "f32"), 10, None, None, None, dev(W3, "bf16"))])[0]
    assert int(host(i3)[0]) == 3


def test_eigh_nonfinite_sets_info(lrc):
    C = np.eye(200, dtype=np.float32)
    C[3, 7] = np.inf
    lam, V, info = lrc.lrc_eigh(dev(C, "f32"), n_vec=4)
    assert int(host(info)[0]) == 1
    Cj = np.eye(32, dtype=np.float32)[None].repeat(2, 0)
    Cj[1, 0, 5] = np.nan
    lam, V, info = lrc.lrc_eigh(dev(Cj, "f32"), n_vec=4, prec=2)
    assert list(host(info)) == [0, 1]


def test_eigh_diagonal_and_repeated(lrc):
    _say("eigh diagonal with repeated eigenvalues")
    dvals = np.array([5.0] * 40 + [2.0] * 100 + [1.0] * 60, dtype=np.float32)
    perm = np.random.default_rng(0).permutation(200)
    C = np.diag(dvals[perm]).astype(np.float32)
    lam, V, info = lrc.lrc_eigh(dev(C, "f32"), n_vec=200)
    lam, V = host(lam), host(V).astype(np.float64)
    assert np.allclose(lam, np.sort(dvals)[::-1], atol=1e-5 * 5)
    assert np.max(np.abs(V.T @ V - np.eye(200))) <= 1e-5
    P = V[:, :40] @ V[:, :40].T  # projector onto the lambda = 5 eigenspace
    assert np.allclose(P, np.diag((dvals[perm] == 5).astype(float)), atol=1e-5)


# ---------------------------------------------------------------------------------------------
# error curve, factors, Fisher, allocation
# ---------------------------------------------------------------------------------------------

def test_error_curve_bitexact(lrc):
    _say("error curve")
    r = np.random.default_rng(1)
    lam = np.sort(r.exponential(1.0, (5, 777)), axis=1)[:, ::-1].copy()
    lam[:, -3:] = [1e-18, 0.0, -1e-17]
    eps = host(lrc.lrc_error_curve(dev(lam, "f64")))
    assert np.array_equal(eps, oracle.error_curve(lam))


@pytest.mark.parametrize("wdt", ["bf16", "f32"])
def test_factorize_matches_fp64_product(lrc, wdt):
    _say("factorize %s" % wdt)
    W = inputs.weight(520, 1376, wdt, inputs.CFG_BLOCK, 0, 5)
    Q, _ = np.linalg.qr(np.random.default_rng(2).standard_normal((1376, 300)))
    V = Q.astype(np.float32)
    k = 237
    A = torch.empty(520, k, dtype=torch.float32, device="cuda")
    B = torch.empty(k, 1376, dtype=torch.float32, device="cuda")
    lrc.lrc_factorize(dev(W, wdt), dev(V, "f32"), k, A, B)
    W64 = oracle.widen(W, wdt)
    ref = W64 @ V[:, :k].astype(np.float64)
    Ah = host(A).astype(np.float64)
    assert np.linalg.norm(Ah - ref) <= 1e-6 * np.linalg.norm(ref)
    assert np.array_equal(host(B), V[:, :k].T)
    # transposed weight (maps factors back through W^T): A = W^T V with V d_in x k
    V2 = np.linalg.qr(np.random.default_rng(3).standard_normal((520, 90)))[0].astype(np.float32)
    A2 = torch.empty(1376, 90, dtype=torch.float32, device="cuda")
    lrc.lrc_factorize(dev(W, wdt), dev(V2, "f32"), 90, A2, None, trans_w=1)
    ref2 = W64.T @ V2.astype(np.float64)
    assert np.linalg.norm(host(A2) - ref2) <= 1e-6 * np.linalg.norm(ref2)


@pytest.mark.parametrize("trans,vcols,wdt", [(0, 2850, "bf16"), (1, 2850, "bf16"), (0, 2852, "bf16"),
                                             (1, 2852, "bf16"), (0, 2852, "f32"), (1, 2852, "f64")])
def test_factorize_large_tiles(lrc, trans, vcols, wdt):
    """Products with at least 512 output tiles of 128 x 128 take the kernel's large-tile instance:
    2900 x 2850 outputs over a contraction of 2860 (ragged in every dimension), against the fp64
    product; a batch of two equals the members computed one by one, bit for bit.  V with 2852
    columns (rows 4-element aligned) takes the vector loads, with 2850 the element loads; W in bf16,
    fp32 and fp64 (the fp64 weight holds fp32 values, widened exactly)."""
    _say("factorize 128-wide tiles, trans_w %d, V with %d columns, W %s" % (trans, vcols, wdt))
    rows, red, k = 2900, 2860, 2850
    gen = "bf16" if wdt == "bf16" else "f32"
    W = inputs.weight(rows, red, gen, inputs.CFG_BLOCK, 0, 7) if trans == 0 else \
        inputs.weight(red, rows, gen, inputs.CFG_BLOCK, 0, 7)
    if wdt == "f64":
        W = W.astype(np.float64)
    V = np.random.default_rng(4).standard_normal((red, vcols)).astype(np.float32)
    A = torch.empty(rows, k, dtype=torch.float32, device="cuda")
    Wd, Vd = dev(W, wdt), dev(V, "f32")
    lrc.lrc_factorize(Wd, Vd, k, A, None, trans_w=trans)
    W64 = oracle.widen(W, wdt)
    ref = (W64 if trans == 0 else W64.T) @ V[:, :k].astype(np.float64)
    Ah = host(A).astype(np.float64)
    err = np.linalg.norm(Ah - ref) / np.linalg.norm(ref)
    print("relative Frobenius error %.2e" % err)
    assert err <= 1e-6
    # the fp64 product rounded once to fp32 (half an fp32 ulp), up to the order of the fp64 sums
    # (entries with heavy cancellation, below 1e-6 of the largest, left to the norm check)
    big = np.abs(ref) >= 1e-6 * np.abs(ref).max()
    assert np.max(np.abs(Ah - ref)[big] / np.abs(ref)[big]) <= 2.0 ** -23
    Wb, Vb = torch.stack([Wd, Wd.flip(0)]), torch.stack([Vd, Vd.flip(1)])
    Ab = torch.empty(2, rows, k, dtype=torch.float32, device="cuda")
    lrc.lrc_factorize(Wb, Vb, k, Ab, None, trans_w=trans, d_in=Wd.shape[0], d_out=Wd.shape[1], batch=2,
                      stride_w=Wd.numel(), stride_v=Vd.numel(), stride_a=rows * k)
    A1 = torch.empty(rows, k, dtype=torch.float32, device="cuda")
    lrc.lrc_factorize(Wb[1], Vb[1], k, A1, None, trans_w=trans)
    assert torch.equal(Ab[0], A) and torch.equal(Ab[1], A1)


def test_factorize_per_head_batch(lrc):
    _say("factorize per-head batch")
    W = inputs.weight(512, 512, "bf16", inputs.CFG_HEADS, 0, 0)
    Vh = np.stack([np.linalg.qr(np.random.default_rng(10 + h).standard_normal((128, 128)))[0]
                   for h in range(4)]).astype(np.float32)
    k = 32
    A = torch.empty(4, 512, k, dtype=torch.float32, device="cuda")
    B = torch.empty(4, k, 128, dtype=torch.float32, device="cuda")
    Wd = dev(W, "bf16")
    lrc.lrc_factorize(Wd, dev(Vh, "f32"), k, A, B, d_in=512, d_out=128, batch=4, stride_w=128,
                      stride_v=128 * 128, stride_a=512 * k, stride_b=k * 128)
    W64 = oracle.widen(W, "bf16")
    Ah = host(A)
    for h in range(4):
        ref = W64[:, 128 * h:128 * h + 128] @ Vh[h][:, :k].astype(np.float64)
        assert np.linalg.norm(Ah[h] - ref) <= 1e-6 * np.linalg.norm(ref)
        assert np.array_equal(host(B)[h], Vh[h][:, :k].T)


def test_fisher_scores(lrc):
    _say("fisher")
    shapes = [(37, 41), (256, 128), (1000, 333), (1, 1), (2048, 4096)]
    Gs, Ws = [], []
    for i, (a, b) in enumerate(shapes):
        Gs.append(inputs.gradient(a, b, 1e-4, inputs.CFG_STACK, 0, i))
        Ws.append(inputs.weight(a, b, "bf16", inputs.CFG_STACK, 0, i))
    alpha, info = lrc.lrc_fisher_scores([dev(g, "bf16") for g in Gs], [dev(w, "bf16") for w in Ws])
    alpha, info = host(alpha), host(info)
    for i in range(len(shapes)):
        ref = oracle.fisher(Gs[i], Ws[i])
        assert abs(alpha[i] - ref) <= 1e-12 * ref, i
        assert info[i] == 0
    # unaligned view (offset by one element) goes through the scalar path
    G0 = dev(Gs[4], "bf16").reshape(-1)[1:]
    W0 = dev(Ws[4], "bf16").reshape(-1)[1:]
    a1, _ = lrc.lrc_fisher_scores([G0], [W0])
    ref = oracle.fisher(Gs[4].reshape(-1)[1:], Ws[4].reshape(-1)[1:])
    assert abs(host(a1)[0] - ref) <= 1e-12 * ref
    # fp32 inputs
    g32 = np.random.default_rng(4).standard_normal(5000).astype(np.float32)
    w32 = np.random.default_rng(5).standard_normal(5000).astype(np.float32)
    a2, _ = lrc.lrc_fisher_scores([dev(g32, "f32")], [dev(w32, "f32")])
    ref = float(np.sum((g32.astype(np.float64) * w32.astype(np.float64)) ** 2))
    assert abs(host(a2)[0] - ref) <= 1e-12 * ref


def test_fisher_nonfinite(lrc):
    g = inputs.f32_to_bf16_bits(np.array([1.0, np.inf, 2.0], np.float32))
    w = inputs.f32_to_bf16_bits(np.array([1.0, 1.0, 2.0], np.float32))
    _, info = lrc.lrc_fisher_scores([dev(g, "bf16")], [dev(w, "bf16")])
    assert int(host(info)[0]) == 1


def _alloc_gpu(lrc, alpha, lams, eps0, cost, budget, k_min=None):
    offs = np.concatenate([[0], np.cumsum([len(l) for l in lams])]).astype(np.int64)
    lp = np.concatenate([np.asarray(l, dtype=np.float64) for l in lams]) if offs[-1] else np.zeros(0)
    km = None if k_min is None else dev(np.asarray(k_min, dtype=np.int32), "i32")
    k, info = lrc.lrc_allocate_ranks(dev(np.asarray(alpha, np.float64), "f64"), dev(lp, "f64"),
                                     dev(offs, "i64"), dev(np.asarray(eps0, np.float64), "f64"),
                                     dev(np.asarray(cost, np.int64), "i64"), budget, k_min=km)
    return host(k), int(host(info)[0])


def test_allocate_worked_example(lrc):
    ex = json.load(open(os.path.join(GOLDEN, "alloc_worked_example.json")))
    ms = ex["matrices"]
    args = ([m["alpha"] for m in ms], [m["lam"] for m in ms], [m["eps0"] for m in ms], [m["cost"] for m in ms])
    for case in ex["cases"]:
        k, info = _alloc_gpu(lrc, *args, case["budget"], case["k_min"])
        assert info == case["info"] and list(k) == case["k"], case


def test_allocate_bitexact_random_with_ties(lrc):
    _say("allocation random")
    r = np.random.default_rng(7)
    for trial in range(40):
        M = int(r.integers(1, 12))
        lams = []
        for m in range(M):
            K = int(r.integers(0, 60))
            if trial % 3 == 0:  # many exact ties
                l = np.sort(r.choice([0.0, 0.5, 1.0, 2.0, -1e-9], K))[::-1]
            else:
                l = np.sort(r.exponential(1.0, K))[::-1]
            lams.append(l)
        alpha = r.choice([0.0, 1.0, 3.0], M) if trial % 3 == 0 else r.exponential(1.0, M)
        eps0 = [float(np.sum(np.maximum(l, 0))) for l in lams]
        cost = r.integers(1, 9, M)
        k_min = [int(r.integers(0, len(l) + 1)) if r.random() < 0.3 else 0 for l in lams]
        total = int(sum(len(l) * c for l, c in zip(lams, cost)))
        for budget in (0, total // 3, total // 2 + 1, total, total + 5):
            kg, ig = _alloc_gpu(lrc, alpha, lams, eps0, cost, budget, k_min)
            ko, io = oracle.allocate_ranks(alpha, lams, eps0, cost, budget, k_min)
            assert ig == io and list(kg) == list(ko), (trial, budget)


def test_allocate_bad_scores(lrc):
    k, info = _alloc_gpu(lrc, [1.0, np.nan], [[1.0, 0.5], [2.0]], [1.5, 2.0], [3, 3], 100)
    assert info == 5
    k, info = _alloc_gpu(lrc, [1.0, 1.0], [[1.0, 0.5], [2.0]], [1.5, -2.0], [3, 3], 100)
    assert info == 5


# ---------------------------------------------------------------------------------------------
# the whole path, end to end
# ---------------------------------------------------------------------------------------------

def _pipeline(lrc, X, xdt, W, k, n_blocks=1, prec=1):
    """cov -> eigh -> error curve -> factorize on the GPU; returns host arrays."""
    C = _cov_gpu(lrc, X, xdt, W, n_blocks=n_blocks)
    d_out = W.shape[1]
    hd = d_out // n_blocks
    if n_blocks == 1:
        lam, V, info = lrc.lrc_eigh(C, n_vec=k, prec=prec)
        lam, V = lam[None], V[None]
    else:  # n <= 128: the batched Jacobi path, in fp64 whatever prec says
        lam, V, info = lrc.lrc_eigh(C, n_vec=k, prec=prec)
    assert np.all(host(info) == 0)
    eps = lrc.lrc_error_curve(lam)
    A = torch.empty(n_blocks, W.shape[0], k, dtype=torch.float32, device="cuda")
    B = torch.empty(n_blocks, k, hd, dtype=torch.float32, device="cuda")
    lrc.lrc_factorize(dev(W, xdt), V, k, A, B, d_in=W.shape[0], d_out=hd, batch=n_blocks, stride_w=hd,
                      stride_v=hd * k, stride_a=W.shape[0] * k, stride_b=k * hd)
    Ch = host(C)
    return host(lam), host(V), host(eps), host(A), host(B), (Ch[None] if n_blocks == 1 else Ch)


def _check_pipeline(X, xdt, W, k, lam, V, eps, A, B, n_blocks=1, C_gpu=None, prec=1):
    C = oracle.covariance(X, xdt, W, xdt, n_blocks=n_blocks)
    C = C[None] if n_blocks == 1 else C
    W64 = oracle.widen(W, xdt)
    X64 = oracle.widen(X, xdt)
    hd = W.shape[1] // n_blocks
    for h in range(n_blocks):
        lam_r, V_r = oracle.eigh(C[h])
        eps_r = oracle.error_curve(lam_r)
        if C_gpu is not None:  # diagnostic: the accumulation's share of the error (LAPACK on the GPU's C)
            Cg = np.triu(C_gpu[h]).astype(np.float64)
            lg = np.linalg.eigvalsh(Cg + np.triu(Cg, 1).T)[::-1]
            eg = oracle.error_curve(lg)
            big = eps_r >= 1e-4 * eps_r[0]
            print("head %d accumulation only: eps rel %.2e, tail %.2e eps_0" % (
                h, np.max(np.abs(eg[big] - eps_r[big]) / eps_r[big]),
                np.max(np.abs(eg[~big] - eps_r[~big])) / eps_r[0] if (~big).any() else 0.0))
        el = check_lambda(lam[h], lam_r)
        s = sin_theta_max(V[h], V_r, k)
        Wh = W64[:, h * hd:(h + 1) * hd]
        # the GPU factors reach the closed-form error: ||X W - X A B||^2 = eps_k (test-side fp64)
        R = X64 @ (Wh - A[h].astype(np.float64) @ B[h].astype(np.float64))
        direct = float(np.sum(R * R))
        big = eps_r >= 1e-4 * eps_r[0]
        print("head %d: lambda %.2e, eps rel %.2e, tail %.2e eps_0, sin theta %.2e (gap %.2e), direct/eps_k - 1 = %.2e"
              % (h, el, np.max(np.abs(eps[h][big] - eps_r[big]) / eps_r[big]),
                 np.max(np.abs(eps[h][~big] - eps_r[~big])) / eps_r[0] if (~big).any() else 0.0, s, gap(lam_r, k),
                 direct / eps_r[k] - 1))
        check_eps(eps[h], eps_r, prec=prec)
        assert s <= 1e-3
        assert abs(direct - eps_r[k]) <= 1e-4 * eps_r[k] + 1e-6 * eps_r[0]


@pytest.mark.parametrize("prec", [1, 2])
def test_pipeline_single_layer(lrc, prec):
    _say("pipeline single layer 2048 x 256 -> 256, k = 64, prec %d" % prec)
    d = inputs.single_layer()
    out = _pipeline(lrc, d["X"], "f32", d["W"], 64, prec=prec)
    _check_pipeline(d["X"], "f32", d["W"], 64, *out[:5], C_gpu=out[5], prec=prec)


@pytest.mark.parametrize("prec", [1, 2])
def test_pipeline_block_scaled(lrc, prec):
    _say("pipeline scaled block 16384 x 512 -> 640, prec %d" % prec)
    X = inputs.block_activations(512, 16384)
    W = inputs.weight(512, 640, "bf16", inputs.CFG_BLOCK, 0, 0)
    k = inputs.rank_at_ratio(512, 640, 0.6)
    out = _pipeline(lrc, X, "bf16", W, k, prec=prec)
    _check_pipeline(X, "bf16", W, k, *out[:5], C_gpu=out[5], prec=prec)


def test_pipeline_per_head_scaled(lrc):
    _say("pipeline per-head 8192 x 512, 4 heads of 128, k = 32")
    d = inputs.per_head(n_tok=8192, d_model=512, head_dim=128)
    out = _pipeline(lrc, d["X"], "bf16", d["W"], 32, n_blocks=4)  # default prec: the Jacobi path is fp64
    _check_pipeline(d["X"], "bf16", d["W"], 32, *out[:5], n_blocks=4, C_gpu=out[5], prec=2)


def test_allocate_proportional_bitexact(lrc):
    """FLRC proportional ranks (and a non-increasing budget schedule) bit-exact against the oracle:
    224 lognormal importances with repeated values (ties), 7 importances, and bad scores (info 5)."""
    _say("allocate proportional: 224 and 7 matrices, 6 budgets")
    rng = np.random.default_rng(11)
    a224 = rng.lognormal(0.0, 2.0, size=224)
    a224[10:20] = a224[5]  # ties in the remainders
    budgets = np.array([500000, 400000, 123457, 2241, 7, 0], dtype=np.int64)
    for a in (a224, np.array([3.0, 1.0, 4.0, 1.0, 5.0, 9.0, 2.0])):
        r, info = lrc.lrc_allocate_proportional(dev(a.astype(np.float64), "f64"), dev(budgets, "i64"))
        r_o, info_o = oracle.allocate_proportional(a, budgets.tolist())
        assert int(host(info)[0]) == info_o == 0
        assert np.array_equal(host(r), r_o)
        assert np.array_equal(host(r).sum(axis=1), budgets)
    r, info = lrc.lrc_allocate_proportional(dev(np.array([1.0, -2.0, 3.0]), "f64"), dev(budgets, "i64"))
    assert int(host(info)[0]) == 5 and np.all(host(r) == 0)
