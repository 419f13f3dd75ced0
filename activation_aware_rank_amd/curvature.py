"""Curvature-weighted truncation (LASER page, "LASER: Loss-Aware Singular-value Decomposition
and Rank Allocation", method 1), composed from liblrc entry points on one stream.

With X the calibration activations (N x d_in) and G the gradients of the layer output Y = X W
(N x d_out), the loss increase of a weight change dW is approximated through the Kronecker-
factored curvature Sigma_g (x) Sigma_x, Sigma_x = X^T X / N, Sigma_g = G^T G / N.  With lower
Cholesky factors Sigma = L L^T the weight moves to W~ = L_x^T W L_g, whose truncated SVD is the
optimum in that metric; the left singular vectors U come from the eigenvectors of W~ W~^T, and the
truncation maps back to W_k = A B with

    A = L_x^{-T} U_k          (d_in x k),
    B = U_k^T L_x^T W         (k x d_out),

so that L_x^T (W - W_k) L_g = (I - U_k U_k^T) W~ and its squared Frobenius norm is the sum of the
discarded eigenvalues of W~ W~^T.  (The page writes the factors with S_k^{+-1} split between them;
the product A B is the same.)

Only buffer allocation and call order live here; every arithmetic step runs in liblrc's kernels.
"""
from __future__ import annotations

import torch

from . import lrc


def curvature_truncation(X: torch.Tensor, G: torch.Tensor, W: torch.Tensor, k: int, prec: int = lrc.LRC_F64,
                         stream=None, marks: list | None = None) -> dict:
    """Run the chain on device tensors X (N x d_in), G (N x d_out), W (d_in x d_out).

    Returns a dict of device tensors: Lx, Lg (fp64 lower factors), W1 = L_x^T W (fp64),
    Wt = W~ (fp64), lam (fp64, eigenvalues of W~ W~^T descending), U (fp32 d_in x k),
    A (fp64 d_in x k), Bt (fp32 d_out x k, B transposed) and info (int32 per step:
    cov_x, cov_g, chol_x, chol_g, eigh).  With a list ``marks``, a (stage, torch.cuda.Event) pair is
    appended after each stage (recorded on the stream used).
    """
    n_tok, d_in = X.shape
    d_out = W.shape[1]
    if G.shape != (n_tok, d_out) or W.shape[0] != d_in:
        raise ValueError("X (N x d_in), G (N x d_out) and W (d_in x d_out) disagree")
    st = stream if stream is not None else torch.cuda.current_stream()
    with torch.cuda.stream(st):  # torch's own allocations and fills go to the same stream
        return _chain(X, G, W, k, prec, st, marks)


def _chain(X, G, W, k, prec, st, marks):
    n_tok, d_in = X.shape
    d_out = W.shape[1]
    dev = X.device
    stream = st

    def mark(name):
        if marks is not None:
            e = torch.cuda.Event(enable_timing=True)
            e.record(st)
            marks.append((name, e))

    mark("start")
    info = torch.zeros(5, dtype=torch.int32, device=dev)
    Cx = torch.zeros(d_in, d_in, dtype=torch.float32, device=dev)
    Cg = torch.zeros(d_out, d_out, dtype=torch.float32, device=dev)
    lrc.lrc_cov_accumulate(X, None, Cx, info=info[0:1], stream=stream)
    lrc.lrc_cov_accumulate(G, None, Cg, info=info[1:2], stream=stream)
    Lx = lrc.lrc_sym_to_f64(Cx, 1.0 / n_tok, stream=stream)
    Lg = lrc.lrc_sym_to_f64(Cg, 1.0 / n_tok, stream=stream)
    del Cx, Cg
    mark("covariances")
    lrc.lrc_cholesky(Lx, info=info[2:3], stream=stream)
    lrc.lrc_cholesky(Lg, info=info[3:4], stream=stream)
    mark("cholesky")
    W1 = lrc.lrc_to_f64(W, stream=stream)
    lrc.lrc_trmm(0, 1, Lx, W1, stream=stream)            # W1 = L_x^T W
    Wt = lrc.lrc_to_f64(W1, stream=stream)
    lrc.lrc_trmm(1, 0, Lg, Wt, stream=stream)            # W~ = L_x^T W L_g
    mark("whiten")
    M = lrc.lrc_gram_f64(Wt, stream=stream)              # upper of W~ W~^T
    mark("gram")
    lam, U, _ = lrc.lrc_eigh(M, k, prec, info=info[4:5], stream=stream)
    del M
    mark("eigh")
    A = lrc.lrc_to_f64(U, stream=stream)
    lrc.lrc_trsm(0, 1, Lx, A, stream=stream)             # A = L_x^{-T} U_k
    Bt = torch.empty(d_out, k, dtype=torch.float32, device=dev)
    lrc.lrc_factorize(W1, U, k, Bt, trans_w=1, stream=stream)  # B^T = W1^T U_k
    mark("map_back")
    return {"Lx": Lx, "Lg": Lg, "W1": W1, "Wt": Wt, "lam": lam, "U": U, "A": A, "Bt": Bt, "info": info}
