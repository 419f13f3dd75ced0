"""Thin ctypes binding of liblrc (include/lrc.h), with the same entry-point names.

Only argument marshalling happens here: tensors are checked for device, dtype and layout, their
data pointers, leading dimensions and torch's current stream are passed to the C ABI, and
workspace is allocated as a torch uint8 tensor.  Every computation runs in the HIP kernels of
liblrc.so.  Importing this module fails loudly when the library has not been built.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblrc.so")

if not os.path.exists(LIB_PATH):
    raise ImportError("liblrc.so is not built; run `python -m activation_aware_rank_amd.build` "
                      "(or __graft_entry__.build()) first")

_lib = ctypes.CDLL(LIB_PATH)

LRC_BF16, LRC_F32, LRC_F64 = 0, 1, 2
STATUS = {0: "LRC_OK", 1: "LRC_ERR_ARG", 2: "LRC_ERR_DTYPE", 3: "LRC_ERR_WORKSPACE", 4: "LRC_ERR_HIP",
          5: "LRC_ERR_UNIMPLEMENTED"}
INFO = {0: "ok", 1: "non-finite input", 2: "no convergence", 3: "not positive definite",
        4: "mandatory ranks exceed the budget", 5: "negative or NaN score"}

_vp, _i64, _i32, _sz, _int = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t, ctypes.c_int


def _sig(name, res, *args):
    f = getattr(_lib, name)
    f.restype = res
    f.argtypes = list(args)
    return f


_abi = _sig("lrc_abi_version", _int)
_status_string = _sig("lrc_status_string", ctypes.c_char_p, _int)
_last_error = _sig("lrc_last_error", ctypes.c_char_p)
_cov_ws = _sig("lrc_cov_accumulate_workspace", _sz, _int, _i64, _i64, _int, _i64, _i32)
_cov = _sig("lrc_cov_accumulate", _int, _vp, _int, _i64, _i64, _i64, _vp, _int, _i64, _i64, _i32, _vp, _i64, _vp, _sz,
            _vp, _vp)
_eigh_ws = _sig("lrc_eigh_workspace", _sz, _i64, _i64, _i64, _int)
_eigh = _sig("lrc_eigh", _int, _vp, _i64, _i64, _i64, _i64, _int, _vp, _vp, _i64, _i64, _i64, _vp, _sz, _vp, _vp)
_err = _sig("lrc_error_curve", _int, _vp, _i64, _i64, _vp, _vp)
_fac = _sig("lrc_factorize", _int, _vp, _int, _i32, _i64, _i64, _i64, _vp, _i64, _i64, _i64, _i64, _i64, _vp, _i64,
            _i64, _vp, _i64, _i64, _vp)
_fsh_ws = _sig("lrc_fisher_scores_workspace", _sz, _i32, _vp)
_fsh = _sig("lrc_fisher_scores", _int, _i32, _vp, _vp, _vp, _int, _vp, _vp, _sz, _vp, _vp)
_fsh_na = _sig("lrc_fisher_scores_noalloc", _int, _i32, _vp, _vp, _vp, _int, _vp, _vp, _vp)
_alc_ws = _sig("lrc_allocate_ranks_workspace", _sz, _i32, _i64)
_alc = _sig("lrc_allocate_ranks", _int, _i32, _vp, _vp, _vp, _i64, _vp, _vp, _vp, _i64, _vp, _vp, _sz, _vp, _vp)
_chol_ws = _sig("lrc_cholesky_workspace", _sz, _i64)
_chol = _sig("lrc_cholesky", _int, _vp, _i64, _i64, _vp, _sz, _vp, _vp)
_trmm_ws = _sig("lrc_trmm_workspace", _sz, _i64, _i64)
_trmm = _sig("lrc_trmm", _int, _i32, _i32, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _sz, _vp)
_trsm_ws = _sig("lrc_trsm_workspace", _sz, _i32, _i64, _i64)
_trsm = _sig("lrc_trsm", _int, _i32, _i32, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _sz, _vp)
_sym64 = _sig("lrc_sym_to_f64", _int, _vp, _i64, _i64, ctypes.c_double, _vp, _i64, _vp)
_to64 = _sig("lrc_to_f64", _int, _vp, _int, _i64, _i64, _i64, ctypes.c_double, _vp, _i64, _vp)
_gram64 = _sig("lrc_gram_f64", _int, _vp, _i64, _i64, _i64, _vp, _i64, _vp)
_cfi_ws = _sig("lrc_cov_from_input_workspace", _sz, _i64, _i64)
_aprop = _sig("lrc_allocate_proportional", _int, _i32, _vp, _i32, _vp, _vp, _vp, _vp)
_cfi = _sig("lrc_cov_from_input", _int, _vp, _i64, _i64, _vp, _int, _i64, _i64, _vp, _i64, _vp, _sz, _vp)
_aswift = _sig("lrc_allocate_swift", _int, _i32, _vp, _vp, _vp, _vp, _vp, ctypes.c_double, _i32, _vp, _i64, _vp, _vp,
               _vp, _vp)
_cfsh_ws = _sig("lrc_component_fisher_workspace", _sz, _i64, _i64, _i64)
_cfsh = _sig("lrc_component_fisher", _int, _vp, _vp, _int, _i64, _i64, _i64, _i64, _vp, _i64, _i64, _i64, _i64, _i64,
             _i64, _vp, _i64, _vp, _sz, _vp)
_acomp_ws = _sig("lrc_allocate_components_workspace", _sz, _i32, _i64)
_acomp = _sig("lrc_allocate_components", _int, _i32, _vp, _vp, _i64, _vp, _vp, _i64, _vp, _vp, _vp, _sz, _vp, _vp)
_rfac_ws = _sig("lrc_range_factor_workspace", _sz, _i64, _i64)
_rfac = _sig("lrc_range_factor", _int, _vp, _int, _i64, _i64, _i64, _vp, _i64, _vp, _sz, _vp, _vp)
_covr_ws = _sig("lrc_cov_accumulate_range_workspace", _sz, _i64, _i64)
_covr = _sig("lrc_cov_accumulate_range", _int, _vp, _int, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _sz, _vp, _vp)
_tim_en = _sig("lrc_timing_enable", _int, _int)
_tim_st = _sig("lrc_timing_set_stride", _int, ctypes.c_char_p, _int)
_tim_rd = _sig("lrc_timing_read", _int, ctypes.c_char_p, ctypes.POINTER(ctypes.c_int64),
               ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double), _int)

EXPORTED = ("lrc_abi_version", "lrc_status_string", "lrc_last_error", "lrc_cov_accumulate_workspace",
            "lrc_cov_accumulate", "lrc_eigh_workspace", "lrc_eigh", "lrc_eigh_multi_workspace", "lrc_eigh_multi",
            "lrc_error_curve", "lrc_factorize",
            "lrc_fisher_scores_workspace", "lrc_fisher_scores", "lrc_fisher_scores_noalloc",
            "lrc_allocate_ranks_workspace",
            "lrc_allocate_ranks", "lrc_cholesky_workspace", "lrc_cholesky", "lrc_trmm_workspace", "lrc_trmm",
            "lrc_trsm_workspace", "lrc_trsm", "lrc_sym_to_f64", "lrc_to_f64", "lrc_gram_f64",
            "lrc_cov_from_input_workspace", "lrc_cov_from_input", "lrc_allocate_proportional",
            "lrc_allocate_swift", "lrc_component_fisher_workspace", "lrc_component_fisher",
            "lrc_allocate_components_workspace", "lrc_allocate_components",
            "lrc_range_factor_workspace", "lrc_range_factor", "lrc_cov_accumulate_range_workspace",
            "lrc_cov_accumulate_range", "lrc_timing_enable", "lrc_timing_set_stride", "lrc_timing_read")


class LrcError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__("%s: %s" % (STATUS.get(code, str(code)), msg))
        self.code = code


def _check(code: int):
    if code != 0:
        raise LrcError(code, (_last_error() or b"").decode())


def lrc_abi_version() -> int:
    return _abi()


def lrc_status_string(code: int) -> str:
    return _status_string(code).decode()


def lrc_last_error() -> str:
    return (_last_error() or b"").decode()


# ----------------------------------------------------------------------------------------------
# marshalling helpers
# ----------------------------------------------------------------------------------------------
_DT = {torch.bfloat16: LRC_BF16, torch.float32: LRC_F32, torch.float64: LRC_F64}


def _dt(t: torch.Tensor) -> int:
    if t.dtype not in _DT:
        raise TypeError("unsupported dtype %s" % t.dtype)
    return _DT[t.dtype]


def _dev(t: torch.Tensor, name: str):
    if not t.is_cuda:
        raise ValueError("%s must be a GPU tensor" % name)


def _rows(t: torch.Tensor, name: str) -> int:
    """Leading dimension of a matrix (or batch of matrices) with a contiguous last axis."""
    _dev(t, name)
    if t.dim() < 2 or t.stride(-1) != 1:
        raise ValueError("%s must be a matrix with a contiguous last dimension" % name)
    return t.stride(-2)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _workspace(nbytes: int, device, ws=None):
    if nbytes == 0:
        return None, 0
    if ws is not None and ws.numel() >= nbytes:
        return ws, ws.numel()
    return torch.empty(nbytes, dtype=torch.uint8, device=device), nbytes


def _info(info, n, device):
    if info is None:
        info = torch.empty(n, dtype=torch.int32, device=device)
    if info.dtype != torch.int32 or info.numel() < n:
        raise ValueError("info must be int32 with at least %d entries" % n)
    return info


# ----------------------------------------------------------------------------------------------
# entry points
# ----------------------------------------------------------------------------------------------
def lrc_cov_accumulate_workspace(x_dtype: int, n_tok: int, d_in: int, has_w: bool, d_out: int, n_blocks: int = 1) -> int:
    return _cov_ws(x_dtype, n_tok, d_in, int(bool(has_w)), d_out, n_blocks)


def lrc_cov_accumulate(X: torch.Tensor, W: torch.Tensor | None, C: torch.Tensor, n_blocks: int = 1, info=None,
                       ws=None, stream=None) -> torch.Tensor:
    """C[upper] += (X W)^T (X W).  X (n_tok, d_in); W (d_in, d_out) or None; C (d_out, d_out) fp32,
    or (n_blocks, hd, hd) for the per-head diagonal blocks.  Returns the int32 info tensor."""
    ldx = _rows(X, "X")
    n_tok, d_in = X.shape
    if W is not None:
        ldw = _rows(W, "W")
        d_out = W.shape[1]
        wt = _dt(W)
    else:
        ldw, d_out, wt = 0, d_in, _dt(X)
    ldc = _rows(C, "C")
    if C.dtype != torch.float32:
        raise TypeError("C must be float32")
    nbytes = lrc_cov_accumulate_workspace(_dt(X), n_tok, d_in, W is not None, d_out, n_blocks)
    w, wn = _workspace(nbytes, X.device, ws)
    info = _info(info, 1, X.device)
    _check(_cov(_ptr(X), _dt(X), n_tok, d_in, ldx, _ptr(W), wt, d_out, ldw, n_blocks, _ptr(C), ldc, _ptr(w), wn,
                _ptr(info), _stream(stream)))
    return info


def lrc_eigh_workspace(n: int, batch: int, n_vec: int, prec: int = LRC_F32) -> int:
    return _eigh_ws(n, batch, n_vec, prec)


class _EighGroup(ctypes.Structure):
    """struct lrc_eigh_group of include/lrc.h."""
    _fields_ = [("C", _vp), ("n", _i64), ("ldc", _i64), ("batch", _i64), ("stride_c", _i64), ("lambda_", _vp),
                ("V", _vp), ("ldv", _i64), ("n_vec", _i64), ("stride_v", _i64), ("info", _vp),
                ("W", _vp), ("w_t", _int), ("d_in", _i64), ("ldw", _i64), ("stride_w", _i64),
                ("projected", _i32), ("L", _vp), ("ldl", _i64), ("stride_l", _i64),
                ("A", _vp), ("lda", _i64), ("stride_a", _i64)]


_eigh_mws = _sig("lrc_eigh_multi_workspace", _sz, ctypes.POINTER(_EighGroup), _i32, _int)
_eigh_m = _sig("lrc_eigh_multi", _int, ctypes.POINTER(_EighGroup), _i32, _int, _vp, _sz, _vp)


def _eigh_args(C, n_vec, lam, V, info, W=None, projected=False, L=None, A=None):
    """Marshals one lrc_eigh call (W: the optional range basis of lrc_eigh_multi, d_in x n or
    batch x d_in x n; projected: C is B = Q^T C Q, d_in x d_in): (struct, squeeze flag, lam, V,
    info)."""
    ldc = _rows(C, "C")
    squeeze = C.dim() == 2
    Cb = C.unsqueeze(0) if squeeze else C
    batch, n = Cb.shape[0], Cb.shape[1]
    if projected:
        if W is None:
            raise ValueError("a projected group needs its range basis W")
        n = W.shape[-1]
    dev = C.device
    if lam is None:
        lam = torch.empty(batch, n, dtype=torch.float64, device=dev)
    if V is None and n_vec > 0:
        V = torch.empty(batch, n, n_vec, dtype=torch.float32, device=dev)
    if squeeze:  # a caller's lam (n,) and V (n, n_vec) for a single matrix, as batches of one (views)
        if lam.dim() == 1:
            lam = lam.unsqueeze(0)
        if V is not None and V.dim() == 2:
            V = V.unsqueeze(0)
    ldv = _rows(V, "V") if V is not None else max(n_vec, 1)
    stride_v = (V.stride(0) if V.dim() == 3 else 0) if V is not None else 0
    info = _info(info, batch, dev)
    g = _EighGroup(_ptr(C), n, ldc, batch, Cb.stride(0), _ptr(lam), _ptr(V), ldv, n_vec, stride_v, _ptr(info))
    if W is not None:
        g.W, g.w_t, g.d_in, g.ldw = _ptr(W), _dt(W), W.shape[-2], _rows(W, "W")
        g.stride_w = W.stride(0) if W.dim() == 3 else 0
        g.projected = int(bool(projected))
        if L is not None:
            g.L, g.ldl = _ptr(L), _f64_matrix(L, "L")
            g.stride_l = L.stride(0) if L.dim() == 3 else 0
        if A is not None:
            if A.dtype != torch.float32:
                raise TypeError("A must be float32")
            g.A, g.lda = _ptr(A), _rows(A, "A")
            g.stride_a = A.stride(0) if A.dim() == 3 else 0
    return g, squeeze, lam, V, info


def _eigh_out(squeeze, lam, V, info):
    if squeeze:
        return lam[0], (V[0] if V is not None else None), info
    return lam, V, info


def lrc_eigh(C: torch.Tensor, n_vec: int, prec: int = LRC_F32, lam=None, V=None, info=None, ws=None, stream=None):
    """Eigenpairs of the symmetric fp32 matrix (or batch) C, upper triangle read.
    Returns (lambda fp64 (batch, n) descending, V fp32 (batch, n, n_vec), info int32 (batch,))."""
    g, squeeze, lam, V, info = _eigh_args(C, n_vec, lam, V, info)
    nbytes = lrc_eigh_workspace(g.n, g.batch, n_vec, prec)
    w, wn = _workspace(nbytes, C.device, ws)
    _check(_eigh(g.C, g.n, g.ldc, g.batch, g.stride_c, prec, g.lambda_, g.V, g.ldv, n_vec, g.stride_v, _ptr(w), wn,
                 g.info, _stream(stream)))
    return _eigh_out(squeeze, lam, V, info)


def lrc_eigh_multi_workspace(groups, prec: int = LRC_F32) -> int:
    """groups: sequence of (n, batch, n_vec), (n, batch, n_vec, d_in) for a group with a range basis
    of d_in rows (only its presence and d_in matter for the size) or (n, batch, n_vec, d_in, projected)."""
    gs = []
    for grp in groups:
        n, b, nv = grp[:3]
        g = _EighGroup(None, n, n, b, 0, None, None, nv, nv, 0, None)
        if len(grp) > 3 and grp[3]:
            g.W, g.d_in, g.ldw = 1, grp[3], n  # any non-NULL pointer: the query reads no memory
            g.projected = int(bool(grp[4])) if len(grp) > 4 else 0
        gs.append(g)
    arr = (_EighGroup * len(gs))(*gs)
    return _eigh_mws(arr, len(gs), prec)


def lrc_eigh_multi(groups, prec: int = LRC_F32, ws=None, stream=None):
    """Several lrc_eigh calls in one.  groups: sequence of (C, n_vec), (C, n_vec, lam, V, info),
    (C, n_vec, lam, V, info, W), (C, n_vec, lam, V, info, W, projected) or (..., projected, L) with
    the meaning of lrc_eigh's arguments; W is the optional range basis (d_in x n, or batch x d_in x
    n: C = (X W)^T (X W)); projected: C is B = Q^T C Q (d_in x d_in) from lrc_cov_accumulate_range;
    L: the factor of W W^T from lrc_range_factor (d_in x d_in, or batch x d_in x d_in); an optional
    ninth element A (d_in x n_vec fp32, or batched) of a projected group receives W V = L U.  Returns a
    list of (lambda, V, info) per group."""
    parts = []
    for grp in groups:
        C, n_vec = grp[0], grp[1]
        lam, V, info, W, pj, L, A = (tuple(grp[2:9]) + (None, None, None, None, False, None, None))[:7]
        parts.append(_eigh_args(C, n_vec, lam, V, info, W, bool(pj), L, A))
    if not parts:
        raise ValueError("lrc_eigh_multi needs at least one group")
    arr = (_EighGroup * len(parts))(*[p[0] for p in parts])
    nbytes = _eigh_mws(arr, len(parts), prec)
    w, wn = _workspace(nbytes, groups[0][0].device, ws)
    _check(_eigh_m(arr, len(parts), prec, _ptr(w), wn, _stream(stream)))
    return [_eigh_out(*p[1:]) for p in parts]


def lrc_range_factor_workspace(d_in: int, n: int) -> int:
    return _rfac_ws(d_in, n)


def lrc_range_factor(W: torch.Tensor, L=None, info=None, ws=None, stream=None):
    """L (d_in, d_in) fp64 with W W^T = L L^T (lower triangle written) for W (d_in, n), n >= d_in.
    Returns (L, info)."""
    ldw = _rows(W, "W")
    d_in, n = W.shape
    if L is None:
        L = torch.zeros(d_in, d_in, dtype=torch.float64, device=W.device)
    ldl = _f64_matrix(L, "L")
    w, wn = _workspace(_rfac_ws(d_in, n), W.device, ws)
    info = _info(info, 1, W.device)
    _check(_rfac(_ptr(W), _dt(W), d_in, n, ldw, _ptr(L), ldl, _ptr(w), wn, _ptr(info), _stream(stream)))
    return L, info


def lrc_cov_accumulate_range_workspace(n_tok: int, d_in: int) -> int:
    return _covr_ws(n_tok, d_in)


def lrc_cov_accumulate_range(X: torch.Tensor, L: torch.Tensor, B: torch.Tensor, info=None, ws=None,
                             stream=None) -> torch.Tensor:
    """B[upper] += (X L)^T (X L): X (n_tok, d_in) bf16, L (d_in, d_in) fp64 from lrc_range_factor,
    B (d_in, d_in) fp32.  Returns the int32 info tensor."""
    ldx = _rows(X, "X")
    n_tok, d_in = X.shape
    ldl = _f64_matrix(L, "L")
    ldb = _rows(B, "B")
    if B.dtype != torch.float32:
        raise TypeError("B must be float32")
    w, wn = _workspace(_covr_ws(n_tok, d_in), X.device, ws)
    info = _info(info, 1, X.device)
    _check(_covr(_ptr(X), _dt(X), n_tok, d_in, ldx, _ptr(L), ldl, _ptr(B), ldb, _ptr(w), wn, _ptr(info),
                 _stream(stream)))
    return info


def lrc_error_curve(lam: torch.Tensor, eps=None, stream=None) -> torch.Tensor:
    """eps[b][k] = sum of lam[b][i] for i >= k, k = 0..n (fp64)."""
    _dev(lam, "lambda")
    if lam.dtype != torch.float64 or not lam.is_contiguous():
        raise ValueError("lambda must be contiguous float64")
    n = lam.shape[-1]
    batch = lam.numel() // n
    if eps is None:
        eps = torch.empty(lam.shape[:-1] + (n + 1,), dtype=torch.float64, device=lam.device)
    _check(_err(_ptr(lam), n, batch, _ptr(eps), _stream(stream)))
    return eps


def lrc_factorize(W: torch.Tensor, V: torch.Tensor, k: int, A: torch.Tensor | None, B: torch.Tensor | None = None,
                  trans_w: int = 0, d_in: int | None = None, d_out: int | None = None, batch: int = 1,
                  stride_w: int = 0, stride_v: int = 0, stride_a: int = 0, stride_b: int = 0, stream=None):
    """A = W V[:, :k] (trans_w 0) or W^T V[:, :k] (trans_w 1) when A is given; B = V[:, :k]^T when
    given.  Batched matrices are addressed by element strides (a per-head W_h is a column slice)."""
    ldw, ldv = _rows(W, "W"), _rows(V, "V")
    lda = _rows(A, "A") if A is not None else 0
    ldb = _rows(B, "B") if B is not None else 0
    d_in = W.shape[-2] if d_in is None else d_in
    d_out = W.shape[-1] if d_out is None else d_out
    if V.dtype != torch.float32 or (A is not None and A.dtype != torch.float32) or \
            (B is not None and B.dtype != torch.float32):
        raise TypeError("V, A and B must be float32")
    _check(_fac(_ptr(W), _dt(W), trans_w, d_in, d_out, ldw, _ptr(V), ldv, k, batch, stride_w, stride_v, _ptr(A), lda,
                stride_a, _ptr(B), ldb, stride_b, _stream(stream)))
    return A, B


def lrc_fisher_scores(Gs, Ws, alpha=None, info=None, ws=None, stream=None):
    """alpha[m] = sum (G_m * W_m)^2 in fp64 for lists of same-dtype contiguous GPU tensors."""
    n = len(Gs)
    if n != len(Ws) or n == 0:
        raise ValueError("G and W lists must have the same non-zero length")
    for g, w in zip(Gs, Ws):
        _dev(g, "G")
        _dev(w, "W")
        if g.numel() != w.numel() or not g.is_contiguous() or not w.is_contiguous() or g.dtype != w.dtype:
            raise ValueError("G[m] and W[m] must be contiguous, same size and dtype")
    dev = Gs[0].device
    gp = (ctypes.c_void_p * n)(*[g.data_ptr() for g in Gs])
    wp = (ctypes.c_void_p * n)(*[w.data_ptr() for w in Ws])
    ne = (ctypes.c_int64 * n)(*[g.numel() for g in Gs])
    nbytes = _fsh_ws(n, ne)
    w, wn = _workspace(nbytes, dev, ws)
    if alpha is None:
        alpha = torch.empty(n, dtype=torch.float64, device=dev)
    info = _info(info, n, dev)
    _check(_fsh(n, gp, wp, ne, _dt(Gs[0]), _ptr(alpha), _ptr(w), wn, _ptr(info), _stream(stream)))
    return alpha, info


def lrc_fisher_scores_noalloc(Gs, Ws, alpha, info, stream=None):
    """lrc_fisher_scores with the partials in the library's own device scratch array: no workspace
    and no allocation in the call (alpha fp64 and info int32 must be given)."""
    n = len(Gs)
    if n != len(Ws) or n == 0:
        raise ValueError("G and W lists must have the same non-zero length")
    for g, w in zip(Gs, Ws):
        _dev(g, "G")
        _dev(w, "W")
        if g.numel() != w.numel() or not g.is_contiguous() or not w.is_contiguous() or g.dtype != w.dtype:
            raise ValueError("G[m] and W[m] must be contiguous, same size and dtype")
    if alpha.dtype != torch.float64 or alpha.numel() < n or info.dtype != torch.int32 or info.numel() < n:
        raise ValueError("alpha (fp64) and info (int32) must hold n_mats entries")
    gp = (ctypes.c_void_p * n)(*[g.data_ptr() for g in Gs])
    wp = (ctypes.c_void_p * n)(*[w.data_ptr() for w in Ws])
    ne = (ctypes.c_int64 * n)(*[g.numel() for g in Gs])
    _check(_fsh_na(n, gp, wp, ne, _dt(Gs[0]), _ptr(alpha), _ptr(info), _stream(stream)))
    return alpha, info


def lrc_fisher_scores_workspace(numel) -> int:
    ne = (ctypes.c_int64 * len(numel))(*[int(x) for x in numel])
    return _fsh_ws(len(numel), ne)


def lrc_allocate_ranks_workspace(n_mats: int, n_items: int) -> int:
    return _alc_ws(n_mats, n_items)


def lrc_cholesky_workspace(n: int) -> int:
    return _chol_ws(n)


def lrc_allocate_ranks(alpha, lambda_packed, offsets, eps0, cost, budget: int, k_min=None, k_out=None, info=None,
                       ws=None, stream=None):
    """Greedy rank allocation; all arrays device tensors (alpha, lambda_packed, eps0 fp64; offsets,
    cost int64; k_min int32 or None).  Returns (k int32 per matrix, info int32 (1,))."""
    n = alpha.numel()
    for t, nm in ((alpha, "alpha"), (eps0, "eps0"), (lambda_packed, "lambda")):
        _dev(t, nm)
        if t.dtype != torch.float64 or not t.is_contiguous():
            raise ValueError("%s must be contiguous float64" % nm)
    for t, nm in ((offsets, "offsets"), (cost, "cost")):
        _dev(t, nm)
        if t.dtype != torch.int64 or not t.is_contiguous():
            raise ValueError("%s must be contiguous int64" % nm)
    if k_min is not None and (k_min.dtype != torch.int32 or not k_min.is_cuda):
        raise ValueError("k_min must be a GPU int32 tensor")
    n_items = lambda_packed.numel()
    dev = alpha.device
    nbytes = _alc_ws(n, n_items)
    w, wn = _workspace(nbytes, dev, ws)
    if k_out is None:
        k_out = torch.empty(n, dtype=torch.int32, device=dev)
    info = _info(info, 1, dev)
    _check(_alc(n, _ptr(alpha), _ptr(lambda_packed), _ptr(offsets), n_items, _ptr(eps0), _ptr(cost), _ptr(k_min),
                int(budget), _ptr(k_out), _ptr(w), wn, _ptr(info), _stream(stream)))
    return k_out, info


def lrc_cholesky(A: torch.Tensor, info=None, ws=None, stream=None):
    lda = _rows(A, "A")
    n = A.shape[0]
    w, wn = _workspace(_chol_ws(n), A.device, ws)
    info = _info(info, 1, A.device)
    _check(_chol(_ptr(A), n, lda, _ptr(w), wn, _ptr(info), _stream(stream)))
    return A, info


def lrc_timing_enable(enable=True):
    """True (or 1): record every launch of the instrumented kernels; an int s > 1: every s-th
    launch of each kernel; False / 0: off."""
    stride = int(enable) if not isinstance(enable, bool) else (1 if enable else 0)
    _check(_tim_en(stride))


def lrc_timing_set_stride(kernel: str, stride: int):
    """Record every stride-th launch of one kernel (overrides the stride given to lrc_timing_enable)."""
    _check(_tim_st(kernel.encode(), int(stride)))


def lrc_timing_read(kernel: str, reset: bool = True):
    """(launches, total_ms, total_algorithmic_flops) recorded for one kernel name."""
    n = ctypes.c_int64(0)
    ms = ctypes.c_double(0.0)
    fl = ctypes.c_double(0.0)
    _check(_tim_rd(kernel.encode(), ctypes.byref(n), ctypes.byref(ms), ctypes.byref(fl), 1 if reset else 0))
    return n.value, ms.value, fl.value


def _f64_matrix(t: torch.Tensor, name: str) -> int:
    if t.dtype != torch.float64:
        raise ValueError("%s must be float64" % name)
    return _rows(t, name)


def lrc_trmm_workspace(m: int, n: int) -> int:
    return _trmm_ws(m, n)


def lrc_trsm_workspace(side: int, m: int, n: int) -> int:
    return _trsm_ws(side, m, n)


def lrc_trmm(side: int, trans: int, L: torch.Tensor, B: torch.Tensor, ws=None, stream=None):
    """B <- op(L) B (side 0) or B op(L) (side 1), op(L) = L or L^T; L lower, fp64, in place."""
    ldl, ldb = _f64_matrix(L, "L"), _f64_matrix(B, "B")
    m, n = B.shape
    w, wn = _workspace(_trmm_ws(m, n), B.device, ws)
    _check(_trmm(side, trans, m, n, _ptr(L), ldl, _ptr(B), ldb, _ptr(w), wn, _stream(stream)))
    return B


def lrc_trsm(side: int, trans: int, L: torch.Tensor, B: torch.Tensor, ws=None, stream=None):
    """B <- op(L)^{-1} B (side 0) or B op(L)^{-1} (side 1); L lower, fp64, in place."""
    ldl, ldb = _f64_matrix(L, "L"), _f64_matrix(B, "B")
    m, n = B.shape
    w, wn = _workspace(_trsm_ws(side, m, n), B.device, ws)
    _check(_trsm(side, trans, m, n, _ptr(L), ldl, _ptr(B), ldb, _ptr(w), wn, _stream(stream)))
    return B


def lrc_sym_to_f64(C: torch.Tensor, scale: float = 1.0, A=None, stream=None):
    """fp64 symmetric A = scale * C from the upper triangle of the fp32 matrix C."""
    if C.dtype != torch.float32:
        raise ValueError("C must be float32")
    ldc = _rows(C, "C")
    n = C.shape[-1]
    if A is None:
        A = torch.empty(n, n, dtype=torch.float64, device=C.device)
    lda = _f64_matrix(A, "A")
    _check(_sym64(_ptr(C), n, ldc, float(scale), _ptr(A), lda, _stream(stream)))
    return A


def lrc_to_f64(X: torch.Tensor, scale: float = 1.0, Y=None, stream=None):
    """fp64 Y = scale * X for a bf16, fp32 or fp64 matrix X."""
    ldx = _rows(X, "X")
    rows, cols = X.shape
    if Y is None:
        Y = torch.empty(rows, cols, dtype=torch.float64, device=X.device)
    ldy = _f64_matrix(Y, "Y")
    _check(_to64(_ptr(X), _dt(X), rows, cols, ldx, float(scale), _ptr(Y), ldy, _stream(stream)))
    return Y


def lrc_gram_f64(B: torch.Tensor, G=None, stream=None):
    """Upper triangle of the fp32 matrix G = B B^T, summed in fp64 from the fp64 matrix B."""
    ldb = _f64_matrix(B, "B")
    m, n = B.shape
    if G is None:
        G = torch.zeros(m, m, dtype=torch.float32, device=B.device)
    if G.dtype != torch.float32:
        raise ValueError("G must be float32")
    _check(_gram64(_ptr(B), m, n, ldb, _ptr(G), _rows(G, "G"), _stream(stream)))
    return G


def lrc_cov_from_input_workspace(d_in: int, d_out: int) -> int:
    return _cfi_ws(d_in, d_out)


def lrc_cov_from_input(H: torch.Tensor, W: torch.Tensor, C=None, ws=None, stream=None) -> torch.Tensor:
    """Upper triangle of C = W^T H W (fp32), from the input covariance H = X^T X (fp32 d_in x d_in, upper
    triangle read, as lrc_cov_accumulate writes it with W = None) and W (d_in x d_out): the covariance
    of Y = X W, formed in fp64."""
    ldh = _rows(H, "H")
    if H.dtype != torch.float32:
        raise ValueError("H must be float32")
    d_in = H.shape[0]
    ldw = _rows(W, "W")
    if W.shape[0] != d_in:
        raise ValueError("W must have d_in rows")
    d_out = W.shape[1]
    if C is None:
        C = torch.zeros(d_out, d_out, dtype=torch.float32, device=H.device)
    if C.dtype != torch.float32:
        raise ValueError("C must be float32")
    w, wn = _workspace(_cfi_ws(d_in, d_out), H.device, ws)
    _check(_cfi(_ptr(H), d_in, ldh, _ptr(W), _dt(W), d_out, ldw, _ptr(C), _rows(C, "C"), _ptr(w), wn, _stream(stream)))
    return C


def lrc_allocate_proportional(alpha: torch.Tensor, budgets: torch.Tensor, r_out=None, info=None, stream=None):
    """Ranks r[t][m] = round(alpha_m / S * budgets[t]), the rows brought to sum to budgets[t] by largest
    remainders (see include/lrc.h).  alpha fp64 (n_mats,), budgets int64 (n_budgets,) on the GPU.
    Returns (r int64 (n_budgets, n_mats), info int32 (1,))."""
    _dev(alpha, "alpha")
    _dev(budgets, "budgets")
    if alpha.dtype != torch.float64 or not alpha.is_contiguous():
        raise ValueError("alpha must be a contiguous float64 vector")
    if budgets.dtype != torch.int64 or not budgets.is_contiguous():
        raise ValueError("budgets must be a contiguous int64 vector")
    n, nb = alpha.numel(), budgets.numel()
    if r_out is None:
        r_out = torch.empty(nb, n, dtype=torch.int64, device=alpha.device)
    info = _info(info, 1, alpha.device)
    _check(_aprop(n, _ptr(alpha), nb, _ptr(budgets), _ptr(r_out), _ptr(info), _stream(stream)))
    return r_out, info


def _vec(t: torch.Tensor, name: str, dtype):
    _dev(t, name)
    if t.dtype != dtype or not t.is_contiguous():
        raise ValueError("%s must be a contiguous %s GPU tensor" % (name, dtype))


def lrc_allocate_swift(beta, eps_kbar, kbar, cost, k_cap, delta: float, alpha_grid, budget: int, scores=None,
                       k_out=None, info=None, stream=None):
    """Swift-SVD candidate allocations, one per alpha of the grid (see include/lrc.h).  beta, eps_kbar,
    alpha_grid fp64; kbar, cost, k_cap int64; all GPU vectors.  Returns (scores fp64 (n_alpha, n),
    k int32 (n_alpha, n), info int32 (n_alpha,))."""
    for t, nm in ((beta, "beta"), (eps_kbar, "eps_kbar"), (alpha_grid, "alpha_grid")):
        _vec(t, nm, torch.float64)
    for t, nm in ((kbar, "kbar"), (cost, "cost"), (k_cap, "k_cap")):
        _vec(t, nm, torch.int64)
    n, na = beta.numel(), alpha_grid.numel()
    if not (eps_kbar.numel() == kbar.numel() == cost.numel() == k_cap.numel() == n):
        raise ValueError("per-matrix vectors must have the same length")
    dev = beta.device
    if scores is None:
        scores = torch.empty(na, n, dtype=torch.float64, device=dev)
    if k_out is None:
        k_out = torch.empty(na, n, dtype=torch.int32, device=dev)
    info = _info(info, na, dev)
    _check(_aswift(n, _ptr(beta), _ptr(eps_kbar), _ptr(kbar), _ptr(cost), _ptr(k_cap), float(delta), na,
                   _ptr(alpha_grid), int(budget), _ptr(scores), _ptr(k_out), _ptr(info), _stream(stream)))
    return scores, k_out, info


def lrc_component_fisher_workspace(d_in: int, k: int, batch: int = 1) -> int:
    return _cfsh_ws(d_in, k, batch)


def lrc_component_fisher(W: torch.Tensor, G: torch.Tensor, V: torch.Tensor, k: int, score=None, d_in=None, d_out=None,
                         batch: int = 1, stride_w: int = 0, stride_g: int = 0, stride_v: int = 0, stride_s: int = 0,
                         ws=None, stream=None) -> torch.Tensor:
    """score[b][i] = ((W v_i) . (G v_i))^2 for the first k columns of V (fp64); batched by element strides."""
    ldw, ldg, ldv = _rows(W, "W"), _rows(G, "G"), _rows(V, "V")
    if W.dtype != G.dtype:
        raise TypeError("W and G must have the same dtype")
    if V.dtype != torch.float32:
        raise TypeError("V must be float32")
    d_in = W.shape[-2] if d_in is None else d_in
    d_out = W.shape[-1] if d_out is None else d_out
    if score is None:
        score = torch.empty(batch, k, dtype=torch.float64, device=W.device)
        stride_s = k
    w, wn = _workspace(_cfsh_ws(d_in, k, batch), W.device, ws)
    _check(_cfsh(_ptr(W), _ptr(G), _dt(W), d_in, d_out, ldw, ldg, _ptr(V), ldv, k, batch, stride_w, stride_g,
                 stride_v, _ptr(score), stride_s, _ptr(w), wn, _stream(stream)))
    return score


def lrc_allocate_components_workspace(n_mats: int, n_items: int) -> int:
    return _acomp_ws(n_mats, n_items)


def lrc_allocate_components(score_packed, offsets, cost, budget: int, k_min=None, k_out=None, selected=None,
                            info=None, ws=None, stream=None):
    """Greedy selection of single components by score per parameter (see include/lrc.h).  Returns
    (k int32 per matrix, selected uint8 per component, info int32 (1,))."""
    _vec(score_packed, "score_packed", torch.float64)
    _vec(offsets, "offsets", torch.int64)
    _vec(cost, "cost", torch.int64)
    if k_min is not None:
        _vec(k_min, "k_min", torch.int32)
    n = cost.numel()
    n_items = score_packed.numel()
    dev = cost.device
    w, wn = _workspace(_acomp_ws(n, n_items), dev, ws)
    if k_out is None:
        k_out = torch.empty(n, dtype=torch.int32, device=dev)
    if selected is None:
        selected = torch.empty(max(n_items, 1), dtype=torch.uint8, device=dev)
    info = _info(info, 1, dev)
    _check(_acomp(n, _ptr(score_packed), _ptr(offsets), n_items, _ptr(cost), _ptr(k_min), int(budget), _ptr(k_out),
                  _ptr(selected), _ptr(w), wn, _ptr(info), _stream(stream)))
    return k_out, selected[:n_items], info
