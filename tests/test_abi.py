"""The C-ABI library loads, exports every entry point include/lrc.h declares, and rejects bad
arguments synchronously (no kernel is launched on these paths, so no GPU is needed)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lrc.h")
LIB = os.path.join(ROOT, "activation_aware_rank_amd", "liblrc.so")


def declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(lrc_[a-z_0-9]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("liblrc.so not built (run __graft_entry__.build())")
    return ctypes.CDLL(LIB)


def test_header_declares_the_six_path_entry_points():
    d = declared()
    for name in ("lrc_cov_accumulate", "lrc_eigh", "lrc_factorize", "lrc_error_curve", "lrc_fisher_scores",
                 "lrc_allocate_ranks"):
        assert name in d


def test_every_declared_symbol_is_exported(lib):
    missing = [n for n in declared() if not hasattr(lib, n)]
    assert not missing, missing


def test_binding_covers_every_declared_symbol():
    from activation_aware_rank_amd import lrc
    assert sorted(lrc.EXPORTED) == declared()
    for n in declared():
        assert callable(getattr(lrc, n))


def test_abi_version_and_status_strings(lib):
    from activation_aware_rank_amd import lrc
    assert lrc.lrc_abi_version() == 1
    assert lrc.lrc_status_string(0) == "ok"
    assert lrc.lrc_status_string(3).startswith("workspace")


def test_argument_errors_are_synchronous():
    from activation_aware_rank_amd import lrc
    fake = ctypes.c_void_p(256)  # never dereferenced: validation fails first
    # NULL X
    rc = lrc._cov(None, 0, 10, 8, 8, fake, 0, 8, 8, 1, fake, 8, None, 0, fake, None)
    assert rc == 1 and "non-NULL" in lrc.lrc_last_error()
    # ldx < d_in
    rc = lrc._cov(fake, 0, 10, 8, 4, fake, 0, 8, 8, 1, fake, 8, None, 0, fake, None)
    assert rc == 1 and "ldx" in lrc.lrc_last_error()
    # n_blocks does not divide d_out
    rc = lrc._cov(fake, 0, 10, 8, 8, fake, 0, 12, 12, 5, fake, 12, None, 0, fake, None)
    assert rc == 1
    # dtype mismatch
    rc = lrc._cov(fake, 0, 10, 8, 8, fake, 1, 8, 8, 1, fake, 8, None, 0, fake, None)
    assert rc == 2
    # identity W with d_out != d_in
    rc = lrc._cov(fake, 0, 10, 8, 8, None, 0, 16, 0, 1, fake, 16, None, 0, fake, None)
    assert rc == 1
    # range-projected covariance: d_in not a multiple of 32, NULL L, fp32 X, small ldb
    rc = lrc._covr(fake, 0, 10, 48, 48, fake, 48, fake, 48, fake, 1 << 20, fake, None)
    assert rc == 1 and "multiple of 32" in lrc.lrc_last_error()
    rc = lrc._covr(fake, 0, 10, 64, 64, None, 64, fake, 64, fake, 1 << 20, fake, None)
    assert rc == 1
    rc = lrc._covr(fake, 1, 10, 64, 64, fake, 64, fake, 64, fake, 1 << 20, fake, None)
    assert rc == 2
    rc = lrc._covr(fake, 0, 10, 64, 64, fake, 64, fake, 32, fake, 1 << 20, fake, None)
    assert rc == 1
    # range factor: n < d_in
    rc = lrc._rfac(fake, 0, 64, 32, 32, fake, 64, fake, 1 << 20, fake, None)
    assert rc == 1
    # a projected eigendecomposition group without its basis, or with n_vec > d_in
    g = lrc._EighGroup(fake, 400, 200, 1, 0, fake, fake, 8, 8, 0, fake)
    g.projected = 1
    arr = (lrc._EighGroup * 1)(g)
    assert lrc._eigh_m(arr, 1, 1, fake, 1 << 30, None) == 1
    g.W, g.w_t, g.d_in, g.ldw, g.n_vec, g.ldv = fake, 0, 200, 400, 201, 201
    arr = (lrc._EighGroup * 1)(g)
    assert lrc._eigh_m(arr, 1, 1, fake, 1 << 30, None) == 1
    # a caller's factor with ldl < d_in, or without the basis
    g.n_vec, g.ldv, g.L, g.ldl = 8, 8, fake, 100
    arr = (lrc._EighGroup * 1)(g)
    assert lrc._eigh_m(arr, 1, 1, fake, 1 << 30, None) == 1 and "ldl" in lrc.lrc_last_error()
    g2 = lrc._EighGroup(fake, 400, 400, 1, 0, fake, fake, 8, 8, 0, fake)
    g2.L, g2.ldl = fake, 400
    arr = (lrc._EighGroup * 1)(g2)
    assert lrc._eigh_m(arr, 1, 1, fake, 1 << 30, None) == 1
    # covariance from the input covariance: NULL H, W dtype, ldh < d_in, workspace too small
    need = lrc.lrc_cov_from_input_workspace(8, 12)
    up = lambda b: (b + 255) // 256 * 256  # noqa: E731
    assert need == up(8 * 8 * 8) + 2 * up(8 * 12 * 8)  # fp64 H, W and H W
    assert lrc._cfi(None, 8, 8, fake, 0, 12, 12, fake, 12, fake, need, None) == 1
    assert lrc._cfi(fake, 8, 8, fake, 7, 12, 12, fake, 12, fake, need, None) == 2
    assert lrc._cfi(fake, 8, 7, fake, 0, 12, 12, fake, 12, fake, need, None) == 1
    rc = lrc._cfi(fake, 8, 8, fake, 0, 12, 12, fake, 12, fake, need - 1, None)
    assert rc == 3 and "workspace" in lrc.lrc_last_error()
    # workspace too small
    need = lrc.lrc_cov_accumulate_workspace(0, 1000, 64, True, 64, 1)
    assert need > 0
    rc = lrc._cov(fake, 0, 1000, 64, 64, fake, 0, 64, 64, 1, fake, 64, fake, need - 1, fake, None)
    assert rc == 3
    # eigh: n_vec > n, bad prec
    rc = lrc._eigh(fake, 10, 10, 1, 0, 1, fake, fake, 11, 11, 0, None, 0, fake, None)
    assert rc == 1
    rc = lrc._eigh(fake, 10, 10, 1, 0, 0, fake, fake, 4, 4, 0, None, 0, fake, None)
    assert rc == 2
    # factorize: k larger than V's rows
    rc = lrc._fac(fake, 0, 0, 8, 4, 4, fake, 8, 5, 1, 0, 0, fake, 8, 0, None, 0, 0, None)
    assert rc == 1
    # error curve: n <= 0
    assert lrc._err(fake, 0, 1, fake, None) == 1
    # fisher: negative numel
    ne = (ctypes.c_int64 * 1)(-1)
    ptrs = (ctypes.c_void_p * 1)(256)
    assert lrc._fsh(1, ptrs, ptrs, ne, 0, fake, None, 0, fake, None) == 1
    # allocate: negative budget
    assert lrc._alc(1, fake, fake, fake, 3, fake, fake, None, -1, fake, None, 0, fake, None) == 1
    # triangular: bad side flag
    assert lrc._trsm(2, 0, 4, 4, fake, 4, fake, 4, fake, 1 << 20, None) == 1
    # triangular: workspace too small, leading dimension too small
    need = lrc.lrc_trsm_workspace(0, 100, 8)
    assert need >= 2 * 64 * 64 * 8
    assert lrc._trsm(0, 0, 100, 8, fake, 100, fake, 8, fake, need - 1, None) == 3
    assert lrc._trmm(0, 1, 100, 8, fake, 99, fake, 8, fake, 1 << 20, None) == 1
    assert lrc._trmm(1, 0, 8, 100, fake, 100, fake, 100, fake, lrc.lrc_trmm_workspace(8, 100) - 1, None) == 3
    # cholesky: lda < n; conversions: bad dtype, ldx < cols; gram: ldg < m
    assert lrc._chol(fake, 10, 9, fake, 1 << 20, fake, None) == 1
    assert lrc._to64(fake, 7, 4, 4, 4, 1.0, fake, 4, None) == 2
    assert lrc._to64(fake, 0, 4, 4, 3, 1.0, fake, 4, None) == 1
    assert lrc._sym64(fake, 8, 7, 1.0, fake, 8, None) == 1
    assert lrc._gram64(fake, 8, 4, 4, fake, 7, None) == 1
    # eigh_multi: NULL groups, count 0, a group with n_vec > n, bad prec, small workspace
    G = lrc._EighGroup
    assert lrc._eigh_m(None, 1, 1, None, 0, None) == 1
    ok = G(256, 300, 300, 2, 90000, 256, 256, 8, 8, 2400, 256)
    bad = G(256, 300, 300, 1, 0, 256, 256, 8, 301, 0, 256)
    arr = (G * 2)(ok, bad)
    assert lrc._eigh_m(arr, 0, 1, None, 0, None) == 1
    assert lrc._eigh_m(arr, 2, 1, fake, 1 << 40, None) == 1 and "n_vec" in lrc.lrc_last_error()
    assert lrc._eigh_m(arr, 1, 7, fake, 1 << 40, None) == 2
    need = lrc._eigh_mws(arr, 1, 1)
    assert lrc._eigh_m(arr, 1, 1, fake, need - 1, None) == 3
    # range basis: bad dtype, ldw < n, bases of a batch overlapping
    for w_t, ldw, stride_w, code, word in ((5, 300, 200 * 300, 2, "w_t"), (0, 299, 200 * 300, 1, "ldw"),
                                           (0, 300, 100, 1, "stride_w")):
        g = G(256, 300, 300, 2, 90000, 256, 256, 8, 8, 2400, 256, 256, w_t, 200, ldw, stride_w)
        assert lrc._eigh_m((G * 1)(g), 1, 1, fake, 1 << 40, None) == code and word in lrc.lrc_last_error()


def test_workspace_queries_are_consistent():
    from activation_aware_rank_amd import lrc
    a = lrc.lrc_cov_accumulate_workspace(0, 100000, 4096, True, 4096, 1)
    b = lrc.lrc_cov_accumulate_workspace(0, 100000, 4096, True, 11008, 1)
    assert 0 < a < b
    assert lrc.lrc_eigh_workspace(4096, 1, 1228, 1) > lrc.lrc_eigh_workspace(4096, 1, 0, 1)
    assert lrc.lrc_eigh_workspace(128, 32, 32, 2) == 0  # Jacobi keeps everything in LDS
    # batched members run up to eight at a time, each with a region of its own
    one = lrc.lrc_eigh_workspace(4096, 1, 1228, 1)
    assert lrc.lrc_eigh_workspace(4096, 3, 1228, 1) == 3 * one
    assert lrc.lrc_eigh_workspace(4096, 9, 1228, 1) == 8 * one
    # several groups: as many regions as concurrent members, each sized for the largest group
    assert lrc.lrc_eigh_multi_workspace([(4096, 3, 1228)], 1) == 3 * one
    big = lrc.lrc_eigh_workspace(11008, 1, 1791, 1)
    assert lrc.lrc_eigh_multi_workspace([(4096, 5, 1228), (11008, 2, 1791), (128, 32, 32)], 1) == 7 * big
    assert lrc.lrc_eigh_multi_workspace([(4096, 8, 1228), (11008, 2, 1791)], 1) == 8 * big
    # the largest n and the largest n_vec may come from different groups
    assert lrc.lrc_eigh_multi_workspace([(4096, 1, 1791), (11008, 1, 1228)], 1) == 2 * big
    assert lrc.lrc_eigh_multi_workspace([(64, 4, 8)], 2) == 0
    assert lrc.lrc_eigh_multi_workspace([(64, 4, 65)], 2) == 0
    # a range basis of d_in rows (128 < d_in < n, n_vec <= d_in): the region also holds the basis, n x n
    # and d_in x n fp64 products, and the decomposition of the d_in x d_in matrix; otherwise ignored
    rng = lrc.lrc_eigh_multi_workspace([(11008, 2, 1791, 4096)], 1)
    assert rng > 2 * 8 * 11008 * 11008 and rng != 2 * big
    assert lrc.lrc_eigh_multi_workspace([(11008, 2, 1791, 4096), (4096, 5, 1228)], 1) == 7 * (rng // 2)
    assert lrc.lrc_eigh_multi_workspace([(11008, 1, 1791, 12000)], 1) == big
    assert lrc.lrc_eigh_multi_workspace([(11008, 1, 1791, 100)], 1) == big
    assert lrc.lrc_eigh_multi_workspace([(4096, 1, 1791, 1228)], 1) == lrc.lrc_eigh_workspace(4096, 1, 1791, 1)
    assert lrc.lrc_allocate_ranks_workspace(224, 548704) > 548704 * 8


def test_allocation_scores_argument_errors():
    from activation_aware_rank_amd import lrc
    fake = ctypes.c_void_p(256)
    # Swift-SVD candidates: NULL pointer, n_mats out of range, n_alpha 0, negative budget
    assert lrc._aswift(3, None, fake, fake, fake, fake, 0.5, 2, fake, 10, fake, fake, fake, None) == 1
    assert lrc._aswift(1025, fake, fake, fake, fake, fake, 0.5, 2, fake, 10, fake, fake, fake, None) == 1
    assert lrc._aswift(3, fake, fake, fake, fake, fake, 0.5, 0, fake, 10, fake, fake, fake, None) == 1
    assert lrc._aswift(3, fake, fake, fake, fake, fake, 0.5, 2, fake, -1, fake, fake, fake, None) == 1
    # component scores: dtype, k > d_out, ldv < k, workspace
    ws = lrc.lrc_component_fisher_workspace(100, 20, 1)
    assert ws >= 2 * 20 * 8
    assert lrc._cfsh(fake, fake, 2, 100, 50, 50, 50, fake, 20, 20, 1, 0, 0, 0, fake, 20, fake, ws, None) == 2
    assert lrc._cfsh(fake, fake, 0, 100, 50, 50, 50, fake, 60, 60, 1, 0, 0, 0, fake, 60, fake, 1 << 30, None) == 1
    assert lrc._cfsh(fake, fake, 0, 100, 50, 50, 50, fake, 10, 20, 1, 0, 0, 0, fake, 20, fake, ws, None) == 1
    assert lrc._cfsh(fake, fake, 0, 100, 50, 50, 50, fake, 20, 20, 1, 0, 0, 0, fake, 20, fake, ws - 1, None) == 3
    # component greedy: NULL offsets, negative budget, small workspace
    need = lrc.lrc_allocate_components_workspace(4, 100)
    assert need == lrc.lrc_allocate_ranks_workspace(4, 100)
    assert lrc._acomp(4, fake, None, 100, fake, None, 10, fake, None, fake, need, fake, None) == 1
    assert lrc._acomp(4, fake, fake, 100, fake, None, -1, fake, None, fake, need, fake, None) == 1
    assert lrc._acomp(4, fake, fake, 100, fake, None, 10, fake, None, fake, need - 1, fake, None) == 3
