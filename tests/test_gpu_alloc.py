"""Parity of the two further allocation rules against the oracle, through the C ABI.

* Swift-SVD allocation candidates (Swift-SVD page, section 2-na): the GPU's scores within 1e-14
  relative of the oracle's (device and host pow/log may differ in the last bit), and its ranks for
  every alpha of a grid bit-exact against the oracle's allocation from the same scores; the
  hand-worked cases; bad inputs.
* LASER per-component empirical-Fisher scores (LASER page, method 2): the GPU's
  ((W v_i) . (G v_i))^2 against the oracle's diagonal of V^T (W^T G) V, relative to the scale
  ||W v_i||^2 ||G v_i||^2 that bounds the rounding of a cancelling dot product; per-head batches
  with column-slice strides; the greedy selection bit-exact (ranks and kept components) against the
  oracle on the same scores, ties included; the hand-worked cases.
"""
import json
import os

import numpy as np
import pytest

import oracle
from activation_aware_rank_amd import inputs
from parity_utils import dev, host

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module")
def lrc():
    from activation_aware_rank_amd import lrc as m
    return m


def _say(msg):
    print("\n[case] " + msg, flush=True)


# ---------------------------------------------------------------------------------------------
# Swift-SVD candidates
# ---------------------------------------------------------------------------------------------

def _swift_gpu(lrc, beta, eps, kbar, cost, k_cap, delta, alphas, budget):
    f64 = lambda a: dev(np.asarray(a, dtype=np.float64), "f64")  # noqa: E731
    i64 = lambda a: dev(np.asarray(a, dtype=np.int64), "i64")  # noqa: E731
    s, k, info = lrc.lrc_allocate_swift(f64(beta), f64(eps), i64(kbar), i64(cost), i64(k_cap), delta, f64(alphas),
                                        budget)
    return host(s), host(k), host(info)


def test_swift_worked_example(lrc):
    """alpha = 1 makes the scores the importances exactly (x^1 and y^0 are exact)."""
    ex = json.load(open(os.path.join(GOLDEN, "swift_alloc_worked_example.json")))
    for case in ex["cases"]:
        s, k, info = _swift_gpu(lrc, case["scores"], [5.0, 6.0, 7.0], ex["kbar"], ex["cost"], ex["k_cap"],
                                case["delta"], [1.0], case["budget"])
        assert np.array_equal(s[0], np.array(case["scores"]))
        assert int(info[0]) == case["info"] and list(k[0]) == case["k"], case


def test_swift_stack_grid_bitexact(lrc):
    """224 matrices of a 32-layer stack (the LLaMA-7B shapes), an 80 % parameter budget, uniform ranks
    at 80 %, delta 0.5 and 0.9, an alpha grid of 11 values."""
    _say("Swift-SVD candidates: 224 matrices, 11 alphas")
    shapes = inputs.block_shapes()
    r = np.random.default_rng(31)
    di = np.array([shapes[m][0] for _ in range(32) for m in inputs.BLOCK_MATRICES], dtype=np.int64)
    do = np.array([shapes[m][1] for _ in range(32) for m in inputs.BLOCK_MATRICES], dtype=np.int64)
    cost = di + do
    k_cap = (di * do) // cost
    kbar = np.floor(0.8 * di * do / cost).astype(np.int64)
    budget = int(np.floor(0.8 * np.sum(di * do)))
    beta = r.lognormal(0.0, 1.5, 224)
    eps = r.lognormal(12.0, 2.0, 224)
    eps[5] = 0.0
    eps[6] = -3e-9  # rounding residue of a tail sum
    alphas = np.linspace(0.0, 1.0, 11)
    for delta in (0.5, 0.9):
        s, k, info = _swift_gpu(lrc, beta, eps, kbar, cost, k_cap, delta, alphas, budget)
        assert np.all(info == 0)
        for a_i, al in enumerate(alphas):
            s_ref = oracle.swift_scores(beta, eps, float(al))
            assert np.max(np.abs(s[a_i] - s_ref) / s_ref) <= 1e-14, al
            k_ref, info_ref = oracle.swift_allocate(s[a_i], kbar, cost, k_cap, delta, budget)
            assert info_ref == 0 and np.array_equal(k[a_i], k_ref), (delta, al)
            k_own, _ = oracle.swift_allocate(s_ref, kbar, cost, k_cap, delta, budget)
            used = int(np.sum(k[a_i].astype(np.int64) * cost))
            assert used <= budget
            print("delta %.1f alpha %.1f: ranks %d..%d, %d of %d parameters, same as from the oracle's own "
                  "scores: %s" % (delta, al, k[a_i].min(), k[a_i].max(), used, budget,
                                  np.array_equal(k[a_i], k_own)))


def test_swift_bad_inputs(lrc):
    ones = [1.0, 1.0]
    s, k, info = _swift_gpu(lrc, [1.0, -2.0], ones, [1, 1], [2, 2], [3, 3], 0.5, [0.5, 0.0], 10)
    assert list(info) == [5, 0]  # (-2)^0.5 is NaN; (-2)^0 = 1 is a valid score
    s, k, info = _swift_gpu(lrc, ones, [1.0, np.nan], [1, 1], [2, 2], [3, 3], 0.5, [0.5], 10)
    assert int(info[0]) == 5
    s, k, info = _swift_gpu(lrc, ones, ones, [1, 4], [2, 2], [3, 3], 0.5, [0.5], 10)  # kbar > k_cap
    assert int(info[0]) == 5
    s, k, info = _swift_gpu(lrc, ones, ones, [1, 1], [2, 2], [3, 3], 0.5, [1.5], 10)  # alpha > 1
    assert int(info[0]) == 5
    s, k, info = _swift_gpu(lrc, ones, ones, [2, 2], [2, 2], [3, 3], 1.0, [0.5], 7)  # minima 8 > 7
    assert int(info[0]) == 4 and list(k[0]) == [2, 2]


# ---------------------------------------------------------------------------------------------
# LASER per-component scores and the component greedy
# ---------------------------------------------------------------------------------------------

def _check_scores(s_gpu, W64, G64, V, k):
    Vk = np.asarray(V, dtype=np.float64)[:, :k]
    ref = oracle.component_fisher(W64, G64, V, k)
    scale = (np.linalg.norm(W64 @ Vk, axis=0) * np.linalg.norm(G64 @ Vk, axis=0)) ** 2
    err = np.max(np.abs(s_gpu - ref) / scale)
    print("component scores: max |ds| / (||W v|| ||G v||)^2 = %.2e, relative to the score %.2e"
          % (err, np.max(np.abs(s_gpu - ref) / np.maximum(ref, 1e-300))))
    assert err <= 1e-13
    return ref


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_component_fisher_vs_oracle(lrc, dtype):
    """200 x 330 (ragged tiles in both directions), k = 150, V from the oracle's eigendecomposition of a
    block-shaped covariance."""
    _say("component scores %s 200 x 330, k = 150" % dtype)
    d_in, d_out, k = 200, 330, 150
    X = inputs.block_activations(d_in, 3000)
    Wb = inputs.weight(d_in, d_out, "bf16", inputs.CFG_BLOCK, 0, 5)
    Gb = inputs.gradient(d_in, d_out, 1e-4, inputs.CFG_BLOCK, 0, 5)
    _, V = oracle.eigh(oracle.covariance(X, "bf16", Wb, "bf16"))
    V32 = V.astype(np.float32)
    if dtype == "bf16":
        W, G = Wb, Gb
    else:
        W, G = oracle.widen(Wb, "bf16").astype(np.float32), oracle.widen(Gb, "bf16").astype(np.float32)
    s = host(lrc.lrc_component_fisher(dev(W, dtype), dev(G, dtype), dev(V32, "f32"), k))[0]
    _check_scores(s, oracle.widen(W, dtype), oracle.widen(G, dtype), V32, k)


def test_component_fisher_per_head_batch(lrc):
    """Four heads of 64 columns of a 256 x 256 matrix: W_h, G_h column slices (stride 64), V_h stacked."""
    _say("component scores per head: 4 x (256 x 64), k = 40")
    d_in, hd, nh, k = 256, 64, 4, 40
    Wb = inputs.weight(d_in, hd * nh, "bf16", inputs.CFG_HEADS, 0, 3)
    Gb = inputs.gradient(d_in, hd * nh, 1e-4, inputs.CFG_HEADS, 0, 3)
    r = np.random.default_rng(5)
    Vs = np.stack([np.linalg.qr(r.standard_normal((hd, hd)))[0] for _ in range(nh)]).astype(np.float32)
    s = host(lrc.lrc_component_fisher(dev(Wb, "bf16"), dev(Gb, "bf16"), dev(Vs, "f32"), k, d_in=d_in, d_out=hd,
                                      batch=nh, stride_w=hd, stride_g=hd, stride_v=hd * hd))
    W64, G64 = oracle.widen(Wb, "bf16"), oracle.widen(Gb, "bf16")
    for h in range(nh):
        _check_scores(s[h], W64[:, h * hd:(h + 1) * hd], G64[:, h * hd:(h + 1) * hd], Vs[h], k)


def _comp_gpu(lrc, scores, cost, budget, k_min=None):
    offs = np.concatenate([[0], np.cumsum([len(x) for x in scores])]).astype(np.int64)
    sp = np.concatenate([np.asarray(x, dtype=np.float64) for x in scores])
    km = None if k_min is None else dev(np.asarray(k_min, dtype=np.int32), "i32")
    k, sel, info = lrc.lrc_allocate_components(dev(sp, "f64"), dev(offs, "i64"), dev(np.asarray(cost, np.int64), "i64"),
                                               budget, k_min=km)
    sel = host(sel)
    return host(k), [sel[offs[m]:offs[m + 1]].astype(bool) for m in range(len(scores))], int(host(info)[0])


def test_component_alloc_worked_example(lrc):
    ex = json.load(open(os.path.join(GOLDEN, "component_alloc_worked_example.json")))
    for case in ex["cases"]:
        k, masks, info = _comp_gpu(lrc, ex["scores"], ex["cost"], case["budget"], case["k_min"])
        assert info == case["info"], case
        assert list(k) == case["k"], case
        assert [list(m.astype(int)) for m in masks] == case["masks"], case


def test_component_alloc_bitexact_random_with_ties(lrc):
    _say("component allocation random")
    r = np.random.default_rng(32)
    for trial in range(30):
        M = int(r.integers(1, 10))
        scores = []
        for m in range(M):
            K = int(r.integers(1, 80))
            x = r.lognormal(0.0, 2.0, K)
            if trial % 3 == 0:
                x = r.choice([0.0, 0.5, 1.0, 3.0], K)
            scores.append(x)
        cost = r.integers(1, 9, M)
        k_min = [int(r.integers(0, len(x) + 1)) if r.random() < 0.3 else 0 for x in scores]
        total = int(sum(len(x) * c for x, c in zip(scores, cost)))
        for budget in (0, total // 3, total // 2 + 1, total, total + 5):
            kg, mg, ig = _comp_gpu(lrc, scores, cost, budget, k_min)
            ko, mo, io = oracle.allocate_components(scores, cost, budget, k_min)
            assert ig == io and list(kg) == list(ko), (trial, budget)
            assert all(np.array_equal(a, b) for a, b in zip(mg, mo)), (trial, budget)


def test_component_alloc_bad_scores(lrc):
    k, masks, info = _comp_gpu(lrc, [[1.0, np.nan], [2.0]], [3, 3], 100)
    assert info == 5
    k, masks, info = _comp_gpu(lrc, [[1.0, -0.5], [2.0]], [3, 3], 100)
    assert info == 5


def test_laser_chain_small(lrc):
    """Covariance -> eigendecomposition -> component scores -> greedy over three matrices on the GPU,
    against the oracle's chain: scores within the eigenvectors' own precision, the selection
    bit-exact on the GPU's scores."""
    _say("LASER chain: 3 matrices, 4096 tokens")
    import torch
    X = inputs.block_activations(160, 4096)
    mats = [(160, 200), (160, 160), (160, 240)]
    scores_g, costs, checks = [], [], []
    for i, (di, do) in enumerate(mats):
        W = inputs.weight(di, do, "bf16", inputs.CFG_BLOCK, 1, i)
        G = inputs.gradient(di, do, 1e-4, inputs.CFG_BLOCK, 1, i)
        C = torch.zeros(do, do, dtype=torch.float32, device="cuda")
        lrc.lrc_cov_accumulate(dev(X, "bf16"), dev(W, "bf16"), C)
        K = (di * do) // (di + do)
        lam, V, info = lrc.lrc_eigh(C, n_vec=K, prec=2)
        assert int(host(info)[0]) == 0
        s = host(lrc.lrc_component_fisher(dev(W, "bf16"), dev(G, "bf16"), V, K))[0]
        _, V_r = oracle.eigh(oracle.covariance(X, "bf16", W, "bf16"))
        s_r = oracle.component_fisher(oracle.widen(W, "bf16"), oracle.widen(G, "bf16"), V_r, K)
        checks.append(np.max(np.abs(s - s_r)) / np.max(s_r))
        scores_g.append(s)
        costs.append(di + do)
    print("scores against the oracle's chain: max |ds| / max s = %s" % ["%.1e" % c for c in checks])
    assert max(checks) <= 1e-3
    budget = int(0.5 * sum(di * do for di, do in mats))
    kg, mg, ig = _comp_gpu(lrc, scores_g, costs, budget)
    ko, mo, io = oracle.allocate_components(scores_g, costs, budget)
    assert ig == io == 0 and list(kg) == list(ko)
    assert all(np.array_equal(a, b) for a, b in zip(mg, mo))
