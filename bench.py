"""Benchmark: activation-aware truncated SVD of one LLaMA-7B-shaped block on one MI355X.

Workload (one "step" = the whole path over one batch of synthetic calibration data):
  * block: q/k/v/o 4096x4096, gate/up 4096x11008, down 11008x4096 (Y = X W orientation), bf16
    weights ~ N(0, 0.02^2); calibration 256 sequences x 2048 tokens = 524288 tokens, X = N(0,1)
    times a per-channel lognormal(0,1) scale, bf16 (the down projection gets its own X of width
    11008 drawn the same way); rank for 60% of each matrix's parameters (1228 / 1791).
  * per matrix: covariance C = sum Y^T Y (lrc_cov_accumulate), eigendecomposition (lrc_eigh),
    error curve (lrc_error_curve), factors A = W V_k, B = V_k^T (lrc_factorize);
  * over the block: Fisher scores of synthetic gradients ~ N(0, 1e-4^2) (lrc_fisher_scores) and
    the greedy allocation of the same 60% parameter budget from the error curves
    (lrc_allocate_ranks; its ranks are reported, the factors use the per-matrix 60% ranks).
Inputs are generated on the GPU (torch's seeded generator) and are resident in HBM before the
timed region.  Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6  # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
MATS = ("q_proj", "k_proj", "v_proj", "o_proj", "gate_proj", "up_proj", "down_proj")


def shapes(d_model, d_ff):
    return {"q_proj": (d_model, d_model), "k_proj": (d_model, d_model), "v_proj": (d_model, d_model),
            "o_proj": (d_model, d_model), "gate_proj": (d_model, d_ff), "up_proj": (d_model, d_ff),
            "down_proj": (d_ff, d_model)}


def cov_flops(n_tok, d_in, d_out):
    """Algorithmic flops of C += (XW)^T(XW): the GEMM plus the upper triangle of the SYRK."""
    return n_tok * (2 * d_in * d_out + d_out * (d_out + 1))


def _profile_record(name, source_key="source"):
    """A committed rocprofv3 counter record under profiles/, if the kernel source it names is unchanged
    since the counters were taken (else None)."""
    import hashlib
    try:
        rec = json.load(open(os.path.join(ROOT, "profiles", name)))
        src = open(os.path.join(ROOT, rec[source_key]), "rb").read()
    except (OSError, ValueError, KeyError):
        return None
    if hashlib.sha256(src).hexdigest() != rec.get("source_sha256"):
        return None
    return rec


def measured_traffic(kernel, algorithmic_bytes_per_launch=None):
    """HBM bytes per launch from the committed FETCH_SIZE/WRITE_SIZE record. With the algorithmic bytes
    per launch of this run given, the record's ratio of measured to algorithmic bytes scales them (for
    a kernel whose launches carry a different amount of work here than in the counted run)."""
    rec = _profile_record("%s_traffic.json" % kernel)
    if rec is None:
        return None
    if algorithmic_bytes_per_launch is not None:
        return rec["traffic_bytes_per_launch"] / rec["algorithmic_bytes_per_launch"] * algorithmic_bytes_per_launch
    return rec["traffic_bytes_per_launch"]


def mfma_counters(kernel):
    """Executed MFMA rate, shader clock and busy fraction from the committed counter record."""
    rec = _profile_record("k_cov_mfma_counters.json")
    if rec is None or kernel not in rec.get("kernels", {}):
        return None
    k = rec["kernels"][kernel]
    return {"executed_tflops": k["executed_mfma_tflops"], "shader_clock_ghz": k["shader_clock_ghz"],
            "mfma_busy": k["mfma_busy_fraction"], "counted_launch_ms": k["mean_launch_ms"],
            "source": "profiles/k_cov_mfma_counters.json (rocprofv3 MFMA and GRBM counters, one step with "
                      "--overlap off)"}


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(d_model, d_ff, sample_tok, layer_tokens, heads_sample):
    """The fp64 oracle timed on the host's cores, on bounded samples of the workloads.

    value: the oracle's direct covariance (Y = X W, C = Y^T Y) of all 7 block matrices over
    sample_tok tokens, as tokens/s (the headline's unit).  Beside it: the oracle's seconds per
    4096 x 4096 layer at layer_tokens tokens (covariance, cyclic Jacobi eigendecomposition, factors,
    error curve), and one-core times of the single fp32 layer (whole) and of the per-head case (a
    heads_sample-token slice of its 32768 tokens, all 32 heads)."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle
    from activation_aware_rank_amd import inputs
    threads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or (os.cpu_count() or 1)
    X = inputs.block_activations(d_model, sample_tok)
    Xd = inputs.block_activations(d_ff, sample_tok, feeds_down=True)
    Ws = {m: inputs.block_weight(m, d_model, d_ff) for m in MATS}
    t0 = time.perf_counter()
    for m in MATS:
        oracle.covariance(Xd if m == "down_proj" else X, "bf16", Ws[m], "bf16")
    dt = time.perf_counter() - t0
    out = {"value": sample_tok / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
           "cpu_model": _cpu_model(),
           "sample": "fp64 direct covariance (Y = XW, C = Y^T Y) of all 7 block matrices over %d tokens "
                     "(%.1f s); eigendecomposition, error curve and factors excluded, so this is an upper "
                     "bound on the oracle's whole-step throughput" % (sample_tok, dt),
           "seconds": dt}
    del X, Xd
    if layer_tokens > 0:
        # one 4096 x 4096 layer at its calibration size: O1 + O2 + O3 + O4
        k = int(np.floor(0.6 * d_model * d_model / (2 * d_model)))
        Xl = inputs.block_activations(d_model, layer_tokens, layer=1)
        Wl = inputs.weight(d_model, d_model, "bf16", inputs.CFG_STACK, 1, 0)
        t0 = time.perf_counter()
        C = oracle.covariance(Xl, "bf16", Wl, "bf16")
        t1 = time.perf_counter()
        lam, V = oracle.eigh_large(C)
        t2 = time.perf_counter()
        oracle.truncate(oracle.widen(Wl, "bf16"), V, k)
        oracle.error_curve(lam)
        t3 = time.perf_counter()
        out["sec_per_4096_layer"] = t3 - t0
        out["sec_per_4096_layer_note"] = (
            "%d tokens, k = %d, %d threads: covariance %.1f s, eigendecomposition %.1f s (LAPACK start "
            "basis, then the cyclic Jacobi sweeps), factors and error curve %.1f s"
            % (layer_tokens, k, threads, t1 - t0, t2 - t1, t3 - t2))
        del Xl, C, V
    with threadpool_limits(limits=1):
        d = inputs.single_layer()
        t0 = time.perf_counter()
        C = oracle.covariance(d["X"], "f32", d["W"], "f32")
        lam, V = oracle.eigh(C)
        oracle.truncate(oracle.widen(d["W"], "f32"), V, 64)
        oracle.error_curve(lam)
        t1 = time.perf_counter()
        out["one_core_single_layer_s"] = t1 - t0
        if heads_sample > 0:
            dh = inputs.per_head(n_tok=heads_sample)
            t0 = time.perf_counter()
            Ch = oracle.covariance(dh["X"], "bf16", dh["W"], "bf16", n_blocks=32)
            for h in range(32):
                lam_h, V_h = oracle.eigh(Ch[h])
                oracle.error_curve(lam_h)
            t1 = time.perf_counter()
            out["one_core_per_head_tokens_per_s"] = heads_sample / (t1 - t0)
        out["one_core_note"] = ("one thread: the single fp32 layer whole (2048 tokens, 256 -> 256: covariance, "
                                "Jacobi, factors at k = 64, error curve); the per-head keys over a %d-token slice "
                                "(covariances of all 32 heads of 128, Jacobi and error curve of each), as tokens/s"
                                % heads_sample)
    return out


PEAK_F64_TFLOPS = 78.6  # MI355X dense fp64 (MFMA and vector)


def curvature_leg(torch, lrc, n_tok, seed, prec, dev, d_in=5120, d_out=13824, k=1024):
    """The curvature-weighted chain (LASER page, method 1) on a 13B-shaped FFN matrix: one warm-up
    run, then one timed run with per-stage events and the fp64 product kernel's own timings."""
    from activation_aware_rank_amd import inputs
    from activation_aware_rank_amd.curvature import curvature_truncation
    d = inputs.curvature_layer_gpu(n_tok, d_in, d_out, seed + 5, dev)
    curvature_truncation(d["X"], d["G"], d["W"], k, prec)
    torch.cuda.synchronize()
    for kern in ("k_dgemm", "k_cov_syrk", "k_cov_gemm_y"):
        lrc.lrc_timing_read(kern, reset=True)
    lrc.lrc_timing_enable(1)
    lrc.lrc_timing_set_stride("k_trd_symv", 16)
    marks = []
    t0 = time.perf_counter()
    out = curvature_truncation(d["X"], d["G"], d["W"], k, prec, marks=marks)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    lrc.lrc_timing_enable(False)
    dg_n, dg_ms, dg_fl = lrc.lrc_timing_read("k_dgemm", reset=False)
    sy_n, sy_ms, sy_fl = lrc.lrc_timing_read("k_cov_syrk", reset=True)  # a reset drops every record
    assert int(out["info"].sum().item()) == 0, "curvature chain info flags: %s" % out["info"].tolist()
    stages = {marks[i][0]: round(marks[i - 1][1].elapsed_time(marks[i][1]), 3) for i in range(1, len(marks))}
    dg_tf = dg_fl / (dg_ms / 1000.0) / 1e12 if dg_ms > 0 else 0.0
    return {
        "workload": "13B-shaped FFN matrix W %dx%d bf16, %d calibration tokens (activations and output "
                    "gradients), k = %d, eig prec %s" % (d_in, d_out, n_tok, k, "f64" if prec == 2 else "f32"),
        "seconds_per_layer": wall,
        "stage_ms": stages,
        "roofline_dgemm": {"kernel": "k_dgemm", "bound": "mfma", "achieved": dg_tf, "peak": PEAK_F64_TFLOPS,
                           "unit": "TFLOP/s", "frac": dg_tf / PEAK_F64_TFLOPS, "launches": dg_n, "total_ms": dg_ms,
                           "per_launch": "algorithmic flops = 2 M N K of the launch; a triangular output "
                                         "counts M (M + 1) K, a triangular operand M N (K + 1)"},
        "syrk_ms": sy_ms, "syrk_tflops": (sy_fl / (sy_ms / 1000.0) / 1e12) if sy_ms > 0 else 0.0,
    }


def _events(torch):
    def ev(st=None):
        e = torch.cuda.Event(enable_timing=True)
        e.record(st)
        return e
    return ev


def single_layer_leg(torch, lrc, dev, runs=5):
    """The single fp32 linear layer (2048 tokens, 256 -> 256, k = 64): covariance (fp32 path), fp32
    eigendecomposition, error curve, factors; mean of `runs` after one warm-up."""
    from activation_aware_rank_amd import inputs
    ev = _events(torch)
    d = inputs.single_layer()
    X = torch.from_numpy(d["X"]).to(dev)
    W = torch.from_numpy(d["W"]).to(dev)
    k = 64
    C = torch.empty(256, 256, dtype=torch.float32, device=dev)
    A = torch.empty(256, k, dtype=torch.float32, device=dev)
    B = torch.empty(k, 256, dtype=torch.float32, device=dev)
    info = torch.zeros(2, dtype=torch.int32, device=dev)
    ws_cov = torch.empty(lrc.lrc_cov_accumulate_workspace(lrc.LRC_F32, 2048, 256, True, 256, 1) + 256,
                         dtype=torch.uint8, device=dev)

    def run():
        C.zero_()
        lrc.lrc_cov_accumulate(X, W, C, info=info[0:1], ws=ws_cov)
        lam, V, _ = lrc.lrc_eigh(C, k, prec=lrc.LRC_F32, info=info[1:2])
        lrc.lrc_error_curve(lam[None])
        lrc.lrc_factorize(W, V, k, A, B)

    run()
    torch.cuda.synchronize()
    e0 = ev()
    for _ in range(runs):
        run()
    e1 = ev()
    torch.cuda.synchronize()
    assert int(info.sum().item()) == 0
    s = e0.elapsed_time(e1) / 1000.0 / runs
    return {"workload": "single fp32 linear layer: 2048 tokens, W 256x256, k = 64, eig prec f32",
            "seconds_per_layer": s, "tokens_per_s": 2048 / s}


def per_head_leg(torch, lrc, n_tok, seed, dev, d_model=4096, hd=128, k=32, runs=3):
    """Per-head keys (WSVD page, methodology 1): X n_tok x 4096 bf16 Student-t(3) with 8 outlier
    channels x50, W_K 4096 x 4096 bf16, 32 heads of 128: the diagonal-block covariances, 32 batched
    Jacobi eigendecompositions, error curves and factors at k = 32; mean of `runs` after a warm-up."""
    from activation_aware_rank_amd import inputs
    ev = _events(torch)
    d = inputs.per_head_gpu(n_tok, d_model, seed + 11, dev)
    X, W = d["X"], d["W"]
    nh = d_model // hd
    C = torch.empty(nh, hd, hd, dtype=torch.float32, device=dev)
    lam = torch.empty(nh, hd, dtype=torch.float64, device=dev)
    V = torch.empty(nh, hd, k, dtype=torch.float32, device=dev)
    eps = torch.empty(nh, hd + 1, dtype=torch.float64, device=dev)
    A = torch.empty(nh, d_model, k, dtype=torch.float32, device=dev)
    B = torch.empty(nh, k, hd, dtype=torch.float32, device=dev)
    info = torch.zeros(nh + 1, dtype=torch.int32, device=dev)
    ws_cov = torch.empty(lrc.lrc_cov_accumulate_workspace(lrc.LRC_BF16, n_tok, d_model, True, d_model, nh),
                         dtype=torch.uint8, device=dev)

    def run(marks):
        C.zero_()
        marks.append(ev())
        lrc.lrc_cov_accumulate(X, W, C, n_blocks=nh, info=info[0:1], ws=ws_cov)
        marks.append(ev())
        lrc.lrc_eigh(C, k, lam=lam, V=V, info=info[1:])
        lrc.lrc_error_curve(lam, eps=eps)
        marks.append(ev())
        lrc.lrc_factorize(W, V, k, A, B, d_in=d_model, d_out=hd, batch=nh, stride_w=hd, stride_v=hd * k,
                          stride_a=d_model * k, stride_b=k * hd)
        marks.append(ev())

    run([])
    torch.cuda.synchronize()
    recs = []
    for _ in range(runs):
        m = []
        run(m)
        recs.append(m)
    torch.cuda.synchronize()
    assert int(info.sum().item()) == 0, "per-head info flags: %s" % info.tolist()
    cov = sum(m[0].elapsed_time(m[1]) for m in recs) / runs
    eig = sum(m[1].elapsed_time(m[2]) for m in recs) / runs
    fac = sum(m[2].elapsed_time(m[3]) for m in recs) / runs
    tot = (cov + eig + fac) / 1000.0
    fl = n_tok * (2 * d_model * d_model + nh * hd * (hd + 1))
    return {"workload": "per-head keys: %d tokens x 4096 (Student-t(3), 8 outlier channels x50), W_K 4096x4096, "
                        "32 heads of 128, k = 32" % n_tok,
            "tokens_per_s": n_tok / tot, "cov_tokens_per_s": n_tok / (cov / 1000.0),
            "cov_tflops_algorithmic": fl / (cov / 1000.0) / 1e12,
            "stage_ms": {"covariance": round(cov, 3), "eigh_and_error_curve": round(eig, 3), "factors": round(fac, 3)}}


def stack_leg(torch, lrc, n_layers, n_tok, seed, prec, dev, d_model=4096, d_ff=11008, rho=0.8, sets=3,
              cov_range=True):
    """The 32-layer stack end to end (FLRC page, method 1; LASER page, method 2): for every layer its
    own n_tok calibration tokens, the 7 covariances (cov_range: gate/up's in the coordinates of
    range(W^T), B = (X L)^T (X L) with W W^T = L L^T), one call decomposing all 7 (gate/up through a
    basis of range(W^T)) with k_cap = floor(d_in d_out / (d_in + d_out)) vectors each, the error curves; then
    the Fisher scores of all 224 matrices, the greedy allocation of rho of the parameters from the real
    eigenvalues, and the factors of every matrix at its allocated rank.  One timed pass (inputs drawn
    before the clock starts, except each layer's calibration tokens, which are drawn into the same
    buffers before that layer's covariances and timed apart)."""
    import numpy as np

    from activation_aware_rank_amd import inputs
    ev = _events(torch)
    sh = shapes(d_model, d_ff)
    g = torch.Generator(device=dev)
    g.manual_seed(seed + 7)
    Ws, Gs = inputs.stack_weights_gpu(g, n_layers, d_model, d_ff, dev)
    X = torch.empty(n_tok, d_model, dtype=torch.bfloat16, device=dev)
    Xd = torch.empty(n_tok, d_ff, dtype=torch.bfloat16, device=dev)
    kcap = {m: (di * do) // (di + do) for m, (di, do) in sh.items()}
    groups = {}
    for m in MATS:
        groups.setdefault((sh[m][1], kcap[m]), []).append(m)
    where = {m: (gk, ms.index(m)) for gk, ms in groups.items() for m in ms}
    V = [{m: torch.empty(sh[m][1], kcap[m], dtype=torch.float32, device=dev) for m in MATS} for _ in range(n_layers)]
    lam = [{m: torch.empty(sh[m][1], dtype=torch.float64, device=dev) for m in MATS} for _ in range(n_layers)]
    eps = [{m: torch.empty(sh[m][1] + 1, dtype=torch.float64, device=dev) for m in MATS} for _ in range(n_layers)]
    # `sets` sets of the per-layer buffers: layer l's decompositions (on side stream l % sets, from a
    # host thread of their own) overlap the next layers' covariances on the main stream; a set is
    # reused `sets` layers later, after its decompositions and copies are done
    NS = max(1, sets)
    proj = {gk: cov_range and sh[ms[0]][0] < gk[0] for gk, ms in groups.items()}  # B = (X L)^T (X L)
    gd = {gk: sh[ms[0]][0] if proj[gk] else gk[0] for gk, ms in groups.items()}  # order of the stored matrices
    gC = [{gk: torch.empty(len(ms), gd[gk], gd[gk], dtype=torch.float32, device=dev) for gk, ms in groups.items()}
          for _ in range(NS)]
    # the factors of W W^T, per buffer set (a set's decompositions read them on their side stream)
    gL = [{gk: torch.zeros(len(ms), sh[ms[0]][0], sh[ms[0]][0], dtype=torch.float64, device=dev)
           for gk, ms in groups.items() if proj[gk]} for _ in range(NS)]
    Lf = [{m: gL[si][where[m][0]][where[m][1]] for m in MATS if proj[where[m][0]]} for si in range(NS)]
    ginfo_g = [{gk: torch.zeros(len(ms), dtype=torch.int32, device=dev) for gk, ms in groups.items()} for _ in range(NS)]
    cinfo = torch.zeros(1, dtype=torch.int32, device=dev)
    bad = [torch.zeros(1, dtype=torch.int64, device=dev) for _ in range(NS + 1)]  # per set, and the covariances'
    # each group decomposes from stacked buffers (the range bases of gate/up included) and its
    # eigenvalues and vectors are copied out to the per-matrix buffers
    gV = [{gk: torch.empty(len(ms), gk[0], gk[1], dtype=torch.float32, device=dev) for gk, ms in groups.items()}
          for _ in range(NS)]
    glam = [{gk: torch.empty(len(ms), gk[0], dtype=torch.float64, device=dev) for gk, ms in groups.items()}
            for _ in range(NS)]
    ws_cov = torch.empty(max([lrc.lrc_cov_accumulate_workspace(lrc.LRC_BF16, n_tok, di, True, do, 1)
                              for di, do in sh.values()] +
                             [lrc.lrc_cov_accumulate_range_workspace(n_tok, sh[m][0]) for m in Lf[0]]),
                         dtype=torch.uint8, device=dev)
    ws_eig = [torch.empty(lrc.lrc_eigh_multi_workspace(
        [(gk[0], len(ms), gk[1], sh[ms[0]][0] if sh[ms[0]][0] < gk[0] else 0, proj[gk]) for gk, ms in groups.items()],
        prec), dtype=torch.uint8, device=dev) for _ in range(NS)]
    gW = [{gk: torch.empty(len(ms), sh[ms[0]][0], gk[0], dtype=torch.bfloat16, device=dev)
           for gk, ms in groups.items() if sh[ms[0]][0] < gk[0]} for _ in range(NS)]
    side = [torch.cuda.Stream(device=dev) for _ in range(NS)]
    # the range factors of a layer on streams of their own, beside that layer's first covariances
    fst = {m: torch.cuda.Stream(device=dev) for m in Lf[0]}
    ws_rfm = {m: torch.empty(lrc.lrc_range_factor_workspace(*sh[m]), dtype=torch.uint8, device=dev) for m in Lf[0]}
    finfo = {m: torch.zeros(1, dtype=torch.int32, device=dev) for m in Lf[0]}
    offs_h = [0] + list(np.cumsum([kcap[m] for _ in range(n_layers) for m in MATS]))
    offs = torch.tensor(offs_h, dtype=torch.int64, device=dev)
    lam_packed = torch.empty(int(offs_h[-1]), dtype=torch.float64, device=dev)
    eps0 = torch.empty(n_layers * 7, dtype=torch.float64, device=dev)
    cost = torch.tensor([sum(sh[m]) for _ in range(n_layers) for m in MATS], dtype=torch.int64, device=dev)
    budget = int(np.floor(rho * n_layers * sum(di * do for di, do in sh.values())))
    alpha = torch.empty(n_layers * 7, dtype=torch.float64, device=dev)
    k_out = torch.empty(n_layers * 7, dtype=torch.int32, device=dev)
    ws_alc = torch.empty(lrc.lrc_allocate_ranks_workspace(n_layers * 7, lam_packed.numel()), dtype=torch.uint8,
                         device=dev)
    Gl = [Gs[l][m] for l in range(n_layers) for m in MATS]
    Wl = [Ws[l][m] for l in range(n_layers) for m in MATS]
    ws_fsh = torch.empty(lrc.lrc_fisher_scores_workspace([w.numel() for w in Wl]), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    gen_ev, cov_ev, eig_ev = [], [], []

    def decompose(layer, si, ready):
        # runs on a host thread of its own: the library call returns once its launches are enqueued
        sd = side[si]
        with torch.cuda.stream(sd):
            sd.wait_event(ready)
            e0 = ev(sd)
            lrc.lrc_eigh_multi([(gC[si][gk], gk[1], glam[si][gk], gV[si][gk], ginfo_g[si][gk], gW[si].get(gk),
                                 proj[gk], gL[si].get(gk)) for gk in groups], prec=prec, ws=ws_eig[si], stream=sd)
            for gk, ms in groups.items():
                bad[si] += ginfo_g[si][gk].abs().sum()
                for j, m in enumerate(ms):
                    lam[layer][m].copy_(glam[si][gk][j])
                    V[layer][m].copy_(gV[si][gk][j])
            for i, m in enumerate(MATS):
                lrc.lrc_error_curve(lam[layer][m][None], eps=eps[layer][m][None], stream=sd)
                q = layer * 7 + i
                lam_packed[offs_h[q]:offs_h[q] + kcap[m]].copy_(lam[layer][m][:kcap[m]])
                eps0[q:q + 1].copy_(eps[layer][m][0:1])
            eig_ev.append((e0, ev(sd)))

    threads = [None] * NS
    done = [None] * NS
    t0 = time.perf_counter()
    for layer in range(n_layers):
        si = layer % NS
        if threads[si] is not None:  # this set's previous decompositions enqueued; the GPU waits for them
            threads[si].join()
            stream.wait_stream(side[si])
        a0 = ev(stream)
        fev = {}
        for m in Lf[si]:  # after this set's previous decompositions (the stream waited for them above)
            fst[m].wait_stream(stream)
            lrc.lrc_range_factor(Ws[layer][m], L=Lf[si][m], info=finfo[m], ws=ws_rfm[m], stream=fst[m])
            fev[m] = ev(fst[m])
        inputs.stack_layer_gpu(g, n_tok, d_model, d_ff, dev, X, Xd)
        a1 = ev(stream)
        for i, m in enumerate(MATS):
            gk, j = where[m]
            C = gC[si][gk][j]
            C.zero_()
            if m in Lf[si]:
                stream.wait_event(fev[m])
                bad[NS] += finfo[m]
                lrc.lrc_cov_accumulate_range(X, Lf[si][m], C, info=cinfo, ws=ws_cov)
            else:
                lrc.lrc_cov_accumulate(Xd if m == "down_proj" else X, Ws[layer][m], C, info=cinfo, ws=ws_cov)
            bad[NS] += cinfo
        for gk, ms in groups.items():
            if gk in gW[si]:
                for j, m in enumerate(ms):
                    gW[si][gk][j].copy_(Ws[layer][m])
        a2 = ev(stream)
        gen_ev.append((a0, a1))
        cov_ev.append((a1, a2))
        threads[si] = threading.Thread(target=decompose, args=(layer, si, a2))
        threads[si].start()
    for t in threads:
        if t is not None:
            t.join()
    for sd in side:
        stream.wait_stream(sd)
    b0 = ev()
    lrc.lrc_fisher_scores(Gl, Wl, alpha=alpha, ws=ws_fsh)
    lrc.lrc_allocate_ranks(alpha, lam_packed, offs, eps0, cost, budget, k_out=k_out, ws=ws_alc)
    b1 = ev()
    kk = k_out.cpu().tolist()
    # the factors at the allocated ranks, into buffers of the largest rank (no allocation per matrix)
    kmax = max(kk)
    A_buf = torch.empty(max(di for di, do in sh.values()) * kmax, dtype=torch.float32, device=dev)
    B_buf = torch.empty(max(do for di, do in sh.values()) * kmax, dtype=torch.float32, device=dev)
    fac_ev = []
    for layer in range(n_layers):
        for i, m in enumerate(MATS):
            km = kk[layer * 7 + i]
            if km <= 0:
                continue
            di, do = sh[m]
            f0 = ev(stream)
            lrc.lrc_factorize(Ws[layer][m], V[layer][m], km, A_buf[:di * km].view(di, km), B_buf[:km * do].view(km, do))
            fac_ev.append((f0, ev(stream)))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    t_gen = sum(x.elapsed_time(y) for x, y in gen_ev) / 1000.0
    fac_ms = sum(x.elapsed_time(y) for x, y in fac_ev)
    marks = {"cov": sum(x.elapsed_time(y) for x, y in cov_ev), "eig": sum(x.elapsed_time(y) for x, y in eig_ev)}
    assert int(sum(b.item() for b in bad)) == 0, "stack: device info flags set"
    used = sum(kk[q] * sum(sh[MATS[q % 7]]) for q in range(len(kk)))
    return {"workload": "%d-layer LLaMA-7B-shaped stack (%d matrices, %d parameters), %d calibration tokens per "
                        "layer, eig prec %s, k_cap vectors per matrix, greedy allocation of %.0f%% of the parameters%s"
                        % (n_layers, n_layers * 7, n_layers * sum(di * do for di, do in sh.values()), n_tok,
                           "f32" if prec == lrc.LRC_F32 else "f64", rho * 100,
                           "; gate/up covariances in the coordinates of range(W^T)" if Lf[0] else ""),
            "seconds": wall, "seconds_per_layer": wall / n_layers,
            "tokens_per_s": n_layers * n_tok / wall,
            "stage_s": {"covariances": marks["cov"] / 1000.0, "eigh_and_error_curves": marks["eig"] / 1000.0,
                        "fisher_and_allocation": b0.elapsed_time(b1) / 1000.0, "factors": fac_ms / 1000.0},
            "stage_note": "layer l's decompositions and error curves run on a side stream during layer l+1's "
                          "input generation and covariances, so the stage times overlap and add up to more than "
                          "the wall time",
            "input_generation_s_included": t_gen,
            "allocated_parameters": used, "budget": budget,
            "rank_range": [min(kk), max(kk)]}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--tokens", type=int, default=524288)
    ap.add_argument("--d-model", type=int, default=4096)
    ap.add_argument("--d-ff", type=int, default=11008)
    ap.add_argument("--ratio", type=float, default=0.6)
    ap.add_argument("--prec", choices=("f32", "f64"), default="f32", help="eigensolver working precision")
    ap.add_argument("--cpu-sample", type=int, default=1024, help="tokens for the CPU oracle baseline (0: skip)")
    ap.add_argument("--seed", type=int, default=20261203)
    ap.add_argument("--breakdown", action="store_true", help="print per-call timings to stderr")
    ap.add_argument("--calib-copy-mb", type=int, default=1024, help="size of the byte-counter reference copy")
    ap.add_argument("--curvature-tokens", type=int, default=131072,
                    help="tokens of the curvature-weighted 13B FFN leg, timed after the block (0: skip)")
    ap.add_argument("--curvature-prec", choices=("f32", "f64"), default="f64")
    ap.add_argument("--layer-runs", type=int, default=2,
                    help="runs of one 4096x4096 layer on its own after the timed steps (0: skip)")
    ap.add_argument("--overlap", choices=("on", "off"), default="on",
                    help="decompose each group of matrices (grouped by output width and rank) as soon as its "
                         "covariances are done, on a side stream from a host thread of its own, while the "
                         "remaining covariances run")
    ap.add_argument("--overlap-chunk", type=int, default=0,
                    help="with --overlap on: split groups into parts of this many matrices (0: whole groups)")
    ap.add_argument("--overlap-order", choices=("small-first", "large-first", "most-first", "rank-small", "rank-large"),
                    default="rank-small",
                    help="small-first: the groups of one output width decomposed in one call (the library "
                         "tridiagonalises matrices of one order in lockstep), narrow widths first; large-first / "
                         "most-first: one group at a time, largest n or most matrices first; rank-small / "
                         "rank-large: the groups of one tridiagonal order (d_in for a projected covariance) and "
                         "rank in one call (lockstep and batched throughout), smaller or larger rank first")
    ap.add_argument("--factored-steps", type=int, default=2,
                    help="timed steps of the variant that forms the covariances from X^T X (0: skip)")
    ap.add_argument("--eig-range", choices=("on", "off"), default="on",
                    help="on: covariances of Y = X W with d_in < d_out (gate/up) are decomposed through a basis of "
                         "range(W^T) (their rank is at most d_in); off: the full decomposition of every covariance")
    ap.add_argument("--cov-range", choices=("on", "off"), default="on",
                    help="with --eig-range on: those covariances are accumulated in the coordinates of the basis, "
                         "B = (X L)^T (X L) with W W^T = L L^T (d_in x d_in), and decomposed from B; off: the full "
                         "d_out x d_out covariance is accumulated and projected by the decomposition")
    ap.add_argument("--full-steps", type=int, default=2,
                    help="timed steps of the variant that forms every covariance in full (gate/up 11008 x 11008, "
                         "then projected by the decomposition), stages in series (0: skip; only with --cov-range on)")
    ap.add_argument("--timing-stride", type=int, default=16,
                    help="time every s-th launch of the per-column symmetric product in the timed steps")
    ap.add_argument("--layer-tokens", type=int, default=65536,
                    help="also time one 4096x4096 layer over this many tokens (a stack layer's calibration size; 0: skip)")
    ap.add_argument("--heads-tokens", type=int, default=32768, help="tokens of the per-head keys leg (0: skip)")
    ap.add_argument("--single", choices=("on", "off"), default="on", help="the single fp32 layer leg")
    ap.add_argument("--stack-layers", type=int, default=32, help="layers of the stack leg (0: skip)")
    ap.add_argument("--stack-tokens", type=int, default=65536, help="calibration tokens per layer of the stack leg")
    ap.add_argument("--stack-sets", type=int, default=3,
                    help="buffer sets of the stack leg: layers whose decompositions may run at once")
    ap.add_argument("--cpu-layer-tokens", type=int, default=65536,
                    help="tokens of the oracle's 4096x4096 layer in the CPU baseline (0: skip)")
    ap.add_argument("--cpu-heads-sample", type=int, default=4096,
                    help="token slice of the per-head keys for the oracle's one-core time (0: skip)")
    a = ap.parse_args()
    if a.gpus != 1:
        print("bench.py runs on exactly one GPU; --gpus %d is not supported (the path would shard matrices "
              "or token ranges across GPUs)" % a.gpus, file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from activation_aware_rank_amd import lrc

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    prec = lrc.LRC_F32 if a.prec == "f32" else lrc.LRC_F64
    sh = shapes(a.d_model, a.d_ff)
    ks = {m: int(np.floor(a.ratio * di * do / (di + do))) for m, (di, do) in sh.items()}
    from activation_aware_rank_amd import inputs
    blk = inputs.block_gpu(a.tokens, a.d_model, a.d_ff, a.seed, dev)
    X, Xd, W, G = blk["X"], blk["Xd"], blk["W"], blk["G"]
    del blk
    # outputs and workspaces allocated once, outside the timed region.  The matrices are grouped
    # by output width and rank (q/k/v/o: 4096 and 1228, down: 4096 and 1791, gate/up: 11008 and
    # 1791); each group's covariances sit in one stack, and all groups go through one call that
    # decomposes up to eight matrices at once.
    groups = {}
    for m in MATS:
        groups.setdefault((sh[m][1], ks[m]), []).append(m)
    # groups whose covariance has rank <= d_in < d_out: their weights in one stack (the range bases of
    # the decomposition; the covariance calls read the same storage)
    gW = {}
    if a.eig_range == "on":
        for g, ms in groups.items():
            if sh[ms[0]][0] < g[0]:
                gW[g] = torch.stack([W[m] for m in ms])
                for i, m in enumerate(ms):
                    W[m] = gW[g][i]
    # --cov-range on: those groups' covariances in the basis's coordinates, B = (X L)^T (X L), d_in x d_in,
    # from the factor L of W W^T (one per matrix, formed in the step)
    gP = set(gW) if a.cov_range == "on" else set()
    gd = {g: (sh[ms[0]][0] if g in gP else g[0]) for g, ms in groups.items()}  # order of the stored matrices
    gC = {g: torch.empty(len(ms), gd[g], gd[g], dtype=torch.float32, device=dev) for g, ms in groups.items()}
    gL = {g: torch.zeros(len(groups[g]), gd[g], gd[g], dtype=torch.float64, device=dev) for g in gP}
    glam = {g: torch.empty(len(ms), g[0], dtype=torch.float64, device=dev) for g, ms in groups.items()}
    # V's rows padded to a multiple of four values (16 bytes), so that the factor products can load
    # four consecutive values of V at a time; the decompositions write the first n_vec of each row
    gV = {g: torch.empty(len(ms), g[0], (g[1] + 3) // 4 * 4, dtype=torch.float32, device=dev)[:, :, :g[1]]
          for g, ms in groups.items()}
    geps = {g: torch.empty(len(ms), g[0] + 1, dtype=torch.float64, device=dev) for g, ms in groups.items()}
    ginfo = {g: torch.zeros(len(ms), dtype=torch.int32, device=dev) for g, ms in groups.items()}
    where = {m: (g, ms.index(m)) for g, ms in groups.items() for m in ms}
    Lf = {m: gL[where[m][0]][where[m][1]] for m in MATS if where[m][0] in gP}
    rinfo = torch.zeros(len(MATS), dtype=torch.int32, device=dev)
    C = {m: gC[where[m][0]][where[m][1]] for m in MATS}
    lam = {m: glam[where[m][0]][where[m][1]] for m in MATS}
    V = {m: gV[where[m][0]][where[m][1]] for m in MATS}
    eps = {m: geps[where[m][0]][where[m][1]] for m in MATS}
    A = {m: torch.empty(di, ks[m], dtype=torch.float32, device=dev) for m, (di, do) in sh.items()}
    # a projected group's factors A = W V = L U come out of its decomposition (stacked per group)
    gA = {g: torch.empty(len(groups[g]), sh[groups[g][0]][0], g[1], dtype=torch.float32, device=dev) for g in gP}
    for g in gP:
        for i, m in enumerate(groups[g]):
            A[m] = gA[g][i]
    B = {m: torch.empty(ks[m], do, dtype=torch.float32, device=dev) for m, (di, do) in sh.items()}
    info = torch.zeros(8, dtype=torch.int32, device=dev)
    ws_cov = torch.empty(max([lrc.lrc_cov_accumulate_workspace(lrc.LRC_BF16, a.tokens, di, True, do, 1)
                              for di, do in sh.values()] +
                             [lrc.lrc_cov_accumulate_range_workspace(a.tokens, gd[g]) for g in gP]),
                         dtype=torch.uint8, device=dev)
    ws_rf = {m: torch.empty(lrc.lrc_range_factor_workspace(*sh[m]), dtype=torch.uint8, device=dev)
             for m in MATS if where[m][0] in gP}
    ws_eig = torch.empty(lrc.lrc_eigh_multi_workspace(
        [(g[0], len(ms), g[1], sh[ms[0]][0] if g in gW else 0, g in gP) for g, ms in groups.items()], prec),
        dtype=torch.uint8, device=dev)
    eig_groups = [(gC[g], g[1], glam[g], gV[g], ginfo[g], gW.get(g), g in gP, gL.get(g), gA.get(g)) for g in groups]
    gkey = "+".join("%dx%d_k%d" % (len(ms), g[0], g[1]) for g, ms in groups.items())
    # overlap: covariances group by group, largest n first; each group's eigendecompositions and
    # error curves on a side stream of its own (default priority) with a workspace of its own
    # phases: the covariances of a phase's groups, then (on a side stream) one call decomposing them all
    # a phase is a list of parts (g, lo, hi): members lo .. hi-1 of group g; --overlap-chunk splits
    # larger groups into parts of that many members, each a phase of its own
    def parts_of(g):
        n, c = len(groups[g]), a.overlap_chunk if a.overlap_chunk > 0 else len(groups[g])
        return [(g, lo, min(lo + c, n)) for lo in range(0, n, c)]
    if a.overlap_order == "small-first":  # groups of one output width together, narrow widths first
        widths = sorted({g[0] for g in groups})
        phases = [[pt for g in groups if g[0] == wd for pt in parts_of(g)] for wd in widths]
    elif a.overlap_order in ("rank-small", "rank-large"):  # groups of one tridiagonal order and rank together
        keys = sorted({(gd[g], g[1]) for g in groups}, key=lambda x: (x[1], x[0]),
                      reverse=a.overlap_order == "rank-large")
        phases = [[pt for g in groups if (gd[g], g[1]) == kk for pt in parts_of(g)] for kk in keys]
    else:
        g_order = sorted(groups, key=lambda g: -g[0] if a.overlap_order == "large-first" else len(groups[g]) * -1)
        phases = [[pt] for g in g_order for pt in parts_of(g)]
    side = [torch.cuda.Stream(device=dev) for _ in phases]
    ws_eig_g = [torch.empty(lrc.lrc_eigh_multi_workspace(
        [(g[0], hi - lo, g[1], sh[groups[g][0]][0] if g in gW else 0, g in gP) for g, lo, hi in ph], prec),
        dtype=torch.uint8, device=dev) for ph in phases] if a.overlap == "on" else []
    pname = ["+".join("%dx%d_k%d" % (hi - lo, g[0], g[1]) for g, lo, hi in ph) for ph in phases]
    kcap = {m: (di * do) // (di + do) for m, (di, do) in sh.items()}
    offs_h = [0] + list(np.cumsum([kcap[m] for m in MATS]))
    offs = torch.tensor(offs_h, dtype=torch.int64, device=dev)
    lam_packed = torch.empty(int(offs_h[-1]), dtype=torch.float64, device=dev)
    eps0 = torch.empty(len(MATS), dtype=torch.float64, device=dev)
    cost = torch.tensor([sum(sh[m]) for m in MATS], dtype=torch.int64, device=dev)
    budget = int(np.floor(a.ratio * sum(di * do for di, do in sh.values())))
    ws_alc = torch.empty(lrc.lrc_allocate_ranks_workspace(len(MATS), lam_packed.numel()), dtype=torch.uint8,
                         device=dev)
    ws_fsh = torch.empty(lrc.lrc_fisher_scores_workspace([G[m].numel() for m in MATS]), dtype=torch.uint8,
                         device=dev)
    alpha = torch.empty(len(MATS), dtype=torch.float64, device=dev)
    k_out = torch.empty(len(MATS), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()

    def ev(st):
        e = torch.cuda.Event(enable_timing=True)
        e.record(st)
        return e

    fstream = torch.cuda.Stream(device=dev)  # the range factors, off the covariance stream
    fready = {}

    def factors(times):
        # L of every matrix with a projected covariance, on a side stream from the step's start; the
        # covariance stream waits for each only where it needs it (it also serves the decomposition)
        fstream.wait_stream(stream)
        for m in MATS:
            if m in Lf:
                i = MATS.index(m)
                e0 = ev(fstream)
                lrc.lrc_range_factor(W[m], L=Lf[m], info=rinfo[i:i + 1], ws=ws_rf[m], stream=fstream)
                fready[m] = ev(fstream)
                times.append((m + ".factor", e0, fready[m]))

    def cov(m, times):
        i = MATS.index(m)
        xin = Xd if m == "down_proj" else X
        C[m].zero_()
        e0 = ev(stream)
        if m in Lf:  # B = (X L)^T (X L) in the coordinates of range(W^T), L from W W^T = L L^T
            stream.wait_event(fready[m])
            lrc.lrc_cov_accumulate_range(xin, Lf[m], C[m], info=info[i:i + 1], ws=ws_cov)
        else:
            lrc.lrc_cov_accumulate(xin, W[m], C[m], info=info[i:i + 1], ws=ws_cov)
        e1 = ev(stream)
        times.append((m + ".cov", e0, e1))

    def eig_group(pi, ready, times):
        # runs on a host thread of its own: the library call returns once its launches are
        # enqueued, which takes about as long as they run
        sg = side[pi]
        sg.wait_event(ready)
        e0 = ev(sg)
        lrc.lrc_eigh_multi([(gC[g][lo:hi], g[1], glam[g][lo:hi], gV[g][lo:hi], ginfo[g][lo:hi],
                             gW[g][lo:hi] if g in gW else None, g in gP, gL[g][lo:hi] if g in gP else None,
                             gA[g][lo:hi] if g in gP else None)
                            for g, lo, hi in phases[pi]], prec=prec, ws=ws_eig_g[pi], stream=sg)
        for g, lo, hi in phases[pi]:
            lrc.lrc_error_curve(glam[g][lo:hi], eps=geps[g][lo:hi], stream=sg)
        e1 = ev(sg)
        times.append(("eigh." + pname[pi], e0, e1))
        # the group's factors at the fixed ranks right after its eigenvectors, on the same stream
        # (they do not depend on the allocation), so that only the last group's stay in the tail
        for g, lo, hi in phases[pi]:
            for m in groups[g][lo:hi]:
                f0 = ev(sg)
                lrc.lrc_factorize(W[m], V[m], ks[m], None if m in Lf else A[m], B[m], stream=sg)
                f1 = ev(sg)
                times.append((m + ".fac", f0, f1))

    def tail(times, factors=True, a_from_eig=True):
        # a_from_eig: the projected groups' decompositions formed A (only B is formed here for them)
        for m in MATS if factors else ():
            e0 = ev(stream)
            lrc.lrc_factorize(W[m], V[m], ks[m], None if (a_from_eig and m in Lf) else A[m], B[m])
            e1 = ev(stream)
            times.append((m + ".fac", e0, e1))
        e5 = ev(stream)
        lrc.lrc_fisher_scores([G[m] for m in MATS], [W[m] for m in MATS], alpha=alpha, ws=ws_fsh)
        e6 = ev(stream)
        for i, m in enumerate(MATS):  # gather lambda_m[:K_m] and eps_{m,0} (device copies)
            lam_packed[offs_h[i]:offs_h[i] + kcap[m]].copy_(lam[m][:kcap[m]])
            eps0[i:i + 1].copy_(eps[m][0:1])
        e7 = ev(stream)
        lrc.lrc_allocate_ranks(alpha, lam_packed, offs, eps0, cost, budget, k_out=k_out, ws=ws_alc)
        e8 = ev(stream)
        times.append(("fisher", e5, e6))
        times.append(("alloc", e7, e8))

    def step(times):
        factors(times)
        if a.overlap == "on":
            threads = []
            for pi, ph in enumerate(phases):
                for g, lo, hi in ph:
                    for m in groups[g][lo:hi]:
                        cov(m, times)
                t = threading.Thread(target=eig_group, args=(pi, ev(stream), times))
                t.start()
                threads.append(t)
            for t in threads:
                t.join()
            for sd in side:
                stream.wait_stream(sd)
            tail(times, factors=False)
            return
        else:
            for m in MATS:
                cov(m, times)
            # every eigendecomposition of the block in one call: the library runs up to eight at once
            e0 = ev(stream)
            lrc.lrc_eigh_multi(eig_groups, prec=prec, ws=ws_eig)
            for g in groups:
                lrc.lrc_error_curve(glam[g], eps=geps[g])
            e1 = ev(stream)
            times.append(("eigh." + gkey, e0, e1))
        tail(times)

    def factored_leg():
        """The same step with the covariances formed from the input covariances (H = X^T X for the six
        matrices that read X, H_d = X_d^T X_d for down, then C_m = W_m^T H W_m in fp64), the stages in
        series; timed like the main step."""
        H = torch.empty(a.d_model, a.d_model, dtype=torch.float32, device=dev)
        Hd = torch.empty(a.d_ff, a.d_ff, dtype=torch.float32, device=dev)
        ws_h = torch.empty(max(lrc.lrc_cov_accumulate_workspace(lrc.LRC_BF16, a.tokens, d, False, d, 1)
                               for d in (a.d_model, a.d_ff)), dtype=torch.uint8, device=dev)
        ws_f = torch.empty(max(lrc.lrc_cov_from_input_workspace(di, gd[where[m][0]]) for m, (di, do) in sh.items()),
                           dtype=torch.uint8, device=dev)

        def fstep(times):
            e0 = ev(stream)
            H.zero_()
            lrc.lrc_cov_accumulate(X, None, H, info=info[0:1], ws=ws_h)
            Hd.zero_()
            lrc.lrc_cov_accumulate(Xd, None, Hd, info=info[1:2], ws=ws_h)
            e1 = ev(stream)
            for m in MATS:
                if m in Lf:  # B = L^T H L for the matrices decomposed from the basis's coordinates
                    lrc.lrc_range_factor(W[m], L=Lf[m], info=rinfo[MATS.index(m):MATS.index(m) + 1], ws=ws_rf[m])
                lrc.lrc_cov_from_input(Hd if m == "down_proj" else H, Lf.get(m, W[m]), C=C[m], ws=ws_f)
            e2 = ev(stream)
            lrc.lrc_eigh_multi(eig_groups, prec=prec, ws=ws_eig)
            for g in groups:
                lrc.lrc_error_curve(glam[g], eps=geps[g])
            e3 = ev(stream)
            times += [("input_cov", e0, e1), ("cov_from_input", e1, e2), ("eigh", e2, e3)]
            tail(times)

        for _ in range(a.warmup):
            fstep([])
        torch.cuda.synchronize()
        recs_f = []
        t0f = time.perf_counter()
        for _ in range(a.factored_steps):
            r = []
            fstep(r)
            recs_f.append(r)
        torch.cuda.synchronize()
        wall_f = time.perf_counter() - t0f
        assert int(info.sum().item()) == 0, "device info flags set: %s" % info.tolist()
        per_f = {}
        for r in recs_f:
            for key, x0, x1 in r:
                per_f.setdefault(key, []).append(x0.elapsed_time(x1))
        avg_f = {k: round(float(np.mean(v)), 3) for k, v in per_f.items() if k in ("input_cov", "cov_from_input", "eigh")}
        ms_f = wall_f * 1000.0 / a.factored_steps
        return {"metric": "calibration tokens/s into Y^T Y", "value": a.tokens / (ms_f / 1000.0), "unit": "tokens/s",
                "ms_per_step": ms_f, "steps": a.factored_steps, "breakdown_ms": avg_f,
                "cov_tokens_per_s": a.tokens / ((avg_f["input_cov"] + avg_f["cov_from_input"]) / 1000.0),
                "note": "same block, inputs, eigendecompositions, factors, Fisher scores and allocation as the main "
                        "step; the covariances by C_m = W_m^T (X^T X) W_m (one bf16 SYRK of X and one of X_d, then "
                        "two fp64 products per matrix; %s) instead of the fused GEMM + split SYRK; stages in series"
                        % ("for gate/up B = L^T (X^T X) L, W W^T = L L^T" if gP else "all in full")}

    def full_leg():
        """The same step with every covariance formed in full (gate/up as 11008 x 11008 C, decomposed
        through their range basis), the stages in series; timed like the main step."""
        Cfull = {g: torch.empty(len(groups[g]), g[0], g[0], dtype=torch.float32, device=dev) for g in gP}
        ws_covf = torch.empty(max(lrc.lrc_cov_accumulate_workspace(lrc.LRC_BF16, a.tokens, di, True, do, 1)
                                  for di, do in sh.values()), dtype=torch.uint8, device=dev)
        ws_eigf = torch.empty(lrc.lrc_eigh_multi_workspace(
            [(g[0], len(ms), g[1], sh[ms[0]][0] if g in gW else 0) for g, ms in groups.items()], prec),
            dtype=torch.uint8, device=dev)
        groups_f = [((Cfull[g] if g in gP else gC[g]), g[1], glam[g], gV[g], ginfo[g], gW.get(g)) for g in groups]

        def fstep(times):
            e0 = ev(stream)
            for m in MATS:
                i = MATS.index(m)
                g, j = where[m]
                Cm = Cfull[g][j] if g in gP else C[m]
                Cm.zero_()
                lrc.lrc_cov_accumulate(Xd if m == "down_proj" else X, W[m], Cm, info=info[i:i + 1], ws=ws_covf)
            e1 = ev(stream)
            lrc.lrc_eigh_multi(groups_f, prec=prec, ws=ws_eigf)
            for g in groups:
                lrc.lrc_error_curve(glam[g], eps=geps[g])
            e2 = ev(stream)
            times += [("cov", e0, e1), ("eigh", e1, e2)]
            tail(times, a_from_eig=False)

        for _ in range(a.warmup):
            fstep([])
        torch.cuda.synchronize()
        recs_f = []
        t0f = time.perf_counter()
        for _ in range(a.full_steps):
            r = []
            fstep(r)
            recs_f.append(r)
        torch.cuda.synchronize()
        wall_f = time.perf_counter() - t0f
        assert int(info.sum().item()) == 0, "device info flags set: %s" % info.tolist()
        per_f = {}
        for r in recs_f:
            for key, x0, x1 in r:
                per_f.setdefault(key, []).append(x0.elapsed_time(x1))
        avg_f = {k: round(float(np.mean(v)), 3) for k, v in per_f.items() if k in ("cov", "eigh")}
        ms_f = wall_f * 1000.0 / a.full_steps
        kf = k_out.cpu().tolist()
        del Cfull, ws_covf, ws_eigf
        return {"metric": "calibration tokens/s into Y^T Y", "value": a.tokens / (ms_f / 1000.0), "unit": "tokens/s",
                "ms_per_step": ms_f, "steps": a.full_steps, "breakdown_ms": avg_f,
                "cov_tokens_per_s": a.tokens / (avg_f["cov"] / 1000.0),
                "allocated_ranks": dict(zip(MATS, kf)),
                "note": "same block, inputs, factors, Fisher scores and allocation as the main step, with every "
                        "covariance C = (X W)^T (X W) formed in full (gate/up 11008 x 11008 by the fused GEMM + "
                        "split SYRK, decomposed through their range basis, which projects C itself); stages in "
                        "series"}

    # a plain copy of known size, outside the timed region: the reference that scales HBM byte
    # counters (FETCH_SIZE / WRITE_SIZE) of a profiled run into bytes
    calib_src = torch.empty(a.calib_copy_mb << 20, dtype=torch.uint8, device=dev)
    calib_dst = torch.empty_like(calib_src)
    calib_dst.copy_(calib_src)
    del calib_src, calib_dst
    for _ in range(a.warmup):
        step([])
    torch.cuda.synchronize()
    lrc.lrc_timing_read("k_cov_syrk", reset=True)  # a reset drops the records of every kernel
    lrc.lrc_timing_enable(1)  # every launch of the long kernels
    lrc.lrc_timing_set_stride("k_trd_symv", a.timing_stride)  # one launch per column: a sample
    recs = []
    t0 = time.perf_counter()
    for _ in range(a.steps):
        r = []
        step(r)
        recs.append(r)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    lrc.lrc_timing_enable(False)
    syrk_n, syrk_ms, syrk_fl = lrc.lrc_timing_read("k_cov_syrk", reset=False)
    gemm_n, gemm_ms, gemm_fl = lrc.lrc_timing_read("k_cov_gemm_y", reset=False)
    geml_n, geml_ms, geml_fl = lrc.lrc_timing_read("k_cov_gemm_l", reset=False)
    symv_n, symv_ms, symv_by = lrc.lrc_timing_read("k_trd_symv", reset=True)
    assert int(info.sum().item()) == 0, "device info flags set: %s" % info.tolist()
    assert int(rinfo.sum().item()) == 0, "range factor info flags set: %s" % rinfo.tolist()
    for g, gi in ginfo.items():
        assert int(gi.sum().item()) == 0, "eigh info flags set (n = %d): %s" % (g[0], gi.tolist())

    # one 4096x4096 layer on its own, after the timed steps: covariance, eigendecomposition (alone,
    # not batched), error curve, factors; mean of --layer-runs runs
    def one_layer(m="q_proj", n_tok=None):
        C[m].zero_()
        e0 = ev(stream)
        lrc.lrc_cov_accumulate(X if n_tok is None else X[:n_tok], W[m], C[m], info=info[0:1], ws=ws_cov)
        lrc.lrc_eigh(C[m], ks[m], prec=prec, lam=lam[m][None], V=V[m][None], info=info[7:8], ws=ws_eig)
        lrc.lrc_error_curve(lam[m][None], eps=eps[m][None])
        lrc.lrc_factorize(W[m], V[m], ks[m], A[m], B[m])
        e1 = ev(stream)
        return e0, e1

    layer_runs = [one_layer() for _ in range(a.layer_runs)]
    torch.cuda.synchronize()
    layer_alone_s = float(np.mean([x.elapsed_time(y) for x, y in layer_runs])) / 1000.0 if layer_runs else None
    layer_s_short = None
    if a.layer_tokens > 0 and a.layer_runs > 0:
        one_layer(n_tok=a.layer_tokens)  # warm-up at this size
        short_runs = [one_layer(n_tok=a.layer_tokens) for _ in range(a.layer_runs)]
        torch.cuda.synchronize()
        layer_s_short = float(np.mean([x.elapsed_time(y) for x, y in short_runs])) / 1000.0
    assert int(info.sum().item()) == 0, "device info flags set: %s" % info.tolist()

    # per-call times from the events (ms), averaged over steps
    def el(x, y):
        return x.elapsed_time(y)

    per = {}
    for r in recs:
        for key, e0, e1 in r:
            per.setdefault(key, []).append(el(e0, e1))
    avg = {k: float(np.mean(v)) for k, v in per.items()}
    step_ms = wall * 1000.0 / a.steps
    cov_ms = sum(avg[m + ".cov"] for m in MATS)
    eig_ms = sum(v for k, v in avg.items() if k.startswith("eigh."))
    cov_flops_total = sum(cov_flops(a.tokens, di, do) for di, do in sh.values())
    cov_tflops = cov_flops_total / (cov_ms / 1000.0) / 1e12
    # one 4096x4096 layer: its covariance, its share of the block's eigendecompositions and error
    # curves (their time split over the matrices in proportion to n^3, with n = d_in for a matrix
    # decomposed through a range basis: its GEMMs are left out, which overstates q_proj's share), its
    # factors
    n3 = {m: float(sh[m][0] if where[m][0] in gW else sh[m][1]) ** 3 for m in MATS}
    share = n3["q_proj"] / sum(n3.values())
    # the step's wall time outside the covariance, factor, Fisher and allocation calls: the part of
    # the eigendecompositions not hidden behind the covariances (all of them with --overlap off)
    # with --overlap on the factors run on the side streams after each group's eigendecompositions,
    # so the wall time outside the covariance, Fisher and allocation calls holds the unhidden part of
    # the decompositions, error curves and factors; with --overlap off the factor calls are in series
    fac_ms = sum(avg[m + ".fac"] for m in MATS) if a.overlap == "off" else 0.0
    eig_wall_ms = max(0.0, step_ms - cov_ms - fac_ms - avg["fisher"] - avg["alloc"])
    layer_s = (avg["q_proj.cov"] + eig_wall_ms * share + (avg["q_proj.fac"] if a.overlap == "off" else 0.0)) / 1000.0
    if a.breakdown:
        for k in sorted(avg):
            print("%-20s %10.3f ms" % (k, avg[k]), file=sys.stderr)
    # rooflines from HIP events the library records around each launch on its launch stream during
    # the timed steps; "roofline" is the kernel with the largest summed time
    syrk_tf = syrk_fl / (syrk_ms / 1000.0) / 1e12
    roof_syrk = {"kernel": "k_cov_syrk", "bound": "mfma", "achieved": syrk_tf, "peak": PEAK_BF16_TFLOPS,
                 "unit": "TFLOP/s", "frac": syrk_tf / PEAK_BF16_TFLOPS, "traffic": measured_traffic("k_cov_syrk"),
                 "launches": syrk_n, "avg_launch_ms": syrk_ms / max(syrk_n, 1),
                 "total_ms_per_step": syrk_ms / a.steps,
                 "per_launch": "algorithmic flops = tokens in the chunk x d_out (d_out + 1) (upper triangle incl. "
                               "diagonal); the kernel executes 3 fp16 MFMA products per flop pair (scaled hi/lo "
                               "split: hi hi + hi lo + lo hi; the diagonal's sum of lo^2 is a separate pass)",
                 "mfma_counters": mfma_counters("k_cov_syrk")}
    gemm_tf = gemm_fl / (gemm_ms / 1000.0) / 1e12 if gemm_ms > 0 else 0.0
    roof_gemm = {"kernel": "k_cov_gemm_y", "bound": "mfma", "achieved": gemm_tf, "peak": PEAK_BF16_TFLOPS,
                 "unit": "TFLOP/s", "frac": gemm_tf / PEAK_BF16_TFLOPS, "launches": gemm_n,
                 "avg_launch_ms": gemm_ms / max(gemm_n, 1),
                 "total_ms_per_step": gemm_ms / a.steps,
                 "per_launch": "algorithmic flops = 2 x tokens in the chunk x d_in x d_out",
                 "mfma_counters": mfma_counters("k_cov_gemm_y")}
    geml_tf = geml_fl / (geml_ms / 1000.0) / 1e12 if geml_ms > 0 else 0.0
    roof_geml = {"kernel": "k_cov_gemm_l", "bound": "mfma", "achieved": geml_tf, "peak": PEAK_BF16_TFLOPS,
                 "unit": "TFLOP/s", "frac": geml_tf / PEAK_BF16_TFLOPS, "launches": geml_n,
                 "avg_launch_ms": geml_ms / max(geml_n, 1), "total_ms_per_step": geml_ms / a.steps,
                 "per_launch": "algorithmic flops = tokens in the chunk x d_in (d_in + 1) (X L, L lower triangular); "
                               "the kernel executes 3 bf16 MFMA products (hi, mid and lo pieces of L) over the "
                               "nonzero block columns of each block row"}
    symv_gbs = symv_by / (symv_ms / 1000.0) / 1e9 if symv_ms > 0 else 0.0
    roof_symv = {"kernel": "k_trd_symv", "bound": "hbm", "achieved": symv_gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                 "frac": symv_gbs / PEAK_HBM_GBS,
                 "traffic": measured_traffic("k_trd_symv", symv_by / max(symv_n, 1)) if symv_n else None,
                 "traffic_note": "measured HBM bytes per algorithmic byte of the counted run (seven decompositions "
                                 "per launch, profiles/k_trd_symv_traffic.json) x this run's algorithmic bytes per "
                                 "launch", "launches": symv_n,
                 "avg_launch_ms": symv_ms / max(symv_n, 1),
                 "total_ms_per_step": symv_ms * a.timing_stride / a.steps,
                 "avg_bytes_per_launch": symv_by / max(symv_n, 1),
                 "per_launch": "algorithmic bytes = upper triangle of the trailing matrix read once, "
                               "(n-c-1)(n-c)/2 x 4 bytes for column c (one launch per column)"}
    for r in (roof_syrk, roof_gemm, roof_geml):
        r["sampled"] = "every launch in the timed steps (start/stop events recorded by the dispatch)"
    roof_symv["sampled"] = ("every %d-th launch in the timed steps (start/stop events recorded by the dispatch)"
                            % a.timing_stride)
    roof_symv["overlap"] = ("launches on up to eight helper streams overlap (several eigendecompositions at once, "
                            "and with --overlap on the covariance kernels of later groups): a launch's event-timed "
                            "duration includes time its workgroups wait for CUs held by the other streams' kernels, "
                            "and summed durations exceed the eigendecomposition stage's wall time")
    if a.overlap == "on":
        for r in (roof_syrk, roof_gemm, roof_geml):
            r["overlap"] = ("the eigendecompositions of earlier groups run on side streams during later groups' "
                            "covariances: a launch's event-timed duration includes time its workgroups wait for "
                            "CUs held by those kernels (--overlap off times the covariance alone)")
    # the roofline entry is the kernel with the largest summed launch time in the timed steps (events
    # recorded by the dispatches; for k_trd_symv every timing_stride-th launch, scaled up)
    cands = [roof_syrk, roof_symv, roof_gemm] + ([roof_geml] if geml_n else [])
    roof = dict(max(cands, key=lambda r: r["total_ms_per_step"]))
    roof["dominant_by"] = ("largest summed launch time per step among %s (%s ms)"
                           % (", ".join(r["kernel"] for r in cands),
                              ", ".join("%.1f" % r["total_ms_per_step"] for r in cands)))
    out = {
        "metric": "calibration tokens/s into Y^T Y; sec per 4096x4096 layer compressed (eig incl.)",
        "value": a.tokens / (step_ms / 1000.0),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": a.steps, "warmup": a.warmup, "ms_per_step": step_ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (seeded, generated on the GPU)",
        "config": {"workload": "LLaMA-7B-shaped block: q/k/v/o 4096x4096, gate/up 4096x11008, down 11008x4096, "
                               "%d calibration tokens, 60%% params per matrix, eig prec %s%s"
                               % (a.tokens, a.prec, ("; gate/up (rank <= 4096) decomposed through a basis of range(W^T)"
                                  + ("; their covariances accumulated in its coordinates, B = (X L)^T (X L) with "
                                     "W W^T = L L^T (the factor formed in the step)" if gP else ""))
                                  if gW else ""),
                   "tokens": a.tokens, "d_model": a.d_model, "d_ff": a.d_ff, "ranks": ks,
                   "allocated_ranks": dict(zip(MATS, k_out.cpu().tolist()))},
        "sec_per_4096_layer": layer_alone_s,
        "sec_per_4096_layer_note": "q_proj compressed on its own (covariance over all tokens, eigendecomposition, "
                                   "error curve, factors), after the timed steps",
        "sec_per_4096_layer_at_%d_tokens" % a.layer_tokens: layer_s_short,
        "sec_per_4096_layer_in_block": layer_s,
        "sec_per_4096_layer_in_block_note": "an attribution estimate, not a measurement: q_proj covariance + %.4f "
                                            "of the step's wall time outside the covariance, Fisher and allocation "
                                            "calls (the eigendecompositions, error curves and factors of %s not "
                                            "hidden behind the covariances: %.1f ms; with --overlap off the factor "
                                            "calls are left out of that time and q_proj's is added; the share is "
                                            "q_proj's n^3 over the sum, n = d_in for the matrices decomposed "
                                            "through a range basis)" % (share, gkey, eig_wall_ms),
        "cov_tokens_per_s": a.tokens / (cov_ms / 1000.0),
        "cov_ms": cov_ms, "eigh_ms": eig_ms,
        "overlap": a.overlap,
        "overlap_note": (("covariances group by group (%s), each group's eigendecompositions and error curves "
                          "on a side stream as soon as its covariances are done: cov_ms and eigh_ms are summed "
                          "call times that overlap in the step" % ", ".join(pname))
                         if a.overlap == "on" else "covariances, then one call for every eigendecomposition"),
        "breakdown_ms": {k: round(v, 3) for k, v in avg.items()},
        "roofline": roof,
        "rooflines": {"k_cov_syrk": roof_syrk, "k_trd_symv": roof_symv, "k_cov_gemm_y": roof_gemm,
                      **({"k_cov_gemm_l": roof_geml} if geml_n else {})},
    }
    if a.factored_steps > 0:
        out["factored"] = factored_leg()
    if a.full_steps > 0 and gP:
        out["full_covariance"] = full_leg()
    if a.single == "on":
        out["single_layer"] = single_layer_leg(torch, lrc, dev)
    if a.heads_tokens > 0:
        out["per_head"] = per_head_leg(torch, lrc, a.heads_tokens, a.seed, dev)
    if a.curvature_tokens > 0:
        del X, Xd, W, G, C, V, A, B, gC, gV, glam, geps, lam, eps, ws_cov, ws_eig
        torch.cuda.empty_cache()
        out["curvature_layer"] = curvature_leg(torch, lrc, a.curvature_tokens, a.seed,
                                               lrc.LRC_F32 if a.curvature_prec == "f32" else lrc.LRC_F64, dev)
    if a.stack_layers > 0:
        torch.cuda.empty_cache()
        out["stack"] = stack_leg(torch, lrc, a.stack_layers, a.stack_tokens, a.seed, prec, dev, a.d_model, a.d_ff,
                                 sets=a.stack_sets, cov_range=a.cov_range == "on" and a.eig_range == "on")
    if a.cpu_sample > 0:
        out["cpu_baseline"] = cpu_baseline(a.d_model, a.d_ff, a.cpu_sample, a.cpu_layer_tokens, a.cpu_heads_sample)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
