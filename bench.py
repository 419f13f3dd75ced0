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


def measured_traffic(kernel):
    """HBM bytes per launch from the committed rocprofv3 counter record, if the kernel's source is
    unchanged since the counters were taken (else None)."""
    import hashlib
    rec_path = os.path.join(ROOT, "profiles", "%s_traffic.json" % kernel)
    try:
        rec = json.load(open(rec_path))
        src = open(os.path.join(ROOT, rec["source"]), "rb").read()
    except (OSError, ValueError, KeyError):
        return None
    if hashlib.sha256(src).hexdigest() != rec.get("source_sha256"):
        return None
    return rec.get("traffic_bytes_per_launch")


def cpu_baseline(d_model, d_ff, sample_tok):
    """The fp64 oracle's covariance throughput on a bounded token sample of the same block."""
    import numpy as np

    import oracle
    from activation_aware_rank_amd import inputs
    X = inputs.block_activations(d_model, sample_tok)
    Xd = inputs.block_activations(d_ff, sample_tok, feeds_down=True)
    Ws = {m: inputs.block_weight(m, d_model, d_ff) for m in MATS}
    threads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or (os.cpu_count() or 1)
    t0 = time.perf_counter()
    for m in MATS:
        oracle.covariance(Xd if m == "down_proj" else X, "bf16", Ws[m], "bf16")
    dt = time.perf_counter() - t0
    return {"value": sample_tok / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": "fp64 direct covariance (Y = XW, C = Y^T Y) of all 7 block matrices over %d tokens "
                      "(%.1f s); eigendecomposition, error curve and factors excluded, so this is an upper "
                      "bound on the oracle's whole-step throughput" % (sample_tok, dt),
            "seconds": dt}


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
    ap.add_argument("--overlap-order", choices=("large-first", "most-first"), default="large-first",
                    help="group order: largest n first, or the group with the most matrices first")
    ap.add_argument("--factored-steps", type=int, default=2,
                    help="timed steps of the variant that forms the covariances from X^T X (0: skip)")
    ap.add_argument("--eig-range", choices=("on", "off"), default="on",
                    help="on: covariances of Y = X W with d_in < d_out (gate/up) are decomposed through a basis of "
                         "range(W^T) (their rank is at most d_in); off: the full decomposition of every covariance")
    ap.add_argument("--timing-stride", type=int, default=16,
                    help="time every s-th launch of the per-column symmetric product in the timed steps")
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
    gC = {g: torch.empty(len(ms), g[0], g[0], dtype=torch.float32, device=dev) for g, ms in groups.items()}
    glam = {g: torch.empty(len(ms), g[0], dtype=torch.float64, device=dev) for g, ms in groups.items()}
    gV = {g: torch.empty(len(ms), g[0], g[1], dtype=torch.float32, device=dev) for g, ms in groups.items()}
    geps = {g: torch.empty(len(ms), g[0] + 1, dtype=torch.float64, device=dev) for g, ms in groups.items()}
    ginfo = {g: torch.zeros(len(ms), dtype=torch.int32, device=dev) for g, ms in groups.items()}
    where = {m: (g, ms.index(m)) for g, ms in groups.items() for m in ms}
    # groups whose covariance has rank <= d_in < d_out: their weights in one stack too (the range
    # bases of the decomposition; the covariance calls read the same storage)
    gW = {}
    if a.eig_range == "on":
        for g, ms in groups.items():
            if sh[ms[0]][0] < g[0]:
                gW[g] = torch.stack([W[m] for m in ms])
                for i, m in enumerate(ms):
                    W[m] = gW[g][i]
    C = {m: gC[where[m][0]][where[m][1]] for m in MATS}
    lam = {m: glam[where[m][0]][where[m][1]] for m in MATS}
    V = {m: gV[where[m][0]][where[m][1]] for m in MATS}
    eps = {m: geps[where[m][0]][where[m][1]] for m in MATS}
    A = {m: torch.empty(di, ks[m], dtype=torch.float32, device=dev) for m, (di, do) in sh.items()}
    B = {m: torch.empty(ks[m], do, dtype=torch.float32, device=dev) for m, (di, do) in sh.items()}
    info = torch.zeros(8, dtype=torch.int32, device=dev)
    ws_cov = torch.empty(max(lrc.lrc_cov_accumulate_workspace(lrc.LRC_BF16, a.tokens, di, True, do, 1)
                             for di, do in sh.values()), dtype=torch.uint8, device=dev)
    ws_eig = torch.empty(lrc.lrc_eigh_multi_workspace(
        [(g[0], len(ms), g[1], sh[ms[0]][0] if g in gW else 0) for g, ms in groups.items()], prec),
        dtype=torch.uint8, device=dev)
    eig_groups = [(gC[g], g[1], glam[g], gV[g], ginfo[g], gW.get(g)) for g in groups]
    gkey = "+".join("%dx%d_k%d" % (len(ms), g[0], g[1]) for g, ms in groups.items())
    # overlap: covariances group by group, largest n first; each group's eigendecompositions and
    # error curves on a side stream of its own (default priority) with a workspace of its own
    g_order = sorted(groups, key=lambda g: -g[0] if a.overlap_order == "large-first" else len(groups[g]) * -1)
    side = {g: torch.cuda.Stream(device=dev) for g in groups}
    ws_eig_g = {g: torch.empty(lrc.lrc_eigh_multi_workspace(
        [(g[0], len(groups[g]), g[1], sh[groups[g][0]][0] if g in gW else 0)], prec), dtype=torch.uint8, device=dev)
        for g in groups} if a.overlap == "on" else {}
    gname = {g: "%dx%d_k%d" % (len(groups[g]), g[0], g[1]) for g in groups}
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

    def cov(m, times):
        i = MATS.index(m)
        xin = Xd if m == "down_proj" else X
        C[m].zero_()
        e0 = ev(stream)
        lrc.lrc_cov_accumulate(xin, W[m], C[m], info=info[i:i + 1], ws=ws_cov)
        e1 = ev(stream)
        times.append((m + ".cov", e0, e1))

    def eig_group(g, ready, times):
        # runs on a host thread of its own: the library call returns once its launches are
        # enqueued, which takes about as long as they run
        sg = side[g]
        sg.wait_event(ready)
        e0 = ev(sg)
        lrc.lrc_eigh_multi([eig_groups[list(groups).index(g)]], prec=prec, ws=ws_eig_g[g], stream=sg)
        lrc.lrc_error_curve(glam[g], eps=geps[g], stream=sg)
        e1 = ev(sg)
        times.append(("eigh." + gname[g], e0, e1))

    def tail(times):
        for m in MATS:
            e0 = ev(stream)
            lrc.lrc_factorize(W[m], V[m], ks[m], A[m], B[m])
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
        if a.overlap == "on":
            threads = []
            for g in g_order:
                for m in groups[g]:
                    cov(m, times)
                t = threading.Thread(target=eig_group, args=(g, ev(stream), times))
                t.start()
                threads.append(t)
            for t in threads:
                t.join()
            for g in groups:
                stream.wait_stream(side[g])
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
        ws_f = torch.empty(max(lrc.lrc_cov_from_input_workspace(di, do) for di, do in sh.values()),
                           dtype=torch.uint8, device=dev)

        def fstep(times):
            e0 = ev(stream)
            H.zero_()
            lrc.lrc_cov_accumulate(X, None, H, info=info[0:1], ws=ws_h)
            Hd.zero_()
            lrc.lrc_cov_accumulate(Xd, None, Hd, info=info[1:2], ws=ws_h)
            e1 = ev(stream)
            for m in MATS:
                lrc.lrc_cov_from_input(Hd if m == "down_proj" else H, W[m], C=C[m], ws=ws_f)
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
                        "two fp64 products per matrix) instead of the fused GEMM + split SYRK; stages in series"}

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
    symv_n, symv_ms, symv_by = lrc.lrc_timing_read("k_trd_symv", reset=True)
    assert int(info.sum().item()) == 0, "device info flags set: %s" % info.tolist()
    for g, gi in ginfo.items():
        assert int(gi.sum().item()) == 0, "eigh info flags set (n = %d): %s" % (g[0], gi.tolist())

    # one 4096x4096 layer on its own, after the timed steps: covariance, eigendecomposition (alone,
    # not batched), error curve, factors; mean of --layer-runs runs
    def one_layer(m="q_proj"):
        C[m].zero_()
        e0 = ev(stream)
        lrc.lrc_cov_accumulate(X, W[m], C[m], info=info[0:1], ws=ws_cov)
        lrc.lrc_eigh(C[m], ks[m], prec=prec, lam=lam[m][None], V=V[m][None], info=info[7:8], ws=ws_eig)
        lrc.lrc_error_curve(lam[m][None], eps=eps[m][None])
        lrc.lrc_factorize(W[m], V[m], ks[m], A[m], B[m])
        e1 = ev(stream)
        return e0, e1

    layer_runs = [one_layer() for _ in range(a.layer_runs)]
    torch.cuda.synchronize()
    layer_alone_s = float(np.mean([x.elapsed_time(y) for x, y in layer_runs])) / 1000.0 if layer_runs else None
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
    fac_ms = sum(avg[m + ".fac"] for m in MATS)
    eig_wall_ms = max(0.0, step_ms - cov_ms - fac_ms - avg["fisher"] - avg["alloc"])
    layer_s = (avg["q_proj.cov"] + eig_wall_ms * share + avg["q_proj.fac"]) / 1000.0
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
                               "split: hi hi + hi lo + lo hi; the diagonal's sum of lo^2 is a separate pass), so "
                               "executed MFMA utilisation is 3x frac"}
    gemm_tf = gemm_fl / (gemm_ms / 1000.0) / 1e12 if gemm_ms > 0 else 0.0
    roof_gemm = {"kernel": "k_cov_gemm_y", "bound": "mfma", "achieved": gemm_tf, "peak": PEAK_BF16_TFLOPS,
                 "unit": "TFLOP/s", "frac": gemm_tf / PEAK_BF16_TFLOPS, "launches": gemm_n,
                 "avg_launch_ms": gemm_ms / max(gemm_n, 1),
                 "total_ms_per_step": gemm_ms / a.steps,
                 "per_launch": "algorithmic flops = 2 x tokens in the chunk x d_in x d_out"}
    symv_gbs = symv_by / (symv_ms / 1000.0) / 1e9 if symv_ms > 0 else 0.0
    roof_symv = {"kernel": "k_trd_symv", "bound": "hbm", "achieved": symv_gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                 "frac": symv_gbs / PEAK_HBM_GBS, "traffic": measured_traffic("k_trd_symv"), "launches": symv_n,
                 "avg_launch_ms": symv_ms / max(symv_n, 1),
                 "total_ms_per_step": symv_ms * a.timing_stride / a.steps,
                 "avg_bytes_per_launch": symv_by / max(symv_n, 1),
                 "per_launch": "algorithmic bytes = upper triangle of the trailing matrix read once, "
                               "(n-c-1)(n-c)/2 x 4 bytes for column c (one launch per column)"}
    for r in (roof_syrk, roof_gemm):
        r["sampled"] = "every launch in the timed steps (start/stop events recorded by the dispatch)"
    roof_symv["sampled"] = ("every %d-th launch in the timed steps (start/stop events recorded by the dispatch)"
                            % a.timing_stride)
    roof_symv["overlap"] = ("launches on up to eight helper streams overlap (several eigendecompositions at once, "
                            "and with --overlap on the covariance kernels of later groups): a launch's event-timed "
                            "duration includes time its workgroups wait for CUs held by the other streams' kernels, "
                            "and summed durations exceed the eigendecomposition stage's wall time")
    if a.overlap == "on":
        for r in (roof_syrk, roof_gemm):
            r["overlap"] = ("the eigendecompositions of earlier groups run on side streams during later groups' "
                            "covariances: a launch's event-timed duration includes time its workgroups wait for "
                            "CUs held by those kernels (--overlap off times the covariance alone)")
    # the roofline entry is the covariance SYRK: the kernel with the largest time
    roof = roof_syrk
    out = {
        "metric": "calibration tokens/s into Y^T Y; sec per 4096x4096 layer compressed (eig incl.)",
        "value": a.tokens / (step_ms / 1000.0),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": a.steps, "warmup": a.warmup, "ms_per_step": step_ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (seeded, generated on the GPU)",
        "config": {"workload": "LLaMA-7B-shaped block: q/k/v/o 4096x4096, gate/up 4096x11008, down 11008x4096, "
                               "%d calibration tokens, 60%% params per matrix, eig prec %s%s"
                               % (a.tokens, a.prec, "; gate/up (rank <= 4096) decomposed through a basis of range(W^T)"
                                  if gW else ""),
                   "tokens": a.tokens, "d_model": a.d_model, "d_ff": a.d_ff, "ranks": ks,
                   "allocated_ranks": dict(zip(MATS, k_out.cpu().tolist()))},
        "sec_per_4096_layer": layer_alone_s,
        "sec_per_4096_layer_note": "q_proj compressed on its own (covariance over all tokens, eigendecomposition, "
                                   "error curve, factors), after the timed steps",
        "sec_per_4096_layer_in_block": layer_s,
        "sec_per_4096_layer_in_block_note": "q_proj covariance + q_proj factors + %.4f of the step's wall time "
                                            "outside the covariance, factor, Fisher and allocation calls (the "
                                            "eigendecompositions and error curves of %s not hidden behind the "
                                            "covariances: %.1f ms; the share is q_proj's n^3 over the sum, n = d_in "
                                            "for the matrices decomposed through a range basis)"
                                            % (share, gkey, eig_wall_ms),
        "cov_tokens_per_s": a.tokens / (cov_ms / 1000.0),
        "cov_ms": cov_ms, "eigh_ms": eig_ms,
        "overlap": a.overlap,
        "overlap_note": (("covariances group by group (%s), each group's eigendecompositions and error curves "
                          "on a side stream as soon as its covariances are done: cov_ms and eigh_ms are summed "
                          "call times that overlap in the step" % ", ".join(gname[g] for g in g_order))
                         if a.overlap == "on" else "covariances, then one call for every eigendecomposition"),
        "breakdown_ms": {k: round(v, 3) for k, v in avg.items()},
        "roofline": roof,
        "rooflines": {"k_cov_syrk": roof_syrk, "k_trd_symv": roof_symv, "k_cov_gemm_y": roof_gemm},
    }
    if a.factored_steps > 0:
        out["factored"] = factored_leg()
    if a.curvature_tokens > 0:
        del X, Xd, W, G, C, V, A, B, gC, gV, glam, geps, lam, eps, ws_cov, ws_eig
        torch.cuda.empty_cache()
        out["curvature_layer"] = curvature_leg(torch, lrc, a.curvature_tokens, a.seed,
                                               lrc.LRC_F32 if a.curvature_prec == "f32" else lrc.LRC_F64, dev)
    if a.cpu_sample > 0:
        out["cpu_baseline"] = cpu_baseline(a.d_model, a.d_ff, a.cpu_sample)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
