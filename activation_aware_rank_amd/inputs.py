"""Seeded synthetic inputs for activation-aware low-rank compression.

This module only draws random numbers and rounds them to the storage type
(fp32, or bf16 kept as raw uint16 bit patterns).  It holds none of the
method's arithmetic, so both the GPU path and the fp64 oracle can take the
same bytes from it.

Every draw uses numpy's PCG64 seeded by
``SeedSequence(entropy=20261203, spawn_key=(cfg, layer, matrix, stream, chunk))``
and row chunks of 8192, so the bytes do not depend on how many threads fill
them.  Values are drawn in fp64, rounded to fp32, and for bf16 rounded once
more to nearest-even.

Workload recipes (the pages print no data; these stand in for the calibration
corpora they name -- 256 sequences x 2048 tokens of Wikitext2 on the FLRC page,
"Experimental setup"; C4 on the Swift-SVD page, section 4 -- and for trained
weights, which are not available):

* ``single``   one fp32 linear layer: W ~ N(0, 0.02^2); X = N(0,1) * s_j with a
               per-column scale s_j = 10^U(-1,1).
* ``heads``    per-head key projection (WSVD page, "per-head SVD"): W ~ N(0,0.02^2)
               bf16, X bf16 Student-t(3) entries, 8 outlier columns scaled x50.
* ``block``    LLaMA-7B-shaped block: bf16 weights ~ N(0,0.02^2); X = N(0,1)
               * exp(z_j), z_j ~ N(0,1) per channel, bf16.  The down projection
               gets its own independent X of width d_ff drawn the same way.
* ``grad``     synthetic gradients G ~ N(0, sigma^2) bf16, shape of W.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

ENTROPY = 20261203
CHUNK_ROWS = 8192

# stream ids inside the spawn key
S_WEIGHT, S_ACT, S_SCALE, S_GRAD, S_OUTLIER = 0, 1, 2, 3, 4

# config ids inside the spawn key
CFG_SINGLE, CFG_HEADS, CFG_BLOCK, CFG_STACK, CFG_KFAC = 1, 2, 3, 4, 5

# matrix ids of a transformer block, in the order used everywhere
BLOCK_MATRICES = ("q_proj", "k_proj", "v_proj", "o_proj", "gate_proj", "up_proj", "down_proj")


def rng(cfg: int, layer: int, matrix: int, stream: int, chunk: int) -> np.random.Generator:
    ss = np.random.SeedSequence(entropy=ENTROPY, spawn_key=(cfg, layer, matrix, stream, chunk))
    return np.random.default_rng(ss)


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


# ----------------------------------------------------------------------------------------------
# storage rounding
# ----------------------------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even); returns the uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def as_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of a stored array ('bf16' bits or 'f32') to fp64."""
    if dtype == "bf16":
        return bf16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a, dtype=np.float32).astype(np.float64)


def _store(x64: np.ndarray, dtype: str) -> np.ndarray:
    x32 = x64.astype(np.float32)
    return f32_to_bf16_bits(x32) if dtype == "bf16" else x32


# ----------------------------------------------------------------------------------------------
# chunked fills
# ----------------------------------------------------------------------------------------------

def _fill_rows(rows: int, cols: int, dtype: str, make_chunk) -> np.ndarray:
    """Fill a rows x cols array chunk by chunk; make_chunk(c, r0, r1) returns fp64 rows."""
    out = np.empty((rows, cols), dtype=np.uint16 if dtype == "bf16" else np.float32)
    n_chunks = (rows + CHUNK_ROWS - 1) // CHUNK_ROWS

    def work(c):
        r0 = c * CHUNK_ROWS
        r1 = min(rows, r0 + CHUNK_ROWS)
        out[r0:r1] = _store(make_chunk(c, r0, r1), dtype)

    if n_chunks == 1:
        work(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, range(n_chunks)))
    return out


def gaussian(rows: int, cols: int, std: float, dtype: str, cfg: int, layer: int, matrix: int,
             stream: int) -> np.ndarray:
    """rows x cols of N(0, std^2)."""
    def mk(c, r0, r1):
        return rng(cfg, layer, matrix, stream, c).standard_normal((r1 - r0, cols)) * std
    return _fill_rows(rows, cols, dtype, mk)


def weight(d_in: int, d_out: int, dtype: str, cfg: int, layer: int, matrix: int,
           std: float = 0.02) -> np.ndarray:
    """Weight W (d_in x d_out, Y = X W orientation) ~ N(0, std^2)."""
    return gaussian(d_in, d_out, std, dtype, cfg, layer, matrix, S_WEIGHT)


def gradient(d_in: int, d_out: int, std: float, cfg: int, layer: int, matrix: int) -> np.ndarray:
    """Synthetic gradient of W, same shape, ~ N(0, std^2), bf16."""
    return gaussian(d_in, d_out, std, "bf16", cfg, layer, matrix, S_GRAD)


def channel_scales_lognormal(cols: int, cfg: int, layer: int, matrix: int) -> np.ndarray:
    """exp(z_j), z_j ~ N(0,1), one per input channel."""
    return np.exp(rng(cfg, layer, matrix, S_SCALE, 0).standard_normal(cols))


def channel_scales_loguniform(cols: int, cfg: int, layer: int, matrix: int) -> np.ndarray:
    """10^u_j, u_j ~ U(-1, 1): log-uniform in [0.1, 10]."""
    return 10.0 ** rng(cfg, layer, matrix, S_SCALE, 0).uniform(-1.0, 1.0, cols)


def activations_scaled(rows: int, cols: int, scales: np.ndarray, dtype: str, cfg: int, layer: int,
                       matrix: int, row_offset_chunks: int = 0) -> np.ndarray:
    """X = N(0,1) * scales[j]; chunk c of the result uses chunk id row_offset_chunks + c."""
    def mk(c, r0, r1):
        return rng(cfg, layer, matrix, S_ACT, row_offset_chunks + c).standard_normal((r1 - r0, cols)) * scales
    return _fill_rows(rows, cols, dtype, mk)


def activations_student_t(rows: int, cols: int, df: float, n_outliers: int, outlier_scale: float,
                          dtype: str, cfg: int, layer: int, matrix: int) -> np.ndarray:
    """Student-t(df) entries (unit scale); n_outliers columns multiplied by outlier_scale."""
    cols_out = rng(cfg, layer, matrix, S_OUTLIER, 0).choice(cols, n_outliers, replace=False)
    scale = np.ones(cols)
    scale[cols_out] = outlier_scale

    def mk(c, r0, r1):
        return rng(cfg, layer, matrix, S_ACT, c).standard_t(df, (r1 - r0, cols)) * scale
    return _fill_rows(rows, cols, dtype, mk)


# ----------------------------------------------------------------------------------------------
# whole workloads
# ----------------------------------------------------------------------------------------------

def single_layer(n_tok: int = 2048, d_in: int = 256, d_out: int = 256) -> dict:
    """One fp32 layer; full size is 2048 tokens, 256 -> 256, rank 64."""
    s = channel_scales_loguniform(d_in, CFG_SINGLE, 0, 0)
    return {
        "X": activations_scaled(n_tok, d_in, s, "f32", CFG_SINGLE, 0, 0),
        "W": weight(d_in, d_out, "f32", CFG_SINGLE, 0, 0),
        "dtype": "f32",
    }


def per_head(n_tok: int = 32768, d_model: int = 4096, head_dim: int = 128) -> dict:
    """Key projection cut into heads of head_dim columns; full size 32768 tokens, 32 heads."""
    return {
        "X": activations_student_t(n_tok, d_model, 3.0, 8, 50.0, "bf16", CFG_HEADS, 0, 0),
        "W": weight(d_model, d_model, "bf16", CFG_HEADS, 0, 0),
        "dtype": "bf16",
        "n_blocks": d_model // head_dim,
    }


def block_shapes(d_model: int = 4096, d_ff: int = 11008) -> dict:
    """(d_in, d_out) of each block matrix in the Y = X W orientation."""
    return {
        "q_proj": (d_model, d_model), "k_proj": (d_model, d_model), "v_proj": (d_model, d_model),
        "o_proj": (d_model, d_model), "gate_proj": (d_model, d_ff), "up_proj": (d_model, d_ff),
        "down_proj": (d_ff, d_model),
    }


def block_weight(name: str, d_model: int = 4096, d_ff: int = 11008, cfg: int = CFG_BLOCK,
                 layer: int = 0) -> np.ndarray:
    d_in, d_out = block_shapes(d_model, d_ff)[name]
    return weight(d_in, d_out, "bf16", cfg, layer, BLOCK_MATRICES.index(name))


def block_activations(width: int, n_tok: int, feeds_down: bool = False, cfg: int = CFG_BLOCK,
                      layer: int = 0, row_offset_chunks: int = 0) -> np.ndarray:
    """Calibration input of a block: width d_model feeds q/k/v/o/gate/up (matrix id 0 in the
    spawn key), width d_ff feeds down (matrix id 6), so the two are independent draws."""
    which = 6 if feeds_down else 0
    s = channel_scales_lognormal(width, cfg, layer, which)
    return activations_scaled(n_tok, width, s, "bf16", cfg, layer, which, row_offset_chunks)


def rank_at_ratio(d_in: int, d_out: int, ratio: float) -> int:
    """Rank whose factor parameters k (d_in + d_out) keep the given fraction of d_in d_out."""
    return int(np.floor(ratio * d_in * d_out / (d_in + d_out)))


def curvature_layer(n_tok: int = 131072, d_in: int = 5120, d_out: int = 13824) -> dict:
    """Curvature-weighted case of one FFN matrix (13B shape at full size): activations N(0,1)
    with lognormal channel scales, output gradients N(0, 1e-3^2), weight N(0, 0.02^2); all bf16."""
    s = channel_scales_lognormal(d_in, CFG_KFAC, 0, 0)
    return {
        "X": activations_scaled(n_tok, d_in, s, "bf16", CFG_KFAC, 0, 0),
        "G": gaussian(n_tok, d_out, 1e-3, "bf16", CFG_KFAC, 0, 1, S_GRAD),
        "W": weight(d_in, d_out, "bf16", CFG_KFAC, 0, 2),
        "dtype": "bf16",
    }


def curvature_layer_gpu(n_tok: int, d_in: int, d_out: int, seed: int, device) -> dict:
    """The curvature_layer recipe drawn on the GPU by torch's seeded generator (other numbers than
    the host draw; used at full size, where results are checked through properties)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    scale = torch.exp(torch.randn(d_in, generator=g, device=device, dtype=torch.float32))
    X = torch.empty(n_tok, d_in, dtype=torch.bfloat16, device=device)
    G = torch.empty(n_tok, d_out, dtype=torch.bfloat16, device=device)
    for r0 in range(0, n_tok, 16384):
        r1 = min(n_tok, r0 + 16384)
        X[r0:r1] = (torch.randn(r1 - r0, d_in, generator=g, device=device) * scale).to(torch.bfloat16)
        G[r0:r1] = (torch.randn(r1 - r0, d_out, generator=g, device=device) * 1e-3).to(torch.bfloat16)
    W = (torch.randn(d_in, d_out, generator=g, device=device) * 0.02).to(torch.bfloat16)
    return {"X": X, "G": G, "W": W}


def block_gpu(n_tok: int, d_model: int, d_ff: int, seed: int, device) -> dict:
    """The block recipe drawn on the GPU by torch's seeded generator: X (n_tok x d_model) and X_d
    (n_tok x d_ff) N(0,1) times per-channel exp(N(0,1)) scales, weights N(0, 0.02^2) and gradients
    N(0, 1e-4^2) of every block matrix, all bf16.  Other numbers than the host draw; used where
    the sizes are the full ones."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)

    def act(width):
        scale = torch.exp(torch.randn(width, generator=g, device=device, dtype=torch.float32))
        X = torch.empty(n_tok, width, dtype=torch.bfloat16, device=device)
        for r0 in range(0, n_tok, 65536):
            r1 = min(n_tok, r0 + 65536)
            X[r0:r1] = (torch.randn(r1 - r0, width, generator=g, device=device, dtype=torch.float32) * scale).to(
                torch.bfloat16)
        return X

    X = act(d_model)
    Xd = act(d_ff)
    W, G = {}, {}
    for m, (di, do) in block_shapes(d_model, d_ff).items():
        W[m] = (torch.randn(di, do, generator=g, device=device) * 0.02).to(torch.bfloat16)
        G[m] = (torch.randn(di, do, generator=g, device=device) * 1e-4).to(torch.bfloat16)
    return {"X": X, "Xd": Xd, "W": W, "G": G}


def stack_spectra(n_layers: int = 32, d_model: int = 4096, d_ff: int = 11008, cfg: int = CFG_STACK) -> dict:
    """Synthetic inputs of the cross-layer allocation over a stack of blocks: for every matrix a
    decaying spectrum lambda_i = c (i + 1)^-p of its first K = floor(d_in d_out / (d_in + d_out))
    values (c lognormal, p uniform in [0.5, 1.5]), eps_0 = the spectrum's sum times (1 + u), u
    uniform in [0, 0.2) (the part beyond K), and an importance alpha lognormal; all fp64."""
    shapes = block_shapes(d_model, d_ff)
    lams, eps0, alpha, cost = [], [], [], []
    for layer in range(n_layers):
        for mi, name in enumerate(BLOCK_MATRICES):
            di, do = shapes[name]
            k = (di * do) // (di + do)
            r = rng(cfg, layer, mi, S_SCALE, 1)
            c, p = np.exp(r.standard_normal()), r.uniform(0.5, 1.5)
            lam = c * (np.arange(k, dtype=np.float64) + 1.0) ** (-p)
            lams.append(lam)
            eps0.append(float(lam.sum()) * (1.0 + r.uniform(0.0, 0.2)))
            alpha.append(float(np.exp(r.standard_normal())))
            cost.append(di + do)
    return {"lams": lams, "eps0": np.array(eps0), "alpha": np.array(alpha), "cost": np.array(cost, dtype=np.int64)}



def per_head_gpu(n_tok: int, d_model: int, seed: int, device, n_outliers: int = 8, outlier_scale: float = 50.0,
                 df: int = 3) -> dict:
    """The per_head recipe drawn on the GPU by torch's seeded generator: X Student-t(df) entries (a
    normal over the root of a chi-square(df) / df, the chi-square as a sum of df squared normals)
    with n_outliers columns scaled by outlier_scale, W ~ N(0, 0.02^2), both bf16.  Other numbers than
    the host draw; used at full size for timing."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    cols = torch.randperm(d_model, generator=g, device=device)[:n_outliers]
    scale = torch.ones(d_model, device=device)
    scale[cols] = outlier_scale
    X = torch.empty(n_tok, d_model, dtype=torch.bfloat16, device=device)
    for r0 in range(0, n_tok, 8192):
        r1 = min(n_tok, r0 + 8192)
        z = torch.randn(r1 - r0, d_model, generator=g, device=device)
        chi = torch.zeros_like(z)
        for _ in range(df):
            chi += torch.randn(r1 - r0, d_model, generator=g, device=device) ** 2
        X[r0:r1] = (z / torch.sqrt(chi / df) * scale).to(torch.bfloat16)
    W = (torch.randn(d_model, d_model, generator=g, device=device) * 0.02).to(torch.bfloat16)
    return {"X": X, "W": W}


def stack_layer_gpu(g, n_tok: int, d_model: int, d_ff: int, device, X=None, Xd=None) -> tuple:
    """The calibration inputs of one stack layer (the block recipe) drawn on the GPU from the torch
    generator g, into X (n_tok x d_model) and Xd (n_tok x d_ff) when given: N(0,1) times per-channel
    exp(N(0,1)) scales, bf16."""
    import torch

    def act(width, out):
        scale = torch.exp(torch.randn(width, generator=g, device=device, dtype=torch.float32))
        if out is None:
            out = torch.empty(n_tok, width, dtype=torch.bfloat16, device=device)
        for r0 in range(0, n_tok, 16384):
            r1 = min(n_tok, r0 + 16384)
            out[r0:r1] = (torch.randn(r1 - r0, width, generator=g, device=device) * scale).to(torch.bfloat16)
        return out

    return act(d_model, X), act(d_ff, Xd)


def stack_weights_gpu(g, n_layers: int, d_model: int, d_ff: int, device) -> tuple:
    """Weights N(0, 0.02^2) and gradients N(0, 1e-4^2) of every matrix of an n_layers stack (block
    shapes), bf16, drawn on the GPU from the torch generator g: lists of dicts per layer."""
    import torch
    Ws, Gs = [], []
    for _ in range(n_layers):
        W, G = {}, {}
        for m, (di, do) in block_shapes(d_model, d_ff).items():
            W[m] = (torch.randn(di, do, generator=g, device=device) * 0.02).to(torch.bfloat16)
            G[m] = (torch.randn(di, do, generator=g, device=device) * 1e-4).to(torch.bfloat16)
        Ws.append(W)
        Gs.append(G)
    return Ws, Gs
