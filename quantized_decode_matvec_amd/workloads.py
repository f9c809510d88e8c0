"""Seeded synthetic inputs shaped like the pages' heads and experts.

This module draws random numbers and nothing else: it holds none of the
quantization or matvec arithmetic, so both the GPU path and the CPU oracle can
be fed from it. Every generator uses ``numpy.random.default_rng(seed)`` (PCG64)
and draws in the order written in its docstring; fp32 values are drawn first
and cast to fp16 at the end where the workload is fp16.

Weight statistics: N(0, 0.02) (standard deviation 0.02). The pages measured
real checkpoints (LFM2.5-1.2B, Qwen3.6-35B-A3B, MiniCPM5 heads), which are not
available; these tensors stand in for them with the pages' shapes.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

SIGMA = 0.02


def _normal(rng, shape, sigma=SIGMA, chunk_rows=8192):
    """N(0, sigma) fp32, drawn row-chunk by row-chunk (same stream as one call)."""
    out = np.empty(shape, np.float32)
    flat = out.reshape(shape[0], -1)
    for r in range(0, flat.shape[0], chunk_rows):
        blk = rng.standard_normal(size=flat[r:r + chunk_rows].shape, dtype=np.float32)
        blk *= np.float32(sigma)
        flat[r:r + chunk_rows] = blk
    return out


@dataclass
class DenseCase:
    name: str
    fmt: str            # "int4" | "fp4" | "int8" | "km4"
    W: np.ndarray       # [N, K] fp32 or fp16
    x: np.ndarray       # [B, K] fp32 or fp16


def tiny_int4(seed: int = 0) -> DenseCase:
    """256 x 512 fp32 weights with 2% outlier input columns, x fp32 [1, 512].

    Draws: W ~ N(0, 0.02) [256, 512]; 10 = round(0.02 * 512) columns chosen
    without replacement, multiplied by 20 (fp32); x ~ N(0, 1) [1, 512].
    """
    rng = np.random.default_rng(seed)
    N, K = 256, 512
    W = _normal(rng, (N, K))
    cols = rng.choice(K, size=int(round(0.02 * K)), replace=False)
    W[:, cols] *= np.float32(20.0)
    x = rng.standard_normal(size=(1, K), dtype=np.float32)
    return DenseCase("tiny_int4_256x512", "int4", W, x)


def fp4_square(seed: int = 0, n: int = 4096, batch: int = 4) -> DenseCase:
    """4096 x 4096 fp16 weights with 1% outlier input columns, x fp16 [4, 4096].

    Draws: W ~ N(0, 0.02) fp32; 41 = round(0.01 * 4096) columns without
    replacement scaled by 20 in fp32; cast to fp16; x ~ N(0, 1) [batch, n] fp16.
    Batch 1 uses the first row of x.
    """
    rng = np.random.default_rng(seed)
    W = _normal(rng, (n, n))
    cols = rng.choice(n, size=int(round(0.01 * n)), replace=False)
    W[:, cols] *= np.float32(20.0)
    W = W.astype(np.float16)
    x = rng.standard_normal(size=(batch, n), dtype=np.float32).astype(np.float16)
    return DenseCase("fp4_%dx%d" % (n, n), "fp4", W, x)


def lm_head_km4(seed: int = 0, N: int = 248320, K: int = 2048, batch: int = 8) -> DenseCase:
    """lm_head-shaped weights 248320 x 2048 fp16, x fp16 [8, 2048].

    Draws: W ~ N(0, 0.02) fp32 -> fp16; x ~ N(0, 1) [batch, K] fp16.
    Batch 1 uses the first row of x.
    """
    rng = np.random.default_rng(seed)
    W = _normal(rng, (N, K)).astype(np.float16)
    x = rng.standard_normal(size=(batch, K), dtype=np.float32).astype(np.float16)
    return DenseCase("lm_head_km4_%dx%d" % (N, K), "km4", W, x)


def int8_head(seed: int = 0, N: int = 130560, K: int = 2560, heavy_frac: float = 0.05) -> DenseCase:
    """130560 x 2560 fp16 head with heavy-tailed rows, x fp16 [1, 2560].

    Draws: W ~ N(0, 0.02) fp32; round(0.05 * N) rows chosen without
    replacement are redrawn as 0.02 * Student-t(3) (not variance-normalised);
    cast to fp16; x ~ N(0, 1) [1, K] fp16.
    """
    rng = np.random.default_rng(seed)
    W = _normal(rng, (N, K))
    rows = np.sort(rng.choice(N, size=int(round(heavy_frac * N)), replace=False))
    W[rows] = (np.float32(SIGMA) * rng.standard_t(3, size=(len(rows), K))).astype(np.float32)
    W = W.astype(np.float16)
    x = rng.standard_normal(size=(1, K), dtype=np.float32).astype(np.float16)
    return DenseCase("int8_head_%dx%d" % (N, K), "int8", W, x)


@dataclass
class MoECase:
    name: str
    W_gate_up: np.ndarray   # [E, 2I, H] fp16: rows 0..I-1 gate, I..2I-1 up
    W_down: np.ndarray      # [E, H, I] fp16
    logits: np.ndarray      # [T, E] fp32
    x: np.ndarray           # [T, H] fp16
    topk: int


def moe(seed: int = 0, E: int = 256, H: int = 2048, I: int = 512, T: int = 8, topk: int = 8) -> MoECase:
    """256 experts, gate/up 2 x (512 x 2048) and down 2048 x 512, top-8 routing.

    Draws: gate/up ~ N(0, 0.02) [E, 2I, H] fp16; down ~ N(0, 0.02) [E, H, I]
    fp16; router logits ~ N(0, 1) [T, E] fp32; x ~ N(0, 1) [T, H] fp16.
    Smaller token counts use the first T rows of logits and x.
    """
    rng = np.random.default_rng(seed)
    gu = _normal(rng, (E * 2 * I, H)).astype(np.float16).reshape(E, 2 * I, H)
    dn = _normal(rng, (E * H, I)).astype(np.float16).reshape(E, H, I)
    logits = rng.standard_normal(size=(T, E), dtype=np.float32)
    x = rng.standard_normal(size=(T, H), dtype=np.float32).astype(np.float16)
    return MoECase("moe_E%d_H%d_I%d_T%d" % (E, H, I, T), gu, dn, logits, x, topk)


def small_dense(fmt: str, N: int, K: int, batch: int = 1, seed: int = 0,
                dtype=np.float16, outlier_frac: float = 0.0) -> DenseCase:
    """Generic small case for parity sweeps: N(0, 0.02) weights, N(0, 1) x.

    Draws: W [N, K]; optional outlier columns (x20) without replacement; x [batch, K].
    """
    rng = np.random.default_rng(seed)
    W = _normal(rng, (N, K))
    if outlier_frac > 0:
        cols = rng.choice(K, size=max(1, int(round(outlier_frac * K))), replace=False)
        W[:, cols] *= np.float32(20.0)
    x = rng.standard_normal(size=(batch, K), dtype=np.float32)
    return DenseCase("%s_%dx%d_b%d" % (fmt, N, K, batch), fmt, W.astype(dtype), x.astype(dtype))
