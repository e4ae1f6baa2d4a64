"""Grouped GEMM over the per-expert layout, and its device-side tile metadata (test
infrastructure only).

"Add Triton grouped-GEMM for MoE experts on Ampere/Ada" (DeepSpeed PR 8180), "What this
PR does": one grouped GEMM multiplies a 2D row block with a 3D weight stack using the
per-group cumulative offsets `offs`, with the tile -> group map computed on the device
from `offs` (no device -> host sync), and weights kept in their native [E, N, K]
layout (trans_b).  Here the groups are experts: rows [expert_offset[e],
expert_offset[e] + expert_count[e]) of the slot-indexed expert inputs belong to expert
e, and

    y[r, n] = bf16( sum_k x[r, k] * w[e, n, k] )      for r in expert e's rows

The definition is the exact sum (computed here in float64) rounded once to bf16; a
GPU computing it with fp32 accumulation differs from it by less than its own fp32
rounding error, which the parity tests bound.

gemm_tiles: the GEMM's row tiles, experts in ascending id, each expert's rows cut into
tiles of `tile_m` (the last one shorter): entries (expert, first row, rows).
"""
from __future__ import annotations

import numpy as np

from .numerics import bf16_to_f32


def gemm_tiles(expert_offset: np.ndarray, expert_count: np.ndarray, tile_m: int):
    tiles = []
    for e in range(len(expert_count)):
        c = int(expert_count[e])
        for i in range((c + tile_m - 1) // tile_m):
            tiles.append((e, int(expert_offset[e]) + i * tile_m, min(tile_m, c - i * tile_m)))
    return tiles


def grouped_gemm(x: np.ndarray, w: np.ndarray, expert_offset: np.ndarray,
                 expert_count: np.ndarray) -> np.ndarray:
    """x: bf16 bits [rows, K]; w: bf16 bits [G, Nout, K].  Returns the exact products
    (float64 [rows, Nout]; rows of no expert stay 0).  The result y is these values
    rounded once to bf16."""
    rows, K = x.shape
    G, Nout, _ = w.shape
    exact = np.zeros((rows, Nout), dtype=np.float64)
    xf = bf16_to_f32(x).astype(np.float64)
    for e in range(G):
        r0, c = int(expert_offset[e]), int(expert_count[e])
        if c == 0:
            continue
        exact[r0:r0 + c] = xf[r0:r0 + c] @ bf16_to_f32(w[e]).astype(np.float64).T
    return exact


def magnitude(x: np.ndarray, w: np.ndarray, expert_offset: np.ndarray,
              expert_count: np.ndarray) -> np.ndarray:
    """sum_k |x[r, k] * w[e, n, k]|, the scale of the fp32 accumulation error."""
    return grouped_gemm(np.asarray(x) & 0x7FFF, np.asarray(w) & 0x7FFF, expert_offset,
                        expert_count)
