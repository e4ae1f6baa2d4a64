"""Combine: routing-weighted top-k sum back in token order (test infrastructure only).

y[t, i] = bf16( sum over j = 0..k-1 of w[t, j] * expert_out[slot[t, j], i] )

The floating-point operation order is fixed by the determinism rule of "Purlin:
Separating Orchestration from the Datapath of Collectives", section 3.3 (SCORE): one
owner per output element and accumulation in source order.  Read here as: an fp32
accumulator that starts at +0.0, then for j ascending one fp32 product (rounded) and
one fp32 add (rounded) -- no fused multiply-add -- and a single round-to-nearest-even
to bf16 at the end.  numpy's float32 ufuncs are unfused IEEE single operations, so
the loop below is that sequence literally, vectorised over tokens and elements.
"""
from __future__ import annotations

import numpy as np

from .numerics import bf16_to_f32, f32_to_bf16_rne


def combine(expert_out: np.ndarray, weights: np.ndarray, slot: np.ndarray,
            chunk_tokens: int = 1024) -> np.ndarray:
    """expert_out: uint16 bf16 bits [rows, N]; weights float32 [M, k]; slot int [M, k].
    Returns y as uint16 bf16 bits [M, N]."""
    expert_out = np.asarray(expert_out, dtype=np.uint16)
    w = np.asarray(weights, dtype=np.float32)
    M, k = slot.shape
    N = expert_out.shape[1]
    y = np.empty((M, N), dtype=np.uint16)
    for t0 in range(0, M, chunk_tokens):
        t1 = min(M, t0 + chunk_tokens)
        acc = np.zeros((t1 - t0, N), dtype=np.float32)
        for j in range(k):
            rows = bf16_to_f32(expert_out[slot[t0:t1, j]])
            prod = w[t0:t1, j:j + 1] * rows          # fp32 multiply, rounded
            acc = acc + prod                          # fp32 add, rounded
        y[t0:t1] = f32_to_bf16_rne(acc)
    return y
