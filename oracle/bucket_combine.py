"""Receiver-side expansion and the per-(token, bucket) pre-reduced combine (test
infrastructure only).

In dedup mode a token crosses to a destination bucket once ("Zyphra says
routing-pattern expert placement ...", the copy-reduction item).  The steps on
either side of the path then are:

* expand (receiver): every (t, j) whose expert lives in bucket b needs its own
  expert-major input row, so the received row of (t, b) is copied to the slot of each
  such (t, j):  expert_in[slot[t, j]] = recv[send_row[t, j]]  (raw bytes; scales
  follow the rows).
* combine_partial (receiver, on the way back): the token's experts inside one bucket
  are summed before the return, one row per (t, b) instead of one per (t, j):
      partial[r] = bf16( sum over j with send_row[t, j] = r, j ascending,
                         of fl32(w[t, j] * expert_out[slot[t, j]]) )
  with an fp32 accumulator starting at +0.0, unfused, one round to nearest even.
* combine_reduce (sender): the token's partials, one per distinct bucket, are added
  in ascending bucket order -- which is ascending send row, since send rows are
  bucket-major:
      y[t] = bf16( sum over distinct r in send_row[t, :], ascending, of f32(partial[r]) )
  again from +0.0, unfused, one final rounding.

The pages describe the one-copy-per-destination dispatch but not the return path;
this mirror image of it, with bf16 partials (the return carries the same format as
the forward rows) and the orders above, is the reading taken.  The operation order
follows the same one-owner, source-order rule as the flat combine ("Purlin ...",
section 3.3, SCORE).
"""
from __future__ import annotations

from typing import Optional

import numpy as np

from .numerics import bf16_to_f32, f32_to_bf16_rne


def expand(recv: np.ndarray, send_row: np.ndarray, slot: np.ndarray, expert_rows: int,
           recv_scale: Optional[np.ndarray] = None, fill: int = 0):
    """expert_in[slot[t, j]] = recv[send_row[t, j]] for every (t, j)."""
    src = send_row.reshape(-1).astype(np.int64)
    dst = slot.reshape(-1).astype(np.int64)
    out = np.full((expert_rows,) + recv.shape[1:], fill, dtype=recv.dtype)
    out[dst] = recv[src]
    out_scale = None
    if recv_scale is not None:
        out_scale = np.full((expert_rows,) + recv_scale.shape[1:], np.nan, dtype=np.float32)
        out_scale[dst] = recv_scale[src]
    return out, out_scale


def combine_partial(expert_out: np.ndarray, weights: np.ndarray, slot: np.ndarray,
                    send_row: np.ndarray, partial_rows: int) -> np.ndarray:
    """Per-(token, bucket) partial sums, bf16 bits [partial_rows, N]."""
    M, k = slot.shape
    N = expert_out.shape[1]
    w = np.asarray(weights, dtype=np.float32)
    acc = np.zeros((partial_rows, N), dtype=np.float32)
    for j in range(k):
        # for a fixed j the rows send_row[:, j] belong to different tokens, so they
        # are distinct and the indexed update touches each row once
        r = send_row[:, j].astype(np.int64)
        prod = w[:, j:j + 1] * bf16_to_f32(expert_out[slot[:, j]])
        acc[r] = acc[r] + prod
    return f32_to_bf16_rne(acc)


def combine_reduce(partial: np.ndarray, send_row: np.ndarray) -> np.ndarray:
    """y[t] = bf16(sum of the token's distinct partial rows in ascending row order)."""
    M, k = send_row.shape
    N = partial.shape[1]
    rows = np.sort(send_row.astype(np.int64), axis=1)
    acc = np.zeros((M, N), dtype=np.float32)
    for i in range(k):
        r = rows[:, i]
        first = np.ones(M, dtype=bool) if i == 0 else r != rows[:, i - 1]
        acc = np.where(first[:, None], acc + bf16_to_f32(partial[r]), acc)
    return f32_to_bf16_rne(acc)
