"""Dispatch: copy each token's row into its send rows (test infrastructure only).

"All2all performance comparison between Triton-distributed and DeepEP" ("Test Code
Snippet", and the note under the results table) names the gather of token rows into
the destination-grouped send buffer, with the optional per-row scales travelling
beside the data (WITH_SCALE).  With dedup ("Zyphra says routing-pattern expert
placement ...") several (t, j) share one send row; they all carry the same token, so
writing it once or several times is the same.

Rows are raw bytes: dispatch does no arithmetic.
"""
from __future__ import annotations

from typing import Optional

import numpy as np


def dispatch(x: np.ndarray, send_row: np.ndarray, out_rows: int,
             x_scale: Optional[np.ndarray] = None, fill: int = 0):
    """Return (out [out_rows, ...] same dtype as x, out_scale or None).

    ``out[send_row[t, j]] = x[t]`` and ``out_scale[send_row[t, j]] = x_scale[t]`` for
    every (t, j); rows nobody writes keep ``fill`` (bytes) / NaN (scales).
    """
    x = np.asarray(x)
    M, k = send_row.shape
    out = np.full((out_rows,) + x.shape[1:], fill, dtype=x.dtype)
    rows = send_row.reshape(-1).astype(np.int64)
    tok = np.repeat(np.arange(M), k)
    out[rows] = x[tok]
    out_scale = None
    if x_scale is not None:
        out_scale = np.full((out_rows,) + x_scale.shape[1:], np.nan, dtype=np.float32)
        out_scale[rows] = x_scale[tok]
    return out, out_scale
