"""Expert stand-ins between dispatch and combine (test infrastructure only).

No trained experts are involved: each expert is a fixed elementwise map of the row it
receives, so that combine has inputs whose correct result is known in closed form.

* identity: the output row is the dispatched bf16 row.
* scale:    o = bf16( f32(x) * (1 + e/256) ), the factor exact in fp32.
* dequant:  o = bf16( f32(q) * s ), q an fp8 e4m3 code and s the fp32 scale of its
            128-element block.

Per-expert buffers are slot-indexed (M*k rows, expert-major).  With dedup on, the
send buffer has one row per (token, bucket); the stand-in reads each (t, j)'s row
through ``send_row`` and writes it to ``slot`` -- the receiver-side expansion.
"""
from __future__ import annotations

from typing import Optional

import numpy as np

from .numerics import bf16_to_f32, f32_to_bf16_rne, e4m3_to_f32


def expert_outputs(kind: str, sent: np.ndarray, send_row: np.ndarray, slot: np.ndarray,
                   topk_idx: np.ndarray, sent_scale: Optional[np.ndarray] = None,
                   block: int = 128) -> np.ndarray:
    """Return expert_out, uint16 bf16 bits [M*k, N], indexed by slot."""
    M, k = slot.shape
    src = send_row.reshape(-1).astype(np.int64)
    dst = slot.reshape(-1).astype(np.int64)
    e = np.asarray(topk_idx, dtype=np.int64).reshape(-1)
    N = sent.shape[1]
    out = np.empty((M * k, N), dtype=np.uint16)
    chunk = 4096
    for c0 in range(0, M * k, chunk):
        c1 = min(M * k, c0 + chunk)
        rows = sent[src[c0:c1]]
        if kind == "identity":
            o = rows
        elif kind == "scale":
            factor = (np.float32(1.0) + e[c0:c1].astype(np.float32) / np.float32(256.0))
            o = f32_to_bf16_rne(bf16_to_f32(rows) * factor[:, None].astype(np.float32))
        elif kind == "dequant":
            s = sent_scale[src[c0:c1]]
            q = e4m3_to_f32(rows).reshape(c1 - c0, N // block, block)
            o = f32_to_bf16_rne((q * s[:, :, None]).reshape(c1 - c0, N))
        else:
            raise ValueError(kind)
        out[dst[c0:c1]] = o
    return out
