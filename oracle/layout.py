"""Dispatch layout: counts, cumulative offsets, slot map and dedup send rows.

Test infrastructure only.  What is computed, and where it comes from:

* "All2all performance comparison between Triton-distributed and DeepEP", "Test Code
  Snippet": the exchange consumes a send buffer grouped by destination rank, the
  per-destination split counts and their cumulative sums; experts are grouped
  EXPERTS_PER_RANK to a rank out of NUM_TOT_EXPERTS.  Here a destination is a
  *bucket* and the expert -> bucket map is arbitrary.
* "Add Triton grouped-GEMM for MoE experts on Ampere/Ada", "What this PR does": the
  grouped GEMM reads per-expert row offsets ``offs`` from device memory, so every
  expert's rows are contiguous and its offset is exported.
* "Zyphra says routing-pattern expert placement ...": with dedup, each (token, bucket)
  pair is one send row, whatever the number of the token's experts in that bucket.
* "Purlin ...", section 3.1 (Layouts): the send buffer is scattered-V, partitions
  indexed by destination with variable sizes.

Readings where the pages are silent:

* Experts are laid out in memory ordered by (bucket, expert id); with a contiguous
  map that is plain ascending id.
* Inside an expert's run, entries are ordered by flat index t*k + j (ascending token,
  then top-k position): the slot map is a *stable* counting sort.
* A token may name the same expert twice; each occurrence gets its own slot.
* With dedup on, the send buffer is bucket-major and, inside a bucket, ordered by
  ascending token.  With dedup off the send rows are the slots.
* An expert id outside [0, G) makes ``status`` = first bad flat index + 1; a map
  entry outside [0, B) makes it -(first bad expert + 1), checked first.  The pages
  define no error behaviour; either way the other outputs are unspecified.

Two formulations are given: ``dispatch_layout`` (array form, the one tests compare
the GPU with) and ``dispatch_layout_loops`` (per-entry counting loops, for small
inputs).  Tests pin both against a third, tuple-sorting form and against
invariants.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np


@dataclass
class Layout:
    status: int                                   # 0 ok, else first bad flat index + 1
    expert_count: Optional[np.ndarray] = None     # [G]   entries routed to each expert
    expert_offset: Optional[np.ndarray] = None    # [G]   first slot of each expert's run
    bucket_count: Optional[np.ndarray] = None     # [B]   rows sent to each bucket
    bucket_offset: Optional[np.ndarray] = None    # [B+1] exclusive cumsum, [B] = R
    slot: Optional[np.ndarray] = None             # [M,k] expert-major position of (t, j)
    send_row: Optional[np.ndarray] = None         # [M,k] send-buffer row of (t, j)
    send_token: Optional[np.ndarray] = None       # [R]   token of each send row

    @property
    def R(self) -> int:
        return int(self.bucket_offset[-1])


def _first_bad(flat: np.ndarray, ebkt: np.ndarray, B: int) -> int:
    bad_map = np.flatnonzero((ebkt < 0) | (ebkt >= B))
    if bad_map.size:
        return -(int(bad_map[0]) + 1)
    G = ebkt.shape[0]
    bad = np.flatnonzero((flat < 0) | (flat >= G))
    return int(bad[0]) + 1 if bad.size else 0


def dispatch_layout(topk_idx: np.ndarray, expert_bucket: np.ndarray, B: int,
                    dedup: bool) -> Layout:
    """Array formulation of the layout."""
    idx = np.asarray(topk_idx, dtype=np.int64)
    M, k = idx.shape
    ebkt = np.asarray(expert_bucket, dtype=np.int64)
    G = ebkt.shape[0]
    flat = idx.reshape(-1)
    status = _first_bad(flat, ebkt, B)
    if status:
        return Layout(status=status)

    # Memory order of experts: sigma = experts sorted by (bucket, id).
    sigma = np.lexsort((np.arange(G), ebkt))
    sigma_pos = np.empty(G, dtype=np.int64)
    sigma_pos[sigma] = np.arange(G)

    count = np.bincount(flat, minlength=G)
    run_start = np.concatenate(([0], np.cumsum(count[sigma])[:-1]))
    expert_offset = np.empty(G, dtype=np.int64)
    expert_offset[sigma] = run_start

    # slot = position of entry (t, j) when all M*k entries are stably sorted by the
    # memory position of their expert.
    order = np.argsort(sigma_pos[flat], kind="stable")
    slot = np.empty(M * k, dtype=np.int64)
    slot[order] = np.arange(M * k)

    token = np.repeat(np.arange(M, dtype=np.int64), k)
    entry_bucket = ebkt[flat]
    if not dedup:
        bucket_count = np.bincount(entry_bucket, minlength=B)
        send_row = slot
        send_token = np.empty(M * k, dtype=np.int64)
        send_token[slot] = token
    else:
        # distinct (bucket, token) pairs, bucket-major then ascending token
        key = entry_bucket * M + token
        pairs = np.unique(key)
        bucket_count = np.bincount(pairs // M, minlength=B)
        send_row = np.searchsorted(pairs, key)
        send_token = pairs % M
    bucket_offset = np.concatenate(([0], np.cumsum(bucket_count)))

    i32 = lambda a: np.asarray(a, dtype=np.int32)
    return Layout(status=0, expert_count=i32(count), expert_offset=i32(expert_offset),
                  bucket_count=i32(bucket_count), bucket_offset=i32(bucket_offset),
                  slot=i32(slot).reshape(M, k), send_row=i32(send_row).reshape(M, k),
                  send_token=i32(send_token))


def dispatch_layout_loops(topk_idx, expert_bucket, B: int, dedup: bool) -> Layout:
    """The same layout as explicit counting loops (pure Python: small inputs only)."""
    idx = [[int(e) for e in row] for row in np.asarray(topk_idx)]
    ebkt = [int(b) for b in np.asarray(expert_bucket)]
    M, k, G = len(idx), (len(idx[0]) if idx else 0), len(ebkt)
    for e in range(G):
        if not 0 <= ebkt[e] < B:
            return Layout(status=-(e + 1))
    for t in range(M):
        for j in range(k):
            if not 0 <= idx[t][j] < G:
                return Layout(status=t * k + j + 1)

    # 1. count entries per expert
    count = [0] * G
    for t in range(M):
        for j in range(k):
            count[idx[t][j]] += 1
    # 2. expert runs in (bucket, id) order
    expert_offset = [0] * G
    running = 0
    for b in range(B):
        for e in range(G):
            if ebkt[e] == b:
                expert_offset[e] = running
                running += count[e]
    # 3. one cursor per expert, entries visited in (t, j) order
    cursor = list(expert_offset)
    slot = [[0] * k for _ in range(M)]
    for t in range(M):
        for j in range(k):
            e = idx[t][j]
            slot[t][j] = cursor[e]
            cursor[e] += 1

    if not dedup:
        bucket_count = [sum(count[e] for e in range(G) if ebkt[e] == b) for b in range(B)]
        send_row = [row[:] for row in slot]
        send_token = [0] * (M * k)
        for t in range(M):
            for j in range(k):
                send_token[slot[t][j]] = t
    else:
        token_buckets = [set(ebkt[e] for e in idx[t]) for t in range(M)]
        bucket_count = [sum(1 for t in range(M) if b in token_buckets[t]) for b in range(B)]
        start = [0] * B
        for b in range(1, B):
            start[b] = start[b - 1] + bucket_count[b - 1]
        cur = list(start)
        drow = {}
        for t in range(M):                      # ascending token inside each bucket
            for b in range(B):
                if b in token_buckets[t]:
                    drow[(t, b)] = cur[b]
                    cur[b] += 1
        send_row = [[drow[(t, ebkt[idx[t][j]])] for j in range(k)] for t in range(M)]
        send_token = [0] * sum(bucket_count)
        for (t, b), r in drow.items():
            send_token[r] = t
    bucket_offset = [0]
    for c in bucket_count:
        bucket_offset.append(bucket_offset[-1] + c)

    a = lambda v: np.asarray(v, dtype=np.int32)
    return Layout(status=0, expert_count=a(count), expert_offset=a(expert_offset),
                  bucket_count=a(bucket_count), bucket_offset=a(bucket_offset),
                  slot=a(slot).reshape(M, k), send_row=a(send_row).reshape(M, k),
                  send_token=a(send_token))
