"""Correlation-aware expert placement (test infrastructure only).

"Zyphra says routing-pattern expert placement speeds MoE token communication up to
2.63x on AMD MI300X": experts that tokens often choose together are placed on the
same destination, so a token's copies to that destination collapse into one (the
pair statistics item: a few expert pairs carry a large share of tokens).  The page
gives the idea, not an algorithm.  What is built here, and its reading:

* pair_counts: C[a, b] = number of tokens whose expert set contains both a and b
  (a token's repeated expert counts once; ids outside [0, G) are left out); the
  diagonal C[a, a] is the number of tokens that choose a.  With S the 0/1
  token-by-expert incidence matrix this is exactly C = S^T S, which is how it is
  computed here.
* greedy_place(C, B): every bucket holds G/B experts.  Steps, in order:
    1. every expert starts as its own cluster;
    2. the pairs (a < b) with C[a, b] > 0 are visited by count descending, ties by
       (a, b) ascending; a pair joins its two clusters when they differ and the merged
       size is at most G/B (the merged cluster is named by its smaller expert);
    3. clusters are ordered by size descending, ties by smallest member;
    4. each cluster goes whole into the lowest-numbered bucket with room for it; a
       cluster that fits nowhere waits;
    5. the experts of the waiting clusters, in that cluster order and ascending id
       inside each, fill the lowest-numbered buckets with a free place.
"""
from __future__ import annotations

import numpy as np


def pair_counts(topk_idx: np.ndarray, G: int) -> np.ndarray:
    """int64 [G, G] co-occurrence counts, C = S^T S."""
    idx = np.asarray(topk_idx, dtype=np.int64)
    M = idx.shape[0]
    S = np.zeros((M, G), dtype=np.int64)
    tok = np.repeat(np.arange(M), idx.shape[1])
    e = idx.reshape(-1)
    ok = (e >= 0) & (e < G)
    S[tok[ok], e[ok]] = 1
    return S.T @ S


def _visit_order(a_idx: np.ndarray, b_idx: np.ndarray, cnt: np.ndarray) -> np.ndarray:
    """Step 2's visiting order of the pairs: count descending, then a, then b."""
    return np.lexsort((b_idx, a_idx, -cnt))


def _bucket_order(B: int):
    """Steps 4 and 5 try the buckets lowest-numbered first."""
    return range(B)


def greedy_clusters(C: np.ndarray, cap: int) -> list[list[int]]:
    """Steps 1-2: clusters of at most `cap` experts, each a sorted member list, in
    step-3 order (size descending, then smallest member)."""
    C = np.asarray(C, dtype=np.int64)
    G = C.shape[0]
    parent = list(range(G))
    size = [1] * G

    def find(a: int) -> int:
        while parent[a] != a:
            a = parent[a]
        return a

    a_idx, b_idx = np.triu_indices(G, k=1)
    cnt = C[a_idx, b_idx]
    keep = cnt > 0
    a_idx, b_idx, cnt = a_idx[keep], b_idx[keep], cnt[keep]
    for p in _visit_order(a_idx, b_idx, cnt):
        ra, rb = find(int(a_idx[p])), find(int(b_idx[p]))
        if ra != rb and size[ra] + size[rb] <= cap:
            lo, hi = min(ra, rb), max(ra, rb)
            parent[hi] = lo
            size[lo] += size[hi]

    members: dict[int, list[int]] = {}
    for e in range(G):
        members.setdefault(find(e), []).append(e)
    return sorted(members.values(), key=lambda m: (-len(m), m[0]))


def greedy_place(C: np.ndarray, B: int) -> np.ndarray:
    """int32 [G] expert -> bucket map, G/B experts per bucket (steps 1-5)."""
    G = np.asarray(C).shape[0]
    if G % B:
        raise ValueError("G must be a multiple of B")
    cap = G // B
    bucket = np.full(G, -1, dtype=np.int32)
    fill = [0] * B
    waiting = []
    for m in greedy_clusters(C, cap):
        for b in _bucket_order(B):
            if fill[b] + len(m) <= cap:
                bucket[m] = b
                fill[b] += len(m)
                break
        else:
            waiting.append(m)
    for m in waiting:
        for e in m:
            b = next(b for b in _bucket_order(B) if fill[b] < cap)
            bucket[e] = b
            fill[b] += 1
    return bucket
