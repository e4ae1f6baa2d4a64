"""Seeded synthetic MoE routing workloads.

This module only *draws inputs*: routing (top-k expert ids), the expert-to-bucket
map, routing weights and the token rows.  It contains none of the dispatch/combine
arithmetic, so both the HIP path and the CPU oracle can consume its outputs
without sharing any code of the method.

Shapes follow the problem statement of "All2all performance comparison between
Triton-distributed and DeepEP" (section "Benchmark Configuration": hidden 7168,
256 experts, top-8, bfloat16) and the expert-pair statistics of "Zyphra says
routing-pattern expert placement speeds MoE token communication up to 2.63x on
AMD MI300X" (64 of the 8,128 expert pairs of a 128-expert layer carry 42% of
tokens).  Skewed routing uses a Zipf law, the synthetic stand-in that "Diagnosing
Overhead in Dispatch Operations: Cross-architecture Observatory" (abstract)
discusses; real routing traces are not available, so all routing here is
synthetic and seeded.

Every workload is drawn from ``numpy.random.default_rng([1234, cfg_id])`` in a
fixed order: routing, then routing logits, then token rows.

Conversions to bf16 and fp8 use torch's CPU casts (round-to-nearest-even); the
oracle has its own independent codecs that tests pin against these.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

SEED = 1234

# Zipf exponent, hot-pair fraction and pair count of the five standard workloads.
ZIPF_S = 1.2
HOT_PAIR_FRACTION = 0.42
N_HOT_PAIRS = 64
FP8_BLOCK = 128
FP8_MAX = 448.0


@dataclass
class Workload:
    """One seeded MoE dispatch/combine problem (all arrays are host numpy)."""

    name: str
    cfg_id: int
    M: int                      # tokens
    N: int                      # hidden size (elements per row)
    G: int                      # experts
    k: int                      # top-k
    B: int                      # destination buckets
    dtype: str                  # "bf16" or "fp8"
    topk_idx: np.ndarray        # int32 [M, k], expert ids
    expert_bucket: np.ndarray   # int32 [G], bucket of each expert
    weights: np.ndarray         # float32 [M, k], routing weights
    x: np.ndarray               # uint16 [M, N] bf16 bits, or uint8 [M, N] e4m3 bits
    x_scale: Optional[np.ndarray]  # float32 [M, N/128] (fp8 only) else None
    standin: str                # expert stand-in: "identity", "scale", "dequant"
    dedup: bool                 # the mode the workload is quoted in
    meta: dict = field(default_factory=dict)

    @property
    def row_bytes(self) -> int:
        return self.N * (2 if self.dtype == "bf16" else 1)


# --------------------------------------------------------------------------- routing


def uniform_topk(rng: np.random.Generator, M: int, G: int, k: int) -> np.ndarray:
    """k distinct experts per token, uniformly at random, in random draw order."""
    keys = rng.random((M, G), dtype=np.float32)
    return np.argsort(keys, axis=1, kind="stable")[:, :k].astype(np.int32)


def zipf_topk(rng: np.random.Generator, M: int, G: int, k: int,
              s: float = ZIPF_S) -> tuple[np.ndarray, np.ndarray]:
    """k experts per token drawn without replacement from Zipf(s) over a permutation.

    Rank r (0-based) has weight (r+1)^-s; the expert of rank r is perm[r].  Successive
    draws without replacement with renormalisation are sampled exactly by the
    Gumbel-top-k construction: the k largest of log p_r + Gumbel noise, in
    descending order, are the draws in order.
    """
    perm = rng.permutation(G).astype(np.int32)
    logp = -s * np.log(np.arange(1, G + 1, dtype=np.float64))
    keys = logp[None, :] + rng.gumbel(size=(M, G))
    ranks = np.argsort(-keys, axis=1, kind="stable")[:, :k]
    return perm[ranks].astype(np.int32), perm


def correlated_pair_topk(rng: np.random.Generator, M: int, G: int, k: int,
                         n_pairs: int = N_HOT_PAIRS,
                         q: float = HOT_PAIR_FRACTION) -> tuple[np.ndarray, np.ndarray]:
    """Top-k routing with correlated expert pairs.

    ``n_pairs`` disjoint hot pairs are consecutive entries of a seeded permutation of
    the experts.  Each token has k//2 pair slots; each slot becomes, with probability
    ``q``, a hot pair chosen uniformly among those whose experts the token does not
    already hold.  The remaining slots are filled with distinct uniform experts and
    the token's k entries are then put in a random order.
    """
    assert 2 * n_pairs <= G and k % 2 == 0
    perm = rng.permutation(G).astype(np.int32)
    pairs = perm[: 2 * n_pairs].reshape(n_pairs, 2)
    out = np.empty((M, k), dtype=np.int32)
    slot_hot = rng.random((M, k // 2)) < q
    pair_pick = rng.random((M, k // 2))
    fill_keys = rng.random((M, G))
    order_keys = rng.random((M, k))
    for t in range(M):
        chosen: list[int] = []
        taken = np.zeros(G, dtype=bool)
        for s in range(k // 2):
            if not slot_hot[t, s]:
                continue
            free = np.flatnonzero(~(taken[pairs[:, 0]] | taken[pairs[:, 1]]))
            if free.size == 0:
                continue
            a, b = pairs[free[int(pair_pick[t, s] * free.size)]]
            chosen += [int(a), int(b)]
            taken[a] = taken[b] = True
        need = k - len(chosen)
        if need:
            keys = np.where(taken, np.inf, fill_keys[t])
            chosen += [int(e) for e in np.argsort(keys, kind="stable")[:need]]
        out[t] = np.asarray(chosen, dtype=np.int32)[np.argsort(order_keys[t], kind="stable")]
    return out, pairs.astype(np.int32)


def softmax_weights(rng: np.random.Generator, M: int, k: int) -> np.ndarray:
    """Routing weights: softmax over each token's k N(0,1) logits (fp64, then fp32)."""
    logits = rng.standard_normal((M, k))
    z = np.exp(logits - logits.max(axis=1, keepdims=True))
    return (z / z.sum(axis=1, keepdims=True)).astype(np.float32)


def contiguous_buckets(G: int, B: int) -> np.ndarray:
    """Bucket b holds experts [b*G/B, (b+1)*G/B): EXPERTS_PER_RANK consecutive experts."""
    assert G % B == 0
    return (np.arange(G, dtype=np.int32) // (G // B)).astype(np.int32)


def pair_aware_buckets(pairs: np.ndarray, G: int, B: int) -> np.ndarray:
    """Hot pair i goes whole to bucket i mod B; every other expert fills the buckets
    in ascending id order so that each bucket holds G/B experts."""
    per = G // B
    m = np.full(G, -1, dtype=np.int32)
    fill = np.zeros(B, dtype=np.int64)
    for i, (a, b) in enumerate(pairs):
        m[a] = m[b] = i % B
        fill[i % B] += 2
    for e in range(G):
        if m[e] < 0:
            bkt = int(np.flatnonzero(fill < per)[0])
            m[e] = bkt
            fill[bkt] += 1
    return m


def round_robin_buckets(G: int, B: int) -> np.ndarray:
    return (np.arange(G, dtype=np.int32) % B).astype(np.int32)


# --------------------------------------------------------------------------- rows


def bf16_bits_from_f32(v: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round-to-nearest-even, via torch's cast."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def normal_bf16_rows(rng: np.random.Generator, M: int, N: int,
                     chunk_rows: int = 8192) -> np.ndarray:
    out = np.empty((M, N), dtype=np.uint16)
    for r0 in range(0, M, chunk_rows):
        r1 = min(M, r0 + chunk_rows)
        out[r0:r1] = bf16_bits_from_f32(rng.standard_normal((r1 - r0, N), dtype=np.float32))
    return out


def fp8_quantise_blocks(v: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Per-128-element block fp8 e4m3 (OCP, 'fn') quantisation of float32 rows.

    scale = amax/448 in fp32 (1.0 for an all-zero block); code = RNE(v/scale)
    saturated to +-448.  Returns (uint8 codes [M,N], float32 scales [M,N/128]).
    """
    import torch
    M, N = v.shape
    assert N % FP8_BLOCK == 0
    blk = v.reshape(M, N // FP8_BLOCK, FP8_BLOCK)
    amax = np.abs(blk).max(axis=2)
    scale = np.where(amax > 0, amax / np.float32(FP8_MAX), np.float32(1.0)).astype(np.float32)
    q = np.clip(blk / scale[:, :, None], -FP8_MAX, FP8_MAX).astype(np.float32)
    codes = torch.from_numpy(np.ascontiguousarray(q)).to(torch.float8_e4m3fn)
    return codes.view(torch.uint8).numpy().reshape(M, N), scale


def normal_fp8_rows(rng: np.random.Generator, M: int, N: int,
                    chunk_rows: int = 8192) -> tuple[np.ndarray, np.ndarray]:
    codes = np.empty((M, N), dtype=np.uint8)
    scales = np.empty((M, N // FP8_BLOCK), dtype=np.float32)
    for r0 in range(0, M, chunk_rows):
        r1 = min(M, r0 + chunk_rows)
        codes[r0:r1], scales[r0:r1] = fp8_quantise_blocks(
            rng.standard_normal((r1 - r0, N), dtype=np.float32))
    return codes, scales


# --------------------------------------------------------------------------- workloads

# Full sizes of the five standard workloads.
STANDARD_M = {1: 64, 2: 4096, 3: 16384, 4: 16384, 5: 65536}

WORKLOAD_NAMES = {
    1: "uniform-top8-M64",
    2: "uniform-top8-M4096-scaled-experts",
    3: "zipf1.2-top8-M16384",
    4: "correlated-pairs-top8-M16384-N2048-G128",
    5: "uniform-top8-M65536-fp8",
}


def make_workload(cfg_id: int, M: Optional[int] = None, map_kind: str = "pair",
                  with_rows: bool = True) -> Workload:
    """Draw standard workload ``cfg_id`` (1..5), optionally at a reduced token count M.

    cfg 1: M=64, N=7168 bf16, G=256, top-8 uniform distinct, B=8 contiguous buckets,
           identity experts.
    cfg 2: M=4096, as cfg 1, dedup on, experts scale rows by (1 + e/256).
    cfg 3: M=16384, N=7168 bf16, top-8 without replacement from Zipf(1.2) over a
           seeded expert permutation, B=8 contiguous buckets, identity experts.
    cfg 4: M=16384, N=2048 bf16, G=128, 64 hot pairs carry 42% of slots;
           map_kind "pair" (each hot pair in one bucket) or "roundrobin" (e mod 8).
    cfg 5: M=65536, N=7168 fp8 e4m3 + one fp32 scale per 128 elements, G=256,
           top-8 uniform, B=8; experts dequantise to bf16.
    """
    if cfg_id not in STANDARD_M:
        raise ValueError(f"unknown workload {cfg_id}")
    M = STANDARD_M[cfg_id] if M is None else int(M)
    rng = np.random.default_rng([SEED, cfg_id])
    meta: dict = {}
    if cfg_id in (1, 2, 3, 5):
        N, G, k, B = 7168, 256, 8, 8
        if cfg_id == 3:
            idx, perm = zipf_topk(rng, M, G, k)
            meta["zipf_perm"] = perm
        else:
            idx = uniform_topk(rng, M, G, k)
        ebkt = contiguous_buckets(G, B)
    else:
        N, G, k, B = 2048, 128, 8, 8
        idx, pairs = correlated_pair_topk(rng, M, G, k)
        meta["hot_pairs"] = pairs
        if map_kind == "pair":
            ebkt = pair_aware_buckets(pairs, G, B)
        elif map_kind == "roundrobin":
            ebkt = round_robin_buckets(G, B)
        else:
            raise ValueError(map_kind)
        meta["map_kind"] = map_kind
    w = softmax_weights(rng, M, k)
    dtype = "fp8" if cfg_id == 5 else "bf16"
    x = None
    xs = None
    if with_rows:
        if dtype == "fp8":
            x, xs = normal_fp8_rows(rng, M, N)
        else:
            x = normal_bf16_rows(rng, M, N)
    standin = {1: "identity", 2: "scale", 3: "identity", 4: "identity", 5: "dequant"}[cfg_id]
    name = WORKLOAD_NAMES[cfg_id] + (f"-{map_kind}" if cfg_id == 4 else "")
    return Workload(name=name, cfg_id=cfg_id, M=M, N=N, G=G, k=k, B=B, dtype=dtype,
                    topk_idx=idx, expert_bucket=ebkt, weights=w, x=x, x_scale=xs,
                    standin=standin, dedup=(cfg_id in (2, 4)), meta=meta)


def make_custom(M: int, N: int, G: int, k: int, B: int, dtype: str = "bf16",
                routing: str = "uniform", seed: int = 0, standin: str = "identity",
                bucket_map: str = "contiguous") -> Workload:
    """Small workloads for edge cases: any shape, uniform distinct / with-repeats /
    single-expert / random routing, contiguous or random bucket maps."""
    rng = np.random.default_rng([SEED, 100, seed])
    if routing == "uniform":
        idx = uniform_topk(rng, M, G, k)
    elif routing == "repeats":          # ids drawn with replacement: duplicates allowed
        idx = rng.integers(0, G, size=(M, k), dtype=np.int32)
    elif routing == "one_expert":       # every slot to the same expert
        idx = np.full((M, k), G - 1, dtype=np.int32)
    else:
        raise ValueError(routing)
    if bucket_map == "contiguous" and G % B == 0:
        ebkt = contiguous_buckets(G, B)
    elif bucket_map in ("contiguous", "random"):
        ebkt = rng.integers(0, B, size=G, dtype=np.int32)
    elif bucket_map == "roundrobin":
        ebkt = round_robin_buckets(G, B)
    else:
        raise ValueError(bucket_map)
    w = softmax_weights(rng, M, k)
    if dtype == "fp8" and N % FP8_BLOCK == 0:
        x, xs = normal_fp8_rows(rng, M, N)
    elif dtype == "fp8":                # no whole 128-blocks: raw codes, no scales
        x, xs = rng.integers(0, 256, size=(M, N), dtype=np.uint8), None
    else:
        x, xs = normal_bf16_rows(rng, M, N), None
    return Workload(name=f"custom-M{M}-N{N}-G{G}-k{k}-B{B}-{routing}", cfg_id=0, M=M, N=N,
                    G=G, k=k, B=B, dtype=dtype, topk_idx=idx, expert_bucket=ebkt,
                    weights=w, x=x, x_scale=xs, standin=standin, dedup=False)
