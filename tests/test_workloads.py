"""Generator checks: shapes, seeding, statistics against closed forms or an
independent sampler, page constants, and the row codecs against the oracle's own."""
import json
import os
from math import comb

import numpy as np
import pytest

from combine_dispatch_layout_amd import workloads as wl
from oracle import f32_to_bf16_rne, f32_to_e4m3_rne_sat, e4m3_to_f32

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_constants.json")


def golden():
    with open(GOLDEN) as f:
        return {k: v["value"] for k, v in json.load(f).items() if not k.startswith("_")}


def test_page_constants_fix_the_workloads():
    g = golden()
    w = wl.make_workload(1, with_rows=False)
    assert (w.N, w.G, w.k) == (g["hidden_N"], g["experts_G"], g["topk"])
    # 8,128 possible pairs is C(128, 2): the pair workload has 128 experts
    assert comb(128, 2) == g["possible_expert_pairs"]
    w4 = wl.make_workload(4, M=64, with_rows=False)
    assert w4.G == 128 and wl.N_HOT_PAIRS == g["hot_pairs"]
    assert wl.HOT_PAIR_FRACTION == g["hot_pair_token_share"]
    assert w4.B == g["gpus_in_placement_study"]
    assert g["graph_invocations"] * g["timed_replays"] == g["latency_divisor"]


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_shapes_ranges_and_seeding(cfg):
    w = wl.make_workload(cfg, M=128)
    assert w.topk_idx.shape == (128, w.k) and w.topk_idx.dtype == np.int32
    assert w.topk_idx.min() >= 0 and w.topk_idx.max() < w.G
    # distinct experts within each token
    assert all(len(set(r)) == w.k for r in w.topk_idx.tolist())
    assert w.expert_bucket.shape == (w.G,) and w.expert_bucket.max() < w.B
    assert np.allclose(w.weights.sum(axis=1), 1.0, atol=1e-6) and np.all(w.weights > 0)
    if w.dtype == "fp8":
        assert w.x.dtype == np.uint8 and w.x_scale.shape == (128, w.N // 128)
    else:
        assert w.x.dtype == np.uint16 and w.x_scale is None
    w2 = wl.make_workload(cfg, M=128)
    assert np.array_equal(w.topk_idx, w2.topk_idx) and np.array_equal(w.x, w2.x)


def test_bf16_rows_match_oracle_codec():
    rng = np.random.default_rng([wl.SEED, 77])
    v = rng.standard_normal((64, 512), dtype=np.float32)
    assert np.array_equal(wl.bf16_bits_from_f32(v), f32_to_bf16_rne(v))


def test_fp8_rows_match_oracle_codec():
    rng = np.random.default_rng([wl.SEED, 78])
    v = rng.standard_normal((32, 1024), dtype=np.float32)
    v[3, :128] = 0.0                                     # an all-zero block: scale 1
    codes, scale = wl.fp8_quantise_blocks(v)
    blk = v.reshape(32, 8, 128)
    amax = np.abs(blk).max(axis=2)
    assert np.array_equal(scale, np.where(amax > 0, amax / np.float32(448), 1).astype(np.float32))
    q = (blk / scale[:, :, None]).astype(np.float32)
    assert np.array_equal(codes, f32_to_e4m3_rne_sat(q).reshape(32, 1024))
    # every block's largest magnitude maps to +-448
    deq = np.abs(e4m3_to_f32(codes).reshape(32, 8, 128)).max(axis=2)
    assert np.all(deq[amax > 0] == 448.0)


def test_uniform_routing_is_uniform():
    w = wl.make_workload(2, with_rows=False)
    counts = np.bincount(w.topk_idx.reshape(-1), minlength=w.G)
    mean = w.M * w.k / w.G
    # chi-square with 255 degrees of freedom: far below 400 unless badly non-uniform
    assert ((counts - mean) ** 2 / mean).sum() < 400


def test_zipf_matches_sequential_sampler():
    """Gumbel-top-k equals successive renormalised draws: compare the frequency with
    which the rank-0 and rank-1 experts are selected against a direct sequential
    sampler (an independent algorithm)."""
    G, k, M = 256, 8, 4000
    rng = np.random.default_rng(5)
    idx, perm = wl.zipf_topk(rng, M, G, k)
    p = (np.arange(1, G + 1, dtype=np.float64)) ** -wl.ZIPF_S
    rng2 = np.random.default_rng(6)
    seq_hits = np.zeros(2)
    for _ in range(M):
        avail = np.ones(G, bool)
        for _ in range(k):
            q = np.where(avail, p, 0)
            r = rng2.choice(G, p=q / q.sum())
            avail[r] = False
        seq_hits += ~avail[:2]
    gum_hits = np.array([(idx == perm[0]).any(axis=1).sum(), (idx == perm[1]).any(axis=1).sum()])
    # binomial std of a frequency over 4000 tokens is < 0.008
    assert np.all(np.abs(gum_hits / M - seq_hits / M) < 0.04), (gum_hits / M, seq_hits / M)
    assert gum_hits[0] / M > 0.85                      # heavily skewed toward rank 0


def test_correlated_pairs_share():
    w = wl.make_workload(4, M=8192, with_rows=False)
    pairs = w.meta["hot_pairs"]
    partner = np.full(w.G, -1)
    partner[pairs[:, 0]] = pairs[:, 1]
    partner[pairs[:, 1]] = pairs[:, 0]
    hot = 0
    for row in w.topk_idx.tolist():
        s = set(row)
        hot += sum(1 for e in row if partner[e] in s)
    share = hot / w.topk_idx.size
    # 42% of slots in hot pairs by construction, plus a little from random fills
    assert 0.40 < share < 0.47, share
    # pair-aware map keeps every hot pair in one bucket; round-robin splits most
    assert np.all(w.expert_bucket[pairs[:, 0]] == w.expert_bucket[pairs[:, 1]])
    rr = wl.round_robin_buckets(w.G, w.B)
    assert np.mean(rr[pairs[:, 0]] == rr[pairs[:, 1]]) < 0.5
    assert np.all(np.bincount(w.expert_bucket, minlength=w.B) == w.G // w.B)
