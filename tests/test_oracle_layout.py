"""Pins for the layout oracle.

* A third formulation, written here from the definition as a sort of explicit
  (bucket, expert, token, position) tuples, must agree with both oracle
  formulations (array form and counting loops) exhaustively on tiny inputs and on
  random draws.
* Invariants of any correct layout, on the five standard workloads.
* Closed-form dedup statistics.
"""
import itertools
from math import comb

import numpy as np
import pytest

from combine_dispatch_layout_amd import workloads as wl
from oracle.layout import dispatch_layout, dispatch_layout_loops


def tuple_sort_layout(idx, ebkt, B, dedup):
    """Positions in the sorted list of (bucket, expert, token, j) are the slots;
    sorted distinct (bucket, token) pairs are the dedup send rows."""
    idx = [list(map(int, r)) for r in idx]
    ebkt = list(map(int, ebkt))
    M, k, G = len(idx), len(idx[0]), len(ebkt)
    entries = sorted((ebkt[e], e, t, j) for t in range(M) for j, e in enumerate(idx[t]))
    slot = np.zeros((M, k), dtype=np.int64)
    for p, (_, _, t, j) in enumerate(entries):
        slot[t, j] = p
    count = np.array([sum(1 for en in entries if en[1] == e) for e in range(G)])
    # an expert's offset = number of entries whose (bucket, expert) sorts before it
    offset = np.array([sum(1 for en in entries if (en[0], en[1]) < (ebkt[e], e))
                       for e in range(G)])
    if not dedup:
        bcount = np.array([sum(1 for en in entries if en[0] == b) for b in range(B)])
        send_row = slot.copy()
        send_token = np.zeros(M * k, dtype=np.int64)
        for (_, _, t, j), p in zip(entries, range(len(entries))):
            send_token[p] = t
    else:
        pairs = sorted(set((ebkt[e], t) for t in range(M) for e in idx[t]))
        pos = {pr: r for r, pr in enumerate(pairs)}
        bcount = np.array([sum(1 for pr in pairs if pr[0] == b) for b in range(B)])
        send_row = np.array([[pos[(ebkt[e], t)] for e in idx[t]] for t in range(M)])
        send_token = np.array([t for (_, t) in pairs], dtype=np.int64)
    boff = np.concatenate(([0], np.cumsum(bcount)))
    return dict(expert_count=count, expert_offset=offset, bucket_count=bcount,
                bucket_offset=boff, slot=slot, send_row=send_row, send_token=send_token)


FIELDS = ["expert_count", "expert_offset", "bucket_count", "bucket_offset",
          "slot", "send_row", "send_token"]


def assert_same(lay, ref, ctx):
    assert lay.status == 0, ctx
    for f in FIELDS:
        a = np.asarray(getattr(lay, f)) if not isinstance(lay, dict) else lay[f]
        b = np.asarray(ref[f])
        assert a.shape == b.shape and np.array_equal(a, b), (ctx, f, a, b)


def as_dict(lay):
    return {f: getattr(lay, f) for f in FIELDS}


@pytest.mark.parametrize("M,k,G,B", [(1, 1, 1, 1), (2, 2, 3, 2), (3, 2, 3, 2), (2, 3, 2, 2),
                                     (1, 2, 4, 3)])
def test_exhaustive_tiny(M, k, G, B):
    n = 0
    for flat in itertools.product(range(G), repeat=M * k):
        idx = np.array(flat, dtype=np.int32).reshape(M, k)
        for emap in itertools.product(range(B), repeat=G):
            ebkt = np.array(emap, dtype=np.int32)
            for dedup in (False, True):
                ref = tuple_sort_layout(idx, ebkt, B, dedup)
                a = dispatch_layout(idx, ebkt, B, dedup)
                b = dispatch_layout_loops(idx, ebkt, B, dedup)
                assert_same(a, ref, (flat, emap, dedup))
                assert_same(b, as_dict(a), (flat, emap, dedup))
                n += 1
    assert n > 0


@pytest.mark.parametrize("seed", range(12))
def test_random_small(seed):
    rng = np.random.default_rng(seed)
    M = int(rng.integers(1, 70))
    G = int(rng.integers(1, 40))
    k = int(rng.integers(1, min(G, 9) + 1))
    B = int(rng.integers(1, 9))
    idx = rng.integers(0, G, size=(M, k)).astype(np.int32)     # repeats allowed
    ebkt = rng.integers(0, B, size=G).astype(np.int32)
    for dedup in (False, True):
        ref = tuple_sort_layout(idx, ebkt, B, dedup)
        assert_same(dispatch_layout(idx, ebkt, B, dedup), ref, seed)
        assert_same(dispatch_layout_loops(idx, ebkt, B, dedup), ref, seed)


def test_invalid_expert_status():
    idx = np.array([[0, 1], [2, 7], [-1, 0]], dtype=np.int32)
    ebkt = np.zeros(4, dtype=np.int32)
    for f in (dispatch_layout, dispatch_layout_loops):
        assert f(idx, ebkt, 1, False).status == 4      # flat index 3 is the first bad
    idx[1, 1] = 3
    assert dispatch_layout(idx, ebkt, 1, True).status == 5
    # a bucket outside [0, B) is reported first, as -(expert + 1)
    ebkt[2] = 1
    for f in (dispatch_layout, dispatch_layout_loops):
        assert f(idx, ebkt, 1, False).status == -3


def check_invariants(w, lay, dedup):
    M, k, G, B = w.M, w.k, w.G, w.B
    idx = w.topk_idx
    ebkt = w.expert_bucket
    assert lay.status == 0
    # I1: counts sum to M*k
    assert lay.expert_count.sum() == M * k
    # I2: slot is a bijection of [0, M*k)
    assert np.array_equal(np.sort(lay.slot.reshape(-1)), np.arange(M * k))
    # expert runs: every slot of expert e lies in [offset, offset + count)
    e_flat = idx.reshape(-1)
    s_flat = lay.slot.reshape(-1)
    assert np.all(s_flat >= lay.expert_offset[e_flat])
    assert np.all(s_flat < lay.expert_offset[e_flat] + lay.expert_count[e_flat])
    # I3: token strictly increases inside each run (distinct top-k)
    tok_of_slot = np.empty(M * k, dtype=np.int64)
    tok_of_slot[s_flat] = np.repeat(np.arange(M), k)
    for e in range(G):
        o, c = lay.expert_offset[e], lay.expert_count[e]
        assert np.all(np.diff(tok_of_slot[o:o + c]) > 0)
    if not dedup:
        # I4: bucket b's experts tile [bucket_offset[b], bucket_offset[b+1])
        for b in range(B):
            es = np.flatnonzero(ebkt == b)
            lo, hi = lay.bucket_offset[b], lay.bucket_offset[b + 1]
            assert lay.expert_count[es].sum() == hi - lo
            if es.size:
                assert lay.expert_offset[es].min() == lo
        assert np.array_equal(lay.send_row, lay.slot)
    else:
        # I5: dedup rows = distinct (t, b), each once, ascending t inside each bucket
        pairs = {(t, int(ebkt[e])) for t in range(M) for e in idx[t]}
        assert lay.R == len(pairs)
        seen = set()
        for b in range(B):
            lo, hi = lay.bucket_offset[b], lay.bucket_offset[b + 1]
            toks = lay.send_token[lo:hi]
            assert np.all(np.diff(toks) > 0)
            seen |= {(int(t), b) for t in toks}
        assert seen == pairs
        # I6: U_b <= M, sum <= M*min(k, B)
        assert np.all(lay.bucket_count <= M) and lay.R <= M * min(k, B)
        # every (t, j) points at a row holding its own token and its expert's bucket
        r = lay.send_row.reshape(-1)
        assert np.array_equal(lay.send_token[r], np.repeat(np.arange(M), k))
        b_of_row = np.searchsorted(lay.bucket_offset, r, side="right") - 1
        assert np.array_equal(b_of_row, ebkt[e_flat])
    assert np.array_equal(lay.bucket_offset, np.concatenate(([0], np.cumsum(lay.bucket_count))))


@pytest.mark.parametrize("cfg,M", [(1, None), (2, None), (3, 4096), (4, 4096), (5, 4096)])
@pytest.mark.parametrize("dedup", [False, True])
def test_invariants_standard_workloads(cfg, M, dedup):
    w = wl.make_workload(cfg, M=M, with_rows=False)
    lay = dispatch_layout(w.topk_idx, w.expert_bucket, w.B, dedup)
    check_invariants(w, lay, dedup)


def test_loops_agree_on_standard_workload():
    w = wl.make_workload(2, M=512, with_rows=False)
    for dedup in (False, True):
        a = dispatch_layout(w.topk_idx, w.expert_bucket, w.B, dedup)
        b = dispatch_layout_loops(w.topk_idx, w.expert_bucket, w.B, dedup)
        assert_same(b, as_dict(a), dedup)


def test_uniform_dedup_rows_closed_form():
    """Uniform distinct top-8 of 256 experts in 8 buckets of 32: the expected number of
    distinct buckets per token is 8 * (1 - C(224, 8) / C(256, 8)) = 5.2947."""
    expect = 8 * (1 - comb(224, 8) / comb(256, 8))
    assert abs(expect - 5.2947) < 1e-4
    w = wl.make_workload(2, with_rows=False)
    lay = dispatch_layout(w.topk_idx, w.expert_bucket, w.B, True)
    per_token = lay.R / w.M
    # std of the per-token count is < 1, so the mean over 4096 tokens is within 0.05
    assert abs(per_token - expect) < 0.05, per_token
