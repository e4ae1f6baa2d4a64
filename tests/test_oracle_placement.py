"""Pins for the placement oracle.

* pair counts against brute-force set counting (repeats allowed); symmetry; the
  diagonal is the per-expert token count; the off-diagonal sum is exactly
  sum_t |S_t| (|S_t| - 1), so for k distinct experts per token the off-diagonal mean
  is exactly M k (k-1) / (G (G-1)).
* greedy placement: balanced buckets; a block-structured count matrix (intra-block
  counts above all inter-block ones) is recovered exactly; cluster partitions are
  equivariant under relabeling experts (tie-free counts); the 64 hot pairs of the
  correlated-pair workload stay together and the realised dedup saving beats
  round-robin; hand-worked maps fix the tie order of the pair visits, the cluster
  order and the bucket numbering (steps 2-5), and planted mistakes in each (ties by
  (b, a), highest bucket first, clusters by smallest member) fail a pin.
"""
import itertools

import numpy as np
import pytest

from combine_dispatch_layout_amd import workloads as wl
from oracle import dispatch_layout
from oracle.placement import greedy_clusters, greedy_place, pair_counts


@pytest.mark.parametrize("seed", range(5))
def test_pair_counts_brute_force(seed):
    rng = np.random.default_rng(seed)
    M, k, G = int(rng.integers(1, 40)), int(rng.integers(1, 6)), int(rng.integers(2, 12))
    idx = rng.integers(-1, G + 1, size=(M, k))      # repeats and out-of-range ids
    C = pair_counts(idx, G)
    for a, b in itertools.product(range(G), repeat=2):
        want = sum(1 for t in range(M) if a in set(idx[t]) and b in set(idx[t]))
        assert C[a, b] == want


def test_pair_count_identities():
    w = wl.make_workload(2, with_rows=False)
    C = pair_counts(w.topk_idx, w.G)
    assert np.array_equal(C, C.T)
    assert np.array_equal(np.diag(C), np.bincount(w.topk_idx.reshape(-1), minlength=w.G))
    off = C.sum() - np.trace(C)
    assert off == w.M * w.k * (w.k - 1)
    assert abs(off / (w.G * (w.G - 1)) - w.M * w.k * (w.k - 1) / (w.G * (w.G - 1))) == 0


@pytest.mark.parametrize("G,B", [(8, 2), (12, 3), (64, 8), (128, 8)])
def test_balanced(G, B):
    rng = np.random.default_rng(G)
    idx = np.argsort(rng.random((500, G)), axis=1)[:, :min(8, G // 2)]
    m = greedy_place(pair_counts(idx, G), B)
    assert np.all(np.bincount(m, minlength=B) == G // B)


def _block_matrix(G, B, seed):
    rng = np.random.default_rng(seed)
    groups = rng.permutation(G).reshape(B, G // B)
    C = rng.integers(1, 50, size=(G, G))
    for g in groups:
        C[np.ix_(g, g)] = rng.integers(100, 200, size=(len(g), len(g)))
    C = np.triu(C, 1)
    return C + C.T, groups


@pytest.mark.parametrize("seed", range(4))
def test_block_structure_recovered(seed):
    C, groups = _block_matrix(32, 4, seed)
    m = greedy_place(C, 4)
    for g in groups:
        assert len(set(m[g].tolist())) == 1
    assert len({int(m[g[0]]) for g in groups}) == 4


def _tie_free(G, seed):
    rng = np.random.default_rng(seed)
    vals = rng.permutation(G * (G - 1) // 2) + 1
    C = np.zeros((G, G), dtype=np.int64)
    C[np.triu_indices(G, 1)] = vals
    return C + C.T


@pytest.mark.parametrize("seed", range(4))
def test_clusters_equivariant_under_relabeling(seed):
    G, cap = 24, 6
    C = _tie_free(G, seed)
    perm = np.random.default_rng(100 + seed).permutation(G)    # new label of expert e
    Cp = np.empty_like(C)
    Cp[np.ix_(perm, perm)] = C
    a = {frozenset(m) for m in greedy_clusters(C, cap)}
    inv = np.argsort(perm)
    b = {frozenset(int(inv[e]) for e in m) for m in greedy_clusters(Cp, cap)}
    assert a == b


def _saving(w, ebkt):
    lay = dispatch_layout(w.topk_idx, ebkt, w.B, True)
    return 1 - lay.R / (w.M * w.k)


def test_hot_pairs_and_savings():
    w = wl.make_workload(4, M=8192, with_rows=False)
    pairs = w.meta["hot_pairs"]
    m = greedy_place(pair_counts(w.topk_idx, w.G), w.B)
    assert np.all(m[pairs[:, 0]] == m[pairs[:, 1]])
    s_greedy = _saving(w, m)
    s_rr = _saving(w, wl.round_robin_buckets(w.G, w.B))
    s_pair = _saving(w, wl.pair_aware_buckets(pairs, w.G, w.B))
    assert s_greedy > s_rr + 0.05
    assert s_greedy >= s_pair - 0.01


def test_planted_mistakes_fail_a_pin():
    C, groups = _block_matrix(32, 4, 0)

    def ascending(C, B):                   # visit pairs by count ascending
        return greedy_place(C.max() + 1 - np.where(C > 0, C, C.max() + 1), B)

    m = ascending(C, 4)
    assert not all(len(set(m[g].tolist())) == 1 for g in groups)


# ---- hand-worked maps: the tie order of step 2 and the bucket numbering of steps 4-5
#
# Each expected map below was derived by hand from the five steps, written out in the
# comment, and not by running the oracle.

def _sym(G, counts):
    C = np.zeros((G, G), dtype=np.int64)
    for (a, b), c in counts.items():
        C[a, b] = C[b, a] = c
    return C


# G=6, B=2 (cap 3).  C[3,4]=10 merges {3,4}.  C[0,4] and C[1,3] tie at 5; visiting
# (a, b) ascending takes (0,4) first: {0,3,4}, and (1,3) would make 4 > 3, so it is
# skipped.  Clusters by size, then smallest member: [0,3,4], [1], [2], [5].  [0,3,4]
# takes bucket 0 (full), the singletons fill bucket 1.  Visiting ties by (b, a) would
# take (1,3) first and give [1,3,4] in bucket 0 instead.
TIE_CASE = (_sym(6, {(3, 4): 10, (0, 4): 5, (1, 3): 5}), 2,
            [[0, 3, 4], [1], [2], [5]], [0, 1, 1, 0, 0, 1])

# G=8, B=2 (cap 4).  Merges {0,1} (count 3), {2,3} (2), then (3,4) makes {2,3,4}.
# Order: [2,3,4] (size 3), [0,1], [5], [6], [7].  [2,3,4] -> bucket 0; [0,1] does not
# fit there (3+2 > 4) -> bucket 1; [5] -> bucket 0 (now full); [6], [7] -> bucket 1.
SIZE_CASE = (_sym(8, {(0, 1): 3, (2, 3): 2, (3, 4): 1}), 2,
             [[2, 3, 4], [0, 1], [5], [6], [7]], [1, 1, 0, 0, 0, 0, 1, 1])

# G=6, B=2 (cap 3).  Three pair clusters [0,1], [2,3], [4,5].  [0,1] -> bucket 0,
# [2,3] -> bucket 1 (bucket 0 would hold 4), [4,5] fits nowhere and waits.  Step 5:
# expert 4 takes the lowest bucket with a free place (0), then 5 takes bucket 1.
WAIT_CASE = (_sym(6, {(0, 1): 3, (2, 3): 2, (4, 5): 1}), 2,
             [[0, 1], [2, 3], [4, 5]], [0, 0, 1, 1, 0, 1])

HAND_CASES = {"tie": TIE_CASE, "size": SIZE_CASE, "wait": WAIT_CASE}


def _hand_pins_hold():
    for C, B, clusters, m in HAND_CASES.values():
        cap = C.shape[0] // B
        if greedy_clusters(C, cap) != clusters:
            return False
        if greedy_place(C, B).tolist() != m:
            return False
    return True


@pytest.mark.parametrize("case", sorted(HAND_CASES))
def test_hand_worked_maps(case):
    C, B, clusters, m = HAND_CASES[case]
    assert greedy_clusters(C, C.shape[0] // B) == clusters
    assert greedy_place(C, B).tolist() == m


def test_hand_worked_maps_are_tie_sensitive():
    """The tie case really is one: under the (b, a) order its clusters differ, so the
    pin above decides between the two orders."""
    C = TIE_CASE[0]
    a_idx, b_idx = np.triu_indices(6, k=1)
    cnt = C[a_idx, b_idx]
    keep = cnt > 0
    a_idx, b_idx, cnt = a_idx[keep], b_idx[keep], cnt[keep]
    ab = [(int(a_idx[p]), int(b_idx[p])) for p in np.lexsort((b_idx, a_idx, -cnt))]
    ba = [(int(a_idx[p]), int(b_idx[p])) for p in np.lexsort((a_idx, b_idx, -cnt))]
    assert ab[:3] == [(3, 4), (0, 4), (1, 3)]
    assert ba[:3] == [(3, 4), (1, 3), (0, 4)]


def _mutant_ties_ba(a_idx, b_idx, cnt):
    return np.lexsort((a_idx, b_idx, -cnt))         # ties by (b, a)


def _mutant_highest_bucket(B):
    return range(B - 1, -1, -1)                     # highest-numbered bucket first


@pytest.mark.parametrize("name,mutant", [("_visit_order", _mutant_ties_ba),
                                         ("_bucket_order", _mutant_highest_bucket)])
def test_planted_tie_and_bucket_mistakes_fail_a_pin(monkeypatch, name, mutant):
    import oracle.placement as pl
    assert _hand_pins_hold()
    monkeypatch.setattr(pl, name, mutant)
    assert not _hand_pins_hold()


def test_planted_cluster_order_mistake_fails_a_pin(monkeypatch):
    """Step 3 taken as smallest member first (size ignored) changes the size case."""
    import oracle.placement as pl
    real = pl.greedy_clusters

    def by_member(C, cap):
        return sorted(real(C, cap), key=lambda m: m[0])

    monkeypatch.setattr(pl, "greedy_clusters", by_member)
    C, B, _, m = SIZE_CASE
    assert pl.greedy_place(C, B).tolist() != m
