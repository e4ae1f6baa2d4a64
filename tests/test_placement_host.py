"""The host greedy placement in libmoedl (moe_place_experts, host code, no GPU)
against the oracle: identical maps on tie-free, tie-heavy, block-structured and
workload-derived count matrices, plus argument errors."""
import numpy as np
import pytest

from combine_dispatch_layout_amd import moedl
from combine_dispatch_layout_amd import workloads as wl
from oracle.placement import greedy_place, pair_counts


def both(C, B):
    return moedl.moe_place_experts(np.asarray(C, dtype=np.int32), B), greedy_place(C, B)


@pytest.mark.parametrize("G,B,seed", [(8, 2, 0), (12, 3, 1), (64, 8, 2), (128, 8, 3),
                                      (256, 8, 4), (1024, 64, 5), (30, 5, 6)])
def test_random_counts(G, B, seed):
    rng = np.random.default_rng(seed)
    C = rng.integers(0, 6, size=(G, G))          # many ties
    C = np.triu(C, 1)
    C = C + C.T
    a, b = both(C, B)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("cfg,map_kind", [(4, "pair"), (3, "pair"), (2, "pair")])
def test_workload_counts(cfg, map_kind):
    w = wl.make_workload(cfg, M=4096, with_rows=False)
    C = pair_counts(w.topk_idx, w.G)
    a, b = both(C, w.B)
    assert np.array_equal(a, b)


def test_fragmented_packing_path():
    # clusters of 3 with capacity 4 cannot all be placed whole: step 4 is used
    G, B = 12, 3
    C = np.zeros((G, G), dtype=np.int64)
    for g in range(4):
        for i in range(3):
            for j in range(3):
                if i != j:
                    C[3 * g + i, 3 * g + j] = 10 + g
    a, b = both(C, B)
    assert np.array_equal(a, b)
    assert np.all(np.bincount(a, minlength=B) == 4)


def test_errors():
    lib = moedl.load()
    C = np.zeros((12, 12), dtype=np.int32)
    out = np.zeros(12, dtype=np.int32)
    assert lib.moe_place_experts(C.ctypes.data, 12, 5, out.ctypes.data) == 1
    assert lib.moe_place_experts(None, 12, 3, out.ctypes.data) == 1
    assert lib.moe_place_experts(C.ctypes.data, 12, 65, out.ctypes.data) == 2
    assert lib.moe_expert_pair_counts(1 << 20, 10, 8, 2048, 1 << 20, None) == 2
    assert lib.moe_expert_pair_counts(1 << 20, -1, 8, 64, 1 << 20, None) == 1
    assert lib.moe_expert_pair_counts(1 << 20, 10, 8, 64, None, None) == 1


def test_hand_worked_maps():
    """The host greedy gives the hand-derived maps that pin the oracle's tie order,
    cluster order and bucket numbering."""
    from test_oracle_placement import HAND_CASES
    for C, B, _, m in HAND_CASES.values():
        got = moedl.moe_place_experts(np.asarray(C, dtype=np.int32), B)
        assert got.tolist() == m
