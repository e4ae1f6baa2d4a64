"""GPU parity of the dedup round trip around the path: layout (dedup) -> dispatch ->
moe_expand -> expert stand-in -> moe_combine_partial -> moe_combine_reduce, against
the oracle step by step (expanded rows, partial rows and outputs bit for bit)."""
import numpy as np
import pytest
import torch

import oracle
from combine_dispatch_layout_amd import harness, moedl
from combine_dispatch_layout_amd import workloads as wl
from gpu_util import (as_u16, assert_bits_equal, assert_layout_equal, dev, gpu_dispatch,
                      gpu_layout, host, say)

pytestmark = pytest.mark.gpu


def run_both(w):
    ref = oracle.dispatch_layout(w.topk_idx, w.expert_bucket, w.B, True)
    sent, sent_scale = oracle.dispatch(w.x, ref.send_row, ref.R, w.x_scale)
    ein_ref, ein_scale_ref = oracle.expand(sent, ref.send_row, ref.slot, w.M * w.k, sent_scale)
    eo_ref = oracle.expert_outputs(w.standin, ein_ref, ref.slot, ref.slot, w.topk_idx,
                                   ein_scale_ref)
    part_ref = oracle.combine_partial(eo_ref, w.weights, ref.slot, ref.send_row, ref.R)
    y_ref = oracle.combine_reduce(part_ref, ref.send_row)

    lay = gpu_layout(w, True)
    out, out_scale = gpu_dispatch(w, lay)
    ein, ein_scale = moedl.moe_expand(out, lay.send_row, lay.slot, w.M * w.k, out_scale)
    eo = harness.expert_outputs(w.standin, ein, lay.slot, lay.slot, dev(w.topk_idx), ein_scale)
    part = moedl.moe_combine_partial(eo, dev(w.weights), lay.slot, lay.send_row, lay.capacity)
    y = moedl.moe_combine_reduce(part, lay.send_row)
    torch.cuda.synchronize()
    return ref, (ein_ref, ein_scale_ref, part_ref, y_ref), lay, (ein, ein_scale, part, y)


def check(w, ctx):
    ref, (ein_ref, eins_ref, part_ref, y_ref), lay, (ein, eins, part, y) = run_both(w)
    assert_layout_equal(lay, ref, ctx)
    got = host(ein)
    assert np.array_equal(as_u16(got) if w.dtype == "bf16" else got, ein_ref), ctx + " expand"
    if eins_ref is not None:
        assert np.array_equal(host(eins), eins_ref), ctx + " expand scales"
    assert_bits_equal(host(part[:ref.R]), part_ref, ctx + " partial")
    assert_bits_equal(host(y), y_ref, ctx + " reduce")


@pytest.mark.parametrize("cfg,M,map_kind", [(1, None, "pair"), (2, 1000, "pair"),
                                            (3, 1000, "pair"), (4, 1000, "pair"),
                                            (4, 1000, "roundrobin"), (5, 300, "pair")])
def test_round_trip_reduced(gpu_lib, cfg, M, map_kind):
    w = wl.make_workload(cfg, M=M, map_kind=map_kind)
    say(f"bucket round trip {w.name} M={w.M}")
    check(w, w.name)


@pytest.mark.parametrize("cfg,map_kind", [(2, "pair"), (4, "pair"), (4, "roundrobin")])
def test_round_trip_full_size(gpu_lib, cfg, map_kind):
    w = wl.make_workload(cfg, map_kind=map_kind)
    say(f"bucket round trip full {w.name}")
    check(w, w.name)


EDGE = [  # (M, N, G, k, B, routing, bucket_map)
    (1, 7168, 256, 8, 8, "uniform", "contiguous"),
    (300, 64, 16, 1, 4, "uniform", "contiguous"),          # k = 1
    (300, 128, 16, 4, 1, "uniform", "contiguous"),          # one bucket
    (513, 136, 37, 5, 3, "repeats", "random"),              # duplicate ids
    (700, 1024, 1024, 16, 64, "uniform", "random"),         # maximum G, k, B
    (257, 64, 12, 3, 12, "uniform", "roundrobin"),
]


@pytest.mark.parametrize("case", EDGE, ids=[f"M{c[0]}-N{c[1]}-G{c[2]}-k{c[3]}-B{c[4]}-{c[5]}"
                                            for c in EDGE])
def test_round_trip_edges(gpu_lib, case):
    M, N, G, k, B, routing, bmap = case
    w = wl.make_custom(M, N, G, k, B, routing=routing, bucket_map=bmap, seed=M + 7)
    w.standin = "scale"
    say(f"bucket round trip {w.name}")
    check(w, w.name)


def test_single_bucket_matches_flat_combine(gpu_lib):
    """B = 1: partial + reduce reproduce the flat combine bit for bit on the GPU too."""
    w = wl.make_custom(600, 512, 64, 8, 1, routing="uniform", seed=5)
    w.standin = "scale"
    ref, _, lay, (ein, eins, part, y) = run_both(w)
    eo = harness.expert_outputs("scale", ein, lay.slot, lay.slot, dev(w.topk_idx))
    y_flat = moedl.moe_combine(eo, dev(w.weights), lay.slot)
    torch.cuda.synchronize()
    assert torch.equal(y, y_flat)


def _random_cases(n=12, seed=20261204):
    """Seeded random shapes for the round trip (bf16 rows, scaled-expert stand-in), across
    layout paths, repeats and all bucket maps; small enough for the oracle."""
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        G = int(rng.choice([1, 3, 16, 64, 256, 1000]))
        k = int(rng.integers(1, min(16, G) + 1))
        B = int(rng.integers(1, 65))
        M = int(np.exp(rng.uniform(0, np.log(20000 // k))))
        N = int(rng.integers(1, 1024 // 8 + 1)) * 8
        if M * k * N * 2 > (24 << 20):
            continue
        routing = "repeats" if rng.random() < 0.3 else "uniform"
        bmap = str(rng.choice(["contiguous", "random", "roundrobin"]))
        cases.append((M, N, G, k, B, routing, bmap))
    return cases


RANDOM = _random_cases()


@pytest.mark.parametrize("case", RANDOM, ids=[f"M{c[0]}-N{c[1]}-G{c[2]}-k{c[3]}-B{c[4]}-{c[5]}-{c[6]}"
                                              for c in RANDOM])
def test_round_trip_random(gpu_lib, case):
    M, N, G, k, B, routing, bmap = case
    w = wl.make_custom(M, N, G, k, B, routing=routing, bucket_map=bmap, seed=M + N + 11)
    w.standin = "scale"
    say(f"bucket round trip {w.name} map={bmap}")
    check(w, f"{w.name} map={bmap}")
