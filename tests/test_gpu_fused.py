"""GPU parity of moe_layout_dispatch (layout and row scatter in one launch, M <= 512)
against the oracle: every layout array, the status word and every send row bit for
bit, rows past the send count untouched; and identical bytes to the two-call path."""
import numpy as np
import pytest
import torch

import oracle
from combine_dispatch_layout_amd import moedl
from combine_dispatch_layout_amd import workloads as wl
from gpu_util import (SENTINEL_BF16, SENTINEL_FP8, assert_dispatch_equal, assert_layout_equal,
                      dev, gpu_dispatch, gpu_layout, host, rows_dev, say)

pytestmark = pytest.mark.gpu


def fused(w, dedup):
    x = rows_dev(w)
    lay = moedl.alloc_layout(w.M, w.k, w.G, w.B, dedup)
    out = torch.empty((lay.capacity, w.N), dtype=x.dtype, device="cuda")
    out.fill_(SENTINEL_BF16 if w.dtype == "bf16" else SENTINEL_FP8)
    xs = dev(w.x_scale) if w.x_scale is not None else None
    out_scale = None
    if xs is not None:
        out_scale = torch.full((lay.capacity, xs.shape[1]), float("nan"), dtype=torch.float32,
                               device="cuda")
    return moedl.moe_layout_dispatch(dev(w.topk_idx), dev(w.expert_bucket), w.B, dedup, x,
                                     x_scale=xs, lay=lay, out=out, out_scale=out_scale)


def check(w, dedup, ctx):
    say(ctx)
    ref = oracle.dispatch_layout(w.topk_idx, w.expert_bucket, w.B, dedup)
    lay, out, out_scale = fused(w, dedup)
    assert_layout_equal(lay, ref, ctx)
    if ref.status == 0:
        assert_dispatch_equal(w, out, out_scale, ref, ctx=ctx)
    return lay, out, out_scale


STANDARD = [(1, None), (2, 128), (3, 256), (3, 257), (3, 512), (4, 384), (5, 300)]


@pytest.mark.parametrize("cfg,M", STANDARD)
@pytest.mark.parametrize("dedup", [False, True])
def test_fused_standard_workloads(gpu_lib, cfg, M, dedup):
    w = wl.make_workload(cfg, M=M)
    check(w, dedup, f"fused {w.name} M={w.M} dedup={dedup}")


EDGE = [  # (M, N, G, k, B, dtype, routing, bucket_map)
    (1, 7168, 256, 8, 8, "bf16", "uniform", "contiguous"),
    (2, 8, 4, 1, 1, "bf16", "uniform", "contiguous"),           # one 16-byte vector rows
    (257, 64, 1, 1, 1, "bf16", "uniform", "contiguous"),         # G = 1, two tiles
    (300, 128, 16, 4, 4, "bf16", "one_expert", "contiguous"),    # all to one expert
    (511, 136, 37, 5, 3, "bf16", "repeats", "random"),           # duplicates, odd shapes
    (512, 1024, 1024, 16, 64, "bf16", "uniform", "random"),      # maximum M, G, k, B
    (333, 16, 64, 8, 8, "fp8", "uniform", "contiguous"),         # fp8, no scales
    (90, 12288, 64, 3, 4, "bf16", "uniform", "contiguous"),      # rows above 16 KiB
]


@pytest.mark.parametrize("case", EDGE, ids=[f"M{c[0]}-N{c[1]}-G{c[2]}-k{c[3]}-B{c[4]}-{c[5]}-{c[6]}"
                                            for c in EDGE])
@pytest.mark.parametrize("dedup", [False, True])
def test_fused_edge_shapes(gpu_lib, case, dedup):
    M, N, G, k, B, dtype, routing, bmap = case
    w = wl.make_custom(M, N, G, k, B, dtype=dtype, routing=routing, bucket_map=bmap, seed=M)
    if dtype == "fp8":
        w.x_scale = None
    check(w, dedup, f"fused {w.name} dedup={dedup}")


@pytest.mark.parametrize("dedup", [False, True])
def test_fused_matches_two_calls(gpu_lib, dedup):
    w = wl.make_workload(3, M=448)
    lay_f, out_f, _ = fused(w, dedup)
    lay = gpu_layout(w, dedup)
    out, _ = gpu_dispatch(w, lay)
    torch.cuda.synchronize()
    for f in ("expert_count", "expert_offset", "bucket_count", "bucket_offset", "slot",
              "send_row", "send_token", "status"):
        a, b = host(getattr(lay_f, f)), host(getattr(lay, f))
        if f == "send_token":
            R = int(host(lay.bucket_offset)[-1])
            a, b = a[:R], b[:R]
        assert np.array_equal(a, b), f
    assert torch.equal(out_f, out)


def test_fused_empty_batch(gpu_lib):
    idx = torch.empty((0, 8), dtype=torch.int32, device="cuda")
    ebkt = dev((np.arange(256) // 32).astype(np.int32))
    x = torch.empty((0, 7168), dtype=torch.int16, device="cuda")
    for dedup in (False, True):
        lay, out, _ = moedl.moe_layout_dispatch(idx, ebkt, 8, dedup, x)
        torch.cuda.synchronize()
        assert int(lay.status.item()) == 0
        assert int(lay.expert_count.abs().sum().item()) == 0
        assert int(lay.expert_offset.abs().sum().item()) == 0
        assert host(lay.bucket_offset).tolist() == [0] * 9
        assert out.shape == (0, 7168)


@pytest.mark.parametrize("dedup", [False, True])
def test_fused_bad_ids_and_map(gpu_lib, dedup):
    w = wl.make_custom(400, 64, 32, 4, 4, seed=3)
    idx = w.topk_idx.copy()
    idx[300, 2] = 32            # first bad entry: flat 1202
    idx[311, 0] = -5
    w.topk_idx = idx
    lay, _, _ = check(w, dedup, f"fused bad ids dedup={dedup}")
    assert int(lay.status.item()) == 300 * 4 + 2 + 1
    ebkt = w.expert_bucket.copy()
    ebkt[7] = 4
    w.expert_bucket = ebkt
    lay, _, _ = fused(w, dedup)
    torch.cuda.synchronize()
    assert int(lay.status.item()) == -8


def _random_fused_cases(n=20, seed=20261204):
    """Seeded random shapes within the one-launch path (M <= 512): one tile and two,
    both row dtypes (fp8 with scales when N is a multiple of 128), repeats, every
    bucket map, both modes."""
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        G = int(rng.choice([1, 2, 7, 32, 64, 256, 1000, 1024]))
        k = int(rng.integers(1, min(16, G) + 1))
        B = int(rng.integers(1, 65))
        M = int(rng.integers(1, moedl.FUSED_MAX_TOKENS + 1))
        dtype = "fp8" if rng.random() < 0.3 else "bf16"
        if dtype == "fp8":
            N = int(rng.integers(1, 17)) * 128 if rng.random() < 0.6 else int(rng.integers(1, 128)) * 16
        else:
            N = int(rng.integers(1, 1025)) * 8
        routing = "repeats" if rng.random() < 0.3 else "uniform"
        bmap = str(rng.choice(["contiguous", "random", "roundrobin"]))
        dedup = bool(rng.random() < 0.5)
        cases.append((M, N, G, k, B, dtype, routing, bmap, dedup))
    return cases


RANDOM_FUSED = _random_fused_cases()


@pytest.mark.parametrize("case", RANDOM_FUSED, ids=[
    f"M{c[0]}-N{c[1]}-G{c[2]}-k{c[3]}-B{c[4]}-{c[5]}-{c[6]}-{c[7]}-{'dedup' if c[8] else 'flat'}"
    for c in RANDOM_FUSED])
def test_fused_random_shapes(gpu_lib, case):
    M, N, G, k, B, dtype, routing, bmap, dedup = case
    w = wl.make_custom(M, N, G, k, B, dtype=dtype, routing=routing, bucket_map=bmap, seed=M + N)
    check(w, dedup, f"fused {w.name} map={bmap} scales={w.x_scale is not None} dedup={dedup}")


@pytest.mark.parametrize("dedup", [False, True])
def test_prepared_calls_match_immediate_calls(gpu_lib, dedup):
    """Prepared calls (arguments checked and marshalled once) give the immediate calls'
    bytes, follow in-place changes of their inputs' contents, and run on the stream they
    were prepared with."""
    say(f"prepared calls dedup={dedup}")
    w1 = wl.make_workload(1)                                        # M = 64
    w2 = wl.make_custom(w1.M, w1.N, w1.G, w1.k, w1.B, seed=7)      # same shapes, new contents
    idx, ebkt = dev(w1.topk_idx).clone(), dev(w1.expert_bucket)
    x = rows_dev(w1).clone()
    wts = dev(w1.weights).clone()
    side = torch.cuda.Stream()
    p_lay, lay = moedl.prepare_dispatch_layout(idx, ebkt, w1.B, dedup)
    p_disp, out, _ = moedl.prepare_dispatch(x, lay.send_row, lay.capacity, dedup=dedup)
    p_fused, flay, fout, _ = moedl.prepare_layout_dispatch(idx, ebkt, w1.B, dedup, x,
                                                           stream=side)
    p_comb, y = moedl.prepare_combine(out, wts, lay.slot) if not dedup else (None, None)
    p_na, nlay = moedl.prepare_dispatch_layout_noalloc(idx, ebkt, w1.B, dedup)
    for w in (w1, w2, w1):
        idx.copy_(dev(w.topk_idx))
        x.copy_(rows_dev(w))
        wts.copy_(dev(w.weights))
        p_lay()
        p_na()
        p_disp()
        if p_comb is not None:
            p_comb()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            p_fused()
        torch.cuda.current_stream().wait_stream(side)
        ref_lay = moedl.moe_dispatch_layout(idx, ebkt, w.B, dedup)
        ref_out, _ = moedl.moe_dispatch(x, ref_lay.send_row, ref_lay.capacity, dedup=dedup)
        torch.cuda.synchronize()
        R = int(ref_lay.bucket_offset[w.B].item())
        for got in (lay, flay, nlay):
            for name in ("expert_count", "expert_offset", "bucket_count", "bucket_offset",
                         "slot", "send_row", "status"):
                assert torch.equal(getattr(got, name), getattr(ref_lay, name)), name
            assert torch.equal(got.send_token[:R], ref_lay.send_token[:R])
        assert torch.equal(out[:R], ref_out[:R]) and torch.equal(fout[:R], ref_out[:R])
        if p_comb is not None:
            ref_y = moedl.moe_combine(ref_out, wts, ref_lay.slot)
            torch.cuda.synchronize()
            assert torch.equal(y, ref_y)
