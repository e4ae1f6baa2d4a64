"""The library's calls captured in a HIP graph (torch.cuda.CUDAGraph) and replayed:
every replay must reproduce the eager result bit for bit.  Between replays the program
does eager work of its own (clearing the outputs) and synchronises, so a replay that
skipped a node, or depended on state left by an earlier launch, shows up."""
import numpy as np
import pytest
import torch

from combine_dispatch_layout_amd import moedl
from combine_dispatch_layout_amd import workloads as wl
from gpu_util import dev, say

pytestmark = pytest.mark.gpu

REPLAYS = 3


def _replay_and_compare(fn, outputs, ctx):
    """outputs: the tensors (or views) every call writes in full, or a function that
    returns them once the eager call has run."""
    fn()                                            # eager reference
    torch.cuda.synchronize()
    if callable(outputs):
        outputs = outputs()
    want = [o.clone() for o in outputs]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()                                        # warm-up on a side stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    for r in range(REPLAYS):
        for o in outputs:                           # eager work between replays
            o.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (o, w_) in enumerate(zip(outputs, want)):
            assert torch.equal(o, w_), f"{ctx}: replay {r}, output {i} differs"


@pytest.mark.parametrize("cfg,M", [(1, None), (3, 1000), (3, None)])
@pytest.mark.parametrize("dedup", [False, True])
def test_pipeline_in_graph(gpu_lib, cfg, M, dedup):
    w = wl.make_workload(cfg, M=M)
    say(f"graph {w.name} M={w.M} dedup={dedup}")
    idx, ebkt = dev(w.topk_idx), dev(w.expert_bucket)
    x = dev(w.x.view(np.int16))
    wts = dev(w.weights)
    lay = moedl.alloc_layout(w.M, w.k, w.G, w.B, dedup)
    out = torch.empty((lay.capacity, w.N), dtype=torch.int16, device="cuda")
    ein = torch.empty((w.M * w.k, w.N), dtype=torch.int16, device="cuda")
    y = torch.empty((w.M, w.N), dtype=torch.int16, device="cuda")

    def fn():
        moedl.moe_dispatch_layout(idx, ebkt, w.B, dedup, out=lay)
        moedl.moe_dispatch(x, lay.send_row, lay.capacity, out=out, dedup=dedup)
        src = out
        if dedup:
            moedl.moe_expand(out, lay.send_row, lay.slot, w.M * w.k, out=ein)
            src = ein
        moedl.moe_combine(src, wts, lay.slot, y=y)

    outs = [lay.expert_count, lay.expert_offset, lay.bucket_count, lay.bucket_offset,
            lay.slot, lay.send_row, lay.status, y]
    _replay_and_compare(fn, outs, f"{w.name} dedup={dedup}")


def test_fused_small_m_in_graph(gpu_lib):
    w = wl.make_workload(1)
    idx, ebkt = dev(w.topk_idx), dev(w.expert_bucket)
    x = dev(w.x.view(np.int16))
    wts = dev(w.weights)
    lay = moedl.alloc_layout(w.M, w.k, w.G, w.B, False)
    out = torch.empty((lay.capacity, w.N), dtype=torch.int16, device="cuda")
    y = torch.empty((w.M, w.N), dtype=torch.int16, device="cuda")

    def fn():
        moedl.moe_layout_dispatch(idx, ebkt, w.B, False, x, lay=lay, out=out)
        moedl.moe_combine(out, wts, lay.slot, y=y)

    _replay_and_compare(fn, [lay.slot, lay.send_row, lay.expert_offset, lay.status, out, y],
                        "fused")


def test_pair_counts_and_gemm_in_graph(gpu_lib):
    """The pair counts clear their output with a fill kernel (no memset node), and the
    grouped GEMM's tile metadata is rebuilt on the device in every replay."""
    w = wl.make_workload(4, M=2000, with_rows=False)
    idx = dev(w.topk_idx)
    C = torch.empty((w.G, w.G), dtype=torch.int32, device="cuda")
    lay = moedl.alloc_layout(w.M, w.k, w.G, w.B, False)
    rows = w.M * w.k
    tiles = moedl.moe_grouped_gemm_tiles(
        torch.zeros(w.G, dtype=torch.int32, device="cuda"),
        torch.zeros(w.G, dtype=torch.int32, device="cuda"), rows)
    g = torch.Generator(device="cuda").manual_seed(3)
    xg = torch.randn((rows, 256), generator=g, device="cuda").to(torch.bfloat16).view(torch.int16)
    wg = (torch.randn((w.G, 128, 256), generator=g, device="cuda") * 0.05).to(
        torch.bfloat16).view(torch.int16)
    yg = torch.empty((rows, 128), dtype=torch.int16, device="cuda")
    ebkt = dev(w.expert_bucket)

    def fn():
        moedl.moe_expert_pair_counts(idx, w.G, out=C)
        moedl.moe_dispatch_layout(idx, ebkt, w.B, False, out=lay)
        moedl.moe_grouped_gemm_tiles(lay.expert_offset, lay.expert_count, rows, out=tiles)
        moedl.moe_grouped_gemm(xg, wg, tiles, y=yg)

    def written():
        n = int(tiles.num_tiles.item())             # row0 / rows are written up to n
        return [C, tiles.expert, tiles.row0[:n], tiles.rows[:n], tiles.num_tiles, yg]

    _replay_and_compare(fn, written, "pairs+gemm")
