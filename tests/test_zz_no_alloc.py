"""The no-allocation layout call (moe_dispatch_layout_noalloc, static device
workspace) against moe_dispatch_layout with a caller workspace, through the C ABI:
every output bit for bit, on two calls in a row with the second one smaller, for
each kernel path (one launch for 2..64 tiles of 256 tokens or, at k <= 8, of 1024
tokens; three launches above; one tile below) and both modes; then a longer mixed sequence that alternates the two
entry points, since the static array keeps each call's state for the next."""
import numpy as np
import pytest
import torch

from combine_dispatch_layout_amd import moedl
from combine_dispatch_layout_amd import workloads as wl
from gpu_util import dev, say

pytestmark = pytest.mark.gpu

FIELDS = ("expert_count", "expert_offset", "bucket_count", "bucket_offset", "slot",
          "send_row", "status")


def _both(w, dedup):
    idx, ebkt = dev(w.topk_idx), dev(w.expert_bucket)
    a = moedl.moe_dispatch_layout_noalloc(idx, ebkt, w.B, dedup)
    b = moedl.moe_dispatch_layout(idx, ebkt, w.B, dedup)
    torch.cuda.synchronize()
    return a, b


def _assert_same(a, b, ctx):
    assert int(b.status.item()) == 0, ctx
    for f in FIELDS:
        assert torch.equal(getattr(a, f), getattr(b, f)), (ctx, f)
    R = int(b.bucket_offset[-1].item())
    assert torch.equal(a.send_token[:R], b.send_token[:R]), (ctx, "send_token")


@pytest.mark.parametrize("first,second", [
    ((3, 16384), (2, 4096)),      # one launch, then one launch with fewer tiles
    ((5, 65536), (3, 300)),       # one launch of 1024-token tiles, then two tiles
    ((5, 70000), (2, 4096)),      # three launches, then one launch
    ((4, 16384), (3, 200)),       # one launch (G=128), then a single tile
])
@pytest.mark.parametrize("dedup", [False, True])
def test_noalloc_matches_workspace_call(gpu_lib, first, second, dedup):
    for cfg, M in (first, second):
        w = wl.make_workload(cfg, M=M, with_rows=False)
        ctx = f"{w.name} M={M} dedup={dedup}"
        say(ctx)
        a, b = _both(w, dedup)
        _assert_same(a, b, ctx)


def test_noalloc_mixed_sequence(gpu_lib):
    seq = [(3, 16384, True), (2, 4096, False), (4, 8192, True), (5, 65536, True),
           (5, 70000, False), (3, 1000, False), (2, 100, True), (3, 16384, False),
           (4, 300, False)]
    for rep in range(2):
        for cfg, M, dedup in seq:
            w = wl.make_workload(cfg, M=M, with_rows=False)
            ctx = f"{w.name} M={M} dedup={dedup} pass {rep}"
            say(ctx)
            a, b = _both(w, dedup)
            _assert_same(a, b, ctx)


def test_noalloc_refuses_sizes_beyond_its_array(gpu_lib):
    """Sizes whose workspace exceeds the static array are refused before any launch."""
    M, k, G, B = 1 << 20, 8, 1024, 64
    assert moedl.workspace_bytes(M, k, G, B) > moedl.LAYOUT_SCRATCH_BYTES
    idx = torch.zeros((M, k), dtype=torch.int32, device="cuda")
    ebkt = torch.zeros(G, dtype=torch.int32, device="cuda")
    with pytest.raises(moedl.MoeError, match="status 3"):
        moedl.moe_dispatch_layout_noalloc(idx, ebkt, B, False)
