"""GPU parity of the grouped-GEMM tile metadata (bit for bit) and of the MFMA grouped
GEMM against the exact (float64) products of the oracle.

Tolerance, from the arithmetic: the GPU accumulates K products in fp32 (each product of
two bf16 is exact in fp32; K - 1 rounded adds give |error| < K * 2^-24 * sum|x w| with
round-to-nearest, K * 2^-23 * sum|x w| even with truncation) and rounds once to bf16
(|error| <= 2^-8 |value|, half an ulp of an 8-bit significand), so every element must
satisfy
    |y - exact| <= 2^-8 |exact| + K * 2^-22 * sum_k |x w|.
The second assertion keeps the check from being vacuous: almost every element is
within one bf16 rounding of the exact value.
"""
import numpy as np
import pytest
import torch

import oracle
from combine_dispatch_layout_amd import moedl
from combine_dispatch_layout_amd import workloads as wl
from gpu_util import dev, host, say
from oracle.grouped_gemm import magnitude

pytestmark = pytest.mark.gpu


def _bf16(rng, shape, scale=1.0):
    return oracle.f32_to_bf16_rne((rng.standard_normal(shape) * scale).astype(np.float32))


def _check_tiles(lay_gpu, ref, rows):
    tiles = moedl.moe_grouped_gemm_tiles(lay_gpu.expert_offset, lay_gpu.expert_count, rows)
    torch.cuda.synchronize()
    want = oracle.gemm_tiles(ref.expert_offset, ref.expert_count, moedl.GEMM_TILE_M)
    n = int(tiles.num_tiles.item())
    assert n == len(want)
    got = list(zip(host(tiles.expert)[:n].tolist(), host(tiles.row0)[:n].tolist(),
                   host(tiles.rows)[:n].tolist()))
    assert got == want
    assert np.all(host(tiles.expert)[n:] == -1)
    return tiles


def _bound_check(got, exact, mag, K, ctx):
    err = np.abs(got - exact)
    bound = 2.0 ** -8 * np.abs(exact) + K * 2.0 ** -22 * mag
    assert np.all(err <= bound), (ctx, float((err - bound).max()))
    assert np.mean(err <= 2.0 ** -8 * np.abs(exact)) > 0.99, ctx


def _check_gemm(x, w, ref, tiles, ctx=""):
    """Whole output against the oracle; x, w host bf16 bits."""
    K = x.shape[1]
    y = moedl.moe_grouped_gemm(dev(x.view(np.int16)), dev(w.view(np.int16)), tiles)
    torch.cuda.synchronize()
    exact = oracle.grouped_gemm(x, w, ref.expert_offset, ref.expert_count)
    mag = magnitude(x, w, ref.expert_offset, ref.expert_count)
    got = oracle.bf16_to_f32(host(y).view(np.uint16)).astype(np.float64)
    _bound_check(got, exact, mag, K, ctx)


def _row_owner(ref, rows):
    owner = np.full(rows, -1, dtype=np.int64)
    for e in range(len(ref.expert_count)):
        o, c = int(ref.expert_offset[e]), int(ref.expert_count[e])
        owner[o:o + c] = e
    return owner


@pytest.mark.parametrize("cfg,M,K,Nout", [(2, 512, 1024, 256), (3, 512, 1024, 256),
                                          (4, 700, 512, 384)])
def test_grouped_gemm_reduced(gpu_lib, cfg, M, K, Nout):
    w_ = wl.make_workload(cfg, M=M, with_rows=False)
    say(f"grouped gemm {w_.name} M={M} K={K} Nout={Nout}")
    ref = oracle.dispatch_layout(w_.topk_idx, w_.expert_bucket, w_.B, False)
    lay = moedl.moe_dispatch_layout(dev(w_.topk_idx), dev(w_.expert_bucket), w_.B, False)
    rows = w_.M * w_.k
    tiles = _check_tiles(lay, ref, rows)
    rng = np.random.default_rng([cfg, M])
    x = _bf16(rng, (rows, K))
    w = _bf16(rng, (w_.G, Nout, K), scale=0.05)
    _check_gemm(x, w, ref, tiles, ctx=w_.name)


def test_grouped_gemm_edges(gpu_lib):
    """Experts whose row counts sit at and around the 32-row MFMA blocks and the row
    tile (0, 1, 5, 33, 96, 97, 127 ... 300); K = 64 and 192, Nout = 128 and 256."""
    counts = [0, 1, 127, 128, 129, 300, 0, 5, 255, 256, 257, 33, 96, 97]
    G = len(counts)
    idx = np.concatenate([np.full(c, e, np.int32) for e, c in enumerate(counts)]).reshape(-1, 1)
    rng = np.random.default_rng(1)
    idx = idx[rng.permutation(len(idx))]
    ebkt = np.zeros(G, np.int32)
    ref = oracle.dispatch_layout(idx, ebkt, 1, False)
    lay = moedl.moe_dispatch_layout(dev(idx), dev(ebkt), 1, False)
    rows = len(idx)
    tiles = _check_tiles(lay, ref, rows)
    for K, Nout in ((64, 128), (192, 256)):
        x = _bf16(rng, (rows, K))
        w = _bf16(rng, (G, Nout, K), scale=0.1)
        _check_gemm(x, w, ref, tiles, ctx=f"K={K} Nout={Nout}")


def test_grouped_gemm_full_size_sampled(gpu_lib):
    """Zipf M=16384 top-8 (131072 rows, the hottest expert ~15k of them), K=7168,
    Nout=256: 200 sampled rows plus the first and last, each against the oracle run
    on that row and its expert's weights."""
    w_ = wl.make_workload(3, with_rows=False)
    say("grouped gemm full size, sampled rows")
    ref = oracle.dispatch_layout(w_.topk_idx, w_.expert_bucket, w_.B, False)
    lay = moedl.moe_dispatch_layout(dev(w_.topk_idx), dev(w_.expert_bucket), w_.B, False)
    rows, K, Nout = w_.M * w_.k, 7168, 256
    tiles = _check_tiles(lay, ref, rows)
    g = torch.Generator(device="cuda").manual_seed(5)
    xd = torch.randn((rows, K), generator=g, device="cuda").to(torch.bfloat16).view(torch.int16)
    wd = (torch.randn((w_.G, Nout, K), generator=g, device="cuda") * 0.02).to(
        torch.bfloat16).view(torch.int16)
    y = moedl.moe_grouped_gemm(xd, wd, tiles)
    torch.cuda.synchronize()
    rng = np.random.default_rng(3)
    sample = np.unique(np.concatenate([rng.choice(rows, 200, replace=False), [0, rows - 1]]))
    owner = _row_owner(ref, rows)[sample]
    assert np.all(owner >= 0)
    xs = host(xd[dev(sample)]).view(np.uint16)
    ws = host(wd[dev(owner)]).view(np.uint16)                     # [s, Nout, K]
    # each sampled row is a one-row group of its own expert
    one = np.ones(len(sample), dtype=np.int64)
    offs = np.arange(len(sample), dtype=np.int64)
    exact = np.zeros((len(sample), Nout))
    mag = np.zeros((len(sample), Nout))
    for i in range(len(sample)):
        exact[i] = oracle.grouped_gemm(xs[i:i + 1], ws[i:i + 1], offs[:1], one[:1])[0]
        mag[i] = magnitude(xs[i:i + 1], ws[i:i + 1], offs[:1], one[:1])[0]
    got = oracle.bf16_to_f32(host(y[dev(sample)]).view(np.uint16)).astype(np.float64)
    _bound_check(got, exact, mag, K, "full size")


def _tiles_of(entries, size=None):
    """GemmTiles holding the given (expert, first row, rows) entries, padded with expert
    -1 to `size` entries."""
    size = size or len(entries)
    pad = [(-1, 0, 0)] * (size - len(entries))
    i32 = dict(dtype=torch.int32, device="cuda")
    cols = list(zip(*(list(entries) + pad)))
    return moedl.GemmTiles(torch.tensor(cols[0], **i32), torch.tensor(cols[1], **i32),
                           torch.tensor(cols[2], **i32), torch.tensor([len(entries)], **i32))


@pytest.mark.parametrize("K", [64, 128])
@pytest.mark.parametrize("size", [6, 260])
def test_grouped_gemm_bad_tiles(gpu_lib, size, K):
    """Hand-made tile arrays holding an expert id past G, a negative one, a first row
    past the end, a negative first row and a tile running past the last row: the bad
    tiles are skipped, the long one is clipped at the last row, the valid ones are
    computed, and rows no valid tile names keep their previous contents.  Six entries
    launch the split shape (128-row halves), 260 the whole-tile shape (256-row body):
    register-staged at K = 64, direct-to-LDS at K = 128 (whose grid, rounded up to a
    multiple of 8 tiles, also has workgroups past the last entry)."""
    rows, Nout, G = 400, 128, 3
    rng = np.random.default_rng(11)
    x = _bf16(rng, (rows, K))
    w = _bf16(rng, (G, Nout, K), scale=0.1)
    tiles = _tiles_of([(0, 0, 128),      # valid
                       (3, 128, 62),     # expert == G: skipped
                       (1, 190, 256),    # runs past the last row: clipped to rows 190..399
                       (2, 450, 16),     # first row past the end: skipped
                       (-5, 128, 8),     # negative expert: skipped
                       (1, -3, 64)],     # negative first row: skipped
                      size)
    sentinel = 0x7FC1
    y = torch.full((rows, Nout), sentinel, dtype=torch.int16, device="cuda")
    moedl.moe_grouped_gemm(dev(x.view(np.int16)), dev(w.view(np.int16)), tiles, y=y)
    torch.cuda.synchronize()
    yh = host(y).view(np.uint16)
    offs = np.array([0, 190, 0], dtype=np.int64)
    cnts = np.array([128, 210, 0], dtype=np.int64)
    exact = oracle.grouped_gemm(x, w, offs, cnts)
    mag = magnitude(x, w, offs, cnts)
    got = oracle.bf16_to_f32(yh).astype(np.float64)
    for lo, hi in ((0, 128), (190, 400)):
        _bound_check(got[lo:hi], exact[lo:hi], mag[lo:hi], K, f"rows {lo}..{hi}")
    assert np.all(yh[128:190] == sentinel)


@pytest.mark.parametrize("K", [192, 256])
def test_grouped_gemm_launch_shapes_agree(gpu_lib, K):
    """The kernel has three launch shapes, chosen by how far the grid fills the chip:
    256-column blocks, 128-column blocks, and 128-column blocks with every tile split
    over two workgroups.  One problem, with experts whose row counts straddle the 128-
    and 256-row bodies, is driven through all three by sizing the tile arrays (the exact
    bound, 200 entries, 300 entries; unused entries carry expert -1): the outputs must
    be identical bit for bit and within the oracle's bound.  At K = 256 the first two
    shapes run the direct-to-LDS body and the split one the register-staged body, so
    the two bodies are compared bit for bit too."""
    counts = [0, 1, 127, 128, 129, 300, 0, 5, 255, 256, 257, 33, 96, 97, 520]
    G, Nout = len(counts), 256
    idx = np.concatenate([np.full(c, e, np.int32) for e, c in enumerate(counts)]).reshape(-1, 1)
    rng = np.random.default_rng(5)
    idx = idx[rng.permutation(len(idx))]
    rows = len(idx)
    ebkt = np.zeros(G, np.int32)
    ref = oracle.dispatch_layout(idx, ebkt, 1, False)
    lay = moedl.moe_dispatch_layout(dev(idx), dev(ebkt), 1, False)
    exact_size = _check_tiles(lay, ref, rows)
    assert exact_size.max_tiles * (Nout // 128) < 256                  # split shape
    outs = [exact_size]
    i32 = dict(dtype=torch.int32, device="cuda")
    for size in (200, 300):                       # 128-column, then 256-column blocks
        t = moedl.GemmTiles(torch.empty(size, **i32), torch.empty(size, **i32),
                            torch.empty(size, **i32), torch.empty(1, **i32))
        outs.append(moedl.moe_grouped_gemm_tiles(lay.expert_offset, lay.expert_count, rows,
                                                 out=t))
    x = _bf16(rng, (rows, K))
    w = _bf16(rng, (G, Nout, K), scale=0.1)
    xd, wd = dev(x.view(np.int16)), dev(w.view(np.int16))
    ys = [moedl.moe_grouped_gemm(xd, wd, t) for t in outs]
    torch.cuda.synchronize()
    assert torch.equal(ys[0], ys[1]) and torch.equal(ys[0], ys[2])
    exact = oracle.grouped_gemm(x, w, ref.expert_offset, ref.expert_count)
    mag = magnitude(x, w, ref.expert_offset, ref.expert_count)
    got = oracle.bf16_to_f32(host(ys[0]).view(np.uint16)).astype(np.float64)
    _bound_check(got, exact, mag, K, "launch shapes")


def _random_gemm_cases(n=10, seed=20261205):
    """Seeded random grouped problems: skewed expert sizes (some empty, some several
    tiles), K a multiple of 64 (so both the direct-to-LDS and the register-staged bodies
    run) and Nout a multiple of 128 (so all three launch shapes run)."""
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        G = int(rng.integers(1, 65))
        sizes = np.floor(rng.pareto(1.2, G) * 60).astype(np.int64)
        sizes[rng.random(G) < 0.15] = 0
        sizes = np.minimum(sizes, 1500)
        K = int(rng.choice([64, 128, 192, 256, 384, 512, 1024]))
        Nout = int(rng.choice([128, 256, 384, 512, 768]))
        cases.append((tuple(int(v) for v in sizes), K, Nout))
    return cases


GEMM_RANDOM = _random_gemm_cases()


@pytest.mark.parametrize("case", GEMM_RANDOM, ids=[f"G{len(c[0])}-rows{sum(c[0])}-K{c[1]}-N{c[2]}"
                                                   for c in GEMM_RANDOM])
def test_grouped_gemm_random(gpu_lib, case):
    counts, K, Nout = case
    G = len(counts)
    rows = sum(counts)
    say(f"grouped gemm random G={G} rows={rows} K={K} Nout={Nout}")
    idx = np.concatenate([np.full(c, e, np.int32) for e, c in enumerate(counts)] +
                         [np.zeros(0, np.int32)]).reshape(-1, 1)
    rng = np.random.default_rng([G, rows, K, Nout])
    idx = idx[rng.permutation(len(idx))]
    ebkt = np.zeros(G, np.int32)
    ref = oracle.dispatch_layout(idx, ebkt, 1, False)
    lay = moedl.moe_dispatch_layout(dev(idx), dev(ebkt), 1, False)
    tiles = _check_tiles(lay, ref, rows)
    if rows == 0:
        return
    x = _bf16(rng, (rows, K))
    w = _bf16(rng, (G, Nout, K), scale=0.1)
    _check_gemm(x, w, ref, tiles, ctx=f"G={G} rows={rows} K={K} Nout={Nout}")
