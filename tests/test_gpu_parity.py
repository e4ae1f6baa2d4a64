"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the same
seeded inputs.

Layout, counts, slot/send maps and dispatched rows must match bit for bit; combine
must match the oracle's bf16 output bit for bit (the oracle fixes the fp32 op order,
so the 2e-3 relative tolerance on bf16 outputs leaves no room for any other
result; the relative error is also computed and checked against 2e-3).

Sizes: every standard workload at a reduced token count that spans several
256-token layout tiles with a ragged last tile (full comparison), and at its full
size (full comparison of layout and dispatch, combine on sampled tokens) in the
launch configuration the bench times.
"""
import numpy as np
import pytest
import torch

import oracle
from combine_dispatch_layout_amd import moedl
from combine_dispatch_layout_amd import workloads as wl
from gpu_util import (SENTINEL_BF16, SENTINEL_FP8, assert_bits_equal, assert_dispatch_equal,
                      assert_layout_equal, dev, gpu_combine, gpu_dispatch, gpu_expert_outputs,
                      gpu_layout, host, oracle_combine_tokens, oracle_pipeline, rows_dev, say)

pytestmark = pytest.mark.gpu

REL_TOL = 2e-3


def max_rel_err(got_u16, want_u16):
    g = oracle.bf16_to_f32(got_u16.view(np.uint16)).astype(np.float64)
    r = oracle.bf16_to_f32(want_u16).astype(np.float64)
    nz = r != 0
    assert np.all(g[~nz] == 0)
    return float(np.max(np.abs(g[nz] - r[nz]) / np.abs(r[nz]))) if nz.any() else 0.0


REDUCED = [  # (cfg, M, map_kind)
    (1, None, "pair"), (2, 1000, "pair"), (3, 1000, "pair"), (4, 1000, "pair"),
    (4, 1000, "roundrobin"), (5, 300, "pair"),
]


@pytest.mark.parametrize("cfg,M,map_kind", REDUCED)
@pytest.mark.parametrize("dedup", [False, True])
def test_pipeline_reduced(gpu_lib, cfg, M, map_kind, dedup):
    w = wl.make_workload(cfg, M=M, map_kind=map_kind)
    ctx = f"{w.name} M={w.M} dedup={dedup}"
    say(ctx)
    ref, sent, sent_scale, eo_ref, y_ref = oracle_pipeline(w, dedup)
    lay = gpu_layout(w, dedup)
    assert_layout_equal(lay, ref, ctx)
    out, out_scale = gpu_dispatch(w, lay)
    assert_dispatch_equal(w, out, out_scale, ref, ctx=ctx)
    eo = gpu_expert_outputs(w, lay, out, out_scale)
    y = gpu_combine(w, lay, eo)
    torch.cuda.synchronize()
    got = host(y)
    assert max_rel_err(got, y_ref) <= REL_TOL
    assert_bits_equal(got, y_ref, ctx)


@pytest.mark.parametrize("cfg,map_kind", [(1, "pair"), (2, "pair"), (3, "pair"), (4, "pair"),
                                          (4, "roundrobin"), (5, "pair")])
@pytest.mark.parametrize("dedup", [False, True])
def test_layout_full_size(gpu_lib, cfg, map_kind, dedup):
    w = wl.make_workload(cfg, map_kind=map_kind, with_rows=False)
    say(f"layout {w.name} M={w.M} dedup={dedup}")
    ref = oracle.dispatch_layout(w.topk_idx, w.expert_bucket, w.B, dedup)
    assert_layout_equal(gpu_layout(w, dedup), ref, w.name)


@pytest.fixture(scope="module")
def cfg3():
    return wl.make_workload(3)


@pytest.mark.parametrize("dedup", [False, True])
def test_bench_workload_full_size(gpu_lib, cfg3, dedup):
    """Zipf(1.2) M=16384 N=7168 G=256 top-8: the bench's workload and launch
    configuration (combine reads the dispatched rows in place when dedup is off)."""
    w = cfg3
    say(f"full {w.name} dedup={dedup}")
    ref = oracle.dispatch_layout(w.topk_idx, w.expert_bucket, w.B, dedup)
    lay = gpu_layout(w, dedup)
    assert_layout_equal(lay, ref, w.name)
    out, out_scale = gpu_dispatch(w, lay)
    assert_dispatch_equal(w, out, out_scale, ref, ctx=w.name)
    eo = gpu_expert_outputs(w, lay, out, out_scale)
    y = gpu_combine(w, lay, eo)
    torch.cuda.synchronize()
    rng = np.random.default_rng(99)
    tokens = np.sort(rng.choice(w.M, size=384, replace=False))
    tokens[0], tokens[-1] = 0, w.M - 1
    want = oracle_combine_tokens(w, ref, tokens)
    got = host(y[dev(tokens).long()])
    assert max_rel_err(got, want) <= REL_TOL
    assert_bits_equal(got, want, w.name)
    # identity experts: every output row is its input row (closed form)
    x = torch.from_numpy(w.x.view(np.int16)).cuda()
    x = torch.where(x == -32768, torch.zeros_like(x), x)       # -0 comes back as +0
    assert bool((y == x).all().item())


def fp8_closed_form_check(w, y, chunk=8192):
    """Every token of the fp8 workload, on the device: the stand-in experts all emit
    e = bf16(f32(q) * s) for a token's row, and the token's weights sum to one within a
    few fp32 ulps, so y must equal e bit for bit (a -0 comes back as +0): the
    perturbation is far below half a bf16 ulp.  torch's own fp8 decode and RNE cast
    compute e, independently of the library."""
    xs = dev(w.x_scale)
    x = dev(w.x)
    for t0 in range(0, w.M, chunk):
        t1 = min(w.M, t0 + chunk)
        q = x[t0:t1].view(torch.float8_e4m3fn).float()
        e = (q * xs[t0:t1].repeat_interleave(128, dim=1)).to(torch.bfloat16).view(torch.int16)
        e = torch.where(e == -32768, torch.zeros_like(e), e)
        bad = int((y[t0:t1] != e).sum().item())
        assert bad == 0, f"{w.name}: {bad} elements of tokens [{t0}, {t1}) off the closed form"


@pytest.mark.parametrize("dedup", [False, True])
def test_fp8_workload_full_size(gpu_lib, dedup):
    """M=65536, fp8 e4m3 rows + fp32 per-128 scales, > 2^31-byte buffers, both modes:
    layout and dispatch compared in full, combine on sampled tokens against the oracle
    and on every token against the closed form."""
    w = wl.make_workload(5)
    say(f"full {w.name} dedup={dedup}")
    ref = oracle.dispatch_layout(w.topk_idx, w.expert_bucket, w.B, dedup)
    lay = gpu_layout(w, dedup)
    assert_layout_equal(lay, ref, w.name)
    out, out_scale = gpu_dispatch(w, lay, sentinel=dedup)
    assert_dispatch_equal(w, out, out_scale, ref, chunk=65536, ctx=w.name)
    eo = gpu_expert_outputs(w, lay, out, out_scale)
    del out, out_scale
    y = gpu_combine(w, lay, eo)
    torch.cuda.synchronize()
    del eo
    rng = np.random.default_rng(5)
    tokens = np.sort(rng.choice(w.M, size=256, replace=False))
    tokens[0], tokens[-1] = 0, w.M - 1
    want = oracle_combine_tokens(w, ref, tokens)
    got = host(y[dev(tokens).long()])
    assert max_rel_err(got, want) <= REL_TOL
    assert_bits_equal(got, want, w.name)
    fp8_closed_form_check(w, y)


@pytest.mark.parametrize("cfg,map_kind", [(2, "pair"), (4, "pair"), (4, "roundrobin")])
@pytest.mark.parametrize("dedup", [False, True])
def test_full_size_full_compare(gpu_lib, cfg, map_kind, dedup):
    """Full size, every output compared, in the workload's quoted mode (dedup on) and
    in the other one."""
    w = wl.make_workload(cfg, map_kind=map_kind)
    say(f"full {w.name} dedup={dedup}")
    ref, sent, sent_scale, eo_ref, y_ref = oracle_pipeline(w, dedup)
    lay = gpu_layout(w, dedup)
    assert_layout_equal(lay, ref, w.name)
    out, out_scale = gpu_dispatch(w, lay)
    assert_dispatch_equal(w, out, out_scale, ref, ctx=w.name)
    y = gpu_combine(w, lay, gpu_expert_outputs(w, lay, out, out_scale))
    torch.cuda.synchronize()
    got = host(y)
    assert max_rel_err(got, y_ref) <= REL_TOL
    assert_bits_equal(got, y_ref, w.name)


EDGE = [  # (M, N, G, k, B, dtype, routing, bucket_map)
    (1, 7168, 256, 8, 8, "bf16", "uniform", "contiguous"),
    (2, 8, 4, 1, 1, "bf16", "uniform", "contiguous"),           # one 16-byte vector rows
    (257, 64, 1, 1, 1, "bf16", "uniform", "contiguous"),         # G = 1
    (300, 128, 16, 4, 4, "bf16", "one_expert", "contiguous"),    # all to one expert
    (513, 136, 37, 5, 3, "bf16", "repeats", "random"),           # duplicates, odd shapes
    (700, 1024, 1024, 16, 64, "bf16", "uniform", "random"),      # maximum G, k, B
    (640, 512, 96, 6, 7, "bf16", "uniform", "roundrobin"),
    (333, 16, 64, 8, 8, "fp8", "uniform", "contiguous"),         # fp8, no scales
    (200, 8192, 128, 2, 2, "bf16", "uniform", "contiguous"),     # 16 KiB rows
    (90, 12288, 64, 3, 4, "bf16", "uniform", "contiguous"),      # rows above 16 KiB
    (257, 64, 32, 5, 4, "bf16", "repeats", "random"),            # 5 tiles of 64 tokens (k >= 5)
    (384, 96, 1024, 16, 64, "bf16", "uniform", "random"),        # 6 tiles of 64 at max G, k, B
    (2048, 64, 256, 8, 8, "bf16", "uniform", "random"),          # 32 tiles of 64 tokens
    (2049, 64, 256, 8, 8, "bf16", "uniform", "random"),          # 17 tiles of 128 tokens
    (8192, 64, 256, 8, 8, "bf16", "uniform", "roundrobin"),      # 64 tiles of 128 tokens
    (8193, 64, 256, 8, 8, "bf16", "uniform", "roundrobin"),      # 33 tiles of 256 tokens
    (8192, 64, 64, 4, 8, "bf16", "uniform", "random"),           # k = 4: 32 tiles of 256
    (16384, 64, 1024, 16, 64, "bf16", "uniform", "random"),      # 64 tiles, one launch, max G, k, B
    (16385, 64, 256, 8, 8, "bf16", "uniform", "random"),         # one launch, 33 tiles of 512
    (32768, 32, 256, 8, 8, "bf16", "repeats", "random"),         # 64 tiles of 512 tokens
    (32769, 32, 256, 8, 8, "bf16", "uniform", "roundrobin"),     # 33 tiles of 1024 tokens
    (16385, 64, 256, 9, 8, "bf16", "uniform", "random"),         # k = 9 there: three launches
    (65537, 16, 64, 2, 4, "bf16", "uniform", "random"),          # 65 tiles of 1024: three launches
]


@pytest.mark.parametrize("case", EDGE, ids=[f"M{c[0]}-N{c[1]}-G{c[2]}-k{c[3]}-B{c[4]}-{c[5]}-{c[6]}"
                                            for c in EDGE])
@pytest.mark.parametrize("dedup", [False, True])
def test_edge_shapes(gpu_lib, case, dedup):
    M, N, G, k, B, dtype, routing, bmap = case
    w = wl.make_custom(M, N, G, k, B, dtype=dtype, routing=routing, bucket_map=bmap, seed=M)
    if dtype == "fp8":
        w.x_scale = None
    ctx = f"{w.name} dedup={dedup}"
    say(ctx)
    ref = oracle.dispatch_layout(w.topk_idx, w.expert_bucket, w.B, dedup)
    lay = gpu_layout(w, dedup)
    assert_layout_equal(lay, ref, ctx)
    out, out_scale = gpu_dispatch(w, lay)
    assert_dispatch_equal(w, out, out_scale, ref, ctx=ctx)
    if dtype == "bf16":
        sent, _ = oracle.dispatch(w.x, ref.send_row, ref.R)
        eo_ref = oracle.expert_outputs("identity", sent, ref.send_row, ref.slot, w.topk_idx)
        y_ref = oracle.combine(eo_ref, w.weights, ref.slot)
        eo = gpu_expert_outputs(w, lay, out, out_scale)
        y = gpu_combine(w, lay, eo)
        torch.cuda.synchronize()
        assert_bits_equal(host(y), y_ref, ctx)


def _random_cases(n=24, seed=20261203):
    """Seeded random shapes across every layout path below 65,536 tokens (one tile,
    one launch with 256- or 1024-token tiles), both row dtypes, repeats and all bucket
    maps, bounded so that the oracle finishes each in well under a second."""
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        G = int(rng.choice([1, 3, 16, 64, 128, 256, 1000, 1024]))
        k = int(rng.integers(1, min(16, G) + 1))
        B = int(rng.integers(1, 65))
        if rng.random() < 0.2:  # above 64 tiles of 256 tokens: the 1024-token tiles
            k = min(k, 2)
            M = int(rng.integers(16385, 40000 // k + 1))
        else:
            M = int(np.exp(rng.uniform(0, np.log(40000 // k))))
        dtype = "fp8" if rng.random() < 0.25 else "bf16"
        step = 16 if dtype == "fp8" else 8
        N = int(rng.integers(1, 2048 // step + 1)) * step
        if M * N * 2 > (32 << 20):
            continue
        routing = "repeats" if rng.random() < 0.3 else "uniform"
        bmap = str(rng.choice(["contiguous", "random", "roundrobin"]))
        dedup = bool(rng.random() < 0.5)
        cases.append((M, N, G, k, B, dtype, routing, bmap, dedup))
    return cases


RANDOM = _random_cases()


@pytest.mark.parametrize("case", RANDOM, ids=[
    f"M{c[0]}-N{c[1]}-G{c[2]}-k{c[3]}-B{c[4]}-{c[5]}-{c[6]}-{c[7]}-{'dedup' if c[8] else 'flat'}"
    for c in RANDOM])
def test_random_shapes(gpu_lib, case):
    M, N, G, k, B, dtype, routing, bmap, dedup = case
    w = wl.make_custom(M, N, G, k, B, dtype=dtype, routing=routing, bucket_map=bmap, seed=M + N)
    if dtype == "fp8":
        w.x_scale = None
    ctx = f"{w.name} map={bmap} dedup={dedup}"
    say(ctx)
    ref = oracle.dispatch_layout(w.topk_idx, w.expert_bucket, w.B, dedup)
    lay = gpu_layout(w, dedup)
    assert_layout_equal(lay, ref, ctx)
    out, out_scale = gpu_dispatch(w, lay)
    assert_dispatch_equal(w, out, out_scale, ref, ctx=ctx)
    if dtype == "bf16":
        sent, _ = oracle.dispatch(w.x, ref.send_row, ref.R)
        eo_ref = oracle.expert_outputs("identity", sent, ref.send_row, ref.slot, w.topk_idx)
        y_ref = oracle.combine(eo_ref, w.weights, ref.slot)
        y = gpu_combine(w, lay, gpu_expert_outputs(w, lay, out, out_scale))
        torch.cuda.synchronize()
        assert_bits_equal(host(y), y_ref, ctx)


def test_empty_batch(gpu_lib):
    from combine_dispatch_layout_amd import moedl
    idx = torch.empty((0, 8), dtype=torch.int32, device="cuda")
    ebkt = dev((np.arange(256) // 32).astype(np.int32))
    for dedup in (False, True):
        lay = moedl.moe_dispatch_layout(idx, ebkt, 8, dedup)
        torch.cuda.synchronize()
        assert int(lay.status.item()) == 0
        assert int(lay.expert_count.abs().sum().item()) == 0
        assert int(lay.expert_offset.abs().sum().item()) == 0
        assert host(lay.bucket_offset).tolist() == [0] * 9
        x = torch.empty((0, 7168), dtype=torch.int16, device="cuda")
        out, _ = moedl.moe_dispatch(x, lay.send_row, 0)
        y = moedl.moe_combine(out, torch.empty((0, 8), dtype=torch.float32, device="cuda"),
                              lay.slot)
        torch.cuda.synchronize()
        assert y.shape == (0, 7168)


@pytest.mark.parametrize("dedup", [False, True])
def test_bad_ids_status(gpu_lib, dedup):
    w = wl.make_custom(600, 64, 32, 4, 4, seed=3)
    idx = w.topk_idx.copy()
    idx[300, 2] = 32            # first bad entry: flat 1202
    idx[511, 0] = -5
    w.topk_idx = idx
    ref = oracle.dispatch_layout(idx, w.expert_bucket, w.B, dedup)
    assert ref.status == 300 * 4 + 2 + 1
    lay = gpu_layout(w, dedup)
    assert_layout_equal(lay, ref, "bad ids")
    # the erroneous layout must still be safe to dispatch and combine with
    out, _ = gpu_dispatch(w, lay)
    gpu_combine(w, lay, out)
    torch.cuda.synchronize()
    ebkt = w.expert_bucket.copy()
    ebkt[7] = 4
    w.expert_bucket = ebkt
    lay = gpu_layout(w, dedup)
    torch.cuda.synchronize()
    assert int(lay.status.item()) == -8


def test_deterministic_and_stream_ordered(gpu_lib):
    w = wl.make_workload(3, M=2048)
    results = []
    for _ in range(2):
        lay = gpu_layout(w, False)
        out, _ = gpu_dispatch(w, lay)
        y = gpu_combine(w, lay, out)
        results.append([host(lay.slot), host(out), host(y)])
    for a, b in zip(*results):
        assert np.array_equal(a, b)
    # on a side stream, with the inputs produced on that stream
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        lay = gpu_layout(w, False)
        out, _ = gpu_dispatch(w, lay)
        y = gpu_combine(w, lay, out)
    s.synchronize()
    assert np.array_equal(host(y), results[0][2])


@pytest.mark.parametrize("cfg,M,dedup", [(3, 2048, False), (3, 2048, True), (5, 1024, False),
                                         (4, 1536, True)])
def test_dispatch_shapes_agree(gpu_lib, cfg, M, dedup):
    """Launch geometry must not change any output: moe_dispatch's two kernel shapes (k
    single-store waves, or two waves sharing a token's distinct rows; its dedup flag
    picks the shape) write identical bytes, scales included, for a layout of either
    mode."""
    w = wl.make_workload(cfg, M=M)
    say(f"dispatch shapes {w.name} M={M} dedup-layout={dedup}")
    lay = gpu_layout(w, dedup)
    x = rows_dev(w)
    xs = dev(w.x_scale) if w.x_scale is not None else None
    outs = []
    for shape_flag in (False, True):
        out = torch.full((lay.capacity, w.N), SENTINEL_BF16 if w.dtype == "bf16" else SENTINEL_FP8,
                         dtype=x.dtype, device="cuda")
        osc = (torch.full((lay.capacity, xs.shape[1]), float("nan"), device="cuda")
               if xs is not None else None)
        moedl.moe_dispatch(x, lay.send_row, lay.capacity, xs, out=out, out_scale=osc,
                           dedup=shape_flag)
        outs.append((out, osc))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0], outs[1][0])
    if xs is not None:
        assert torch.equal(outs[0][1].isnan(), outs[1][1].isnan())
        assert torch.equal(torch.nan_to_num(outs[0][1]), torch.nan_to_num(outs[1][1]))
    ref = oracle.dispatch_layout(w.topk_idx, w.expert_bucket, w.B, dedup)
    assert_dispatch_equal(w, outs[0][0], outs[0][1], ref, ctx=w.name)


def test_concurrent_streams(gpu_lib):
    """Calls are reentrant across streams when their buffers differ: two workloads run
    layout -> dispatch -> combine at the same time on two streams, each with its own
    layout workspace, and both match their results from one stream, bit for bit."""
    ws = [wl.make_workload(3, M=3000), wl.make_workload(2, M=2500)]
    modes = [False, True]

    def run(w, dedup):
        lay = gpu_layout(w, dedup)
        out, out_scale = gpu_dispatch(w, lay)
        y = gpu_combine(w, lay, gpu_expert_outputs(w, lay, out, out_scale))
        return lay, out, y

    seq = [run(w, d) for w, d in zip(ws, modes)]
    torch.cuda.synchronize()
    seq = [(host(l.slot), host(l.send_row), host(o), host(y)) for l, o, y in seq]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    conc = []
    for s, w, d in zip(streams, ws, modes):
        with torch.cuda.stream(s):
            conc.append(run(w, d))
    for s in streams:
        s.synchronize()
    for (lay, out, y), (slot_h, row_h, out_h, y_h) in zip(conc, seq):
        assert np.array_equal(host(lay.slot), slot_h)
        assert np.array_equal(host(lay.send_row), row_h)
        assert np.array_equal(host(out), out_h)
        assert np.array_equal(host(y), y_h)


def test_workspace_shared_across_sizes_and_modes(gpu_lib):
    """One zero-filled workspace serves a sequence of layouts of different sizes,
    modes, expert counts and kernel paths (one launch for 2..64 tiles of 256 tokens
    and, at k <= 8, up to 64 tiles of 1024; three launches above; one tile below):
    each call clears what the previous
    one-launch call published and publishes in the other region, so every result must
    match the oracle bit for bit whatever came before it."""
    seq = [(3, 16384, False), (2, 4096, True), (4, 16384, True), (3, 300, False),
           (5, 65536, False), (2, 1000, False), (3, 100, True), (4, 8192, False),
           (5, 70000, True), (3, 16384, True), (2, 4096, False)]
    ws_bytes = max(moedl.workspace_bytes(M, 8, wl.make_workload(c, M=M, with_rows=False).G, 8)
                   for c, M, _ in seq)
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device="cuda")
    for rep in range(2):
        for cfg, M, dedup in seq:
            w = wl.make_workload(cfg, M=M, with_rows=False)
            ctx = f"{w.name} M={M} dedup={dedup} pass {rep}"
            say(ctx)
            lay = moedl.alloc_layout(w.M, w.k, w.G, w.B, dedup)
            lay.workspace = ws
            moedl.moe_dispatch_layout(dev(w.topk_idx), dev(w.expert_bucket), w.B, dedup, out=lay)
            ref = oracle.dispatch_layout(w.topk_idx, w.expert_bucket, w.B, dedup)
            assert_layout_equal(lay, ref, ctx)
