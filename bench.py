"""Benchmark: MoE dispatch layout + dispatch + combine on one MI355X.

Workload (the headline configuration): M=16384 tokens, N=7168 bf16 hidden, G=256
experts, top-8 drawn without replacement from Zipf(1.2) over a seeded expert
permutation, 8 buckets of 32 consecutive experts, softmax routing weights, identity
experts, dedup off.  One step = moe_dispatch_layout + moe_dispatch + moe_combine
(combine reads the dispatched rows in place: identity experts need no copy).  All
inputs are resident in HBM before timing starts.

Printed: one JSON line with algorithmic HBM GB/s (value), us per step, the roofline
of the dominant kernel (per-kernel durations from HIP events recorded on the
library's stream inside the timed region), a graph-replay latency following the
microbenchmark method of "Purlin: Separating Orchestration from the Datapath of
Collectives" (section 5: 128 invocations captured in a graph, one warm-up replay,
eight timed replays, divided by 1,024), a plain copy-kernel ceiling, and the CPU
oracle timed on the same inputs.

    python bench.py [--gpus 1] [--steps 100] [--warmup 20] [--cfg 1-5] [--dedup] [--no-cpu]
    python bench.py --path bucket    # dedup round trip: layout, dispatch, moe_expand,
                                     # moe_combine_partial, moe_combine_reduce
    python bench.py --path placement --cfg 4   # pair counts, greedy placement, savings
    python bench.py --path gemm      # tile metadata + MFMA grouped GEMM over the layout
    python bench.py --path small     # small M: fused layout+dispatch vs separate calls
    python bench.py --path chain     # one layer in order: layout, dispatch, grouped GEMM
                                     # (hidden -> hidden per expert), combine
    python bench.py --path dispatch-x  # dispatch (chosen shape, two-wave) at a fixed 1.88 GB send
                                       # buffer while x grows from 235 MB to 1.88 GB
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time
from typing import Optional

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "dispatch+combine µs and HBM GB/s (% of peak), M=16384,N=7168,G=256,k=8"
HBM_PEAK_GBPS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = {
    "dispatch": "combine_dispatch_layout_amd/csrc/dispatch.hip",
    "combine": "combine_dispatch_layout_amd/csrc/combine.hip",
    "grouped_gemm": "combine_dispatch_layout_amd/csrc/gemm.hip",
    "expand": "combine_dispatch_layout_amd/csrc/bucket.hip",
    "combine_partial": "combine_dispatch_layout_amd/csrc/bucket.hip",
    "combine_reduce": "combine_dispatch_layout_amd/csrc/bucket.hip",
    "layout": "combine_dispatch_layout_amd/csrc/layout.hip",
    "layout_dispatch": "combine_dispatch_layout_amd/csrc/layout.hip",
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # 100 timed and 20 warm-up iterations: the event-loop method of "All2all performance
    # comparison between Triton-distributed and DeepEP" ("Test Code Snippet")
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--dedup", action="store_true", help="time dedup mode instead")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle leg")
    ap.add_argument("--no-graph", action="store_true", help="skip the graph-replay leg")
    ap.add_argument("--path", choices=["flat", "bucket", "placement", "gemm", "small", "chain",
                                       "dispatch-x"],
                    default="flat",
                    help="flat: layout+dispatch+combine; bucket: the dedup round trip; "
                         "placement: pair counts + greedy placement and their dedup savings; "
                         "gemm: grouped-GEMM tile metadata + the MFMA grouped GEMM; "
                         "small: latency at M <= 512, fused layout+dispatch vs three calls; "
                         "chain: layout, dispatch, grouped GEMM (N -> N), combine in order; "
                         "dispatch-x: dispatch shapes at a fixed send buffer, growing x")
    ap.add_argument("--nout", type=int, default=2048, help="grouped GEMM output width")
    ap.add_argument("--small-m", default="64,128,256,512",
                    help="token counts of the small path (comma-separated, each <= 512)")
    ap.add_argument("--cfg", type=int, default=3, choices=[1, 2, 3, 4, 5],
                    help="workload: 1 uniform M=64; 2 uniform M=4096, scaled experts; "
                         "3 Zipf M=16384 (the headline); 4 correlated pairs, N=2048, G=128; "
                         "5 uniform M=65536 fp8 with scales")
    return ap.parse_args()


def source_hash(rel: str) -> str:
    with open(os.path.join(ROOT, rel), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def recorded_traffic(kernel: str, workload: str, path: Optional[str] = None):
    """HBM bytes per launch from the committed rocprofv3 counter summary of this
    workload, if it was taken on the current kernel source (else None)."""
    path = path or os.path.join(PROFILES, f"hbm_traffic_{workload}.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get(f"{kernel}.source_sha256") != source_hash(KERNEL_SOURCES[kernel]):
        return None
    if vals.get("workload") != workload:
        return None
    try:
        return float(vals[f"{kernel}.hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def host_cores() -> str:
    cpu_model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu_model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return f"1 of {len(os.sched_getaffinity(0))} host cores ({cpu_model})"


def event_steps(K: int, n: int = 5) -> list:
    """The timed steps that carry per-kernel HIP events: n evenly spaced ones, centred
    in n equal runs of steps so that the first (which starts from an idle queue) is
    not one of them; all steps when K <= n.  An event record costs the stream ~3.3 us
    on MI355X (a step with four of them: 680.5 vs 668.0 us at the headline, 200.9 vs
    187.7 us at M=4096), so recording them on every step would inflate the wall time
    that `value` is taken from; the kernels' durations are steady enough for a few
    samples."""
    if K <= n:
        return list(range(K))
    return sorted({((2 * i + 1) * K) // (2 * n) for i in range(n)})


def hbm_roofline(kernel: str, alg_bytes: float, launch_us: float, traffic=None, **extra):
    achieved = alg_bytes / (launch_us * 1e-6) / 1e9
    r = {"bound": "hbm", "kernel": kernel, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
         "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
         "alg_bytes_per_launch": int(alg_bytes), "launch_us": round(launch_us, 2)}
    r.update(extra)
    return r


def cpu_baseline(w, dedup: bool, max_tokens: int = 16384):
    """The oracle as it stands, single-threaded, on the same inputs: layout, dispatch
    and combine on the first min(M, max_tokens) tokens (the whole workload up to 16384
    tokens), each phase timed; the stand-in expert step between dispatch and combine
    runs but, as on the GPU, is not counted."""
    import oracle
    Ms = min(w.M, max_tokens)
    idx, x, wts = w.topk_idx[:Ms], w.x[:Ms], w.weights[:Ms]
    xs = w.x_scale[:Ms] if w.x_scale is not None else None
    t0 = time.perf_counter()
    lay = oracle.dispatch_layout(idx, w.expert_bucket, w.B, dedup)
    t1 = time.perf_counter()
    sent, sent_scale = oracle.dispatch(x, lay.send_row, lay.R, xs)
    t2 = time.perf_counter()
    if w.standin == "identity" and not dedup and w.dtype == "bf16":
        eo = sent                                   # combine reads the dispatched rows
    else:
        eo = oracle.expert_outputs(w.standin, sent, lay.send_row, lay.slot, idx, sent_scale)
    t3 = time.perf_counter()
    oracle.combine(eo, wts, lay.slot)
    t4 = time.perf_counter()
    dt = (t1 - t0) + (t2 - t1) + (t4 - t3)
    scale_bytes = xs.shape[1] * 4 if xs is not None else 0
    alg = (Ms + lay.R) * (w.row_bytes + scale_bytes) + (Ms * w.k + Ms) * w.N * 2
    return {
        "value": round(alg / dt / 1e9, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
        "sample": (f"{'whole workload' if Ms == w.M else 'first'} {Ms} tokens, one pass of "
                   f"layout+dispatch+combine ({dt:.2f} s; stand-in expert step excluded), "
                   f"{host_cores()}"),
        "seconds": round(dt, 3),
        "phase_seconds": {"layout": round(t1 - t0, 3), "dispatch": round(t2 - t1, 3),
                          "combine": round(t4 - t3, 3)},
    }


def bench_bucket(args, w, dev):
    """Dedup round trip with identity experts: layout (dedup) -> dispatch -> expand ->
    combine_partial -> combine_reduce.  Prints one JSON line (not the headline)."""
    import torch
    from combine_dispatch_layout_amd import moedl
    M, N, G, k, B = w.M, w.N, w.G, w.k, w.B
    rb = w.row_bytes
    idx = torch.from_numpy(w.topk_idx).to(dev)
    ebkt = torch.from_numpy(w.expert_bucket).to(dev)
    x = torch.from_numpy(w.x.view(np.int16)).to(dev)
    wts = torch.from_numpy(w.weights).to(dev)
    lay = moedl.alloc_layout(M, k, G, B, True, dev)
    cap = lay.capacity
    out = torch.empty((cap, N), dtype=torch.int16, device=dev)
    ein = torch.empty((M * k, N), dtype=torch.int16, device=dev)
    part = torch.empty((cap, N), dtype=torch.int16, device=dev)
    y = torch.empty((M, N), dtype=torch.int16, device=dev)
    calls = [
        lambda: moedl.moe_dispatch_layout(idx, ebkt, B, True, out=lay),
        lambda: moedl.moe_dispatch(x, lay.send_row, cap, out=out, dedup=True),
        lambda: moedl.moe_expand(out, lay.send_row, lay.slot, M * k, out=ein),
        lambda: moedl.moe_combine_partial(ein, wts, lay.slot, lay.send_row, cap, partial=part),
        lambda: moedl.moe_combine_reduce(part, lay.send_row, y=y),
    ]
    for _ in range(max(1, args.warmup)):
        for c in calls:
            c()
    torch.cuda.synchronize()
    assert int(lay.status.item()) == 0
    R = int(lay.bucket_offset[B].item())
    rows = {"layout": 0, "dispatch": M + R, "expand": R + M * k, "combine_partial": M * k + R,
            "combine_reduce": R + M}
    names = list(rows)
    stream = torch.cuda.current_stream()
    K = args.steps
    sampled = event_steps(K)
    ev = {i: [torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)]
          for i in sampled}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        e = ev.get(i)
        if e is None:
            for c in calls:
                c()
            continue
        e[0].record(stream)
        for c, ec in zip(calls, e[1:]):
            c()
            ec.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = {n: float(np.mean([e[q].elapsed_time(e[q + 1]) for e in ev.values()]))
           for q, n in enumerate(names)}
    total = sum(rows.values()) * rb
    ms = wall * 1e3 / K
    # identity experts, weights summing to one: y is x to within two bf16 roundings
    diff = (y.view(torch.bfloat16).float() - x.view(torch.bfloat16).float()).abs()
    assert bool((diff <= x.view(torch.bfloat16).float().abs() * (2 * 2.0 ** -8) + 1e-30).all().item())
    # a 2 GiB plain copy: calibrates the HBM byte counters of a profiled run of this path
    from combine_dispatch_layout_amd import harness
    src = torch.empty(1 << 30, dtype=torch.int16, device=dev)
    dst = torch.empty_like(src)
    harness.copy(src, dst)
    torch.cuda.synchronize()
    del src, dst
    # roofline of the slowest data-moving kernel of the round trip
    wl_name = w.name + "-dedup-roundtrip"
    dom = max((n for n in names if rows[n]), key=lambda n: per[n])
    roofline = hbm_roofline(dom, rows[dom] * rb, per[dom] * 1e3,
                            traffic=recorded_traffic(dom, wl_name))
    cpu = None if args.no_cpu else cpu_bucket_baseline(w, 8192)
    res = {"metric": METRIC + " [dedup round trip]", "value": round(total / (ms * 1e-3) / 1e9, 1),
           "unit": "GB/s", "n_gpus": 1, "steps": K, "warmup": args.warmup,
           "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16 rows, f32 accumulation", "data": "synthetic",
           "config": {"workload": wl_name, "M": M, "N": N, "G": G, "k": k,
                      "B": B, "send_rows": R, "dedup_saving": round(1 - R / (M * k), 4)},
           "us_per_step": round(ms * 1e3, 2), "alg_bytes_per_step": total,
           "event_us": {n: round(per[n] * 1e3, 2) for n in names},
           "event_steps": len(sampled),
           "kernel_gbps": {n: round(rows[n] * rb / (per[n] * 1e-3) / 1e9, 1)
                           for n in names if rows[n]},
           "roofline": roofline, "cpu_baseline": cpu}
    print(json.dumps(res))


def cpu_bucket_baseline(w, max_tokens: int):
    """The oracle's dedup round trip (layout, dispatch, expand, combine_partial,
    combine_reduce), single-threaded, on the first min(M, max_tokens) tokens."""
    import oracle
    Ms = min(w.M, max_tokens)
    idx, x, wts = w.topk_idx[:Ms], w.x[:Ms], w.weights[:Ms]
    k, rb = w.k, w.row_bytes
    t = [time.perf_counter()]
    lay = oracle.dispatch_layout(idx, w.expert_bucket, w.B, True)
    t.append(time.perf_counter())
    sent, _ = oracle.dispatch(x, lay.send_row, lay.R)
    t.append(time.perf_counter())
    ein, _ = oracle.expand(sent, lay.send_row, lay.slot, Ms * k)
    t.append(time.perf_counter())
    part = oracle.combine_partial(ein, wts, lay.slot, lay.send_row, lay.R)
    t.append(time.perf_counter())
    oracle.combine_reduce(part, lay.send_row)
    t.append(time.perf_counter())
    dt = t[-1] - t[0]
    R = lay.R
    alg = ((Ms + R) + (R + Ms * k) + (Ms * k + R) + (R + Ms)) * rb
    names = ["layout", "dispatch", "expand", "combine_partial", "combine_reduce"]
    return {"value": round(alg / dt / 1e9, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": (f"{'whole workload' if Ms == w.M else 'first'} {Ms} tokens, one pass of "
                       f"the dedup round trip ({dt:.2f} s), {host_cores()}"),
            "seconds": round(dt, 3),
            "phase_seconds": {n: round(t[i + 1] - t[i], 3) for i, n in enumerate(names)}}


def bench_placement(args, w, dev):
    """Expert pair counts on the GPU, greedy placement on the host, and the send rows
    a dedup layout needs under round-robin, pair-aware and greedy maps."""
    import torch
    from combine_dispatch_layout_amd import moedl, workloads
    M, G, k, B = w.M, w.G, w.k, w.B
    idx = torch.from_numpy(w.topk_idx).to(dev)
    C = moedl.moe_expert_pair_counts(idx, G)
    for _ in range(max(1, args.warmup)):
        moedl.moe_expert_pair_counts(idx, G, out=C)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(args.steps):
        moedl.moe_expert_pair_counts(idx, G, out=C)
    e.record()
    torch.cuda.synchronize()
    counts_us = s.elapsed_time(e) * 1e3 / args.steps
    t0 = time.perf_counter()
    greedy = moedl.moe_place_experts(C, B)
    greedy_ms = (time.perf_counter() - t0) * 1e3
    maps = {"round_robin": workloads.round_robin_buckets(G, B), "greedy": greedy}
    if "hot_pairs" in w.meta:
        maps["pair_aware"] = workloads.pair_aware_buckets(w.meta["hot_pairs"], G, B)
    if G % B == 0:
        maps["contiguous"] = workloads.contiguous_buckets(G, B)
    rows = {}
    for name, m in maps.items():
        lay = moedl.moe_dispatch_layout(idx, torch.from_numpy(m).to(dev), B, True)
        torch.cuda.synchronize()
        rows[name] = int(lay.bucket_offset[B].item())
    saving = {n: round(1 - r / (M * k), 4) for n, r in rows.items()}
    # out of sample: place from the first half of the tokens, measure on the second
    h = M // 2
    Ch = moedl.moe_expert_pair_counts(idx[:h].contiguous(), G)
    holdout_map = moedl.moe_place_experts(Ch, B)
    holdout = {}
    for name, m in (("greedy_from_first_half", holdout_map), ("round_robin", maps["round_robin"])) + \
            ((("pair_aware", maps["pair_aware"]),) if "pair_aware" in maps else ()):
        lay = moedl.moe_dispatch_layout(idx[h:].contiguous(), torch.from_numpy(m).to(dev), B, True)
        torch.cuda.synchronize()
        holdout[name] = round(1 - int(lay.bucket_offset[B].item()) / ((M - h) * k), 4)
    # pair counts: read the routing table once, write the G x G counts
    roofline = hbm_roofline("pair_counts", M * k * 4 + G * G * 4, counts_us)
    cpu = None
    if not args.no_cpu:
        import oracle
        t0 = time.perf_counter()
        Co = oracle.pair_counts(w.topk_idx, G)
        t1 = time.perf_counter()
        omap = oracle.greedy_place(Co, B)
        t2 = time.perf_counter()
        cpu = {"value": round((t1 - t0) * 1e6, 1), "unit": "us (pair counts)", "cores": 1,
               "kind": "oracle", "greedy_ms": round((t2 - t1) * 1e3, 3),
               "same_map_as_library": bool(np.array_equal(omap, greedy)),
               "sample": f"whole workload, M={M}, G={G}, one pass, {host_cores()}"}
    res = {"metric": "expert placement: dedup saving (fraction of token copies removed)",
           "value": saving["greedy"], "unit": "fraction", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "higher_is_better": True, "vs_baseline": None,
           "dtype": "int32",
           "data": "synthetic", "config": {"workload": w.name, "M": M, "G": G, "k": k, "B": B},
           "send_rows": rows, "dedup_saving": saving, "dedup_saving_second_half": holdout,
           "pair_counts_us": round(counts_us, 2), "greedy_host_ms": round(greedy_ms, 3),
           "roofline": roofline, "cpu_baseline": cpu}
    print(json.dumps(res))


MFMA_BF16_PEAK_TFLOPS = 2500.0


def _time_calls(torch, calls, steps):
    """Mean event time (us) of each call over `steps` rounds, after one warm-up round."""
    for c in calls:
        c()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)]
          for _ in range(steps)]
    for i in range(steps):
        ev[i][0].record(stream)
        for c, e in zip(calls, ev[i][1:]):
            c()
            e.record(stream)
    torch.cuda.synchronize()
    return [float(np.mean([e[q].elapsed_time(e[q + 1]) for e in ev])) * 1e3
            for q in range(len(calls))]


def _time_gemm(moedl, torch, x, wt, tiles, y, lay_offset, lay_count, steps, warmup):
    """Mean event time (us) of moe_grouped_gemm_tiles and moe_grouped_gemm over `steps`."""
    rows = x.shape[0]
    calls = [lambda: moedl.moe_grouped_gemm_tiles(lay_offset, lay_count, rows, out=tiles),
             lambda: moedl.moe_grouped_gemm(x, wt, tiles, y=y)]
    for _ in range(max(1, warmup)):
        for c in calls:
            c()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for i in range(steps):
        ev[i][0].record(stream)
        for c, e in zip(calls, ev[i][1:]):
            c()
            e.record(stream)
    torch.cuda.synchronize()
    return [float(np.mean([e[q].elapsed_time(e[q + 1]) for e in ev])) * 1e3 for q in range(2)]


def bench_gemm(args, w, dev):
    """The expert step over the headline layout: every dispatched row (M*k of them,
    slot-indexed by expert) times its expert's [Nout, N] bf16 weights, fp32 accumulate.
    Also the grouped-GEMM shape the DeepSpeed page measures (16 experts, 760 tokens,
    dim 2048 -> hidden 768, unbalanced), as context, and the regular form of the
    headline problem (M*k/G rows per expert) run by the vendor's batched product and by
    this library, interleaved, as the reference for the grouped kernel."""
    import torch
    from combine_dispatch_layout_amd import moedl
    M, N, G, k, B = w.M, w.N, w.G, w.k, w.B
    Nout = args.nout
    idx = torch.from_numpy(w.topk_idx).to(dev)
    ebkt = torch.from_numpy(w.expert_bucket).to(dev)
    x = torch.from_numpy(w.x.view(np.int16)).to(dev)
    lay = moedl.alloc_layout(M, k, G, B, False, dev)
    moedl.moe_dispatch_layout(idx, ebkt, B, False, out=lay)
    xe = torch.empty((M * k, N), dtype=torch.int16, device=dev)
    moedl.moe_dispatch(x, lay.send_row, M * k, out=xe)
    gen = torch.Generator(device=dev).manual_seed(11)
    wt = (torch.randn((G, Nout, N), generator=gen, device=dev) * 0.02).to(
        torch.bfloat16).view(torch.int16)
    tiles = moedl.moe_grouped_gemm_tiles(lay.expert_offset, lay.expert_count, M * k)
    y = torch.empty((M * k, Nout), dtype=torch.int16, device=dev)
    t_tiles, t_gemm = _time_gemm(moedl, torch, xe, wt, tiles, y, lay.expert_offset,
                                 lay.expert_count, args.steps, args.warmup)
    torch.cuda.synchronize()
    flops = 2.0 * M * k * N * Nout
    tflops = flops / (t_gemm * 1e-6) / 1e12
    # sanity: one sampled row per 4096 against a float32 product on the GPU
    off_h, cnt_h = lay.expert_offset.cpu().numpy(), lay.expert_count.cpu().numpy()
    owner = np.full(M * k, -1, dtype=np.int64)
    for e in range(G):
        owner[off_h[e]:off_h[e] + cnt_h[e]] = e
    r = np.arange(0, M * k, 4096)
    rd, ed = torch.from_numpy(r).to(dev), torch.from_numpy(owner[r]).to(dev)
    ref = torch.bmm(wt[ed].view(torch.bfloat16).float().contiguous(),
                    xe[rd].view(torch.bfloat16).float().unsqueeze(2).contiguous()).squeeze(2)
    got = y[rd].view(torch.bfloat16).float()
    assert bool(((got - ref).abs() <= ref.abs() * 2.0 ** -7 + 1e-2).all().item()), "gemm check"

    # the DeepSpeed page's grouped-GEMM shape: 16 experts, 760 tokens, 2048 -> 768
    Gs, Ms, Ks, Ns = 16, 760, 2048, 768
    rng = np.random.default_rng(12)
    cnt = rng.multinomial(Ms, rng.dirichlet(np.ones(Gs))).astype(np.int32)
    off = np.concatenate([[0], np.cumsum(cnt)[:-1]]).astype(np.int32)
    xs = (torch.randn((Ms, Ks), generator=gen, device=dev)).to(torch.bfloat16).view(torch.int16)
    ws = (torch.randn((Gs, Ns, Ks), generator=gen, device=dev) * 0.02).to(
        torch.bfloat16).view(torch.int16)
    offd, cntd = torch.from_numpy(off).to(dev), torch.from_numpy(cnt).to(dev)
    ts = moedl.moe_grouped_gemm_tiles(offd, cntd, Ms)
    ys = torch.empty((Ms, Ns), dtype=torch.int16, device=dev)
    s_tiles, s_gemm = _time_gemm(moedl, torch, xs, ws, ts, ys, offd, cntd, args.steps, args.warmup)

    # The vendor library on the regular form of the same problem: every expert given
    # M*k/G rows, so that hipBLASLt's batched product (torch.bmm, per-expert weights,
    # contiguous operands) can run it; this library's grouped GEMM on the same regular
    # layout beside it, interleaved.  The batched product has no ragged rows to handle,
    # so it is the reference for the grouped kernel's own bodies.
    E = (M * k) // G
    xb = xe[:G * E].view(torch.bfloat16).view(G, E, N)
    w_kn = wt.view(torch.bfloat16).transpose(1, 2).contiguous()
    yb = torch.empty((G, E, Nout), dtype=torch.bfloat16, device=dev)
    offr = torch.arange(0, G, device=dev, dtype=torch.int32) * E
    cntr = torch.full((G,), E, dtype=torch.int32, device=dev)
    tr = moedl.moe_grouped_gemm_tiles(offr, cntr, G * E)
    yr = torch.empty((G * E, Nout), dtype=torch.int16, device=dev)
    flops_r = 2.0 * G * E * N * Nout
    vend, lib_r = [], []
    for _ in range(3):
        vend.append(flops_r / (_time_calls(torch, [lambda: torch.bmm(xb, w_kn, out=yb)], 5)[0]
                               * 1e-6) / 1e12)
        lib_r.append(flops_r / (_time_gemm(moedl, torch, xe[:G * E], wt, tr, yr, offr, cntr, 5,
                                           1)[1] * 1e-6) / 1e12)
    del w_kn, yb, yr
    torch.cuda.synchronize()

    # a 2 GiB plain copy: calibrates the HBM byte counters of a profiled run of this leg
    from combine_dispatch_layout_amd import harness
    src = torch.empty(1 << 30, dtype=torch.int16, device=dev)
    dst = torch.empty_like(src)
    harness.copy(src, dst)
    torch.cuda.synchronize()
    del src, dst

    cpu = None if args.no_cpu else cpu_gemm_baseline(w, wt, Nout, 8192)

    wl_name = f"{w.name}-grouped-gemm-K{N}-N{Nout}"
    traffic = recorded_traffic("grouped_gemm", wl_name,
                               os.path.join(PROFILES, f"hbm_traffic_{wl_name}.txt"))
    res = {"metric": "grouped GEMM TFLOP/s over the per-expert layout (bf16 in/out, fp32 acc)",
           "value": round(tflops, 1), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": round((t_tiles + t_gemm) * 1e-3, 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "bf16 operands, f32 accumulation",
           "data": "synthetic",
           "config": {"workload": wl_name, "rows": M * k, "K": N, "Nout": Nout, "G": G},
           "roofline": {"bound": "mfma", "achieved": round(tflops, 1),
                        "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                        "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": traffic,
                        "min_hbm_bytes_per_launch": int(G * Nout * N * 2 + M * k * N * 2
                                                        + M * k * Nout * 2)},
           "cpu_baseline": cpu,
           "event_us": {"grouped_gemm_tiles": round(t_tiles, 2), "grouped_gemm": round(t_gemm, 2)},
           "regular_layout_reference": {
               "experts": G, "rows_per_expert": E, "K": N, "Nout": Nout,
               "vendor_batched_tflops": [round(v, 1) for v in vend],
               "grouped_gemm_tflops": [round(v, 1) for v in lib_r],
               "vendor": "torch.bmm (hipBLASLt), per-expert weights, contiguous operands"},
           "deepspeed_page_shape": {"experts": Gs, "tokens": Ms, "K": Ks, "Nout": Ns,
                                    "tiles_us": round(s_tiles, 2), "gemm_us": round(s_gemm, 2),
                                    "tflops": round(2.0 * Ms * Ks * Ns / (s_gemm * 1e-6) / 1e12, 2)}}
    print(json.dumps(res))


def bench_chain(args, w, dev):
    """One MoE layer in the order it runs, on the headline routing: moe_dispatch_layout,
    moe_dispatch, moe_grouped_gemm_tiles + moe_grouped_gemm (each expert's rows times its
    own [N, N] bf16 weights, so the expert outputs have the hidden size and are the
    combine's input, as the grouped-GEMM page places the GEMM between the two), and
    moe_combine.  Per-kernel event times in that order, and beside them the same
    dispatch and combine run back to back (identity experts), in the same process."""
    import torch
    from combine_dispatch_layout_amd import moedl
    M, N, G, k, B = w.M, w.N, w.G, w.k, w.B
    assert w.dtype == "bf16"
    idx = torch.from_numpy(w.topk_idx).to(dev)
    ebkt = torch.from_numpy(w.expert_bucket).to(dev)
    x = torch.from_numpy(w.x.view(np.int16)).to(dev)
    wts = torch.from_numpy(w.weights).to(dev)
    rows = M * k
    lay = moedl.alloc_layout(M, k, G, B, False, dev)
    xe = torch.empty((rows, N), dtype=torch.int16, device=dev)
    ye = torch.empty((rows, N), dtype=torch.int16, device=dev)
    y = torch.empty((M, N), dtype=torch.int16, device=dev)
    # expert weights N(0, 1/N): the outputs keep the inputs' scale
    gen = torch.Generator(device=dev).manual_seed(13)
    wt = torch.empty((G, N, N), dtype=torch.int16, device=dev)
    for e in range(G):
        wt[e] = (torch.randn((N, N), generator=gen, device=dev) * N ** -0.5).to(
            torch.bfloat16).view(torch.int16)
    moedl.moe_dispatch_layout(idx, ebkt, B, False, out=lay)
    tiles = moedl.moe_grouped_gemm_tiles(lay.expert_offset, lay.expert_count, rows)

    calls = [
        ("layout", lambda: moedl.moe_dispatch_layout(idx, ebkt, B, False, out=lay)),
        ("dispatch", lambda: moedl.moe_dispatch(x, lay.send_row, rows, out=xe)),
        ("gemm_tiles", lambda: moedl.moe_grouped_gemm_tiles(lay.expert_offset, lay.expert_count,
                                                             rows, out=tiles)),
        ("grouped_gemm", lambda: moedl.moe_grouped_gemm(xe, wt, tiles, y=ye)),
        ("combine", lambda: moedl.moe_combine(ye, wts, lay.slot, y=y)),
    ]
    y_flat = torch.empty_like(y)
    flat = [calls[0], calls[1],
            ("combine", lambda: moedl.moe_combine(xe, wts, lay.slot, y=y_flat))]

    def timed(seq, steps, warmup):
        for _ in range(max(1, warmup)):
            for _, c in seq:
                c()
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(seq) + 1)]
              for _ in range(steps)]
        t0 = time.perf_counter()
        for i in range(steps):
            ev[i][0].record(stream)
            for (_, c), e in zip(seq, ev[i][1:]):
                c()
                e.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        per = {n: float(np.mean([e[q].elapsed_time(e[q + 1]) for e in ev])) * 1e3
               for q, (n, _) in enumerate(seq)}
        return wall * 1e6 / steps, per

    # the same chain with the dispatch shape of two waves per token (moe_dispatch's
    # dedup flag selects it): after the GEMM's weight stream x is no longer in the
    # last-level cache, where that shape holds up better
    calls_2w = list(calls)
    calls_2w[1] = ("dispatch", lambda: moedl.moe_dispatch(x, lay.send_row, rows, out=xe,
                                                         dedup=True))
    us_step, per = timed(calls, args.steps, args.warmup)
    _, per_2w = timed(calls_2w, max(2, args.steps // 4), 1)
    _, per_flat = timed(flat, args.steps, args.warmup)
    for _, c in calls:  # the chain's outputs for the check below
        c()
    torch.cuda.synchronize()
    assert int(lay.status.item()) == 0

    # sanity on 8 sampled tokens: y[t] against float32 sums of the bf16 expert outputs
    # (each a float32 mat-vec rounded once to bf16), within two bf16 roundings of the
    # magnitude
    for t in range(0, M, M // 8):
        xt = x[t].view(torch.bfloat16).float()
        ref = torch.zeros(N, device=dev)
        mag = torch.zeros(N, device=dev)
        for j in range(k):
            o = (wt[int(idx[t, j])].view(torch.bfloat16).float() @ xt).to(torch.bfloat16).float()
            ref += float(wts[t, j]) * o
            mag += abs(float(wts[t, j])) * o.abs()
        got = y[t].view(torch.bfloat16).float()
        assert bool(((got - ref).abs() <= mag * 2.0 ** -6 + 1e-3).all().item()), "chain check"

    flops = 2.0 * rows * N * N
    gemm_tflops = flops / (per["grouped_gemm"] * 1e-6) / 1e12
    row_bytes = N * 2
    disp_bytes = (M + rows) * row_bytes
    comb_bytes = (rows + M) * row_bytes
    rates = {"dispatch_gbps": round(disp_bytes / (per["dispatch"] * 1e-6) / 1e9, 1),
             "combine_gbps": round(comb_bytes / (per["combine"] * 1e-6) / 1e9, 1),
             "grouped_gemm_tflops": round(gemm_tflops, 1)}
    rates_flat = {"dispatch_gbps": round(disp_bytes / (per_flat["dispatch"] * 1e-6) / 1e9, 1),
                  "combine_gbps": round(comb_bytes / (per_flat["combine"] * 1e-6) / 1e9, 1)}
    wl_name = f"{w.name}-chain-K{N}-N{N}"
    traffic = recorded_traffic("grouped_gemm", wl_name,
                               os.path.join(PROFILES, f"hbm_traffic_{wl_name}.txt"))

    # a 2 GiB plain copy: calibrates the HBM byte counters of a profiled run of this leg
    from combine_dispatch_layout_amd import harness
    src = torch.empty(1 << 30, dtype=torch.int16, device=dev)
    dst = torch.empty_like(src)
    harness.copy(src, dst)
    torch.cuda.synchronize()
    del src, dst

    cpu = None if args.no_cpu else cpu_chain_baseline(w, wt, lay)
    res = {"metric": "MoE layer step in order (layout, dispatch, grouped GEMM N->N, combine), "
                     "us per step, M=16384,N=7168,G=256,k=8",
           "value": round(us_step, 1), "unit": "us", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": round(us_step * 1e-3, 4),
           "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
           "dtype": "bf16 rows and weights, f32 accumulation", "data": "synthetic",
           "config": {"workload": wl_name, "M": M, "N": N, "G": G, "k": k, "B": B,
                      "rows": rows, "dedup": False},
           "event_us": {n: round(v, 2) for n, v in per.items()},
           "rates_in_chain": rates,
           "event_us_two_wave_dispatch": {n: round(v, 2) for n, v in per_2w.items()},
           "event_us_back_to_back": {n: round(v, 2) for n, v in per_flat.items()},
           "rates_back_to_back": rates_flat,
           "roofline": {"bound": "mfma", "kernel": "grouped_gemm", "achieved": round(gemm_tflops, 1),
                        "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                        "frac": round(gemm_tflops / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": traffic,
                        "min_hbm_bytes_per_launch": int(G * N * N * 2 + 2 * rows * N * 2),
                        "launch_us": round(per["grouped_gemm"], 2)},
           "cpu_baseline": cpu}
    print(json.dumps(res))


def bench_dispatch_x(args, dev):
    """moe_dispatch at one send-buffer size, 131,072 rows of N=7168 bf16 (1.88 GB),
    while the rows read grow: M=16384 tokens at k=8, 32768 at k=4, 65536 at k=2, 131072
    at k=1 (x from 235 MB to 1.88 GB), uniform distinct routing over G=256 experts, 8
    buckets.  Two calls per case: `auto` (dedup=0: the call picks k single-store waves
    while x fits the 256 MB Infinity Cache or k = 1, else two waves sharing a token's
    rows) and `two_waves` (dedup=1: always the shared shape).  Each launch follows a
    combine of the dispatched rows, as in the step."""
    import torch
    from combine_dispatch_layout_amd import moedl, workloads
    N, G, B, R = 7168, 256, 8, 131072
    rows = []
    for k in (8, 4, 2, 1):
        M = R // k
        rng = np.random.default_rng([1234, 90, k])
        idx = torch.from_numpy(workloads.uniform_topk(rng, M, G, k)).to(dev)
        ebkt = torch.from_numpy(workloads.contiguous_buckets(G, B)).to(dev)
        lay = moedl.moe_dispatch_layout(idx, ebkt, B, False)
        gen = torch.Generator(device=dev).manual_seed(k)
        x = torch.randn((M, N), generator=gen, device=dev).to(torch.bfloat16).view(torch.int16)
        wts = torch.full((M, k), 1.0 / k, dtype=torch.float32, device=dev)
        out = torch.empty((R, N), dtype=torch.int16, device=dev)
        y = torch.empty((M, N), dtype=torch.int16, device=dev)
        shapes = {"auto": False, "two_waves": True}
        for flag in shapes.values():  # warm-up
            moedl.moe_combine(out, wts, lay.slot, y=y)
            moedl.moe_dispatch(x, lay.send_row, R, out=out, dedup=flag)
        torch.cuda.synchronize()
        ev = {n: [] for n in shapes}
        for _ in range(max(4, args.steps // 10)):
            for n, flag in shapes.items():
                moedl.moe_combine(out, wts, lay.slot, y=y)
                s_, e_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                s_.record()
                moedl.moe_dispatch(x, lay.send_row, R, out=out, dedup=flag)
                e_.record()
                ev[n].append((s_, e_))
        torch.cuda.synchronize()
        st = lay.send_token
        samp = torch.randint(0, R, (1024,), device=dev)
        assert torch.equal(out[samp], x[st[samp].long()]), "dispatch check"
        alg = (M + R) * N * 2
        row = {"M": M, "k": k, "x_MB": round(M * N * 2 / 1e6), "send_MB": round(R * N * 2 / 1e6)}
        for n in shapes:
            us = float(np.median([s_.elapsed_time(e_) * 1e3 for s_, e_ in ev[n]]))
            row[f"{n}_us"] = round(us, 1)
            row[f"{n}_gbps"] = round(alg / us / 1e3, 1)
        rows.append(row)
        del out, x, y, lay, idx

    # a 2 GiB plain copy: calibrates the HBM byte counters of a profiled run of this leg
    from combine_dispatch_layout_amd import harness
    src = torch.empty(1 << 30, dtype=torch.int16, device=dev)
    dst = torch.empty_like(src)
    harness.copy(src, dst)
    torch.cuda.synchronize()
    del src, dst

    worst = rows[-1]
    cpu = None
    if not args.no_cpu:
        import oracle
        Ms = 8192
        w1 = workloads.make_custom(Ms, N, G, 1, B, seed=90)
        lay_o = oracle.dispatch_layout(w1.topk_idx, w1.expert_bucket, B, False)
        t0 = time.perf_counter()
        oracle.dispatch(w1.x, lay_o.send_row, lay_o.R)
        dt = time.perf_counter() - t0
        cpu = {"value": round(2 * Ms * N * 2 / dt / 1e9, 3), "unit": "GB/s", "cores": 1,
               "kind": "oracle",
               "sample": f"dispatch of {Ms} tokens at k=1 ({dt:.3f} s), {host_cores()}"}
    res = {"metric": "dispatch GB/s at a fixed 1.88 GB send buffer, x from 235 MB to 1.88 GB",
           "value": worst["auto_gbps"], "unit": "GB/s", "n_gpus": 1,
           "steps": max(4, args.steps // 10), "warmup": 1, "ms_per_step": round(worst["auto_us"] * 1e-3, 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "bf16 rows (byte copy)", "data": "synthetic",
           "config": {"workload": "uniform-N7168-send131072-rows", "G": G, "B": B, "rows": R},
           "cases": rows,
           "roofline": hbm_roofline("dispatch", (worst["M"] + R) * N * 2, worst["auto_us"]),
           "cpu_baseline": cpu}
    print(json.dumps(res))


def cpu_chain_baseline(w, wt, lay):
    """The oracle on a bounded sample of the chain: layout, dispatch and combine of the
    whole workload (single-threaded, as the flat leg), plus the oracle's grouped GEMM
    (float64 products, one BLAS thread) on 64 rows of the busiest expert, extrapolated
    to all rows by their FLOP count."""
    import oracle
    from threadpoolctl import threadpool_limits
    base = cpu_baseline(w, False)
    cnt = lay.expert_count.cpu().numpy()
    e = int(np.argmax(cnt))
    S = 64
    lay_o = oracle.dispatch_layout(w.topk_idx, w.expert_bucket, w.B, False)
    xe, _ = oracle.dispatch(w.x, lay_o.send_row, w.M * w.k)
    r0 = int(lay_o.expert_offset[e])
    x_s = np.ascontiguousarray(xe[r0:r0 + S])
    del xe
    w_s = wt[e:e + 1].cpu().numpy().view(np.uint16)
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        oracle.grouped_gemm(x_s, w_s, np.array([0]), np.array([S]))
        dt = time.perf_counter() - t0
    gemm_s = dt * (w.M * w.k) / S
    total = base["seconds"] + gemm_s
    return {"value": round(total * 1e6, 0), "unit": "us", "cores": 1, "kind": "oracle",
            "sample": (f"layout+dispatch+combine on all {w.M} tokens ({base['seconds']:.2f} s) "
                       f"plus the grouped GEMM on {S} rows of expert {e} ({dt:.2f} s), "
                       f"extrapolated by FLOP count to {w.M * w.k} rows ({gemm_s:.0f} s); "
                       f"{host_cores()}"),
            "seconds": round(total, 1)}


def cpu_gemm_baseline(w, wt, Nout: int, sample_rows: int):
    """The oracle's grouped GEMM (float64 products), one BLAS thread, on the first
    `sample_rows` rows of the per-expert layout.  Its inputs come from the oracle's own
    layout and dispatch of the host tokens; the weights of the experts those rows
    belong to are copied from the device tensor the GPU leg uses."""
    import oracle
    from threadpoolctl import threadpool_limits
    lay = oracle.dispatch_layout(w.topk_idx, w.expert_bucket, w.B, False)
    S = min(sample_rows, w.M * w.k)
    xe, _ = oracle.dispatch(w.x, lay.send_row, w.M * w.k)
    off = lay.expert_offset.astype(np.int64)
    cnt = np.clip(np.minimum(off + lay.expert_count, S) - off, 0, None)
    experts = np.nonzero(cnt)[0]
    x_s = np.ascontiguousarray(xe[:S])
    del xe
    w_s = wt[experts.tolist()].cpu().numpy().view(np.uint16)
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        oracle.grouped_gemm(x_s, w_s, off[experts], cnt[experts])
        dt = time.perf_counter() - t0
    return {"value": round(2.0 * S * w.N * Nout / dt / 1e12, 5), "unit": "TFLOP/s", "cores": 1,
            "kind": "oracle",
            "sample": (f"first {S} of {w.M * w.k} rows of the per-expert layout "
                       f"({len(experts)} experts), K={w.N}, Nout={Nout}, float64 products "
                       f"({dt:.2f} s), {host_cores()}"),
            "seconds": round(dt, 3)}


def graph_replay_us(torch, step, invocations=128, timed=8):
    """[PURLIN] section 5 method: `invocations` steps captured in one graph, one warm-up
    replay, `timed` timed replays; microseconds per step."""
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for _ in range(invocations):
            step()
    g.replay()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(timed):
        g.replay()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) * 1e3 / (invocations * timed)


def bench_small(args, dev):
    """Small batches (N=7168 bf16, G=256, top-8 uniform, 8 contiguous buckets, identity
    experts): a step is dispatch layout + row scatter + combine, either as three calls
    or with moe_layout_dispatch doing the first two in one launch."""
    import torch
    from combine_dispatch_layout_amd import moedl, workloads
    rows = []
    ms = [int(v) for v in args.small_m.split(",")]
    if not ms or min(ms) < 1 or max(ms) > 512:
        raise SystemExit("--small-m: token counts in 1..512")
    kern_us, kern_bytes = {}, {}
    for M in ms:
        w = workloads.make_workload(1, M=M)
        N, G, k, B = w.N, w.G, w.k, w.B
        idx = torch.from_numpy(w.topk_idx).to(dev)
        ebkt = torch.from_numpy(w.expert_bucket).to(dev)
        x = torch.from_numpy(w.x.view(np.int16)).to(dev)
        wts = torch.from_numpy(w.weights).to(dev)
        res = {"M": M}
        for dedup in (False, True):
            lay = moedl.alloc_layout(M, k, G, B, dedup, dev)
            cap = lay.capacity
            out = torch.empty((cap, N), dtype=torch.int16, device=dev)
            y = torch.empty((M, N), dtype=torch.int16, device=dev)
            eo = out
            if dedup:   # combine reads slot-indexed rows: expand once, untimed
                moedl.moe_layout_dispatch(idx, ebkt, B, True, x, lay=lay, out=out)
                eo, _ = moedl.moe_expand(out, lay.send_row, lay.slot, M * k)

            def three():
                moedl.moe_dispatch_layout(idx, ebkt, B, dedup, out=lay)
                moedl.moe_dispatch(x, lay.send_row, cap, out=out, dedup=dedup)
                moedl.moe_combine(eo, wts, lay.slot, y=y)

            def fused():
                moedl.moe_layout_dispatch(idx, ebkt, B, dedup, x, lay=lay, out=out)
                moedl.moe_combine(eo, wts, lay.slot, y=y)

            # the same two forms as prepared calls (arguments checked and marshalled
            # once): eager steps without the binding's per-call checks
            p_lay, _ = moedl.prepare_dispatch_layout(idx, ebkt, B, dedup, out=lay)
            p_disp, _, _ = moedl.prepare_dispatch(x, lay.send_row, cap, out=out, dedup=dedup)
            p_comb, _ = moedl.prepare_combine(eo, wts, lay.slot, y=y)
            p_fused, _, _, _ = moedl.prepare_layout_dispatch(idx, ebkt, B, dedup, x, lay=lay,
                                                             out=out)

            def three_prepared():
                p_lay()
                p_disp()
                p_comb()

            def fused_prepared():
                p_fused()
                p_comb()

            tag = "dedup" if dedup else "flat"
            for name, fn in (("three_calls", three), ("fused", fused),
                             ("three_calls_prepared", three_prepared),
                             ("fused_prepared", fused_prepared)):
                for _ in range(max(1, args.warmup)):
                    fn()
                torch.cuda.synchronize()
                t0 = time.perf_counter()
                for _ in range(args.steps):
                    fn()
                torch.cuda.synchronize()
                res[f"{tag}_{name}_eager_us"] = round((time.perf_counter() - t0) * 1e6 / args.steps, 2)
                res[f"{tag}_{name}_graph_us"] = round(graph_replay_us(torch, fn), 2)
                xz = torch.where(x == -32768, torch.zeros_like(x), x)
                assert bool((y == xz).all().item()), f"M={M} {tag} {name}: y != x"
            if M == ms[0] and not dedup:
                # duration of each kernel, for the roofline of whichever form is faster:
                # graph replay of the kernel alone (eager launches of a kernel this short
                # measure the host's launch rate, not the kernel)
                rb = w.row_bytes
                kern = {
                    "layout": (lambda: moedl.moe_dispatch_layout(idx, ebkt, B, False, out=lay),
                               4 * M * k * 4 + 3 * G * 4),
                    "dispatch": (lambda: moedl.moe_dispatch(x, lay.send_row, cap, out=out),
                                 (M + M * k) * rb),
                    "combine": (lambda: moedl.moe_combine(eo, wts, lay.slot, y=y),
                                (M * k + M) * N * 2),
                    "layout_dispatch": (lambda: moedl.moe_layout_dispatch(idx, ebkt, B, False, x,
                                                                          lay=lay, out=out),
                                        (M + M * k) * rb),
                }
                kern_us = {name: graph_replay_us(torch, fn) for name, (fn, _) in kern.items()}
                kern_bytes = {n: b for n, (_, b) in kern.items()}
        rows.append(res)
    head = rows[0]
    # the step is reported on the faster of its two forms; the roofline is that form's
    # longest kernel
    best = min(("three_calls", "fused"), key=lambda p: head[f"flat_{p}_graph_us"])
    members = ["layout", "dispatch", "combine"] if best == "three_calls" else ["layout_dispatch", "combine"]
    dom = max(members, key=lambda n: kern_us[n])
    # a 2 GiB plain copy: calibrates the HBM byte counters of a profiled run of this leg
    from combine_dispatch_layout_amd import harness
    src = torch.empty(1 << 30, dtype=torch.int16, device=dev)
    dst = torch.empty_like(src)
    harness.copy(src, dst)
    torch.cuda.synchronize()
    del src, dst
    traffic = recorded_traffic(dom, f"uniform-top8-M{head['M']}-small-path")
    roofline = hbm_roofline(dom, kern_bytes[dom], kern_us[dom], traffic=traffic, M=head["M"],
                            graph_us_per_kernel={n: round(v, 2) for n, v in kern_us.items()})
    cpu = None if args.no_cpu else cpu_small_baseline(workloads.make_workload(1, M=ms[0]))
    out = {"metric": "small-M layout+dispatch+combine latency (graph replay, us per step)",
           "value": head[f"flat_{best}_graph_us"], "unit": "us", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "higher_is_better": False, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16 rows, f32 accumulation", "data": "synthetic",
           "config": {"workload": "uniform-top8-N7168-G256-B8", "M": [r["M"] for r in rows],
                      "value_at": {"M": head["M"], "dedup": False, "form": best}},
           "roofline": roofline, "cpu_baseline": cpu, "rows": rows}
    print(json.dumps(out))


def cpu_small_baseline(w, seconds: float = 3.0):
    """The oracle's layout + dispatch + combine at the small workload's M, repeated for
    about `seconds`; microseconds per step, single-threaded."""
    import oracle
    n, t0 = 0, time.perf_counter()
    while True:
        lay = oracle.dispatch_layout(w.topk_idx, w.expert_bucket, w.B, False)
        sent, _ = oracle.dispatch(w.x, lay.send_row, lay.R)
        oracle.combine(sent, w.weights, lay.slot)
        n += 1
        dt = time.perf_counter() - t0
        if dt >= seconds:
            break
    return {"value": round(dt * 1e6 / n, 1), "unit": "us", "cores": 1, "kind": "oracle",
            "sample": (f"M={w.M} flat layout+dispatch+combine, {n} repetitions ({dt:.2f} s), "
                       f"{host_cores()}"),
            "seconds": round(dt, 3)}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the path has no multi-GPU part to measure)", file=sys.stderr)
        sys.exit(2)
    for var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
        os.environ[var] = "1"

    import torch
    from combine_dispatch_layout_amd import harness, moedl, workloads

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    moedl.load()
    dev = torch.device("cuda:0")
    dedup = bool(args.dedup)
    if args.path == "small":
        bench_small(args, dev)
        return
    if args.path == "dispatch-x":
        bench_dispatch_x(args, dev)
        return
    w = workloads.make_workload(args.cfg)
    if args.path == "bucket":
        bench_bucket(args, w, dev)
        return
    if args.path == "placement":
        bench_placement(args, w, dev)
        return
    if args.path == "gemm":
        bench_gemm(args, w, dev)
        return
    if args.path == "chain":
        bench_chain(args, w, dev)
        return

    M, N, G, k, B = w.M, w.N, w.G, w.k, w.B
    row_bytes = w.row_bytes
    fp8 = w.dtype == "fp8"

    idx = torch.from_numpy(w.topk_idx).to(dev)
    ebkt = torch.from_numpy(w.expert_bucket).to(dev)
    x = torch.from_numpy(w.x if fp8 else w.x.view(np.int16)).to(dev)
    xs = torch.from_numpy(w.x_scale).to(dev) if w.x_scale is not None else None
    wts = torch.from_numpy(w.weights).to(dev)
    lay = moedl.alloc_layout(M, k, G, B, dedup, dev)
    cap = lay.capacity
    out = torch.empty((cap, N), dtype=x.dtype, device=dev)
    out_scale = (torch.empty((cap, xs.shape[1]), dtype=torch.float32, device=dev)
                 if xs is not None else None)
    y = torch.empty((M, N), dtype=torch.int16, device=dev)
    # identity experts without dedup: combine reads the dispatched rows in place;
    # otherwise the stand-in expert step (untimed) writes slot-indexed bf16 outputs
    in_place = w.standin == "identity" and not dedup and not fp8
    eo = out if in_place else torch.empty((M * k, N), dtype=torch.int16, device=dev)
    slot_eo = lay.slot

    def step():
        moedl.moe_dispatch_layout(idx, ebkt, B, dedup, out=lay)
        moedl.moe_dispatch(x, lay.send_row, cap, x_scale=xs, out=out, out_scale=out_scale,
                           dedup=dedup)
        moedl.moe_combine(eo, wts, slot_eo, y=y)

    # ---- graph replay (128 invocations, 1 warm-up replay, 8 timed replays, / 1024).
    # It runs before the warm-up: ~1,150 steps of load, so the eager steps timed below
    # start after the power manager's clock dip at the start of a load (~15 ms), also
    # when the warm-up is short. The timed region itself is unchanged.
    # one untimed expert step so combine has real inputs
    step()
    if not in_place:
        harness.expert_outputs(w.standin, out, lay.send_row, lay.slot, idx, out_scale, out=eo)
    torch.cuda.synchronize()

    graph_us = None
    if not args.no_graph:
        try:
            g = torch.cuda.CUDAGraph()
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                step()
            torch.cuda.current_stream().wait_stream(side)
            torch.cuda.synchronize()
            with torch.cuda.graph(g):
                for _ in range(128):
                    step()
            g.replay()
            torch.cuda.synchronize()
            s, e_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record()
            for _ in range(8):
                g.replay()
            e_.record()
            torch.cuda.synchronize()
            graph_us = s.elapsed_time(e_) * 1e3 / 1024
            del g
        except Exception as exc:  # report, never hide: the eager figure stands alone
            print(f"graph replay skipped: {exc!r}", file=sys.stderr)

    # warm-up
    for _ in range(max(1, args.warmup)):
        step()
    torch.cuda.synchronize()
    R = int(lay.bucket_offset[B].item())
    assert int(lay.status.item()) == 0

    # algorithmic bytes: read x (and scales) once, write R send rows (and scales), read
    # M*k bf16 expert rows, write M bf16 rows
    scale_bytes = xs.shape[1] * 4 if xs is not None else 0
    disp_bytes = (M + R) * (row_bytes + scale_bytes)
    comb_bytes = (M * k + M) * N * 2
    total_bytes = disp_bytes + comb_bytes

    # ---- timed region: exactly `steps` steps; per-kernel HIP events on the same stream,
    # on a few evenly spaced steps (event_steps)
    stream = torch.cuda.current_stream()
    K = args.steps
    sampled = event_steps(K)
    ev = {i: [torch.cuda.Event(enable_timing=True) for _ in range(4)] for i in sampled}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        e = ev.get(i)
        if e is None:
            step()
            continue
        e[0].record(stream)
        moedl.moe_dispatch_layout(idx, ebkt, B, dedup, out=lay)
        e[1].record(stream)
        moedl.moe_dispatch(x, lay.send_row, cap, x_scale=xs, out=out, out_scale=out_scale,
                           dedup=dedup)
        e[2].record(stream)
        moedl.moe_combine(eo, wts, slot_eo, y=y)
        e[3].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    evs = list(ev.values())
    lay_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    disp_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    comb_ms = float(np.mean([e[2].elapsed_time(e[3]) for e in evs]))
    span_ms = float(np.mean([e[0].elapsed_time(e[3]) for e in evs]))
    ms_per_step = wall * 1e3 / K
    gbps = total_bytes / (ms_per_step * 1e-3) / 1e9

    # ---- plain copy ceiling (2 GiB, 16-byte non-temporal streaming copy)
    nbytes = 2 << 30
    src = torch.empty(nbytes // 2, dtype=torch.int16, device=dev)
    dst = torch.empty_like(src)
    harness.copy(src, dst)
    torch.cuda.synchronize()
    cs, ce = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    cs.record()
    for _ in range(10):
        harness.copy(src, dst)
    ce.record()
    torch.cuda.synchronize()
    copy_gbps = 2 * nbytes * 10 / (cs.elapsed_time(ce) * 1e-3) / 1e9
    dst.copy_(src)                      # device-to-device memcpy of the same 2 GiB
    torch.cuda.synchronize()
    cs.record()
    for _ in range(10):
        dst.copy_(src)
    ce.record()
    torch.cuda.synchronize()
    memcpy_gbps = 2 * nbytes * 10 / (cs.elapsed_time(ce) * 1e-3) / 1e9
    del src, dst

    # correctness guard on the timed buffers, closed forms of the stand-in experts
    # (weights of a token sum to one): identity y == x exactly; scaled experts
    # y ~ x * sum_j w_j (1 + e_j / 256) within two bf16 roundings; fp8 experts
    # y ~ dequant(x) * sum_j w_j within one rounding (sampled tokens)
    torch.cuda.synchronize()
    if w.standin == "identity":
        xz = torch.where(x == -32768, torch.zeros_like(x), x)
        assert bool((y == xz).all().item()), "combine output differs from the input rows"
    else:
        ts = torch.arange(0, M, 61, device=dev)
        wt = wts[ts].double()
        if w.standin == "scale":
            f = (wt * (1.0 + idx[ts].double() / 256.0)).sum(1, keepdim=True)
            ref = x[ts].view(torch.bfloat16).double() * f
            tol = 2.0 ** -7
        else:
            q = x[ts].cpu().view(torch.float8_e4m3fn).double()
            sc = xs[ts].cpu().double().repeat_interleave(128, dim=1)
            ref = (q * sc).to(dev) * wt.sum(1, keepdim=True)
            tol = 2.0 ** -8 * 1.001
        got = y[ts].view(torch.bfloat16).double()
        assert bool(((got - ref).abs() <= ref.abs() * tol + 1e-30).all().item()), \
            f"combine output off the {w.standin} closed form"

    # ---- roofline of the dominant kernel
    kernels = {"dispatch": (disp_ms, disp_bytes), "combine": (comb_ms, comb_bytes)}
    dom = max(kernels, key=lambda n: kernels[n][0])
    dms, dbytes = kernels[dom]
    achieved = dbytes / (dms * 1e-3) / 1e9
    traffic = recorded_traffic(dom, w.name + ("-dedup" if dedup else ""))
    roofline = {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                "traffic": traffic, "alg_bytes_per_launch": dbytes,
                "launch_us": round(dms * 1e3, 2)}

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(w, dedup, 16384 if in_place else 8192)

    res = {
        "metric": METRIC, "value": round(gbps, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": K, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": ("bf16 rows, f32 accumulation" if not fp8 else
                  "fp8_e4m3 rows + f32 scales, f32 accumulation, bf16 out"), "data": "synthetic",
        "config": {"workload": w.name + ("-dedup" if dedup else ""), "M": M, "N": N, "G": G,
                   "k": k, "B": B, "dtype": w.dtype, "experts": w.standin, "dedup": dedup,
                   "send_rows": R, "parallelism": "single-gpu"},
        "us_per_step": round(ms_per_step * 1e3, 2),
        "frac_of_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4),
        "alg_bytes_per_step": total_bytes,
        "event_us": {"layout": round(lay_ms * 1e3, 2), "dispatch": round(disp_ms * 1e3, 2),
                     "combine": round(comb_ms * 1e3, 2), "span": round(span_ms * 1e3, 2)},
        "event_steps": len(sampled),
        "kernel_gbps": {n: round(b / (t * 1e-3) / 1e9, 1) for n, (t, b) in kernels.items()},
        "graph_replay_us_per_step": None if graph_us is None else round(graph_us, 2),
        "graph_replay_gbps": None if graph_us is None else round(total_bytes / (graph_us * 1e-6) / 1e9, 1),
        "copy_ceiling_gbps": round(copy_gbps, 1),
        "memcpy_dtod_gbps": round(memcpy_gbps, 1),
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(res))


if __name__ == "__main__":
    main()
