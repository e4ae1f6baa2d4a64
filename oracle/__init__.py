"""CPU oracle for MoE dispatch layout, dispatch and combine -- TEST INFRASTRUCTURE ONLY.

This package is a plain, slow, obviously correct host implementation of what the HIP
library computes.  It is used by ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` and by nothing else: the product path never
imports it and has no CPU fallback.  It shares no code with the HIP library and
imports nothing from the product package.

Sources (web pages, cited by title and section):

* "All2all performance comparison between Triton-distributed and DeepEP"
  (Triton-distributed issue 117), sections "Test Code Snippet" and "Benchmark
  Configuration": a send buffer grouped by destination, per-destination splits and
  their cumulative sums, optional per-row scales, hidden size, experts per rank and
  total experts; dispatch and combine as the two phases.
* "Zyphra says routing-pattern expert placement speeds MoE token communication up to
  2.63x on AMD MI300X": a (token, destination) pair travels as one copy even when several
  of the token's experts sit at that destination (dedup mode), under an arbitrary expert placement.
* "Add Triton grouped-GEMM for MoE experts on Ampere/Ada" (DeepSpeed PR 8180),
  "What this PR does": per-expert row offsets ``offs`` that stay on the device.
* "Purlin: Separating Orchestration from the Datapath of Collectives", section 3.3
  (The Atom, SCORE): one owner per output element and accumulation in source order,
  which fixes combine's floating-point operation order; section 3.1 (Layouts): the
  send buffer is a scattered-V layout indexed by destination.

Modules: ``numerics`` (bf16 / fp8 e4m3 codecs), ``layout`` (counts, offsets, slot
map, dedup rows), ``dispatch`` (row scatter), ``combine`` (weighted top-k sum),
``bucket_combine`` (receiver-side expansion of dedup rows, per-(token, bucket)
pre-reduced combine), ``placement`` (expert pair co-occurrence counts and the greedy
correlation-aware expert -> bucket placement), ``grouped_gemm`` (the expert GEMM over
the per-expert layout and its tile metadata), ``standins`` (expert stand-ins used between dispatch and
combine in tests).

Parity pins: every function here is pinned in ``tests/test_oracle_*.py`` against
something other than itself (library codecs, brute-force enumeration, invariants,
closed forms and exact step-by-step evaluation).  No function is parity-unpinned.
"""
from .numerics import (bf16_to_f32, f32_to_bf16_rne, e4m3_to_f32, f32_to_e4m3_rne_sat)
from .layout import Layout, dispatch_layout, dispatch_layout_loops
from .dispatch import dispatch
from .combine import combine
from .standins import expert_outputs
from .bucket_combine import expand, combine_partial, combine_reduce
from .placement import pair_counts, greedy_clusters, greedy_place
from .grouped_gemm import gemm_tiles, grouped_gemm

__all__ = [
    "bf16_to_f32", "f32_to_bf16_rne", "e4m3_to_f32", "f32_to_e4m3_rne_sat",
    "Layout", "dispatch_layout", "dispatch_layout_loops", "dispatch", "combine",
    "expert_outputs", "expand", "combine_partial", "combine_reduce",
    "pair_counts", "greedy_clusters", "greedy_place", "gemm_tiles", "grouped_gemm",
]
