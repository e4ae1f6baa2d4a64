"""Build libmoedl.so and libmoedl_harness.so in-tree with hipcc for gfx950.

Run as ``python -m combine_dispatch_layout_amd.build``.  Every call recompiles.
Objects go to ``_build/`` at the repository root; the shared libraries land next to
this file, where the binding loads them.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++20", "-fPIC", "-Wall",
    "-Wno-unused-command-line-argument",
    # no packed fp32 instructions anywhere in the library
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # combine's fp32 op order is part of its definition: never fuse multiply-add
    "-ffp-contract=off",
    "-I", INCLUDE, "-I", CSRC,
]

# Per-source additions.  layout.hip: no atomic optimizer.  It would turn the one-lane
# fetch-add with which a layout tile leaves into a wave reduction that waits for the
# returned value at once; the kernel issues that atomic early and reads the value only
# at its end, so that the round trip overlaps the rest of the tile's work.  (Every other
# atomic there on a wave-uniform address is on an error path.)
EXTRA = {
    "layout.hip": ["-mllvm", "-amdgpu-atomic-optimizer-strategy=None"],
}

LIBS = {
    "libmoedl.so": ["api.cpp", "layout.hip", "noalloc.hip", "dispatch.hip", "combine.hip",
                    "bucket.hip", "placement.hip", "gemm.hip"],
    "libmoedl_harness.so": ["harness.hip"],
}


def _run(cmd: list[str]) -> None:
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "is not a recognized feature for this target" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if out.strip():
        print(out, file=sys.stderr)


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    _run([HIPCC, "-x", "hip", *COMMON, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src),
          "-o", obj])
    return obj


def build(verbose: bool = False) -> dict[str, str]:
    """Compile every source and link both libraries; returns {name: path}."""
    if not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted({s for v in LIBS.values() for s in v})
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = dict(zip(srcs, ex.map(_compile, srcs)))
    out = {}
    for lib, parts in LIBS.items():
        tmp = os.path.join(BUILD, lib)
        _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp,
              *[objs[s] for s in parts]])
        dst = os.path.join(PKG, lib)
        shutil.copyfile(tmp, dst + ".tmp")
        os.replace(dst + ".tmp", dst)
        out[lib] = dst
        if verbose:
            print(f"built {dst}")
    return out


if __name__ == "__main__":
    build(verbose=True)
