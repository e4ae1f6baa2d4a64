"""Host-side checks of the C ABI (no GPU needed, no kernel is launched).

* libmoedl.so / libmoedl_harness.so load and export every function declared in
  include/*.h.
* The workspace query and the synchronous argument checks return the documented
  status codes.  Every call here is rejected before any HIP call; pointers are
  fake non-null values that are never dereferenced.
"""
import ctypes
import os
import re

import pytest

from combine_dispatch_layout_amd import moedl, harness

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3
P = 1 << 20            # fake, 16-byte aligned, never dereferenced


def declared(header):
    text = open(os.path.join(ROOT, "include", header)).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def test_headers_declare_the_three_calls():
    names = declared("moe_dispatch.h")
    for n in ("moe_dispatch_layout", "moe_dispatch", "moe_combine",
              "moe_dispatch_layout_workspace_bytes"):
        assert n in names


@pytest.mark.parametrize("header,loader", [("moe_dispatch.h", moedl.load),
                                           ("moe_harness.h", harness.load)])
def test_library_exports_every_declared_symbol(header, loader):
    lib = loader()
    for name in declared(header):
        assert hasattr(lib, name), name
    assert moedl.SIGNATURES.keys() >= set(declared("moe_dispatch.h"))


def test_version_and_strings():
    lib = moedl.load()
    assert lib.moe_abi_version() == 3
    assert lib.moe_status_string(0) == b"ok"
    assert lib.moe_status_string(3) == b"workspace too small"


def test_workspace_query():
    lib = moedl.load()
    assert lib.moe_dispatch_layout_workspace_bytes(16384, 8, 256, 8) > 64 * 256 * 4
    assert lib.moe_dispatch_layout_workspace_bytes(0, 8, 256, 8) > 0
    assert lib.moe_dispatch_layout_workspace_bytes(-1, 8, 256, 8) == 0
    assert lib.moe_dispatch_layout_workspace_bytes(10, 8, 4096, 8) == 0
    # grows with M
    assert (lib.moe_dispatch_layout_workspace_bytes(1 << 20, 8, 256, 8) >
            lib.moe_dispatch_layout_workspace_bytes(1 << 10, 8, 256, 8))


def layout_call(M=64, k=8, G=256, B=8, dedup=0, ptr=P, idx=P, ws=P, ws_bytes=1 << 30):
    lib = moedl.load()
    return lib.moe_dispatch_layout(idx, M, k, ptr, G, B, dedup, ptr, ptr, ptr, ptr, ptr, ptr,
                                   ptr, ptr, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(M=-1), INVALID), (dict(k=0), INVALID), (dict(G=0), INVALID), (dict(B=0), INVALID),
    (dict(k=9, G=8), INVALID), (dict(dedup=2), INVALID), (dict(ptr=None), INVALID),
    (dict(idx=None), INVALID), (dict(ws=None), INVALID), (dict(ws=P + 4), INVALID),
    (dict(G=1025), UNSUPPORTED), (dict(k=17, G=64), UNSUPPORTED), (dict(B=65), UNSUPPORTED),
    (dict(M=1 << 28, k=8), UNSUPPORTED), (dict(ws_bytes=16), WORKSPACE),
])
def test_layout_argument_errors(kw, status):
    assert layout_call(**kw) == status


def dispatch_call(x=P, dtype=0, M=64, N=7168, xs=None, sr=P, k=8, dd=0, out=P, os_=None, rows=512):
    return moedl.load().moe_dispatch(x, dtype, M, N, xs, sr, k, dd, out, os_, rows, None)


@pytest.mark.parametrize("kw,status", [
    (dict(M=-1), INVALID), (dict(N=0), INVALID), (dict(k=0), INVALID), (dict(rows=-1), INVALID),
    (dict(dtype=7), INVALID), (dict(x=None), INVALID), (dict(sr=None), INVALID),
    (dict(dd=2), INVALID),
    (dict(out=None), INVALID), (dict(x=P + 8), INVALID), (dict(out=P + 2), INVALID),
    (dict(xs=P), INVALID),                          # scales without out_scale
    (dict(xs=P, os_=P), INVALID),                   # scales with bf16
    (dict(k=17), UNSUPPORTED), (dict(N=7164), UNSUPPORTED),     # 14328 B rows
    (dict(dtype=1, N=7160), UNSUPPORTED),                        # fp8 rows of 7160 B
    (dict(dtype=1, N=7184, xs=P, os_=P), UNSUPPORTED),           # scales, N % 128 != 0
])
def test_dispatch_argument_errors(kw, status):
    assert dispatch_call(**kw) == status


def combine_call(eo=P, rows=512, w=P, slot=P, M=64, k=8, N=7168, y=P):
    return moedl.load().moe_combine(eo, rows, w, slot, M, k, N, y, None)


@pytest.mark.parametrize("kw,status", [
    (dict(M=-1), INVALID), (dict(N=0), INVALID), (dict(k=0), INVALID), (dict(rows=-1), INVALID),
    (dict(eo=None), INVALID), (dict(w=None), INVALID), (dict(slot=None), INVALID),
    (dict(y=None), INVALID), (dict(eo=P + 2), INVALID), (dict(y=P + 8), INVALID),
    (dict(k=17), UNSUPPORTED), (dict(N=7164), UNSUPPORTED),
])
def test_combine_argument_errors(kw, status):
    assert combine_call(**kw) == status


def test_harness_argument_errors():
    lib = harness.load()
    assert lib.moe_harness_copy(P, P, 15, None) == 1
    assert lib.moe_harness_copy(P + 4, P, 16, None) == 1
    assert lib.moe_harness_copy(P, P, 0, None) == 0
    assert lib.moe_harness_expert_outputs(5, P, None, 1, 128, P, P, P, 1, 1, P, 1, None) == 1


def expand_call(recv=P, dtype=0, R=512, N=7168, rs=None, sr=P, sl=P, M=64, k=8, ein=P, es=None,
                rows=512):
    return moedl.load().moe_expand(recv, dtype, R, N, rs, sr, sl, M, k, ein, es, rows, None)


@pytest.mark.parametrize("kw,status", [
    (dict(M=-1), INVALID), (dict(N=0), INVALID), (dict(k=0), INVALID), (dict(R=-1), INVALID),
    (dict(rows=-1), INVALID), (dict(dtype=3), INVALID), (dict(recv=None), INVALID),
    (dict(sr=None), INVALID), (dict(sl=None), INVALID), (dict(ein=None), INVALID),
    (dict(recv=P + 4), INVALID), (dict(rs=P), INVALID), (dict(rs=P, es=P), INVALID),
    (dict(k=17), UNSUPPORTED), (dict(N=7164), UNSUPPORTED),
    (dict(dtype=1, N=7184, rs=P, es=P), UNSUPPORTED),
])
def test_expand_argument_errors(kw, status):
    assert expand_call(**kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(M=-1), INVALID), (dict(k=0), INVALID), (dict(rows=-1), INVALID), (dict(prow=-1), INVALID),
    (dict(w=None), INVALID), (dict(sr=None), INVALID), (dict(part=None), INVALID),
    (dict(eo=P + 2), INVALID), (dict(k=17), UNSUPPORTED), (dict(N=100), UNSUPPORTED),
])
def test_combine_partial_argument_errors(kw, status):
    a = dict(eo=P, rows=512, w=P, slot=P, sr=P, M=64, k=8, N=7168, part=P, prow=512)
    a.update(kw)
    lib = moedl.load()
    assert lib.moe_combine_partial(a["eo"], a["rows"], a["w"], a["slot"], a["sr"], a["M"], a["k"],
                                   a["N"], a["part"], a["prow"], None) == status


@pytest.mark.parametrize("kw,status", [
    (dict(M=-1), INVALID), (dict(k=0), INVALID), (dict(prow=-1), INVALID), (dict(part=None), INVALID),
    (dict(sr=None), INVALID), (dict(y=None), INVALID), (dict(y=P + 8), INVALID),
    (dict(k=17), UNSUPPORTED), (dict(N=7164), UNSUPPORTED),
])
def test_combine_reduce_argument_errors(kw, status):
    a = dict(part=P, prow=512, sr=P, M=64, k=8, N=7168, y=P)
    a.update(kw)
    lib = moedl.load()
    assert lib.moe_combine_reduce(a["part"], a["prow"], a["sr"], a["M"], a["k"], a["N"], a["y"],
                                  None) == status


def test_grouped_gemm_max_tiles():
    lib = moedl.load()
    assert lib.moe_grouped_gemm_max_tiles(131072, 256, 128) == 1024 + 256
    assert lib.moe_grouped_gemm_max_tiles(0, 8, 128) == 8
    assert lib.moe_grouped_gemm_max_tiles(1, 8, 128) == 9
    assert lib.moe_grouped_gemm_max_tiles(-1, 8, 128) == 0
    assert lib.moe_grouped_gemm_max_tiles(10, 0, 128) == 0
    assert lib.moe_grouped_gemm_max_tiles(10, 8, 0) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(off=None), INVALID), (dict(cnt=None), INVALID), (dict(num=None), INVALID),
    (dict(G=0), INVALID), (dict(tm=0), INVALID), (dict(mt=-1), INVALID),
    (dict(te=None), INVALID), (dict(tr=None), INVALID), (dict(tn=None), INVALID),
    (dict(G=1025), UNSUPPORTED),
])
def test_grouped_gemm_tiles_argument_errors(kw, status):
    a = dict(off=P, cnt=P, G=256, tm=128, te=P, tr=P, tn=P, mt=1280, num=P)
    a.update(kw)
    lib = moedl.load()
    assert lib.moe_grouped_gemm_tiles(a["off"], a["cnt"], a["G"], a["tm"], a["te"], a["tr"],
                                      a["tn"], a["mt"], a["num"], None) == status


@pytest.mark.parametrize("kw,status", [
    (dict(rows=-1), INVALID), (dict(K=0), INVALID), (dict(G=0), INVALID), (dict(Nout=0), INVALID),
    (dict(mt=-1), INVALID), (dict(w=None), INVALID), (dict(te=None), INVALID),
    (dict(x=None), INVALID), (dict(y=None), INVALID), (dict(x=P + 2), INVALID),
    (dict(w=P + 8), INVALID), (dict(K=7160), UNSUPPORTED), (dict(Nout=2000), UNSUPPORTED),
    (dict(K=1 << 23), UNSUPPORTED), (dict(K=1 << 22), UNSUPPORTED),  # 256-row tile offsets
    (dict(mt=1 << 21, Nout=1024), UNSUPPORTED), (dict(rows=0, x=None, y=None), OK),
])
def test_grouped_gemm_argument_errors(kw, status):
    a = dict(x=P, rows=512, K=7168, w=P, G=256, Nout=2048, te=P, tr=P, tn=P, mt=260, y=P)
    a.update(kw)
    lib = moedl.load()
    assert lib.moe_grouped_gemm(a["x"], a["rows"], a["K"], a["w"], a["G"], a["Nout"], a["te"],
                                a["tr"], a["tn"], a["mt"], a["y"], None) == status


def fused_call(idx=P, M=64, k=8, eb=P, G=256, B=8, dd=0, x=P, dtype=0, N=7168, xs=None, o=P,
               st=P, out=P, os_=None, rows=512):
    return moedl.load().moe_layout_dispatch(idx, M, k, eb, G, B, dd, x, dtype, N, xs, o, o, o, o,
                                            o, o, o, st, out, os_, rows, None)


@pytest.mark.parametrize("kw,status", [
    (dict(M=-1), INVALID), (dict(k=0), INVALID), (dict(k=9, G=8), INVALID), (dict(N=0), INVALID),
    (dict(rows=-1), INVALID), (dict(dd=2), INVALID), (dict(dtype=2), INVALID),
    (dict(idx=None), INVALID), (dict(eb=None), INVALID), (dict(o=None), INVALID),
    (dict(st=None), INVALID), (dict(x=None), INVALID), (dict(out=None), INVALID),
    (dict(x=P + 4), INVALID), (dict(out=P + 8), INVALID), (dict(xs=P), INVALID),
    (dict(xs=P, os_=P), INVALID), (dict(M=513), UNSUPPORTED), (dict(k=17, G=64), UNSUPPORTED),
    (dict(G=1025), UNSUPPORTED), (dict(B=65), UNSUPPORTED), (dict(N=7164), UNSUPPORTED),
    (dict(dtype=1, N=7184, xs=P, os_=P), UNSUPPORTED),
])
def test_layout_dispatch_argument_errors(kw, status):
    assert fused_call(**kw) == status


def test_noalloc_layout_argument_errors():
    """The no-allocation layout call checks like moe_dispatch_layout, and refuses sizes
    whose workspace exceeds its static array, all before any HIP call."""
    lib = moedl.load()

    def call(M=100, k=8, G=256, B=8, dedup=0, idx=P, ptr=P):
        return lib.moe_dispatch_layout_noalloc(idx, M, k, ptr, G, B, dedup, ptr, ptr, ptr, ptr,
                                               ptr, ptr, ptr, ptr, None)

    assert call(M=-1) == INVALID
    assert call(k=0) == INVALID
    assert call(k=9, G=8) == INVALID
    assert call(dedup=2) == INVALID
    assert call(G=2048) == UNSUPPORTED
    assert call(idx=None) == INVALID
    assert moedl.workspace_bytes(1 << 20, 8, 1024, 64) > moedl.LAYOUT_SCRATCH_BYTES
    assert call(M=1 << 20, G=1024, B=64) == WORKSPACE
