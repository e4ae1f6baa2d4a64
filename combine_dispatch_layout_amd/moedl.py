"""Thin Python binding over libmoedl (include/moe_dispatch.h).

Argument marshalling only: every step of the path runs in the library's HIP kernels.
torch is used for device memory and streams -- tensors' data pointers and the
current HIP stream are passed straight through.  Output tensors are allocated here
when the caller does not pass them.  There is no fallback: if the shared library is
missing, every call raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoedl.so")

MOE_OK = 0
MOE_BF16 = 0
MOE_FP8_E4M3 = 1
MAX_EXPERTS = 1024
MAX_TOPK = 16
MAX_BUCKETS = 64
SCALE_BLOCK = 128

_lib: Optional[ctypes.CDLL] = None

_i32p = ctypes.c_void_p
_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32

# name -> (restype, argtypes), mirroring include/moe_dispatch.h
SIGNATURES = {
    "moe_abi_version": (ctypes.c_int32, []),
    "moe_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "moe_dispatch_layout_workspace_bytes": (ctypes.c_size_t, [_i64, _i32, _i32, _i32]),
    "moe_dispatch_layout": (ctypes.c_int, [
        _i32p, _i64, _i32, _i32p, _i32, _i32, _i32, _i32p, _i32p, _i32p, _i32p, _i32p,
        _i32p, _i32p, _i32p, _vp, ctypes.c_size_t, _vp]),
    "moe_dispatch_layout_noalloc": (ctypes.c_int, [
        _i32p, _i64, _i32, _i32p, _i32, _i32, _i32, _i32p, _i32p, _i32p, _i32p, _i32p,
        _i32p, _i32p, _i32p, _vp]),
    "moe_dispatch": (ctypes.c_int, [
        _vp, ctypes.c_int, _i64, _i32, _vp, _i32p, _i32, _i32, _vp, _vp, _i64, _vp]),
    "moe_layout_dispatch": (ctypes.c_int, [
        _i32p, _i64, _i32, _i32p, _i32, _i32, _i32, _vp, ctypes.c_int, _i32, _vp, _i32p, _i32p,
        _i32p, _i32p, _i32p, _i32p, _i32p, _i32p, _vp, _vp, _i64, _vp]),
    "moe_combine": (ctypes.c_int, [_vp, _i64, _vp, _i32p, _i64, _i32, _i32, _vp, _vp]),
    "moe_expand": (ctypes.c_int, [
        _vp, ctypes.c_int, _i64, _i32, _vp, _i32p, _i32p, _i64, _i32, _vp, _vp, _i64, _vp]),
    "moe_combine_partial": (ctypes.c_int, [
        _vp, _i64, _vp, _i32p, _i32p, _i64, _i32, _i32, _vp, _i64, _vp]),
    "moe_combine_reduce": (ctypes.c_int, [_vp, _i64, _i32p, _i64, _i32, _i32, _vp, _vp]),
    "moe_expert_pair_counts": (ctypes.c_int, [_i32p, _i64, _i32, _i32, _i32p, _vp]),
    "moe_place_experts": (ctypes.c_int, [_vp, _i32, _i32, _vp]),
    "moe_grouped_gemm_max_tiles": (ctypes.c_int32, [_i64, _i32, _i32]),
    "moe_grouped_gemm_tiles": (ctypes.c_int, [
        _i32p, _i32p, _i32, _i32, _i32p, _i32p, _i32p, _i32, _i32p, _vp]),
    "moe_grouped_gemm": (ctypes.c_int, [
        _vp, _i64, _i32, _vp, _i32, _i32, _i32p, _i32p, _i32p, _i32, _vp, _vp]),
}

GEMM_TILE_M = 256


class MoeError(RuntimeError):
    def __init__(self, call: str, status: int):
        self.status = status
        msg = lib().moe_status_string(status).decode() if _lib is not None else str(status)
        super().__init__(f"{call} failed: status {status} ({msg})")


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libmoedl.so (built by combine_dispatch_layout_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: run `python -m combine_dispatch_layout_amd.build`")
        lib_ = ctypes.CDLL(path)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib_, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib_
    return _lib


def lib() -> ctypes.CDLL:
    return load()


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors passed to libmoedl must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors passed to libmoedl must be contiguous")
    return t.data_ptr() if t.numel() > 0 else None


_I32 = (torch.int32,)
_F32 = (torch.float32,)
_ROW16 = (torch.bfloat16, torch.int16, torch.uint16)


def _want(t: Optional[torch.Tensor], name: str, dtypes, min_numel: int, cols: int = 0) -> None:
    """Sizes reach the library separately from the tensors, so a tensor the kernels
    index must hold at least min_numel elements of an accepted dtype (and, for row
    buffers, `cols` columns), or the call is refused before any pointer is passed."""
    if t is None:
        return
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype}, expected one of {[str(d) for d in dtypes]}")
    if cols and (t.dim() != 2 or t.shape[1] != cols):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected [rows, {cols}]")
    if t.numel() < min_numel:
        raise ValueError(f"{name}: {t.numel()} elements, the call needs {min_numel}")


def _row_dtypes(x: torch.Tensor):
    """Row buffers of one call share the element size of x."""
    return _ROW16 if _dtype_code(x) == MOE_BF16 else (torch.uint8, torch.float8_e4m3fn)


def _check_layout(lay: "Layout", M: int, k: int, G: int, B: int, dedup: bool) -> None:
    _want(lay.expert_count, "expert_count", _I32, G)
    _want(lay.expert_offset, "expert_offset", _I32, G)
    _want(lay.bucket_count, "bucket_count", _I32, B)
    _want(lay.bucket_offset, "bucket_offset", _I32, B + 1)
    _want(lay.slot, "slot", _I32, M * k)
    _want(lay.send_row, "send_row", _I32, M * k)
    _want(lay.send_token, "send_token", _I32, send_capacity(M, k, B, dedup))
    _want(lay.status, "status", _I32, 1)


# torch's current HIP stream of a device as a raw handle: the accessor torch's own
# extensions use (~0.1 us), falling back to the public call (~2.7 us per call).
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(stream, like: Optional[torch.Tensor] = None) -> int:
    """The stream to launch on: `stream` if given, else the current stream of the
    device of `like` (a tensor argument of the call)."""
    if stream is None:
        if _raw_stream is not None and like is not None and like.is_cuda:
            return _raw_stream(like.get_device())
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _check(call: str, status: int) -> None:
    if status != MOE_OK:
        raise MoeError(call, status)


def workspace_bytes(M: int, k: int, G: int, B: int) -> int:
    return int(lib().moe_dispatch_layout_workspace_bytes(M, k, G, B))


@dataclass
class Layout:
    expert_count: torch.Tensor   # int32 [G]
    expert_offset: torch.Tensor  # int32 [G]
    bucket_count: torch.Tensor   # int32 [B]
    bucket_offset: torch.Tensor  # int32 [B+1]
    slot: torch.Tensor           # int32 [M, k]
    send_row: torch.Tensor       # int32 [M, k]
    send_token: torch.Tensor     # int32 [capacity]
    status: torch.Tensor         # int32 [1]
    workspace: torch.Tensor      # uint8 scratch
    dedup: bool

    @property
    def capacity(self) -> int:
        return self.send_token.numel()


def send_capacity(M: int, k: int, B: int, dedup: bool) -> int:
    """Rows the send buffer needs, known on the host: M*k, or M*min(k, B) with dedup."""
    return M * (min(k, B) if dedup else k)


def alloc_layout(M: int, k: int, G: int, B: int, dedup: bool, device="cuda") -> Layout:
    i32 = dict(dtype=torch.int32, device=device)
    return Layout(
        expert_count=torch.empty(G, **i32), expert_offset=torch.empty(G, **i32),
        bucket_count=torch.empty(B, **i32), bucket_offset=torch.empty(B + 1, **i32),
        slot=torch.empty((M, k), **i32), send_row=torch.empty((M, k), **i32),
        send_token=torch.empty(send_capacity(M, k, B, dedup), **i32),
        status=torch.empty(1, **i32),
        # zero-filled once: the layout's counters start at zero and every call
        # leaves them there
        workspace=torch.zeros(max(1, workspace_bytes(M, k, G, B)), dtype=torch.uint8,
                              device=device),
        dedup=dedup)


def _layout_tensors(lay: "Layout") -> tuple:
    return (lay.expert_count, lay.expert_offset, lay.bucket_count, lay.bucket_offset, lay.slot,
            lay.send_row, lay.send_token, lay.status, lay.workspace)


def _dispatch_layout_args(topk_idx, expert_bucket, B, dedup, out):
    """Checked arguments of moe_dispatch_layout (all but the stream), the tensors they
    point into, and the Layout."""
    M, k = topk_idx.shape
    G = expert_bucket.shape[0]
    if topk_idx.dtype != torch.int32 or expert_bucket.dtype != torch.int32:
        raise TypeError("topk_idx and expert_bucket must be int32")
    if out is None:
        lay = alloc_layout(M, k, G, B, dedup, topk_idx.device)
    else:
        lay = out
        _check_layout(lay, M, k, G, B, dedup)
    args = (_ptr(topk_idx), M, k, _ptr(expert_bucket), G, B, int(dedup), _ptr(lay.expert_count),
            _ptr(lay.expert_offset), _ptr(lay.bucket_count), _ptr(lay.bucket_offset),
            _ptr(lay.slot), _ptr(lay.send_row), _ptr(lay.send_token), _ptr(lay.status),
            _ptr(lay.workspace), lay.workspace.numel())
    return args, (topk_idx, expert_bucket) + _layout_tensors(lay), lay


def moe_dispatch_layout(topk_idx: torch.Tensor, expert_bucket: torch.Tensor, B: int,
                        dedup: bool, out: Optional[Layout] = None, stream=None) -> Layout:
    """topk_idx int32 [M, k], expert_bucket int32 [G] -> Layout (device tensors)."""
    args, _, lay = _dispatch_layout_args(topk_idx, expert_bucket, B, dedup, out)
    _check("moe_dispatch_layout", lib().moe_dispatch_layout(*args, _stream(stream, topk_idx)))
    return lay


LAYOUT_SCRATCH_BYTES = 4 << 20  # the library's static workspace per GPU


def _dispatch_layout_noalloc_args(topk_idx, expert_bucket, B, dedup, out):
    M, k = topk_idx.shape
    G = expert_bucket.shape[0]
    if topk_idx.dtype != torch.int32 or expert_bucket.dtype != torch.int32:
        raise TypeError("topk_idx and expert_bucket must be int32")
    if out is None:
        i32 = dict(dtype=torch.int32, device=topk_idx.device)
        lay = Layout(
            expert_count=torch.empty(G, **i32), expert_offset=torch.empty(G, **i32),
            bucket_count=torch.empty(B, **i32), bucket_offset=torch.empty(B + 1, **i32),
            slot=torch.empty((M, k), **i32), send_row=torch.empty((M, k), **i32),
            send_token=torch.empty(send_capacity(M, k, B, dedup), **i32),
            status=torch.empty(1, **i32),
            workspace=torch.empty(0, dtype=torch.uint8, device=topk_idx.device), dedup=dedup)
    else:
        lay = out
        _check_layout(lay, M, k, G, B, dedup)
    args = (_ptr(topk_idx), M, k, _ptr(expert_bucket), G, B, int(dedup), _ptr(lay.expert_count),
            _ptr(lay.expert_offset), _ptr(lay.bucket_count), _ptr(lay.bucket_offset),
            _ptr(lay.slot), _ptr(lay.send_row), _ptr(lay.send_token), _ptr(lay.status))
    return args, (topk_idx, expert_bucket) + _layout_tensors(lay), lay


def moe_dispatch_layout_noalloc(topk_idx: torch.Tensor, expert_bucket: torch.Tensor, B: int,
                                dedup: bool, out: Optional[Layout] = None,
                                stream=None) -> Layout:
    """moe_dispatch_layout with the library's static workspace (no workspace buffer).
    The Layout's workspace field is an empty tensor."""
    args, _, lay = _dispatch_layout_noalloc_args(topk_idx, expert_bucket, B, dedup, out)
    _check("moe_dispatch_layout_noalloc",
           lib().moe_dispatch_layout_noalloc(*args, _stream(stream, topk_idx)))
    return lay


def _dtype_code(x: torch.Tensor) -> int:
    if x.dtype in (torch.bfloat16, torch.int16, torch.uint16):
        return MOE_BF16
    if x.dtype in (torch.uint8, torch.float8_e4m3fn):
        return MOE_FP8_E4M3
    raise TypeError(f"unsupported row dtype {x.dtype}")


def _dispatch_args(x, send_row, out_rows, x_scale, out, out_scale, dedup):
    M, N = x.shape
    k = send_row.shape[1] if send_row.dim() == 2 else 1
    if out is None:
        out = torch.empty((out_rows, N), dtype=x.dtype, device=x.device)
    if x_scale is not None and out_scale is None:
        out_scale = torch.empty((out_rows, x_scale.shape[1]), dtype=torch.float32,
                                device=x.device)
    sc = N // SCALE_BLOCK
    _want(send_row, "send_row", _I32, M * k)
    _want(out, "out", _row_dtypes(x), out_rows * N, cols=N)
    _want(x_scale, "x_scale", _F32, M * sc)
    _want(out_scale, "out_scale", _F32, out_rows * sc)
    args = (_ptr(x), _dtype_code(x), M, N, _ptr(x_scale), _ptr(send_row), k, int(dedup),
            _ptr(out), _ptr(out_scale), out_rows)
    return args, (x, send_row, x_scale, out, out_scale), out, out_scale


def moe_dispatch(x: torch.Tensor, send_row: torch.Tensor, out_rows: int,
                 x_scale: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                 out_scale: Optional[torch.Tensor] = None, dedup: bool = False, stream=None):
    """x [M, N] (bf16 bits or fp8 codes), send_row int32 [M, k] -> (out [out_rows, N],
    out_scale [out_rows, N/128] or None).  dedup: send_row came from a dedup layout
    (selects the kernel shape only)."""
    args, _, out, out_scale = _dispatch_args(x, send_row, out_rows, x_scale, out, out_scale,
                                             dedup)
    _check("moe_dispatch", lib().moe_dispatch(*args, _stream(stream, x)))
    return out, out_scale


FUSED_MAX_TOKENS = 512


def _layout_dispatch_args(topk_idx, expert_bucket, B, dedup, x, x_scale, lay, out, out_scale):
    M, k = topk_idx.shape
    G = expert_bucket.shape[0]
    N = x.shape[1]
    if topk_idx.dtype != torch.int32 or expert_bucket.dtype != torch.int32:
        raise TypeError("topk_idx and expert_bucket must be int32")
    if lay is None:
        lay = alloc_layout(M, k, G, B, dedup, topk_idx.device)
    else:
        _check_layout(lay, M, k, G, B, dedup)
    rows = lay.capacity
    if out is None:
        out = torch.empty((rows, N), dtype=x.dtype, device=x.device)
    if x_scale is not None and out_scale is None:
        out_scale = torch.empty((rows, x_scale.shape[1]), dtype=torch.float32, device=x.device)
    sc = N // SCALE_BLOCK
    # M comes from topk_idx, and the kernel reads M rows of x
    _want(x, "x", _row_dtypes(x), M * N, cols=N)
    _want(out, "out", _row_dtypes(x), 0, cols=N)
    _want(x_scale, "x_scale", _F32, M * sc)
    _want(out_scale, "out_scale", _F32, out.shape[0] * sc)
    args = (_ptr(topk_idx), M, k, _ptr(expert_bucket), G, B, int(dedup), _ptr(x), _dtype_code(x),
            N, _ptr(x_scale), _ptr(lay.expert_count), _ptr(lay.expert_offset),
            _ptr(lay.bucket_count), _ptr(lay.bucket_offset), _ptr(lay.slot), _ptr(lay.send_row),
            _ptr(lay.send_token), _ptr(lay.status), _ptr(out), _ptr(out_scale), out.shape[0])
    keep = (topk_idx, expert_bucket, x, x_scale, out, out_scale) + _layout_tensors(lay)
    return args, keep, lay, out, out_scale


def moe_layout_dispatch(topk_idx: torch.Tensor, expert_bucket: torch.Tensor, B: int,
                        dedup: bool, x: torch.Tensor, x_scale: Optional[torch.Tensor] = None,
                        lay: Optional[Layout] = None, out: Optional[torch.Tensor] = None,
                        out_scale: Optional[torch.Tensor] = None, stream=None):
    """moe_dispatch_layout + moe_dispatch in one launch (M <= 512) -> (Layout, out,
    out_scale).  The Layout's workspace is not used."""
    args, _, lay, out, out_scale = _layout_dispatch_args(topk_idx, expert_bucket, B, dedup, x,
                                                         x_scale, lay, out, out_scale)
    _check("moe_layout_dispatch", lib().moe_layout_dispatch(*args, _stream(stream, topk_idx)))
    return lay, out, out_scale


def _combine_args(expert_out, weights, slot, y):
    rows, N = expert_out.shape
    M, k = slot.shape
    _want(expert_out, "expert_out", _ROW16, 0)
    _want(weights, "weights", _F32, M * k)
    _want(slot, "slot", _I32, M * k)
    if y is None:
        y = torch.empty((M, N), dtype=expert_out.dtype, device=expert_out.device)
    _want(y, "y", _ROW16, M * N, cols=N)
    args = (_ptr(expert_out), rows, _ptr(weights), _ptr(slot), M, k, N, _ptr(y))
    return args, (expert_out, weights, slot, y), y


def moe_combine(expert_out: torch.Tensor, weights: torch.Tensor, slot: torch.Tensor,
                y: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """expert_out bf16 [rows, N], weights fp32 [M, k], slot int32 [M, k] -> y bf16 [M, N]."""
    args, _, y = _combine_args(expert_out, weights, slot, y)
    _check("moe_combine", lib().moe_combine(*args, _stream(stream, slot)))
    return y


class Prepared:
    """One library call whose arguments were checked and marshalled once, for loops
    that repeat a call on the same buffers (a serving step at small M spends more
    time in the binding than on the GPU).  It holds references to every tensor it was
    built from, so their storage, and the device pointers taken from it, stay valid
    while it lives.  Calling it launches on the stream given when it was prepared,
    else on the current stream of the tensors' device, and raises MoeError on an error
    status.  The tensors' contents may change between calls; for other tensors or
    sizes, prepare a new call."""

    __slots__ = ("_name", "_fn", "_args", "_dev", "_stream", "_keep")

    def __init__(self, name: str, args: tuple, like: torch.Tensor, keep: tuple, stream):
        self._name = name
        self._fn = getattr(lib(), name)
        self._args = args
        self._dev = like.get_device()
        self._stream = None if stream is None else _stream(stream)
        self._keep = keep

    def __call__(self) -> None:
        s = self._stream
        if s is None:
            s = (_raw_stream(self._dev) if _raw_stream is not None
                 else torch.cuda.current_stream(self._dev).cuda_stream)
        st = self._fn(*self._args, s)
        if st != MOE_OK:
            raise MoeError(self._name, st)


def prepare_dispatch_layout(topk_idx: torch.Tensor, expert_bucket: torch.Tensor, B: int,
                            dedup: bool, out: Optional[Layout] = None, stream=None):
    """moe_dispatch_layout as a Prepared call -> (Prepared, Layout).  Nothing is
    launched until the Prepared is called."""
    args, keep, lay = _dispatch_layout_args(topk_idx, expert_bucket, B, dedup, out)
    return Prepared("moe_dispatch_layout", args, topk_idx, keep, stream), lay


def prepare_dispatch_layout_noalloc(topk_idx: torch.Tensor, expert_bucket: torch.Tensor,
                                    B: int, dedup: bool, out: Optional[Layout] = None,
                                    stream=None):
    """moe_dispatch_layout_noalloc as a Prepared call -> (Prepared, Layout): nothing is
    allocated when it is called."""
    args, keep, lay = _dispatch_layout_noalloc_args(topk_idx, expert_bucket, B, dedup, out)
    return Prepared("moe_dispatch_layout_noalloc", args, topk_idx, keep, stream), lay


def prepare_dispatch(x: torch.Tensor, send_row: torch.Tensor, out_rows: int,
                     x_scale: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                     out_scale: Optional[torch.Tensor] = None, dedup: bool = False,
                     stream=None):
    """moe_dispatch as a Prepared call -> (Prepared, out, out_scale)."""
    args, keep, out, out_scale = _dispatch_args(x, send_row, out_rows, x_scale, out, out_scale,
                                                dedup)
    return Prepared("moe_dispatch", args, x, keep, stream), out, out_scale


def prepare_layout_dispatch(topk_idx: torch.Tensor, expert_bucket: torch.Tensor, B: int,
                            dedup: bool, x: torch.Tensor, x_scale: Optional[torch.Tensor] = None,
                            lay: Optional[Layout] = None, out: Optional[torch.Tensor] = None,
                            out_scale: Optional[torch.Tensor] = None, stream=None):
    """moe_layout_dispatch as a Prepared call -> (Prepared, Layout, out, out_scale)."""
    args, keep, lay, out, out_scale = _layout_dispatch_args(topk_idx, expert_bucket, B, dedup, x,
                                                            x_scale, lay, out, out_scale)
    return Prepared("moe_layout_dispatch", args, topk_idx, keep, stream), lay, out, out_scale


def prepare_combine(expert_out: torch.Tensor, weights: torch.Tensor, slot: torch.Tensor,
                    y: Optional[torch.Tensor] = None, stream=None):
    """moe_combine as a Prepared call -> (Prepared, y)."""
    args, keep, y = _combine_args(expert_out, weights, slot, y)
    return Prepared("moe_combine", args, slot, keep, stream), y


def moe_expand(recv: torch.Tensor, send_row: torch.Tensor, slot: torch.Tensor, expert_rows: int,
               recv_scale: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
               out_scale: Optional[torch.Tensor] = None, stream=None):
    """Receiver-side expansion: out[slot[t, j]] = recv[send_row[t, j]] (+ scales)."""
    R, N = recv.shape
    M, k = slot.shape
    if out is None:
        out = torch.empty((expert_rows, N), dtype=recv.dtype, device=recv.device)
    if recv_scale is not None and out_scale is None:
        out_scale = torch.empty((expert_rows, recv_scale.shape[1]), dtype=torch.float32,
                                device=recv.device)
    sc = N // SCALE_BLOCK
    _want(send_row, "send_row", _I32, M * k)
    _want(slot, "slot", _I32, M * k)
    _want(out, "out", _row_dtypes(recv), expert_rows * N, cols=N)
    _want(recv_scale, "recv_scale", _F32, R * sc)
    _want(out_scale, "out_scale", _F32, expert_rows * sc)
    st = lib().moe_expand(_ptr(recv), _dtype_code(recv), R, N, _ptr(recv_scale), _ptr(send_row),
                          _ptr(slot), M, k, _ptr(out), _ptr(out_scale), expert_rows,
                          _stream(stream, slot))
    _check("moe_expand", st)
    return out, out_scale


def moe_combine_partial(expert_out: torch.Tensor, weights: torch.Tensor, slot: torch.Tensor,
                        send_row: torch.Tensor, partial_rows: int,
                        partial: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Per-(token, bucket) partial sums, bf16 [partial_rows, N]."""
    rows, N = expert_out.shape
    M, k = slot.shape
    _want(expert_out, "expert_out", _ROW16, 0)
    _want(weights, "weights", _F32, M * k)
    _want(slot, "slot", _I32, M * k)
    _want(send_row, "send_row", _I32, M * k)
    if partial is None:
        partial = torch.empty((partial_rows, N), dtype=expert_out.dtype, device=expert_out.device)
    _want(partial, "partial", _ROW16, partial_rows * N, cols=N)
    st = lib().moe_combine_partial(_ptr(expert_out), rows, _ptr(weights), _ptr(slot),
                                   _ptr(send_row), M, k, N, _ptr(partial), partial_rows,
                                   _stream(stream, slot))
    _check("moe_combine_partial", st)
    return partial


def moe_combine_reduce(partial: torch.Tensor, send_row: torch.Tensor,
                       y: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """y[t] = bf16(sum of the token's distinct partial rows, ascending)."""
    rows, N = partial.shape
    M, k = send_row.shape
    _want(partial, "partial", _ROW16, 0)
    _want(send_row, "send_row", _I32, M * k)
    if y is None:
        y = torch.empty((M, N), dtype=partial.dtype, device=partial.device)
    _want(y, "y", _ROW16, M * N, cols=N)
    st = lib().moe_combine_reduce(_ptr(partial), rows, _ptr(send_row), M, k, N, _ptr(y),
                                  _stream(stream, send_row))
    _check("moe_combine_reduce", st)
    return y


def moe_expert_pair_counts(topk_idx: torch.Tensor, G: int, out: Optional[torch.Tensor] = None,
                           stream=None) -> torch.Tensor:
    """Expert pair co-occurrence counts, int32 [G, G] on the device."""
    M, k = topk_idx.shape
    _want(topk_idx, "topk_idx", _I32, M * k)
    if out is None:
        out = torch.empty((G, G), dtype=torch.int32, device=topk_idx.device)
    _want(out, "pair_counts", _I32, G * G)
    st = lib().moe_expert_pair_counts(_ptr(topk_idx), M, k, G, _ptr(out), _stream(stream, topk_idx))
    _check("moe_expert_pair_counts", st)
    return out


def moe_place_experts(pair_counts, B: int):
    """Greedy expert -> bucket placement on the host.  pair_counts: int32 [G, G]
    (numpy array or tensor, copied to host).  Returns a numpy int32 [G] map."""
    import numpy as np
    C = pair_counts.cpu().numpy() if isinstance(pair_counts, torch.Tensor) else pair_counts
    C = np.ascontiguousarray(C, dtype=np.int32)
    if C.ndim != 2 or C.shape[0] != C.shape[1]:
        raise ValueError(f"pair_counts: shape {C.shape}, expected [G, G]")
    G = C.shape[0]
    out = np.empty(G, dtype=np.int32)
    st = lib().moe_place_experts(C.ctypes.data, G, B, out.ctypes.data)
    _check("moe_place_experts", st)
    return out


@dataclass
class GemmTiles:
    expert: torch.Tensor     # int32 [max_tiles], -1 past the last tile
    row0: torch.Tensor       # int32 [max_tiles]
    rows: torch.Tensor       # int32 [max_tiles]
    num_tiles: torch.Tensor  # int32 [1]

    @property
    def max_tiles(self) -> int:
        return self.expert.numel()


def _check_tiles(t: GemmTiles) -> None:
    _want(t.expert, "tile_expert", _I32, 0)
    _want(t.row0, "tile_row0", _I32, t.max_tiles)
    _want(t.rows, "tile_rows", _I32, t.max_tiles)
    _want(t.num_tiles, "num_tiles", _I32, 1)


def moe_grouped_gemm_tiles(expert_offset: torch.Tensor, expert_count: torch.Tensor, rows: int,
                           tile_m: int = GEMM_TILE_M, out: Optional[GemmTiles] = None,
                           stream=None) -> GemmTiles:
    """Row tiles of each expert's run, built on the device (no host sync)."""
    G = expert_count.numel()
    _want(expert_count, "expert_count", _I32, G)
    _want(expert_offset, "expert_offset", _I32, G)
    if out is None:
        mt = int(lib().moe_grouped_gemm_max_tiles(rows, G, tile_m))
        i32 = dict(dtype=torch.int32, device=expert_count.device)
        out = GemmTiles(torch.empty(mt, **i32), torch.empty(mt, **i32), torch.empty(mt, **i32),
                        torch.empty(1, **i32))
    _check_tiles(out)
    st = lib().moe_grouped_gemm_tiles(_ptr(expert_offset), _ptr(expert_count), G, tile_m,
                                      _ptr(out.expert), _ptr(out.row0), _ptr(out.rows),
                                      out.max_tiles, _ptr(out.num_tiles), _stream(stream, expert_count))
    _check("moe_grouped_gemm_tiles", st)
    return out


def moe_grouped_gemm(x: torch.Tensor, w: torch.Tensor, tiles: GemmTiles,
                     y: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """y = per-expert x @ w[e].T (bf16 bits in and out, fp32 accumulation)."""
    rows, K = x.shape
    G, Nout, Kw = w.shape
    if Kw != K:
        raise ValueError(f"w: shape {tuple(w.shape)}, expected [G, Nout, {K}]")
    _want(x, "x", _ROW16, 0)
    _want(w, "w", _ROW16, 0)
    _check_tiles(tiles)
    if y is None:
        y = torch.empty((rows, Nout), dtype=x.dtype, device=x.device)
    _want(y, "y", _ROW16, rows * Nout, cols=Nout)
    st = lib().moe_grouped_gemm(_ptr(x), rows, K, _ptr(w), G, Nout, _ptr(tiles.expert),
                                _ptr(tiles.row0), _ptr(tiles.rows), tiles.max_tiles, _ptr(y),
                                _stream(stream, y))
    _check("moe_grouped_gemm", st)
    return y
