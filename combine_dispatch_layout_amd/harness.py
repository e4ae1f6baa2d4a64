"""Binding of libmoedl_harness (include/moe_harness.h): expert stand-ins and a plain
streaming copy.  These sit beside the dispatch/combine path -- tests use the
stand-ins to produce combine inputs, the bench uses the copy as a bandwidth and
traffic-counter reference.  Neither is part of the path."""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoedl_harness.so")

STANDIN = {"identity": 0, "scale": 1, "dequant": 2}
_lib = None


def load() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: run `python -m combine_dispatch_layout_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        v, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
        lib.moe_harness_expert_outputs.restype = ctypes.c_int
        lib.moe_harness_expert_outputs.argtypes = [i32, v, v, i64, i32, v, v, v, i64, i32, v, i64, v]
        lib.moe_harness_copy.restype = ctypes.c_int
        lib.moe_harness_copy.argtypes = [v, v, ctypes.c_size_t, v]
        _lib = lib
    return _lib


def _p(t):
    return None if t is None or t.numel() == 0 else t.data_ptr()


def expert_outputs(kind: str, sent: torch.Tensor, send_row: torch.Tensor, slot: torch.Tensor,
                   topk_idx: torch.Tensor, sent_scale: Optional[torch.Tensor] = None,
                   out: Optional[torch.Tensor] = None) -> torch.Tensor:
    M, k = slot.shape
    N = sent.shape[1]
    if out is None:
        out = torch.empty((M * k, N), dtype=torch.int16, device=sent.device)
    st = load().moe_harness_expert_outputs(
        STANDIN[kind], _p(sent), _p(sent_scale), sent.shape[0], N, _p(send_row), _p(slot),
        _p(topk_idx), M, k, _p(out), out.shape[0], torch.cuda.current_stream().cuda_stream)
    if st != 0:
        raise RuntimeError(f"moe_harness_expert_outputs failed: {st}")
    return out


def copy(src: torch.Tensor, dst: torch.Tensor, stream=None) -> None:
    nbytes = src.numel() * src.element_size()
    s = torch.cuda.current_stream().cuda_stream if stream is None else stream.cuda_stream
    st = load().moe_harness_copy(_p(src), _p(dst), nbytes, s)
    if st != 0:
        raise RuntimeError(f"moe_harness_copy failed: {st}")
