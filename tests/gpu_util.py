"""Helpers for the GPU parity tests: run the HIP path through the C ABI, run the
oracle on the same seeded inputs (whole, or restricted to sampled tokens), and
compare element by element."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
from combine_dispatch_layout_amd import harness, moedl

LAYOUT_FIELDS = ("expert_count", "expert_offset", "bucket_count", "bucket_offset", "slot",
                 "send_row")
SENTINEL_BF16 = 0x7FA5          # a NaN pattern no dispatch ever writes
SENTINEL_FP8 = 0x7F


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy()


def rows_dev(w) -> torch.Tensor:
    return dev(w.x.view(np.int16)) if w.dtype == "bf16" else dev(w.x)


def as_u16(a: np.ndarray) -> np.ndarray:
    return a.view(np.uint16) if a.dtype == np.int16 else a


def gpu_layout(w, dedup: bool):
    return moedl.moe_dispatch_layout(dev(w.topk_idx), dev(w.expert_bucket), w.B, dedup)


def assert_layout_equal(lay, ref, ctx=""):
    torch.cuda.synchronize()
    st = int(lay.status.item())
    assert st == ref.status, (ctx, "status", st, ref.status)
    if ref.status:
        return
    for f in LAYOUT_FIELDS:
        got = host(getattr(lay, f))
        want = getattr(ref, f)
        if not np.array_equal(got, want):
            bad = np.flatnonzero(got.reshape(-1) != want.reshape(-1))
            raise AssertionError(f"{ctx}: {f} differs at {bad.size} positions, first "
                                 f"{bad[:5]}: got {got.reshape(-1)[bad[:5]]} want "
                                 f"{want.reshape(-1)[bad[:5]]}")
    R = ref.R
    assert np.array_equal(host(lay.send_token[:R]), ref.send_token), (ctx, "send_token")


def gpu_dispatch(w, lay, sentinel=True):
    x = rows_dev(w)
    cap = lay.capacity
    out = torch.empty((cap, w.N), dtype=x.dtype, device="cuda")
    if sentinel:
        out.fill_(SENTINEL_BF16 if w.dtype == "bf16" else SENTINEL_FP8)
    xs = dev(w.x_scale) if w.x_scale is not None else None
    out_scale = None
    if xs is not None:
        out_scale = torch.full((cap, xs.shape[1]), float("nan"), dtype=torch.float32,
                               device="cuda")
    moedl.moe_dispatch(x, lay.send_row, cap, xs, out=out, out_scale=out_scale, dedup=lay.dedup)
    return out, out_scale


def assert_dispatch_equal(w, out, out_scale, ref, chunk=8192, ctx=""):
    """Every send row r < R equals x[send_token[r]] (oracle's send_token) and rows
    >= R still hold the sentinel.  Compared in chunks to bound host memory."""
    torch.cuda.synchronize()
    R = ref.R
    for r0 in range(0, R, chunk):
        r1 = min(R, r0 + chunk)
        got = host(out[r0:r1])
        want = w.x[ref.send_token[r0:r1]]
        got = as_u16(got) if w.dtype == "bf16" else got
        if not np.array_equal(got, want):
            bad = r0 + np.flatnonzero((got != want).any(axis=1))
            raise AssertionError(f"{ctx}: {bad.size} dispatched rows differ, first {bad[:5]}")
        if out_scale is not None:
            assert np.array_equal(host(out_scale[r0:r1]), w.x_scale[ref.send_token[r0:r1]]), ctx
    if R < out.shape[0]:
        tail = out[R:]
        s = SENTINEL_BF16 if w.dtype == "bf16" else SENTINEL_FP8
        val = torch.tensor(s, dtype=torch.int32).to(out.dtype).item()
        assert bool((tail == val).all().item()), f"{ctx}: rows >= R were written"
        if out_scale is not None:
            assert bool(torch.isnan(out_scale[R:]).all().item()), ctx


def gpu_expert_outputs(w, lay, out, out_scale):
    if w.standin == "identity" and not lay.dedup:
        return out                                   # combine reads the send rows in place
    return harness.expert_outputs(w.standin, out, lay.send_row, lay.slot, dev(w.topk_idx),
                                  out_scale)


def gpu_combine(w, lay, eo):
    return moedl.moe_combine(eo, dev(w.weights), lay.slot)


def oracle_pipeline(w, dedup):
    ref = oracle.dispatch_layout(w.topk_idx, w.expert_bucket, w.B, dedup)
    sent, sent_scale = oracle.dispatch(w.x, ref.send_row, ref.R, w.x_scale)
    eo = oracle.expert_outputs(w.standin, sent, ref.send_row, ref.slot, w.topk_idx, sent_scale)
    y = oracle.combine(eo, w.weights, ref.slot)
    return ref, sent, sent_scale, eo, y


def oracle_combine_tokens(w, ref, tokens: np.ndarray) -> np.ndarray:
    """Oracle combine output for the given tokens only: the oracle's dispatch, stand-in
    and combine run on the sub-problem made of those tokens' send rows and slots,
    renumbered densely (the arithmetic per output element is unchanged)."""
    tokens = np.asarray(tokens)
    srow = ref.send_row[tokens]
    slot = ref.slot[tokens]
    u_rows, srow_local = np.unique(srow, return_inverse=True)
    srow_local = srow_local.reshape(srow.shape)
    sent_tok = ref.send_token[u_rows]
    sent = w.x[sent_tok]
    sent_scale = w.x_scale[sent_tok] if w.x_scale is not None else None
    slot_local = np.arange(slot.size).reshape(slot.shape)
    eo = oracle.expert_outputs(w.standin, sent, srow_local, slot_local, w.topk_idx[tokens],
                               sent_scale)
    return oracle.combine(eo, w.weights[tokens], slot_local)


def assert_bits_equal(got: np.ndarray, want: np.ndarray, ctx=""):
    got = as_u16(got)
    if np.array_equal(got, want):
        return
    bad = np.argwhere(got != want)
    t, i = bad[0]
    raise AssertionError(f"{ctx}: {len(bad)} elements differ; first at token {t} element "
                         f"{i}: got {got[t, i]:#06x} want {want[t, i]:#06x}")
