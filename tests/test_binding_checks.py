"""The Python binding refuses tensors too small, of the wrong dtype or of the wrong row
width for the sizes it passes to the library, before any pointer leaves Python (CPU:
these checks run before the device check, so CPU tensors reach them)."""
import numpy as np
import pytest
import torch

from combine_dispatch_layout_amd import moedl

i32 = dict(dtype=torch.int32)


def _raises(exc, match, fn, *a, **kw):
    with pytest.raises(exc, match=match):
        fn(*a, **kw)


def test_layout_fields(built_lib):
    M, k, G, B = 10, 4, 16, 2
    idx = torch.zeros((M, k), **i32)
    ebkt = torch.zeros(G, **i32)
    lay = moedl.alloc_layout(M, k, G, B, False, device="cpu")
    lay.slot = torch.empty(M * k - 1, **i32)
    _raises(ValueError, "slot: 39 elements, the call needs 40", moedl.moe_dispatch_layout,
            idx, ebkt, B, False, out=lay)
    lay = moedl.alloc_layout(M, k, G, B, False, device="cpu")      # dedup-sized send_token
    _raises(ValueError, "send_token", moedl.moe_dispatch_layout, idx, ebkt, B, False,
            out=moedl.alloc_layout(M, k, G, B, True, device="cpu"))
    lay.bucket_offset = torch.empty(B, **i32)
    _raises(ValueError, "bucket_offset", moedl.moe_dispatch_layout, idx, ebkt, B, False, out=lay)
    lay = moedl.alloc_layout(M, k, G, B, False, device="cpu")
    lay.expert_count = torch.empty(G, dtype=torch.int64)
    _raises(TypeError, "expert_count: dtype torch.int64", moedl.moe_dispatch_layout, idx, ebkt,
            B, False, out=lay)


def test_dispatch_buffers(built_lib):
    M, N, k = 6, 256, 3
    x = torch.zeros((M, N), dtype=torch.int16)
    send_row = torch.zeros((M, k), **i32)
    _raises(ValueError, "out: shape", moedl.moe_dispatch, x, send_row, M * k,
            out=torch.empty((M * k, N + 8), dtype=torch.int16))
    _raises(ValueError, "out: 256 elements", moedl.moe_dispatch, x, send_row, M * k,
            out=torch.empty((1, N), dtype=torch.int16))
    _raises(TypeError, "out: dtype torch.uint8", moedl.moe_dispatch, x, send_row, M * k,
            out=torch.empty((M * k, N), dtype=torch.uint8))
    _raises(ValueError, "send_row: 15 elements", moedl.moe_dispatch, x,
            torch.zeros((M - 1, k), **i32), M * k)
    x8 = torch.zeros((M, N), dtype=torch.uint8)
    xs = torch.zeros((M, N // 128), dtype=torch.float32)
    _raises(ValueError, "out_scale: 2 elements", moedl.moe_dispatch, x8, send_row, M * k,
            x_scale=xs, out=torch.empty((M * k, N), dtype=torch.uint8),
            out_scale=torch.empty((1, 2), dtype=torch.float32))
    _raises(ValueError, "x_scale", moedl.moe_dispatch, x8, send_row, M * k,
            x_scale=xs[:2])


def test_layout_dispatch_rows_of_x(built_lib):
    """The one-launch layout + dispatch takes M from topk_idx and reads M rows of x, so
    an x with fewer rows is refused before any pointer is passed."""
    M, N, k, G, B = 6, 256, 2, 16, 2
    idx = torch.zeros((M, k), **i32)
    ebkt = torch.zeros(G, **i32)
    _raises(ValueError, "x: 256 elements, the call needs 1536", moedl.moe_layout_dispatch,
            idx, ebkt, B, False, torch.zeros((1, N), dtype=torch.int16))
    _raises(ValueError, "x: 768 elements", moedl.moe_layout_dispatch, idx, ebkt, B, True,
            torch.zeros((3, N), dtype=torch.uint8))
    # the right number of rows reaches the device check
    _raises(ValueError, "must live on the GPU", moedl.moe_layout_dispatch, idx, ebkt, B,
            False, torch.zeros((M, N), dtype=torch.int16))


def test_combine_and_return_path(built_lib):
    M, k, N, rows = 5, 4, 64, 20
    eo = torch.zeros((rows, N), dtype=torch.int16)
    w = torch.zeros((M, k), dtype=torch.float32)
    slot = torch.zeros((M, k), **i32)
    _raises(TypeError, "weights: dtype torch.float64", moedl.moe_combine, eo, w.double(), slot)
    _raises(ValueError, "weights: 16 elements", moedl.moe_combine, eo, w[:4], slot)
    _raises(ValueError, "y: shape", moedl.moe_combine, eo, w, slot,
            y=torch.empty((M, N // 2), dtype=torch.int16))
    _raises(TypeError, "expert_out: dtype torch.float32", moedl.moe_combine, eo.float(), w, slot)
    send_row = torch.zeros((M, k), **i32)
    _raises(ValueError, "out: 64 elements", moedl.moe_expand, eo, send_row, slot, rows,
            out=torch.empty((1, N), dtype=torch.int16))
    _raises(ValueError, "send_row: 12 elements", moedl.moe_expand, eo,
            torch.zeros((3, k), **i32), slot, rows)
    _raises(ValueError, "partial: 64 elements", moedl.moe_combine_partial, eo, w, slot,
            send_row, 10, partial=torch.empty((1, N), dtype=torch.int16))
    _raises(ValueError, "y: 64 elements", moedl.moe_combine_reduce, eo, send_row,
            y=torch.empty((1, N), dtype=torch.int16))


def test_placement_and_gemm(built_lib):
    idx = torch.zeros((4, 2), **i32)
    _raises(ValueError, "pair_counts: 15 elements", moedl.moe_expert_pair_counts, idx, 4,
            out=torch.empty(15, **i32))
    _raises(ValueError, "pair_counts: shape", moedl.moe_place_experts,
            np.zeros((4, 5), dtype=np.int32), 2)
    x = torch.zeros((10, 64), dtype=torch.int16)
    w = torch.zeros((2, 128, 64), dtype=torch.int16)
    t = moedl.GemmTiles(torch.full((3,), -1, **i32), torch.zeros(2, **i32),
                        torch.zeros(3, **i32), torch.zeros(1, **i32))
    _raises(ValueError, "tile_row0: 2 elements", moedl.moe_grouped_gemm, x, w, t)
    t.row0 = torch.zeros(3, **i32)
    _raises(ValueError, r"w: shape \(2, 128, 32\)", moedl.moe_grouped_gemm, x, w[:, :, :32], t)
    _raises(ValueError, "y: shape", moedl.moe_grouped_gemm, x, w, t,
            y=torch.empty((10, 64), dtype=torch.int16))
    _raises(ValueError, "tile_rows", moedl.moe_grouped_gemm_tiles, torch.zeros(2, **i32),
            torch.zeros(2, **i32), 10,
            out=moedl.GemmTiles(torch.zeros(4, **i32), torch.zeros(4, **i32),
                                torch.zeros(3, **i32), torch.zeros(1, **i32)))


def test_right_sizes_reach_the_device_check(built_lib):
    """With every size right, the next refusal is the device check: the size checks do
    not reject valid calls."""
    M, N, k = 6, 256, 3
    x = torch.zeros((M, N), dtype=torch.int16)
    _raises(ValueError, "must live on the GPU", moedl.moe_dispatch, x,
            torch.zeros((M, k), **i32), M * k)
    _raises(ValueError, "must live on the GPU", moedl.moe_combine,
            torch.zeros((M * k, N), dtype=torch.int16), torch.zeros((M, k)),
            torch.zeros((M, k), **i32))


def test_prepared_calls_check_like_the_calls(built_lib):
    """prepare_* run the checks of the immediate calls when they are built, and the
    device check after them; nothing is launched while preparing."""
    M, k, G, B, N = 10, 4, 16, 2, 256
    idx = torch.zeros((M, k), **i32)
    ebkt = torch.zeros(G, **i32)
    lay = moedl.alloc_layout(M, k, G, B, False, device="cpu")
    lay.slot = torch.empty(M * k - 1, **i32)
    _raises(ValueError, "slot: 39 elements, the call needs 40", moedl.prepare_dispatch_layout,
            idx, ebkt, B, False, out=lay)
    _raises(ValueError, "must live on the GPU", moedl.prepare_dispatch_layout, idx, ebkt, B,
            False, out=moedl.alloc_layout(M, k, G, B, False, device="cpu"))
    _raises(ValueError, "slot: 39 elements", moedl.prepare_dispatch_layout_noalloc, idx, ebkt,
            B, False, out=lay)
    x = torch.zeros((M, N), dtype=torch.int16)
    _raises(ValueError, "out: 256 elements", moedl.prepare_dispatch, x,
            torch.zeros((M, k), **i32), M * k, out=torch.zeros((1, N), dtype=torch.int16))
    _raises(ValueError, "x: 256 elements, the call needs 2560", moedl.prepare_layout_dispatch,
            idx, ebkt, B, False, x[:1])
    eo = torch.zeros((M * k, N), dtype=torch.int16)
    _raises(ValueError, "weights: 16 elements", moedl.prepare_combine, eo,
            torch.zeros((4, k)), torch.zeros((M, k), **i32))
    _raises(ValueError, "must live on the GPU", moedl.prepare_combine, eo,
            torch.zeros((M, k)), torch.zeros((M, k), **i32))
