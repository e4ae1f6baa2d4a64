"""Pins for the oracle's number formats against torch's CPU casts (an independent
library implementation) and hand-checked special values."""
import numpy as np
import pytest
import torch

from oracle.numerics import bf16_to_f32, f32_to_bf16_rne, e4m3_to_f32, f32_to_e4m3_rne_sat


def _torch_bf16_bits(f32):
    return torch.from_numpy(np.ascontiguousarray(f32, dtype=np.float32)).to(
        torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_bf16_widen_matches_torch_all_patterns():
    u = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ours = bf16_to_f32(u)
    ref = torch.from_numpy(u.view(np.int16)).view(torch.bfloat16).float().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_bf16_narrow_matches_torch_random_bits():
    rng = np.random.default_rng(7)
    u = rng.integers(0, 1 << 32, size=1 << 20, dtype=np.uint64).astype(np.uint32)
    f = u.view(np.float32)
    nan = np.isnan(f)
    ours = f32_to_bf16_rne(f)
    ref = _torch_bf16_bits(f)
    assert np.array_equal(ours[~nan], ref[~nan])
    # NaN stays NaN (exponent all ones, mantissa nonzero) and keeps its sign
    assert np.all((ours[nan] & 0x7F80) == 0x7F80) and np.all((ours[nan] & 0x7F) != 0)
    assert np.array_equal(ours[nan] >> 15, (u[nan] >> 31).astype(np.uint16))


def test_bf16_narrow_ties_and_edges():
    cases = {
        1.0 + 2.0 ** -8: 0x3F80,          # exact tie, even stays
        1.0 + 3 * 2.0 ** -8: 0x3F82,      # exact tie, odd rounds up
        1.0 + 2.0 ** -8 + 2.0 ** -20: 0x3F81,  # above the tie
        -0.0: 0x8000,
        float("inf"): 0x7F80,
        3.4028234663852886e38: 0x7F80,    # max float rounds to inf
        2.0 ** -133: 0x0001,              # bf16's smallest subnormal, exact
        2.0 ** -134: 0x0000,              # half of it: tie, even (zero) stays
        3 * 2.0 ** -134: 0x0002,          # one and a half: tie, rounds to even 2
        2.0 ** -126: 0x0080,              # smallest normal
    }
    for v, want in cases.items():
        got = int(f32_to_bf16_rne(np.array([v], dtype=np.float32))[0])
        assert got == want, (v, hex(got), hex(want))


def test_e4m3_decode_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ours = e4m3_to_f32(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    nan = np.isnan(ref)
    assert nan.sum() == 2 and np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9


def test_e4m3_encode_matches_torch_in_range():
    rng = np.random.default_rng(3)
    v = np.concatenate([
        rng.standard_normal(1 << 18).astype(np.float32) * 50,
        rng.uniform(-448, 448, 1 << 16).astype(np.float32),
        e4m3_to_f32(np.arange(0, 0x7F, dtype=np.uint8)),             # exact codes
        ((e4m3_to_f32(np.arange(0, 0x7E, dtype=np.uint8)) +
          e4m3_to_f32(np.arange(1, 0x7F, dtype=np.uint8))) / 2).astype(np.float32),  # ties
    ])
    v = np.concatenate([v, -v])
    ours = f32_to_e4m3_rne_sat(v)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_e4m3_encode_saturates():
    v = np.array([448.0, 460.0, 1e6, -1e6, float("inf")], dtype=np.float32)
    assert list(f32_to_e4m3_rne_sat(v)) == [0x7E, 0x7E, 0x7E, 0xFE, 0x7E]
    assert f32_to_e4m3_rne_sat(np.array([np.nan], dtype=np.float32))[0] == 0x7F
