"""Number formats used by the oracle (test infrastructure only).

* bfloat16: the top 16 bits of an IEEE binary32.  Widening is exact (shift left 16);
  narrowing rounds to nearest, ties to even, on the 16 dropped bits; NaN stays a
  quiet NaN.  Combine's output format ("bf16 out, fp32 accumulate").
* fp8 e4m3 in the OCP "fn" variant: 1 sign, 4 exponent (bias 7), 3 mantissa bits, no
  infinities, only S.1111.111 is NaN, largest finite 448.  The per-128-element
  scaled rows of the fp8 workload carry these codes; the problem statement of
  "All2all performance comparison between Triton-distributed and DeepEP"
  ("Test Code Snippet": element size, scale element size, WITH_SCALE) leaves the
  variant open, and OCP e4m3fn is the one gfx950 converts natively.
"""
from __future__ import annotations

import numpy as np


def bf16_to_f32(u: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float32, exactly."""
    return (np.asarray(u, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_bf16_rne(f: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest, ties to even."""
    u = np.ascontiguousarray(f, dtype=np.float32).view(np.uint32).astype(np.uint64)
    is_nan = (u & 0x7FFFFFFF) > 0x7F800000
    lsb = (u >> 16) & 1
    rounded = (u + 0x7FFF + lsb) >> 16
    quiet = (u >> 16) | 0x0040
    return np.where(is_nan, quiet, rounded).astype(np.uint16)


def _e4m3_table() -> np.ndarray:
    """Value of each of the 256 e4m3fn codes (NaN for the two NaN codes)."""
    vals = np.empty(256, dtype=np.float64)
    for code in range(256):
        s = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            vals[code] = np.nan
        elif e == 0:
            vals[code] = s * m * 2.0 ** -9          # subnormal: (m/8) * 2^(1-7)
        else:
            vals[code] = s * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


E4M3_VALUES = _e4m3_table()


def e4m3_to_f32(q: np.ndarray) -> np.ndarray:
    """fp8 e4m3fn codes (uint8) -> float32, exactly."""
    return E4M3_VALUES[np.asarray(q, dtype=np.uint8)].astype(np.float32)


def f32_to_e4m3_rne_sat(v: np.ndarray) -> np.ndarray:
    """float32 -> e4m3fn codes, round to nearest (ties to the even code), saturating
    to +-448; NaN -> 0x7F.  Written as 'nearest representable value' over the code
    table rather than as bit manipulation."""
    v = np.asarray(v, dtype=np.float64)
    pos_codes = np.arange(0x00, 0x7F)              # 0 .. 0x7E: +0 .. +448
    pos_vals = E4M3_VALUES[pos_codes]
    a = np.minimum(np.abs(v), 448.0)
    hi = np.clip(np.searchsorted(pos_vals, a, side="left"), 0, len(pos_vals) - 1)
    lo = np.clip(hi - 1, 0, len(pos_vals) - 1)
    d_lo = a - pos_vals[lo]
    d_hi = pos_vals[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (pos_codes[hi] % 2 == 0))
    code = np.where(pick_hi, pos_codes[hi], pos_codes[lo]).astype(np.uint8)
    code = np.where(np.signbit(v), code | 0x80, code).astype(np.uint8)
    return np.where(np.isnan(v), np.uint8(0x7F), code).astype(np.uint8)
