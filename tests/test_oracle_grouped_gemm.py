"""Pins for the grouped-GEMM oracle and its tile metadata.

* brute-force triple loop on tiny shapes (an independent formulation);
* closed form: W[e] = c_e * I (c_e a power of two) gives y = c_e * x exactly;
* the magnitude helper equals the brute-force sum of |x w|;
* tiles cover every expert row exactly once, in expert order, with the expected
  count sum_e ceil(count_e / tile_m) <= ceil(rows / tile_m) + G.
"""
import numpy as np
import pytest

from oracle import bf16_to_f32, f32_to_bf16_rne, dispatch_layout
from oracle.grouped_gemm import gemm_tiles, grouped_gemm, magnitude


def _bf16(rng, shape, scale=1.0):
    return f32_to_bf16_rne((rng.standard_normal(shape) * scale).astype(np.float32))


@pytest.mark.parametrize("seed", range(3))
def test_brute_force(seed):
    rng = np.random.default_rng(seed)
    G, K, Nout = 3, 5, 4
    counts = rng.integers(0, 4, size=G)
    offs = np.concatenate(([0], np.cumsum(counts)[:-1]))
    rows = int(counts.sum())
    x, w = _bf16(rng, (rows, K)), _bf16(rng, (G, Nout, K))
    exact = grouped_gemm(x, w, offs, counts)
    mag = magnitude(x, w, offs, counts)
    xf, wf = bf16_to_f32(x).astype(np.float64), bf16_to_f32(w).astype(np.float64)
    for e in range(G):
        for r in range(offs[e], offs[e] + counts[e]):
            for n in range(Nout):
                s = sum(xf[r, k] * wf[e, n, k] for k in range(K))
                m = sum(abs(xf[r, k] * wf[e, n, k]) for k in range(K))
                assert exact[r, n] == pytest.approx(s, rel=1e-12, abs=1e-12)
                assert mag[r, n] == pytest.approx(m, rel=1e-12, abs=1e-12)


def test_scaled_identity_closed_form():
    rng = np.random.default_rng(7)
    G, K = 4, 16
    counts = np.array([3, 0, 5, 2])
    offs = np.concatenate(([0], np.cumsum(counts)[:-1]))
    x = _bf16(rng, (counts.sum(), K))
    c = 2.0 ** np.arange(-1, G - 1)
    w = np.stack([f32_to_bf16_rne((np.eye(K) * c[e]).astype(np.float32)) for e in range(G)])
    exact = grouped_gemm(x, w, offs, counts)
    for e in range(G):
        sl = slice(offs[e], offs[e] + counts[e])
        assert np.array_equal(exact[sl], bf16_to_f32(x[sl]).astype(np.float64) * c[e])


@pytest.mark.parametrize("tile_m", [1, 64, 128])
def test_tiles_cover_rows(tile_m):
    rng = np.random.default_rng(tile_m)
    idx = rng.integers(0, 40, size=(700, 6))
    lay = dispatch_layout(idx, (np.arange(40) % 5).astype(np.int32), 5, False)
    tiles = gemm_tiles(lay.expert_offset, lay.expert_count, tile_m)
    seen = np.zeros(700 * 6, dtype=int)
    last_e = -1
    for e, r0, n in tiles:
        assert e >= last_e and 1 <= n <= tile_m
        assert lay.expert_offset[e] <= r0 and r0 + n <= lay.expert_offset[e] + lay.expert_count[e]
        seen[r0:r0 + n] += 1
        last_e = e
    assert np.all(seen == 1)
    want = int(np.sum((lay.expert_count + tile_m - 1) // tile_m))
    assert len(tiles) == want <= (700 * 6 + tile_m - 1) // tile_m + 40
