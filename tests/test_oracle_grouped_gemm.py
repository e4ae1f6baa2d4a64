"""Pins for the grouped-GEMM oracle and its tile metadata.

* brute-force triple loop on tiny shapes (an independent formulation);
* closed form: W[e] = c_e * I (c_e a power of two) gives y = c_e * x exactly;
* the magnitude helper equals the brute-force sum of |x w|;
* tiles cover every expert row exactly once, in expert order, with the expected
  count sum_e ceil(count_e / tile_m) <= ceil(rows / tile_m) + G; a hand-worked example;
* exact equality with a rational-arithmetic formulation (small K, where float64 is
  exact), and planted mistakes (transposed weights, the wrong expert's weights, a
  dropped k slice) that it rejects.
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


def _exact_int(x, w, offs, counts):
    """An independent formulation in exact rational arithmetic: every bf16 value is a
    dyadic rational, so the products and their sums are exact as Fractions.
    Returns {(r, n): Fraction}."""
    from fractions import Fraction

    def as_frac(bits):
        v = float(bf16_to_f32(np.array([bits], dtype=np.uint16))[0])
        return Fraction(v)

    out = {}
    G, Nout, K = w.shape
    for e in range(G):
        for r in range(int(offs[e]), int(offs[e] + counts[e])):
            for n in range(Nout):
                out[(r, n)] = sum(as_frac(x[r, k]) * as_frac(w[e, n, k]) for k in range(K))
    return out


def _matches_exact(exact, ref):
    from fractions import Fraction
    return all(Fraction(float(exact[r, n])) == v for (r, n), v in ref.items())


def test_exact_integer_formulation():
    """With bf16 inputs and small K the float64 sums are exact, so the oracle must equal
    the exact rational sum, not merely approximate it."""
    rng = np.random.default_rng(11)
    G, K, Nout = 3, 6, 6
    counts = np.array([2, 0, 3])
    offs = np.array([0, 2, 2])
    x, w = _bf16(rng, (5, K)), _bf16(rng, (G, Nout, K))
    assert _matches_exact(grouped_gemm(x, w, offs, counts), _exact_int(x, w, offs, counts))


def test_planted_mistakes_fail():
    """Mutated oracles (weights transposed, the next expert's weights, one k slice
    dropped) each disagree with the exact formulation."""
    rng = np.random.default_rng(12)
    G, K, Nout = 3, 6, 6
    counts = np.array([2, 1, 3])
    offs = np.array([0, 2, 3])
    x, w = _bf16(rng, (6, K)), _bf16(rng, (G, Nout, K))
    ref = _exact_int(x, w, offs, counts)
    assert _matches_exact(grouped_gemm(x, w, offs, counts), ref)
    transposed = np.ascontiguousarray(np.swapaxes(w, 1, 2))
    assert not _matches_exact(grouped_gemm(x, transposed, offs, counts), ref)
    rolled = np.roll(w, 1, axis=0)
    assert not _matches_exact(grouped_gemm(x, rolled, offs, counts), ref)
    dropped = x.copy()
    dropped[:, -1] = 0
    assert not _matches_exact(grouped_gemm(dropped, w, offs, counts), ref)


def test_tiles_worked_example():
    """Counts 0, 300, 128, 1 at offsets 0, 0, 300, 428 with 128-row tiles."""
    off = np.array([0, 0, 300, 428])
    cnt = np.array([0, 300, 128, 1])
    assert gemm_tiles(off, cnt, 128) == [(1, 0, 128), (1, 128, 128), (1, 256, 44),
                                         (2, 300, 128), (3, 428, 1)]
    assert gemm_tiles(off, np.zeros(4, dtype=int), 128) == []
