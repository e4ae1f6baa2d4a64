"""Pins for the dispatch, stand-in and combine oracles.

* Dispatch: every send row holds its token's bytes, unwritten rows keep their fill.
* Identity round trip: with identity experts and positive weights summing to 1,
  combine must give back the input rows exactly (closed form: the fp32 sum differs
  from x by ~1e-6 relative, far below half a bf16 ulp).
* Scaled experts: y ~= x * sum_j w_j (1 + e_j/256) within two bf16 roundings.
* fp8 experts: y = bf16(dequant(x) * sum w) within one rounding.
* fp64 bound: |y - sum w o| <= 2^-8 |sum w o| + k 2^-23 sum |w o| for every element.
* Operation order: a hand-built case whose bf16 result depends on the fp32 rounding
  of each step, evaluated here step by step in float64 with one explicit fp32
  rounding per operation.
* Planted mistakes: mutated copies of the combine oracle (a dropped term, weights on
  the wrong expert, reversed order, fused multiply-add) each fail one of the pins.
"""
import numpy as np
import pytest

from combine_dispatch_layout_amd import workloads as wl
from oracle import (bf16_to_f32, f32_to_bf16_rne, e4m3_to_f32, dispatch_layout,
                    dispatch, combine, expert_outputs)


def pipeline(w, dedup, combine_fn=combine):
    lay = dispatch_layout(w.topk_idx, w.expert_bucket, w.B, dedup)
    sent, sent_scale = dispatch(w.x, lay.send_row, lay.R, w.x_scale)
    eo = expert_outputs(w.standin, sent, lay.send_row, lay.slot, w.topk_idx, sent_scale)
    y = combine_fn(eo, w.weights, lay.slot)
    return lay, sent, sent_scale, eo, y


@pytest.mark.parametrize("dedup", [False, True])
def test_dispatch_rows_and_sentinels(dedup):
    w = wl.make_workload(1)
    lay = dispatch_layout(w.topk_idx, w.expert_bucket, w.B, dedup)
    cap = w.M * w.k
    out, _ = dispatch(w.x, lay.send_row, cap, fill=0xABCD)
    for r in range(lay.R):
        assert np.array_equal(out[r], w.x[lay.send_token[r]])
    assert np.all(out[lay.R:] == 0xABCD)
    if dedup:
        assert lay.R < cap


def test_dispatch_scales_follow_rows():
    w = wl.make_workload(5, M=96)
    lay = dispatch_layout(w.topk_idx, w.expert_bucket, w.B, True)
    out, osc = dispatch(w.x, lay.send_row, lay.R, w.x_scale)
    assert np.array_equal(out, w.x[lay.send_token])
    assert np.array_equal(osc, w.x_scale[lay.send_token])


@pytest.mark.parametrize("cfg,M", [(1, None), (3, 1024)])
@pytest.mark.parametrize("dedup", [False, True])
def test_identity_round_trip_is_exact(cfg, M, dedup):
    w = wl.make_workload(cfg, M=M)
    assert np.all(w.weights > 0)
    *_, y = pipeline(w, dedup)
    x = w.x.copy()
    x[x == 0x8000] = 0                      # -0 comes back as +0
    assert np.array_equal(y, x)


def test_scaled_experts_closed_form():
    w = wl.make_workload(2, M=512)
    *_, y = pipeline(w, True)
    factor = (w.weights.astype(np.float64) * (1 + w.topk_idx / 256.0)).sum(axis=1)
    expect = bf16_to_f32(w.x).astype(np.float64) * factor[:, None]
    got = bf16_to_f32(y).astype(np.float64)
    nz = expect != 0
    rel = np.abs(got[nz] - expect[nz]) / np.abs(expect[nz])
    assert rel.max() <= 2 * 2.0 ** -8, rel.max()
    assert np.all(got[~nz] == 0)


def test_fp8_experts_closed_form():
    w = wl.make_workload(5, M=256)
    *_, y = pipeline(w, False)
    deq = (e4m3_to_f32(w.x).reshape(w.M, -1, 128).astype(np.float64) *
           w.x_scale[:, :, None]).reshape(w.M, w.N)
    expect = deq * w.weights.astype(np.float64).sum(axis=1)[:, None]
    got = bf16_to_f32(y).astype(np.float64)
    nz = expect != 0
    rel = np.abs(got[nz] - expect[nz]) / np.abs(expect[nz])
    assert rel.max() <= 2.0 ** -8 * 1.001, rel.max()


def fp64_bound_ok(eo, weights, slot, y):
    k = slot.shape[1]
    terms = weights.astype(np.float64)[:, :, None] * bf16_to_f32(eo[slot]).astype(np.float64)
    exact = terms.sum(axis=1)
    err = np.abs(bf16_to_f32(y).astype(np.float64) - exact)
    bound = 2.0 ** -8 * np.abs(exact) + k * 2.0 ** -23 * np.abs(terms).sum(axis=1)
    return bool(np.all(err <= bound))


@pytest.mark.parametrize("cfg,M", [(2, 256), (4, 256)])
def test_fp64_error_bound(cfg, M):
    w = wl.make_workload(cfg, M=M)
    lay, _, _, eo, y = pipeline(w, w.dedup)
    assert fp64_bound_ok(eo, w.weights, lay.slot, y)


def test_random_signed_inputs_fp64_bound():
    """Mixed-sign weights and rows (cancellation possible): still within the bound."""
    rng = np.random.default_rng(11)
    M, k, N = 64, 6, 256
    eo = f32_to_bf16_rne(rng.standard_normal((M * k, N)).astype(np.float32))
    wts = rng.standard_normal((M, k)).astype(np.float32)
    slot = rng.permutation(M * k).reshape(M, k)
    y = combine(eo, wts, slot)
    assert fp64_bound_ok(eo, wts, slot, y)


def _round_f32(v: float) -> float:
    return float(np.float32(v))


def _stepwise(ws, os_):
    """acc = +0; acc = fl32(acc + fl32(w*o)) for j ascending, in float64 arithmetic with
    an explicit fp32 rounding after each operation (exact here: all operands are
    short enough that float64 represents every intermediate exactly)."""
    acc = 0.0
    for wv, ov in zip(ws, os_):
        acc = _round_f32(acc + _round_f32(wv * ov))
    return acc


ORDER_CASE = dict(
    # j = 0..3.  Sum in source order: 1 + 2^-24 ties back to 1 (twice), then + 2^-8
    # lands exactly on a bf16 tie -> 1.0.  Any other order keeps the 2^-23 and
    # rounds up to 1 + 2^-7.
    w=[1.0, 1.0, 1.0, 1.0], o=[1.0, 2.0 ** -24, 2.0 ** -24, 2.0 ** -8],
)
FMA_CASE = dict(
    # j = 0 contributes -(1 + 2^-7).  j = 1: (1 + 2^-17)(1 + 2^-7) = 1 + 2^-7 + 2^-17 + 2^-24,
    # whose fp32 rounding drops the 2^-24 (a tie to even).  Rounded product: the sum
    # cancels to exactly 2^-17.  Fused: 2^-17 + 2^-24, which bf16 keeps (0x3701).
    w=[1.0, 1.0 + 2.0 ** -17], o=[-(1.0 + 2.0 ** -7), 1.0 + 2.0 ** -7],
)


def _run_case(case, combine_fn=combine):
    k = len(case["w"])
    eo = f32_to_bf16_rne(np.array(case["o"], dtype=np.float32)).reshape(k, 1)
    assert np.array_equal(bf16_to_f32(eo).reshape(-1), np.array(case["o"], dtype=np.float32))
    wts = np.array([case["w"]], dtype=np.float32)
    slot = np.arange(k).reshape(1, k)
    return int(combine_fn(eo, wts, slot)[0, 0])


def _expected_bits(case):
    acc = _stepwise([float(np.float32(v)) for v in case["w"]], case["o"])
    return int(f32_to_bf16_rne(np.array([acc], dtype=np.float32))[0])


def test_operation_order_step_by_step():
    assert _expected_bits(ORDER_CASE) == 0x3F80
    assert _run_case(ORDER_CASE) == 0x3F80


def test_no_fused_multiply_add_step_by_step():
    exp = _expected_bits(FMA_CASE)
    assert exp == 0x3700                       # 2^-17
    assert _run_case(FMA_CASE) == exp
    # a single-rounding (fused) evaluation gives a different bf16 value
    first = FMA_CASE["w"][0] * FMA_CASE["o"][0]
    fused = _round_f32(first + FMA_CASE["w"][1] * FMA_CASE["o"][1])
    assert int(f32_to_bf16_rne(np.array([fused], dtype=np.float32))[0]) == 0x3701


# ---------------------------------------------------------------- planted mistakes


def _combine_dropped_term(eo, wts, slot):
    return combine(eo, wts[:, :-1], slot[:, :-1])


def _combine_weights_misaligned(eo, wts, slot):
    return combine(eo, wts[:, ::-1].copy(), slot)


def _combine_reversed_order(eo, wts, slot):
    return combine(eo, wts[:, ::-1].copy(), slot[:, ::-1].copy())


def _combine_fused(eo, wts, slot):
    acc = np.zeros((slot.shape[0], eo.shape[1]), dtype=np.float64)
    for j in range(slot.shape[1]):
        acc = (acc + wts[:, j:j + 1].astype(np.float64) *
               bf16_to_f32(eo[slot[:, j]]).astype(np.float64)).astype(np.float32).astype(np.float64)
    return f32_to_bf16_rne(acc.astype(np.float32))


def _pins_pass(combine_fn):
    """True if the mutated combine passes every pin above."""
    try:
        w1 = wl.make_workload(1)
        *_, y = pipeline(w1, False, combine_fn)
        x = w1.x.copy()
        x[x == 0x8000] = 0
        if not np.array_equal(y, x):
            return False
        w2 = wl.make_workload(2, M=128)
        *_, y2 = pipeline(w2, True, combine_fn)
        factor = (w2.weights.astype(np.float64) * (1 + w2.topk_idx / 256.0)).sum(axis=1)
        expect = bf16_to_f32(w2.x).astype(np.float64) * factor[:, None]
        nz = expect != 0
        rel = np.abs(bf16_to_f32(y2).astype(np.float64)[nz] - expect[nz]) / np.abs(expect[nz])
        if rel.max() > 2 * 2.0 ** -8:
            return False
        if _run_case(ORDER_CASE, combine_fn) != _expected_bits(ORDER_CASE):
            return False
        if _run_case(FMA_CASE, combine_fn) != _expected_bits(FMA_CASE):
            return False
        return True
    except Exception:
        return False


def test_correct_combine_passes_all_pins():
    assert _pins_pass(combine)


@pytest.mark.parametrize("mutant", [_combine_dropped_term, _combine_weights_misaligned,
                                    _combine_reversed_order, _combine_fused])
def test_planted_mistakes_are_caught(mutant):
    assert not _pins_pass(mutant)
