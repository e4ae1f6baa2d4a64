"""Pins for the receiver-side expansion and the pre-reduced combine oracle.

* expand after a dedup dispatch puts each token's own row at every one of its slots
  (closed form), scales included.
* With one bucket, partial + reduce is exactly the flat combine (a special case that
  reduces to an already pinned routine): one partial per token with the flat
  combine's op order, then bf16 -> f32 -> +0 -> bf16 is the identity.
* With one expert per bucket, every partial is bf16(fl32(w*o)); the result is
  evaluated here step by step with torch's bf16 cast and float64 arithmetic rounded to
  fp32 after each operation.
* fp64 error bound with two bf16 roundings.
* An order-sensitive case (bf16 tie) fixes the ascending-bucket order of the reduce;
  planted mistakes each fail a pin.
"""
import numpy as np
import pytest
import torch

from combine_dispatch_layout_amd import workloads as wl
from oracle import bf16_to_f32, f32_to_bf16_rne, dispatch_layout, dispatch, combine
from oracle.bucket_combine import combine_partial, combine_reduce, expand


def bf16_round_torch(v: float) -> float:
    return float(torch.tensor([v], dtype=torch.float32).to(torch.bfloat16).float()[0])


def f32(v: float) -> float:
    return float(np.float32(v))


@pytest.mark.parametrize("cfg,M", [(1, None), (2, 300), (5, 80)])
def test_expand_puts_token_rows_at_slots(cfg, M):
    w = wl.make_workload(cfg, M=M)
    lay = dispatch_layout(w.topk_idx, w.expert_bucket, w.B, True)
    sent, sent_scale = dispatch(w.x, lay.send_row, lay.R, w.x_scale)
    ein, ein_scale = expand(sent, lay.send_row, lay.slot, w.M * w.k, sent_scale)
    tok = np.repeat(np.arange(w.M), w.k)
    assert np.array_equal(ein[lay.slot.reshape(-1)], w.x[tok])
    if w.x_scale is not None:
        assert np.array_equal(ein_scale[lay.slot.reshape(-1)], w.x_scale[tok])


def _random_problem(M, k, G, B, N, seed, signed=True):
    rng = np.random.default_rng(seed)
    idx = np.argsort(rng.random((M, G)), axis=1)[:, :k].astype(np.int32)
    ebkt = rng.integers(0, B, size=G).astype(np.int32)
    lay = dispatch_layout(idx, ebkt, B, True)
    eo = f32_to_bf16_rne(rng.standard_normal((M * k, N)).astype(np.float32))
    wts = (rng.standard_normal((M, k)) if signed else rng.random((M, k))).astype(np.float32)
    return idx, ebkt, lay, eo, wts


@pytest.mark.parametrize("seed", range(4))
def test_single_bucket_equals_flat_combine(seed):
    M, k, G, N = 50, 6, 20, 64
    idx, _, _, eo, wts = _random_problem(M, k, G, 1, N, seed)
    lay = dispatch_layout(idx, np.zeros(G, np.int32), 1, True)
    part = combine_partial(eo, wts, lay.slot, lay.send_row, lay.R)
    y = combine_reduce(part, lay.send_row)
    assert np.array_equal(y, combine(eo, wts, lay.slot))


def test_singleton_buckets_step_by_step():
    M, k, G, N = 6, 4, 4, 16
    rng = np.random.default_rng(3)
    idx = np.array([rng.permutation(G)[:k] for _ in range(M)], dtype=np.int32)
    ebkt = np.arange(G, dtype=np.int32)                      # expert e alone in bucket e
    lay = dispatch_layout(idx, ebkt, G, True)
    eo = f32_to_bf16_rne(rng.standard_normal((M * k, N)).astype(np.float32))
    wts = rng.standard_normal((M, k)).astype(np.float32)
    y = combine_reduce(combine_partial(eo, wts, lay.slot, lay.send_row, lay.R), lay.send_row)
    eo_f = bf16_to_f32(eo).astype(np.float64)
    for t in range(M):
        order = np.argsort(idx[t])                           # ascending bucket = expert id
        for i in range(N):
            acc = 0.0
            for j in order:
                p = bf16_round_torch(f32(float(wts[t, j]) * eo_f[lay.slot[t, j], i]))
                acc = f32(acc + p)
            want = bf16_round_torch(acc)
            got = float(bf16_to_f32(y[t:t + 1, i:i + 1])[0, 0])
            assert got == want or (np.isnan(got) and np.isnan(want)), (t, i, got, want)


def _bound_ok(eo, wts, slot, send_row, y):
    M, k = slot.shape
    terms = wts.astype(np.float64)[:, :, None] * bf16_to_f32(eo[slot]).astype(np.float64)
    exact = terms.sum(axis=1)
    part_abs = np.zeros_like(exact)
    for t in range(M):
        for r in np.unique(send_row[t]):
            part_abs[t] += np.abs(terms[t][send_row[t] == r].sum(axis=0))
    err = np.abs(bf16_to_f32(y).astype(np.float64) - exact)
    bound = 1.01 * (2.0 ** -8 * np.abs(exact) + 2.0 ** -8 * part_abs) + \
        2 * k * 2.0 ** -23 * np.abs(terms).sum(axis=1)
    return bool(np.all(err <= bound))


@pytest.mark.parametrize("cfg,M", [(2, 200), (4, 200)])
def test_fp64_bound_on_workloads(cfg, M):
    w = wl.make_workload(cfg, M=M)
    lay = dispatch_layout(w.topk_idx, w.expert_bucket, w.B, True)
    sent, _ = dispatch(w.x, lay.send_row, lay.R)
    eo, _ = expand(sent, lay.send_row, lay.slot, w.M * w.k)
    y = combine_reduce(combine_partial(eo, w.weights, lay.slot, lay.send_row, lay.R), lay.send_row)
    assert _bound_ok(eo, w.weights, lay.slot, lay.send_row, y)


def test_fp64_bound_signed_random():
    idx, ebkt, lay, eo, wts = _random_problem(80, 8, 32, 5, 128, seed=9)
    y = combine_reduce(combine_partial(eo, wts, lay.slot, lay.send_row, lay.R), lay.send_row)
    assert _bound_ok(eo, wts, lay.slot, lay.send_row, y)


# One token, experts 0..3 in buckets 0..3, weights 1: the partials are the expert
# values.  Summed in ascending bucket order, 1 + 2^-24 ties back to 1 twice and
# + 2^-8 lands on a bf16 tie -> 1.0 (0x3F80).  Descending order, or the token's j
# order (experts 1, 2, 3, 0), keeps a 2^-23 and rounds to 0x3F81.
ORDER_VALUES = [1.0, 2.0 ** -24, 2.0 ** -24, 2.0 ** -8]


def _order_case(partial_fn=combine_partial, reduce_fn=combine_reduce):
    idx = np.array([[1, 2, 3, 0]], dtype=np.int32)            # j order differs from buckets
    ebkt = np.arange(4, dtype=np.int32)
    lay = dispatch_layout(idx, ebkt, 4, True)
    eo = np.zeros((4, 1), dtype=np.uint16)
    for j in range(4):
        eo[lay.slot[0, j], 0] = f32_to_bf16_rne(np.array([ORDER_VALUES[idx[0, j]]], np.float32))[0]
    wts = np.ones((1, 4), dtype=np.float32)
    part = partial_fn(eo, wts, lay.slot, lay.send_row, lay.R)
    return int(reduce_fn(part, lay.send_row)[0, 0])


def test_reduce_order_case():
    assert _order_case() == 0x3F80


def _reduce_in_order(partial, send_row, descending=False):
    M, k = send_row.shape
    acc = np.zeros((M, partial.shape[1]), dtype=np.float32)
    for t in range(M):
        rows = sorted(set(int(r) for r in send_row[t]), reverse=descending)
        for r in rows:
            acc[t] = acc[t] + bf16_to_f32(partial[r])
    return f32_to_bf16_rne(acc)


def _reduce_j_order(partial, send_row):
    M, k = send_row.shape
    acc = np.zeros((M, partial.shape[1]), dtype=np.float32)
    for t in range(M):
        seen = []
        for r in send_row[t]:
            if int(r) not in seen:
                seen.append(int(r))
                acc[t] = acc[t] + bf16_to_f32(partial[int(r)])
    return f32_to_bf16_rne(acc)


def _partial_fp32_then_flat(eo, wts, slot, send_row, R):
    # mistake: no bf16 rounding of the partials (keeps fp32) -> breaks the singleton case
    acc = np.zeros((R, eo.shape[1]), dtype=np.float32)
    for j in range(slot.shape[1]):
        r = send_row[:, j].astype(np.int64)
        acc[r] = acc[r] + wts[:, j:j + 1] * bf16_to_f32(eo[slot[:, j]])
    return acc.view(np.uint32) >> 16   # truncation instead of RNE


def test_planted_mistakes_fail_a_pin():
    assert _order_case(reduce_fn=lambda p, s: _reduce_in_order(p, s, True)) != 0x3F80
    assert _order_case(reduce_fn=_reduce_j_order) != 0x3F80
    # truncating partials breaks the step-by-step singleton pin
    M, k, G, N = 6, 4, 4, 16
    rng = np.random.default_rng(3)
    idx = np.array([rng.permutation(G)[:k] for _ in range(M)], dtype=np.int32)
    lay = dispatch_layout(idx, np.arange(G, dtype=np.int32), G, True)
    eo = f32_to_bf16_rne(rng.standard_normal((M * k, N)).astype(np.float32))
    wts = rng.standard_normal((M, k)).astype(np.float32)
    good = combine_partial(eo, wts, lay.slot, lay.send_row, lay.R)
    bad = _partial_fp32_then_flat(eo, wts, lay.slot, lay.send_row, lay.R).astype(np.uint16)
    assert not np.array_equal(good, bad)


def _partial_and_rows():
    idx, ebkt, lay, eo, wts = _random_problem(10, 4, 8, 3, 8, seed=1)
    return combine_partial(eo, wts, lay.slot, lay.send_row, lay.R), lay.send_row


def test_reduce_matches_explicit_loop():
    part, rows = _partial_and_rows()
    assert np.array_equal(combine_reduce(part, rows), _reduce_in_order(part, rows))
