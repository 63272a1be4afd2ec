"""Pins for the oracle's router (logits, top-k, weights) and permute.

Top-k is pinned by brute force over every k-subset on tiny inputs and by a
sort-based library routine; weights by hand-worked cases and the sum-to-one
invariant; logits by exact rational arithmetic; permute by Python's stable sort.
"""
import itertools
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
from golden_io import router_cases


def _route_logits(logits, k):
    """Feed logits straight through: x = logits, router = identity, so l[e] = x[e] exactly."""
    l = np.asarray(logits, dtype=np.float64)
    E = l.shape[-1]
    x = l.reshape(-1, E).copy()
    wr = np.eye(E, dtype=np.float32)
    return oracle.route(np.ascontiguousarray(x), wr, None, k)


def test_hand_worked_cases():
    for logits, k, ids, ws in router_cases():
        _, idx, w = _route_logits(logits, k)
        assert idx[0].tolist() == ids
        np.testing.assert_allclose(w[0], ws, rtol=0, atol=4e-16)


def _rank_key(l, e):
    return (1 if math.isnan(l) else 0, 0 if math.isnan(l) else -l, e)


@pytest.mark.parametrize("seed", range(6))
def test_topk_brute_force_pairs(seed):
    """E=16, k=2: the chosen set is the best pair under (sum desc, then lexicographic ids),
    and the order inside it is (logit desc, index asc).  Logits are quantised to force ties."""
    rng = np.random.default_rng(seed)
    T, E, k = 32, 16, 2
    l = np.round(rng.normal(size=(T, E)) * 2) / 2          # many exact ties
    _, idx, _ = _route_logits(l, k)
    for t in range(T):
        best = None
        for pair in itertools.combinations(range(E), k):
            ordered = sorted(pair, key=lambda e: _rank_key(l[t, e], e))
            key = [_rank_key(l[t, e], e) for e in ordered]
            if best is None or key < best[0]:
                best = (key, ordered)
        assert idx[t].tolist() == best[1]


@pytest.mark.parametrize("k", [1, 2, 8])
def test_topk_matches_lexsort(k):
    rng = np.random.default_rng(k)
    T, E = 64, 288
    l = rng.normal(size=(T, E))
    l[:, 10] = l[:, 3]                                    # exact ties between experts 3 and 10
    _, idx, _ = _route_logits(l, k)
    for t in range(T):
        order = np.lexsort((np.arange(E), -l[t]))       # primary: -l, secondary: index
        assert idx[t].tolist() == order[:k].tolist()


def test_nan_logits_rank_last():
    # the identity-router trick would spread NaN to every logit (NaN * 0), so the NaNs
    # come in through the bias
    bias = np.array([np.nan, 1.0, np.nan, -5.0], dtype=np.float32)
    x = np.zeros((1, 4))
    _, idx, _ = oracle.route(x, np.eye(4, dtype=np.float32), bias, 3)
    assert idx[0].tolist() == [1, 3, 0]


def test_weights_sum_to_one_and_formula():
    rng = np.random.default_rng(1)
    l = rng.normal(size=(50, 288))
    _, idx, w = _route_logits(l, 8)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=0, atol=4 * 2.0**-52)
    assert np.all((w > 0) & (w < 1))
    for t in range(50):
        s = np.array([1.0 / (1.0 + math.exp(-l[t, e])) for e in idx[t]])
        np.testing.assert_allclose(w[t], s / s.sum(), rtol=1e-15)


def test_logits_exact_rational():
    """bf16-valued x times small-exponent fp32 router rows: every partial sum is exact in
    fp64, so the oracle's logit equals the exact rational dot product."""
    rng = np.random.default_rng(7)
    T, d, E = 3, 64, 5
    x = (rng.integers(-128, 128, size=(T, d)) * 2.0**-6).astype(np.float64)
    wr = (rng.integers(-2**12, 2**12, size=(E, d)) * 2.0**-12).astype(np.float32)
    bias = (rng.integers(-8, 8, size=E) * 0.125).astype(np.float32)
    logits, _, _ = oracle.route(x, wr, bias, 2)
    for t in range(T):
        for e in range(E):
            exact = sum(Fraction(float(x[t, i])) * Fraction(float(wr[e, i])) for i in range(d))
            exact += Fraction(float(bias[e]))
            assert Fraction(logits[t, e]) == exact


def test_bias_shifts_selection():
    l = np.zeros((1, 4))
    x = l.copy()
    wr = np.eye(4, dtype=np.float32)
    bias = np.array([0, 0, 0.5, 0.25], dtype=np.float32)
    _, idx, w = oracle.route(x, wr, bias, 2)
    assert idx[0].tolist() == [2, 3]
    s = [1 / (1 + math.exp(-0.5)), 1 / (1 + math.exp(-0.25))]
    np.testing.assert_allclose(w[0], [s[0] / sum(s), s[1] / sum(s)], rtol=1e-15)


@pytest.mark.parametrize("T,k,E", [(1, 8, 288), (7, 2, 16), (300, 8, 288), (0, 8, 288)])
def test_permute_matches_stable_sort(T, k, E):
    rng = np.random.default_rng(T)
    idx = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]) if T else \
        np.zeros((0, k), dtype=np.int32)
    idx = idx.astype(np.int32).reshape(T, k)
    offsets, sp, pp = oracle.permute(idx, E)
    flat = idx.reshape(-1)
    want = sorted(range(T * k), key=lambda p: (flat[p], p))   # Python's sort is stable
    assert sp.tolist() == want
    assert offsets[0] == 0 and offsets[E] == T * k
    counts = np.bincount(flat, minlength=E) if T else np.zeros(E, dtype=int)
    np.testing.assert_array_equal(np.diff(offsets), counts)
    # pick_pos is the inverse permutation of sorted_pick
    assert np.array_equal(sp[pp], np.arange(T * k))
    for e in range(E):
        seg = sp[offsets[e]:offsets[e + 1]]
        assert np.all(flat[seg] == e)
        assert np.all(np.diff(seg // k) > 0)      # token ids strictly increasing per expert


def test_permute_rejects_out_of_range():
    with pytest.raises(ValueError):
        oracle.permute(np.array([[0, 16]], dtype=np.int32), 16)


def test_permute_dropped_picks_take_no_position():
    """Expert id -1 (a pick dropped by renorm-skip) takes no position; the others are sorted
    exactly as Python's stable sort sorts them without it; the positions past the last kept pick
    hold -1; any other negative id is still refused."""
    idx = np.array([[3, -1], [0, 3], [-1, 1], [2, 0]], dtype=np.int32)
    offsets, sp, pp = oracle.permute(idx, 4)
    flat = idx.reshape(-1)
    kept = [p for p in range(8) if flat[p] >= 0]
    want = sorted(kept, key=lambda p: (flat[p], p))
    assert sp.tolist() == want + [-1, -1]
    assert offsets.tolist() == [0, 2, 3, 4, 6]
    assert pp[1] == -1 and pp[4] == -1
    assert [pp[p] for p in want] == list(range(6))
    with pytest.raises(ValueError):
        oracle.permute(np.array([[0, -2]], dtype=np.int32), 4)


# -------------------------------------------------------------------------------------------
# renorm-skip: picks after the first whose weight is below the threshold are dropped and the
# kept weights renormalised (Strata-GLM blog, "Uncensoring without touching the weights")
# -------------------------------------------------------------------------------------------

def _route_skip(logits, k, tau):
    l = np.asarray(logits, dtype=np.float64)
    E = l.shape[-1]
    return oracle.route(np.ascontiguousarray(l.reshape(-1, E)), np.eye(E, dtype=np.float32), None, k, tau)


def test_renorm_skip_golden():
    """Logits 3 2 -2 0.5 with k=3: the third pick (logit 0.5) weighs 0.2535 before the skip.  A
    threshold of 0.3 drops it, and the two kept picks then carry exactly the weights of the
    hand-worked two-expert case with logits 3 and 2 (tests/golden/router_cases.txt, first line)."""
    _, ids2, ws2 = router_cases()[0][1:]
    _, idx, w = _route_skip([3, 2, -2, 0.5], 3, 0.3)
    assert idx[0].tolist() == [0, 1, -1]
    np.testing.assert_allclose(w[0], list(ws2) + [0.0], rtol=0, atol=4e-16)
    # a threshold below the third weight keeps all three, bit for bit as without the skip
    _, idx0, w0 = _route_skip([3, 2, -2, 0.5], 3, 0.0)
    _, idx1, w1 = _route_skip([3, 2, -2, 0.5], 3, 0.25)
    assert idx1.tolist() == idx0.tolist() == [[0, 1, 3]]
    np.testing.assert_array_equal(w1, w0)
    # a threshold above every weight but the first keeps the first pick alone, with weight 1
    _, idx, w = _route_skip([3, 2, -2, 0.5], 3, 0.9)
    assert idx[0].tolist() == [0, -1, -1] and w[0].tolist() == [1.0, 0.0, 0.0]


@pytest.mark.parametrize("seed", range(4))
def test_renorm_skip_relations(seed):
    """Against the same routing without the skip: the kept picks are the same experts in the same
    slots, they form a prefix of the rank order that always holds rank 0, a pick is dropped exactly
    when its unskipped weight is below the threshold, and each kept weight is its unskipped weight
    divided by the kept picks' unskipped total."""
    rng = np.random.default_rng(seed)
    l = rng.normal(size=(200, 288)) * rng.uniform(0.5, 3.0)
    tau = float(np.float32(rng.uniform(0.05, 0.2)))
    _, idx0, w0 = _route_skip(l, 8, 0.0)
    _, idx, w = _route_skip(l, 8, tau)
    dropped = idx < 0
    assert not dropped[:, 0].any()
    assert np.all(np.diff(dropped.astype(int), axis=1) >= 0)          # a suffix of the ranks
    np.testing.assert_array_equal(dropped[:, 1:], w0[:, 1:] < tau)
    np.testing.assert_array_equal(np.where(dropped, -1, idx0), idx)
    kept_total = np.where(dropped, 0.0, w0).sum(axis=1, keepdims=True)
    np.testing.assert_allclose(w, np.where(dropped, 0.0, w0 / kept_total), rtol=1e-14, atol=0)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=0, atol=4 * 2.0**-52)
    assert dropped.any() and not dropped.all(axis=1).any()
