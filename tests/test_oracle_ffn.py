"""Pins for the oracle's expert FFN, combine and whole layer.

Special cases that reduce to textbook routines (k=1 is one expert's dense SwiGLU FFN,
checked with numpy float64 matmuls on independently decoded weights; a zero router
makes every logit tie; x = 0 gives y = 0), exact metamorphic relations, and negative
controls: planted mistakes (in copies of the oracle's steps, on the CPU) that the
parity tolerance must catch by a wide margin.
"""
import dataclasses
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from indep import expert_weights, silu

TINY = synth.WORKLOADS["tiny"]
TOL_F32 = 1e-4   # parity tolerance for fp32 output (rel-L2)


def rel_l2(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def _inputs(wl, seed=0, T=None):
    lay = synth.make_layer(wl, 0, seed, "cpu")
    x = synth.make_x(wl, seed, "cpu", tokens=T)
    blobs = [lay["blob"][e].numpy() for e in range(wl.n_experts)]
    bias = None if lay["bias"] is None else lay["bias"].numpy()
    return oracle.to_f64(x), lay["router"].numpy(), bias, blobs


def _layer(wl, x64, wr, bias, blobs, scaling=1.0, residual=None):
    return oracle.layer(x64, wr, bias, blobs, wl.d_model, wl.d_ff, wl.top_k, wl.wformat, scaling, residual)


def _dense_ffn(blob, x, wl):
    Wg, Wu, Wd = expert_weights(blob, wl.d_model, wl.d_ff, wl.wformat)
    g = Wg @ x
    u = Wu @ x
    return Wd @ (silu(g) * u)


@pytest.mark.parametrize("wformat", [synth.MXFP4, synth.NVFP4])
def test_k1_is_dense_ffn(wformat):
    wl = dataclasses.replace(TINY, top_k=1, n_experts=4, wformat=wformat, tokens=5)
    x64, wr, bias, blobs = _inputs(wl)
    y, idx, w, _ = _layer(wl, x64, wr, bias, blobs)
    assert np.all(w == 1.0)
    for t in range(wl.tokens):
        want = _dense_ffn(blobs[idx[t, 0]], x64[t], wl)
        np.testing.assert_allclose(y[t], want, rtol=1e-12, atol=1e-14 * np.abs(want).max())


def test_zero_router_ties_and_mean_of_all_experts():
    wl = dataclasses.replace(TINY, top_k=TINY.n_experts, tokens=2)
    x64, wr, bias, blobs = _inputs(wl)
    y, idx, w, logits = _layer(wl, x64, np.zeros_like(wr), None, blobs)
    assert np.all(logits == 0)
    assert idx.tolist() == [list(range(wl.n_experts))] * 2
    np.testing.assert_allclose(w, 1.0 / wl.n_experts, rtol=1e-15)
    for t in range(2):
        want = np.mean([_dense_ffn(b, x64[t], wl) for b in blobs], axis=0)
        np.testing.assert_allclose(y[t], want, rtol=1e-12, atol=1e-14 * np.abs(want).max())


def test_zero_router_k2_picks_first_two():
    x64, wr, bias, blobs = _inputs(TINY)
    _, idx, w, _ = _layer(TINY, x64, np.zeros_like(wr), None, blobs)
    assert idx.tolist() == [[0, 1]] * TINY.tokens
    assert np.all(w == 0.5)


def test_zero_input_gives_zero_output():
    x64, wr, bias, blobs = _inputs(TINY)
    y, _, _, _ = _layer(TINY, np.zeros_like(x64), wr, bias, blobs)
    assert np.all(y == 0.0)


def test_residual_is_added():
    x64, wr, bias, blobs = _inputs(TINY)
    y0, _, _, _ = _layer(TINY, x64, wr, bias, blobs)
    y1, _, _, _ = _layer(TINY, x64, wr, bias, blobs, residual=x64)
    np.testing.assert_array_equal(y1, y0 + x64)


def test_steps_compose_to_layer():
    x64, wr, bias, blobs = _inputs(TINY)
    y, idx, w, logits = _layer(TINY, x64, wr, bias, blobs)
    l2, idx2, w2 = oracle.route(x64, wr, bias, TINY.top_k)
    off, sp, pp = oracle.permute(idx2, TINY.n_experts)
    o = oracle.expert_ffn(blobs, TINY.d_model, TINY.d_ff, TINY.wformat, x64, TINY.top_k, off, sp)
    y2 = oracle.combine(o, w2, pp)
    np.testing.assert_array_equal(idx, idx2)
    np.testing.assert_array_equal(y, y2)
    # each o row is that pick's dense FFN
    for i, p in enumerate(sp):
        t, j = divmod(int(p), TINY.top_k)
        np.testing.assert_allclose(o[i], _dense_ffn(blobs[idx[t, j]], x64[t], TINY), rtol=1e-12,
                                   atol=1e-14 * np.abs(o[i]).max())


# -------------------------------------------------------------------------------------------
# exact metamorphic relations
# -------------------------------------------------------------------------------------------

def _bump_scales(blobs, wl, part, delta=1):
    off = synth.blob_offsets(wl.d_model, wl.d_ff, wl.wformat)
    so, sn = off[part + "_s"]
    out = []
    for b in blobs:
        b = b.copy()
        b[so:so + sn] = b[so:so + sn] + delta
        out.append(b)
    return out


def test_down_scale_plus_one_doubles_output_exactly():
    x64, wr, bias, blobs = _inputs(TINY)
    y, _, _, _ = _layer(TINY, x64, wr, bias, blobs)
    y2, _, _, _ = _layer(TINY, x64, wr, bias, _bump_scales(blobs, TINY, "down"))
    np.testing.assert_array_equal(y2, 2 * y)


def test_up_scale_plus_one_doubles_output_exactly():
    x64, wr, bias, blobs = _inputs(TINY)
    y, _, _, _ = _layer(TINY, x64, wr, bias, blobs)
    y2, _, _, _ = _layer(TINY, x64, wr, bias, _bump_scales(blobs, TINY, "up"))
    np.testing.assert_array_equal(y2, 2 * y)


def test_scaling_two_doubles_exactly():
    x64, wr, bias, blobs = _inputs(TINY)
    y, _, _, _ = _layer(TINY, x64, wr, bias, blobs)
    y2, _, _, _ = _layer(TINY, x64, wr, bias, blobs, scaling=2.0)
    np.testing.assert_array_equal(y2, 2 * y)


def test_token_permutation_permutes_output():
    wl = dataclasses.replace(TINY, tokens=9)
    x64, wr, bias, blobs = _inputs(wl)
    y, idx, _, _ = _layer(wl, x64, wr, bias, blobs)
    perm = np.random.default_rng(0).permutation(9)
    y2, idx2, _, _ = _layer(wl, np.ascontiguousarray(x64[perm]), wr, bias, blobs)
    np.testing.assert_array_equal(y2, y[perm])
    np.testing.assert_array_equal(idx2, idx[perm])


def test_expert_relabelling_leaves_output_unchanged():
    x64, wr, bias, blobs = _inputs(TINY)
    y, idx, _, _ = _layer(TINY, x64, wr, bias, blobs)
    perm = np.random.default_rng(3).permutation(TINY.n_experts)   # new id of old expert e
    inv = np.argsort(perm)
    wr2 = np.ascontiguousarray(wr[inv])
    blobs2 = [blobs[inv[e]] for e in range(TINY.n_experts)]
    y2, idx2, _, _ = _layer(TINY, x64, wr2, bias, blobs2)
    np.testing.assert_array_equal(idx2, perm[idx])
    np.testing.assert_array_equal(y2, y)


# -------------------------------------------------------------------------------------------
# negative controls: each planted mistake must exceed the fp32 parity tolerance >= 100x
# -------------------------------------------------------------------------------------------

def _baseline():
    x64, wr, bias, blobs = _inputs(TINY)
    y, idx, w, logits = _layer(TINY, x64, wr, bias, blobs)
    return x64, wr, bias, blobs, y, idx, w, logits


def _assert_caught(y_bad, y, name):
    err = rel_l2(y_bad, y)
    assert err > 100 * TOL_F32, f"negative control '{name}' not separated: rel-L2 {err:.3g}"


def test_negative_flipped_nibble_order():
    x64, wr, bias, blobs, y, *_ = _baseline()
    flipped = [((b >> 4) | (b << 4)).astype(np.uint8) for b in blobs]
    off = synth.blob_offsets(TINY.d_model, TINY.d_ff, TINY.wformat)
    for fb, b in zip(flipped, blobs):     # flip only the packed codes, keep the scales
        fb[off["gate_s"][0]:] = b[off["gate_s"][0]:]
    y_bad, *_ = _layer(TINY, x64, wr, bias, flipped)
    _assert_caught(y_bad, y, "flipped nibble order")


def test_negative_routed_scaling():
    x64, wr, bias, blobs, y, *_ = _baseline()
    y_bad, *_ = _layer(TINY, x64, wr, bias, blobs, scaling=2.5)
    _assert_caught(y_bad, y, "routed_scaling 2.5 vs 1.0")


def test_negative_e8m0_bias_off_by_one():
    x64, wr, bias, blobs, y, *_ = _baseline()
    bad = _bump_scales(_bump_scales(_bump_scales(blobs, TINY, "gate"), TINY, "up"), TINY, "down")
    y_bad, *_ = _layer(TINY, x64, wr, bias, bad)
    _assert_caught(y_bad, y, "E8M0 bias off by one")


def _combine_with(w_bad, x64, wr, bias, blobs, idx):
    off, sp, pp = oracle.permute(idx, TINY.n_experts)
    o = oracle.expert_ffn(blobs, TINY.d_model, TINY.d_ff, TINY.wformat, x64, TINY.top_k, off, sp)
    return oracle.combine(o, np.ascontiguousarray(w_bad), pp)


def test_negative_softmax_instead_of_sigmoid():
    x64, wr, bias, blobs, y, idx, w, logits = _baseline()
    sel = np.take_along_axis(logits, idx.astype(np.int64), axis=1)
    soft = np.exp(sel) / np.exp(sel).sum(axis=1, keepdims=True)
    _assert_caught(_combine_with(soft, x64, wr, bias, blobs, idx), y, "softmax scoring")


def test_negative_no_renormalisation():
    x64, wr, bias, blobs, y, idx, w, logits = _baseline()
    sel = np.take_along_axis(logits, idx.astype(np.int64), axis=1)
    raw = 1.0 / (1.0 + np.exp(-sel))
    _assert_caught(_combine_with(raw, x64, wr, bias, blobs, idx), y, "no renormalisation")


def test_negative_higher_index_tie_break():
    x64, wr, bias, blobs, *_ = _baseline()
    wr0 = np.zeros_like(wr)
    b = np.zeros(TINY.n_experts, dtype=np.float32)
    b[3], b[5], b[11] = 1.0, 0.5, 0.5             # second place is a tie between 5 and 11
    y, idx, w, _ = _layer(TINY, x64, wr0, b, blobs)
    assert idx[0].tolist() == [3, 5]
    idx_bad = np.tile(np.array([[3, 11]], dtype=np.int32), (TINY.tokens, 1))
    _assert_caught(_combine_with(w, x64, wr0, b, blobs, idx_bad), y, "higher-index tie-break")


def test_negative_wrong_block_axis():
    """Scales applied down the columns instead of along each row's reduction dim."""
    x64, wr, bias, blobs, y, idx, w, _ = _baseline()
    d, f = TINY.d_model, TINY.d_ff

    def ffn_wrong_axis(blob, x):
        import indep
        nq, ns = f * d // 2, f * d // 32
        mats = []
        for i, (rows, K) in enumerate(((f, d), (f, d), (d, f))):
            q = blob[i * nq:(i + 1) * nq].reshape(rows, K // 2)
            s = blob[3 * nq + i * ns: 3 * nq + (i + 1) * ns].reshape(-1)
            c = indep.codes(q, K)
            sc = torch.from_numpy(s.copy()).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
            r, k = np.meshgrid(np.arange(rows), np.arange(K), indexing="ij")
            mats.append(indep._table()[c] * sc[(k * rows + r) // 32])
        Wg, Wu, Wd = mats
        return Wd @ (silu(Wg @ x) * (Wu @ x))

    y_bad = np.zeros_like(y)
    for t in range(TINY.tokens):
        for j in range(TINY.top_k):
            y_bad[t] += w[t, j] * ffn_wrong_axis(blobs[idx[t, j]], x64[t])
    _assert_caught(y_bad, y, "wrong block axis")


# -------------------------------------------------------------------------------------------
# the weighted combine at non-uniform weights: which weight goes with which pick
# -------------------------------------------------------------------------------------------

def test_combine_pairs_each_weight_with_its_pick():
    """Identity router: token 0's logits are the golden case 1 3 0.5 2 (tests/golden/router_cases.txt:
    k=2 picks experts 1 and 3 with weights 0.5195751544086155 and 0.48042484559138454).  The layer
    output must be w0 * FFN_1(x) + w1 * FFN_3(x), each FFN a numpy matmul on weights decoded by
    tests/indep.py; the same sum with the two weights swapped (a mis-paired combine) must miss the
    oracle by far more than the fp32 tolerance."""
    from golden_io import router_cases
    logits, k, ids, ws = router_cases()[0]
    wl = dataclasses.replace(TINY, n_experts=4, top_k=k, tokens=1)
    lay = synth.make_layer(wl, 0, 7, "cpu")
    blobs = [lay["blob"][e].numpy() for e in range(wl.n_experts)]
    x = synth.make_x(wl, 7, "cpu").double().numpy()
    x[0, :4] = logits                                        # exact in fp32 and fp64
    x64 = np.ascontiguousarray(x)
    wr = np.zeros((wl.n_experts, wl.d_model), dtype=np.float32)
    wr[np.arange(4), np.arange(4)] = 1.0                     # logit e = x[e]
    y, idx, w, _ = _layer(wl, x64, wr, None, blobs)
    assert idx[0].tolist() == ids
    np.testing.assert_allclose(w[0], ws, rtol=0, atol=4e-16)
    f1 = _dense_ffn(blobs[ids[0]], x64[0], wl)
    f3 = _dense_ffn(blobs[ids[1]], x64[0], wl)
    want = ws[0] * f1 + ws[1] * f3
    np.testing.assert_allclose(y[0], want, rtol=1e-12, atol=1e-14 * np.abs(want).max())
    swapped = ws[1] * f1 + ws[0] * f3
    _assert_caught(swapped, y[0], "weights swapped between picks")


def test_combine_matches_numpy_sum_biased_router():
    """k=3 of 16 with a logit bias that spreads the weights (non-uniform), routed_scaling 2.5 and a
    residual: y[t] = 2.5 * sum_j w[t,j] * FFN_{idx[t,j]}(x[t]) + residual[t], with w recomputed in
    numpy from numpy's own logits (sigmoid of the picks over their sum) and each FFN a numpy
    matmul on independently decoded weights."""
    wl = dataclasses.replace(TINY, top_k=3, tokens=6)
    x64, wr, _, blobs = _inputs(wl, seed=11)
    bias = np.float32(1.0) - np.float32(1.2) * (wl.n_experts - 1 - np.arange(wl.n_experts, dtype=np.float32))
    res = np.ascontiguousarray(np.linspace(-1, 1, wl.tokens * wl.d_model).reshape(wl.tokens, wl.d_model))
    y, idx, w, _ = _layer(wl, x64, wr, bias, blobs, scaling=2.5, residual=res)
    l_np = x64 @ wr.astype(np.float64).T + bias.astype(np.float64)
    sel = np.take_along_axis(l_np, idx.astype(np.int64), axis=1)
    sig = 1.0 / (1.0 + np.exp(-sel))
    w_np = sig / sig.sum(axis=1, keepdims=True)
    np.testing.assert_allclose(w, w_np, rtol=1e-13)
    assert (w.max(axis=1) - w.min(axis=1)).min() > 0.2       # the weights really differ
    for t in range(wl.tokens):
        ffns = [_dense_ffn(blobs[e], x64[t], wl) for e in idx[t]]
        want = 2.5 * sum(w_np[t, j] * ffns[j] for j in range(wl.top_k)) + res[t]
        np.testing.assert_allclose(y[t], want, rtol=1e-11, atol=1e-13 * np.abs(want).max())
        rev = 2.5 * sum(w_np[t, wl.top_k - 1 - j] * ffns[j] for j in range(wl.top_k)) + res[t]
        _assert_caught(rev - res[t], y[t] - res[t], "weights paired in reverse rank order")


def test_renorm_skip_layer_matches_numpy_and_catches_missing_renormalisation():
    """With renorm-skip, y[t] = sum over the kept picks of w_kept * FFN(x[t]) (numpy, weights
    recomputed from numpy's logits: the sigmoids of the kept picks over their sum); keeping the
    unrenormalised weights instead is a planted mistake the tolerance must catch."""
    wl = dataclasses.replace(TINY, top_k=4, tokens=6)
    x64, wr, _, blobs = _inputs(wl, seed=5)
    bias = np.float32(1.0) - np.float32(1.2) * (wl.n_experts - 1 - np.arange(wl.n_experts, dtype=np.float32))
    tau = 0.2
    y, idx, w, _ = oracle.layer(x64, wr, bias, blobs, wl.d_model, wl.d_ff, wl.top_k, wl.wformat,
                                renorm_skip=tau)
    _, idx0, w0, _ = oracle.layer(x64, wr, bias, blobs, wl.d_model, wl.d_ff, wl.top_k, wl.wformat)
    assert (idx < 0).any(), "the bias makes some picks light enough to drop"
    l_np = x64 @ wr.astype(np.float64).T + bias.astype(np.float64)
    y_bad = np.zeros_like(y)
    for t in range(wl.tokens):
        kept = [j for j in range(wl.top_k) if idx[t, j] >= 0]
        assert idx[t, kept].tolist() == idx0[t, kept].tolist()
        sig = np.array([1.0 / (1.0 + np.exp(-l_np[t, idx[t, j]])) for j in kept])
        ffns = [_dense_ffn(blobs[idx[t, j]], x64[t], wl) for j in kept]
        want = sum((sig[i] / sig.sum()) * ffns[i] for i in range(len(kept)))
        np.testing.assert_allclose(y[t], want, rtol=1e-11, atol=1e-13 * np.abs(want).max())
        y_bad[t] = sum(w0[t, j] * ffns[i] for i, j in enumerate(kept))
    _assert_caught(y_bad, y, "kept weights not renormalised")


# -------------------------------------------------------------------------------------------
# the shared expert: every token's dense FFN, added outside the routed scaling
# -------------------------------------------------------------------------------------------

def _shared_inputs():
    wl = dataclasses.replace(TINY, n_experts=TINY.n_experts + 1, tokens=5)   # blob E is the shared one
    x64, wr, bias, blobs = _inputs(wl, seed=3)
    return TINY, x64, np.ascontiguousarray(wr[:TINY.n_experts]), blobs[:TINY.n_experts], blobs[TINY.n_experts]


def test_shared_expert_alone_is_its_dense_ffn():
    """With the routed sum scaled to nothing, y is the shared expert's dense SwiGLU FFN of each token
    (numpy matmuls on independently decoded weights) plus the residual."""
    wl, x64, wr, blobs, sb = _shared_inputs()
    res = np.ascontiguousarray(x64 * 0.5)
    y, *_ = oracle.layer(x64, wr, None, blobs, wl.d_model, wl.d_ff, wl.top_k, wl.wformat, 0.0, res,
                         shared_blob=sb)
    for t in range(x64.shape[0]):
        want = _dense_ffn(sb, x64[t], wl) + res[t]
        np.testing.assert_allclose(y[t], want, rtol=1e-12, atol=1e-14 * np.abs(want).max())


def test_shared_expert_sits_outside_routed_scaling():
    """y(shared, routed_scaling 2.5) = 2.5 * y(no shared expert, scaling 1) + FFN_shared(x): the
    shared expert is added with weight 1 after the scaling (the scaling factor of the windlass
    README's negative controls, 2.5); scaling it with the routed sum is caught by far."""
    wl, x64, wr, blobs, sb = _shared_inputs()
    y1, *_ = oracle.layer(x64, wr, None, blobs, wl.d_model, wl.d_ff, wl.top_k, wl.wformat, 1.0)
    y, *_ = oracle.layer(x64, wr, None, blobs, wl.d_model, wl.d_ff, wl.top_k, wl.wformat, 2.5, shared_blob=sb)
    sh = np.stack([_dense_ffn(sb, x64[t], wl) for t in range(x64.shape[0])])
    want = 2.5 * y1 + sh
    np.testing.assert_allclose(y, want, rtol=1e-12, atol=1e-14 * np.abs(want).max())
    _assert_caught(2.5 * (y1 + sh), y, "shared expert inside the routed scaling")
    _assert_caught(y1 + sh, y, "routed scaling ignored")
