"""Pins for the oracle's opt-in MXFP8 activation mode: the E4M3 rounding against torch's
float8_e4m3fn conversion (round to nearest, ties to even), the block scale rule through its
invariants, and the whole layer against an independent numpy/torch implementation."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import synth
from indep import expert_weights, silu

TINY = synth.WORKLOADS["tiny"]


def _torch_e4m3(v):
    """Nearest E4M3FN value (ties to even) by torch's own conversion; v exact in fp32."""
    t = torch.tensor(np.asarray(v, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_e4m3_round_codes_midpoints_and_random():
    codes = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    vals = np.sort(np.unique(np.abs(codes[np.isfinite(codes)])))
    assert vals[-1] == 448.0
    for v in vals:                                   # every value is its own rounding
        assert oracle.e4m3_round(v) == v and oracle.e4m3_round(-v) == -v
    mids = (vals[:-1] + vals[1:]) / 2                # exact ties: go to the even code
    got = np.array([oracle.e4m3_round(m) for m in mids])
    np.testing.assert_array_equal(got, _torch_e4m3(mids))
    rng = np.random.default_rng(0)
    r = np.concatenate([rng.uniform(-447, 447, 4000), rng.uniform(-2**-5, 2**-5, 4000)]).astype(np.float32)
    got = np.array([oracle.e4m3_round(float(v)) for v in r])
    np.testing.assert_array_equal(got, _torch_e4m3(r))


@pytest.mark.parametrize("seed", range(3))
def test_block_quantiser_scale_rule(seed):
    rng = np.random.default_rng(seed)
    v = (rng.normal(size=32 * 64) * np.repeat(2.0 ** rng.integers(-30, 30, 64), 32)).astype(np.float32)
    v[:32] = 0.0                                    # an all-zero block
    v[32:64] = v[32:64] * 2.0**-120                 # a block whose exponent is clamped
    q = oracle.quant_mxfp8(v.astype(np.float64))
    for b in range(64):
        blk, qb = v[32 * b:32 * b + 32].astype(np.float64), q[32 * b:32 * b + 32]
        amax = np.abs(blk).max()
        if amax == 0:
            assert np.all(qb == 0)
            continue
        S = max(int(np.floor(np.log2(amax))) - 7, -126)
        if S > -126:
            assert 128 <= amax / 2.0**S < 256       # the block's top binade lands on [128, 256)
        np.testing.assert_array_equal(qb, _torch_e4m3(blk / 2.0**S) * 2.0**S)
        assert np.all(np.abs(qb) / 2.0**S <= 256)       # no code needs more than the range


def _np_layer_aq(blobs, x64, idx, w, wl):
    """The MXFP8 layer in numpy: x and h quantised per block of 32 with torch's E4M3 rounding."""
    def q(v):
        out = np.empty_like(v)
        for b in range(0, v.size, 32):
            blk = v[b:b + 32]
            amax = np.abs(blk).max()
            S = -126 if amax == 0 else max(int(np.floor(np.log2(amax))) - 7, -126)
            out[b:b + 32] = _torch_e4m3((blk / 2.0**S).astype(np.float32)) * 2.0**S
        return out
    y = np.zeros_like(x64)
    for t in range(x64.shape[0]):
        xq = q(x64[t])
        for j in range(wl.top_k):
            Wg, Wu, Wd = expert_weights(blobs[idx[t, j]], wl.d_model, wl.d_ff, wl.wformat)
            h = silu(Wg @ xq) * (Wu @ xq)
            y[t] += w[t, j] * (Wd @ q(h))
    return y


def test_layer_actquant_matches_numpy():
    wl = TINY
    lay = synth.make_layer(wl, 0, 0, "cpu")
    x64 = oracle.to_f64(synth.make_x(wl, 0, "cpu"))
    blobs = [lay["blob"][e].numpy() for e in range(wl.n_experts)]
    wr = lay["router"].numpy()
    y, idx, w, _ = oracle.layer(x64, wr, None, blobs, wl.d_model, wl.d_ff, wl.top_k, wl.wformat, act_quant=1)
    want = _np_layer_aq(blobs, x64, idx, w, wl)
    np.testing.assert_allclose(y, want, rtol=1e-11, atol=1e-13 * np.abs(want).max())
    # the quantisation is real, of the size a single E4M3 term gives (about 2-3% rel-L2)
    y0, idx0, _, _ = oracle.layer(x64, wr, None, blobs, wl.d_model, wl.d_ff, wl.top_k, wl.wformat)
    np.testing.assert_array_equal(idx, idx0)            # the router sees x exactly
    err = float(np.linalg.norm(y - y0) / np.linalg.norm(y0))
    assert 3e-3 < err < 8e-2, err


def test_actquant_of_representable_input_keeps_x():
    """Inputs already on the MXFP8 grid of their blocks are left as they are."""
    v = np.concatenate([np.array([1.0, -0.5, 3.0, 0.0] * 8), np.array([2.0**-100, -3 * 2.0**-101] * 16)])
    np.testing.assert_array_equal(oracle.quant_mxfp8(v), v)
