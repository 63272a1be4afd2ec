"""The seeded input generators: quantiser rounding, determinism, workload structure."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import synth


def _mx_codes_for(values, scale_exp=0):
    """Quantise one block whose amax fixes the shared exponent to ``scale_exp``."""
    blk = torch.zeros(32)
    blk[0] = 4.0 * 2.0**scale_exp            # amax = 4 * 2^e  -> floor(log2) - 2 = e
    blk[1:1 + len(values)] = torch.tensor(values) * 2.0**scale_exp
    q, s = synth.quantize_mx(blk.reshape(1, 32))
    assert int(s[0, 0]) == 127 + scale_exp
    deq = oracle.dequant(q.numpy(), s.numpy(), 1, 32, oracle.MXFP4)[0]
    return deq[1:1 + len(values)] / 2.0**scale_exp


def test_rne_ties_in_scaled_units():
    vals = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.25, -0.75, -5.0]
    want = [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0, -0.0, -1.0, -4.0]
    np.testing.assert_array_equal(_mx_codes_for(vals, 0), want)
    np.testing.assert_array_equal(_mx_codes_for(vals, -5), want)


def test_saturation_at_six():
    blk = torch.zeros(1, 32)
    blk[0, 0] = 7.9          # amax 7.9 -> exponent 0, 7.9 saturates to 6
    blk[0, 1] = 7.0
    q, s = synth.quantize_mx(blk)
    deq = oracle.dequant(q.numpy(), s.numpy(), 1, 32, oracle.MXFP4)[0]
    assert deq[0] == 6.0 and deq[1] == 6.0


def test_zero_block():
    q, s = synth.quantize_mx(torch.zeros(2, 64))
    assert int(q.sum()) == 0 and int(s.sum()) == 0


def test_quantiser_error_is_small():
    w = torch.randn(64, 256) * 0.02
    q, s = synth.quantize_mx(w)
    deq = oracle.dequant(q.numpy(), s.numpy(), 64, 256, oracle.MXFP4)
    rel = np.linalg.norm(deq - w.double().numpy()) / np.linalg.norm(w.double().numpy())
    assert rel < 0.2
    qn, sn, ts = synth.quantize_nv(w)
    deqn = oracle.dequant(qn.numpy(), sn.numpy(), 64, 256, oracle.NVFP4, ts)
    reln = np.linalg.norm(deqn - w.double().numpy()) / np.linalg.norm(w.double().numpy())
    assert reln < 0.15


def test_generation_is_deterministic_and_subset_independent():
    wl = synth.WORKLOADS["tiny"]
    a = synth.make_experts(wl, 0, 0)
    b = synth.make_experts(wl, 0, 0, group=3)
    c = synth.make_experts(wl, 0, 0, experts=[5, 2])
    assert torch.equal(a, b)
    assert torch.equal(a[5], c[5]) and torch.equal(a[2], c[2]) and int(c[0].sum()) == 0
    d = synth.make_experts(wl, 1, 0)
    assert not torch.equal(a, d)
    assert torch.equal(synth.make_x(wl, 0), synth.make_x(wl, 0))


def test_blob_offsets_match_oracle_stride():
    for (d, f, fmt) in [(256, 128, 0), (4096, 2048, 0), (6144, 2048, 1), (256, 128, 1)]:
        assert synth.blob_offsets(d, f, fmt)["stride"] == oracle.blob_stride(d, f, fmt)


def test_workload_shapes():
    W = synth.WORKLOADS
    assert (W["decode"].d_model, W["decode"].d_ff, W["decode"].n_experts, W["decode"].top_k) == (4096, 2048, 288, 8)
    assert W["decode"].n_layers == 42 and W["prefill"].tokens == 4096 and W["batched"].tokens == 64
    assert W["nvfp4_prefill"].tokens == 2048 and W["nvfp4_decode"].n_experts == 256


def test_flat_router_gives_unit_logits():
    wl = synth.WORKLOADS["prefill"]
    x = synth.make_x(wl, tokens=64).float()
    wr = synth.make_router(wl)
    l = x @ wr.T
    assert 0.85 < float(l.std()) < 1.15


def test_skew_calibration():
    """Hottest 35% of experts take ~74% of picks ("A hot expert cache ...", section
    "Offload more, cache the hot experts")."""
    share = synth.skew_share(synth.SKEW_ALPHA_288, tokens=8000)
    assert abs(share - 0.74) < 0.02
    assert abs(synth.skew_share(0.0, tokens=8000) - 0.35) < 0.03   # flat routing
