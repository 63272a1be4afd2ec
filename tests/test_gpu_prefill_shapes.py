"""Whole-output parity of the many-pick ("prefill") expert GEMMs at the GLM-5.3 layer shapes.

The 4096-token chunk runs the straight-line instances of the LDS-tiled MXFP4 GEMM (K = d_model 4096
for gate/up, d_ff 2048 for down) and the NVFP4 tiled GEMM at d_model 6144.  The oracle cannot
afford every token of that chunk, so these tests reach the same kernel instances with fewer experts
(the many-pick GEMM is chosen once a layer has more than 8 picks per expert) and compare EVERY token
of the output: several tiles per expert, ragged last tiles, the fp32 (four-term) instances too.
"""
import numpy as np
import pytest
import torch

import synth
from gpu_util import DeviceLayer, oracle_layer, rel_l2, run_layer, small, tol

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import routed_expert_ffn_router_amd as m      # must load: no fallback path exists


def _x(wl, T, seed=0, tag="x"):
    return synth.make_x(wl, seed, "cpu", tokens=T, tag=tag).to("cuda").contiguous()


# (E, k, T, dtype): every case has T*k > 8E, so gate/up and down run the many-pick GEMM's
# straight-line instances at K = 4096 and 2048; bf16 uses two activation terms, fp32 four
@pytest.mark.parametrize("E,k,T,dt", [
    (4, 2, 64, synth.BF16),        # one ragged tile per expert
    (4, 2, 48, synth.F32),         # four-term instances (32-pick tiles)
    (16, 8, 512, synth.BF16),      # four tiles per expert and a ragged tail, tiles on every XCD
])
def test_mxfp4_prefill_gemm_full_output(E, k, T, dt):
    wl = small("decode", n_experts=E, top_k=k, act_dtype=dt)
    print(f"mxfp4 glm-shape prefill GEMMs E={E} k={k} T={T} dtype={dt}", flush=True)
    dl = DeviceLayer(m, wl, host_gen=False)
    x = _x(wl, T, tag=f"pf{E}_{T}")
    y, idx, w = run_layer(m, dl, x)
    oy, oidx, ow, _ = oracle_layer(dl, x, idx_hint=idx.cpu().numpy())
    np.testing.assert_array_equal(idx.cpu().numpy(), oidx)
    counts = np.bincount(oidx.reshape(-1), minlength=E)
    assert counts.min() > 8, "every expert takes the many-pick path"
    err = rel_l2(y.float().cpu().numpy(), oy)
    worst_tok = max(rel_l2(y[t].float().cpu().numpy(), oy[t]) for t in range(T))
    print(f"  rel-L2 {err:.3e} (worst token {worst_tok:.3e}, tol {tol(wl):.0e})")
    assert err <= tol(wl)
    assert worst_tok <= 4 * tol(wl)      # no token (tile slot) is wrong while the rest hide it


@pytest.mark.parametrize("staged", [False, True])
def test_nvfp4_prefill_gemm_full_output(staged):
    """NVFP4 at d_model 6144: 16 experts, k=8, T=256 (128 picks per expert, two 64-pick tiles each)."""
    wl = small("nvfp4_prefill", n_experts=16)
    T = 256
    print(f"nvfp4 d=6144 prefill GEMMs staged={staged}", flush=True)
    dl = DeviceLayer(m, wl, host_gen=False)
    x = _x(wl, T, tag="nvpf")
    yy = torch.empty_like(x)
    idx = torch.empty(T, wl.top_k, dtype=torch.int32, device="cuda")
    w = torch.empty(T, wl.top_k, dtype=torch.float32, device="cuda")
    ws = m.workspace(dl.shape, T)
    staging = torch.empty(16, dl.stride, dtype=torch.uint8, device="cuda") if staged else None
    m.moe_layer(dl.shape, x, T, dl.router, None, dl.table, staging, None, yy, idx, w, ws)
    torch.cuda.synchronize()
    oy, oidx, _, _ = oracle_layer(dl, x, idx_hint=idx.cpu().numpy())
    np.testing.assert_array_equal(idx.cpu().numpy(), oidx)
    err = rel_l2(yy.float().cpu().numpy(), oy)
    worst_tok = max(rel_l2(yy[t].float().cpu().numpy(), oy[t]) for t in range(T))
    print(f"  rel-L2 {err:.3e} (worst token {worst_tok:.3e})")
    assert err <= tol(wl)
    assert worst_tok <= 4 * tol(wl)
