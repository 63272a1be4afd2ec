"""Renorm-skip on the GPU against the oracle (Strata-GLM blog, "Uncensoring without touching the
weights": picks with a tiny weight are dropped cleanly and the rest renormalised).  A logit bias
of -2.5 puts the top-8 logits around 0, where the sigmoid weights spread enough for a threshold of
0.11 to drop some picks of most tokens; dropped picks must come out as expert -1 with weight 0,
bit for bit where the oracle drops them, and the layer output must match the oracle's."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import DeviceLayer, oracle_layer, rel_l2, run_layer, small, tol

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import routed_expert_ffn_router_amd as m      # must load: no fallback path exists

TAU = 0.11


def _x(wl, T, tag):
    return synth.make_x(wl, 0, "cpu", tokens=T, tag=tag).to("cuda").contiguous()


def _biased(dl):
    dl.bias = torch.full((dl.wl.n_experts,), -2.5, dtype=torch.float32, device="cuda")
    return dl


@pytest.fixture(scope="module")
def glm64():
    return _biased(DeviceLayer(m, small("decode", n_experts=64, renorm_skip=TAU), host_gen=False))


# T=1: the one-token fused router; 3 and 16: the few-token fused router; 40 and 300: the general
# router, permute and GEMMs
@pytest.mark.parametrize("T", [1, 3, 16, 40, 300])
def test_renorm_skip_layer(glm64, T):
    dl = glm64
    wl = dl.wl
    print(f"renorm-skip layer T={T}", flush=True)
    x = _x(wl, T, f"rs{T}")
    y, idx, w = run_layer(m, dl, x)
    oy, oidx, ow, _ = oracle_layer(dl, x)
    gi = idx.cpu().numpy()
    np.testing.assert_array_equal(gi, oidx)
    np.testing.assert_allclose(w.cpu().numpy(), ow, rtol=2e-7, atol=1e-8)
    assert (oidx[:, 0] >= 0).all()
    if T >= 3:
        assert (oidx < 0).any(), "some picks are dropped"
    err = rel_l2(y.float().cpu().numpy(), oy)
    print(f"  dropped {(oidx < 0).mean():.2f} of picks; rel-L2 {err:.3e}")
    assert err <= tol(wl)


@pytest.mark.parametrize("T", [5, 33])
def test_renorm_skip_route_and_staged_calls(glm64, T):
    """moe_route with the threshold, then the staged permute / expert FFN / combine: the dropped
    picks take no position, and the staged result equals moe_layer's bit for bit."""
    dl = glm64
    wl = dl.wl
    x = _x(wl, T, f"rss{T}")
    y, idx, w = run_layer(m, dl, x)
    sh = dl.shape
    ws = m.workspace(sh, T)
    idx2 = torch.empty_like(idx)
    w2 = torch.empty_like(w)
    m.moe_route(sh, x, T, dl.router, dl.bias, idx2, w2, ws)
    off = torch.empty(wl.n_experts + 1, dtype=torch.int32, device="cuda")
    sp = torch.empty(T * wl.top_k, dtype=torch.int32, device="cuda")
    pp = torch.empty_like(sp)
    m.moe_permute(sh, idx2, T, off, sp, pp, ws, ws.numel())
    o = torch.empty(T * wl.top_k, wl.d_model, dtype=torch.float32, device="cuda")
    m.moe_expert_ffn(sh, dl.table, x, T, off, sp, o, ws)
    y2 = torch.empty_like(y)
    m.moe_combine(sh, o, w2, pp, T, None, y2)
    torch.cuda.synchronize()
    assert m.workspace_status(ws) == 0            # -1 is a dropped pick, not a refused id
    assert torch.equal(idx, idx2) and torch.equal(w, w2)
    dropped = (idx2 < 0).reshape(-1)
    assert dropped.any()
    assert (pp[dropped] == -1).all() and int(off[-1]) == int((~dropped).sum())
    _, oidx, ow = oracle.route(oracle.to_f64(x), dl.router.cpu().numpy(), dl.bias.cpu().numpy(), wl.top_k, TAU)
    np.testing.assert_array_equal(idx2.cpu().numpy(), oidx)
    if T > 16:       # the staged calls and the layer take the same kernels for many tokens
        assert torch.equal(y.view(torch.int16), y2.view(torch.int16))
    else:
        assert rel_l2(y2.float().cpu().numpy(), y.float().cpu().numpy()) <= tol(wl)


@pytest.mark.parametrize("T", [1, 6, 40])
def test_renorm_skip_nvfp4(T):
    wl = small("tiny", wformat=synth.NVFP4, d_model=512, d_ff=256, n_experts=32, top_k=6,
               act_dtype=synth.BF16, renorm_skip=0.12)
    dl = _biased(DeviceLayer(m, wl))
    print(f"renorm-skip nvfp4 T={T}", flush=True)
    x = _x(wl, T, f"rsnv{T}")
    y, idx, w = run_layer(m, dl, x)
    oy, oidx, ow, _ = oracle_layer(dl, x)
    np.testing.assert_array_equal(idx.cpu().numpy(), oidx)
    assert rel_l2(y.float().cpu().numpy(), oy) <= tol(wl)
