"""The opt-in MXFP8 activation mode on the GPU against the oracle's mirrored mode: x and h enter the
FP4 x FP8 matrix cores as one E4M3 term per value (scale 2^(floor(log2 amax) - 7) per block of 32),
which halves the matrix-core work of the exact two-term mode.  The router still sees x exactly, so
indices stay bit-exact; outputs match the mirrored oracle (see gpu_util.tol)."""
import numpy as np
import pytest
import torch

import synth
from gpu_util import DeviceLayer, oracle_layer, rel_l2, run_layer, small, tol

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import routed_expert_ffn_router_amd as m      # must load: no fallback path exists


def _x(wl, T, tag):
    return synth.make_x(wl, 0, "cpu", tokens=T, tag=tag).to("cuda").contiguous()


def _check(dl, T, tag):
    wl = dl.wl
    x = _x(wl, T, tag)
    y, idx, _ = run_layer(m, dl, x)
    oy, oidx, _, _ = oracle_layer(dl, x, idx_hint=idx.cpu().numpy())
    np.testing.assert_array_equal(idx.cpu().numpy(), oidx)
    err = rel_l2(y.float().cpu().numpy(), oy)
    print(f"  T={T}: rel-L2 vs the mirrored oracle {err:.3e} (tol {tol(wl):.0e})")
    assert err <= tol(wl)
    return x, y


# fp32 tiny: 1, 4 fused few-token; 53 general few picks; 200 the many-pick GEMM (4 experts)
@pytest.mark.parametrize("kw,T", [(dict(), 1), (dict(), 4), (dict(), 53), (dict(n_experts=4), 200)])
def test_actquant_tiny_fp32(kw, T):
    wl = small("tiny", act_quant=1, **kw)
    print(f"mxfp8 activations tiny {kw} T={T}", flush=True)
    dl = DeviceLayer(m, wl)
    x, y = _check(dl, T, f"aqt{T}")
    # and it is a different computation from the exact mode (about 2-3% away)
    import dataclasses
    from gpu_util import shape_of
    y0 = torch.empty_like(x)
    exact = shape_of(m, dataclasses.replace(wl, act_quant=0))
    m.moe_layer(exact, x, T, dl.router, None, dl.table, None, None, y0, None, None, m.workspace(exact, T))
    torch.cuda.synchronize()
    assert rel_l2(y.cpu().numpy(), y0.cpu().numpy()) > 3e-3


@pytest.fixture(scope="module")
def glm_aq():
    return DeviceLayer(m, small("decode", n_experts=64, act_quant=1), host_gen=False)


@pytest.mark.parametrize("T", [1, 2, 5, 16, 40, 300])
def test_actquant_glm_shape(glm_aq, T):
    print(f"mxfp8 activations glm shape T={T}", flush=True)
    _check(glm_aq, T, f"aqg{T}")


@pytest.mark.parametrize("T", [64, 256])
def test_actquant_prefill_gemm_full_output(T):
    """Many picks per expert at the GLM width: the single-term many-pick GEMM (128-pick tiles)."""
    wl = small("decode", n_experts=4, top_k=2, act_quant=1)
    print(f"mxfp8 activations prefill GEMMs T={T}", flush=True)
    dl = DeviceLayer(m, wl, host_gen=False)
    _check(dl, T, f"aqp{T}")


def test_actquant_with_shared_expert():
    wl = small("decode", n_experts=32, act_quant=1, n_shared=1, routed_scaling=2.5)
    dl = DeviceLayer(m, wl, host_gen=False)
    for T in (1, 9, 40):
        _check(dl, T, f"aqs{T}")
