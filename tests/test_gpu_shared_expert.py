"""The shared expert on the GPU against the oracle: one more expert (table entry n_experts) that
every token passes through with weight 1, outside the routed scaling ("Project Maya", section
"What is in the 96.5 GB": the shared experts beside the routed ones; routed_scaling_factor 2.5
from the windlass README's negative controls).  It runs in the same launches as the routed
experts - in decode, one more tile in the gate/up and down+combine kernels."""
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


@pytest.fixture(scope="module")
def glm_shared():
    wl = small("decode", n_experts=64, n_shared=1, routed_scaling=2.5)
    return DeviceLayer(m, wl, host_gen=False)


# 1, 2: the one-token / few-token fused paths with h in LDS; 5, 16: the few-token path reading h
# from memory; 40, 300: the general router, permute, plan and GEMMs (many picks per expert at 300)
@pytest.mark.parametrize("T", [1, 2, 5, 16, 40, 300])
def test_shared_expert_layer(glm_shared, T):
    dl = glm_shared
    wl = dl.wl
    print(f"shared expert layer T={T}", flush=True)
    x = _x(wl, T, f"sh{T}")
    res = _x(wl, T, f"shres{T}")
    y, idx, w = run_layer(m, dl, x, residual=res)
    oy, oidx, _, _ = oracle_layer(dl, x, residual=res)
    np.testing.assert_array_equal(idx.cpu().numpy(), oidx)
    # compare the MoE part (y - residual): the residual would hide an error in it
    r64 = res.float().cpu().double().numpy()
    err = rel_l2(y.float().cpu().numpy() - r64, oy - r64)
    print(f"  rel-L2 of y - residual {err:.3e}")
    assert err <= 2 * tol(wl)       # y is rounded to bf16 around the residual: one more rounding


@pytest.mark.parametrize("T", [3, 40])
def test_shared_expert_staged_calls(glm_shared, T):
    """moe_expert_ffn writes the shared expert's rows at T*k + t; moe_combine adds them."""
    dl = glm_shared
    wl = dl.wl
    sh = dl.shape
    x = _x(wl, T, f"shs{T}")
    y, idx, w = run_layer(m, dl, x)
    ws = m.workspace(sh, T)
    off = torch.empty(wl.n_experts + 1, dtype=torch.int32, device="cuda")
    sp = torch.empty(T * wl.top_k, dtype=torch.int32, device="cuda")
    pp = torch.empty_like(sp)
    m.moe_permute(sh, idx, T, off, sp, pp)
    o = torch.empty(T * wl.top_k + T, wl.d_model, dtype=torch.float32, device="cuda")
    m.moe_expert_ffn(sh, dl.table, x, T, off, sp, o, ws)
    y2 = torch.empty_like(y)
    m.moe_combine(sh, o, w, pp, T, None, y2)
    torch.cuda.synchronize()
    oy, _, _, _ = oracle_layer(dl, x)
    assert rel_l2(y2.float().cpu().numpy(), oy) <= tol(wl)
    if T > 16:
        assert torch.equal(y.view(torch.int16), y2.view(torch.int16))


def test_shared_expert_with_renorm_skip(glm_shared):
    import dataclasses
    dl = glm_shared
    dl2 = DeviceLayer.__new__(DeviceLayer)
    dl2.__dict__.update(dl.__dict__)
    dl2.wl = dataclasses.replace(dl.wl, renorm_skip=0.11)
    from gpu_util import shape_of
    dl2.shape = shape_of(m, dl2.wl)
    dl2.bias = torch.full((dl.wl.n_experts,), -2.5, dtype=torch.float32, device="cuda")
    for T in (1, 7, 40):
        x = _x(dl2.wl, T, f"shrs{T}")
        y, idx, w = run_layer(m, dl2, x)
        oy, oidx, _, _ = oracle_layer(dl2, x)
        np.testing.assert_array_equal(idx.cpu().numpy(), oidx)
        assert rel_l2(y.float().cpu().numpy(), oy) <= tol(dl2.wl)


@pytest.mark.parametrize("T,staged", [(1, False), (9, False), (9, True), (120, False), (120, True)])
def test_shared_expert_nvfp4(T, staged):
    wl = small("tiny", wformat=synth.NVFP4, d_model=512, d_ff=256, n_experts=24, top_k=4,
               act_dtype=synth.BF16, n_shared=1, routed_scaling=2.5)
    dl = DeviceLayer(m, wl)
    print(f"shared expert nvfp4 T={T} staged={staged}", flush=True)
    x = _x(wl, T, f"shnv{T}")
    y = torch.empty_like(x)
    idx = torch.empty(T, wl.top_k, dtype=torch.int32, device="cuda")
    staging = torch.empty(wl.n_experts, dl.stride, dtype=torch.uint8, device="cuda") if staged else None
    m.moe_layer(dl.shape, x, T, dl.router, None, dl.table, staging, None, y, idx, None, m.workspace(dl.shape, T))
    torch.cuda.synchronize()
    oy, oidx, _, _ = oracle_layer(dl, x)
    np.testing.assert_array_equal(idx.cpu().numpy(), oidx)
    assert rel_l2(y.float().cpu().numpy(), oy) <= tol(wl)


def test_shared_expert_fp32_tiny():
    wl = small("tiny", n_shared=1, routed_scaling=2.5)
    dl = DeviceLayer(m, wl)
    for T in (1, 4, 53):
        x = _x(wl, T, f"sht{T}")
        y, idx, _ = run_layer(m, dl, x)
        oy, oidx, _, _ = oracle_layer(dl, x)
        np.testing.assert_array_equal(idx.cpu().numpy(), oidx)
        assert rel_l2(y.float().cpu().numpy(), oy) <= tol(wl)
