"""moe_layer_noalloc (the library's own scratch array instead of a workspace) against moe_layer on
the same inputs, through the C ABI: bit-identical routing and output, on calls in a row of falling
token counts (so the second call finds the first call's contents in the array), across the
few-token fused path and the general path, and a refused size beyond the array."""
import ctypes

import numpy as np
import pytest
import torch

import synth
from gpu_util import DeviceLayer, oracle_layer, rel_l2, small, tol

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import routed_expert_ffn_router_amd as m      # must load: no fallback path exists


def _x(wl, T, tag):
    return synth.make_x(wl, 0, "cpu", tokens=T, tag=tag).to("cuda").contiguous()


def _outputs(wl, T, x):
    return (torch.empty_like(x), torch.empty(T, wl.top_k, dtype=torch.int32, device="cuda"),
            torch.empty(T, wl.top_k, dtype=torch.float32, device="cuda"))


@pytest.fixture(scope="module")
def layer():
    return DeviceLayer(m, small("decode", n_experts=64), host_gen=False)


@pytest.mark.parametrize("Ts", [(16, 1), (40, 3), (2, 1)])
def test_noalloc_matches_layer(layer, Ts):
    dl = layer
    wl = dl.wl
    for T in Ts:
        print(f"no-alloc layer T={T} (sequence {Ts})", flush=True)
        x = _x(wl, T, f"na{T}")
        res = _x(wl, T, f"nares{T}")
        y0, i0, w0 = _outputs(wl, T, x)
        m.moe_layer(dl.shape, x, T, dl.router, None, dl.table, None, res, y0, i0, w0, m.workspace(dl.shape, T))
        y1, i1, w1 = _outputs(wl, T, x)
        rc = m.library().moe_layer_noalloc(ctypes.byref(dl.shape), x.data_ptr(), T, dl.router.data_ptr(), None,
                                           dl.table.data_ptr(), res.data_ptr(), y1.data_ptr(), i1.data_ptr(),
                                           w1.data_ptr(), torch.cuda.current_stream().cuda_stream)
        assert rc == m.MOE_OK
        torch.cuda.synchronize()
        assert torch.equal(i0, i1) and torch.equal(w0, w1)
        assert torch.equal(y0.view(torch.int16), y1.view(torch.int16))
        # and the oracle, to the parity bar
        oy, oidx, _, _ = oracle_layer(dl, x, idx_hint=i1.cpu().numpy(), residual=res)
        np.testing.assert_array_equal(i1.cpu().numpy(), oidx)
        assert rel_l2(y1.float().cpu().numpy(), oy) <= tol(wl)


def test_noalloc_refuses_beyond_its_array(layer):
    dl = layer
    T = 4096
    assert m.moe_workspace_bytes(dl.shape, T) > (32 << 20)
    rc = m.library().moe_layer_noalloc(ctypes.byref(dl.shape), 1 << 20, T, 1 << 20, None, 1 << 20, None, 2 << 20,
                                       None, None, torch.cuda.current_stream().cuda_stream)
    assert rc == m.MOE_ERR_WORKSPACE
