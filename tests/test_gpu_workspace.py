"""The workspace contract on the GPU: preparation by moe_workspace_init (a dirty workspace, once
prepared, gives results bit-identical to a fresh one), the status word (a router whose wait gives
up reports it and leaves outputs that fail loudly; refused expert ids are reported and left out),
and the per-call observer."""
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


def _call(dl, x, ws, residual=None):
    wl = dl.wl
    T = x.shape[0]
    y = torch.empty_like(x)
    idx = torch.empty(T, wl.top_k, dtype=torch.int32, device="cuda")
    w = torch.empty(T, wl.top_k, dtype=torch.float32, device="cuda")
    m.moe_layer(dl.shape, x, T, dl.router, dl.bias, dl.table, None, residual, y, idx, w, ws)
    torch.cuda.synchronize()
    return y, idx, w


@pytest.fixture(scope="module")
def mid_layer():
    # 64 experts of the GLM width: the few-token router keeps its table in LDS
    wl = small("decode", n_experts=64)
    return DeviceLayer(m, wl, host_gen=False)


@pytest.mark.parametrize("T", [1, 5, 16, 40])
def test_dirty_workspace_once_prepared_matches_fresh(mid_layer, T):
    dl = mid_layer
    print(f"0xFF workspace, prepared, T={T}", flush=True)
    x = _x(dl.wl, T, tag=f"dirty{T}")
    y0, i0, w0 = run_layer(m, dl, x)
    ws = torch.full((m.moe_workspace_bytes(dl.shape, T),), 0xFF, dtype=torch.uint8, device="cuda")
    m.moe_workspace_init(dl.shape, T, ws)
    for _ in range(2):               # and again on the same workspace
        y1, i1, w1 = _call(dl, x, ws)
        assert m.workspace_status(ws) == 0
        assert torch.equal(i0, i1) and torch.equal(w0, w1)
        assert torch.equal(y0.view(torch.int16), y1.view(torch.int16))


@pytest.mark.parametrize("T", [1, 3, 16])
def test_router_wait_that_gives_up_fails_loudly(mid_layer, T):
    """poll_limit < 0 makes the few-token router give up at once (every kernel still ends normally):
    the status word reports it, indices are -1, weights and y NaN; the workspace stays refused
    until it is prepared again, after which results equal a fresh workspace's."""
    dl = mid_layer
    wl = dl.wl
    print(f"router gives up, T={T}", flush=True)
    x = _x(wl, T, tag=f"to{T}")
    ws = m.workspace(dl.shape, T)
    m.moe_workspace_init(dl.shape, T, ws, poll_limit=-1)
    y, idx, w = _call(dl, x, ws, residual=x)
    assert m.workspace_status(ws) == m.MOE_WS_ROUTE_TIMEOUT
    assert (idx == -1).all()
    assert torch.isnan(w).all()
    assert torch.isnan(y.float()).all()
    # still refused: the status is sticky, and the router does not trust its hand-over slots
    m.moe_workspace_init(dl.shape, T, ws, poll_limit=0)      # default limit, status cleared
    ws_status_set = ws.clone()
    ws_status_set[:4] = torch.tensor([m.MOE_WS_ROUTE_TIMEOUT], dtype=torch.int32).view(torch.uint8).cuda()
    y2, idx2, _ = _call(dl, x, ws_status_set)
    assert (idx2 == -1).all() and torch.isnan(y2.float()).all()
    # prepared again: as fresh
    y3, i3, w3 = _call(dl, x, ws)
    assert m.workspace_status(ws) == 0
    y0, i0, w0 = run_layer(m, dl, x)
    assert torch.equal(i0, i3) and torch.equal(w0, w3)
    assert torch.equal(y0.view(torch.int16), y3.view(torch.int16))


def test_generous_poll_limit_changes_nothing(mid_layer):
    dl = mid_layer
    x = _x(dl.wl, 2, tag="gen")
    ws = m.workspace(dl.shape, 2)
    m.moe_workspace_init(dl.shape, 2, ws, poll_limit=1 << 24)
    y1, i1, _ = _call(dl, x, ws)
    y0, i0, _ = run_layer(m, dl, x)
    assert m.workspace_status(ws) == 0
    assert torch.equal(i0, i1) and torch.equal(y0.view(torch.int16), y1.view(torch.int16))


@pytest.mark.parametrize("T,k,E", [(9, 4, 32), (2000, 8, 288)])
def test_permute_refuses_bad_ids_and_skips_dropped(T, k, E):
    """Expert id -1 is a dropped pick, ids >= E or < -1 are refused (status bit); both take no
    sorted position (pick_pos -1), the valid picks are sorted exactly as without them, the
    positions past offsets[E] hold -1, and the combine leaves such picks out."""
    g = torch.Generator().manual_seed(T)
    idx = torch.stack([torch.randperm(E, generator=g)[:k] for _ in range(T)]).to(torch.int32)
    idx[0, k - 1] = -1
    idx[T // 2, 1] = E + 3
    idx[T - 1, 0] = -7
    idx[1, k - 1] = -1
    flat = idx.reshape(-1).numpy()
    valid = (flat >= 0) & (flat < E)
    # expected: a stable counting sort of the valid picks by expert
    order = np.flatnonzero(valid)[np.argsort(flat[valid], kind="stable")]
    counts = np.bincount(flat[valid], minlength=E)
    want_off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    want_sp = np.full(T * k, -1, dtype=np.int32)
    want_sp[:order.size] = order
    want_pp = np.full(T * k, -1, dtype=np.int32)
    want_pp[order] = np.arange(order.size)
    shape = m.make_shape(256, 128, E, k)
    for with_ws in (False, True):
        off = torch.empty(E + 1, dtype=torch.int32, device="cuda")
        sp = torch.full((T * k,), 12345, dtype=torch.int32, device="cuda")
        pp = torch.full((T * k,), 12345, dtype=torch.int32, device="cuda")
        ws = m.workspace(shape, T) if with_ws else None
        torch.cuda.synchronize()
        m.moe_permute(shape, idx.cuda(), T, off, sp, pp, ws, 0 if ws is None else ws.numel())
        torch.cuda.synchronize()
        np.testing.assert_array_equal(off.cpu().numpy(), want_off)
        np.testing.assert_array_equal(sp.cpu().numpy(), want_sp)
        np.testing.assert_array_equal(pp.cpu().numpy(), want_pp)
        if with_ws:
            assert m.workspace_status(ws) == m.MOE_WS_BAD_EXPERT_ID
    # combine: y[t] = sum over picks with a position of w * o[pos]
    d = 256
    o = torch.randn(T * k, d, generator=g).cuda()
    wts = torch.rand(T, k, generator=g).cuda()
    y = torch.empty(T, d, dtype=torch.float32, device="cuda")
    sh32 = m.make_shape(d, 128, E, k, act_dtype=m.MOE_DT_F32)
    m.moe_combine(sh32, o, wts, pp, T, None, y)
    torch.cuda.synchronize()
    on, wn, ppn = o.cpu().double().numpy(), wts.cpu().double().numpy(), pp.cpu().numpy()
    want = np.zeros((T, d))
    for t in range(T):
        for j in range(k):
            if ppn[t * k + j] >= 0:
                want[t] += wn[t, j] * on[ppn[t * k + j]]
    np.testing.assert_allclose(y.cpu().double().numpy(), want, rtol=1e-5, atol=1e-5)


def test_observer_sees_every_kernel(mid_layer):
    dl = mid_layer
    x = _x(dl.wl, 1, tag="obs")
    seen = []
    obs = m.make_observer(trace=lambda name, phase, stream: seen.append((name, phase)))
    y = torch.empty_like(x)
    m.moe_layer(dl.shape, x, 1, dl.router, None, dl.table, None, None, y, None, None,
                m.workspace(dl.shape, 1), observer=obs)
    torch.cuda.synchronize()
    names = [n for n, p in seen if p == 0]
    assert names == ["route_small", "gemm_gate_up", "down_combine"]
    assert [p for _, p in seen] == [0, 1] * 3
    # the hooks belong to that call only: a plain call afterwards sees none of them
    seen.clear()
    run_layer(m, dl, x)
    assert seen == []
