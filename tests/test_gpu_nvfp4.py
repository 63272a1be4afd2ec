"""GPU parity of the NVFP4 path (E2M1 codes, E4M3 scale per 16, fp32 tensor scale) and of the
device-list gather into staging, through the C ABI, against the fp64 CPU oracle.

Router indices are bit-exact; outputs are within rel-L2 1e-4 (fp32 activations) or 8e-3 (bf16
activations) of the oracle; staged copies are byte-identical to their sources, and a layer run
from staging equals the same layer run in place bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import DeviceLayer, oracle_layer, rel_l2, run_layer, small, tol

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import routed_expert_ffn_router_amd as m      # must load: no fallback path exists


def _x(wl, T, seed=0, tag="x"):
    return synth.make_x(wl, seed, "cpu", tokens=T, tag=tag).to("cuda").contiguous()


def _layer(m, dl, x, staging=None, residual=None):
    wl = dl.wl
    T = x.shape[0]
    y = torch.empty_like(x)
    idx = torch.empty(T, wl.top_k, dtype=torch.int32, device="cuda")
    w = torch.empty(T, wl.top_k, dtype=torch.float32, device="cuda")
    ws = m.workspace(dl.shape, T)
    m.moe_layer(dl.shape, x, T, dl.router, dl.bias, dl.table, staging, residual, y, idx, w, ws)
    torch.cuda.synchronize()
    return y, idx, w


@pytest.mark.parametrize("kw,T", [
    (dict(), 4),                                                   # fp32 activations
    (dict(act_dtype=synth.BF16), 1),
    (dict(act_dtype=synth.BF16), 37),                              # ragged tiles
    (dict(d_model=512, d_ff=384, n_experts=24, top_k=3), 9),        # K not a multiple of 512
    (dict(act_dtype=synth.BF16, n_experts=8, top_k=8), 53),        # every expert, tiles of 8 picks
    (dict(d_model=384, d_ff=256, n_experts=40, top_k=4, act_dtype=synth.BF16), 300),
    # K past the LDS-decoded few-pick kernel's 8192: gate/up (K = d_model) on the tile GEMM, 12
    # blocks of 32 rows (not a multiple of the 8 XCD lanes); then down (K = d_ff, 65 steps of 128)
    (dict(d_model=9216, d_ff=384, n_experts=8, top_k=2, act_dtype=synth.BF16), 13),
    (dict(d_model=384, d_ff=8320, n_experts=8, top_k=2), 7),
])
def test_nvfp4_layer_small(kw, T):
    wl = small("tiny", wformat=synth.NVFP4, **kw)
    print(f"nvfp4 layer parity {kw} T={T}", flush=True)
    dl = DeviceLayer(m, wl)
    x = _x(wl, T)
    y, idx, _ = run_layer(m, dl, x)
    oy, oidx, _, _ = oracle_layer(dl, x)
    np.testing.assert_array_equal(idx.cpu().numpy(), oidx)
    err = rel_l2(y.float().cpu().numpy(), oy)
    print(f"  rel-L2 {err:.3e} (tol {tol(wl):.0e})")
    assert err <= tol(wl)


def test_nvfp4_expert_ffn_rows():
    """moe_expert_ffn's per-pick rows against the oracle's, residual and scaling through the layer."""
    wl = small("tiny", wformat=synth.NVFP4, d_model=512, d_ff=256, n_experts=32, top_k=4, routed_scaling=2.5)
    dl = DeviceLayer(m, wl)
    T = 21
    x = _x(wl, T)
    res = _x(wl, T, tag="res")
    y, idx, w = _layer(m, dl, x, residual=res)
    oy, oidx, _, _ = oracle_layer(dl, x, residual=res)
    np.testing.assert_array_equal(idx.cpu().numpy(), oidx)
    assert rel_l2(y.float().cpu().numpy(), oy) <= tol(wl)
    sh = dl.shape
    off = torch.empty(wl.n_experts + 1, dtype=torch.int32, device="cuda")
    sp = torch.empty(T * wl.top_k, dtype=torch.int32, device="cuda")
    pp = torch.empty_like(sp)
    m.moe_permute(sh, idx, T, off, sp, pp)
    o = torch.empty(T * wl.top_k, wl.d_model, dtype=torch.float32, device="cuda")
    m.moe_expert_ffn(sh, dl.table, x, T, off, sp, o, m.workspace(sh, T))
    torch.cuda.synchronize()
    ooff, osp, _ = oracle.permute(idx.cpu().numpy(), wl.n_experts)
    oo = oracle.expert_ffn(dl.host_blobs(idx.cpu().numpy().reshape(-1)), wl.d_model, wl.d_ff, wl.wformat,
                           oracle.to_f64(x), wl.top_k, ooff, osp)
    err = rel_l2(o.cpu().numpy(), oo)
    print(f"  expert rows rel-L2 {err:.3e}")
    assert err <= tol(wl)


def test_gather_copies_bytes_and_table():
    wl = small("tiny", wformat=synth.NVFP4, n_experts=20)
    dl = DeviceLayer(m, wl)
    lst = torch.tensor([7, 0, 19, 7, 3], dtype=torch.int32, device="cuda")
    n = lst.numel()
    staging = torch.zeros(n, dl.stride, dtype=torch.uint8, device="cuda")
    staged = torch.zeros(n * m.EXPERT_BYTES, dtype=torch.uint8, device="cuda")
    m.moe_gather_experts(dl.shape, dl.table, lst, n, staging, staged)
    torch.cuda.synchronize()
    stride = m.moe_blob_stride(dl.shape)
    for i, e in enumerate(lst.tolist()):
        assert torch.equal(staging[i, :stride], dl.blob[e, :stride]), f"slot {i} (expert {e})"
    tab = staged.cpu().numpy().view(np.uint64).reshape(n, m.EXPERT_BYTES // 8)
    base = staging.data_ptr()
    for i in range(n):
        assert int(tab[i, 0]) == base + i * dl.stride          # gate_q points at the slot


@pytest.mark.parametrize("kw,T", [
    (dict(act_dtype=synth.BF16), 6),                                          # one group
    (dict(act_dtype=synth.BF16, n_experts=160, top_k=8, d_model=256, d_ff=128), 64),   # three groups
])
def test_nvfp4_layer_staged_equals_in_place(kw, T):
    wl = small("tiny", wformat=synth.NVFP4, **kw)
    print(f"nvfp4 staged vs in place {kw} T={T}", flush=True)
    dl = DeviceLayer(m, wl)
    x = _x(wl, T)
    y0, idx0, _ = _layer(m, dl, x)
    staging = torch.empty(min(wl.n_experts, 64), dl.stride, dtype=torch.uint8, device="cuda")
    y1, idx1, _ = _layer(m, dl, x, staging=staging)
    assert torch.equal(idx0, idx1)
    assert torch.equal(y0.view(torch.int16), y1.view(torch.int16))
    oy, oidx, _, _ = oracle_layer(dl, x)
    np.testing.assert_array_equal(idx1.cpu().numpy(), oidx)
    assert rel_l2(y1.float().cpu().numpy(), oy) <= tol(wl)


def test_staging_rejected_for_mxfp4():
    wl = small("tiny")
    dl = DeviceLayer(m, wl)
    x = _x(wl, 2)
    staging = torch.empty(16, dl.stride, dtype=torch.uint8, device="cuda")
    with pytest.raises(m.MoeError) as ei:
        _layer(m, dl, x, staging=staging)
    assert ei.value.status == m.MOE_ERR_INVALID


# ---------------------------------------------------------------------------------------------
# the NVFP4 configuration at full size (d_model 6144, d_ff 2048, 256 experts, top-8)
# ---------------------------------------------------------------------------------------------

def test_nvfp4_few_token_calls_repeat_on_one_workspace():
    """Few-token calls (the fused router, in place) of different token counts in turn on one
    workspace, with the shared expert and a residual, give exactly what the staged path (the
    general router and a separate gather) gives, every time: nothing a call leaves in the
    workspace changes the next one."""
    wl = small("tiny", wformat=synth.NVFP4, d_model=512, d_ff=256, n_experts=24, top_k=4,
               act_dtype=synth.BF16, n_shared=1, routed_scaling=2.5)
    dl = DeviceLayer(m, wl)
    Ts = (5, 1, 16, 3)
    xs = {T: _x(wl, T, tag=f"rep{T}") for T in Ts}
    rs = {T: _x(wl, T, tag=f"rres{T}") for T in Ts}
    staging = torch.empty(wl.n_experts, dl.stride, dtype=torch.uint8, device="cuda")
    ref = {T: _layer(m, dl, xs[T], staging=staging, residual=rs[T])[0] for T in Ts}
    ws = m.workspace(dl.shape, 16)
    for rnd in range(5):
        for T in Ts:
            y = torch.empty_like(xs[T])
            idx = torch.empty(T, wl.top_k, dtype=torch.int32, device="cuda")
            m.moe_layer(dl.shape, xs[T], T, dl.router, dl.bias, dl.table, None, rs[T], y, idx, None, ws)
            torch.cuda.synchronize()
            assert torch.equal(y.view(torch.int16), ref[T].view(torch.int16)), (rnd, T)
    oy, oidx, _, _ = oracle_layer(dl, xs[5], residual=rs[5])
    assert rel_l2(ref[5].float().cpu().numpy(), oy) <= tol(wl)


@pytest.fixture(scope="module")
def nv_layer():
    wl = synth.WORKLOADS["nvfp4_decode"]
    print("generating a 256-expert NVFP4 layer in HBM", flush=True)
    return DeviceLayer(m, wl, layer=0, host_gen=False)


@pytest.mark.parametrize("T", [1, 3])
def test_nvfp4_decode_full_size(nv_layer, T):
    dl = nv_layer
    wl = dl.wl
    print(f"nvfp4 full size T={T}", flush=True)
    x = _x(wl, T, tag=f"x{T}")
    y0, idx0, _ = _layer(m, dl, x)
    staging = torch.empty(64, dl.stride, dtype=torch.uint8, device="cuda")
    y1, idx1, _ = _layer(m, dl, x, staging=staging)
    assert torch.equal(y0.view(torch.int16), y1.view(torch.int16))
    oy, oidx, _, _ = oracle_layer(dl, x, idx_hint=idx0.cpu().numpy())
    np.testing.assert_array_equal(idx0.cpu().numpy(), oidx)
    err = rel_l2(y0.float().cpu().numpy(), oy)
    print(f"  rel-L2 {err:.3e}")
    assert err <= tol(wl)


def test_nvfp4_prefill_sampled(nv_layer):
    """T=2048 with staging (four groups of 64 experts): routing bit-exact on every token,
    output checked on sampled tokens."""
    dl = nv_layer
    wl = dl.wl
    T = 2048
    print("nvfp4 prefill T=2048 staged", flush=True)
    x = _x(wl, T, tag="prefill")
    staging = torch.empty(64, dl.stride, dtype=torch.uint8, device="cuda")
    y, idx, _ = _layer(m, dl, x, staging=staging)
    _, oidx, _ = oracle.route(oracle.to_f64(x), dl.router.cpu().numpy(), None, wl.top_k)
    np.testing.assert_array_equal(idx.cpu().numpy(), oidx)
    sample = [0, 5, 1000, 2047]
    xs = x[sample].contiguous()
    oy, _, _, _ = oracle_layer(dl, xs, idx_hint=oidx[sample])
    err = rel_l2(y[sample].float().cpu().numpy(), oy)
    print(f"  sampled rel-L2 {err:.3e}")
    assert err <= tol(wl)
