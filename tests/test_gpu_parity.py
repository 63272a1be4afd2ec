"""GPU parity of the HIP path (through the C ABI) against the fp64 CPU oracle.

Router indices and permutations must be bit-exact; layer outputs must be within rel-L2 1e-4
(fp32 activations) or 8e-3 (bf16 activations) of the oracle's unrounded fp64 output.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import DeviceLayer, covering_sample, oracle_layer, rel_l2, run_layer, small, tol

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import routed_expert_ffn_router_amd as m      # must load: no fallback path exists


def _x(wl, T, seed=0, tag="x"):
    return synth.make_x(wl, seed, "cpu", tokens=T, tag=tag).to("cuda").contiguous()


# ---------------------------------------------------------------------------------------------
# router and permute
# ---------------------------------------------------------------------------------------------

@pytest.mark.parametrize("name,T", [("tiny", 4), ("tiny", 77), ("decode", 1), ("decode", 64), ("prefill", 300)])
def test_route_bit_exact(name, T):
    wl = small(name)
    print(f"route parity {name} T={T}", flush=True)
    router = synth.make_router(wl, 0, 0, "cpu")
    bias = synth.make_bias(synth.WORKLOADS["batched"], 0, 0, "cpu") if name == "decode" and T == 64 else None
    x = _x(wl, T)
    shape = m.make_shape(wl.d_model, wl.d_ff, wl.n_experts, wl.top_k, wl.wformat, wl.act_dtype)
    idx = torch.empty(T, wl.top_k, dtype=torch.int32, device="cuda")
    w = torch.empty(T, wl.top_k, dtype=torch.float32, device="cuda")
    ws = m.workspace(shape, T)
    m.moe_route(shape, x, T, router.cuda(), None if bias is None else bias.cuda(), idx, w, ws)
    torch.cuda.synchronize()
    _, oidx, ow = oracle.route(oracle.to_f64(x), router.numpy(), None if bias is None else bias.numpy(),
                               wl.top_k)
    np.testing.assert_array_equal(idx.cpu().numpy(), oidx)
    np.testing.assert_allclose(w.cpu().numpy(), ow, rtol=2e-7, atol=1e-8)
    np.testing.assert_allclose(w.sum(dim=1).cpu().numpy(), 1.0, atol=2.0**-21)


def test_route_ties_go_to_lower_index():
    wl = small("tiny", top_k=3)
    T = 8
    router = synth.make_router(wl, 0, 0, "cpu")
    router[9] = router[2]          # experts 2 and 9 tie exactly on every token
    router[13] = router[2]
    x = _x(wl, T)
    shape = m.make_shape(wl.d_model, wl.d_ff, wl.n_experts, wl.top_k, wl.wformat, wl.act_dtype)
    idx = torch.empty(T, 3, dtype=torch.int32, device="cuda")
    w = torch.empty(T, 3, dtype=torch.float32, device="cuda")
    m.moe_route(shape, x, T, router.cuda(), None, idx, w, m.workspace(shape, T))
    torch.cuda.synchronize()
    _, oidx, _ = oracle.route(oracle.to_f64(x), router.numpy(), None, 3)
    np.testing.assert_array_equal(idx.cpu().numpy(), oidx)


@pytest.mark.parametrize("T", [1, 5, 40])
def test_route_nan_rows_and_zero_tokens(T):
    """NaN logits rank after every number (experts 3 and 9 have NaN router rows); a token of
    zeros gives every expert logit 0, so the lowest indices win, with equal weights."""
    wl = small("tiny", top_k=4)
    router = synth.make_router(wl, 0, 0, "cpu")
    router[3] = float("nan")
    router[9] = float("nan")
    x = _x(wl, T)
    x[0] = 0.0
    shape = m.make_shape(wl.d_model, wl.d_ff, wl.n_experts, wl.top_k, wl.wformat, wl.act_dtype)
    idx = torch.empty(T, 4, dtype=torch.int32, device="cuda")
    w = torch.empty(T, 4, dtype=torch.float32, device="cuda")
    m.moe_route(shape, x, T, router.cuda(), None, idx, w, m.workspace(shape, T))
    torch.cuda.synchronize()
    _, oidx, ow = oracle.route(oracle.to_f64(x), router.numpy(), None, 4)
    np.testing.assert_array_equal(idx.cpu().numpy(), oidx)
    np.testing.assert_array_equal(oidx[0], [0, 1, 2, 4])       # 3 is NaN: after every number
    assert not np.isin(oidx[1:], [3, 9]).any()
    np.testing.assert_allclose(w.cpu().numpy(), ow, rtol=2e-7, atol=1e-8)


# with a workspace, 4+ blocks of 1024 picks are sorted by one workgroup per block; (3000, 2, 4) puts
# runs of one expert across every block boundary, (1000, 8, 1024) ends in a ragged block
@pytest.mark.parametrize("with_ws", [False, True])
@pytest.mark.parametrize("T,k,E", [(1, 8, 288), (5, 2, 16), (64, 8, 288), (4096, 8, 288), (1000, 8, 1024),
                                   (3000, 2, 4)])
def test_permute_bit_exact(T, k, E, with_ws):
    g = torch.Generator().manual_seed(T + E)
    idx = torch.stack([torch.randperm(E, generator=g)[:k] for _ in range(T)]).to(torch.int32)
    shape = m.make_shape(256, 128, E, k)
    off = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    sp = torch.empty(T * k, dtype=torch.int32, device="cuda")
    pp = torch.empty(T * k, dtype=torch.int32, device="cuda")
    if with_ws:
        ws = m.workspace(shape, T)
        torch.cuda.synchronize()
        m.moe_permute(shape, idx.cuda(), T, off, sp, pp, ws, ws.numel() * ws.element_size())
    else:
        m.moe_permute(shape, idx.cuda(), T, off, sp, pp)
    torch.cuda.synchronize()
    ooff, osp, opp = oracle.permute(idx.numpy(), E)
    np.testing.assert_array_equal(off.cpu().numpy(), ooff)
    np.testing.assert_array_equal(sp.cpu().numpy(), osp)
    np.testing.assert_array_equal(pp.cpu().numpy(), opp)


# ---------------------------------------------------------------------------------------------
# whole layer
# ---------------------------------------------------------------------------------------------

SMALL_CASES = [
    ("tiny", dict(), 4),                                                     # the fp32 config
    ("tiny", dict(), 1),
    ("tiny", dict(), 53),                                                    # ragged, many tiles
    ("tiny", dict(act_dtype=synth.BF16), 9),
    ("tiny", dict(d_model=512, d_ff=256, n_experts=32, top_k=4, act_dtype=synth.BF16), 37),
    ("tiny", dict(d_model=1024, d_ff=512, n_experts=64, top_k=8, act_dtype=synth.BF16), 300),
    ("tiny", dict(d_model=1024, d_ff=2048, n_experts=8, top_k=2), 11),
    # d_model past the staged-column decode kernels (4096) and d_ff past the LDS down (2048):
    # the tile GEMMs with long K at few picks
    ("tiny", dict(d_model=5120, d_ff=384, n_experts=8, top_k=2, act_dtype=synth.BF16), 5),
    ("tiny", dict(d_model=1024, d_ff=4224, n_experts=8, top_k=2), 6),
    # many picks per expert (LDS-tiled GEMM): fp32 activations in four terms
    ("tiny", dict(n_experts=4, top_k=2), 200),
    # 3 K steps of gate/up, 5 of down; the second block of 256 down rows runs past d_model
    ("tiny", dict(d_model=384, d_ff=640, n_experts=8, top_k=2, act_dtype=synth.BF16), 150),
    # 7 K steps: one full group of four plus a tail of three
    ("tiny", dict(d_model=896, d_ff=256, n_experts=12, top_k=3, act_dtype=synth.BF16), 100),
    # few tokens, router rows not a whole number of 256-element chunks per half (fused router)
    ("tiny", dict(d_model=384, d_ff=256, n_experts=16, top_k=2, act_dtype=synth.BF16), 4),
    ("tiny", dict(d_model=640, d_ff=256, n_experts=9, top_k=3), 2),
    # fused router: k > 8 takes the k-round top-k; E > 320 holds 16 logits per lane
    ("tiny", dict(n_experts=64, top_k=12), 3),
    ("tiny", dict(n_experts=400, top_k=8, act_dtype=synth.BF16), 5),
    ("tiny", dict(n_experts=400, top_k=8, act_dtype=synth.BF16), 1),
    ("tiny", dict(n_experts=400, top_k=8, act_dtype=synth.BF16), 16),
    # fused router, 16 tokens on four experts: an expert's tokens fill more than one tile
    ("tiny", dict(n_experts=4, top_k=2), 16),
    # 8-32 picks per expert on average: the 64-column tile (32 picks with two terms, some experts
    # over two tiles); with fp32 activations (four terms) 16 picks per tile
    ("tiny", dict(d_model=512, d_ff=256, n_experts=16, top_k=4, act_dtype=synth.BF16), 90),
    ("tiny", dict(n_experts=8, top_k=2), 60),
    # fp32 activations on the few-pick tiles of the general path (four terms: 4 picks per tile)
    ("tiny", dict(n_experts=64, top_k=4), 24),
]


@pytest.mark.parametrize("name,kw,T", SMALL_CASES)
def test_layer_small(name, kw, T):
    wl = small(name, **kw)
    print(f"layer parity {kw} T={T}", flush=True)
    dl = DeviceLayer(m, wl)
    x = _x(wl, T)
    y, idx, w = run_layer(m, dl, x)
    oy, oidx, ow, _ = oracle_layer(dl, x)
    np.testing.assert_array_equal(idx.cpu().numpy(), oidx)
    err = rel_l2(y.float().cpu().numpy(), oy)
    print(f"  rel-L2 {err:.3e} (tol {tol(wl):.0e})")
    assert err <= tol(wl)


@pytest.mark.parametrize("T", [1, 3, 16])
def test_fused_route_ties_nan_and_zero_token(T):
    """The few-token router of moe_layer: experts 2, 9 and 13 tie exactly on every token, experts
    3 and 7 have NaN logits (after every number), and token 0 is all zeros (every finite logit 0,
    so the lowest indices win with equal weights)."""
    wl = small("tiny", top_k=4)
    print(f"fused route ties/NaN T={T}", flush=True)
    dl = DeviceLayer(m, wl)
    dl.router[9] = dl.router[2]
    dl.router[13] = dl.router[2]
    dl.router[3] = float("nan")
    dl.router[7] = float("nan")
    x = _x(wl, T)
    x[0] = 0.0
    y, idx, w = run_layer(m, dl, x)
    oy, oidx, ow, _ = oracle_layer(dl, x)
    np.testing.assert_array_equal(idx.cpu().numpy(), oidx)
    np.testing.assert_array_equal(oidx[0], [0, 1, 2, 4])
    np.testing.assert_allclose(w.cpu().numpy(), ow, rtol=2e-7, atol=1e-8)
    assert rel_l2(y.float().cpu().numpy(), oy) <= tol(wl)


def test_fused_route_workspace_shared_across_T():
    """One workspace, sized for 64 tokens, used by the general path (T=64) and then by the
    few-token path (T=1, 16, 1): each result equals the one from a fresh workspace."""
    wl = small("tiny", d_model=512, d_ff=256, n_experts=32, top_k=4, act_dtype=synth.BF16)
    dl = DeviceLayer(m, wl)
    ws = m.workspace(dl.shape, 64)
    for T in (64, 1, 16, 1):
        print(f"shared workspace T={T}", flush=True)
        x = _x(wl, T, tag=f"ws{T}")
        y = torch.empty_like(x)
        idx = torch.empty(T, wl.top_k, dtype=torch.int32, device="cuda")
        w = torch.empty(T, wl.top_k, dtype=torch.float32, device="cuda")
        m.moe_layer(dl.shape, x, T, dl.router, dl.bias, dl.table, None, None, y, idx, w, ws)
        torch.cuda.synchronize()
        y0, i0, w0 = run_layer(m, dl, x)
        assert torch.equal(idx, i0) and torch.equal(w, w0)
        assert torch.equal(y.view(torch.int16), y0.view(torch.int16))


def test_layer_residual_and_scaling():
    wl = small("tiny", routed_scaling=2.5)
    dl = DeviceLayer(m, wl)
    x = _x(wl, 6)
    res = _x(wl, 6, tag="res")
    y, idx, _ = run_layer(m, dl, x, residual=res)
    oy, oidx, _, _ = oracle_layer(dl, x, residual=res)
    np.testing.assert_array_equal(idx.cpu().numpy(), oidx)
    assert rel_l2(y.float().cpu().numpy(), oy) <= tol(wl)


def test_staged_calls_match_layer():
    wl = small("tiny", d_model=512, d_ff=256, n_experts=32, top_k=4, act_dtype=synth.BF16)
    dl = DeviceLayer(m, wl)
    T = 21
    x = _x(wl, T)
    y, idx, w = run_layer(m, dl, x)
    sh = dl.shape
    ws = m.workspace(sh, T)
    idx2 = torch.empty_like(idx)
    w2 = torch.empty_like(w)
    m.moe_route(sh, x, T, dl.router, dl.bias, idx2, w2, ws)
    off = torch.empty(wl.n_experts + 1, dtype=torch.int32, device="cuda")
    sp = torch.empty(T * wl.top_k, dtype=torch.int32, device="cuda")
    pp = torch.empty_like(sp)
    m.moe_permute(sh, idx2, T, off, sp, pp)
    o = torch.empty(T * wl.top_k, wl.d_model, dtype=torch.float32, device="cuda")
    m.moe_expert_ffn(sh, dl.table, x, T, off, sp, o, ws)
    y2 = torch.empty_like(y)
    m.moe_combine(sh, o, w2, pp, T, None, y2)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2) and torch.equal(w, w2)
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))
    # the staged o rows are the oracle's per-pick expert outputs
    ooff, osp, _ = oracle.permute(idx.cpu().numpy(), wl.n_experts)
    oo = oracle.expert_ffn(dl.host_blobs(idx.cpu().numpy().reshape(-1)), wl.d_model, wl.d_ff, wl.wformat,
                           oracle.to_f64(x), wl.top_k, ooff, osp)
    assert rel_l2(o.cpu().numpy(), oo) <= tol(wl)


def test_zero_tokens_is_noop():
    wl = small("tiny")
    dl = DeviceLayer(m, wl)
    ws = torch.empty(256, dtype=torch.uint8, device="cuda")
    m.moe_layer(dl.shape, None, 0, dl.router, None, dl.table, None, None, None, None, None, ws)
    torch.cuda.synchronize()


def test_zero_input_gives_zero_output():
    wl = small("tiny", act_dtype=synth.BF16)
    dl = DeviceLayer(m, wl)
    x = torch.zeros(5, wl.d_model, dtype=torch.bfloat16, device="cuda")
    y, _, _ = run_layer(m, dl, x)
    assert torch.count_nonzero(y.float()) == 0


def test_run_to_run_bit_identical():
    wl = small("tiny", d_model=512, d_ff=256, n_experts=32, top_k=4, act_dtype=synth.BF16)
    dl = DeviceLayer(m, wl)
    x = _x(wl, 40)
    y1, i1, w1 = run_layer(m, dl, x)
    y2, i2, w2 = run_layer(m, dl, x)
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16)) and torch.equal(i1, i2)


def test_down_scale_plus_one_doubles_output():
    """Adding 1 to every E8M0 byte of W_down doubles y exactly (fp32 output)."""
    wl = small("tiny")
    dl = DeviceLayer(m, wl)
    x = _x(wl, 7)
    y1, _, _ = run_layer(m, dl, x)
    off = synth.blob_offsets(wl.d_model, wl.d_ff, wl.wformat)
    so, sn = off["down_s"]
    dl.blob[:, so:so + sn] += 1
    y2, _, _ = run_layer(m, dl, x)
    assert torch.equal(y2, 2 * y1)


# ---------------------------------------------------------------------------------------------
# full-size GLM-5.3-Flash layer shapes (sampled against the oracle)
# ---------------------------------------------------------------------------------------------

@pytest.fixture(scope="module")
def glm_layer():
    wl = synth.WORKLOADS["decode"]
    print("generating a 288-expert MXFP4 layer in HBM", flush=True)
    return DeviceLayer(m, wl, layer=0, host_gen=False)


# T=1 and 2: few-token kernels with the h terms staged in LDS; 5 and 16: the same gate/up kernel
# with the down kernel reading h from memory (and tiles of several picks of one expert); 20, 48
# and 64: the general path (matrix-core router, permute, grouped GEMMs, combine)
@pytest.mark.parametrize("T", [1, 2, 5, 16, 20, 48, 64])
def test_glm_decode_layer(glm_layer, T):
    dl = glm_layer
    wl = dl.wl
    print(f"glm layer T={T}", flush=True)
    x = _x(wl, T, tag=f"x{T}")
    y, idx, w = run_layer(m, dl, x)
    oy, oidx, ow, _ = oracle_layer(dl, x, idx_hint=idx.cpu().numpy())
    np.testing.assert_array_equal(idx.cpu().numpy(), oidx)
    err = rel_l2(y.float().cpu().numpy(), oy)
    print(f"  rel-L2 {err:.3e}")
    assert err <= tol(wl)


def test_glm_decode_zero_token(glm_layer):
    """A zero token at full width: all 288 logits are 0, more candidates than the one-pass top-k
    takes, so the k-round top-k picks experts 0..7 with weights 1/8; token 1 is ordinary."""
    dl = glm_layer
    wl = dl.wl
    print("glm layer zero token", flush=True)
    x = _x(wl, 2, tag="zero")
    x[0] = 0.0
    y, idx, w = run_layer(m, dl, x)
    oy, oidx, ow, _ = oracle_layer(dl, x, idx_hint=idx.cpu().numpy())
    np.testing.assert_array_equal(idx.cpu().numpy(), oidx)
    np.testing.assert_array_equal(oidx[0], np.arange(8))
    np.testing.assert_allclose(w[0].cpu().numpy(), 0.125, rtol=0, atol=0)
    assert rel_l2(y.float().cpu().numpy(), oy) <= tol(wl)


@pytest.mark.parametrize("T", [512, 1024])
def test_glm_mid_chunk_sampled(glm_layer, T):
    """Chunks of 14 and 28 picks per expert on average: the 64-column (32-pick) tiles of the
    many-picks GEMM at full width.  Routing bit-exact on every token; the output on tokens whose
    picks fill every column slot of a 32-pick tile and every eighth of the tile list."""
    dl = glm_layer
    wl = dl.wl
    print(f"glm chunk T={T}", flush=True)
    x = _x(wl, T, tag=f"mid{T}")
    y, idx, w = run_layer(m, dl, x)
    _, oidx, ow = oracle.route(oracle.to_f64(x), dl.router.cpu().numpy(), None, wl.top_k)
    np.testing.assert_array_equal(idx.cpu().numpy(), oidx)
    sample = covering_sample(oidx, wl.n_experts, 32, n_min=48)
    print(f"  {len(sample)} sampled tokens", flush=True)
    xs = x[sample].contiguous()
    oy, _, _, _ = oracle_layer(dl, xs, idx_hint=oidx[sample])
    err = rel_l2(y[sample].float().cpu().numpy(), oy)
    print(f"  sampled rel-L2 {err:.3e}")
    assert err <= tol(wl)


def test_glm_prefill_chunk_sampled(glm_layer):
    """T=4096 chunk, the bench's prefill leg: routing bit-exact on every token; the output checked on
    at least 64 tokens chosen so that their picks fill every column slot of a 64-pick tile, fall in
    every eighth of the tile list (one per XCD) and include ragged last tiles."""
    dl = glm_layer
    wl = dl.wl
    T = 4096
    print("glm prefill T=4096", flush=True)
    x = _x(wl, T, tag="prefill")
    y, idx, w = run_layer(m, dl, x)
    _, oidx, ow = oracle.route(oracle.to_f64(x), dl.router.cpu().numpy(), None, wl.top_k)
    np.testing.assert_array_equal(idx.cpu().numpy(), oidx)
    counts = np.bincount(oidx.reshape(-1), minlength=wl.n_experts)
    assert counts.min() > 0        # nearly every expert active at this chunk size
    sample = covering_sample(oidx, wl.n_experts, 64, n_min=64)
    print(f"  {len(sample)} sampled tokens", flush=True)
    xs = x[sample].contiguous()
    oy, _, _, _ = oracle_layer(dl, xs, idx_hint=oidx[sample])
    err = rel_l2(y[sample].float().cpu().numpy(), oy)
    print(f"  sampled rel-L2 {err:.3e}")
    assert err <= tol(wl)
