"""The C ABI library without a GPU: it loads, exports every function include/moe.h declares,
and rejects bad arguments on the host before anything is launched (stream 0, fake device
pointers that are never dereferenced)."""
import ctypes
import subprocess

import pytest

import oracle
import synth

m = pytest.importorskip("routed_expert_ffn_router_amd")

FAKE = 1 << 20          # a 256-aligned fake device address; never dereferenced on these paths


def test_exports_every_declared_function():
    declared = m.header_functions()
    assert len(declared) >= 11
    out = subprocess.run(["nm", "-D", "--defined-only", m.LIB_PATH], capture_output=True, text=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for name in declared:
        assert name in exported, name
        assert hasattr(m.library(), name)


def test_version_and_status_strings():
    assert m.abi_version() == 2
    for s in range(5):
        assert m.status_string(s)
    assert m.status_string(99) == "unknown status"


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_blob_stride_matches_oracle(name):
    wl = synth.WORKLOADS[name]
    sh = m.make_shape(wl.d_model, wl.d_ff, wl.n_experts, wl.top_k, wl.wformat, wl.act_dtype)
    assert m.moe_blob_stride(sh) == oracle.blob_stride(wl.d_model, wl.d_ff, wl.wformat)
    assert m.moe_blob_stride(sh) == synth.blob_offsets(wl.d_model, wl.d_ff, wl.wformat)["stride"]
    assert m.moe_workspace_bytes(sh, wl.tokens) > 0


def _route(shape, T=1, x=FAKE, wr=FAKE, idx=FAKE, w=FAKE, ws=FAKE, ws_bytes=1 << 40):
    return m.library().moe_route(ctypes.byref(shape), x, T, wr, None, idx, w, ws, ws_bytes, 0)


def test_validation_codes():
    good = m.make_shape(256, 128, 16, 2, 0, 0)
    assert _route(m.make_shape(256, 128, 16, 17)) == m.MOE_ERR_INVALID      # k > E
    assert _route(m.make_shape(256, 128, 16, 0)) == m.MOE_ERR_INVALID       # k = 0
    assert _route(m.make_shape(256, 128, 2000, 8)) == m.MOE_ERR_UNSUPPORTED  # E > 1024
    assert _route(m.make_shape(200, 128, 16, 2)) == m.MOE_ERR_UNSUPPORTED   # d % 128
    assert _route(m.make_shape(256, 96, 16, 2)) == m.MOE_ERR_UNSUPPORTED    # f % 128
    assert _route(m.make_shape(256, 128, 16, 2, 7, 0)) == m.MOE_ERR_INVALID  # bad format enum
    assert _route(m.make_shape(256, 128, 16, 2, 0, 5)) == m.MOE_ERR_INVALID  # bad dtype enum
    assert _route(m.make_shape(256, 128, 16, 2, 0, 0, float("nan"))) == m.MOE_ERR_INVALID
    assert _route(good, T=-1) == m.MOE_ERR_INVALID
    assert _route(good, T=100000) == m.MOE_ERR_UNSUPPORTED
    assert _route(good, T=0, x=None) == m.MOE_OK                             # no-op
    assert _route(good, x=None) == m.MOE_ERR_INVALID
    assert _route(good, x=FAKE + 4) == m.MOE_ERR_INVALID                     # misaligned
    assert _route(good, ws_bytes=16) == m.MOE_ERR_WORKSPACE
    assert m.library().moe_route(None, FAKE, 1, FAKE, None, FAKE, FAKE, FAKE, 1 << 40, 0) == m.MOE_ERR_INVALID
    # the optional parts of the layer: renorm_skip in [0, 1), n_shared 0 or 1, act_quant an enum
    # (MXFP8 activations only with MXFP4 weights)
    assert _route(m.make_shape(256, 128, 16, 2, renorm_skip=-0.1)) == m.MOE_ERR_INVALID
    assert _route(m.make_shape(256, 128, 16, 2, renorm_skip=1.0)) == m.MOE_ERR_INVALID
    assert _route(m.make_shape(256, 128, 16, 2, renorm_skip=float("nan"))) == m.MOE_ERR_INVALID
    assert _route(m.make_shape(256, 128, 16, 2, n_shared=2)) == m.MOE_ERR_INVALID
    assert _route(m.make_shape(256, 128, 16, 2, n_shared=-1)) == m.MOE_ERR_INVALID
    assert _route(m.make_shape(256, 128, 16, 2, act_quant=2)) == m.MOE_ERR_INVALID
    assert _route(m.make_shape(256, 128, 16, 2, 1, 0, act_quant=m.MOE_AQ_MXFP8)) == m.MOE_ERR_UNSUPPORTED


def test_validation_other_entry_points():
    L = m.library()
    sh = m.make_shape(256, 128, 16, 2, 0, 0)
    nv = m.make_shape(256, 128, 16, 2, 1, 0)
    b = ctypes.byref
    assert L.moe_permute(b(sh), None, 4, FAKE, FAKE, FAKE, None, 0, 0) == m.MOE_ERR_INVALID
    # a workspace, when given, must hold the layout for (shape, T)
    assert L.moe_permute(b(sh), FAKE, 4, FAKE, FAKE, FAKE, FAKE, 16, 0) == m.MOE_ERR_WORKSPACE
    assert L.moe_expert_ffn(b(sh), FAKE, FAKE, 4, FAKE, FAKE, FAKE, FAKE, 16, 0) == m.MOE_ERR_WORKSPACE
    assert L.moe_expert_ffn(b(nv), FAKE, FAKE, 4, FAKE, FAKE, FAKE, FAKE, 16, 0) == m.MOE_ERR_WORKSPACE
    # staging belongs to the NVFP4 gather path; it must be 16-byte aligned
    assert L.moe_layer(b(sh), FAKE, 4, FAKE, None, FAKE, FAKE, None, 2 * FAKE, None, None, FAKE, 1 << 40, 0) \
        == m.MOE_ERR_INVALID
    assert L.moe_layer(b(nv), FAKE, 4, FAKE, None, FAKE, FAKE + 8, None, 2 * FAKE, None, None, FAKE, 1 << 40, 0) \
        == m.MOE_ERR_INVALID
    assert L.moe_combine(b(sh), FAKE, FAKE, None, 4, None, FAKE, 0) == m.MOE_ERR_INVALID
    assert L.moe_layer(b(sh), FAKE, 4, FAKE, None, FAKE, None, None, 2 * FAKE, None, None, FAKE, 16, 0) \
        == m.MOE_ERR_WORKSPACE
    assert L.moe_layer(b(sh), FAKE, 4, FAKE, None, FAKE, None, None, FAKE, None, None, FAKE, 1 << 40, 0) \
        == m.MOE_ERR_INVALID                                                # y aliases x
    assert L.moe_gather_experts(b(sh), FAKE, FAKE, -1, FAKE, FAKE, 0) == m.MOE_ERR_INVALID
    assert L.moe_gather_experts(b(sh), FAKE, FAKE, 0, None, None, 0) == m.MOE_OK
    assert L.moe_fill_table(b(sh), FAKE, 100, FAKE, 0) == m.MOE_ERR_INVALID   # stride too small
    assert m.moe_workspace_bytes(m.make_shape(256, 128, 16, 17), 4) == 0
    # workspace preparation: a null or misaligned workspace, or one too small for (shape, T)
    assert L.moe_workspace_init(b(sh), 4, None, 1 << 40, 0, 0) == m.MOE_ERR_INVALID
    assert L.moe_workspace_init(b(sh), 4, FAKE + 16, 1 << 40, 0, 0) == m.MOE_ERR_INVALID
    assert L.moe_workspace_init(b(sh), 4, FAKE, 16, 0, 0) == m.MOE_ERR_WORKSPACE
    assert L.moe_workspace_init(b(sh), -1, FAKE, 1 << 40, 0, 0) == m.MOE_ERR_INVALID
    # moe_permute's workspace, when given, must be 256-byte aligned like every other
    assert L.moe_permute(b(sh), FAKE, 4, FAKE, FAKE, FAKE, FAKE + 16, 1 << 40, 0) == m.MOE_ERR_INVALID
    # the observed layer validates exactly as moe_layer does
    obs = m.make_observer()
    assert L.moe_layer_observed(b(sh), FAKE, 4, FAKE, None, FAKE, None, None, FAKE, None, None, FAKE, 1 << 40, 0,
                                ctypes.byref(obs)) == m.MOE_ERR_INVALID      # y aliases x
    assert L.moe_layer_observed(b(sh), None, 0, None, None, None, None, None, None, None, None, None, 0, 0,
                                None) == m.MOE_OK                           # T = 0 is a no-op


def test_workspace_header_is_first_and_fixed():
    """The status word sits at offset 0 and the hand-over slots right after the header, at the same
    place for every T, so one workspace serves calls of every token count up to its own."""
    sh = m.make_shape(4096, 2048, 288, 8)
    sizes = [m.moe_workspace_bytes(sh, T) for T in (1, 16, 17, 64, 4096)]
    assert sizes == sorted(sizes) and sizes[0] > 256 + 8 * 16 * 288
    assert m.MOE_WS_STATUS_OFFSET == 0
