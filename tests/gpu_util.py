"""Helpers shared by the GPU parity tests: build device inputs from ``synth``, run the HIP
path through the C ABI binding, and gather what the oracle needs back on the host."""
import dataclasses

import numpy as np
import torch

import oracle
import synth


def rel_l2(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def tol(wl) -> float:
    """Parity tolerance on rel-L2 of the layer output: 1e-4 for fp32, 8e-3 for bf16 output.  In the
    opt-in MXFP8 activation mode (compared with the oracle's mirrored mode) fp32 output gets 1e-3:
    both sides quantise x identically, but h is quantised from fp32 sums on the GPU and fp64 sums in
    the oracle, and an h value that lands within their difference of an E4M3 rounding midpoint
    takes the neighbouring code (one step, at most 1/16 of that value)."""
    if wl.act_quant:
        return 1e-3 if wl.act_dtype == synth.F32 else 8e-3
    return 1e-4 if wl.act_dtype == synth.F32 else 8e-3


def shape_of(m, wl):
    return m.make_shape(wl.d_model, wl.d_ff, wl.n_experts, wl.top_k, wl.wformat, wl.act_dtype,
                        wl.routed_scaling, wl.renorm_skip, wl.n_shared, wl.act_quant)


class DeviceLayer:
    """One layer's inputs in HBM plus its expert table."""

    def __init__(self, m, wl, layer=0, seed=0, host_gen=None):
        if host_gen is None:
            host_gen = wl.d_model * wl.d_ff * wl.n_experts <= 64 * 1024 * 1024
        gen_dev = "cpu" if host_gen else "cuda"
        lay = synth.make_layer(wl, layer, seed, gen_dev)
        self.wl = wl
        self.shape = shape_of(m, wl)
        self.router = lay["router"].to("cuda").contiguous()
        self.bias = None if lay["bias"] is None else lay["bias"].to("cuda").contiguous()
        self.blob = lay["blob"].to("cuda").contiguous()
        self.stride = self.blob.shape[1]
        self.table = torch.empty((wl.n_experts + wl.n_shared) * m.EXPERT_BYTES, dtype=torch.uint8, device="cuda")
        m.moe_fill_table(self.shape, self.blob, self.stride, self.table)

    def host_blobs(self, experts):
        """Host copies of the given experts' blobs (None for the others), for the oracle."""
        out = [None] * self.wl.n_experts
        for e in sorted(set(int(v) for v in experts)):
            out[e] = self.blob[e].cpu().numpy()
        return out

    def shared_blob(self):
        """Host copy of the shared expert's blob, or None."""
        return self.blob[self.wl.n_experts].cpu().numpy() if self.wl.n_shared else None


def run_layer(m, dl, x, residual=None):
    wl = dl.wl
    T = x.shape[0]
    y = torch.empty_like(x)
    idx = torch.empty(T, wl.top_k, dtype=torch.int32, device="cuda")
    w = torch.empty(T, wl.top_k, dtype=torch.float32, device="cuda")
    ws = m.workspace(dl.shape, T)
    m.moe_layer(dl.shape, x, T, dl.router, dl.bias, dl.table, None, residual, y, idx, w, ws)
    torch.cuda.synchronize()
    return y, idx, w


def oracle_layer(dl, x, idx_hint=None, residual=None, scaling=None):
    wl = dl.wl
    x64 = oracle.to_f64(x)
    if idx_hint is None:
        _, idx_hint, _ = oracle.route(x64, dl.router.cpu().numpy(),
                                      None if dl.bias is None else dl.bias.cpu().numpy(), wl.top_k)
    hint = np.asarray(idx_hint).reshape(-1)
    blobs = dl.host_blobs(hint[hint >= 0])
    res = None if residual is None else oracle.to_f64(residual)
    return oracle.layer(x64, dl.router.cpu().numpy(), None if dl.bias is None else dl.bias.cpu().numpy(),
                        blobs, wl.d_model, wl.d_ff, wl.top_k, wl.wformat,
                        wl.routed_scaling if scaling is None else scaling, res, wl.renorm_skip,
                        dl.shared_blob(), wl.act_quant)


def small(name="tiny", **kw):
    return dataclasses.replace(synth.WORKLOADS[name], **kw)


def covering_sample(idx, E, tile_picks, n_min=64, seed=0):
    """Tokens whose picks, between them, fill every column slot of a tile of `tile_picks` picks
    that some tile fills,
    land in every eighth of the tile list (the many-pick GEMM hands each of the 8 XCDs one
    contiguous eighth), and include a pick of every ragged last tile, padded with further tokens
    to at least n_min.  idx: [T, k] routing.  Pure bookkeeping of the tile plan (expert ranges in
    sorted order, tiles of tile_picks consecutive positions), no arithmetic of the method."""
    idx = np.asarray(idx)
    T, k = idx.shape
    counts = np.bincount(idx.reshape(-1), minlength=E)
    first = np.concatenate([[0], np.cumsum(counts)])[:-1]
    tiles_per = (counts + tile_picks - 1) // tile_picks
    tile0 = np.concatenate([[0], np.cumsum(tiles_per)])[:-1]
    ntiles = int(tiles_per.sum())
    tpx = (ntiles + 7) // 8
    # sorted position of each pick: stable by (expert, pick id)
    order = np.argsort(idx.reshape(-1), kind="stable")
    pos = np.empty(T * k, dtype=np.int64)
    pos[order] = np.arange(T * k)
    e = idx.reshape(-1)
    rel = pos - first[e]
    slot = rel % tile_picks
    tile = tile0[e] + rel // tile_picks
    xcd = tile // tpx
    ragged = (rel // tile_picks == tiles_per[e] - 1) & (counts[e] % tile_picks != 0)
    # (the slots some tile fills: with few picks per expert no tile reaches the last slots)
    filled = int(min(tile_picks, counts.max())) if counts.size else 0
    need = {("slot", s) for s in range(filled)} | {("xcd", x) for x in range(min(8, ntiles))}
    rng = np.random.default_rng(seed)
    chosen = []
    for t in rng.permutation(T):
        feats = set()
        for p in range(t * k, t * k + k):
            feats |= {("slot", int(slot[p])), ("xcd", int(xcd[p]))}
        if feats & need:
            chosen.append(int(t))
            need -= feats
        if not need:
            break
    assert not need, f"no tokens cover {sorted(need)[:4]}"
    for t in [int(p // k) for p in np.flatnonzero(ragged)[:8]]:
        if t not in chosen:
            chosen.append(t)
    for t in rng.permutation(T):
        if len(chosen) >= n_min:
            break
        if int(t) not in chosen:
            chosen.append(int(t))
    return sorted(chosen)
