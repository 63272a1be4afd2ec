"""Seeded synthetic inputs for the routed mixture-of-experts FFN layer.

This module only *makes inputs*: activations, router weights, logit biases and
expert weight blobs in the MXFP4 / NVFP4 byte formats.  It holds none of the
layer's arithmetic (no routing, no dequantisation, no FFN) and is imported by
both the HIP path's tests/bench and the CPU oracle's tests, so that both sides
consume exactly the same bytes.

Workloads (shapes, value distributions, routing structure) follow the pages:
GLM-5.3-Flash routed layers with 288 experts and 8 picks per token
("Project Maya", section "What is in the 96.5 GB"; Strata-GLM blog, "Why
GLM-5.3-Flash"), flat routing ("Day one: 1.75 tokens per second" of the
Strata-GLM blog), a per-layer skew where the hottest 35% of experts take 74% of
picks ("A hot expert cache ...", section "Offload more, cache the hot
experts"), and MXFP4 / NVFP4 expert weights (windlass README; "A hot expert
cache ...", "The wall: one PCIe transfer per token").

Everything runs through ``torch`` on the device given (``"cpu"`` for small
cases, ``"cuda"`` to build the 162 GB 42-layer stack directly in HBM); the same
seed gives the same bytes on the same device type.
"""
from __future__ import annotations

import dataclasses
import hashlib
import math
from typing import Optional

import torch

MXFP4 = 0
NVFP4 = 1
F32 = 0
BF16 = 1

# --------------------------------------------------------------------------------------------
# workload configurations
# --------------------------------------------------------------------------------------------


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    d_model: int
    d_ff: int
    n_experts: int
    top_k: int
    tokens: int
    n_layers: int
    wformat: int            # MXFP4 or NVFP4
    act_dtype: int          # F32 or BF16
    router_std: float       # std of router weights
    weight_std: float = 0.02
    skew_alpha: float = 0.0  # logit bias b_e = -alpha * ln(rank_e); 0 = flat routing
    routed_scaling: float = 1.0
    renorm_skip: float = 0.0
    n_shared: int = 0        # 1: one more expert blob (index n_experts), the shared expert
    act_quant: int = 0       # 1: the layer's opt-in MXFP8 activation mode

    @property
    def torch_act_dtype(self):
        return torch.float32 if self.act_dtype == F32 else torch.bfloat16


# Skew strength calibrated so that, with N(0,1) logits over 288 experts, the hottest 35%
# (101) of experts take ~74% of the picks (see ``skew_share`` and tests/test_synth.py).
SKEW_ALPHA_288 = 0.395

WORKLOADS = {
    "tiny": Workload("tiny", 256, 128, 16, 2, 4, 1, MXFP4, F32, 0.02),
    "decode": Workload("decode", 4096, 2048, 288, 8, 1, 42, MXFP4, BF16, 1.0 / 64.0),
    "batched": Workload("batched", 4096, 2048, 288, 8, 64, 42, MXFP4, BF16, 1.0 / 64.0,
                        skew_alpha=SKEW_ALPHA_288),
    "prefill": Workload("prefill", 4096, 2048, 288, 8, 4096, 1, MXFP4, BF16, 1.0 / 64.0),
    "nvfp4_decode": Workload("nvfp4_decode", 6144, 2048, 256, 8, 1, 1, NVFP4, BF16,
                             1.0 / math.sqrt(6144.0)),
    "nvfp4_prefill": Workload("nvfp4_prefill", 6144, 2048, 256, 8, 2048, 1, NVFP4, BF16,
                              1.0 / math.sqrt(6144.0)),
}

# --------------------------------------------------------------------------------------------
# canonical expert blob layout: [gate_q | up_q | down_q | gate_s | up_s | down_s] (+ tensor scales)
# --------------------------------------------------------------------------------------------


def block_size(wformat: int) -> int:
    return 32 if wformat == MXFP4 else 16


def blob_offsets(d: int, f: int, wformat: int) -> dict:
    """Byte offsets of the six sub-tensors (and NVFP4 tensor scales) in one expert blob."""
    B = block_size(wformat)
    gq = f * d // 2
    dq = d * f // 2
    gs = f * d // B
    ds = d * f // B
    off = {}
    o = 0
    for name, n in (("gate_q", gq), ("up_q", gq), ("down_q", dq),
                    ("gate_s", gs), ("up_s", gs), ("down_s", ds)):
        off[name] = (o, n)
        o += n
    if wformat == NVFP4:
        off["ts"] = (o, 12)
        o += 12
        o = (o + 255) // 256 * 256
    off["stride"] = o
    return off


# --------------------------------------------------------------------------------------------
# quantisers (input generation only: both sides read the bytes these produce)
# --------------------------------------------------------------------------------------------

_E2M1_MIDPOINTS = (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)


def _e2m1_round(v: torch.Tensor) -> torch.Tensor:
    """Round-to-nearest-even onto the E2M1 grid, saturating at 6; returns 4-bit codes (int16)."""
    a = v.abs()
    code = torch.zeros(v.shape, dtype=torch.int16, device=v.device)
    for i, m in enumerate(_E2M1_MIDPOINTS):
        if i % 2 == 1:
            code += (a >= m).to(torch.int16)
        else:
            code += (a > m).to(torch.int16)
    code |= (torch.signbit(v).to(torch.int16) << 3)
    return code


def _pack_nibbles(code: torch.Tensor) -> torch.Tensor:
    """Element 2i goes to the low nibble, element 2i+1 to the high nibble."""
    lo = code[..., 0::2]
    hi = code[..., 1::2]
    return (lo | (hi << 4)).to(torch.uint8)


def quantize_mx(w: torch.Tensor):
    """MXFP4: blocks of 32 along the last dim, one E8M0 scale each.

    Shared exponent = floor(log2(amax)) - 2 (2 = largest E2M1 exponent), clamped to the E8M0
    range; an all-zero block gets scale byte 0 and zero codes.
    Returns (codes [.., K/2] uint8, scales [.., K/32] uint8).
    """
    *lead, K = w.shape
    assert K % 32 == 0
    wb = w.float().reshape(*lead, K // 32, 32)
    amax = wb.abs().amax(dim=-1)
    _, ex = torch.frexp(amax)                       # amax = m * 2^ex, m in [0.5, 1)
    e = (ex.to(torch.int32) - 1) - 2
    e = torch.clamp(e, -127, 127)
    zero = amax == 0
    e = torch.where(zero, torch.full_like(e, -127), e)
    scale_byte = (e + 127).to(torch.uint8)
    v = torch.ldexp(wb, (-e).to(torch.float32)[..., None])
    code = _e2m1_round(v)
    code = torch.where(zero[..., None], torch.zeros_like(code), code)
    return _pack_nibbles(code.reshape(*lead, K)), scale_byte


def quantize_nv(w: torch.Tensor):
    """NVFP4: blocks of 16 along the last dim, E4M3 block scale, one fp32 tensor scale.

    ts = amax(tensor) / (6 * 448); block scale = E4M3(amax_block / (6 * ts)); codes =
    E2M1(x / (block_scale * ts)).  Returns (codes uint8, scales uint8 (E4M3 bytes), ts float).
    """
    *lead, K = w.shape
    assert K % 16 == 0
    w = w.float()
    amax_t = float(w.abs().max())
    ts = amax_t / (6.0 * 448.0) if amax_t > 0 else 1.0
    ts = float(torch.tensor(ts, dtype=torch.float32))
    wb = w.reshape(*lead, K // 16, 16)
    amax = wb.abs().amax(dim=-1)
    target = torch.clamp(amax / (6.0 * ts), max=448.0)
    bs8 = target.to(torch.float8_e4m3fn)
    bs = bs8.float()
    denom = bs * ts
    v = torch.where(denom[..., None] > 0, wb / denom[..., None], torch.zeros_like(wb))
    code = _e2m1_round(v)
    return _pack_nibbles(code.reshape(*lead, K)), bs8.view(torch.uint8), ts


# --------------------------------------------------------------------------------------------
# seeded generation
# --------------------------------------------------------------------------------------------


def sub_seed(*parts) -> int:
    """Deterministic 63-bit seed from (seed, config, layer, tensor, ...)."""
    h = hashlib.sha256("/".join(str(p) for p in parts).encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def _gen(device, *parts) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(sub_seed(*parts))
    return g


def make_x(wl: Workload, seed: int = 0, device="cpu", tokens: Optional[int] = None,
           tag: str = "x") -> torch.Tensor:
    """Activations x ~ N(0, 1) in the workload's activation dtype, [T, d]."""
    T = wl.tokens if tokens is None else tokens
    g = _gen(device, seed, wl.name, tag)
    x = torch.randn(T, wl.d_model, generator=g, device=device, dtype=torch.float32)
    return x.to(wl.torch_act_dtype)


def make_router(wl: Workload, layer: int = 0, seed: int = 0, device="cpu") -> torch.Tensor:
    """Router weights [E, d] fp32 ~ N(0, router_std^2)."""
    g = _gen(device, seed, wl.name, layer, "router")
    w = torch.randn(wl.n_experts, wl.d_model, generator=g, device=device, dtype=torch.float32)
    return w * wl.router_std


def make_bias(wl: Workload, layer: int = 0, seed: int = 0, device="cpu") -> Optional[torch.Tensor]:
    """Per-layer logit bias b_e = -alpha * ln(rank_e), rank a seeded permutation of 1..E.

    None for flat-routing workloads.
    """
    if wl.skew_alpha == 0.0:
        return None
    g = _gen("cpu", seed, wl.name, layer, "rank")
    rank = torch.randperm(wl.n_experts, generator=g).to(torch.float64) + 1.0
    b = (-wl.skew_alpha * torch.log(rank)).to(torch.float32)
    return b.to(device)


def skew_share(alpha: float, E: int = 288, k: int = 8, tokens: int = 20000, seed: int = 0,
               top_frac: float = 0.35) -> float:
    """Share of picks taken by the hottest ``top_frac`` of experts under bias -alpha*ln(rank)."""
    g = torch.Generator().manual_seed(seed)
    logits = torch.randn(tokens, E, generator=g, dtype=torch.float64)
    bias = -alpha * torch.log(torch.arange(1, E + 1, dtype=torch.float64))
    sel = torch.topk(logits + bias, k, dim=1).indices.reshape(-1)
    counts = torch.bincount(sel, minlength=E).to(torch.float64)
    top = int(round(top_frac * E))
    return float(torch.sort(counts, descending=True).values[:top].sum() / counts.sum())


def make_experts(wl: Workload, layer: int = 0, seed: int = 0, device="cpu",
                 experts: Optional[list] = None, group: int = 16) -> torch.Tensor:
    """Expert blobs [E + n_shared, stride] uint8 for one layer, quantised from N(0, weight_std^2)
    (blob n_experts is the shared expert when there is one).

    ``experts`` restricts generation to a subset (others stay zero); each expert's bytes
    depend only on (seed, workload, layer, expert), never on the subset or the group size.
    """
    d, f, E = wl.d_model, wl.d_ff, wl.n_experts + wl.n_shared
    off = blob_offsets(d, f, wl.wformat)
    blob = torch.zeros(E, off["stride"], dtype=torch.uint8, device=device)
    fill_experts(blob, wl, layer, seed, experts, group)
    return blob


def fill_experts(blob: torch.Tensor, wl: Workload, layer: int = 0, seed: int = 0,
                 experts: Optional[list] = None, group: int = 16) -> None:
    d, f, E = wl.d_model, wl.d_ff, wl.n_experts + wl.n_shared
    off = blob_offsets(d, f, wl.wformat)
    ids = list(range(E)) if experts is None else list(experts)
    device = blob.device
    shapes = {"gate": (f, d), "up": (f, d), "down": (d, f)}
    for i0 in range(0, len(ids), group):
        chunk = ids[i0:i0 + group]
        for part in ("gate", "up", "down"):
            rows, K = shapes[part]
            ws = []
            for e in chunk:
                g = _gen(device, seed, wl.name, layer, part, e)
                ws.append(torch.randn(rows, K, generator=g, device=device, dtype=torch.float32))
            w = torch.stack(ws) * wl.weight_std
            qo, qn = off[part + "_q"]
            so, sn = off[part + "_s"]
            idx = torch.tensor(chunk, device=device)
            if wl.wformat == MXFP4:
                q, s = quantize_mx(w)
                blob[idx, qo:qo + qn] = q.reshape(len(chunk), -1)
                blob[idx, so:so + sn] = s.reshape(len(chunk), -1)
            else:
                for j, e in enumerate(chunk):
                    q, s, ts = quantize_nv(w[j])
                    blob[e, qo:qo + qn] = q.reshape(-1)
                    blob[e, so:so + sn] = s.reshape(-1)
                    tso, _ = off["ts"]
                    k = ("gate", "up", "down").index(part)
                    tsb = torch.tensor([ts], dtype=torch.float32).view(torch.uint8).to(device)
                    blob[e, tso + 4 * k: tso + 4 * k + 4] = tsb
            del w, ws


def make_layer(wl: Workload, layer: int = 0, seed: int = 0, device="cpu", experts=None):
    """One layer's inputs: dict(router=[E,d] f32, bias=[E] f32 or None, blob=[E,stride] u8)."""
    return {
        "router": make_router(wl, layer, seed, device),
        "bias": make_bias(wl, layer, seed, device),
        "blob": make_experts(wl, layer, seed, device, experts),
    }
