#!/usr/bin/env python3
"""Benchmark of the routed mixture-of-experts FFN layer on one MI355X.

Headline (one JSON line): MoE-layer tokens/s of the 42-layer GLM-5.3-Flash-class decode stack
(d_model 4096, d_ff 2048, 288 MXFP4 experts, top-8, T=1, bf16 activations, flat routing), one
step = one token through all 42 layers, replayed as one HIP graph, inputs resident in HBM.
Each layer reads its own unit-scale input (the normalised hidden state a transformer block hands
its MoE layer) and writes y_l = x_l + MoE_l(x_l), the residual fused.  The same line carries the
dominant kernel's roofline (its duration from HIP events recorded by its own dispatch), the
oracle timed on the host cores, and secondary measurements: the 4096-token prefill chunk, the
64-token batched decode with skewed routing, and the NVFP4 configuration.  Every leg is checked
against the oracle in the same run (router indices bit-exact, rel-L2 of y within tolerance);
if any check fails the line carries no value and the exit status is 1.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                  [--only decode|prefill|batched|nvfp4]
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
FP4_PEAK_TFLOPS = 10100.0      # dense MX-FP4 MFMA, published
FP8_PEAK_TFLOPS = 5000.0       # dense FP8 MFMA, published
BF16_PEAK_TFLOPS = 2500.0
METRIC = "MoE-layer tokens/s (decode T=1, prefill T=4096) + % of HBM/MFMA peak"


# ---------------------------------------------------------------------------------------------
# HIP runtime plumbing (events, graphs) through ctypes
# ---------------------------------------------------------------------------------------------
class Hip:
    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so.7")
        P = ctypes.c_void_p
        L = self.lib
        L.hipEventCreate.argtypes = [ctypes.POINTER(P)]
        L.hipEventRecord.argtypes = [P, P]
        L.hipEventSynchronize.argtypes = [P]
        L.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), P, P]
        L.hipStreamBeginCapture.argtypes = [P, ctypes.c_int]
        L.hipStreamEndCapture.argtypes = [P, ctypes.POINTER(P)]
        L.hipGraphInstantiate.argtypes = [ctypes.POINTER(P), P, P, P, ctypes.c_size_t]
        L.hipGraphLaunch.argtypes = [P, P]
        L.hipStreamSynchronize.argtypes = [P]
        L.hipGraphExecDestroy.argtypes = [P]
        L.hipGraphDestroy.argtypes = [P]
        L.hipGetErrorString.restype = ctypes.c_char_p

    def _ok(self, rc, what):
        if rc != 0:
            raise RuntimeError(f"{what}: {self.lib.hipGetErrorString(rc).decode()}")

    def event(self):
        ev = ctypes.c_void_p()
        self._ok(self.lib.hipEventCreate(ctypes.byref(ev)), "hipEventCreate")
        return ev.value

    def record(self, ev, stream):
        self._ok(self.lib.hipEventRecord(ev, stream), "hipEventRecord")

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        self._ok(self.lib.hipEventSynchronize(b), "hipEventSynchronize")
        self._ok(self.lib.hipEventElapsedTime(ctypes.byref(ms), a, b), "hipEventElapsedTime")
        return ms.value

    def capture(self, stream, fn):
        """Capture fn() enqueued on `stream` into an instantiated graph."""
        self._ok(self.lib.hipStreamBeginCapture(stream, 2), "hipStreamBeginCapture")   # relaxed mode
        try:
            fn()
        finally:
            g = ctypes.c_void_p()
            self._ok(self.lib.hipStreamEndCapture(stream, ctypes.byref(g)), "hipStreamEndCapture")
        ex = ctypes.c_void_p()
        self._ok(self.lib.hipGraphInstantiate(ctypes.byref(ex), g, None, None, 0), "hipGraphInstantiate")
        return ex.value, g.value

    def launch(self, graph_exec, stream):
        self._ok(self.lib.hipGraphLaunch(graph_exec, stream), "hipGraphLaunch")

    def sync(self, stream):
        self._ok(self.lib.hipStreamSynchronize(stream), "hipStreamSynchronize")


def kernel_times(hip, m, stream, step, reps=3):
    """Per-kernel durations (us) of step(observer): every moe_layer call of the step carries an
    observer whose event hook hands the library a pair of HIP events for each kernel; the kernel's
    own dispatch records them at its start and end (hipExtLaunchKernel) on the stream it runs on,
    so a duration holds no launch gap (the same timestamps a profiler reads).  The step runs
    eagerly, reps times; returns {kernel: [durations]}."""
    pairs = []
    pool = []

    def events(kernel):
        a = pool.pop() if pool else hip.event()
        b = pool.pop() if pool else hip.event()
        pairs.append((kernel, a, b))
        return a, b

    obs = m.make_observer(events=events)
    per = {}
    for _ in range(reps):
        step(obs)
        hip.sync(stream)
        for k, a, b in pairs:
            per.setdefault(k, []).append(1000.0 * hip.elapsed_ms(a, b))
            pool += [a, b]
        pairs.clear()
    return per


# ---------------------------------------------------------------------------------------------
# workloads
# ---------------------------------------------------------------------------------------------
class Stack:
    """n_layers MoE layers of one workload, all experts resident in HBM."""

    def __init__(self, m, synth, torch, wl, n_layers, seed=0, log=print):
        self.wl = wl
        self.n = n_layers
        d, E = wl.d_model, wl.n_experts
        self.shape = m.make_shape(wl.d_model, wl.d_ff, E, wl.top_k, wl.wformat, wl.act_dtype, wl.routed_scaling)
        stride = m.moe_blob_stride(self.shape)
        t0 = time.time()
        self.blob = torch.empty(n_layers, E, stride, dtype=torch.uint8, device="cuda")
        self.router = torch.empty(n_layers, E, d, dtype=torch.float32, device="cuda")
        self.bias = [None] * n_layers
        self.table = torch.empty(n_layers, E * m.EXPERT_BYTES, dtype=torch.uint8, device="cuda")
        for l in range(n_layers):
            synth.fill_experts(self.blob[l], wl, l, seed)
            self.router[l] = synth.make_router(wl, l, seed, "cuda")
            b = synth.make_bias(wl, l, seed, "cuda")
            self.bias[l] = None if b is None else b.contiguous()
            m.moe_fill_table(self.shape, self.blob[l], stride, self.table[l])
            if (l + 1) % 7 == 0 or l + 1 == n_layers:
                torch.cuda.synchronize()
                log(f"# generated {l + 1}/{n_layers} layers ({self.blob[:l + 1].numel() / 1e9:.1f} GB) "
                    f"in {time.time() - t0:.1f} s")
        torch.cuda.synchronize()


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed counter summary (profiles/), or None when
    the kernel sources have changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get(kernel)
    if not rec:
        return None
    h = hashlib.sha256()
    for name in rec["sources"]:         # the kernel's file and the header its helpers live in
        h.update(open(os.path.join(ROOT, "routed_expert_ffn_router_amd", "csrc", name), "rb").read())
    if h.hexdigest() != rec["sources_sha256"]:
        return None
    return rec["bytes_per_launch"]


def algorithmic_layer_bytes(wl, experts_touched, T):
    """Bytes a layer must move at least: touched experts' blobs, the router, x and y."""
    B = 32 if wl.wformat == 0 else 16
    fd = wl.d_model * wl.d_ff
    stride = 3 * fd // 2 + 3 * fd // B
    act = 2 if wl.act_dtype == 1 else 4
    return experts_touched * stride + wl.n_experts * wl.d_model * 4 + 2 * T * wl.d_model * act


def gate_up_bytes(wl, experts):
    B = 32 if wl.wformat == 0 else 16
    fd = wl.d_model * wl.d_ff
    return experts * (2 * fd // 2 + 2 * fd // B)


def rel_l2(a, b):
    import numpy as np
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def oracle_check(oracle, np, torch, wl, blob_of, router, bias, x, y, idx, tokens=None, shared_blob=None):
    """Parity of one layer call against the oracle: router indices of every token bit-exact,
    rel-L2 of y (computed without a residual) on `tokens` (all when None).  blob_of(e) returns
    expert e's blob as a host array; the workload's renorm_skip, act_quant and routed_scaling (and
    the shared expert's blob, if any) are the layer's.  Returns (exact, rel_l2, oracle seconds)."""
    x64 = oracle.to_f64(x)
    wr = router.cpu().numpy()
    b = None if bias is None else bias.cpu().numpy()
    gidx = idx.cpu().numpy()
    t0 = time.perf_counter()
    _, oidx, _ = oracle.route(x64, wr, b, wl.top_k, wl.renorm_skip)
    exact = bool(np.array_equal(oidx, gidx))
    sel = np.arange(x.shape[0]) if tokens is None else np.asarray(tokens)
    blobs = [None] * wl.n_experts
    for e in np.unique(oidx[sel].reshape(-1)):
        if e >= 0:
            blobs[int(e)] = blob_of(int(e))
    xs = np.ascontiguousarray(x64[sel])
    oy, _, _, _ = oracle.layer(xs, wr, b, blobs, wl.d_model, wl.d_ff, wl.top_k, wl.wformat, wl.routed_scaling, None,
                               wl.renorm_skip, shared_blob, wl.act_quant)
    secs = time.perf_counter() - t0
    err = rel_l2(oracle.to_f64(y)[sel], oy)
    return exact, err, secs


def tolerance(wl):
    return 1e-4 if wl.act_dtype == 0 else 8e-3


def parity_entry(wl, exact, err, what):
    ok = bool(exact and err == err and err <= tolerance(wl))
    return {"checked": what, "router_indices_exact": exact, "rel_l2_y": err, "tolerance": tolerance(wl), "pass": ok}


def host_info():
    info = {"nproc": os.cpu_count(), "omp_num_threads": os.environ.get("OMP_NUM_THREADS"), "cpu_model": None}
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    info["cpu_model"] = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        info["affinity_cpus"] = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        pass
    return info


def expert_entry(m, synth, wl, ptr):
    """The 64-byte moe_expert record of a blob at device address ptr (host bytes)."""
    off = synth.blob_offsets(wl.d_model, wl.d_ff, wl.wformat)
    e = m.moe_expert()
    for f in ("gate_q", "up_q", "down_q", "gate_s", "up_s", "down_s"):
        setattr(e, f, ptr + off[f][0])
    e.gate_ts = e.up_ts = e.down_ts = 1.0
    return bytes(e)


def issued_mfma(flops, terms, ms, kern):
    """MFMA use against the instruction rate actually issued: the split activations make `terms`
    FP8 columns per value, so the scaled FP4 x FP8 MFMAs issue terms x the algorithmic FLOPs, at the
    FP8 rate; over the layer and over its two GEMM kernels alone."""
    issued = terms * flops
    gemm_us = kern.get("gemm_gate_up", 0.0) + kern.get("gemm_down", 0.0)
    return {"activation_terms": terms,
            "issued_fp8_mfma_frac": issued / (ms * 1e-3) / (FP8_PEAK_TFLOPS * 1e12),
            "gemm_issued_fp8_mfma_frac": issued / (gemm_us * 1e-6) / (FP8_PEAK_TFLOPS * 1e12) if gemm_us else None}


def time_graph(hip, S, step, reps, warm=3):
    """Capture step() on stream S as one graph; returns (ms per replay, graph)."""
    gexec, _ = hip.capture(S, step)
    for _ in range(warm):
        hip.launch(gexec, S)
    hip.sync(S)
    e0, e1 = hip.event(), hip.event()
    hip.record(e0, S)
    for _ in range(reps):
        hip.launch(gexec, S)
    hip.record(e1, S)
    return hip.elapsed_ms(e0, e1) / reps, gexec


def time_calls(hip, S, call, reps, warm=2):
    for _ in range(warm):
        call()
    hip.sync(S)
    e0, e1 = hip.event(), hip.event()
    hip.record(e0, S)
    for _ in range(reps):
        call()
    hip.record(e1, S)
    return hip.elapsed_ms(e0, e1) / reps


def rows_legs(args, m, synth, torch, np, hip, stream, S, stack, oracle, parity, log):
    """The layer's optional parts, each timed on the decode stack's weights and checked against the
    oracle in the same run: the shared expert with routed_scaling 2.5 (42-layer decode graph),
    renorm-skip (42-layer decode graph under low-confidence routing, against the same routing
    unskipped), the opt-in MXFP8 activations (the 4096-token chunk), and chunks of 16 to 2048
    tokens between the decode and prefill paths."""
    import dataclasses
    wl0 = synth.WORKLOADS["decode"]
    nl, E, d = stack.n, wl0.n_experts, wl0.d_model
    rec = {}
    steps = max(5, args.steps // 2)
    xs = [synth.make_x(wl0, args.seed, "cuda", tokens=1, tag=f"x_rows_{l}") for l in range(nl)]
    bufs = [torch.empty_like(xs[0]), torch.empty_like(xs[0])]
    stride = stack.blob.shape[2]

    # -- shared expert (routed_scaling 2.5): table of E + 1 entries, the last a blob of its own --
    wl_sh = dataclasses.replace(wl0, n_shared=1, routed_scaling=2.5)
    sh_shape = m.make_shape(d, wl0.d_ff, E, wl0.top_k, wl0.wformat, wl0.act_dtype, 2.5, 0.0, 1)
    sh_blob = torch.empty(nl, 1, stride, dtype=torch.uint8, device="cuda")
    sh_table = torch.empty(nl, (E + 1) * m.EXPERT_BYTES, dtype=torch.uint8, device="cuda")
    tmp = torch.zeros(E + 1, stride, dtype=torch.uint8, device="cuda")   # fill_experts addresses blob E
    for l in range(nl):
        synth.fill_experts(tmp, wl_sh, l, args.seed, experts=[E])
        sh_blob[l, 0] = tmp[E]
        sh_table[l, :E * m.EXPERT_BYTES] = stack.table[l]
        ent = torch.frombuffer(bytearray(expert_entry(m, synth, wl0, sh_blob[l, 0].data_ptr())), dtype=torch.uint8)
        sh_table[l, E * m.EXPERT_BYTES:] = ent.cuda()
    del tmp
    ws = m.workspace(sh_shape, 1)
    torch.cuda.synchronize()

    def sh_step(observer=None):
        for l in range(nl):
            m.moe_layer(sh_shape, xs[l], 1, stack.router[l], None, sh_table[l], None, xs[l], bufs[l % 2], None, None,
                        ws, stream=S, observer=observer)
    ms, _ = time_graph(hip, S, sh_step, steps)
    per = kernel_times(hip, m, S, sh_step, reps=2)
    lb = 9 * m.moe_blob_stride(stack.shape) + E * d * 4 + 4 * d
    rec["shared_expert"] = {"workload": "decode stack + one shared expert per layer, routed_scaling 2.5, T=1",
                            "us_per_layer": 1000 * ms / nl, "layer_tokens_per_s": nl / (ms * 1e-3),
                            "hbm_frac_layer": lb / (ms * 1e-3 / nl) / (HBM_PEAK_GBS * 1e9),
                            "kernels_us": {k: float(np.mean(v)) for k, v in per.items()}}
    log(f"# shared expert: {1000 * ms / nl:.2f} us/layer ({100 * rec['shared_expert']['hbm_frac_layer']:.1f}% of HBM "
        f"on 9 experts/layer)")
    if oracle is not None:
        y0 = torch.empty_like(xs[0])
        i0 = torch.empty(1, wl0.top_k, dtype=torch.int32, device="cuda")
        errs, ok = [], True
        for l in (0, nl - 1):
            with torch.cuda.stream(stream):
                m.moe_layer(sh_shape, xs[l], 1, stack.router[l], None, sh_table[l], None, None, y0, i0, None, ws,
                            stream=S)
            hip.sync(S)
            exact, err, _ = oracle_check(oracle, np, torch, wl_sh, lambda e, l=l: stack.blob[l, e].cpu().numpy(),
                                         stack.router[l], None, xs[l], y0, i0, None,
                                         shared_blob=sh_blob[l, 0].cpu().numpy())
            ok = ok and exact
            errs.append(err)
        parity["shared_expert"] = parity_entry(wl_sh, ok, max(errs), f"layers 0 and {nl - 1}, the token")
    del sh_blob, sh_table

    # -- renorm-skip: low-confidence routing (logit bias -2.5 puts the top picks near 0, where the
    #    sigmoid weights spread), threshold 0.11, against the same routing without the skip --
    bias = torch.full((E,), -2.5, dtype=torch.float32, device="cuda")
    wl_rs = dataclasses.replace(wl0, renorm_skip=0.11)
    res = {}
    for tau in (0.0, 0.11):
        sh = m.make_shape(d, wl0.d_ff, E, wl0.top_k, wl0.wformat, wl0.act_dtype, 1.0, tau)
        ws = m.workspace(sh, 1)
        idx = torch.empty(nl, 1, wl0.top_k, dtype=torch.int32, device="cuda")
        torch.cuda.synchronize()

        def rs_step(observer=None, sh=sh, ws=ws, idx=idx):
            for l in range(nl):
                m.moe_layer(sh, xs[l], 1, stack.router[l], bias, stack.table[l], None, xs[l], bufs[l % 2], idx[l],
                            None, ws, stream=S, observer=observer)
        ms, _ = time_graph(hip, S, rs_step, steps)
        kept = float((idx >= 0).sum().item()) / nl
        res[tau] = {"us_per_layer": 1000 * ms / nl, "experts_per_layer": kept}
        if oracle is not None and tau > 0:
            y0 = torch.empty_like(xs[0])
            i0 = torch.empty(1, wl0.top_k, dtype=torch.int32, device="cuda")
            with torch.cuda.stream(stream):
                m.moe_layer(sh, xs[0], 1, stack.router[0], bias, stack.table[0], None, None, y0, i0, None, ws,
                            stream=S)
            hip.sync(S)
            exact, err, _ = oracle_check(oracle, np, torch, wl_rs, lambda e: stack.blob[0, e].cpu().numpy(),
                                         stack.router[0], bias, xs[0], y0, i0)
            parity["renorm_skip"] = parity_entry(wl_rs, exact, err, "layer 0, the token")
    rec["renorm_skip"] = {"workload": "decode stack, logit bias -2.5 (low-confidence routing), threshold 0.11",
                          "skip": res[0.11], "no_skip": res[0.0],
                          "speedup": res[0.0]["us_per_layer"] / res[0.11]["us_per_layer"]}
    log(f"# renorm-skip: {res[0.11]['us_per_layer']:.2f} us/layer with {res[0.11]['experts_per_layer']:.2f} experts "
        f"against {res[0.0]['us_per_layer']:.2f} us with 8")

    # -- opt-in MXFP8 activations, the 4096-token chunk --
    wl_aq = dataclasses.replace(synth.WORKLOADS["prefill"], act_quant=1)
    aq_shape = m.make_shape(d, wl0.d_ff, E, wl0.top_k, wl0.wformat, wl0.act_dtype, 1.0, 0.0, 0, 1)
    T = 4096
    x = synth.make_x(wl_aq, args.seed, "cuda", tokens=T, tag="x_prefill")
    y = torch.empty_like(x)
    idx = torch.empty(T, wl0.top_k, dtype=torch.int32, device="cuda")
    ws = m.workspace(aq_shape, T)
    torch.cuda.synchronize()
    call = lambda observer=None: m.moe_layer(aq_shape, x, T, stack.router[0], None, stack.table[0], None, None, y, idx,
                                             None, ws, stream=S, observer=observer)
    ms = time_calls(hip, S, call, max(3, steps // 3))
    per = kernel_times(hip, m, S, call, reps=2)
    flops = 2.0 * 3 * d * wl0.d_ff * T * wl0.top_k
    rec["mxfp8_activations"] = {"workload": "prefill chunk T=4096, opt-in MXFP8 activations (one E4M3 term)",
                                "ms_per_layer": ms, "tokens_per_s": T / (ms * 1e-3),
                                "fp4_mfma_frac": flops / (ms * 1e-3) / (FP4_PEAK_TFLOPS * 1e12),
                                **issued_mfma(flops, 1, ms, {k: float(np.mean(v)) for k, v in per.items()}),
                                "kernels_us": {k: float(np.mean(v)) for k, v in per.items()}}
    log(f"# MXFP8 activations, prefill T=4096: {ms:.3f} ms/layer; kernels (us): "
        + ", ".join(f"{k} {v:.1f}" for k, v in rec["mxfp8_activations"]["kernels_us"].items()))
    if oracle is not None:
        sample = [0, 2047, 4095]
        exact, err, _ = oracle_check(oracle, np, torch, wl_aq, lambda e: stack.blob[0, e].cpu().numpy(),
                                     stack.router[0], None, x, y, idx, sample)
        parity["mxfp8_activations"] = parity_entry(wl_aq, exact, err, f"T=4096, against the oracle's mirrored mode, "
                                                   f"y of tokens {sample}")
    del x, y, ws

    # -- chunks between decode and prefill (layer 0) --
    wl_p = synth.WORKLOADS["prefill"]
    Tmax = 2048
    ws = m.workspace(stack.shape, Tmax)
    mid = {}
    worst, exact_all = 0.0, True
    for T in (16, 32, 48, 64, 128, 256, 512, 1024, 2048):
        x = synth.make_x(wl_p, args.seed, "cuda", tokens=T, tag=f"x_mid{T}")
        y = torch.empty_like(x)
        idx = torch.empty(T, wl0.top_k, dtype=torch.int32, device="cuda")
        torch.cuda.synchronize()
        call = lambda observer=None: m.moe_layer(stack.shape, x, T, stack.router[0], None, stack.table[0], None, None,
                                                 y, idx, None, ws, stream=S, observer=observer)
        ms = time_calls(hip, S, call, max(5, steps // 2))
        touched = len(np.unique(idx.cpu().numpy()))
        b = algorithmic_layer_bytes(wl_p, touched, T)
        mid[str(T)] = {"ms_per_layer": ms, "tokens_per_s": T / (ms * 1e-3), "experts": touched,
                       "hbm_frac": b / (ms * 1e-3) / (HBM_PEAK_GBS * 1e9)}
        if oracle is not None:
            exact, err, _ = oracle_check(oracle, np, torch, wl_p, lambda e: stack.blob[0, e].cpu().numpy(),
                                         stack.router[0], None, x, y, idx, [0, T - 1])
            exact_all = exact_all and exact
            worst = err if err != err else max(worst, err)
    rec["mid_chunks"] = mid
    log("# chunks: " + ", ".join(f"T={t}: {r['ms_per_layer'] * 1000:.0f} us ({r['tokens_per_s'] / 1e3:.0f}k tok/s, "
                                 f"{100 * r['hbm_frac']:.0f}% HBM)" for t, r in mid.items()))
    if oracle is not None:
        parity["mid_chunks"] = parity_entry(wl_p, exact_all, worst, "T=16..2048: indices of every token, y of the "
                                            "first and last token")
    return rec


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--layers", type=int, default=42)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=20.0)
    ap.add_argument("--only", choices=["decode", "prefill", "batched", "nvfp4", "rows"], default=None)
    ap.add_argument("--nv-layers", type=int, default=8, help="NVFP4 decode stack depth")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (for scaling HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import routed_expert_ffn_router_amd as m
    import synth

    def log(*a):
        print(*a, file=sys.stderr, flush=True)

    torch.cuda.set_device(0)
    if args.copy_calibration:
        # a plain copy of known size: what FETCH_SIZE / WRITE_SIZE read for it scales the counters
        n = 1 << 30
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n, "copies": 3}), flush=True)
        return
    check = not args.no_cpu_baseline
    oracle = None
    if check:
        import oracle
    hip = Hip()
    stream = torch.cuda.Stream()
    S = stream.cuda_stream
    out = {}
    parity = {}
    want = (lambda w: args.only is None or args.only == w)

    # ---------------- decode stack (headline) ----------------
    wl_dec = synth.WORKLOADS["decode"]
    nl = args.layers
    stack = None
    if want("decode") or want("batched") or want("prefill") or want("rows"):
        log(f"# building the {nl}-layer decode stack in HBM")
        stack = Stack(m, synth, torch, wl_dec, nl, args.seed, log)

    def run_stack(T, biases, xs, bufs, ws, keep=None):
        """One step: every layer l reads its own input xs[l] and writes y_l = xs[l] + MoE_l(xs[l])
        (residual fused).  Each input stands in for the normalised hidden state a transformer block
        hands its MoE layer; feeding one layer's output straight into the next, with no norm
        between them, grows the activations without bound (past bf16's range by layer 19)."""
        def fn(observer=None):
            for l in range(nl):
                m.moe_layer(stack.shape, xs[l], T, stack.router[l], biases[l], stack.table[l], None, xs[l],
                            bufs[l % 2], None if keep is None else keep[0][l],
                            None if keep is None else keep[1][l], ws, stream=S, observer=observer)
        return fn

    for name, T in (("decode", 1), ("batched", 64)):
        if not want(name):
            continue
        wl = synth.WORKLOADS[name]
        biases = [synth.make_bias(wl, l, args.seed, "cuda") for l in range(nl)]
        xs = [synth.make_x(wl, args.seed, "cuda", tokens=T, tag=f"x_{name}_{l}") for l in range(nl)]
        bufs = [torch.empty_like(xs[0]), torch.empty_like(xs[0])]
        ws = m.workspace(stack.shape, T)
        idx_keep = torch.empty(nl, T, wl.top_k, dtype=torch.int32, device="cuda")
        w_keep = torch.empty(nl, T, wl.top_k, dtype=torch.float32, device="cuda")
        # the inputs and the zero-filled workspace come from torch's stream; S (a non-blocking
        # stream) does not wait for it by itself
        torch.cuda.synchronize()
        # eager reference step (keeps every layer's routing), then the graph
        with torch.cuda.stream(stream):
            run_stack(T, biases, xs, bufs, ws, keep=(idx_keep, w_keep))()
        hip.sync(S)
        y_eager = bufs[(nl - 1) % 2].clone()
        gexec, _ = hip.capture(S, run_stack(T, biases, xs, bufs, ws, keep=(idx_keep, w_keep)))
        for _ in range(3):      # replays reproduce the eager step bit for bit
            hip.launch(gexec, S)
            hip.sync(S)
            assert torch.equal(bufs[(nl - 1) % 2].view(torch.int16), y_eager.view(torch.int16)), \
                "graph replay differs from the eager step"
        for _ in range(args.warmup):
            hip.launch(gexec, S)
        hip.sync(S)
        e0, e1 = hip.event(), hip.event()
        torch.cuda.synchronize()
        hip.record(e0, S)
        for _ in range(args.steps):
            hip.launch(gexec, S)
        hip.record(e1, S)
        ms = hip.elapsed_ms(e0, e1) / args.steps
        torch.cuda.synchronize()
        assert m.workspace_status(ws) == 0, "workspace status word set"
        # per-kernel durations: events recorded by each kernel's own dispatch, same step
        per = kernel_times(hip, m, S, run_stack(T, biases, xs, bufs, ws))
        kern = {k: float(np.mean(v)) for k, v in per.items()}
        touched = [len(np.unique(idx_keep[l].cpu().numpy())) for l in range(nl)]
        layer_bytes = float(np.mean([algorithmic_layer_bytes(wl, u, T) for u in touched]))
        us_layer = 1000.0 * ms / nl
        rec = {
            "ms_per_step": ms, "us_per_layer": us_layer, "tokens": T, "layers": nl,
            "layer_tokens_per_s": nl * T / (ms / 1000.0), "stack_tokens_per_s": T / (ms / 1000.0),
            "algorithmic_bytes_per_layer": layer_bytes, "mean_experts_per_layer": float(np.mean(touched)),
            "hbm_frac_layer": layer_bytes / (us_layer * 1e-6) / (HBM_PEAK_GBS * 1e9),
            "kernels_us": kern,
        }
        gu_bytes = float(np.mean([gate_up_bytes(wl, u) for u in touched]))
        rec["gate_up_roofline"] = {"bound": "hbm", "achieved": gu_bytes / (kern["gemm_gate_up"] * 1e-6) / 1e9,
                                   "peak": HBM_PEAK_GBS, "unit": "GB/s", "bytes_per_launch": gu_bytes}
        rec["gate_up_roofline"]["frac"] = rec["gate_up_roofline"]["achieved"] / HBM_PEAK_GBS
        out[name] = rec
        out[name + "_state"] = (idx_keep, w_keep, xs, bufs, ws, biases)
        log(f"# {name}: {ms:.3f} ms/step, {us_layer:.2f} us/layer, "
            f"{rec['layer_tokens_per_s']:.0f} layer-tokens/s, {100 * rec['hbm_frac_layer']:.1f}% of HBM peak")
        log(f"#   kernels (us): " + ", ".join(f"{k} {v:.2f}" for k, v in kern.items()))

    # ---------------- prefill chunk (layer 0 of the stack, T=4096) ----------------
    if want("prefill"):
        wl = synth.WORKLOADS["prefill"]
        T = wl.tokens
        x = synth.make_x(wl, args.seed, "cuda", tokens=T, tag="x_prefill")
        y = torch.empty_like(x)
        idx = torch.empty(T, wl.top_k, dtype=torch.int32, device="cuda")
        wts = torch.empty(T, wl.top_k, dtype=torch.float32, device="cuda")
        ws = m.workspace(stack.shape, T)
        torch.cuda.synchronize()        # inputs and workspace ready before S uses them
        call = lambda observer=None: m.moe_layer(stack.shape, x, T, stack.router[0], None, stack.table[0], None,
                                                 None, y, idx, wts, ws, stream=S, observer=observer)
        for _ in range(max(2, args.warmup)):
            call()
        hip.sync(S)
        e0, e1 = hip.event(), hip.event()
        steps = max(3, args.steps // 5)
        hip.record(e0, S)
        for _ in range(steps):
            call()
        hip.record(e1, S)
        ms = hip.elapsed_ms(e0, e1) / steps
        per = kernel_times(hip, m, S, call)
        kern = {k: float(np.mean(v)) for k, v in per.items()}
        flops = 2.0 * 3 * wl.d_model * wl.d_ff * T * wl.top_k
        touched = len(np.unique(idx.cpu().numpy()))
        bytes_ = algorithmic_layer_bytes(wl, touched, T)
        floor_ms = max(bytes_ / (HBM_PEAK_GBS * 1e9), flops / (FP4_PEAK_TFLOPS * 1e12)) * 1e3
        out["prefill"] = {
            "ms_per_layer": ms, "tokens": T, "tokens_per_s": T / (ms / 1000.0),
            "experts_active": touched, "algorithmic_bytes": bytes_, "algorithmic_tflop": flops / 1e12,
            "hbm_frac": bytes_ / (ms * 1e-3) / (HBM_PEAK_GBS * 1e9),
            "fp4_mfma_frac": flops / (ms * 1e-3) / (FP4_PEAK_TFLOPS * 1e12),
            "roofline_frac": floor_ms / ms, "kernels_us": kern,
            # the MFMAs actually issued: each activation as `terms` FP8 columns, FP4 x FP8 at the FP8 rate
            **issued_mfma(flops, 2 if wl.act_dtype == 1 else 4, ms, kern),
        }
        log(f"# prefill T={T}: {ms:.3f} ms/layer, {T / ms * 1e3:.0f} tokens/s, "
            f"{100 * out['prefill']['roofline_frac']:.1f}% of the roofline bound")
        log(f"#   kernels (us): " + ", ".join(f"{k} {v:.1f}" for k, v in kern.items()))
        if check:
            # routing of all 4096 tokens, y on 8 tokens spread over the chunk
            sample = [0, 1, 511, 1024, 2047, 2048, 3333, 4095]
            exact, err, secs = oracle_check(oracle, np, torch, wl, lambda e: stack.blob[0, e].cpu().numpy(),
                                            stack.router[0], None, x, y, idx, sample)
            parity["prefill"] = parity_entry(wl, exact, err, f"T=4096: indices of all tokens, y of tokens {sample}")
            out["prefill"]["oracle_sample"] = {"tokens": len(sample), "seconds": secs}
            log(f"#   parity {parity['prefill']}")

    # ---------------- NVFP4 configuration: decode T=1 and a 2048-token chunk, staged or not ------
    if want("nvfp4"):
        wl = synth.WORKLOADS["nvfp4_decode"]
        nvl = args.nv_layers
        log(f"# building the {nvl}-layer NVFP4 stack in HBM")
        nst = Stack(m, synth, torch, wl, nvl, args.seed, log)
        stride = m.moe_blob_stride(nst.shape)
        staging = torch.empty(min(wl.n_experts, 64), nst.blob.shape[2], dtype=torch.uint8, device="cuda")
        rec = {}
        for T in (1, 2048):
            # each layer its own input, as in the decode stack
            xs = [synth.make_x(wl, args.seed, "cuda", tokens=T, tag=f"x_nv{T}_{l}") for l in range(nvl)]
            bufs = [torch.empty_like(xs[0]), torch.empty_like(xs[0])]
            ws = m.workspace(nst.shape, T)
            idx = torch.empty(nvl, T, wl.top_k, dtype=torch.int32, device="cuda")
            torch.cuda.synchronize()    # inputs and workspace ready before S uses them
            for staged in (False, True):
                def step(observer=None, staged=staged):
                    for l in range(nvl):
                        m.moe_layer(nst.shape, xs[l], T, nst.router[l], None, nst.table[l],
                                    staging if staged else None, xs[l], bufs[l % 2], idx[l], None, ws, stream=S,
                                    observer=observer)
                with torch.cuda.stream(stream):
                    step()
                hip.sync(S)
                if T == 1:
                    gexec, _ = hip.capture(S, step)
                    run = lambda: hip.launch(gexec, S)
                else:
                    run = step
                reps = max(3, args.steps // (1 if T == 1 else 10))
                for _ in range(2):
                    run()
                hip.sync(S)
                e0, e1 = hip.event(), hip.event()
                hip.record(e0, S)
                for _ in range(reps):
                    run()
                hip.record(e1, S)
                ms = hip.elapsed_ms(e0, e1) / reps / nvl
                kern = {k: float(np.mean(v)) for k, v in kernel_times(hip, m, S, step, reps=2).items()}
                touched = float(np.mean([len(np.unique(idx[l].cpu().numpy())) for l in range(nvl)]))
                ffn_bytes = touched * stride + wl.n_experts * wl.d_model * 4
                stage_bytes = 2 * touched * stride if staged else 0
                key = f"T{T}_{'staged' if staged else 'in_place'}"
                rec[key] = {"ms_per_layer": ms, "tokens_per_s": T / (ms * 1e-3), "experts_per_layer": touched,
                            "bytes_without_staging": ffn_bytes, "staging_bytes": stage_bytes,
                            "hbm_frac_without_staging": ffn_bytes / (ms * 1e-3) / (HBM_PEAK_GBS * 1e9),
                            "hbm_frac_with_staging": (ffn_bytes + stage_bytes) / (ms * 1e-3) / (HBM_PEAK_GBS * 1e9),
                            "kernels_us": kern}
                log(f"# nvfp4 {key}: {1000 * ms:.1f} us/layer, {T / (ms * 1e-3):.0f} tokens/s, "
                    f"{touched:.0f} experts/layer; kernels (us): " + ", ".join(f"{k} {v:.1f}" for k, v in kern.items()))
                if check:
                    # layer 0 once more without the residual, against the oracle (T=1: the token;
                    # T=2048: indices of every token, y of 4 tokens)
                    y0 = torch.empty_like(xs[0])
                    i0 = torch.empty(T, wl.top_k, dtype=torch.int32, device="cuda")
                    with torch.cuda.stream(stream):
                        m.moe_layer(nst.shape, xs[0], T, nst.router[0], None, nst.table[0],
                                    staging if staged else None, None, y0, i0, None, ws, stream=S)
                    hip.sync(S)
                    sample = None if T == 1 else [0, 5, 1000, 2047]
                    exact, err, secs = oracle_check(oracle, np, torch, wl, lambda e: nst.blob[0, e].cpu().numpy(),
                                                    nst.router[0], None, xs[0], y0, i0, sample)
                    parity["nvfp4_" + key] = parity_entry(wl, exact, err, "layer 0, indices of every token, y of "
                                                          + ("the token" if T == 1 else f"tokens {sample}"))
                    rec[key]["oracle_sample"] = {"tokens": T if sample is None else len(sample), "seconds": secs}
                    log(f"#   parity {parity['nvfp4_' + key]}")
        out["nvfp4"] = rec
        del nst

    # ---------------- the layer's optional parts and the mid-size chunks ----------------
    if want("rows"):
        out["rows"] = rows_legs(args, m, synth, torch, np, hip, stream, S, stack, oracle if check else None, parity,
                                log)

    # ---------------- batched parity: layers 0 and 41, all 64 tokens ----------------
    if want("batched") and check:
        wl = synth.WORKLOADS["batched"]
        idx_keep, w_keep, xs, bufs, ws, biases = out["batched_state"]
        worst, exact_all, secs_all = 0.0, True, 0.0
        for l in (0, nl - 1):
            y_l = torch.empty_like(xs[l])
            i_l = torch.empty(64, wl.top_k, dtype=torch.int32, device="cuda")
            with torch.cuda.stream(stream):
                m.moe_layer(stack.shape, xs[l], 64, stack.router[l], biases[l], stack.table[l], None, None, y_l,
                            i_l, None, ws, stream=S)
            hip.sync(S)
            exact, err, secs = oracle_check(oracle, np, torch, wl, lambda e, l=l: stack.blob[l, e].cpu().numpy(),
                                            stack.router[l], biases[l], xs[l], y_l, i_l)
            exact_all = exact_all and exact and torch.equal(i_l, idx_keep[l])
            worst = err if err != err else max(worst, err)
            secs_all += secs
        parity["batched"] = parity_entry(wl, exact_all, worst, f"layers 0 and {nl - 1}, all 64 tokens")
        out["batched"]["oracle_sample"] = {"layers": 2, "tokens": 64, "seconds": secs_all}
        log(f"#   batched parity {parity['batched']}")

    # ---------------- oracle on the host cores (bounded sample of the decode stack) ------------
    cpu = None
    if want("decode") and check:
        idx_keep, w_keep, xs, bufs, ws, _ = out["decode_state"]
        # every layer's output y_l without the residual, on its own input x_l
        ys = []
        with torch.cuda.stream(stream):
            for l in range(nl):
                y_l = torch.empty_like(xs[l])
                m.moe_layer(stack.shape, xs[l], 1, stack.router[l], None, stack.table[l], None, None, y_l, None,
                            None, ws, stream=S)
                ys.append(y_l)
        hip.sync(S)
        t_cpu = 0.0
        n_done = 0
        worst = 0.0
        exact = True
        for l in range(nl):
            sel = idx_keep[l].cpu().numpy().reshape(-1)
            blobs = [None] * wl_dec.n_experts
            for e in sel:
                blobs[int(e)] = stack.blob[l, int(e)].cpu().numpy()
            x64 = oracle.to_f64(xs[l])
            wr = stack.router[l].cpu().numpy()
            t0 = time.perf_counter()
            oy, oidx, ow, _ = oracle.layer(x64, wr, None, blobs, wl_dec.d_model, wl_dec.d_ff, wl_dec.top_k,
                                           wl_dec.wformat, 1.0, None)
            t_cpu += time.perf_counter() - t0
            n_done += 1
            exact = exact and bool(np.array_equal(oidx, idx_keep[l].cpu().numpy()))
            err = rel_l2(oracle.to_f64(ys[l]), oy)
            worst = err if not np.isfinite(err) else max(worst, err)     # a NaN or inf fails the check
            if not np.isfinite(worst):
                break
            if t_cpu > args.cpu_seconds:
                break
        cpu = {"value": n_done / t_cpu, "unit": "layer-tokens/s", "cores": oracle.num_threads(), "kind": "oracle",
               "sample": f"decode stack, T=1, first {n_done} of {nl} layers on the GPU's own layer inputs "
                         f"({t_cpu:.1f} s of fp64 oracle time)",
               "host": host_info()}
        # the other legs' oracle samples, as rates (tokens per second of oracle time)
        also = {}
        if "prefill" in out and "oracle_sample" in out["prefill"]:
            o_ = out["prefill"]["oracle_sample"]
            also["prefill_T4096_tokens_per_s"] = o_["tokens"] / o_["seconds"]
        if "nvfp4" in out:
            for key in ("T1_in_place", "T2048_in_place"):
                o_ = out["nvfp4"].get(key, {}).get("oracle_sample")
                if o_:
                    also[f"nvfp4_{key}_tokens_per_s"] = o_["tokens"] / o_["seconds"]
        if "batched" in out and "oracle_sample" in out["batched"]:
            o_ = out["batched"]["oracle_sample"]
            also["batched_layer_tokens_per_s"] = o_["layers"] * o_["tokens"] / o_["seconds"]
        cpu["other_samples"] = also
        parity["decode"] = parity_entry(wl_dec, exact, worst, f"{n_done} of {nl} layers, the token")
        log(f"# oracle: {cpu['value']:.3f} layer-tokens/s on {cpu['cores']} threads; parity {parity['decode']}")

    # ---------------- the one JSON line ----------------
    all_pass = bool(parity) and all(p["pass"] for p in parity.values())
    dec = out.get("decode")
    line = {"metric": METRIC, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "mxfp4 x fp8-terms, fp32 accumulate", "data": "synthetic"}
    if dec is not None:
        line.update({
            "value": dec["layer_tokens_per_s"], "unit": "layer-tokens/s", "ms_per_step": dec["ms_per_step"],
            "config": {"workload": "decode: 42 stacked MoE layers, d_model 4096, d_ff 2048, 288 MXFP4 experts "
                                   "(E2M1 + E8M0/32), top-8 sigmoid router, T=1, bf16 activations, flat routing; "
                                   "each layer reads its own unit-scale input (the normalised hidden state), "
                                   "residual fused",
                       "layers": nl, "tokens_per_step": 1, "parallelism": "single GPU"},
            "stack_tokens_per_s": dec["stack_tokens_per_s"], "us_per_layer": dec["us_per_layer"],
            "hbm_frac_layer": dec["hbm_frac_layer"],
            "roofline": {"bound": "hbm", "kernel": "gemm_gate_up (k_mx_gateup_dec: gate and up of 8 experts, "
                                                  "8.9 MB each)",
                         "achieved": dec["gate_up_roofline"]["achieved"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": dec["gate_up_roofline"]["frac"], "traffic": measured_traffic("k_mx_gateup_dec"),
                         "bytes_per_launch": dec["gate_up_roofline"]["bytes_per_launch"],
                         "avg_launch_us": dec["kernels_us"]["gemm_gate_up"],
                         "timer": "HIP events recorded by the kernel's own dispatch (hipExtLaunchKernel) on its "
                                  "stream, mean over 3 eager steps of 42 layers"},
            "kernels_us": dec["kernels_us"],
        })
    else:
        first = next((k for k in ("prefill", "batched", "nvfp4") if k in out), None)
        if first is None:         # only the optional rows ran: their figures are under "rows"
            line.update({"value": None, "unit": "layer-tokens/s", "ms_per_step": None,
                         "config": {"workload": "rows"}})
        else:
            r = out[first] if first != "nvfp4" else out["nvfp4"]["T1_in_place"]
            line.update({"value": r.get("tokens_per_s", r.get("layer_tokens_per_s")), "unit": "tokens/s",
                         "ms_per_step": r.get("ms_per_layer", r.get("ms_per_step")),
                         "config": {"workload": first}})
    line["cpu_baseline"] = cpu
    line["parity"] = dict(parity, all_pass=all_pass) if parity else None
    for k in ("prefill", "batched", "nvfp4", "rows"):
        if k in out:
            line[k] = {kk: vv for kk, vv in out[k].items()}
    failed = bool(parity) and not all_pass
    if failed:
        line["value"] = None          # no number without a passing parity check in the same run
    print(json.dumps(line), flush=True)
    if failed:
        sys.exit(1)


if __name__ == "__main__":
    main()
