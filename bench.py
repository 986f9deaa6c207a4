"""Benchmark of the YOCO shared-KV attention hot path on one MI355X.

Default workload (the one the headline metric is quoted on): the 3B-shaped
bf16 prefill -- batch 1, 4096 tokens, hidden 3072, 24 query / 8 KV heads,
head_dim 128; 8 sliding-window layers (window 1024), one global KV
projection, 8 causal cross-decoder layers over the one shared cache.
One step = that whole pass over one batch; value = algorithmic TFLOP/s of
the step (unmasked query-key pairs only, 2 flops per MAC, exp not counted).

The same run also measures the cross-attention decode kernel at its own
headline shape (batch 16, context 32768, 32/8 heads, 16 cross layers x 128
steps) and reports its HBM GB/s, the 512K fp8-cache decode, the one-token
generation step at the decode shape (16 self-decoder ring layers, the
one-row KV projection, 16 cross layers), the 1M-token early-exit prefill,
and times the float64 CPU oracle on a bounded sample of the prefill step
("cpu_baseline").

Prints ONE JSON line.  Inputs are seeded synthetic tensors already resident
in HBM when timing starts.
"""
import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import shared_kv_attention_amd as yk  # noqa: E402
from shared_kv_attention_amd.synth import WORKLOADS, randn, seed_for  # noqa: E402

METRIC = "cross-attn decode KV GB/s (% HBM peak); prefill TFLOP/s (% MFMA peak)"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
PROFILES = os.path.join(ROOT, "profiles")


# ---------------------------------------------------------------- counting
def swa_pairs(n, w):
    """Number of (query, key) pairs with t - W < s <= t."""
    full = min(n, w)
    return full * (full + 1) // 2 + (n - full) * w


def causal_pairs(nq, q_offset=0):
    """Pairs with s <= q_offset + i for query rows i = 0..nq-1."""
    return nq * q_offset + nq * (nq + 1) // 2


def attn_flops(pairs, heads, d, batch):
    return 4.0 * d * heads * batch * pairs          # QK^T and PV, 2 flops per MAC


def proj_flops(batch, n, hidden, kv_width):
    return 2.0 * batch * n * hidden * 2 * kv_width


def decode_bytes(batch, hkv, ctx, d, hq, kv_bytes, q_bytes):
    return 2.0 * batch * hkv * ctx * d * kv_bytes + 2.0 * batch * hq * d * q_bytes


# ---------------------------------------------------------------- helpers
def events_ms(pairs):
    return [s.elapsed_time(e) for s, e in pairs]


def kernel_source_digest(name):
    with open(os.path.join(ROOT, "shared_kv_attention_amd", "csrc", name), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def traffic_from_profile(summary_name, kernel_file, per_launch_key):
    """HBM bytes per launch from a committed counter summary, if the kernel is unchanged."""
    path = os.path.join(PROFILES, summary_name)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"source sha256/16:\s*([0-9a-f]+)", text)
    if not m or m.group(1) != kernel_source_digest(kernel_file):
        return None
    m = re.search(per_launch_key + r":\s*([0-9.eE+]+)", text)
    return float(m.group(1)) if m else None


# ---------------------------------------------------------------- prefill step
class PrefillStep:
    def __init__(self, wl, dev):
        self.wl = wl
        B, N, D, Hq, Hkv, d = wl.batch, wl.seq, wl.hidden, wl.n_heads, wl.n_kv_heads, wl.head_dim
        wid = wl.wid
        self.x = randn((B, N, D), seed_for(wid, 0), device=dev)
        self.wk = randn((Hkv * d, D), seed_for(wid, 1), std=wl.weight_std, device=dev)
        self.wv = randn((Hkv * d, D), seed_for(wid, 2), std=wl.weight_std, device=dev)
        self.swa = []
        for layer in range(wl.n_self_layers):
            s0 = seed_for(wid, 10 + 3 * layer)
            self.swa.append((randn((B, Hq, N, d), s0, device=dev),
                             randn((B, Hkv, N, d), s0 + 1, device=dev),
                             randn((B, Hkv, N, d), s0 + 2, device=dev)))
        self.cross_q = [randn((B, Hq, N, d), seed_for(wid, 200 + layer), device=dev)
                        for layer in range(wl.n_cross_layers)]
        self.kc = torch.empty(B, Hkv, N, d, dtype=torch.bfloat16, device=dev)
        self.vc = torch.empty_like(self.kc)
        self.o_swa = [torch.empty(B, Hq, N, d, dtype=torch.bfloat16, device=dev) for _ in self.swa]
        self.o_cross = [torch.empty(B, Hq, N, d, dtype=torch.bfloat16, device=dev) for _ in self.cross_q]
        self.flops_swa = attn_flops(swa_pairs(N, wl.window), Hq, d, B)
        self.flops_cross = attn_flops(causal_pairs(N), Hq, d, B)
        self.flops_proj = proj_flops(B, N, D, Hkv * d)
        self.flops = (wl.n_self_layers * self.flops_swa + self.flops_proj
                      + wl.n_cross_layers * self.flops_cross)

    def run(self, ev=None):
        wl = self.wl
        for (q, k, v), o in zip(self.swa, self.o_swa):
            yk.yoco_swa_attn(q, k, v, wl.window, o=o)
        yk.yoco_global_kv_proj(self.x, self.wk, self.wv, self.kc, self.vc)
        # the cross layers run back to back; one event pair around all of
        # them (an event between two launches opens a gap of several
        # microseconds in the stream), so a launch's duration is the span / L
        if ev is not None:
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record()
        for q, o in zip(self.cross_q, self.o_cross):
            yk.yoco_cross_attn_prefill(q, self.kc, self.vc, o=o)
        if ev is not None:
            e.record()
            ev.append((s, e))


def cpu_baseline_prefill(step, budget_s):
    """Time the float64 oracle on a sample of the prefill step's rows."""
    import numpy as np

    import oracle
    wl = step.wl
    N, Hq, d, W = wl.seq, wl.n_heads, wl.head_dim, wl.window
    f = lambda t: t.double().cpu().numpy()  # noqa: E731
    # sample: every `stride`-th query row of every head of one SWA layer and
    # one cross layer, and every `stride`-th token of the projection
    stride = 64
    rows = list(range(stride // 2, N, stride))
    q, k, v = (f(t) for t in step.swa[0])
    kc, vc, qc = f(step.kc), f(step.vc), f(step.cross_q[0])
    x, wk, wv = f(step.x), f(step.wk), f(step.wv)
    flops = 0.0
    t0 = time.perf_counter()
    reps = 0
    while True:
        oracle.swa_attention(q, k, v, W, rows=rows)
        flops += sum(4.0 * d * Hq * min(t + 1, W) for t in rows)
        oracle.cross_prefill_attention(qc, kc, vc, rows=rows)
        flops += sum(4.0 * d * Hq * (t + 1) for t in rows)
        oracle.global_kv_proj(x, wk, wv, wl.n_kv_heads, d, rows=rows)
        flops += proj_flops(1, len(rows), wl.hidden, wl.n_kv_heads * d)
        reps += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    threads = None
    try:
        from threadpoolctl import threadpool_info
        threads = max((p.get("num_threads", 1) for p in threadpool_info()), default=1)
    except Exception:  # noqa: BLE001
        pass
    cores = len(os.sched_getaffinity(0))
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": threads or cores,
        "host_cores": cores,
        "kind": "oracle",
        "sample": (f"{reps}x: {len(rows)} query rows (every {stride}th) x {Hq} heads of one SWA layer "
                   f"and one cross layer, plus {len(rows)} projection tokens; float64 numpy, "
                   f"{dt:.1f} s wall"),
    }


def _threads():
    try:
        from threadpoolctl import threadpool_info
        return max((p.get("num_threads", 1) for p in threadpool_info()), default=1)
    except Exception:  # noqa: BLE001
        return len(os.sched_getaffinity(0))


def _time_until(fn, budget_s):
    t0 = time.perf_counter()
    reps = 0
    while True:
        fn()
        reps += 1
        if time.perf_counter() - t0 >= budget_s:
            return (time.perf_counter() - t0) / reps, reps


def cpu_baseline_decode(smp, budget_s):
    """The oracle's decode (float64) on the sampled (sequence, KV head) groups
    of one call, extrapolated to every group of the call and to the
    workload's calls."""
    import numpy as np

    import oracle
    groups = smp["groups"]

    def one():
        for i in range(len(groups)):
            if smp["fp8"]:
                k = oracle.dequantize_kv_fp8(smp["k"][i][None, None], np.array([smp["ks"][i]], dtype=np.float32))
                v = oracle.dequantize_kv_fp8(smp["v"][i][None, None], np.array([smp["vs"][i]], dtype=np.float32))
            else:
                k, v = smp["k"][i][None, None], smp["v"][i][None, None]
            oracle.decode_attention(smp["q"][i][None], k, v, [smp["ctx"]])

    per_sample, reps = _time_until(one, budget_s)
    per_call = per_sample / len(groups) * smp["B"] * smp["Hkv"]
    return {
        "workload": smp["workload"], "extrapolated": True,
        "value": smp["bytes_per_call"] / per_call / 1e9, "unit": "GB/s",
        "oracle_s_per_call": per_call, "oracle_s_workload": per_call * smp["calls"], "calls": smp["calls"],
        "cores": _threads(), "kind": "oracle",
        "sample": (f"{reps}x: {len(groups)} of {smp['B'] * smp['Hkv']} (sequence, KV head) groups of one call "
                   f"({smp['g']} query heads x {smp['ctx']} keys each"
                   + (", codes decoded to float64 first" if smp["fp8"] else "")
                   + "), float64 numpy; extrapolated to the whole call and to every call"),
    }


def cpu_baseline_early_exit(smp, budget_s):
    """The oracle on samples of the 1M-token early exit: window rows of one
    layer, projection rows, and the last position's decode over one KV head
    of the full cache -- each extrapolated to the whole flow."""
    import numpy as np

    import oracle
    N, W, Ls, Lc, Hkv, d = smp["N"], smp["W"], smp["Ls"], smp["Lc"], smp["Hkv"], smp["d"]
    rows = smp["rows"]

    def swa_rows():
        # each sampled row with its window of keys: the query sits at the
        # window's last position and sees all of it (the window's allowed set)
        for q, k, v in smp["swa"]:
            oracle.cross_prefill_attention(q, k, v, n_kv=k.shape[2], q_offset=k.shape[2] - 1)

    def proj_rows():
        oracle.global_kv_proj(smp["x"], smp["wk"], smp["wv"], Hkv, d)

    def decode_head():
        oracle.decode_attention(smp["dec_q"], smp["dec_k"], smp["dec_v"], [N])

    t_swa, r1 = _time_until(swa_rows, budget_s / 3)
    t_proj, r2 = _time_until(proj_rows, budget_s / 3)
    t_dec, r3 = _time_until(decode_head, budget_s / 3)
    s_swa = t_swa / len(rows) * N * Ls
    s_proj = t_proj / len(rows) * N
    s_dec = t_dec * Hkv * Lc
    total = s_swa + s_proj + s_dec
    flops = (Ls * attn_flops(swa_pairs(N, W), Hkv * smp["g"], d, 1) + proj_flops(1, N, smp["x"].shape[-1], Hkv * d)
             + Lc * attn_flops(N, Hkv * smp["g"], d, 1))
    return {
        "workload": smp["workload"], "extrapolated": True,
        "value": flops / total / 1e12, "unit": "TFLOP/s",
        "oracle_s_per_step": total,
        "parts_s": {"swa": s_swa, "kv_proj": s_proj, "last_token_decode": s_dec},
        "cores": _threads(), "kind": "oracle",
        "sample": (f"window layer: {len(rows)} query rows x all heads ({r1}x), projection: {len(rows)} rows "
                   f"({r2}x), decode of the last position over one KV head of the 2^20-row cache ({r3}x); "
                   "float64 numpy; extrapolated to every row, layer and KV head"),
    }


# ---------------------------------------------------------------- decode
def run_decode(wl, dev, steps, sample=None, n_groups=2):
    """Times the decode calls; with `sample` (a dict), also copies n_groups
    (sequence, KV head) groups of the cache and one call's queries to the host
    for the oracle timing."""
    B, ctx, Hq, Hkv, d, L = wl.batch, wl.seq, wl.n_heads, wl.n_kv_heads, wl.head_dim, wl.n_cross_layers
    wid = wl.wid
    fp8 = wl.dtype == "fp8-kv"
    if fp8:
        kf = randn((B, Hkv, ctx, d), seed_for(wid, 0), dtype="f32", device=dev)
        kc, ks = yk.yoco_kv_quantize_fp8(kf)
        del kf
        vf = randn((B, Hkv, ctx, d), seed_for(wid, 1), dtype="f32", device=dev)
        vc, vs = yk.yoco_kv_quantize_fp8(vf)
        del vf
        kv_bytes = 1
    else:
        kc = randn((B, Hkv, ctx, d), seed_for(wid, 0), device=dev)
        vc = randn((B, Hkv, ctx, d), seed_for(wid, 1), device=dev)
        ks = vs = None
        kv_bytes = 2
    qs = randn((L, B, Hq, d), seed_for(wid, 2), device=dev)
    o = torch.empty(B, Hq, d, dtype=torch.bfloat16, device=dev)
    ws = torch.empty(yk.yoco_cross_attn_decode_workspace_bytes(B, Hq, Hkv, ctx, d), dtype=torch.uint8, device=dev)

    def call(layer):
        yk.yoco_cross_attn_decode(qs[layer], kc, vc, ctx, k_scale=ks, v_scale=vs, o=o, workspace=ws)

    if sample is not None:
        g = Hq // Hkv
        groups = [((7 * i) % B, (3 * i + 1) % Hkv) for i in range(n_groups)]
        sample.update(workload=wl.name, groups=groups, g=g, B=B, Hkv=Hkv, ctx=ctx, d=d, fp8=fp8,
                      calls=steps * L, bytes_per_call=decode_bytes(B, Hkv, ctx, d, Hq, kv_bytes, 2),
                      q=[qs[0, b, kvh * g:(kvh + 1) * g].float().cpu().numpy() for b, kvh in groups],
                      k=[kc[b, kvh].cpu().numpy() if fp8 else kc[b, kvh].float().cpu().numpy() for b, kvh in groups],
                      v=[vc[b, kvh].cpu().numpy() if fp8 else vc[b, kvh].float().cpu().numpy() for b, kvh in groups],
                      ks=None if not fp8 else [float(ks[kvh]) for _, kvh in groups],
                      vs=None if not fp8 else [float(vs[kvh]) for _, kvh in groups])

    for layer in range(min(L, 4)):   # warm-up
        call(layer)
    torch.cuda.synchronize()
    ev = []
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    # one event pair per step around its L back-to-back calls (an event
    # between two launches opens a gap of several microseconds)
    for _ in range(steps):
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for layer in range(L):
            call(layer)
        e.record()
        ev.append((s, e))
    t1.record()
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)
    per_call = sum(events_ms(ev)) / (len(ev) * L)
    nbytes = decode_bytes(B, Hkv, ctx, d, Hq, kv_bytes, 2)
    gbs = nbytes / (per_call * 1e-3) / 1e9
    return {
        "workload": wl.name,
        "calls": len(ev) * L,
        "ms_per_call": per_call,
        "total_ms": total_ms,
        "bytes_per_call": nbytes,
        "GB/s": gbs,
        "frac_hbm_peak": gbs / HBM_PEAK_GBS,
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS,
                     "traffic": traffic_from_profile(f"decode_split_{wl.name}.txt", "decode.hip",
                                                     "hbm bytes per launch")},
        "timing": "HIP events around each step's back-to-back calls (split kernel + combine kernel per call); per call = span / calls",
    }


# ---------------------------------------------------------------- 8-bit cache writer
def run_quantize(wl, dev, reps=5):
    """Times yoco_kv_quantize_fp8 on one bf16 cache tensor of the decode
    workload's shape (its K).  The per-head scale needs every row's maximum
    before any code is written, so the writer reads the input twice (maxima,
    then encode) and writes the codes once: those are the bytes counted."""
    B, ctx, Hkv, d = wl.batch, wl.seq, wl.n_kv_heads, wl.head_dim
    kv = randn((B, Hkv, ctx, d), seed_for(wl.wid, 0), device=dev)
    codes = torch.empty(kv.shape, dtype=torch.uint8, device=dev)
    scale = torch.empty(Hkv, dtype=torch.float32, device=dev)
    ws = torch.empty(max(yk.yoco_kv_quantize_fp8_workspace_bytes(Hkv), 16), dtype=torch.uint8, device=dev)
    call = lambda: yk.yoco_kv_quantize_fp8(kv, codes, scale, ws)  # noqa: E731
    call()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(reps):
        call()
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / reps
    n = kv.numel()
    nbytes = 2 * n * 2 + n
    gbs = nbytes / (ms * 1e-3) / 1e9
    out = {"shape": [B, Hkv, ctx, d], "input": "bf16", "calls": reps, "ms_per_call": ms, "bytes_per_call": nbytes,
           "GB/s": gbs, "frac_hbm_peak": gbs / HBM_PEAK_GBS,
           "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": gbs / HBM_PEAK_GBS,
                        "traffic": traffic_from_profile("quant_fp8_decode_32k_bf16.txt", "fp8_quant.hip",
                                                        "hbm bytes per call")},
           "bytes": "input read twice (per-head maxima, then encode), codes written once",
           "timing": "HIP events around back-to-back calls (clear + maxima + encode kernels per call)"}
    del kv, codes
    return out


# ---------------------------------------------------------------- generation
def run_generation(wl, dev, steps):
    """One generated token per sequence: every self-decoder layer appends the
    token's K/V to its W-slot ring and attends over the window; the hidden
    state is projected into row ctx-1 of the global cache; every cross layer
    attends over rows 0..ctx-1.  Synthetic queries, new K/V and hidden state
    per layer; full rings."""
    B, ctx, Hq, Hkv, d, W, D = wl.batch, wl.seq, wl.n_heads, wl.n_kv_heads, wl.head_dim, wl.window, wl.hidden
    Ls, Lc, wid = wl.n_self_layers, wl.n_cross_layers, wl.wid
    rings = [(randn((B, Hkv, W, d), seed_for(wid, 10 + 2 * i), device=dev),
              randn((B, Hkv, W, d), seed_for(wid, 11 + 2 * i), device=dev)) for i in range(Ls)]
    kc = randn((B, Hkv, ctx, d), seed_for(wid, 0), device=dev)
    vc = randn((B, Hkv, ctx, d), seed_for(wid, 1), device=dev)
    wk = randn((Hkv * d, D), seed_for(wid, 3), std=wl.weight_std, device=dev)
    wv = randn((Hkv * d, D), seed_for(wid, 4), std=wl.weight_std, device=dev)
    qs_self = randn((Ls, B, Hq, d), seed_for(wid, 5), device=dev)
    kn = randn((Ls, B, Hkv, d), seed_for(wid, 6), device=dev)
    vn = randn((Ls, B, Hkv, d), seed_for(wid, 7), device=dev)
    hid = randn((B, 1, D), seed_for(wid, 8), device=dev)
    qs_cross = randn((Lc, B, Hq, d), seed_for(wid, 2), device=dev)
    o = torch.empty(B, Hq, d, dtype=torch.bfloat16, device=dev)
    ws_self = torch.empty(yk.yoco_swa_decode_workspace_bytes(B, Hq, Hkv, W, d), dtype=torch.uint8, device=dev)
    ws_cross = torch.empty(yk.yoco_cross_attn_decode_workspace_bytes(B, Hq, Hkv, ctx, d), dtype=torch.uint8,
                           device=dev)
    pos = ctx - 1    # the token being generated sits at the last cached position

    parts = {"self_decoder": [], "kv_append": [], "cross_decoder": []}

    def ev_call(key, fn, record):
        if record:
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record()
            fn()
            e.record()
            parts[key].append((s, e))
        else:
            fn()

    def step(record):
        for i in range(Ls):
            ev_call("self_decoder", lambda: yk.yoco_swa_decode(qs_self[i], rings[i][0], rings[i][1], pos,
                                                               k_new=kn[i], v_new=vn[i], o=o, workspace=ws_self),
                    record)
        ev_call("kv_append", lambda: yk.yoco_global_kv_proj(hid, wk, wv, kc, vc, pos0=pos), record)
        for i in range(Lc):
            ev_call("cross_decoder", lambda: yk.yoco_cross_attn_decode(qs_cross[i], kc, vc, ctx, o=o,
                                                                       workspace=ws_cross), record)

    step(False)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(steps):
        step(True)
    t1.record()
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / steps
    part_ms = {k: sum(events_ms(v)) / steps for k, v in parts.items()}
    # the same step replayed from a HIP graph (no host launch gaps between its
    # ~100 short kernels; the append rewrites the same ring slot each replay)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(False)
    graph.replay()
    torch.cuda.synchronize()
    t0.record()
    for _ in range(steps):
        graph.replay()
    t1.record()
    torch.cuda.synchronize()
    ms_graph = t0.elapsed_time(t1) / steps
    del graph
    self_bytes = Ls * (B * Hkv * W * d * 2 * 2 + B * Hq * d * 2 * 2 + B * Hkv * d * 2 * 2)
    proj_bytes = 2 * Hkv * d * D * 2 + B * D * 2 + 2 * B * Hkv * d * 2
    cross_bytes = Lc * decode_bytes(B, Hkv, ctx, d, Hq, 2, 2)
    nbytes = self_bytes + proj_bytes + cross_bytes
    gbs = nbytes / (ms_step * 1e-3) / 1e9
    return {
        "workload": wl.name,
        "steps": steps,
        "ms_per_step": ms_step,
        "tokens_per_s": B / (ms_step * 1e-3),
        "bytes_per_step": nbytes,
        "GB/s": gbs,
        "frac_hbm_peak": gbs / HBM_PEAK_GBS,
        "parts_ms_per_step": part_ms,
        "graph": {"ms_per_step": ms_graph, "tokens_per_s": B / (ms_graph * 1e-3),
                  "GB/s": nbytes / (ms_graph * 1e-3) / 1e9},
        "parts_GB/s": {"self_decoder": self_bytes / (part_ms["self_decoder"] * 1e-3) / 1e9,
                       "kv_append": proj_bytes / (part_ms["kv_append"] * 1e-3) / 1e9,
                       "cross_decoder": cross_bytes / (part_ms["cross_decoder"] * 1e-3) / 1e9},
        "timing": "HIP events around the whole step and around every call; graph: the step captured once "
                  "and replayed",
    }


# ---------------------------------------------------------------- gated retention
def run_gret(wl, dev, reps, decode_batch=16, chunk=256, tau=16.0, n_states=16):
    """Gated-retention self-decoder layer (chunkwise prefill) at the 3B shape,
    and its recurrent decode step.  Gate logits ~ N(3, 1) with tau 16 (decay
    close to 1, the regime the temperature is there to produce).  The calls
    cycle over distinct per-layer tensors (the workload's self-decoder layers
    for the prefill, 800 MB; n_states decode states, 400 MB), so that no
    layer's data is still in the 256 MB last-level cache when it comes round
    again, as in a model step."""
    B, N, H, d, wid = wl.batch, wl.seq, wl.n_heads, wl.head_dim, wl.wid
    L = wl.n_self_layers
    s = d ** -0.25
    layers = []
    for layer in range(L):
        s0 = seed_for(wid, 20 + 4 * layer)
        layers.append((randn((B, H, N, d), s0, std=s, device=dev), randn((B, H, N, d), s0 + 1, std=s, device=dev),
                       randn((B, H, N, d), s0 + 2, device=dev),
                       randn((B, H, N), s0 + 3, dtype="f32", device=dev) + 3.0,
                       torch.empty(B, H, N, d, dtype=torch.bfloat16, device=dev),
                       torch.empty(B, H, d, d, dtype=torch.float32, device=dev)))
    ws = torch.empty(yk.yoco_gret_prefill_workspace_bytes(B, H, N, d, chunk), dtype=torch.uint8, device=dev)
    it = {"p": 0, "d": 0}

    def prefill():
        q, k, v, z, o, st = layers[it["p"] % L]
        it["p"] += 1
        yk.yoco_gret_prefill(q, k, v, z, tau, o=o, state_out=st, chunk=chunk, workspace=ws)

    Bd = decode_batch
    qd = randn((Bd, H, d), seed_for(wid, 4), std=s, device=dev)
    kd = randn((Bd, H, d), seed_for(wid, 5), std=s, device=dev)
    vd = randn((Bd, H, d), seed_for(wid, 6), device=dev)
    zd = randn((Bd, H), seed_for(wid, 7), dtype="f32", device=dev) + 3.0
    states = [randn((Bd, H, d, d), seed_for(wid, 100 + i), std=0.1, dtype="f32", device=dev) for i in range(n_states)]
    od = torch.empty_like(qd)

    def decode():
        sd = states[it["d"] % n_states]
        it["d"] += 1
        yk.yoco_gret_decode(qd, kd, vd, zd, tau, sd, o=od)

    # `reps` calls back to back, captured once in a HIP graph and replayed
    # between two events (as the layers of a model would run): the
    # microsecond-scale decode step is then not paced by the host's per-call
    # launch latency.  The kernels use no memset, so the graph holds kernel
    # nodes only.
    res = {}
    for name, fn in (("prefill", prefill), ("decode", decode)):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(reps):
                fn()
        graph.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        graph.replay()
        b.record()
        torch.cuda.synchronize()
        res[name] = events_ms([(a, b)])[0] / reps
        del graph
    nc = (N + chunk - 1) // chunk
    pairs = sum(min(chunk, N - c * chunk) * (min(chunk, N - c * chunk) + 1) // 2 for c in range(nc))
    flops = B * H * (4.0 * d * pairs + 2 * 2.0 * N * d * d)      # inner QK^T and WV; cross Q R and state K^T V
    pbytes = B * H * N * (4 * d * 2 + 4)                            # q, k, v, o (bf16) and the gate logits
    dbytes = Bd * H * (2 * d * d * 4 + 4 * d * 2 + 4)               # state read + written, q, k, v, o, gate
    pgbs = pbytes / (res["prefill"] * 1e-3) / 1e9
    dgbs = dbytes / (res["decode"] * 1e-3) / 1e9
    return {
        "workload": wl.name,
        "prefill": {"batch": B, "seq_len": N, "heads": H, "head_dim": d, "chunk": chunk,
                    "ms_per_layer": res["prefill"], "TFLOP/s": flops / (res["prefill"] * 1e-3) / 1e12,
                    "GB/s": pgbs,
                    "roofline": {"bound": "hbm", "achieved": pgbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                 "frac": pgbs / HBM_PEAK_GBS,
                                 "traffic": traffic_from_profile(f"gret_prefill_{wl.name}.txt", "gret.hip",
                                                                 "hbm bytes per layer")},
                    "flops_per_layer": flops, "bytes_per_layer": pbytes},
        "decode": {"batch": Bd, "heads": H, "head_dim": d, "ms_per_step": res["decode"], "GB/s": dgbs,
                   "roofline": {"bound": "hbm", "achieved": dgbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                "frac": dgbs / HBM_PEAK_GBS,
                                "traffic": traffic_from_profile(f"gret_decode_{wl.name}.txt", "gret.hip",
                                                                "hbm bytes per step")},
                   "bytes_per_step": dbytes},
        "timing": "HIP events around one replay of a HIP graph of back-to-back calls (prefill: 3 kernels; decode: 1 kernel)",
    }


# ---------------------------------------------------------------- whole block
class BlockForward:
    """The 3B-shaped YOCO block with every step on the GPU: per self-decoder
    layer the pre-norm Q/K/V projection, sliding-window attention, the output
    projection (residual) and the SwiGLU feed-forward (gate/up, then down with
    the residual); the global KV projection; per cross-decoder layer the query
    projection, causal cross attention over the shared cache, the output
    projection and the feed-forward.  Early exit runs the cross-decoder for
    the last position only."""

    def __init__(self, wl, dev):
        self.wl = wl
        B, N, D, Hq, Hkv, d, F = wl.batch, wl.seq, wl.hidden, wl.n_heads, wl.n_kv_heads, wl.head_dim, wl.ffn_dim
        idx = iter(range(300, 1000))
        r = lambda *shape, std=wl.weight_std: randn(shape, seed_for(wl.wid, next(idx)), std=std, device=dev)  # noqa: E731
        ffn = lambda: (r(F, D), r(F, D), r(D, F, std=wl.weight_std * (D / F) ** 0.5))  # noqa: E731
        self.x0 = randn((B, N, D), seed_for(wl.wid, 299), device=dev)
        self.x = torch.empty_like(self.x0)
        self.swa = [(r(Hq * d, D), r(Hkv * d, D), r(Hkv * d, D), r(D, Hq * d), ffn()) for _ in range(wl.n_self_layers)]
        self.glob = (r(Hkv * d, D), r(Hkv * d, D))
        self.cross = [(r(Hq * d, D), r(D, Hq * d), ffn()) for _ in range(wl.n_cross_layers)]
        bf = dict(dtype=torch.bfloat16, device=dev)
        self.q = torch.empty(B, Hq, N, d, **bf)
        self.k = torch.empty(B, Hkv, N, d, **bf)
        self.v = torch.empty(B, Hkv, N, d, **bf)
        self.o = torch.empty(B, Hq, N, d, **bf)
        self.h = torch.empty(B, N, F, **bf)
        self.kc = torch.empty(B, Hkv, N, d, **bf)
        self.vc = torch.empty(B, Hkv, N, d, **bf)
        self.last = torch.empty(B, 1, D, **bf)
        self.q1 = torch.empty(B, Hq, 1, d, **bf)
        self.o1 = torch.empty(B, Hq, d, **bf)
        self.h1 = torch.empty(B, 1, F, **bf)
        self.ws = torch.empty(yk.yoco_cross_attn_decode_workspace_bytes(B, Hq, Hkv, N, d), dtype=torch.uint8,
                              device=dev)
        g = lambda m, n_, k: 2.0 * m * n_ * k  # noqa: E731
        M = B * N
        self.flops = {
            "qkv_proj": wl.n_self_layers * g(M, (Hq + 2 * Hkv) * d, D) + wl.n_cross_layers * g(M, Hq * d, D),
            "swa_attn": wl.n_self_layers * attn_flops(swa_pairs(N, wl.window), Hq, d, B),
            "kv_proj": proj_flops(B, N, D, Hkv * d),
            "cross_attn": wl.n_cross_layers * attn_flops(causal_pairs(N), Hq, d, B),
            "out_proj": (wl.n_self_layers + wl.n_cross_layers) * g(M, D, Hq * d),
            "swiglu": (wl.n_self_layers + wl.n_cross_layers) * g(M, 2 * F, D),
            "down_proj": (wl.n_self_layers + wl.n_cross_layers) * g(M, D, F),
        }
        L_c = wl.n_cross_layers
        self.flops_early_exit = (sum(v for k_, v in self.flops.items() if k_ != "cross_attn")
                                 - L_c * (g(M - B, Hq * d, D) + g(M - B, D, Hq * d) + g(M - B, 2 * F, D)
                                          + g(M - B, D, F))
                                 + L_c * attn_flops(N, Hq, d, B))

    def _t(self, ev, key, fn):
        if ev is None:
            fn()
            return
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        fn()
        e.record()
        ev.setdefault(key, []).append((s, e))

    def run(self, early_exit=False, ev=None):
        wl = self.wl
        B, N, Hq, d = wl.batch, wl.seq, wl.n_heads, wl.head_dim
        x = self.x
        x.copy_(self.x0)
        t = self._t
        for wq, wk, wv, wo, (wg, wu, wd) in self.swa:
            t(ev, "qkv_proj", lambda: yk.yoco_qkv_proj(x, wq, d, wk, wv, q_out=self.q, k_out=self.k, v_out=self.v))
            t(ev, "swa_attn", lambda: yk.yoco_swa_attn(self.q, self.k, self.v, wl.window, o=self.o))
            t(ev, "out_proj", lambda: yk.yoco_linear_residual(self.o, wo, x, a_heads=Hq))
            t(ev, "swiglu", lambda: yk.yoco_swiglu(x, wg, wu, h=self.h))
            t(ev, "down_proj", lambda: yk.yoco_linear_residual(self.h, wd, x))
        t(ev, "kv_proj", lambda: yk.yoco_global_kv_proj(x, self.glob[0], self.glob[1], self.kc, self.vc))
        if early_exit:
            last = self.last
            last.copy_(x[:, N - 1:N])
            for wq, wo, (wg, wu, wd) in self.cross:
                yk.yoco_qkv_proj(last, wq, d, q_out=self.q1)
                yk.yoco_cross_attn_decode(self.q1.view(B, Hq, d), self.kc, self.vc, N, o=self.o1, workspace=self.ws)
                yk.yoco_linear_residual(self.o1.view(B, Hq, 1, d), wo, last, a_heads=Hq)
                yk.yoco_swiglu(last, wg, wu, h=self.h1)
                yk.yoco_linear_residual(self.h1, wd, last)
            return
        for wq, wo, (wg, wu, wd) in self.cross:
            t(ev, "qkv_proj", lambda: yk.yoco_qkv_proj(x, wq, d, q_out=self.q))
            t(ev, "cross_attn", lambda: yk.yoco_cross_attn_prefill(self.q, self.kc, self.vc, o=self.o))
            t(ev, "out_proj", lambda: yk.yoco_linear_residual(self.o, wo, x, a_heads=Hq))
            t(ev, "swiglu", lambda: yk.yoco_swiglu(x, wg, wu, h=self.h))
            t(ev, "down_proj", lambda: yk.yoco_linear_residual(self.h, wd, x))


def run_block(wl, dev, steps):
    blk = BlockForward(wl, dev)
    res = {}
    for mode in ("full", "early_exit"):
        for _ in range(2):
            blk.run(early_exit=mode == "early_exit")
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(steps):
            blk.run(early_exit=mode == "early_exit")
        b.record()
        torch.cuda.synchronize()
        res[mode] = events_ms([(a, b)])[0] / steps
    ev = {}
    blk.run(ev=ev)
    torch.cuda.synchronize()
    parts = {}
    for key, pairs in ev.items():
        ms = sum(events_ms(pairs))
        tf = blk.flops[key] / (ms * 1e-3) / 1e12
        parts[key] = {"ms": ms, "calls": len(pairs), "TFLOP/s": tf, "frac_mfma_peak": tf / BF16_PEAK_TFLOPS}
    total = sum(blk.flops.values())
    tokens = wl.batch * wl.seq
    out = {
        "workload": wl.name,
        "config": {"batch": wl.batch, "seq_len": wl.seq, "hidden": wl.hidden, "q_heads": wl.n_heads,
                   "kv_heads": wl.n_kv_heads, "head_dim": wl.head_dim, "ffn_dim": wl.ffn_dim,
                   "self_layers": wl.n_self_layers, "cross_layers": wl.n_cross_layers, "window": wl.window},
        "ms_per_forward": res["full"],
        "tokens_per_s": tokens / (res["full"] * 1e-3),
        "TFLOP/s": total / (res["full"] * 1e-3) / 1e12,
        "flops_per_forward": total,
        "parts": parts,
        "early_exit": {"ms_per_prefill": res["early_exit"], "tokens_per_s": tokens / (res["early_exit"] * 1e-3),
                       "TFLOP/s": blk.flops_early_exit / (res["early_exit"] * 1e-3) / 1e12,
                       "speedup_vs_full": res["full"] / res["early_exit"]},
        "timing": ("HIP events around back-to-back forwards (the input copy included); parts: events around "
                   "each call of one forward"),
    }
    del blk
    return out


# ---------------------------------------------------------------- one device's share
def run_shard(wl, dev, parts=8, reps=3):
    """One device's share of the 1M-token early-exit flow split over `parts`
    devices by sequence chunks: each self-decoder layer over the device's
    2^20 / parts rows plus a 1024-row halo of the previous chunk, the global
    projection of its rows, and per cross-decoder layer the last token's
    decode over its cache shard plus the merge of the `parts` shard results
    (the halo and the partials would arrive over xGMI; that exchange is not
    timed here)."""
    B, N, D, Hq, Hkv, d, W = wl.batch, wl.seq, wl.hidden, wl.n_heads, wl.n_kv_heads, wl.head_dim, wl.window
    C = N // parts
    wid = wl.wid
    q = randn((B, Hq, C, d), seed_for(wid, 500), device=dev)
    k = randn((B, Hkv, C + W, d), seed_for(wid, 501), device=dev)
    v = randn((B, Hkv, C + W, d), seed_for(wid, 502), device=dev)
    o = torch.empty_like(q)
    x = randn((B, C, D), seed_for(wid, 503), device=dev)
    wk = randn((Hkv * d, D), seed_for(wid, 504), std=wl.weight_std, device=dev)
    wv = randn((Hkv * d, D), seed_for(wid, 505), std=wl.weight_std, device=dev)
    kc = torch.empty(B, Hkv, C, d, dtype=torch.bfloat16, device=dev)
    vc = torch.empty_like(kc)
    qd = randn((B, Hq, d), seed_for(wid, 506), device=dev)
    od = torch.empty_like(qd)
    lse = torch.empty(B, Hq, dtype=torch.float32, device=dev)
    ws = torch.empty(yk.yoco_cross_attn_decode_workspace_bytes(B, Hq, Hkv, C, d), dtype=torch.uint8, device=dev)
    o_parts = randn((parts, B, Hq, d), seed_for(wid, 507), device=dev)
    lse_parts = randn((parts, B, Hq), seed_for(wid, 508), dtype="f32", device=dev)
    om = torch.empty_like(qd)

    def timed(fn):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return events_ms([(a, b)])[0] / reps

    swa_ms = timed(lambda: yk.yoco_swa_attn_halo(q, k, v, W, o=o))
    proj_ms = timed(lambda: yk.yoco_global_kv_proj(x, wk, wv, kc, vc))
    dec_ms = timed(lambda: yk.yoco_cross_attn_decode(qd, kc, vc, C, o=od, lse=lse, workspace=ws))
    merge_ms = timed(lambda: yk.yoco_attn_merge(o_parts, lse_parts, o=om))
    f_swa = attn_flops(C * W, Hq, d, B)                 # every shard row sees a full window
    f_proj = proj_flops(B, C, D, Hkv * d)
    dbytes = decode_bytes(B, Hkv, C, d, Hq, 2, 2)
    step = wl.n_self_layers * swa_ms + proj_ms + wl.n_cross_layers * (dec_ms + merge_ms)
    return {
        "workload": wl.name, "devices": parts, "rows_per_device": C, "halo_rows": W,
        "swa_layer": {"ms": swa_ms, "TFLOP/s": f_swa / (swa_ms * 1e-3) / 1e12,
                      "frac_mfma_peak": f_swa / (swa_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS},
        "kv_proj": {"ms": proj_ms, "TFLOP/s": f_proj / (proj_ms * 1e-3) / 1e12},
        "decode_shard": {"ms": dec_ms, "GB/s": dbytes / (dec_ms * 1e-3) / 1e9,
                         "frac_hbm_peak": dbytes / (dec_ms * 1e-3) / 1e9 / HBM_PEAK_GBS},
        "merge_ms": merge_ms,
        "device_ms_per_step": step,
        "timing": "HIP events around back-to-back calls of each part; the exchanges between devices are not timed",
    }


# ---------------------------------------------------------------- early exit
def run_early_exit(wl, dev, steps, sample=None):
    """1M-token early-exit prefill: L_s SWA layers over all tokens, the global
    KV projection of all tokens, then the cross-decoder for the last position
    only (one decode call per cross layer over the full cache).  With
    `sample` (a dict), copies to the host what the oracle timing needs:
    sampled query rows of one window layer with their windows, sampled
    projection rows with the weights, one KV head of the full cache and its
    last-position queries."""
    B, N, D, Hq, Hkv, d, W = wl.batch, wl.seq, wl.hidden, wl.n_heads, wl.n_kv_heads, wl.head_dim, wl.window
    wid = wl.wid
    layers = []
    for layer in range(wl.n_self_layers):
        s0 = seed_for(wid, 10 + 3 * layer)
        layers.append((randn((B, Hq, N, d), s0, device=dev), randn((B, Hkv, N, d), s0 + 1, device=dev),
                       randn((B, Hkv, N, d), s0 + 2, device=dev)))
    o = torch.empty(B, Hq, N, d, dtype=torch.bfloat16, device=dev)
    x = randn((B, N, D), seed_for(wid, 0), device=dev)
    wk = randn((Hkv * d, D), seed_for(wid, 1), std=wl.weight_std, device=dev)
    wv = randn((Hkv * d, D), seed_for(wid, 2), std=wl.weight_std, device=dev)
    kc = torch.empty(B, Hkv, N, d, dtype=torch.bfloat16, device=dev)
    vc = torch.empty_like(kc)
    ql = randn((wl.n_cross_layers, B, Hq, d), seed_for(wid, 300), device=dev)
    od = torch.empty(B, Hq, d, dtype=torch.bfloat16, device=dev)
    ws = torch.empty(yk.yoco_cross_attn_decode_workspace_bytes(B, Hq, Hkv, N, d), dtype=torch.uint8, device=dev)
    ev = {"swa": [], "proj": [], "decode": []}

    def timed(key, fn):
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        fn()
        e.record()
        ev[key].append((s, e))

    def step(record):
        for q, k, v in layers:
            f = lambda: yk.yoco_swa_attn(q, k, v, W, o=o)  # noqa: E731
            timed("swa", f) if record else f()
        f = lambda: yk.yoco_global_kv_proj(x, wk, wv, kc, vc)  # noqa: E731
        timed("proj", f) if record else f()
        for layer in range(wl.n_cross_layers):
            f = lambda: yk.yoco_cross_attn_decode(ql[layer], kc, vc, N, o=od, workspace=ws)  # noqa: E731
            timed("decode", f) if record else f()

    step(False)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(steps):
        step(True)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    if sample is not None:
        # window rows: the first rows (partial windows), both sides of the
        # first full window, and spread over the sequence
        rows = sorted({0, 1, W - 2, W - 1, W, W + 1, N // 2, N - 1} | {(N // 8) * i + 333 for i in range(8)})
        q0, k0, v0 = layers[0]
        g = Hq // Hkv
        sample.update(workload=wl.name, N=N, W=W, Ls=wl.n_self_layers, Lc=wl.n_cross_layers, Hkv=Hkv, g=g, d=d,
                      rows=rows,
                      swa=[(q0[:, :, t:t + 1].float().cpu().numpy(),
                            k0[:, :, max(0, t - W + 1):t + 1].float().cpu().numpy(),
                            v0[:, :, max(0, t - W + 1):t + 1].float().cpu().numpy()) for t in rows],
                      x=x[:, rows].float().cpu().numpy(), wk=wk.float().cpu().numpy(), wv=wv.float().cpu().numpy(),
                      dec_q=ql[0][:, 0:g].float().cpu().numpy(), dec_k=kc[:, 0:1].float().cpu().numpy(),
                      dec_v=vc[:, 0:1].float().cpu().numpy())
    swa_ms = sum(events_ms(ev["swa"])) / len(ev["swa"])
    proj_ms = sum(events_ms(ev["proj"])) / len(ev["proj"])
    dec_ms = sum(events_ms(ev["decode"])) / len(ev["decode"])
    f_swa = attn_flops(swa_pairs(N, W), Hq, d, B)
    f_proj = proj_flops(B, N, D, Hkv * d)
    dbytes = decode_bytes(B, Hkv, N, d, Hq, 2, 2)
    flops = wl.n_self_layers * f_swa + f_proj + wl.n_cross_layers * attn_flops(N, Hq, d, B)
    full_cross = wl.n_cross_layers * attn_flops(causal_pairs(N), Hq, d, B)
    return {
        "workload": wl.name,
        "ms_per_step": ms,
        "steps": steps,
        "TFLOP/s": flops / (ms * 1e-3) / 1e12,
        "swa": {"ms": swa_ms, "TFLOP/s": f_swa / (swa_ms * 1e-3) / 1e12,
                "frac_mfma_peak": f_swa / (swa_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS},
        "kv_proj": {"ms": proj_ms, "TFLOP/s": f_proj / (proj_ms * 1e-3) / 1e12,
                    "frac_mfma_peak": f_proj / (proj_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS},
        "last_token_decode": {"ms": dec_ms, "GB/s": dbytes / (dec_ms * 1e-3) / 1e9,
                              "frac_hbm_peak": dbytes / (dec_ms * 1e-3) / 1e9 / HBM_PEAK_GBS},
        "cross_decoder_flops_skipped_by_early_exit": full_cross,
        "timing": "HIP events around every call of each step",
    }


# ---------------------------------------------------------------- achievable peaks
def run_peaks(dev, reps=5):
    """What this chip reaches at its clock under load: a streaming read of a
    4 GiB buffer and a register-resident bf16 matrix-core loop."""
    buf = torch.zeros(1 << 30, dtype=torch.int32, device=dev)
    part = torch.empty(2048, dtype=torch.int32, device=dev)
    mout = torch.empty(4 * 1024, dtype=torch.float32, device=dev)
    iters = 20000
    res = {}
    for name, fn in (("read", lambda: yk.yoco_peak_hbm_read(buf, blocks=2048, partial=part)),
                     ("mfma", lambda: yk.yoco_peak_mfma_bf16(iters, blocks=1024, out=mout)),
                     ("mfma_toggling", lambda: yk.yoco_peak_mfma_bf16_toggling(iters, blocks=1024, out=mout))):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        res[name] = events_ms([(a, b)])[0] / reps
    read_gbs = buf.numel() * 4 / (res["read"] * 1e-3) / 1e9
    mfma_tf = 1024 * 4 * iters * 8 * 32768 / (res["mfma"] * 1e-3) / 1e12
    mfma_tog_tf = 1024 * 4 * iters * 8 * 32768 / (res["mfma_toggling"] * 1e-3) / 1e12
    del buf
    return {"hbm_read_GB/s": read_gbs, "frac_of_spec_hbm": read_gbs / HBM_PEAK_GBS,
            "mfma_bf16_TFLOP/s": mfma_tf, "frac_of_spec_mfma": mfma_tf / BF16_PEAK_TFLOPS,
            "mfma_bf16_toggling_TFLOP/s": mfma_tog_tf,
            "what": "libyoco peak microbenchmarks: one streaming read of 4 GiB; 1024 workgroups x 4 waves x "
                    "20000 rounds of 8 independent 32x32x16 bf16 MFMAs from registers, on operands of ones "
                    "and on operands that change every instruction (the matrix core then draws more power "
                    "and the clock drops, as with real data)"}


# ---------------------------------------------------------------- main
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--decode-steps", type=int, default=128,
                    help="decode steps (x16 cross layers) of the 32K-context decode measurement")
    ap.add_argument("--cpu-budget", type=float, default=12.0,
                    help="seconds of oracle CPU work on the prefill sample (as much again on the other configs)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--calibrate-copy-mb", type=int, default=0,
                    help="run one elementwise bf16 copy (x * 1) of this many MiB, read and written once, "
                         "as the known-size reference for HBM byte counters")
    ap.add_argument("--no-fp8-decode", action="store_true",
                    help="skip the 512K fp8-cache decode measurement (allocates ~26 GB)")
    ap.add_argument("--no-early-exit", action="store_true",
                    help="skip the 1M-token early-exit flow measurement (allocates ~110 GB)")
    ap.add_argument("--extra-steps", type=int, default=3, help="steps of the 1M early-exit flow")
    ap.add_argument("--no-generation", action="store_true", help="skip the one-token generation step measurement")
    ap.add_argument("--no-gret", action="store_true", help="skip the gated-retention measurement")
    ap.add_argument("--gret-reps", type=int, default=50, help="calls per timed HIP graph of the gated-retention layer")
    ap.add_argument("--no-block", action="store_true",
                    help="skip the whole-block measurement (3B shape with all layer glue on the GPU)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for {args.gpus} GPUs, WORLD_SIZE={world}); "
              "the library has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = "cuda:0"
    torch.cuda.set_device(0)
    yk.lib()

    if args.calibrate_copy_mb:
        n = args.calibrate_copy_mb * (1 << 20) // 2
        src = torch.ones(n, dtype=torch.bfloat16, device=dev)
        dst = torch.mul(src, 1)
        torch.cuda.synchronize()
        del src, dst

    wl = WORKLOADS["prefill_3b_bf16"]
    step = PrefillStep(wl, dev)
    for _ in range(args.warmup):
        step.run()
    torch.cuda.synchronize()

    ev = []
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for _ in range(args.steps):
        step.run(ev)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    tflops = step.flops / (ms * 1e-3) / 1e12

    attn_ms = sum(events_ms(ev)) / (len(ev) * wl.n_cross_layers)
    attn_tflops = step.flops_cross / (attn_ms * 1e-3) / 1e12
    roofline = {
        "bound": "mfma",
        "kernel": "attn_fwd_kernel<bf16,128,causal> (yoco_cross_attn_prefill)",
        "achieved": attn_tflops,
        "peak": BF16_PEAK_TFLOPS,
        "unit": "TFLOP/s",
        "frac": attn_tflops / BF16_PEAK_TFLOPS,
        "traffic": traffic_from_profile("attn_fwd_prefill_3b_bf16.txt", "attn_fwd.hip", "hbm bytes per launch"),
        "flops_per_launch": step.flops_cross,
        "ms_per_launch": attn_ms,
        "timing": "HIP events around the back-to-back cross-layer launches of every timed step; per launch = span / layers",
    }

    # the same step captured once as a HIP graph and replayed (no host launch
    # gaps between its 17 kernels); the headline value stays the stream-launched step
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step.run()
    for _ in range(2):
        g.replay()
    torch.cuda.synchronize()
    g0 = torch.cuda.Event(enable_timing=True)
    g1 = torch.cuda.Event(enable_timing=True)
    g0.record()
    for _ in range(args.steps):
        g.replay()
    g1.record()
    torch.cuda.synchronize()
    ms_graph = g0.elapsed_time(g1) / args.steps
    del g

    peaks = run_peaks(dev)
    roofline["measured_peak"] = peaks["mfma_bf16_TFLOP/s"]
    roofline["frac_of_measured_peak"] = attn_tflops / peaks["mfma_bf16_TFLOP/s"]
    roofline["measured_peak_toggling"] = peaks["mfma_bf16_toggling_TFLOP/s"]
    roofline["frac_of_measured_peak_toggling"] = attn_tflops / peaks["mfma_bf16_toggling_TFLOP/s"]

    out = {
        "metric": METRIC,
        "value": tflops,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) activations/queries/keys/values, N(0,0.02) weights)",
        "config": {
            "workload": wl.name, "batch": wl.batch, "seq_len": wl.seq, "hidden": wl.hidden,
            "q_heads": wl.n_heads, "kv_heads": wl.n_kv_heads, "head_dim": wl.head_dim,
            "self_layers": wl.n_self_layers, "window": wl.window, "cross_layers": wl.n_cross_layers,
            "step": "8x sliding-window attention + 1x global KV projection + 8x causal cross prefill",
            "flops_per_step": step.flops,
        },
        "frac_mfma_peak": tflops / BF16_PEAK_TFLOPS,
        "graph": {"ms_per_step": ms_graph, "TFLOP/s": step.flops / (ms_graph * 1e-3) / 1e12,
                  "timing": "the step captured once as a HIP graph; events around back-to-back replays"},
        "roofline": roofline,
        "measured_peaks": peaks,
    }
    del step
    torch.cuda.empty_cache()

    smp_dec, smp_fp8, smp_ee = {}, {}, {}
    want_cpu = not args.no_cpu_baseline
    if not args.no_decode:
        out["decode"] = run_decode(WORKLOADS["decode_32k_bf16"], dev, args.decode_steps,
                                   sample=smp_dec if want_cpu else None)
        out["decode"]["roofline"]["measured_peak"] = peaks["hbm_read_GB/s"]
        out["decode"]["roofline"]["frac_of_measured_peak"] = out["decode"]["GB/s"] / peaks["hbm_read_GB/s"]
        torch.cuda.empty_cache()
    if not args.no_fp8_decode:
        out["quantize_fp8"] = run_quantize(WORKLOADS["decode_32k_bf16"], dev)
        out["decode_fp8"] = run_decode(WORKLOADS["decode_512k_fp8"], dev, WORKLOADS["decode_512k_fp8"].decode_steps,
                                       sample=smp_fp8 if want_cpu else None, n_groups=1)
        torch.cuda.empty_cache()
    if not args.no_generation:
        wg = WORKLOADS["generation_32k_bf16"]
        out["generation"] = run_generation(wg, dev, wg.decode_steps)
        torch.cuda.empty_cache()
    if not args.no_block:
        out["block_prefill"] = run_block(wl, dev, 3)
        torch.cuda.empty_cache()
    if not args.no_gret:
        out["gated_retention"] = run_gret(WORKLOADS["gret_3b_bf16"], dev, args.gret_reps)
        torch.cuda.empty_cache()
    if not args.no_early_exit:
        out["early_exit_1m"] = run_early_exit(WORKLOADS["early_exit_1m_bf16"], dev, args.extra_steps,
                                              sample=smp_ee if want_cpu else None)
        torch.cuda.empty_cache()
        out["early_exit_1m_one_of_8_devices"] = run_shard(WORKLOADS["early_exit_1m_bf16"], dev)
        torch.cuda.empty_cache()

    if want_cpu:
        step = PrefillStep(wl, dev)
        out["cpu_baseline"] = cpu_baseline_prefill(step, args.cpu_budget)
        del step
        # the same oracle beside the other measured configurations (sampled,
        # extrapolated), each on its own slice of the CPU budget
        per = {}
        budget = args.cpu_budget / 3
        if smp_dec:
            per["decode_32k_bf16"] = cpu_baseline_decode(smp_dec, budget)
        if smp_fp8:
            per["decode_512k_fp8"] = cpu_baseline_decode(smp_fp8, budget)
        if smp_ee:
            per["early_exit_1m_bf16"] = cpu_baseline_early_exit(smp_ee, budget)
        out["cpu_baseline"]["per_config"] = per
    else:
        out["cpu_baseline"] = None

    print(json.dumps(out))


if __name__ == "__main__":
    main()
