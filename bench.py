#!/usr/bin/env python3
"""Benchmark of the causal attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 4]
                    [--no-also] [--no-cpu] [--cpu-seconds S] [--no-graph]
                    [--calib-copy | --calib-mfma | --calib-hbm]

A step is one pass of the hot path over one batch of the workload's seeded
synthetic inputs, resident in HBM before timing starts:
    prefill with RoPE (workloads 3, 4): one attn_fwd_rope call -- the RoPE
    pass rotates k in place and writes the angle table, then the fused causal
    attention rotates each query row as it loads it;
    prefill without RoPE (workloads 1, 2): the fused causal attention;
    decode (workload 5): RoPE on the new query row, then the split-K decode.
For the RoPE prefills the same step as two calls (rope_apply on q and k,
then attention) is timed beside it ("ms_per_step_rope_then_attn").

The headline workload (default 4: bf16 GQA + RoPE prefill B1 Hq32 Hkv8
T16384 d128, the largest configuration; it fits one GPU) is timed for K
steps after W warm-up steps (at least 10): an event is recorded on the
stream the kernels run on before the first step and after every step, so
the line carries the mean step time (total / K, "ms_per_step", from which
"value" is computed) and the median of the K step times
("ms_per_step_median").  The K steps are launched back to back through the
C ABI with their arguments checked and marshalled once (Bound calls), so
short kernels are not timed against Python's argument checks.  For
comparison the same steps are also timed as replays of a HIP graph holding
10 steps (unless --no-graph), after checking that a one-step graph replayed
three times (inputs restored, outputs poisoned in between) reproduces the
eager step bit for bit.  The other workloads are timed the same way with
at least 10 warm-up steps (about 30 ms) and at least 50 timed steps (about
50 ms) each.

FLOPs (causal-adjusted): 4 * B * Hq * d * N_vis, N_vis = sum_i min(Tk,
q_offset + i + 1), i.e. two matrix products over the visible (query, key)
pairs only ("Transformer" (ai-notes) -- Discussion (Compute)).  Algorithmic
bytes of attention: elt * d * (2 B Hq Tq + 2 B Hkv Tk) (q and o once, k and
v once per K/V head).  RoPE bytes: read + write of q and k.

Roofline of every workload: its arithmetic intensity (FLOPs / algorithmic
bytes) against the ridge of the published peaks (2516.6 TFLOP/s dense bf16
/ 8000 GB/s = 314.6 FLOP/B) decides the bound -- "mfma" at or above the
ridge, "hbm" below; "frac" is the fraction of that bound's peak, and the
fractions of both peaks are reported beside it.  Measured ceilings (a
matrix-core loop and a streaming read, librocattn_calib.so) are reported in
"measured_peaks" next to the published ones.

Also printed in the same line (unless --no-also): the other workloads'
rates, each timed the same way, so every part of the path has a live
number; and a CPU baseline: the fp64 oracle timed on the host cores on a
bounded sample of the headline workload.  The attention gradients
(attn_bwd) are timed on the shapes of workloads 2 and 3 ("backward"), and
attention with values of their own width (attn_fwd_dv) on workload 3's
shape ("value_width").

--calib-copy runs only a plain device copy of a known size (used to scale
the HBM byte counters of a profiler run); --calib-mfma and --calib-hbm run
only the matrix-core loop or the streaming read and print their rates.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6      # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3        # MI355X fp32 vector
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
KERNEL_SOURCES = {
    "prefill_bf16_d128": "transformer_causal_self_amd/csrc/attn_prefill_bf16.hip",
    "prefill_bf16_d64": "transformer_causal_self_amd/csrc/attn_prefill_bf16.hip",
    "decode_bf16": "transformer_causal_self_amd/csrc/attn_decode_bf16.hip",
    "rope": "transformer_causal_self_amd/csrc/rope.hip",
    "attn_f32": "transformer_causal_self_amd/csrc/attn_f32.hip",
    # one attn_fwd_rope call: the RoPE pass on k, then the prefill kernel
    # that rotates q as it loads it
    "attn_fwd_rope_bf16_d128": ("transformer_causal_self_amd/csrc/rope.hip",
                                "transformer_causal_self_amd/csrc/attn_prefill_bf16.hip"),
}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")


def n_visible(Tq, Tk, causal, q_offset):
    if not causal:
        return Tq * Tk
    return sum(min(Tk, q_offset + i + 1) for i in range(Tq))


def attn_flops(w):
    return 4.0 * w.B * w.Hq * w.d * n_visible(w.Tq, w.Tk, w.causal, w.q_offset)


def elt_bytes(w):
    return 4 if w.dtype == "f32" else 2


def attn_bytes(w):
    return elt_bytes(w) * w.d * (2.0 * w.B * w.Hq * w.Tq + 2.0 * w.B * w.Hkv * w.Tk)


def rope_bytes(w, decode):
    e = elt_bytes(w)
    if decode:  # only the new query rows are rotated during the step
        return 2.0 * e * w.d * w.B * w.Hq * w.Tq
    return 2.0 * e * w.d * w.Tq * w.B * (w.Hq + w.Hkv)


def source_hash(kernel):
    src = KERNEL_SOURCES[kernel]
    h = hashlib.sha256()
    for path in ((src,) if isinstance(src, str) else src):
        with open(os.path.join(ROOT, path), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel, workload_name):
    """HBM bytes per launch from the committed profiler counters, if they
    were taken on the current kernel source; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)[f"{kernel}:{workload_name}"]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("source_sha256_16") != source_hash(kernel):
        return None
    return rec.get("bytes_per_launch")


class Timer:
    """HIP events around n runs of fn() on the current stream (the stream
    the bindings launch on): direct launches, or (graph=True) replays of a
    HIP graph holding REPS runs.  Returns the mean time per run in ms; for
    direct launches, last_times holds each run's own time (an event is
    recorded before the first run and after every run)."""

    REPS = 10
    MIN_WARMUP = 10

    def __init__(self, torch, graph=False):
        self.torch = torch
        self.eager = not graph
        self.last_times = []

    def __call__(self, fn, n, warmup):
        torch = self.torch
        for _ in range(max(warmup, self.MIN_WARMUP)):
            fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        if self.eager:
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
            ev[0].record()
            for i in range(n):
                fn()
                ev[i + 1].record()
            torch.cuda.synchronize()
            self.last_times = [ev[i].elapsed_time(ev[i + 1]) for i in range(n)]
            return ev[0].elapsed_time(ev[n]) / n  # ms
        reps = min(self.REPS, n)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(reps):
                fn()
        g.replay()
        torch.cuda.synchronize()
        n_replay = max(1, n // reps)
        e0.record()
        for _ in range(n_replay):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        del g
        return e0.elapsed_time(e1) / (n_replay * reps)  # ms

    def median(self):
        t = sorted(self.last_times)
        return t[len(t) // 2] if len(t) % 2 else 0.5 * (t[len(t) // 2 - 1] + t[len(t) // 2])


RIDGE = PEAK_BF16_TFLOPS / PEAK_HBM_GBS * 1e3   # FLOP per byte where the two roofs meet


def roofline(flops, nbytes, ms, dtype, ms_median=None):
    """Bound from the arithmetic intensity against the ridge of the published
    peaks, the fraction of that bound's peak, and both fractions."""
    tf = flops / (ms * 1e-3) / 1e12
    gbs = nbytes / (ms * 1e-3) / 1e9
    intensity = flops / nbytes
    if dtype == "f32":
        bound, achieved, peak, unit = "alu", tf, PEAK_F32_TFLOPS, "TFLOP/s"
    elif intensity >= RIDGE:
        bound, achieved, peak, unit = "mfma", tf, PEAK_BF16_TFLOPS, "TFLOP/s"
    else:
        bound, achieved, peak, unit = "hbm", gbs, PEAK_HBM_GBS, "GB/s"
    r = {"bound": bound, "achieved": achieved, "peak": peak, "unit": unit, "frac": achieved / peak,
         "intensity_flop_per_byte": intensity, "ridge_flop_per_byte": RIDGE,
         "tflops": tf, "gbs": gbs}
    if dtype != "f32":
        r["frac_of_mfma_peak"] = tf / PEAK_BF16_TFLOPS
        r["frac_of_hbm_peak"] = gbs / PEAK_HBM_GBS
    if ms_median is not None:
        r["achieved_median"] = achieved * ms / ms_median
        r["frac_median"] = r["achieved_median"] / peak
    return r


def check_graph_replay(torch, fn, outputs, inputs, replays=3):
    """A graph of one fn() replayed several times, with eager work and
    synchronisation between replays, gives the eager result bit for bit
    (inputs that fn changes in place are restored before each run)."""
    saved = [x.clone() for x in inputs]

    def restore():
        for x, y in zip(inputs, saved):
            x.copy_(y)

    restore()
    fn()
    torch.cuda.synchronize()
    want = [x.clone() for x in outputs]
    g = torch.cuda.CUDAGraph()
    restore()
    with torch.cuda.graph(g):
        fn()
    ok = True
    pure_outputs = [x for x in outputs if not any(x is y for y in inputs)]
    for _ in range(replays):
        restore()
        for x in pure_outputs:
            x.fill_(float("nan") if x.is_floating_point() else 0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ok = ok and all(torch.equal(x, y) for x, y in zip(outputs, want))
    restore()
    torch.cuda.synchronize()
    del g
    return ok


def setup(w, torch, ra, wl, dev):
    """Device inputs and the step callables of workload w."""
    q, k, v = wl.inputs(w)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    del q, k, v
    od = torch.empty_like(qd)
    decode = w.Tq == 1 and w.dtype == "bf16"
    ws_b = ra.attn_workspace_bytes(w.B, w.Hq, w.Hkv, w.Tq, w.Tk, w.d, w.torch_dtype)
    ws = torch.empty(ws_b, dtype=torch.uint8, device=dev) if ws_b else None
    if w.rope and decode:
        ra.rope_apply(kd, None, pos0=0, base=w.rope_base)  # the cache arrives rotated
        torch.cuda.synchronize()

    def attn():
        ra.attn_fwd_ws(qd, kd, vd, od, ws, None, scale=w.scale, causal=w.causal,
                       q_offset=w.q_offset)

    attn_b = ra.bind_attn_fwd_ws(qd, kd, vd, od, ws, None, scale=w.scale, causal=w.causal,
                                 q_offset=w.q_offset)
    if w.rope and decode:
        def rope():
            ra.rope_apply(qd, None, pos0=w.q_offset, base=w.rope_base)
        rope_b = ra.bind_rope_apply(qd, None, pos0=w.q_offset, base=w.rope_base)
    elif w.rope:
        def rope():
            ra.rope_apply(qd, kd, pos0=0, base=w.rope_base)
        rope_b = ra.bind_rope_apply(qd, kd, pos0=0, base=w.rope_base)
    else:
        rope = rope_b = None

    def step_sep():
        if rope is not None:
            rope()
        attn()

    if rope_b is not None:
        def step_sep_b():
            rope_b()
            attn_b()
    else:
        step_sep_b = attn_b

    step, step_b, sep_b = step_sep, step_sep_b, None
    if w.rope and not decode:   # RoPE fused into the attention call
        tab = torch.empty(ra.attn_fwd_rope_workspace_bytes(w.Tk, w.d), dtype=torch.uint8,
                          device=dev)

        def step():
            ra.attn_fwd_rope(qd, kd, vd, od, scale=w.scale, causal=w.causal, q_offset=w.q_offset,
                             base=w.rope_base, workspace=tab)

        step_b = ra.bind_attn_fwd_rope(qd, kd, vd, od, tab, scale=w.scale, causal=w.causal,
                                       q_offset=w.q_offset, base=w.rope_base)
        sep_b = step_sep_b

    return dict(step=step, attn=attn, rope=rope, step_b=step_b, attn_b=attn_b, rope_b=rope_b,
                sep_b=sep_b, decode=decode, q=qd, k=kd, v=vd, o=od)


def single_launch_ms(torch, dev, fn, cold, n=21, scratch_bytes=512 << 20):
    """Median time of single synchronised launches of fn; with cold=True
    each follows a 512 MiB device write that evicts the inputs from L2 and
    the 256 MB MALL."""
    scratch = torch.empty(scratch_bytes, dtype=torch.uint8, device=dev)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    times = []
    fn()
    for i in range(n):
        if cold:
            scratch.fill_(i & 0xFF)
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    del scratch
    times.sort()
    return times[len(times) // 2]


def measure(w, args, torch, ra, wl, dev, steps=None, warmup=None, cold=False):
    """Times of one workload's step, attention and RoPE launches.  Without
    explicit counts: about 30 ms (at least 10 steps) of warm-up and 50 ms (at
    least 50 steps) of timed steps.  With cold=True also the attention launch
    after a cache-evicting write."""
    s = setup(w, torch, ra, wl, dev)
    timer = Timer(torch)
    if steps is None or warmup is None:
        t_est = timer(s["step_b"], 3, 1) * 1e-3
        warmup = max(10, int(0.03 / t_est))
        steps = max(50, int(0.05 / t_est))
    ms_step = timer(s["step_b"], steps, warmup)
    ms_step_median = timer.median()
    ms_attn = timer(s["attn_b"], steps, warmup)
    ms_attn_median = timer.median()
    out = dict(workload=w.name, steps=steps, warmup=max(warmup, Timer.MIN_WARMUP),
               ms_per_step=ms_step, ms_per_step_median=ms_step_median,
               attn_ms=ms_attn, attn_ms_median=ms_attn_median,
               timing="back-to-back launches, arguments marshalled once; an event after every step")
    if cold:
        out["attn_ms_single_launch_warm"] = single_launch_ms(torch, dev, s["attn_b"], False)
        out["attn_ms_single_launch_cold_mall"] = single_launch_ms(torch, dev, s["attn_b"], True)
    if s["sep_b"] is not None:
        out["ms_per_step_rope_then_attn"] = timer(s["sep_b"], steps, warmup)
    if not args.no_graph:  # the same steps as HIP graph replays, for comparison
        graph_ok = check_graph_replay(torch, s["step"], [s["o"], s["q"], s["k"]],
                                      [s["q"], s["k"], s["v"]])
        out["graph_replay_matches_eager"] = graph_ok
        out["ms_per_step_graph"] = (Timer(torch, graph=True)(s["step"], steps, warmup)
                                    if graph_ok else None)
    fl = attn_flops(w)
    by = attn_bytes(w)
    kernel = ("decode_bf16" if s["decode"] else "attn_f32" if w.dtype == "f32"
              else f"prefill_bf16_d{w.d}")
    out["attn_kernel"] = kernel
    out["attn_tflops"] = fl / (ms_attn * 1e-3) / 1e12
    out["attn_gbs"] = by / (ms_attn * 1e-3) / 1e9
    out["roofline_attn"] = roofline(fl, by, ms_attn, w.dtype, ms_attn_median)
    out["roofline_step"] = roofline(fl, by, ms_step, w.dtype, ms_step_median)
    if s["rope"] is not None:
        ms_rope = timer(s["rope_b"], steps, warmup)
        rb = rope_bytes(w, s["decode"])
        out["rope_ms"] = ms_rope
        out["rope_gbs"] = rb / (ms_rope * 1e-3) / 1e9
        out["rope_pct_hbm_peak"] = 100.0 * out["rope_gbs"] / PEAK_HBM_GBS
    out["step_flops"] = fl
    out["attn_bytes"] = by
    del s
    torch.cuda.empty_cache()
    return out


CACHED_STEPS = [
    # name, B, Hq, Hkv, Tn, Tmax, pos, d
    ("decode_step_bf16_B32_Hq32_Hkv8_pos8191_Tmax8192_d128", 32, 32, 8, 1, 8192, 8191, 128),
    ("chunked_prefill_bf16_B1_Hq32_Hkv8_Tn512_pos3584_Tmax4096_d128", 1, 32, 8, 512, 4096, 3584, 128),
]


def measure_cached_steps(torch, ra, wl, dev):
    """attn_decode_step (one launch for a one-token step: RoPE of the new
    query and key, cache append, split-K attention and the merge of its
    chunks; RoPE and append, then the attention, for a chunk of rows)
    against the same step as separate calls (rope_apply on q and on the new
    keys, two cache copies, attention over the cache prefix).  Inputs are
    seeded draws; each timed call rotates q again in place, which leaves the
    amount of work unchanged."""
    out = {}
    for name, B, Hq, Hkv, Tn, Tmax, pos, d in CACHED_STEPS:
        q, kn, vn = (x.to(dev) for x in wl.random_qkv(B, Hq, Hkv, Tn, Tn, d, seed=2001))
        _, kc, vc = (x.to(dev) for x in wl.random_qkv(1, 1, Hkv * B, 1, Tmax, d, seed=2002))
        kc = kc.view(B, Hkv, Tmax, d).contiguous()
        vc = vc.view(B, Hkv, Tmax, d).contiguous()
        o = torch.empty_like(q)
        scale = 1.0 / (d ** 0.5)
        ws = ra.decode_step_workspace(q, kc)
        nb = ra.attn_workspace_bytes(B, Hq, Hkv, Tn, Tmax, d, torch.bfloat16)
        ws_attn = torch.empty(nb, dtype=torch.uint8, device=dev) if nb else None
        fused = ra.bind_attn_decode_step(q, kn, vn, kc, vc, pos, o, scale=scale, workspace=ws)
        k2 = kn.clone()
        rope_q = ra.bind_rope_apply(q, None, pos0=pos)
        rope_k = ra.bind_rope_apply(k2, None, pos0=pos)
        kview, vview = kc[:, :, :pos + Tn], vc[:, :, :pos + Tn]
        attn = ra.bind_attn_fwd_ws(q, kview, vview, o, ws_attn, None, scale=scale, causal=True,
                                   q_offset=pos)

        def unfused():
            rope_q()
            rope_k()
            kc[:, :, pos:pos + Tn].copy_(k2)
            vc[:, :, pos:pos + Tn].copy_(vn)
            attn()

        timer = Timer(torch)
        t_est = timer(fused, 3, 1) * 1e-3
        warm, steps = max(5, int(0.03 / t_est)), max(10, int(0.05 / t_est))
        ms_f = timer(fused, steps, warm)
        ms_u = timer(unfused, steps, warm)
        kv_bytes = 2.0 * 2 * d * B * Hkv * (pos + Tn)       # cache read once per K/V head
        flops = 4.0 * B * Hq * d * n_visible(Tn, pos + Tn, True, pos)
        out[name] = {"ms_per_step": round(ms_f, 4), "ms_per_step_separate_calls": round(ms_u, 4),
                     "cache_gbs": round(kv_bytes / (ms_f * 1e-3) / 1e9, 1),
                     "tflops": round(flops / (ms_f * 1e-3) / 1e12, 2)}
        print(f"# {name}: fused step {ms_f * 1e3:.1f} us, separate calls {ms_u * 1e3:.1f} us",
              file=sys.stderr)
        del q, kn, vn, kc, vc, o, ws, ws_attn, k2, kview, vview
        torch.cuda.empty_cache()
    return out


VALUE_WIDTHS = ((128, 64), (64, 128))


def measure_value_widths(torch, ra, wl, dev):
    """attn_fwd_dv (values of their own width) on workload 3's shape (B2 Hq32
    Hkv8 T4096, causal) with (d_k, d_v) = (128, 64) and (64, 128).  FLOPs:
    2 (d_k + d_v) per visible pair (the two products)."""
    w = wl.WORKLOADS[3]
    out = {}
    for dk, dv in VALUE_WIDTHS:
        q, k, _ = (x.to(dev) for x in wl.random_qkv(w.B, w.Hq, w.Hkv, w.Tq, w.Tk, dk, seed=3001))
        _, _, v = (x.to(dev) for x in wl.random_qkv(w.B, w.Hq, w.Hkv, 1, w.Tk, dv, seed=3002))
        o = torch.empty(w.B, w.Hq, w.Tq, dv, dtype=q.dtype, device=dev)
        call = ra._fwd_dv_call(q, k, v, o, None, dk ** -0.5, True, 0, None)
        timer = Timer(torch)
        t_est = timer(call, 3, 1) * 1e-3
        ms = timer(call, max(10, int(0.05 / t_est)), max(5, int(0.03 / t_est)))
        flops = 2.0 * (dk + dv) * w.B * w.Hq * n_visible(w.Tq, w.Tk, True, 0)
        tf = flops / (ms * 1e-3) / 1e12
        name = f"bf16_B{w.B}_Hq{w.Hq}_Hkv{w.Hkv}_T{w.Tq}_dk{dk}_dv{dv}"
        out[name] = {"ms": round(ms, 4), "tflops": round(tf, 1),
                     "pct_of_bf16_peak": round(100.0 * tf / PEAK_BF16_TFLOPS, 1)}
        print(f"# value width {name}: {ms * 1e3:.1f} us = {tf:.1f} TFLOP/s", file=sys.stderr)
        del q, k, v, o
        torch.cuda.empty_cache()
    return out


BACKWARD_WORKLOADS = (2, 3)


def measure_backward(torch, ra, wl, dev):
    """attn_bwd (the two gradient kernels: dQ with the rows' statistics, dK/dV) on
    the workloads' shapes, with the upstream gradient a seeded N(0, 1) draw
    and o, lse from the forward on the same inputs.  FLOPs: the five matrix
    products of the gradients (S recomputed, dP, dV, dK, dQ) over the visible
    pairs, 10 * B * Hq * d * N_vis."""
    out = {}
    for key in BACKWARD_WORKLOADS:
        w = wl.WORKLOADS[key]
        q, k, v = (x.to(dev) for x in wl.inputs(w))
        g = torch.Generator(device="cpu").manual_seed(w.seed + 500)
        dO = torch.randn(q.shape, generator=g).to(q.dtype).to(dev)
        o = torch.empty_like(q)
        lse = torch.empty(w.B, w.Hq, w.Tq, dtype=torch.float32, device=dev)
        ra.attn_fwd_ws(q, k, v, o, None, lse, scale=w.scale, causal=w.causal, q_offset=w.q_offset)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        nb = ra.attn_bwd_workspace_bytes(w.B, w.Hq, w.Hkv, w.Tq, w.Tk, w.d, q.dtype)
        ws = torch.empty(nb, dtype=torch.uint8, device=dev)
        bwd = ra.bind_attn_bwd(q, k, v, o, dO, lse, dq, dk, dv, ws, scale=w.scale, causal=w.causal,
                               q_offset=w.q_offset)
        timer = Timer(torch)
        t_est = timer(bwd, 3, 1) * 1e-3
        ms = timer(bwd, max(10, int(0.05 / t_est)), max(5, int(0.03 / t_est)))
        flops = 10.0 * w.B * w.Hq * w.d * n_visible(w.Tq, w.Tk, w.causal, w.q_offset)
        tf = flops / (ms * 1e-3) / 1e12
        out[w.name] = {"ms": round(ms, 4), "tflops": round(tf, 1),
                       "pct_of_bf16_peak": round(100.0 * tf / PEAK_BF16_TFLOPS, 1)}
        print(f"# backward {w.name}: {ms * 1e3:.1f} us = {tf:.1f} TFLOP/s", file=sys.stderr)
        del q, k, v, dO, o, lse, dq, dk, dv, ws
        torch.cuda.empty_cache()
    return out


def cpu_baseline(w, seconds):
    """The fp64 oracle on the host cores, on a bounded sample of workload w:
    whole passes over the workload when one pass fits the time budget, else
    an evenly spread sample of query rows (each with all its visible keys)."""
    import numpy as np

    import oracle
    from transformer_causal_self_amd import workloads as wl

    q, k, v = wl.inputs(w)
    q64 = q.double().numpy(); k64 = k.double().numpy(); v64 = v.double().numpy()
    del q, k, v
    orc = oracle.default()
    if w.rope:
        k64 = orc.rope(k64, 0, w.rope_base)
        q64 = orc.rope(q64, w.q_offset, w.rope_base)
    full_flops = attn_flops(w)
    # calibrate on a small row sample
    rng = np.random.default_rng(0)
    n_rows = w.B * w.Hq * w.Tq
    probe = min(n_rows, 512)
    idx = rng.choice(n_rows, size=probe, replace=False)
    rows = np.stack([idx // (w.Hq * w.Tq), (idx // w.Tq) % w.Hq, idx % w.Tq], axis=1)
    t0 = time.perf_counter()
    orc.attn_rows(q64, k64, v64, rows, w.scale, causal=w.causal, q_offset=w.q_offset)
    t_probe = time.perf_counter() - t0
    est_full = t_probe * n_rows / probe
    flops_done = 0.0
    t_total = 0.0
    if est_full <= seconds:
        passes = 0
        while True:
            t0 = time.perf_counter()
            orc.attn(q64, k64, v64, w.scale, causal=w.causal, q_offset=w.q_offset)
            t_total += time.perf_counter() - t0
            flops_done += full_flops
            passes += 1
            if t_total >= seconds or passes >= 1000:
                break
        sample = f"{passes} full pass(es) over the workload ({w.B * w.Hq * w.Tq} query rows)"
    else:
        n = max(1, int(n_rows * seconds / est_full))
        idx = np.linspace(0, n_rows - 1, n).astype(np.int64)
        rows = np.stack([idx // (w.Hq * w.Tq), (idx // w.Tq) % w.Hq, idx % w.Tq], axis=1)
        t0 = time.perf_counter()
        orc.attn_rows(q64, k64, v64, rows, w.scale, causal=w.causal, q_offset=w.q_offset)
        t_total = time.perf_counter() - t0
        vis = [min(w.Tk, w.q_offset + int(i) + 1) if w.causal else w.Tk for i in rows[:, 2]]
        flops_done = 4.0 * w.d * float(sum(vis))
        sample = f"{n} of {n_rows} query rows, evenly spaced, all visible keys each"
    return {"value": flops_done / t_total / 1e12, "unit": "TFLOP/s",
            "cores": oracle.threads_used(), "kind": "oracle",
            "sample": f"{sample}; {t_total:.1f} s of fp64 work"}


def calib_copy(torch, dev, nbytes=1 << 30, reps=5):
    a = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
    b = torch.empty_like(a)
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"calib_copy_bytes_read": nbytes, "calib_copy_bytes_written": nbytes,
                      "reps": reps}))


CALIB_LIBRARY = os.path.join(ROOT, "transformer_causal_self_amd", "librocattn_calib.so")


def calib_library():
    import ctypes
    if not os.path.exists(CALIB_LIBRARY):
        raise RuntimeError(f"{CALIB_LIBRARY} is not built: run __graft_entry__.build()")
    lib = ctypes.CDLL(CALIB_LIBRARY)
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    lib.calib_mfma_loop.argtypes = [ctypes.c_int, ctypes.c_int, vp, vp]
    lib.calib_mfma_loop_flops.argtypes = [ctypes.c_int, ctypes.c_int]
    lib.calib_mfma_loop_flops.restype = ctypes.c_double
    lib.calib_stream_read.argtypes = [vp, sz, ctypes.c_int, vp, vp]
    lib.calib_stream_copy.argtypes = [vp, vp, sz, ctypes.c_int, vp]
    return lib


MFMA_LOOP_WG, MFMA_LOOP_ITERS = 2048, 4000    # 8 waves per SIMD (two rounds of 4); ~2 ms
STREAM_BYTES = 2 << 30                        # 2 GiB: far past the 256 MB MALL
STREAM_WGS = (256, 512, 1024, 2048)


def measured_peaks(torch, dev, reps=10):
    """The matrix-core loop and the streaming read and copy of
    librocattn_calib.so, timed with events on the current stream (median of
    `reps` launches after 3 warm-up launches)."""
    lib = calib_library()
    stream = torch.cuda.current_stream().cuda_stream

    def med(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        ts.sort()
        return ts[len(ts) // 2]

    sink = torch.empty(max(MFMA_LOOP_WG, max(STREAM_WGS)), dtype=torch.float32, device=dev)

    def mfma():
        if lib.calib_mfma_loop(MFMA_LOOP_WG, MFMA_LOOP_ITERS, sink.data_ptr(), stream) != 0:
            raise RuntimeError("calib_mfma_loop failed")

    ms_mfma = med(mfma)
    tf = lib.calib_mfma_loop_flops(MFMA_LOOP_WG, MFMA_LOOP_ITERS) / (ms_mfma * 1e-3) / 1e12
    src = torch.empty(STREAM_BYTES, dtype=torch.uint8, device=dev).fill_(1)

    # the best of a few grid sizes (one, two, four and eight workgroups of
    # 256 lanes per CU)
    best_read, best_wg = None, None
    for wg in STREAM_WGS:
        def read(wg=wg):
            if lib.calib_stream_read(src.data_ptr(), STREAM_BYTES, wg, sink.data_ptr(), stream) != 0:
                raise RuntimeError("calib_stream_read failed")
        ms = med(read)
        if best_read is None or ms < best_read:
            best_read, best_wg = ms, wg
    ms_read = best_read
    half = STREAM_BYTES // 2
    dst = torch.empty(half, dtype=torch.uint8, device=dev)

    def copy():
        if lib.calib_stream_copy(src.data_ptr(), dst.data_ptr(), half, best_wg, stream) != 0:
            raise RuntimeError("calib_stream_copy failed")

    ms_copy = med(copy)
    del src, dst, sink
    torch.cuda.empty_cache()
    return {
        "mfma_bf16_loop_tflops": tf,
        "mfma_bf16_loop_frac_of_published": tf / PEAK_BF16_TFLOPS,
        "hbm_stream_read_gbs": STREAM_BYTES / (ms_read * 1e-3) / 1e9,
        "hbm_stream_copy_gbs": 2 * half / (ms_copy * 1e-3) / 1e9,
        "published": {"mfma_bf16_tflops": PEAK_BF16_TFLOPS, "hbm_gbs": PEAK_HBM_GBS},
        "how": (f"v_mfma_f32_32x32x16_bf16 loop, {MFMA_LOOP_WG} workgroups x 4 waves x "
                f"{MFMA_LOOP_ITERS} rounds of 4 products; 16-byte non-temporal read of "
                f"{STREAM_BYTES >> 30} GiB (best of {list(STREAM_WGS)} workgroups: {best_wg}) and copy of "
                f"{half >> 30} GiB; median of {reps} launches each"),
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", type=int, default=4, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--no-also", action="store_true", help="skip the other workloads")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--calib-copy", action="store_true")
    ap.add_argument("--calib-mfma", action="store_true")
    ap.add_argument("--calib-hbm", action="store_true")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the HIP graph replay comparison")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(no collectives); run it with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    import transformer_causal_self_amd as ra
    from transformer_causal_self_amd import workloads as wl

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    ra.library()
    dev = torch.device("cuda:0")
    if args.calib_copy:
        calib_copy(torch, dev)
        return
    if args.calib_mfma or args.calib_hbm:
        print(json.dumps(measured_peaks(torch, dev)))
        return

    w = wl.WORKLOADS[args.workload]
    head = measure(w, args, torch, ra, wl, dev, args.steps, args.warmup, cold=(args.workload == 2))
    print(f"# {w.name}: step {head['ms_per_step'] * 1e3:.2f} us (median "
          f"{head['ms_per_step_median'] * 1e3:.2f}), attention {head['attn_ms'] * 1e3:.2f} us",
          file=sys.stderr)

    decode = head["attn_kernel"] == "decode_bf16"
    step_s = head["ms_per_step"] * 1e-3
    if decode:
        metric_val = head["attn_bytes"] / step_s / 1e9
        unit = "GB/s"
    else:
        metric_val = head["step_flops"] / step_s / 1e12
        unit = "TFLOP/s"

    # Roofline of the dominant kernel from the event-timed steps.  For the
    # RoPE prefills a step is one attn_fwd_rope call: the prefill kernel plus
    # the RoPE pass on k (about 1 % of the step at 16384 keys), so the rate
    # is a slight underestimate of the prefill kernel's own.
    kernel = head["attn_kernel"]
    if w.rope and not decode:
        roof = dict(head["roofline_step"])
        roof["kernel"] = f"{kernel} (query-load RoPE) + rope pass on k: one attn_fwd_rope call"
        roof["launch_us"] = head["ms_per_step"] * 1e3
        roof["launch_us_median"] = head["ms_per_step_median"] * 1e3
    else:
        roof = dict(head["roofline_attn"])
        roof["kernel"] = kernel
        roof["launch_us"] = head["attn_ms"] * 1e3
        roof["launch_us_median"] = head["attn_ms_median"] * 1e3
    roof["algorithmic_bytes"] = head["attn_bytes"]
    roof["algorithmic_flops"] = head["step_flops"]
    roof["traffic"] = measured_traffic("attn_fwd_rope_bf16_d128" if w.rope and not decode and w.d == 128
                                       else kernel, w.name)

    line = {
        "metric": "causal attention TFLOP/s + % bf16 MFMA peak (prefill); GB/s + % HBM (decode)",
        "value": metric_val,
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": head["warmup"],
        "ms_per_step": head["ms_per_step"],
        "ms_per_step_median": head["ms_per_step_median"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if w.dtype == "f32" else "bf16",
        "data": "synthetic (seeded N(0, sigma^2) q/k/v, see transformer_causal_self_amd/workloads.py)",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "Tq": w.Tq,
                   "Tk": w.Tk, "d_head": w.d, "causal": w.causal, "q_offset": w.q_offset,
                   "scale": w.scale, "rope": w.rope, "sigma": w.sigma, "parallelism": "single GPU"},
        "pct_of_peak": 100.0 * roof["frac"],
        "roofline": roof,
        "timing": head["timing"],
        "attn_ms_plain_prefill": head["attn_ms"],
        "ms_per_step_graph": head.get("ms_per_step_graph"),
        "attn_ms_single_launch_warm": head.get("attn_ms_single_launch_warm"),
        "attn_ms_single_launch_cold_mall": head.get("attn_ms_single_launch_cold_mall"),
        "ms_per_step_rope_then_attn": head.get("ms_per_step_rope_then_attn"),
        "graph_replay_matches_eager": head.get("graph_replay_matches_eager"),
    }
    line["measured_peaks"] = measured_peaks(torch, dev)
    mp = line["measured_peaks"]
    roof["frac_of_measured_peak"] = (roof["tflops"] / mp["mfma_bf16_loop_tflops"] if roof["bound"] == "mfma"
                                     else roof["gbs"] / mp["hbm_stream_read_gbs"] if roof["bound"] == "hbm"
                                     else None)

    if not args.no_also:
        also = {}
        for key in (1, 2, 3, 4, 5):
            if key == args.workload:
                continue
            wo = wl.WORKLOADS[key]
            r = measure(wo, args, torch, ra, wl, dev, cold=(key == 2))
            r = {kk: (round(vv, 4) if isinstance(vv, float) else vv) for kk, vv in r.items()}
            r["attn_traffic"] = measured_traffic(r["attn_kernel"], wo.name)
            also[str(key)] = r
            print(f"# {wo.name}: attention {r['attn_ms'] * 1e3:.2f} us = "
                  f"{r['attn_tflops']:.1f} TFLOP/s, {r['attn_gbs']:.0f} GB/s", file=sys.stderr)
        line["also"] = also
        line["cached_steps"] = measure_cached_steps(torch, ra, wl, dev)
        line["backward"] = measure_backward(torch, ra, wl, dev)
        line["value_width"] = measure_value_widths(torch, ra, wl, dev)

    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(line))


if __name__ == "__main__":
    main()
