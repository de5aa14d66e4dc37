#!/usr/bin/env python3
"""Benchmark of the cached-prefix flow-matching denoise loop on one MI355X.

Workload: the pi0.5-shaped bf16 action expert at batch 1 (18 layers, width 1024,
8 query heads + 1 KV head of 256, GeGLU MLP 4096, 816 cached prefix tokens, a
50 x 32 action chunk, 10 Euler steps), seeded synthetic weights N(0, 0.02),
prefix K/V and noise N(0, 1).  One "step" of this benchmark is one whole denoise
call (all 10 Euler steps of one action chunk), replayed as a single hipGraph
with the prefix KV and the timestep tables already installed, inputs resident in
HBM.  Timing follows the protocol of the PhyAI reading (10 warm-up and 50 timed
iterations), bracketed by device synchronisation.

Printed JSON fields beyond the metric: per-call latency statistics, the
isolated duration of every loop kernel (one graph replay of back-to-back
launches, timed with HIP events on the context stream), the roofline of the
dominant kernel, and the CPU oracle timed on a bounded sample.
"""
from __future__ import annotations

import argparse
import ctypes
import dataclasses
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "ms per action chunk (10 Euler steps) at batch 1; chunks/sec at batch 32"
HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = 2500.0   # dense bf16
# loop kernels and their ids for phyai_enqueue_kernel_repeat; "attn_merge" combines the
# key splits of the few-row attention (its own launch), and has no algorithmic bytes of its own
# HBM bytes per launch of the batch-1 loop kernels (dispatches inside the loop) from the
# rocprofv3 FETCH_SIZE and WRITE_SIZE passes summarised in profiles/pi05_b1_loop_kernels.md:
# raw KiB scaled by what the same counters read for a 256 MiB device-to-device copy (fetch x2.0,
# write x1.0).  They describe the kernel sources they were taken on: the hash covers every
# source file of the library, and any change makes the bench report traffic null.
PROFILED_TRAFFIC = {
    "sources_sha256": "4813797312d8e5fd7940eff6eb414dd3cd9b37a4ca83d975e56a3f669db1d25c",
    "bytes": {"qkv": 6967297, "attention": 8970755, "attn_merge": 6722561, "o_proj": 7726641,
              "gate_up": 18945027, "down": 13807571, "out_euler": 2170727},
}


def profiled_traffic(kernel):
    """Counted HBM bytes per launch of a loop kernel, or None once the sources changed."""
    csrc = os.path.join(ROOT, "flow_matching_action_cached_amd", "csrc")
    h = hashlib.sha256()
    for n in sorted(os.listdir(csrc)):
        if n.endswith((".hip", ".h", ".cpp")):
            h.update(n.encode())
            with open(os.path.join(csrc, n), "rb") as f:
                h.update(f.read())
    if h.hexdigest() != PROFILED_TRAFFIC["sources_sha256"]:
        return None
    return PROFILED_TRAFFIC["bytes"].get(kernel)


def stage_traffic(stage):
    """Counted bytes per launch of a loop stage (the attention stage: attention + merge)."""
    parts = ["attention", "attn_merge"] if stage == "attention" else [stage]
    vals = [profiled_traffic(k) for k in parts]
    return None if any(v is None for v in vals) else int(sum(vals))


KERNEL_IDS = {"qkv": 0, "attention": 1, "attn_merge": 7, "o_proj": 2, "gate_up": 3, "down": 4, "out_euler": 5}
KERNELS = ["qkv", "attention", "o_proj", "gate_up", "down", "out_euler"]


def algorithmic_bytes(d):
    """Bytes the method must move per launch of each loop kernel (weights of that
    linear, or the layer's K/V for attention); activations stay on chip / in L2."""
    e = 2  # bf16
    qd = d.n_q_heads * d.head_dim
    kv = 2 * (d.prefix_len + d.chunk_len) * d.n_kv_heads * d.head_dim * e
    return {
        "qkv": d.qkv_dim * d.width * e,
        "attention": kv,
        "o_proj": d.width * qd * e,
        "gate_up": 2 * d.mlp_dim * d.width * e,
        "down": d.width * d.mlp_dim * e,
        "out_euler": 2 * d.action_dim * d.width * e,
    }


def chunk_bytes(d):
    """Algorithmic bytes per chunk: N x (all weights + prefix K/V + per-step tables)."""
    e = 2
    per_layer = (d.qkv_dim * d.width + d.width * d.n_q_heads * d.head_dim + 3 * d.mlp_dim * d.width) * e
    io = 2 * d.action_dim * d.width * e
    kv = 2 * d.n_layers * d.prefix_len * d.n_kv_heads * d.head_dim * e
    tables = d.n_mod * 2 * d.width * 4
    return d.n_steps * (d.n_layers * per_layer + io + kv + tables)


def chunk_bytes_int4(d):
    """Per chunk: N x (int4 codes + bf16 scales of the expert linears, bf16 in/out
    projections, prefix K/V, tables)."""
    per_layer = d.qkv_dim * d.width + d.width * d.n_q_heads * d.head_dim + 3 * d.mlp_dim * d.width
    codes = d.n_layers * per_layer // 2
    scales = d.n_layers * per_layer // 128 * 2
    io = 2 * d.action_dim * d.width * 2
    kv = 2 * d.n_layers * d.prefix_len * d.n_kv_heads * d.head_dim * 2
    tables = d.n_mod * 2 * d.width * 4
    return d.n_steps * (codes + scales + io + kv + tables)


def batch_flops(d):
    """Algorithmic MFMA flops of one chunk for the whole batch: the four expert linears
    (2 * rows * params per layer) plus attention (QK^T and PV over prefix + chunk keys),
    times layers and steps.  In/out projections and element-wise work are not counted."""
    rows = d.batch * d.chunk_len
    per_layer = d.qkv_dim * d.width + d.width * d.n_q_heads * d.head_dim + 3 * d.mlp_dim * d.width
    lin = 2 * rows * per_layer
    keys = d.prefix_len + d.chunk_len
    attn = 4 * rows * d.n_q_heads * keys * d.head_dim
    return d.n_steps * d.n_layers * (lin + attn)


def wam_flops(d):
    """Algorithmic MFMA flops of one joint chunk: both guidance branches (2 x T token rows)
    through the four linears of every layer plus full self-attention over the T tokens,
    times layers and steps (in/out projections and element-wise work not counted)."""
    T = d.latent_tokens + d.action_tokens
    rows = 2 * T
    hd = d.n_heads * d.head_dim
    per_layer = 3 * hd * d.width + d.width * hd + 3 * d.mlp_dim * d.width
    return d.n_steps * d.n_layers * (2 * rows * per_layer + 4 * rows * T * hd)


def wam_kernel_flops(d):
    T = d.latent_tokens + d.action_tokens
    rows = 2 * T
    hd = d.n_heads * d.head_dim
    return {"qkv": 2 * rows * 3 * hd * d.width, "attention": 4 * rows * T * hd, "o_proj": 2 * rows * d.width * hd,
            "gate_up": 2 * rows * 2 * d.mlp_dim * d.width, "down": 2 * rows * d.mlp_dim * d.width}


def time_chunks(ex, noise, out, steps, warmup, torch):
    for _ in range(warmup):
        ex.denoise(noise, out)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        ex.denoise(noise, out)
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


def kernel_times(ex, reps, torch, names=KERNELS):
    """Mean duration of each loop kernel, one graph replay of `reps` launches each."""
    res = {}
    for name in names:
        which = KERNEL_IDS[name]
        ex.enqueue_kernel_repeat(which, 0, reps)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        ex.enqueue_kernel_repeat(which, 0, reps)
        b.record()
        torch.cuda.synchronize()
        res[name] = a.elapsed_time(b) * 1000.0 / reps
    return res


def schedule(n):
    import numpy as np
    dt = -1.0 / n
    return np.array([1.0 + k * dt for k in range(n)], dtype=np.float64).astype(np.float32)


def device_inputs(d, inputs, torch):
    el = torch.bfloat16
    keys = ("w_in", "b_in", "w_out", "b_out", "w_mod", "b_mod", "w_qkv", "w_o", "w_gu", "w_d")
    w = {k: torch.from_numpy(inputs[k]).cuda().to(el).contiguous() for k in keys}
    k = torch.from_numpy(inputs["k_pre"]).cuda().to(el).contiguous()
    v = torch.from_numpy(inputs["v_pre"]).cuda().to(el).contiguous()
    noise = torch.from_numpy(inputs["noise"]).cuda().contiguous()
    return w, k, v, noise


def cpu_baseline(d, inputs):
    """The CPU oracle (float64 NumPy) on one whole chunk of the same workload, all cores;
    beside it, labelled extrapolations: one Euler step on one thread (x N steps), the batch-32
    chunk (the oracle evaluates samples one by one), and the joint denoiser's guided pair from
    one layer of one step at full width (x layers x steps)."""
    from oracle import expert as ox
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threadpool_limits = None
        threads = os.cpu_count() or 1
    t = schedule(d.n_steps)
    ts = []
    for _ in range(4):  # one warm-up, three timed
        t0 = time.perf_counter()
        ox.denoise(inputs, d, t=t)
        ts.append(time.perf_counter() - t0)
    sec = statistics.median(ts[1:])
    out = {"value": round(sec * 1000.0, 1), "unit": "ms/chunk", "cores": int(threads), "kind": "oracle",
           "sample": "1 chunk (10 Euler steps) of the pi0.5-shaped workload at batch 1, float64 NumPy; "
                     "median of 3 timed runs after 1 warm-up"}
    # one Euler step (velocity of step 0 and the update) of sample 0 on one thread, x N
    p = ox.as_f64_params(inputs)
    tables = ox.modulation_tables(t, inputs["w_mod"], inputs["b_mod"])
    kp = inputs["k_pre"][0].astype("float64")
    vp = inputs["v_pre"][0].astype("float64")
    x0 = inputs["noise"][0].astype("float64")

    def one_step():
        t0 = time.perf_counter()
        x0 + ox.step_sizes(t)[0] * ox.velocity(x0, tables[0], p, kp, vp, d)
        return time.perf_counter() - t0

    if threadpool_limits is not None:
        with threadpool_limits(limits=1):
            one_step()
            st = one_step()
        out["single_thread"] = {
            "value": round(st * d.n_steps * 1000.0, 1), "unit": "ms/chunk", "cores": 1, "kind": "oracle",
            "extrapolated": True,
            "sample": f"one Euler step of the batch-1 chunk on one thread ({st * 1000.0:.1f} ms), x {d.n_steps} steps"}
    out["batch32_extrapolated"] = {
        "value": round(32 * sec * 1000.0, 1), "unit": "ms per batch-32 chunk",
        "chunks_per_s": round(32 / (32 * sec), 3), "cores": int(threads), "kind": "oracle", "extrapolated": True,
        "sample": "the timed batch-1 chunk x 32 samples (samples never interact; the oracle runs them one by one)"}
    # joint denoiser: both guidance branches through one layer of one step at full width
    import dataclasses as dc
    import synth
    from oracle import wam as ow
    dw = synth.WAM_CONFIGS["wam"]
    d1 = dc.replace(dw, n_layers=1)
    iw = synth.make_wam_inputs(d1, 0)
    keys = ("w_in_lat", "b_in_lat", "w_in_act", "b_in_act", "w_out_lat", "b_out_lat", "w_out_act", "b_out_act",
            "w_qkv", "w_o", "w_gu", "w_d")
    pw = {k: iw[k].astype("float64") for k in keys}
    tw = schedule(dw.n_steps)
    zl, za = iw["z_lat"].astype("float64"), iw["z_act"].astype("float64")
    t0 = time.perf_counter()
    for cond in (iw["c_cond"], iw["c_uncond"]):
        ow.velocity(zl, za, ow.modulation(tw[0], cond, iw["w_mod"], iw["b_mod"]), pw, d1)
    lw = time.perf_counter() - t0
    del pw, iw
    out["joint_extrapolated"] = {
        "value": round(lw * dw.n_layers * dw.n_steps * 1000.0, 1), "unit": "ms/chunk", "cores": int(threads),
        "kind": "oracle", "extrapolated": True,
        "sample": f"one layer of one step of both guidance branches at full width ({dw.latent_tokens + dw.action_tokens}"
                  f" tokens, width {dw.width}; {lw * 1000.0:.0f} ms incl. in/out projections), x {dw.n_layers} layers "
                  f"x {dw.n_steps} steps"}
    return out


PHASE_NAMES = ["QKV", "attention", "merge", "O + residual sum", "gate/up", "down + residual sum"]


def persistent_trace(d, ex, noise, out, np, torch):
    """Per-phase breakdown of the persistent loop (phase-trace build: per workgroup and phase,
    real-time stamps at 100 MHz of the wait's begin and end and of the flag's publication).
    A phase's span on an XCD runs from that XCD's last flag of the previous phase to its last
    flag of this one; the hand-off lag from that previous flag to a workgroup's wait end."""
    lib = ex._lib
    lib.phyai_persist_trace.argtypes = [ctypes.c_void_p]
    slots, max_phases = 8, 4096
    buf = np.zeros(256 * max_phases * slots, np.uint64)
    ex.set_persistent(True)
    if ex.loop_form(1) != 1:
        raise RuntimeError("the persistent loop form is not available for this workload")
    for _ in range(3):
        ex.denoise(noise, out)
    ex.sync()
    lib.phyai_persist_trace(buf.ctypes.data)  # clear
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    ex.denoise(noise, out)
    b.record()
    ex.sync()
    if lib.phyai_persist_trace(buf.ctypes.data) != 0:
        raise RuntimeError("phyai_persist_trace failed")
    L = d.n_layers
    n_ph = 1 + d.n_steps * (6 * L + 1)
    t = buf.reshape(256, max_phases, slots)[:, :n_ph].astype(np.int64)
    xcd = np.arange(256) & 7

    def kind(p):
        q = (p - 1) % (6 * L + 1)
        return "out/Euler/in" if q == 6 * L else PHASE_NAMES[q % 6]

    rows = {}
    for p in range(2, n_ph):
        for x in range(8):
            m = xcd == x
            prev = t[m, p - 1, 2].max()
            rows.setdefault(kind(p), []).append(((t[m, p, 2].max() - prev) / 100.0,
                                                 np.median(t[m, p, 1] - prev) / 100.0,
                                                 np.median(t[m, p, 2] - t[m, p, 1]) / 100.0))
    print(f"persistent loop, {d.n_layers} layers x {d.n_steps} steps, batch 1: traced chunk "
          f"{a.elapsed_time(b):.3f} ms ({n_ph} phases)")
    print("phase                 span_us  lag_us  work_us   (medians over 8 XCDs x instances)")
    per_layer = 0.0
    for k in PHASE_NAMES + ["out/Euler/in"]:
        v = np.array(rows[k])
        med = np.median(v, axis=0)
        if k != "out/Euler/in":
            per_layer += med[0]
        print(f"{k:20s} {med[0]:8.2f} {med[1]:7.2f} {med[2]:8.2f}")
    print(f"sum of the layer's phase spans: {per_layer:.2f} us")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--kernel-reps", type=int, default=200)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-variants", action="store_true")
    ap.add_argument("--variants", default="int4,rope,gated,prefill,persistent,capsule,b32,wam,wam_unipc,wam_tp4",
                    help="comma-separated variants to measure after the batch-1 line: int4, rope, gated, "
                         "prefill, persistent, capsule, b32, wam, wam_unipc (needs wam), wam_tp4")
    ap.add_argument("--persistent-trace", action="store_true",
                    help="instead of the bench line: run the batch-1 loop as the persistent kernel with the "
                         "phase-trace build (libphyai_trace.so) and print its per-phase breakdown")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="before timing, copy a buffer of this many MiB device-to-device (a kernel of "
                         "known traffic for calibrating hardware byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the loop runs on a single MI355X; --gpus {args.gpus} "
              "is not supported)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import synth
    import flow_matching_action_cached_amd as fm

    if args.persistent_trace:
        fm.load_library(fm.LIB_PATH.replace("libphyai.so", "libphyai_trace.so"))
    d = synth.CONFIGS["pi05"]
    inputs = synth.make_expert_inputs(d, 0)
    w, kp, vp, noise = device_inputs(d, inputs, torch)
    ex = fm.ActionExpert.from_dims(d)
    ex.set_weights(w)
    ex.set_prefix_kv(kp, vp)
    ex.set_timestep_tables(schedule(d.n_steps))
    out = torch.empty_like(noise)
    print(f"[bench] setup done: {d}", file=sys.stderr, flush=True)
    if args.persistent_trace:
        persistent_trace(d, ex, noise, out, np, torch)
        ex.close()
        return
    if args.calib_copy_mb:
        n = args.calib_copy_mb << 18  # float32 elements
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    for _ in range(args.warmup):
        ex.denoise(noise, out)
    torch.cuda.synchronize()
    # timed region: K back-to-back chunks
    s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    s0.record()
    for _ in range(args.steps):
        ex.denoise(noise, out)
    s1.record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t_wall) * 1000.0
    ms_per_chunk = s0.elapsed_time(s1) / args.steps
    print(f"[bench] timed {args.steps} chunks: {ms_per_chunk:.4f} ms/chunk (wall {wall_ms / args.steps:.4f})",
          file=sys.stderr, flush=True)

    # per-call latency distribution (each call bracketed by its own events)
    lat = []
    for _ in range(args.steps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        ex.denoise(noise, out)
        b.record()
        b.synchronize()
        lat.append(a.elapsed_time(b))
    lat.sort()
    p99 = lat[min(len(lat) - 1, int(round(0.99 * (len(lat) - 1))))]

    # in-loop kernel durations: the same loop with an event after every launch on the context
    # stream, queued behind a short wait so that it runs back to back; the attention stage is the
    # attention launch plus the merge of its key splits
    # Each event costs the queue a few microseconds, which the intervals include: the loop with
    # marks runs longer than the graph replay by n_events x that cost, so every interval is
    # corrected by the mean cost per event (the graph's kernels run back to back: the sum of
    # their durations is its chunk time).
    stage_reps = max(5, args.steps // 5)
    st_us, loop_ms = ex.time_loop_stages(noise, reps=stage_reps)
    n_marks = 1 + d.n_steps * (6 * d.n_layers + 1)  # launches, each followed by an event
    ev_us = max(0.0, (loop_ms - ms_per_chunk) * 1000.0 / n_marks)
    raw_us = {"qkv": st_us[0], "attention": st_us[1] + st_us[7], "o_proj": st_us[2], "gate_up": st_us[3],
              "down": st_us[4], "out_euler": st_us[5]}
    inloop_us = {k: v - ev_us * (2 if k == "attention" else 1) for k, v in raw_us.items()}
    per_chunk = {k: d.n_steps * d.n_layers for k in KERNELS}
    per_chunk["out_euler"] = d.n_steps
    share = {k: inloop_us[k] * per_chunk[k] for k in KERNELS}
    dominant = max(share, key=share.get)
    abytes = algorithmic_bytes(d)
    ach = abytes[dominant] / (inloop_us[dominant] * 1e-6) / 1e9
    print(f"[bench] in-loop stages (us/launch): {inloop_us}, loop with marks {loop_ms:.4f} ms", file=sys.stderr,
          flush=True)
    # cache-warm figures: one graph replay of back-to-back launches of layer 0 (the same operands
    # can stay in L2 / the memory-side cache between launches)
    per_launch_us = kernel_times(ex, args.kernel_reps, torch, KERNELS + ["attn_merge"])
    print(f"[bench] isolated kernels (us/launch): {per_launch_us}", file=sys.stderr, flush=True)

    ex.denoise(noise, out)
    torch.cuda.synchronize()
    finite = bool(torch.isfinite(out).all().item())
    ex.close()

    # int4 group-128 variant of the same workload (expert linears quantised by the library)
    variants = {}
    todo = set() if args.no_variants else {v.strip() for v in args.variants.split(",") if v.strip()}
    if "int4" in todo:
        d4 = synth.CONFIGS["pi05_int4"]
        inp4 = synth.make_expert_inputs(d4, 0)
        w4 = {}
        for k in ("w_in", "b_in", "w_out", "b_out", "w_mod", "b_mod"):
            w4[k] = w[k]
        for k in ("w_qkv", "w_o", "w_gu", "w_d"):
            p_, s_ = fm.quantize_int4_g128(torch.from_numpy(inp4[k]).cuda())
            w4[k], w4["s" + k[1:]] = p_, s_
        del inp4
        e4 = fm.ActionExpert.from_dims(d4)
        e4.set_weights(w4)
        e4.set_prefix_kv(kp, vp)
        e4.set_timestep_tables(schedule(d.n_steps))
        for _ in range(args.warmup):
            e4.denoise(noise, out)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(args.steps):
            e4.denoise(noise, out)
        b.record()
        torch.cuda.synchronize()
        ms4 = a.elapsed_time(b) / args.steps
        e4.close()
        b4 = chunk_bytes_int4(d)
        variants["int4_g128_batch1"] = {"ms_per_chunk": round(ms4, 4), "chunks_per_s": round(1000.0 / ms4, 2),
                                        "algorithmic_bytes": b4,
                                        "hbm_frac": round(b4 / (ms4 * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        print(f"[bench] int4 variant: {ms4:.4f} ms/chunk", file=sys.stderr, flush=True)

    if "rope" in todo:
        # the same batch-1 workload with the chunk's queries and keys rotated (base 1e4)
        dr = dataclasses.replace(d, rope_theta=1e4)
        er = fm.ActionExpert.from_dims(dr)
        er.set_weights(w)
        er.set_prefix_kv(kp, vp)
        er.set_timestep_tables(schedule(d.n_steps))
        for _ in range(args.warmup):
            er.denoise(noise, out)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(args.steps):
            er.denoise(noise, out)
        b.record()
        torch.cuda.synchronize()
        msr = a.elapsed_time(b) / args.steps
        er.close()
        variants["rope_batch1"] = {"ms_per_chunk": round(msr, 4), "chunks_per_s": round(1000.0 / msr, 2),
                                   "rope_theta": 1e4,
                                   "hbm_frac": round(chunk_bytes(d) / (msr * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        print(f"[bench] rope variant: {msr:.4f} ms/chunk", file=sys.stderr, flush=True)

    if "gated" in todo:
        # the same batch-1 workload with residual gates (a third row block of W_mod, seeded)
        dg = dataclasses.replace(d, gated_residual=True)
        inpg = synth.make_expert_inputs(dg, 0)
        wg = dict(w)
        for k in ("w_mod", "b_mod"):
            wg[k] = torch.from_numpy(inpg[k]).cuda().to(torch.bfloat16).contiguous()
        del inpg
        eg = fm.ActionExpert.from_dims(dg)
        eg.set_weights(wg)
        eg.set_prefix_kv(kp, vp)
        eg.set_timestep_tables(schedule(d.n_steps))
        for _ in range(args.warmup):
            eg.denoise(noise, out)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(args.steps):
            eg.denoise(noise, out)
        b.record()
        torch.cuda.synchronize()
        msg = a.elapsed_time(b) / args.steps
        eg.close()
        variants["gated_residual_batch1"] = {"ms_per_chunk": round(msg, 4), "chunks_per_s": round(1000.0 / msg, 2),
                                             "hbm_frac": round(chunk_bytes(d) / (msg * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        print(f"[bench] gated-residual variant: {msg:.4f} ms/chunk", file=sys.stderr, flush=True)

    if "prefill" in todo:
        # prefix prefill: the prefix network (the expert's layer with a plain RMSNorm) over the
        # 816 prefix tokens, writing every layer's K/V into the cache; eager launches
        pre = synth.make_prefix_inputs(d, 1)
        ep = fm.ActionExpert.from_dims(d, prefill=True)
        ep.set_weights(w)
        ep.set_prefill_weights({k: torch.from_numpy(pre[k]).cuda().to(torch.bfloat16).contiguous()
                                for k in ("w_qkv", "w_o", "w_gu", "w_d")})
        tok = torch.from_numpy(pre["tokens"]).cuda().to(torch.bfloat16).contiguous()
        del pre
        for _ in range(args.warmup):
            ep.prefill(tok)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(args.steps):
            ep.prefill(tok)
        b.record()
        torch.cuda.synchronize()
        msp = a.elapsed_time(b) / args.steps
        ep.sync()
        ep.close()
        # 2 x rows x params of the four linears, plus QK^T and PV over the prefix keys, per layer
        rows, per_layer = d.prefix_len, d.qkv_dim * d.width + d.width * d.n_q_heads * d.head_dim + 3 * d.mlp_dim * d.width
        pf = d.n_layers * (2 * rows * per_layer + 4 * d.n_q_heads * rows * rows * d.head_dim)
        variants["prefill_816_batch1"] = {"ms_per_prefix": round(msp, 4), "algorithmic_tflop": round(pf / 1e12, 4),
                                          "mfma_frac": round(pf / (msp * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS, 4)}
        print(f"[bench] prefill variant: {msp:.4f} ms per prefix", file=sys.stderr, flush=True)

    if "persistent" in todo:
        # the same batch-1 workload as one persistent kernel (opt-in loop form)
        ep = fm.ActionExpert.from_dims(d)
        ep.set_weights(w)
        ep.set_prefix_kv(kp, vp)
        ep.set_timestep_tables(schedule(d.n_steps))
        ep.set_persistent(True)
        form = ep.loop_form(1)
        for _ in range(args.warmup):
            ep.denoise(noise, out)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(args.steps):
            ep.denoise(noise, out)
        b.record()
        ep.sync()
        msq = a.elapsed_time(b) / args.steps
        ep.close()
        variants["persistent_batch1"] = {"ms_per_chunk": round(msq, 4), "chunks_per_s": round(1000.0 / msq, 2),
                                         "loop_form": "persistent" if form == 1 else "graph",
                                         "hbm_frac": round(chunk_bytes(d) / (msq * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        print(f"[bench] persistent variant: {msq:.4f} ms/chunk (form {form})", file=sys.stderr, flush=True)

    if "capsule" in todo:
        # execution-state capsules of the 816-token prefix: save (async kernels), restore
        # (waits for the stream, reads the header, copies back) and fork at batch 1 -> slot 0
        ec = fm.ActionExpert.from_dims(d)
        ec.set_weights(w)
        ec.set_prefix_kv(kp, vp)
        nbytes = ec._lib.phyai_capsule_bytes(ec._h)
        cap = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        capp = ctypes.c_void_p(cap.data_ptr())
        for _ in range(max(args.warmup, 1)):
            ec._check(ec._lib.phyai_capsule_save(ec._h, capp, nbytes))
            ec._check(ec._lib.phyai_capsule_restore(ec._h, capp, nbytes))
        torch.cuda.synchronize()
        reps = max(args.steps, 10)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            ec._check(ec._lib.phyai_capsule_save(ec._h, capp, nbytes))
        b.record()
        torch.cuda.synchronize()
        ms_save = a.elapsed_time(b) / reps
        t0 = time.perf_counter()
        for _ in range(reps):
            ec._check(ec._lib.phyai_capsule_restore(ec._h, capp, nbytes))
        torch.cuda.synchronize()
        ms_restore = (time.perf_counter() - t0) * 1e3 / reps
        ec.close()
        del cap
        moved = 2 * (nbytes - 256)  # payload read once and written once
        variants["capsule_816_batch1"] = {
            "capsule_bytes": int(nbytes), "ms_per_save": round(ms_save, 4), "ms_per_restore": round(ms_restore, 4),
            "save_hbm_frac": round(moved / (ms_save * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        print(f"[bench] capsule variant: save {ms_save:.4f} ms, restore {ms_restore:.4f} ms for {nbytes} B",
              file=sys.stderr, flush=True)

    if "b32" in todo:
        # batch 32: each sample its own prefix and noise; bf16 MFMA GEMMs
        d32 = synth.CONFIGS["pi05_b32"]
        inp32 = synth.make_expert_inputs(d32, 0)
        k32 = torch.from_numpy(inp32["k_pre"]).cuda().to(torch.bfloat16).contiguous()
        v32 = torch.from_numpy(inp32["v_pre"]).cuda().to(torch.bfloat16).contiguous()
        n32 = torch.from_numpy(inp32["noise"]).cuda().contiguous()
        del inp32
        e32 = fm.ActionExpert.from_dims(d32)
        e32.set_weights(w)
        e32.set_prefix_kv(k32, v32)
        e32.set_timestep_tables(schedule(d.n_steps))
        o32 = torch.empty_like(n32)
        ms32 = time_chunks(e32, n32, o32, max(5, args.steps // 5), max(2, args.warmup // 5), torch)
        kt32 = kernel_times(e32, max(10, args.kernel_reps // 10), torch)
        e32.close()
        fl = batch_flops(d32)
        gemm_fl = {"qkv": 2 * 1600 * d32.qkv_dim * d32.width, "o_proj": 2 * 1600 * d32.width * d32.n_q_heads * d32.head_dim,
                   "gate_up": 2 * 1600 * 2 * d32.mlp_dim * d32.width, "down": 2 * 1600 * d32.mlp_dim * d32.width}
        dom32 = max(gemm_fl, key=lambda k: kt32[k])
        variants["bf16_batch32"] = {
            "ms_per_batch_chunk": round(ms32, 4), "chunks_per_s": round(32 * 1000.0 / ms32, 2),
            "algorithmic_tflop": round(fl / 1e12, 3),
            "mfma_frac": round(fl / (ms32 * 1e-3) / MFMA_PEAK_TFLOPS / 1e12, 4),
            "kernel_us": {k: round(v, 2) for k, v in kt32.items()},
            "roofline": {"kernel": dom32, "bound": "mfma", "unit": "TFLOP/s",
                         "achieved": round(gemm_fl[dom32] / (kt32[dom32] * 1e-6) / 1e12, 1),
                         "peak": MFMA_PEAK_TFLOPS,
                         "frac": round(gemm_fl[dom32] / (kt32[dom32] * 1e-6) / 1e12 / MFMA_PEAK_TFLOPS, 4)},
        }
        print(f"[bench] batch-32 variant: {ms32:.3f} ms per batch chunk, {32000.0 / ms32:.1f} chunks/s",
              file=sys.stderr, flush=True)

    if "wam" in todo:
        # joint video/action denoiser, guided pair: 28 layers, width 2048, 4096 + 32 tokens, 8 steps
        dw = synth.WAM_CONFIGS["wam"]
        wdev = synth.wam_device_inputs(dw, 0)
        jd = fm.JointDenoiser.from_dims(dw)
        jd.set_weights(wdev)
        jd.set_conditions(wdev["c_cond"], wdev["c_uncond"], dw.guidance)
        jd.set_timestep_tables(schedule(dw.n_steps))
        ol, oa = torch.empty_like(wdev["z_lat"]), torch.empty_like(wdev["z_act"])
        for _ in range(2):
            jd.denoise(wdev["z_lat"], wdev["z_act"], ol, oa)
        torch.cuda.synchronize()
        nw = max(3, args.steps // 10)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(nw):
            jd.denoise(wdev["z_lat"], wdev["z_act"], ol, oa)
        b.record()
        torch.cuda.synchronize()
        msw = a.elapsed_time(b) / nw
        ktw = kernel_times(jd, 5, torch)
        jd.close()
        if "wam_unipc" in todo:
            # the same chunk with the UniPC solver (predictor order 2, corrector on)
            ju = fm.JointDenoiser.from_dims(dw, solver_order=2)
            ju.set_weights(wdev)
            ju.set_conditions(wdev["c_cond"], wdev["c_uncond"], dw.guidance)
            ju.set_timestep_tables(schedule(dw.n_steps))
            for _ in range(2):
                ju.denoise(wdev["z_lat"], wdev["z_act"], ol, oa)
            torch.cuda.synchronize()
            a.record()
            for _ in range(nw):
                ju.denoise(wdev["z_lat"], wdev["z_act"], ol, oa)
            b.record()
            torch.cuda.synchronize()
            msu = a.elapsed_time(b) / nw
            ktu = kernel_times(ju, 5, torch, names=("out_euler",))
            ju.close()
            variants["wam_joint_cfg_pair_unipc2"] = {
                "ms_per_chunk": round(msu, 3), "chunks_per_s": round(1000.0 / msu, 3),
                "out_update_us": round(ktu["out_euler"], 1), "out_update_us_euler": round(ktw["out_euler"], 1),
                "mfma_frac": round(wam_flops(dw) / (msu * 1e-3) / MFMA_PEAK_TFLOPS / 1e12, 4)}
            print(f"[bench] joint UniPC variant: {msu:.2f} ms per chunk", file=sys.stderr, flush=True)
        del wdev
        flw = wam_flops(dw)
        kfl = wam_kernel_flops(dw)
        domw = max(kfl, key=lambda k: ktw[k])
        variants["wam_joint_cfg_pair"] = {
            "ms_per_chunk": round(msw, 3), "chunks_per_s": round(1000.0 / msw, 3),
            "algorithmic_tflop": round(flw / 1e12, 2),
            "mfma_frac": round(flw / (msw * 1e-3) / MFMA_PEAK_TFLOPS / 1e12, 4),
            "kernel_us": {k: round(v, 1) for k, v in ktw.items()},
            "kernel_mfma_frac": {k: round(kfl[k] / (ktw[k] * 1e-6) / 1e12 / MFMA_PEAK_TFLOPS, 4) for k in kfl},
            "roofline": {"kernel": domw, "bound": "mfma", "unit": "TFLOP/s",
                         "achieved": round(kfl[domw] / (ktw[domw] * 1e-6) / 1e12, 1), "peak": MFMA_PEAK_TFLOPS,
                         "frac": round(kfl[domw] / (ktw[domw] * 1e-6) / 1e12 / MFMA_PEAK_TFLOPS, 4)},
            "config": {"layers": dw.n_layers, "width": dw.width, "heads": f"{dw.n_heads} x {dw.head_dim}",
                       "mlp": dw.mlp_dim, "tokens": f"{dw.latent_tokens}x{dw.latent_dim} latent + "
                                                    f"{dw.action_tokens}x{dw.action_dim} action",
                       "branches": 2, "guidance": dw.guidance, "euler_steps": dw.n_steps},
        }
        print(f"[bench] joint variant: {msw:.2f} ms per chunk", file=sys.stderr, flush=True)

    if "wam_tp4" in todo:
        # the shapes of one rank of a 4-way tensor-parallel split of each guidance branch: 4 of
        # the 16 heads and a quarter of the MLP (column-parallel QKV and gate/up, row-parallel
        # O and down) over all 4128 tokens, both branches as one batch of two (the matching
        # rank pair); the all-reduces after O and down are not run
        dr = dataclasses.replace(synth.WAM_CONFIGS["wam"], n_heads=4, mlp_dim=2048)
        rdev = synth.wam_device_inputs(dr, 0)
        jr = fm.JointDenoiser.from_dims(dr)
        jr.set_weights(rdev)
        jr.set_conditions(rdev["c_cond"], rdev["c_uncond"], dr.guidance)
        jr.set_timestep_tables(schedule(dr.n_steps))
        ol, oa = torch.empty_like(rdev["z_lat"]), torch.empty_like(rdev["z_act"])
        for _ in range(2):
            jr.denoise(rdev["z_lat"], rdev["z_act"], ol, oa)
        torch.cuda.synchronize()
        nr = max(3, args.steps // 10)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(nr):
            jr.denoise(rdev["z_lat"], rdev["z_act"], ol, oa)
        b.record()
        torch.cuda.synchronize()
        msr = a.elapsed_time(b) / nr
        ktr = kernel_times(jr, 5, torch)
        jr.close()
        del rdev
        flr = wam_flops(dr)
        variants["wam_tp4_rank_shard"] = {
            "ms_per_chunk": round(msr, 3), "algorithmic_tflop": round(flr / 1e12, 2),
            "mfma_frac": round(flr / (msr * 1e-3) / MFMA_PEAK_TFLOPS / 1e12, 4),
            "kernel_us": {k: round(v, 1) for k, v in ktr.items()},
            "note": "compute of the matching conditional / unconditional rank pair of a 4-way tensor-parallel "
                    "split of each branch, run as one batch of two; all-reduces and the CFG exchange not run"}
        print(f"[bench] joint TP-4 rank shard: {msr:.2f} ms per chunk", file=sys.stderr, flush=True)

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on one chunk ...", file=sys.stderr, flush=True)
        cpu = cpu_baseline(d, inputs)

    cb = chunk_bytes(d)
    line = {
        "metric": METRIC,
        "value": round(ms_per_chunk, 4),
        "unit": "ms/chunk",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_chunk, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,0.02) weights, N(0,1) prefix K/V and noise)",
        "config": {"workload": "pi0.5-shaped action expert denoise loop, batch 1", "layers": d.n_layers,
                   "width": d.width, "heads": f"{d.n_q_heads}q/{d.n_kv_heads}kv x {d.head_dim}",
                   "mlp": d.mlp_dim, "prefix_len": d.prefix_len, "chunk": f"{d.chunk_len}x{d.action_dim}",
                   "euler_steps": d.n_steps, "batch": 1},
        "chunks_per_s": round(1000.0 / ms_per_chunk, 2),
        "latency_ms": {"median": round(statistics.median(lat), 4), "mean": round(statistics.mean(lat), 4),
                       "p99": round(p99, 4)},
        "chunk_hbm": {"algorithmic_bytes": cb, "achieved_GBs": round(cb / (ms_per_chunk * 1e-3) / 1e9, 1),
                      "frac": round(cb / (ms_per_chunk * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
        "kernel_us": {k: round(v, 3) for k, v in inloop_us.items()},
        "kernel_us_share_of_chunk": {k: round(share[k] / 1000.0 / ms_per_chunk, 4) for k in KERNELS},
        "kernel_us_inloop_raw": {k: round(v, 3) for k, v in raw_us.items()},
        "loop_with_marks_ms": round(loop_ms, 4),
        "event_cost_us": round(ev_us, 3),
        "kernel_us_cache_warm": {k: round(v, 3) for k, v in per_launch_us.items()},
        "roofline": {"kernel": dominant, "bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": stage_traffic(dominant),
                     "algorithmic_bytes_per_launch": abytes[dominant],
                     "avg_launch_us": round(inloop_us[dominant], 3),
                     "timing": "in-loop: HIP events between the launches of the loop on its stream, less the mean "
                               "cost of an event (marked loop time - graph loop time) / events, mean over "
                               f"{stage_reps} runs x {per_chunk[dominant]} launches"
                               + (" (attention launch + split merge)" if dominant == "attention" else ""),
                     "avg_launch_us_cache_warm": round(per_launch_us[dominant] + (per_launch_us["attn_merge"]
                                                       if dominant == "attention" else 0.0), 3)},
        "output_finite": finite,
        "variants": variants,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
