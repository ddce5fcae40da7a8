#!/usr/bin/env python3
"""Benchmark of the batched decode step on one MI355X: aggregate decode tokens/s
versus batch width B, with the step's and the dominant kernel's fraction of
the HBM roofline, and the CPU oracle timed beside it.

Workload (default): the Mistral-7B shape in bf16 (d=4096, 32 layers, 32 query
/ 8 KV heads of 128, FFN 14336, vocab 32000) with seeded synthetic weights
N(0, 0.02); 64 lanes whose KV lengths are uniform in [128, 4096] (seed 2),
holding synthetic post-rotary K/V ~ N(0, 1) (seed 3); one decode step over the
first B lanes, one new token per lane (seed 1).  Each timed step rewrites the
same slot of every lane (the lanes are rolled back to their lengths before
each step), so every step does the same work.  Inputs are resident in HBM
before timing starts.

Prints ONE JSON line.  Only one GPU: --gpus above 1 exits with a message.
"""
from __future__ import annotations

import argparse
import gc
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# Source files of each kernel class: stored counter readings apply only while these are unchanged.
KERNEL_SOURCES = {
    "attention": ["cbd_attn.hip", "cbd_internal.h"],
    "attn_combine": ["cbd_attn.hip", "cbd_internal.h"],
    "gemm_qkv": ["cbd_gemm.hip", "cbd_internal.h"], "gemm_o": ["cbd_gemm.hip", "cbd_internal.h"],
    "gemm_gu": ["cbd_gemm.hip", "cbd_internal.h"], "gemm_down": ["cbd_gemm.hip", "cbd_internal.h"],
    "gemm_head": ["cbd_gemm.hip", "cbd_internal.h"], "rmsnorm": ["cbd_misc.hip", "cbd_internal.h"],
}


def kernel_source_hash(cls: str) -> str:
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES.get(cls, []):
        with open(os.path.join(ROOT, "continuous_batching_decode_step_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def stored_traffic(cls: str, B: int):
    """HBM bytes per launch of `cls` at batch B from profiles/traffic.md (rocprofv3 FETCH_SIZE and
    WRITE_SIZE runs scaled by a plain copy), or None if absent or the kernel source changed since."""
    path = os.path.join(ROOT, "profiles", "traffic.md")
    if not os.path.exists(path):
        return None
    want = kernel_source_hash(cls)
    with open(path) as f:
        for line in f:
            cells = [c.strip() for c in line.strip().strip("|").split("|")]
            if len(cells) >= 8 and cells[0] == cls and cells[1] == str(B) and cells[2] == want:
                try:
                    return float(cells[7])
                except ValueError:
                    return None
    return None


GEMM_CLASSES = ("gemm_qkv", "gemm_o", "gemm_gu", "gemm_down", "gemm_head")


def measure(eng, lanes, lens, toks, B, steps, warmup, cfg, rf, stream):
    """Time `steps` decode steps over the first B lanes (each step rewrites the same slot of every lane),
    each step with its own event pair and the whole run with one more, then a second pass with events
    around every kernel class.  Returns (sweep row, per-class summary).

    ms_per_step is the whole run's time / steps (what the headline value uses); median_ms and best_ms
    are over the per-step intervals, which leave out any gap between steps (a host stall shows up as
    ms_per_step above median_ms).  kernel_sum_ms is the per-class kernel time of the profiled pass per
    step, so ms_per_step - kernel_sum_ms is the time the GPU spent without a kernel of the step."""
    import torch
    pos0 = lens[:B].astype(np.int32)
    lanes_b, toks_b = lanes[:B], toks[:B]

    def step():
        for b in range(B):
            eng.arena.lane_truncate(lanes_b[b], int(pos0[b]))
        eng.step(lanes_b, pos0.copy(), toks_b)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    # Python's cyclic garbage collector off while steps are timed (as timeit
    # does): a collection pass over this process's large heap has stalled the
    # host for tens of ms, longer than the four steps it may run ahead, and the
    # GPU then idles between steps.
    gc_was = gc.isenabled()
    gc.disable()
    ev = lambda: torch.cuda.Event(enable_timing=True)
    e0, e1 = ev(), ev()
    per_step = [(ev(), ev()) for _ in range(steps)]
    w0 = time.perf_counter()
    e0.record(stream)
    for a, b in per_step:
        a.record(stream)
        step()
        b.record(stream)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    if gc_was:
        gc.enable()
    ms = e0.elapsed_time(e1) / steps
    each = sorted(a.elapsed_time(b) for a, b in per_step)
    pos = [int(x) for x in lens[:B]]
    t_roof = rf.roofline_time_s(cfg, pos)
    eng.model.profile_reset()
    eng.model.profile_enable(True)
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    prof = eng.model.profile_read()
    eng.model.profile_enable(False)
    per = rf.per_class_summary(cfg, prof, pos)
    gemm_ms = sum(per[k]["total_ms"] for k in GEMM_CLASSES if k in per) / steps
    gemm_flops = sum(rf.kernel_flops(cfg, k, pos) * (1 if k == "gemm_head" else cfg.n_layers) for k in GEMM_CLASSES)
    kernel_ms = sum(v["total_ms"] for v in per.values()) / steps
    row = {"B": B, "tok_s": B / (ms * 1e-3), "ms_per_step": ms, "median_ms": float(np.median(each)),
           "best_ms": each[0], "worst_ms": each[-1], "kernel_sum_ms": kernel_ms,
           "wall_ms_per_step": wall * 1e3 / steps,
           "step_alg_GB": rf.step_bytes(cfg, pos) / 1e9, "roofline_tok_s": B / t_roof,
           "roofline_frac": t_roof / (ms * 1e-3),
           "gemm_mfma_util": gemm_flops / (gemm_ms * 1e-3) / (rf.MFMA_PEAK_TFLOPS["bf16"] * 1e12),
           "kernels": {k: {"avg_us": round(v["avg_us"], 2), "share": round(v["total_ms"] / max(
               1e-9, sum(x["total_ms"] for x in per.values())), 4),
               "GBs": None if v["achieved_GBs"] is None else round(v["achieved_GBs"], 1)}
               for k, v in per.items()}}
    return row, per


def wide_leg(cfg, dw, args, rf, log):
    """B = 256 and B = 512 with KV U[128,4096] (the headline distribution): tokens/s and the
    projections' bf16 MFMA utilisation (GEMM flops / summed GEMM kernel time / 2.5 PFLOP/s).
    The 512 lanes share one paged KV pool sized to the blocks they hold (~146 GB; an arena
    with every lane at the longest length would need 275 GB)."""
    import gc
    import torch
    import synth
    from continuous_batching_decode_step_amd.driver import Engine
    out = []
    n, hi = 512, 4096
    lens = synth.kv_lengths(n, hi=hi)
    toks = synth.step_tokens(cfg, n)
    blocks = int(((lens + 1 + 63) // 64).sum())  # each lane's blocks, slot len_b included
    eng = Engine(cfg, dw, n, int(lens.max()) + 1, max_batch=n, kv_blocks=blocks)
    eng.model.set_variant(args.variant)
    eng.model.set_graph_replay(args.graph)
    lanes = [eng.arena.lane_alloc() for _ in range(n)]
    t0 = time.time()
    for b in range(n):
        k, v = synth.lane_kv_bf16(cfg, b, int(lens[b]))
        eng.arena.kv_import(lanes[b], int(lens[b]), k, v, eng.stream)
        if (b + 1) % 128 == 0 and b + 1 < n:
            log("wide: KV of %d lanes loaded (%.1fs)" % (b + 1, time.time() - t0))
    torch.cuda.synchronize()
    log("wide: KV of %d lanes (%d blocks, %.1f GB) loaded in %.1fs" % (
        n, blocks, eng.arena_mem.numel() / 1e9, time.time() - t0))
    for B in (256, 512):
        row, _ = measure(eng, lanes, lens, toks, B, max(3, args.steps // 2), max(1, args.warmup), cfg, rf,
                         torch.cuda.current_stream())
        row["kv_lengths"] = "U[128,%d]" % hi
        log("wide B=%3d  %8.1f tok/s  %.3f ms/step  roofline %.3f  projections at %.1f%% of bf16 MFMA peak" % (
            B, row["tok_s"], row["ms_per_step"], row["roofline_frac"], 100 * row["gemm_mfma_util"]))
        out.append(row)
    del eng
    gc.collect()
    torch.cuda.empty_cache()
    return out


def prefill_leg(cfg, dw, args, rf, log, n=8, count=512):
    """Batched chunked prefill at the 7B shape: n lanes each take a count-token prompt (seeded tokens) from
    an empty cache in one cbd_prefill_batch call of n * count rows.  Reports prompt tokens/s and the
    projections' bf16 MFMA utilisation (GEMM flops / summed GEMM kernel time / 2.5 PFLOP/s)."""
    import gc
    import torch
    import synth
    from continuous_batching_decode_step_amd.driver import Engine
    R = n * count
    prompts = [synth.uniform_int(1, 1000 + b, count, 0, cfg.vocab - 1) for b in range(n)]
    toks = np.concatenate(prompts).astype(np.int32)
    eng = Engine(cfg, dw, n, count, max_batch=R)
    eng.model.set_variant(args.variant)
    eng.model.set_graph_replay(args.graph)
    lanes = [eng.arena.lane_alloc() for _ in range(n)]
    stream = torch.cuda.current_stream()

    def call():
        for l in lanes:
            eng.arena.lane_clear(l)
        pos = np.zeros(n, np.int32)
        eng.model.prefill_batch(eng.arena, lanes, pos, [count] * n, toks, eng.logits, eng.argmax, eng.ws,
                                eng.ws_bytes, eng.stream)

    call()
    torch.cuda.synchronize()
    reps = 3
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    eng.model.profile_reset()
    eng.model.profile_enable(True)
    call()
    torch.cuda.synchronize()
    prof = eng.model.profile_read()
    eng.model.profile_enable(False)
    rows = [t for _ in range(n) for t in range(count)]      # every row's position
    per = rf.per_class_summary(cfg, prof, rows)
    gemm_ms = sum(per[k]["total_ms"] for k in GEMM_CLASSES if k in per and k != "gemm_head")
    gemm_flops = sum(rf.kernel_flops(cfg, k, rows) * cfg.n_layers for k in GEMM_CLASSES if k != "gemm_head")
    out = {"lanes": n, "prompt_tokens": count, "rows": R, "ms_per_call": round(ms, 3),
           "prompt_tok_s": round(R / (ms * 1e-3), 1),
           "gemm_mfma_util": round(gemm_flops / (gemm_ms * 1e-3) / (rf.MFMA_PEAK_TFLOPS["bf16"] * 1e12), 4),
           "kernels_ms": {k: round(v["total_ms"], 3) for k, v in per.items()}}
    log("prefill %d lanes x %d tokens: %.1f ms per call, %.0f prompt tok/s, layer projections at %.1f%% of "
        "bf16 MFMA peak" % (n, count, ms, out["prompt_tok_s"], 100 * out["gemm_mfma_util"]))
    del eng
    gc.collect()
    torch.cuda.empty_cache()
    return out


def clone_leg(cfg, dw, log, n=4096, reps=5):
    """Prefix reuse at the 7B shape: cbd_lane_clone of an n-position lane (whole 64-position blocks of
    every layer, K and V, one copy kernel).  Reports the time per clone and the HBM rate of the copy
    (every byte read once and written once) against 8 TB/s."""
    import gc
    import torch
    import synth
    import continuous_batching_decode_step_amd as cbd
    from continuous_batching_decode_step_amd.driver import Engine
    eng = Engine(cfg, dw, 2, n, max_batch=1)
    a, b = eng.arena.lane_alloc(), eng.arena.lane_alloc()
    k, v = synth.lane_kv_bf16(cfg, 0, n)
    eng.arena.kv_import(a, n, k, v, eng.stream)
    eng.arena.lane_clone(a, b, n, eng.stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        eng.arena.lane_clone(a, b, n, eng.stream)  # synchronous
    ms = (time.perf_counter() - t0) * 1e3 / reps
    moved = 2 * ((n + 63) // 64) * cbd.arena_block_bytes(cfg)  # read + write
    out = {"positions": n, "bytes_moved": moved, "ms_per_clone": round(ms, 3),
           "GBs": round(moved / (ms * 1e-3) / 1e9, 1), "frac_of_hbm_peak": round(moved / (ms * 1e-3) / 8e12, 4)}
    log("clone of a %d-position lane: %.3f ms, %.0f GB/s (%.1f%% of 8 TB/s; wall clock, host sync included)" % (
        n, ms, out["GBs"], 100 * out["frac_of_hbm_peak"]))
    # span eviction: drop [1024, 2048) of the clone; the 2048 positions after it move down (keys rotated)
    b0, e0 = 1024, 2048
    ev = []
    for _ in range(reps):
        eng.arena.lane_clone(a, b, n, eng.stream)
        t0 = time.perf_counter()
        eng.arena.lane_evict_span(b, b0, e0, eng.stream)  # synchronous
        ev.append((time.perf_counter() - t0) * 1e3)
    ems = float(np.median(ev))
    per_pos = cbd.arena_block_bytes(cfg) // 64
    moved_e = 2 * (n - e0) * per_pos  # the moved entries read once and written once
    out["evict_span"] = {"positions": n, "span": [b0, e0], "moved_positions": n - e0, "bytes_moved": moved_e,
                         "ms": round(ems, 3), "GBs": round(moved_e / (ems * 1e-3) / 1e9, 1)}
    log("span eviction [%d, %d) of a %d-position lane: %.3f ms, %.0f GB/s of moved entries (through staging)" % (
        b0, e0, n, ems, out["evict_span"]["GBs"]))
    del eng
    gc.collect()
    torch.cuda.empty_cache()
    return out


def q8_leg(args, rf, log):
    """The pages' own benchmark shape: SmolLM2-135M with Q8_0 weights, lanes holding 16 positions
    (the prompt length of that benchmark; synthetic f32 K/V, seed 3), one decode step per lane, at
    B in {1, 64, 256, 512, 960}.  Context only (their figures come from a CPU)."""
    import gc
    import torch
    import synth
    import continuous_batching_decode_step_amd as cbd
    from continuous_batching_decode_step_amd.driver import Engine
    cfg = synth.SMOL135M_Q8
    dw = cbd.upload_weights(synth.make_weights(cfg))
    batches = [int(x) for x in args.q8_batches.split(",")]
    Bmax, ctx = max(batches), 16
    lens = np.full(Bmax, ctx, dtype=np.int64)
    toks = synth.step_tokens(cfg, Bmax)
    eng = Engine(cfg, dw, Bmax, ctx + 1, max_batch=Bmax)
    eng.model.set_graph_replay(args.graph)
    lanes = [eng.arena.lane_alloc() for _ in range(Bmax)]
    for b in range(Bmax):
        k, v = synth.lane_kv_f32(cfg, b, ctx)
        eng.arena.kv_import(lanes[b], ctx, k, v, eng.stream)
    torch.cuda.synchronize()
    out = []
    for B in batches:
        row, _ = measure(eng, lanes, lens, toks, B, args.steps, args.warmup, cfg, rf, torch.cuda.current_stream())
        log("q8-135m B=%3d  %9.1f tok/s  %.3f ms/step" % (B, row["tok_s"], row["ms_per_step"]))
        out.append({"B": B, "tok_s": round(row["tok_s"], 1), "ms_per_step": round(row["ms_per_step"], 4),
                    "roofline_frac": round(row["roofline_frac"], 4)})
    del eng, dw
    gc.collect()
    torch.cuda.empty_cache()
    return out


def trace_leg(cfg, dw, rf, log):
    """Continuous batching at the 7B shape: 8 lanes, 64 seeded jobs with Poisson
    arrivals (mean gap 4 steps), prompts U[32, 1024] fed one token per step, U[16, 256] new tokens
    (seed 4); greedy tokens fed back, so every step waits for its argmax.  Reports generated
    tokens per wall-clock second and the per-step roofline times summed over the trace."""
    import torch
    import synth
    from continuous_batching_decode_step_amd.driver import Engine, run_trace
    jobs = synth.make_trace(cfg)
    max_seq = max(len(j.prompt) + j.max_new_tokens for j in jobs)
    eng = Engine(cfg, dw, 8, max_seq, max_batch=8)
    warm = synth.make_trace(cfg, n_jobs=2, seed=5)  # graph capture of the small B values
    run_trace(eng, warm, 8)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    out, st = run_trace(eng, jobs, 8, record_positions=True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    t_roof = sum(rf.roofline_time_s(cfg, [int(x) for x in p]) for p in st.positions)
    res = {"jobs": len(jobs), "lanes": 8, "steps": st.steps, "idle_steps": st.idle_steps,
           "lane_steps": st.lane_steps, "generated": st.generated, "wall_s": round(wall, 3),
           "tok_s": round(st.generated / wall, 1), "lane_steps_per_s": round(st.lane_steps / wall, 1),
           "mean_occupancy": round(float(np.mean(st.occupancy)), 3),
           "roofline_frac": round(t_roof / wall, 4)}
    log("trace C5: %s" % res)
    del eng
    return res, out


def sched_trace_leg(cfg, dw, rf, log, c5_out=None, prefill_cap=1024):
    """The C5 jobs through the continuous-batching scheduler (cbd_sched over the decode path): the same
    8 lanes and arrivals (in ticks), but whole prompts prefilled in batched calls (up to prefill_cap
    prompt tokens per tick) instead of one token per step.  Reports generated tokens per wall-clock
    second, ticks, occupancy, and whether every job's tokens equal those of the one-token-per-step
    trace."""
    import torch
    import synth
    from continuous_batching_decode_step_amd.driver import Engine, run_sched_trace
    jobs = synth.make_trace(cfg)
    max_seq = max(len(j.prompt) + j.max_new_tokens for j in jobs)
    rows = max(8, prefill_cap, max(len(j.prompt) for j in jobs))
    eng = Engine(cfg, dw, 8, max_seq, max_batch=rows)
    run_sched_trace(eng, synth.make_trace(cfg, n_jobs=2, seed=5), 8, prefill_cap)  # graph capture warm-up
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    out, tel, idle = run_sched_trace(eng, jobs, 8, prefill_cap)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gen = sum(len(v) for v in out.values())
    res = {"jobs": len(jobs), "lanes": 8, "prefill_tokens_per_tick": prefill_cap, "ticks": tel["ticks"],
           "idle_ticks": idle, "decode_ticks": tel["decode_ticks"], "generated": gen,
           "prompt_tokens": tel["prefill_tokens"], "wall_s": round(wall, 3), "tok_s": round(gen / wall, 1),
           "mean_decode_occupancy": round(tel["occupancy_avg"], 3),
           "tokens_equal_c5": None if c5_out is None else all(out[k] == c5_out[k] for k in c5_out)}
    log("scheduler trace: %s" % res)
    del eng
    return res


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--batches", default="1,2,4,8,16,32,64", help="B sweep; the last is the headline B")
    ap.add_argument("--lanes", type=int, default=64)
    ap.add_argument("--kv-max", type=int, default=4096,
                    help="KV lengths are uniform in [128, KV_MAX] (seed 2)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="budget of the CPU oracle sample")
    ap.add_argument("--prewarm-s", type=float, default=1.0,
                    help="untimed decode steps at the widest B for this long before the sweep (a fresh "
                         "process's first timed steps have shown one-off stalls of ~17 ms)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--variant", type=int, default=0, choices=[0, 1, 2, 3],
                    help="projection kernel family (cbd_set_variant): 0 automatic, 1 split-K, 2 wide panels, 3 dense tiles")
    ap.add_argument("--graph", action="store_true",
                    help="replay each decode step as a captured HIP graph (cbd_set_graph_replay) instead of "
                         "plain launches")
    ap.add_argument("--no-q8", action="store_true",
                    help="skip the SmolLM2-135M Q8_0 leg (decode steps at 16-position contexts, B = 1..960)")
    ap.add_argument("--q8-only", action="store_true",
                    help="run the SmolLM2-135M Q8_0 leg alone and print its rows as the JSON line (for profiling "
                         "that leg; not the headline)")
    ap.add_argument("--q8-batches", default="1,64,256,512,960", help="B values of the SmolLM2-135M Q8_0 leg")
    ap.add_argument("--no-wide", action="store_true",
                    help="skip the wide-batch leg (B = 256 and 512 with KV U[128,4096], one paged pool) "
                         "that reports the projections' bf16 MFMA utilisation")
    ap.add_argument("--no-prefill", action="store_true",
                    help="skip the batched prefill leg (8 lanes x 512-token prompts in one call) and the prefix "
                         "clone leg (a 4096-position lane)")
    ap.add_argument("--no-trace", action="store_true",
                    help="skip the continuous-batching trace legs (8 lanes, 64 Poisson-arriving jobs: one token per "
                         "step, then through the scheduler with batched prefill; ~60 s)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="end with one device-to-device copy of MIB MiB (a known-size kernel for "
                         "scaling HBM byte counters)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(--gpus %d, WORLD_SIZE %d requested)" % (args.gpus, world), file=sys.stderr)
        return 2

    import torch
    import synth
    import continuous_batching_decode_step_amd as cbd
    from continuous_batching_decode_step_amd import roofline as rf
    from continuous_batching_decode_step_amd.driver import Engine

    cbd.lib()  # fail loudly if the HIP library is missing
    if args.q8_only:
        print(json.dumps({"context_q8_smollm135m": q8_leg(args, rf, log)}), flush=True)
        return 0
    cfg = synth.MISTRAL7B
    batches = [int(x) for x in args.batches.split(",")]
    n_lanes = max(args.lanes, max(batches))
    t0 = time.time()
    W = synth.make_weights(cfg)
    log("weights generated in %.1fs" % (time.time() - t0))
    dw = cbd.upload_weights(W)
    lens = synth.kv_lengths(n_lanes, hi=args.kv_max)  # U[128, kv_max]
    toks = synth.step_tokens(cfg, n_lanes)
    max_seq = int(lens.max()) + 1
    eng = Engine(cfg, dw, n_lanes, max_seq, max_batch=max(batches))
    eng.model.set_variant(args.variant)
    eng.model.set_graph_replay(args.graph)
    lanes = [eng.arena.lane_alloc() for _ in range(n_lanes)]
    t0 = time.time()
    for b in range(n_lanes):
        k, v = synth.lane_kv_bf16(cfg, b, int(lens[b]))
        eng.arena.kv_import(lanes[b], int(lens[b]), k, v, eng.stream)
    torch.cuda.synchronize()
    log("KV of %d lanes generated and loaded in %.1fs" % (n_lanes, time.time() - t0))

    stream = torch.cuda.current_stream()
    if args.prewarm_s > 0:
        Bw = max(batches)
        pw = lens[:Bw].astype(np.int32)
        t_end = time.perf_counter() + args.prewarm_s
        while time.perf_counter() < t_end:
            for b in range(Bw):
                eng.arena.lane_truncate(lanes[b], int(pw[b]))
            eng.step(lanes[:Bw], pw.copy(), toks[:Bw])
            torch.cuda.synchronize()
    sweep = []
    headline = None
    for B in batches:
        row, per = measure(eng, lanes, lens, toks, B, args.steps, args.warmup, cfg, rf, stream)
        sweep.append(row)
        log("B=%3d  %8.1f tok/s  %.3f ms/step (median %.3f, best %.3f, kernels %.3f)  roofline %.3f  %s" % (
            B, row["tok_s"], row["ms_per_step"], row["median_ms"], row["best_ms"], row["kernel_sum_ms"],
            row["roofline_frac"],
            " ".join("%s=%.1fus/%sGB/s" % (k, v["avg_us"], v["GBs"]) for k, v in row["kernels"].items())))
        headline = (B, row["ms_per_step"], per, [int(x) for x in lens[:B]])

    B, ms, per, pos = headline
    t_roof_step = rf.roofline_time_s(cfg, pos)
    dom = max((k for k in per if per[k]["alg_bytes"] > 0), key=lambda k: per[k]["total_ms"])
    d = per[dom]
    achieved = d["achieved_GBs"]
    traffic = stored_traffic(dom, B)
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": rf.HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / rf.HBM_PEAK_GBS, 4), "traffic": traffic, "kernel": dom,
            "alg_bytes_per_launch": d["alg_bytes"], "avg_launch_us": round(d["avg_us"], 2),
            "launches": d["launches"],
            # the whole step against the same peak: (weight + KV bytes) / 8 TB/s over the step time
            "step_frac": round(t_roof_step / (ms * 1e-3), 4)}

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        M = oracle.Model(W)
        done, t_cpu = 0, 0.0
        for b in range(n_lanes):
            k, v = synth.lane_kv_bf16(cfg, b, int(lens[b]))  # regenerated, not timed
            lane = M.lane(int(lens[b]) + 1)
            lane.set_kv(synth.bf16_to_f32(k), synth.bf16_to_f32(v))
            t1 = time.perf_counter()
            M.step(lane, int(toks[b]))
            t_cpu += time.perf_counter() - t1
            done += 1
            del lane
            if t_cpu >= args.cpu_seconds:
                break
        cpu = {"value": round(done / t_cpu, 4), "unit": "tokens/s", "cores": oracle.num_threads(), "kind": "oracle",
               "sample": "%d lane-steps of the same workload (lanes 0..%d at their KV lengths, one decode step "
                         "each, serial CPU oracle on bf16 weights: sums in double, values stored in f32), %.1f s" % (done, done - 1, t_cpu)}
        log("cpu oracle: %s" % cpu)

    q8 = None
    if not args.no_q8:
        q8 = q8_leg(args, rf, log)

    wide = None
    if not args.no_wide:
        del eng
        import gc
        gc.collect()
        torch.cuda.empty_cache()
        wide = wide_leg(cfg, dw, args, rf, log)

    prefill = clone = None
    if not args.no_prefill:
        prefill = prefill_leg(cfg, dw, args, rf, log)
        clone = clone_leg(cfg, dw, log)

    trace = sched = None
    if not args.no_trace:
        trace, c5_out = trace_leg(cfg, dw, rf, log)
        sched = sched_trace_leg(cfg, dw, rf, log, c5_out)

    if args.calibrate_copy > 0:
        n = args.calibrate_copy << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log("calibration copy: %d bytes read and written" % n)
        del src, dst

    out = {
        "metric": "aggregate decode tokens/s vs batch B; % HBM roofline",
        "value": round(B / (ms * 1e-3), 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "mistral-7b-shape bf16 decode step, ragged KV lengths U[128,%d] (seed 2), "
                               "one token per lane" % args.kv_max, "batch": B, "lanes": n_lanes, "d": cfg.d,
                   "layers": cfg.n_layers, "heads": "%d/%d" % (cfg.n_heads, cfg.n_kv_heads),
                   "head_dim": cfg.head_dim, "ffn": cfg.ffn, "vocab": cfg.vocab,
                   "mean_kv_len": float(np.mean(lens[:B])), "parallelism": "single GPU"},
        "step_roofline_frac": round(sweep[-1]["roofline_frac"], 4),
        "roofline": roof,
        "cpu_baseline": cpu,
        "sweep": [{k: (round(v, 4) if isinstance(v, float) else v) for k, v in r.items()} for r in sweep],
        "context_q8_smollm135m": q8,
        "context_q8_smollm135m_precision": None if q8 is None else (
            "Q8_0 weights (int8 blocks of 32, binary16 scales) dequantised to binary16 in registers; "
            "activations rounded to binary16 at the projections (the matrix cores' f16 operands), "
            "f32 accumulation, residual stream and K/V in f32"),
        "wide": None if wide is None else [{k: (round(v, 4) if isinstance(v, float) else v) for k, v in r.items()}
                                           for r in wide],
        "prefill": prefill,
        "clone": clone,
        "trace_c5": trace,
        "sched_trace": sched,
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
