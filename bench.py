#!/usr/bin/env python3
"""Throughput of the fused GQA exp-sum-div path on one MI355X.

One step = one mga_gqa_forward call (split-KV partial kernel + combine kernel)
over one batch of synthetic input: Q (16, 256, 64), K (16, 64, 4096),
V (16, 4096, 64) fp16 by default (the tutorial graph at batch 8). Inputs sit
in HBM before timing starts. The timed steps cycle through R copies of the
inputs totalling at least --rotate-bytes (default 1 GiB), so that no step finds
its K/V in the 256 MB Infinity Cache; a same-buffer ("hot") figure is reported
beside it.

Timing follows the profiling protocol on the Mirage pages (16 warm-up
iterations, then many timed iterations between two events, mean per
iteration): the steps are captured once in a HIP graph and replayed, so the
host's launch rate does not limit the measurement; events sit on the stream
the kernels run on. The partial kernel (the dominant one) is timed alone the
same way for the roofline entry.

Prints ONE JSON line. --gpus above 1 is refused: this path runs on one GPU.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
MFMA_FP16_PEAK_TFLOPS = 2516.6  # MI355X dense fp16 MFMA (256 CU x 4096 flop/clk x 2.4 GHz)
KERNEL_SRC = os.path.join(ROOT, "gqa_attention_split_amd", "csrc", "gqa_kernels.hip")


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--config", default="gqa_b16_m256_n4096")
    ap.add_argument("--splits", type=int, default=0, help="0 = the library's policy")
    ap.add_argument("--rotate-bytes", type=float, default=float(1 << 30))
    ap.add_argument("--graph-steps", type=int, default=200, help="steps captured per HIP graph")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="target wall time of the oracle baseline sample (the whole workload "
                         "is repeated until it is reached)")
    ap.add_argument("--mode", choices=("graph", "eager"), default="graph",
                    help="graph: replay captured steps (default); eager: plain launches "
                         "(for counter collection, which sees eager dispatches)")
    ap.add_argument("--pmc-calibrate", action="store_true",
                    help="also run one plain device-to-device copy of known size "
                         "(reference dispatch for FETCH_SIZE / WRITE_SIZE scaling)")
    ap.add_argument("--eager", action="store_true", help="also time without graphs")
    ap.add_argument("--qk-norm", action="store_true",
                    help="time the QK-normalised variant (rms_norm of Q rows and key vectors, "
                         "eps 1e-6) instead of the plain graph")
    ap.add_argument("--boundary", action="store_true",
                    help="time the forward's pieces instead: the partial kernel alone, followed by a "
                         "one-block fill kernel, followed by the combine, and followed by the combine "
                         "reading partials written earlier (one JSON line)")
    ap.add_argument("--sweep-splits", default="",
                    help="comma-separated split counts: time the forward at each (same inputs, "
                         "graph replay) and print one JSON line per count instead of the bench line")
    return ap.parse_args()


def kernel_source_sha() -> str:
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def read_traffic(config: str):
    """Counter-derived HBM bytes per partial-kernel launch, if the committed
    counter summary for this workload was taken on the current kernel source;
    else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_gqa_partial_{config.replace('gqa_', '')}.md")
    try:
        text = open(path).read()
    except OSError:
        return None
    sha = re.search(r"kernel_source_sha256:\s*([0-9a-f]{64})", text)
    cfg = re.search(r"workload:\s*(\S+)", text)
    val = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not (sha and cfg and val) or sha.group(1) != kernel_source_sha() or cfg.group(1) != config:
        return None
    return float(val.group(1))


def time_graph(torch, stream, fn, n_steps, graph_steps, warmup):
    """Capture `graph_steps` calls of fn(i) in one graph, replay to cover n_steps,
    return mean ms per call (events on `stream`)."""
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for i in range(graph_steps):
            fn(i)
    torch.cuda.synchronize()
    g.replay()  # untimed first replay
    torch.cuda.synchronize()
    reps = max(1, math.ceil(n_steps / graph_steps))
    # One event between consecutive replays (no host synchronisation): the
    # whole run and each replay's mean per call.
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    with torch.cuda.stream(stream):
        ev[0].record(stream)
        for r in range(reps):
            g.replay()
            ev[r + 1].record(stream)
    ev[-1].synchronize()
    per_replay = [ev[r].elapsed_time(ev[r + 1]) / graph_steps for r in range(reps)]
    return ev[0].elapsed_time(ev[-1]) / (reps * graph_steps), reps * graph_steps, per_replay


def gpu_clocks():
    """Shader clock and power cap of the AMD cards, read from sysfs (plain file
    reads: no child process). Each entry: the card, the current `pp_dpm_sclk`
    level (MHz) and the hwmon power cap (W); None where the files are absent."""
    out = []
    base = "/sys/class/drm"
    try:
        cards = sorted(c for c in os.listdir(base) if re.fullmatch(r"card\d+", c))
    except OSError:
        return None
    for c in cards:
        dev = os.path.join(base, c, "device")
        try:
            if open(os.path.join(dev, "vendor")).read().strip() != "0x1002":
                continue
            sclk = None
            for line in open(os.path.join(dev, "pp_dpm_sclk")):
                if line.rstrip().endswith("*"):
                    m = re.search(r"(\d+)\s*Mhz", line, re.I)
                    sclk = int(m.group(1)) if m else None
            cap = None
            hw = os.path.join(dev, "hwmon")
            for h in sorted(os.listdir(hw)) if os.path.isdir(hw) else []:
                f = os.path.join(hw, h, "power1_cap")
                if os.path.exists(f):
                    cap = round(int(open(f).read()) / 1e6, 1)
            out.append({"card": c, "sclk_mhz": sclk, "power_cap_w": cap})
        except (OSError, ValueError):
            continue
    return out or None


def read_load_clock(config: str, qk_norm: bool = False):
    """Shader clock under load (GHz) from the committed counter pass of this
    workload (and path): SQ_BUSY_CYCLES per shader engine over the dispatch's
    own duration, if that pass was taken on the current kernel source; else
    None."""
    tag = ("qknorm_" if qk_norm else "") + config.replace("gqa_", "")
    path = os.path.join(ROOT, "profiles", f"counters_gqa_partial_{tag}.md")
    try:
        text = open(path).read()
    except OSError:
        return None
    sha = re.search(r"kernel_source_sha256:\s*([0-9a-f]{64})", text)
    val = re.search(r"load_clock_ghz:\s*([0-9.]+)", text)
    if not (sha and val) or sha.group(1) != kernel_source_sha():
        return None
    return float(val.group(1))


def time_eager(torch, stream, fn, n_steps, warmup):
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(n_steps):
        fn(i)
    end.record(stream)
    end.synchronize()
    return start.elapsed_time(end) / n_steps


def eager_per_call(torch, stream, fn, n_steps):
    """Per-call durations (ms) of n_steps back-to-back eager calls: one event
    between consecutive calls on `stream`, no host synchronisation inside."""
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n_steps + 1)]
    ev[0].record(stream)
    for i in range(n_steps):
        fn(i)
        ev[i + 1].record(stream)
    ev[-1].synchronize()
    return sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(n_steps))


def cpu_baseline(cfg, q, k, v, target_s):
    """The oracle as it stands, on the host's cores, over the whole workload
    (every batch row, query row and key), repeated until about `target_s`
    seconds of wall time have passed; reports the mean rate."""
    import oracle
    reps, t_total = 0, 0.0
    while reps == 0 or t_total < target_s:
        t0 = time.perf_counter()
        oracle.gqa_f64(q, k, v)
        t_total += time.perf_counter() - t0
        reps += 1
    dt = t_total / reps
    # The same oracle on one thread, one call (bounded: a few seconds at the
    # largest workloads' batch sizes would be minutes, so only when the
    # all-thread call took under 0.5 s).
    one = None
    n_all = oracle.threads()
    if dt < 0.5 and n_all > 1:
        oracle.set_threads(1)
        try:
            t0 = time.perf_counter()
            oracle.gqa_f64(q, k, v)
            one = time.perf_counter() - t0
        finally:
            oracle.set_threads(n_all)
    return {
        "value": cfg.flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": oracle.threads(),
        "kind": "oracle",
        "sample": (f"whole workload ({cfg.B}x{cfg.M} query rows x {cfg.N} keys, "
                   f"{cfg.flops / 1e9:.2f} GFLOP) x {reps} repeats, {dt:.3f} s each; "
                   "fp64 C loops, OpenMP over query rows"),
        **({"value_1thread": cfg.flops / one / 1e12} if one else {}),
    }


def main():
    args = parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus > 1 or world > 1:
        print(f"bench.py measures one GPU only (asked for {max(args.gpus, world)}); "
              "the fused GQA path shards over the batch axis with no exchange, but no "
              "multi-GPU run is part of it.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import gqa_attention_split_amd as mga
    from gqa_attention_split_amd.inputs import CONFIGS, make_config

    cfg = CONFIGS[args.config]
    B, M, N, D = cfg.B, cfg.M, cfg.N, cfg.D
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.Stream(dev)  # default priority

    q, k, v = make_config(cfg)
    set_bytes = q.nbytes + k.nbytes + v.nbytes + B * M * D * 2
    R = max(1, min(1024, math.ceil(args.rotate_bytes / set_bytes)))
    base = [torch.from_numpy(x).to(dev) for x in (q, k, v)]
    sets = [base] + [[t.clone() for t in base] for _ in range(R - 1)]
    outs = [torch.empty((B, M, D), dtype=torch.float16, device=dev) for _ in range(R)]
    if args.qk_norm:
        splits = args.splits
        eff = mga.mga_gqa_qknorm_plan(B, M, N, D, splits)[2]
    else:
        splits = args.splits if args.splits > 0 else mga.mga_gqa_choose_splits(B, M, N, D)
        eff = mga.mga_gqa_effective_splits(B, M, N, D, splits)
    ws = mga.workspace_for(B, M, N, D, splits, device=dev, qk_norm=args.qk_norm)
    ws_ptr = 0 if ws is None else ws.data_ptr()
    ws_bytes = 0 if ws is None else ws.numel()
    lib = mga._lib.load()
    sh = stream.cuda_stream
    ptrs = [tuple(t.data_ptr() for t in s) for s in sets]
    optr = [o.data_ptr() for o in outs]
    torch.cuda.synchronize()

    def fwd(i, rotate=True):
        j = i % R if rotate else 0
        if args.qk_norm:
            rc = lib.mga_gqa_qknorm_forward(*ptrs[j], optr[j], B, M, N, D, 1e-6, None, splits, ws_ptr,
                                            ws_bytes, sh)
        else:
            rc = lib.mga_gqa_forward(*ptrs[j], optr[j], B, M, N, D, splits, ws_ptr, ws_bytes, sh)
        if rc:
            raise mga.GqaError(rc)

    def partial(i, rotate=True):
        j = i % R if rotate else 0
        rc = lib.mga_gqa_partial(*ptrs[j], optr[j], B, M, N, D, splits, ws_ptr, ws_bytes, sh)
        if rc:
            raise mga.GqaError(rc)

    gsteps = max(1, min(args.graph_steps, args.steps))
    if args.sweep_splits:
        # One JSON line per split count: the forward at that count, same
        # rotating inputs, graph replay (the bench line's timing).
        for sp in (int(x) for x in args.sweep_splits.split(",")):
            eff_sp = mga.mga_gqa_effective_splits(B, M, N, D, sp)
            if eff_sp < 0:
                continue
            ws_sp = mga.workspace_for(B, M, N, D, sp, device=dev)
            wp, wb = (0, 0) if ws_sp is None else (ws_sp.data_ptr(), ws_sp.numel())

            def fwd_sp(i, sp=sp, wp=wp, wb=wb):
                j = i % R
                rc = lib.mga_gqa_forward(*ptrs[j], optr[j], B, M, N, D, sp, wp, wb, sh)
                if rc:
                    raise mga.GqaError(rc)

            def part_sp(i, sp=sp, wp=wp, wb=wb):
                j = i % R
                rc = lib.mga_gqa_partial(*ptrs[j], optr[j], B, M, N, D, sp, wp, wb, sh)
                if rc:
                    raise mga.GqaError(rc)

            with torch.cuda.stream(stream):
                ms_f, _, _ = time_graph(torch, stream, fwd_sp, args.steps, gsteps, args.warmup)
                ms_p, _, _ = time_graph(torch, stream, part_sp, args.steps, gsteps, args.warmup)
            rows = mga.mga_gqa_plan(B, M, N, D, sp)[1]
            print(json.dumps({"workload": cfg.name, "requested_splits": sp, "splits": eff_sp,
                              "tile_rows": rows, "us_per_forward": round(ms_f * 1e3, 3),
                              "us_partial_kernel": round(ms_p * 1e3, 3),
                              "frac_hbm_peak_forward": round(cfg.algorithmic_bytes / (ms_f * 1e-3)
                                                             / (HBM_PEAK_GBPS * 1e9), 4),
                              "rotating_sets": R, "steps": max(1, math.ceil(args.steps / gsteps)) * gsteps}),
                  flush=True)
            del ws_sp
        return

    if args.boundary and (args.qk_norm or eff == 1):
        print("--boundary times the plain forward's combine launch: it needs a split plan "
              f"(this one has {eff} split{'s' if eff > 1 else ''}) and no --qk-norm", file=sys.stderr)
        sys.exit(2)
    if args.boundary:
        # What the second launch costs in the forward: a fill kernel of one
        # workgroup in the combine's place (the kernel boundary alone), the
        # combine itself, and the combine reading partials that an earlier
        # call wrote (not the ones the partial kernel just wrote).
        tiny = torch.zeros(64, device=dev)
        ws_old = mga.workspace_for(B, M, N, D, splits, device=dev)
        old_ptr = ws_old.data_ptr()
        rc = lib.mga_gqa_partial(*ptrs[0], optr[0], B, M, N, D, splits, old_ptr, ws_bytes, sh)
        if rc:
            raise mga.GqaError(rc)

        def comb_ws(i, wp):
            rc = lib.mga_gqa_combine(optr[i % R], B, M, N, D, splits, wp, ws_bytes, sh)
            if rc:
                raise mga.GqaError(rc)

        pieces = {
            "partial": lambda i: partial(i),
            "partial_then_fill": lambda i: (partial(i), tiny.zero_()),
            "forward": lambda i: fwd(i),
            "partial_then_combine_of_older_partials": lambda i: (partial(i), comb_ws(i, old_ptr)),
            "fill_alone": lambda i: tiny.zero_(),
            "combine_alone": lambda i: comb_ws(i, ws_ptr),
        }
        out = {"workload": cfg.name, "splits": eff, "rotating_sets": R,
               "timing": "hip-graph replay, events on the launch stream, us per call"}
        with torch.cuda.stream(stream):
            for name, fn in pieces.items():
                ms, _, _ = time_graph(torch, stream, fn, args.steps, gsteps, args.warmup)
                out[name + "_us"] = round(ms * 1e3, 3)
        print(json.dumps(out), flush=True)
        return

    print(f"[bench] {cfg.name} B={B} M={M} N={N} D={D} splits={eff} rotating sets={R} "
          f"({R * set_bytes / 2**20:.0f} MiB) steps={args.steps} warmup={args.warmup}",
          file=sys.stderr, flush=True)

    def combine(i, rotate=True):
        j = i % R if rotate else 0
        rc = lib.mga_gqa_combine(optr[j], B, M, N, D, splits, ws_ptr, ws_bytes, sh)
        if rc:
            raise mga.GqaError(rc)

    replays = {}

    def timed(fn, name=None):
        if args.mode == "graph":
            ms, _, per = time_graph(torch, stream, fn, args.steps, gsteps, args.warmup)
            if name:
                per = sorted(per)
                replays[name] = {"n": len(per), "us_per_call_min": round(per[0] * 1e3, 3),
                                 "us_per_call_median": round(per[len(per) // 2] * 1e3, 3),
                                 "us_per_call_max": round(per[-1] * 1e3, 3)}
            return ms
        return time_eager(torch, stream, fn, args.steps, args.warmup)

    clocks_before = gpu_clocks()
    with torch.cuda.stream(stream):
        ms_step = timed(fwd, "forward")
        timed_steps = args.steps if args.mode == "eager" else \
            max(1, math.ceil(args.steps / gsteps)) * gsteps
        print(f"[bench] forward {ms_step * 1e3:.3f} us/step", file=sys.stderr, flush=True)
        clocks_after = gpu_clocks()  # just after the forward's timed region
        if args.qk_norm:  # no separate entry points: the pair is timed as one
            ms_partial, ms_combine = ms_step, 0.0
        else:
            ms_partial = timed(partial, "partial_kernel")
            print(f"[bench] partial kernel {ms_partial * 1e3:.3f} us/launch", file=sys.stderr, flush=True)
            ms_combine = timed(combine) if eff > 1 else 0.0
        ms_hot = timed(lambda i: fwd(i, rotate=False))
        ms_eager = time_eager(torch, stream, fwd, args.steps, args.warmup) \
            if args.eager and args.mode == "graph" else None
        per_call = eager_per_call(torch, stream, fwd, args.steps) if args.eager else None
        if args.pmc_calibrate:
            # One plain device-to-device copy of known size: the reference
            # dispatch that FETCH_SIZE / WRITE_SIZE readings are scaled by.
            src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
            dst = torch.empty_like(src)
            dst.copy_(src)
    torch.cuda.synchronize()

    flops = cfg.flops
    alg_bytes = cfg.algorithmic_bytes
    s = ms_step * 1e-3
    tflops = flops / s / 1e12
    gbps = alg_bytes / s / 1e9
    t_mfma = flops / (MFMA_FP16_PEAK_TFLOPS * 1e12)
    t_hbm = alg_bytes / (HBM_PEAK_GBPS * 1e9)
    bound = "hbm" if t_hbm >= t_mfma else "mfma"
    sp = ms_partial * 1e-3
    # The partial kernel's own algorithmic bytes: Q, K and V read once, and O
    # written once only when it runs unsplit (split, it leaves O to the combine).
    kernel_bytes = alg_bytes - (0 if eff == 1 else B * M * D * 2)
    if bound == "hbm":
        achieved, peak, unit = kernel_bytes / sp / 1e9, HBM_PEAK_GBPS, "GB/s"
        achieved_f = alg_bytes / s / 1e9
    else:
        achieved, peak, unit = flops / sp / 1e12, MFMA_FP16_PEAK_TFLOPS, "TFLOP/s"
        achieved_f = flops / s / 1e12
    load_ghz = read_load_clock(cfg.name, args.qk_norm)

    result = {
        "metric": "fused GQA exp-sum-div attention TFLOP/s + HBM GB/s on 1 MI355X",
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": timed_steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "B": B, "M": M, "N": N, "D": cfg.D,
                   "q_k_std": cfg.qk_std, "v_dist": cfg.v_dist, "seed": cfg.seed,
                   "splits": eff, "rotating_sets": R, "qk_norm": bool(args.qk_norm),
                   "timing": ("hip-graph replay" if args.mode == "graph" else "eager launches")
                   + ", events on the launch stream"},
        "hbm_gbps": round(gbps, 1),
        "frac_hbm_peak": round(t_hbm / s, 4),
        "frac_mfma_peak": round(t_mfma / s, 4),
        "hot_ms_per_step": round(ms_hot, 6),
        "partial_kernel_ms": round(ms_partial, 6),
        "combine_kernel_ms": round(ms_combine, 6),
        "roofline": {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
                     "frac": round(achieved / peak, 4),
                     "traffic": None if args.qk_norm else read_traffic(cfg.name),
                     "kernel": "gqa_partial_kernel + gqa_combine_kernel (QK norm)" if args.qk_norm
                     else "gqa_partial_kernel",
                     "scope": "the dominant kernel alone: its algorithmic bytes (Q, K, V read; O only "
                              "when unsplit) over its graph-replayed launch time"},
        "roofline_forward": {"bound": bound, "achieved": round(achieved_f, 2), "peak": peak, "unit": unit,
                             "frac": round(achieved_f / peak, 4),
                             "scope": "the whole forward (partial kernel + combine and the launch "
                                      "boundaries between them): Q, K, V read, O written, over ms_per_step"},
    }
    if load_ghz:
        # MFMA roof at the shader clock measured under load (counter pass of
        # the same kernel source), next to the nominal 2.4 GHz one.
        peak_load = MFMA_FP16_PEAK_TFLOPS * load_ghz / 2.4
        result["mfma_at_load_clock"] = {"clock_ghz": load_ghz, "peak_tflops": round(peak_load, 1),
                                        "frac_forward": round(flops / s / 1e12 / peak_load, 4),
                                        "frac_partial_kernel": round(flops / sp / 1e12 / peak_load, 4)}
    result["gpu_clocks"] = {"before": clocks_before, "after": clocks_after}
    if replays:
        result["replays"] = replays  # spread of the per-replay means within the timed steps
    if ms_eager is not None:
        result["eager_ms_per_step"] = round(ms_eager, 6)
    if per_call:
        pc = lambda f: round(per_call[min(len(per_call) - 1, int(f * len(per_call)))] * 1e3, 3)
        result["eager_us_per_call"] = {"p10": pc(0.1), "median": pc(0.5), "p90": pc(0.9)}
    if not args.no_cpu_baseline:
        cb = cpu_baseline(cfg, q, k, v, args.cpu_seconds)
        cb["value"] = round(cb["value"], 6)
        one = cb.pop("value_1thread", None)
        if one is not None:  # the oracle on one core, one call of the same workload
            result["cpu_baseline_1thread"] = {"value": round(one, 6), "unit": cb["unit"], "cores": 1,
                                              "kind": "oracle"}
        result["cpu_baseline"] = cb
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
