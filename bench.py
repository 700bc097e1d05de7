#!/usr/bin/env python3
"""Benchmark of frame-aligned windowed attention on one MI355X.

One step is one pass of the whole hot path over one batch of synthetic input,
already resident in HBM: fsa_bounds (key mean, key radii, query norms,
eligibility) then fsa_forward (the attention), through the C ABI, on torch's
current stream. The tile plan is built once per shape before timing.

Workload (default): the 720p-shaped super-resolution chunk, 13 frames of
3600 tokens (a 45x80 latent patch grid), 24 heads of width 128, bf16, each
frame attending to frames within +-2 plus reference frame 0; inputs drawn by
frame_aligned_block_amd.inputs with seed 0.

Prints one JSON line. value = valid-tile TFLOP/s of the whole step, with
valid FLOPs = 4 * d * (valid query-key pairs) * B * H (Q.K^T and P.V on live
tiles only). roofline.achieved = the same FLOPs / the forward kernel's mean
launch time, from HIP events recorded on the launch stream around each
forward launch inside the timed loop.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 720p]
    python bench.py --calibrate-copy BYTES   # a plain copy, for counter scaling
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6     # 256 CUs x 4096 bf16 FLOP/clk x 2.4 GHz (dense)
PEAK_FP32_TFLOPS = 157.3      # fp32 vector
METRIC = "valid-tile TFLOP/s and % bf16 MFMA peak, ms/call, 720p-shaped SR attention"
FWD_SOURCES = ("frame_aligned_block_amd/csrc/forward.hip",
               "frame_aligned_block_amd/csrc/fsa_internal.h",
               "frame_aligned_block_amd/csrc/plan.cpp")
PMC_SUMMARY = "profiles/fsa_forward_720p_pmc.txt"


def forward_source_hash() -> str:
    h = hashlib.sha256()
    for rel in FWD_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(config: str):
    """HBM bytes per forward launch from the committed counter summary, or
    None when it is missing, for another workload, or taken on other code."""
    path = os.path.join(ROOT, PMC_SUMMARY)
    if config != "720p" or not os.path.exists(path):
        return None
    text = open(path).read()
    src = re.search(r"^source_sha256:\s*(\w+)", text, re.M)
    tb = re.search(r"^traffic_bytes_per_launch:\s*([0-9.eE+]+)", text, re.M)
    if not src or not tb or src.group(1) != forward_source_hash():
        return None
    return float(tb.group(1))


# Largest worker pool the oracle's timing may use: the GPU machine's host share
# (one GPU's 16 cores), whatever the host reports beyond it.
MAX_CPU_WORKERS = 16


def _oracle_worker_init():
    """One BLAS thread per worker process (set before numpy loads)."""
    for var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS", "BLIS_NUM_THREADS"):
        os.environ[var] = "1"


_HEADS = {}


def _oracle_block(task):
    """One (head, query frame) block of a workload through the fp64 oracle, on
    one core: (seconds, valid FLOPs). The head is drawn on the host by the
    same seeded recipe as the GPU inputs (the host and device generators give
    different values; the work is the same)."""
    import numpy as np
    from oracle import fsa_oracle as orc
    from frame_aligned_block_amd.inputs import CONFIGS, make_head, to_f64
    name, h, f = task
    cfg = CONFIGS[name]
    if (name, h) not in _HEADS:
        _HEADS.clear()
        _HEADS[(name, h)] = tuple(to_f64(t)[None, None] for t in make_head(cfg, 0, 0, h))
    q, k, v = _HEADS[(name, h)]
    rows = np.arange(f * cfg.T, (f + 1) * cfg.T)
    t0 = time.perf_counter()
    orc.attention_rows(q, k, v, cfg.F, cfg.T, cfg.window, cfg.ref_frame, cfg.scale, 0, 0, rows)
    dt = time.perf_counter() - t0
    keys = cfg.T * len(orc.slice_frames(cfg.F, cfg.window, cfg.ref_frame, f))
    return dt, 4.0 * cfg.d * cfg.T * keys


def _blocks(cfg, heads, per_head=None):
    """(head, frame) blocks of the given heads, head by head, each head's
    heaviest frames first (per_head of them, or all)."""
    from oracle import fsa_oracle as orc
    frames = sorted(range(cfg.F), key=lambda f: -len(orc.slice_frames(cfg.F, cfg.window,
                                                                       cfg.ref_frame, f)))
    return [(cfg.name, h % cfg.H, f) for h in heads for f in frames[:per_head]]


def cpu_baseline(cfg, total_flops: float, heads: int = 0, small_heads: int = 0):
    """The fp64 oracle as it stands, on the host's cores: one whole call of the
    workload (or its first `heads` heads, scaled to a call) on a pool of one
    process per core (at most MAX_CPU_WORKERS), one BLAS thread each, each
    worker taking one head's (head, query frame) blocks at a time; and one
    whole call of the small workload on one core (or its first `small_heads`
    heads, scaled). None for the cross-attention and producer workloads."""
    import concurrent.futures as cf
    import multiprocessing as mp
    from frame_aligned_block_amd.inputs import CONFIGS
    if cfg.M or cfg.grid:
        return None
    cores = max(1, min(len(os.sched_getaffinity(0)), MAX_CPU_WORKERS))
    ctx = mp.get_context("spawn")          # a fresh interpreter: nothing of the GPU is inherited
    nh = min(cfg.H, max(heads, cores)) if heads else cfg.H    # at least one head per worker
    tasks = _blocks(cfg, range(nh))
    with cf.ProcessPoolExecutor(max_workers=cores, mp_context=ctx,
                                initializer=_oracle_worker_init) as pool:
        list(pool.map(_oracle_block, [(cfg.name, 0, cfg.F // 2)] * cores))   # imports, warm-up
        t0 = time.perf_counter()
        res = list(pool.map(_oracle_block, tasks, chunksize=cfg.F))
        wall = time.perf_counter() - t0
    flops = sum(r[1] for r in res)
    rate = flops / wall
    small = CONFIGS["small"]
    sh = small_heads or small.H
    with cf.ProcessPoolExecutor(max_workers=1, mp_context=ctx,
                                initializer=_oracle_worker_init) as one:
        list(one.map(_oracle_block, [(small.name, 0, 0)]))                 # imports, warm-up
        t0 = time.perf_counter()
        list(one.map(_oracle_block, _blocks(small, range(sh)), chunksize=small.F))
        s_wall = time.perf_counter() - t0
    scaled = " (scaled to all heads)" if nh < cfg.H else ""
    return {"value": round(rate / 1e12, 6), "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "ms_per_call": round(total_flops / rate * 1e3, 1),
            "small_single_core_ms_per_call": round(s_wall * small.H / sh * 1e3, 1),
            "sample": f"{nh} of {cfg.H} heads of the {cfg.name} workload ({len(tasks)} (head, "
                      f"query-frame) blocks, {flops / 1e9:.0f} of {total_flops / 1e9:.0f} valid "
                      f"GFLOP) in {wall:.1f} s wall on a pool of {cores} processes, one BLAS "
                      f"thread each, fp64 numpy{scaled}; the small workload on one core: {sh} of "
                      f"{small.H} heads in {s_wall:.1f} s" + (" (scaled)" if sh < small.H else "")}


def workload_name(cfg) -> str:
    head = (f"{cfg.name}-shaped SR chunk: F={cfg.F} frames x T={cfg.T} tokens ({cfg.N} "
            f"tokens), H={cfg.H}, d={cfg.d}, {cfg.dtype}, ")
    if cfg.M:
        return head + f"cross-attention of every token to M={cfg.M} reference tokens"
    return head + f"window +-{cfg.window} + reference frame {cfg.ref_frame}"


def current_sclk_mhz():
    """The GPU's current shader clock from the amdgpu sysfs table (the line
    marked '*'), read right after the timed region; None where unavailable."""
    for path in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
        try:
            for ln in open(path).read().splitlines():
                if ln.rstrip().endswith("*"):
                    return int(ln.split(":")[1].strip().lower().split("mhz")[0])
        except (OSError, ValueError, IndexError):
            continue
    return None


def calibrate_copy(nbytes: int) -> None:
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes": nbytes, "launches": 5}))


def timed(fn, launches: int, stream):
    """Median HIP-event time (ms) of `launches` calls of fn on `stream`."""
    import torch
    e = [torch.cuda.Event(enable_timing=True) for _ in range(launches + 1)]
    e[0].record(stream)
    for i in range(launches):
        fn()
        e[i + 1].record(stream)
    torch.cuda.synchronize()
    return statistics.median([e[i].elapsed_time(e[i + 1]) for i in range(launches)])


def bench_producer(args, cfg) -> int:
    """A producer workload: one step is fsa_prep (RMSNorm, Q/K/V projection,
    rotary embedding, head packing, and the bounds' row norms and key sums),
    fsa_bounds_after_prep, then fsa_forward, from tokens already in HBM. The
    roofline line is the producer call's (its short row-scale pre-pass and the
    MFMA-bound projection kernel, timed together); the same
    chain with the separate fsa_bounds pass is timed beside it."""
    import torch
    from frame_aligned_block_amd import fsa
    from frame_aligned_block_amd.inputs import make_prep_inputs

    print(f"[bench] {cfg.name}: drawing inputs", file=sys.stderr, flush=True)
    X, W, g = make_prep_inputs(cfg, seed=0, device="cuda")
    Wp = torch.empty_like(W)
    fsa.fsa_prep_pack_weights(W, g, Wp, cfg.H, cfg.d)
    plan = fsa.fsa_plan_create(fsa.make_shape(cfg.B, cfg.H, cfg.F, cfg.T, cfg.d, cfg.window,
                                              cfg.ref_frame, args.bq, 0, fsa.FSA_BF16))
    ws = torch.zeros(fsa.fsa_workspace_bytes(plan), dtype=torch.uint8, device="cuda")
    shape = (cfg.B, cfg.H, cfg.N, cfg.d)
    Q, K, V, O = (torch.empty(shape, dtype=torch.bfloat16, device="cuda") for _ in range(4))
    Hg, Wg = cfg.grid
    stream = torch.cuda.current_stream()
    C = cfg.H * cfg.d
    proj_flops = 2.0 * cfg.B * cfg.N * C * 3 * C
    attn_flops = 4.0 * cfg.d * fsa.fsa_plan_valid_pairs(plan) * cfg.B * cfg.H

    def prep():
        fsa.fsa_prep(plan, Hg, Wg, X, Wp, Q, K, V, ws, stream)

    def step():
        prep()
        fsa.fsa_bounds_after_prep(plan, K, ws, cfg.scale, stream)
        fsa.fsa_forward(plan, Q, K, V, O, ws, cfg.scale, args.mode, stream)

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    n = max(3, args.steps // 2)
    prep_ms = timed(prep, n, stream)
    bap_ms = timed(lambda: fsa.fsa_bounds_after_prep(plan, K, ws, cfg.scale, stream), n, stream)
    bounds_ms = timed(lambda: fsa.fsa_bounds(plan, Q, K, ws, cfg.scale, stream), n, stream)
    fsa.fsa_bounds_after_prep(plan, K, ws, cfg.scale, stream)
    fwd_ms = timed(lambda: fsa.fsa_forward(plan, Q, K, V, O, ws, cfg.scale, args.mode, stream),
                   n, stream)
    elig = float(fsa.fsa_copy_eligibility(plan, ws, stream).mean())
    achieved = proj_flops / prep_ms / 1e9
    line = {
        "metric": METRIC,
        "value": round((proj_flops + attn_flops) / ms_step / 1e9, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: the SR layer's producer then attention: "
                               f"F={cfg.F} frames of {Hg}x{Wg} patches ({cfg.N} tokens), "
                               f"C={C} channels, H={cfg.H}, d={cfg.d}, bf16, window "
                               f"+-{cfg.window} + reference frame {cfg.ref_frame}",
                   "B": cfg.B, "H": cfg.H, "F": cfg.F, "T": cfg.T, "d": cfg.d, "C": C,
                   "grid": [Hg, Wg], "mode": args.mode,
                   "projection_flops": proj_flops, "attention_valid_flops": attn_flops},
        "prep_ms_median": round(prep_ms, 4),
        "bounds_after_prep_ms_median": round(bap_ms, 4),
        "separate_bounds_ms_median": round(bounds_ms, 4),
        "forward_ms_median": round(fwd_ms, 4),
        "eligible_head_fraction": round(elig, 4),
        "roofline": {"kernel": "fsa_prep (prep_rowscale + prep_qkv)", "bound": "mfma",
                     "achieved": round(achieved, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": None},
        "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)
    return 0


def extra_workload(name: str, launches: int = 5):
    """Forward time of another workload in the same process (not part of the
    timed step): the median of `launches` event-timed launches after two
    warm-ups, its valid-FLOP rate and fraction of peak, the eligible fraction,
    and for mixed-route workloads the same forward with every head online."""
    import torch
    from frame_aligned_block_amd import fsa
    from frame_aligned_block_amd.inputs import CONFIGS, make_inputs
    cfg = CONFIGS[name]
    print(f"[bench] extra workload {name}", file=sys.stderr, flush=True)
    Q, K, V = make_inputs(cfg, seed=0, device="cuda")
    plan = fsa.fsa_plan_create(fsa.make_shape(cfg.B, cfg.H, cfg.F, cfg.T, cfg.d, cfg.window,
                                              cfg.ref_frame, 0, 0, fsa.FSA_BF16))
    ws = torch.zeros(fsa.fsa_workspace_bytes(plan), dtype=torch.uint8, device="cuda")
    O = torch.empty_like(Q)
    flops = 4.0 * cfg.d * fsa.fsa_plan_valid_pairs(plan) * cfg.B * cfg.H
    stream = torch.cuda.current_stream()
    fsa.fsa_bounds(plan, Q, K, ws, cfg.scale, stream)
    out = {"workload": workload_name(cfg), "row_block": fsa.fsa_plan_row_block(plan),
           "valid_flops": flops}
    for mode in (["auto", "online"] if cfg.loose_period else ["auto"]):
        for _ in range(2):
            fsa.fsa_forward(plan, Q, K, V, O, ws, cfg.scale, mode, stream)
        ms = timed(lambda: fsa.fsa_forward(plan, Q, K, V, O, ws, cfg.scale, mode, stream),
                   launches, stream)
        key = "forward_ms_median" if mode == "auto" else "online_only_forward_ms_median"
        out[key] = round(ms, 4)
        if mode == "auto":
            out["tflops"] = round(flops / ms / 1e9, 2)
            out["frac"] = round(flops / ms / 1e9 / PEAK_BF16_TFLOPS, 4)
    if "online_only_forward_ms_median" in out:
        out["fixed_max_speedup"] = round(out["online_only_forward_ms_median"]
                                         / out["forward_ms_median"], 4)
    el = fsa.fsa_copy_eligibility(plan, ws, stream)
    out["eligible_heads"] = f"{int(el.sum())}/{el.size}"
    del Q, K, V, O, ws
    torch.cuda.empty_cache()
    return out


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="720p")
    ap.add_argument("--mode", default="auto", choices=["auto", "online", "fixed", "auto_frame", "auto_rows"])
    ap.add_argument("--ab-launches", type=int, default=5,
                    help="timed online-only forward launches for the A/B figure")
    ap.add_argument("--cpu-heads", type=int, default=0,
                    help="time the oracle on this many heads and scale (0: the whole call)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--bq", type=int, default=0)
    ap.add_argument("--row-block", type=int, default=0,
                    help="rows per workgroup of the bf16 forward (128: 4 waves, 256: 8 waves; "
                         "0: the plan's choice)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES")
    ap.add_argument("--extra", default="stress,1080p",
                    help="other workloads whose forward is timed after the 720p line's "
                         "(comma list; empty for none)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU only; --gpus {args.gpus} is not "
              "supported (the path shards by head across GPUs, which is not built here)",
              file=sys.stderr)
        return 2

    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return 0

    from frame_aligned_block_amd import fsa
    from frame_aligned_block_amd.inputs import CONFIGS, make_inputs

    cfg = CONFIGS[args.config]
    if cfg.grid:
        return bench_producer(args, cfg)
    print(f"[bench] {cfg.name}: drawing inputs", file=sys.stderr, flush=True)
    Q, K, V = make_inputs(cfg, seed=0, device="cuda")
    code = fsa.FSA_BF16 if cfg.dtype == "bf16" else fsa.FSA_F32
    if cfg.M:           # cross-attention to M reference tokens
        plan = fsa.fsa_plan_create_cross(fsa.make_shape(cfg.B, cfg.H, cfg.F, cfg.T, cfg.d, 0, 0,
                                                        args.bq, 0, code), cfg.M)
    else:
        plan = fsa.fsa_plan_create(fsa.make_shape(cfg.B, cfg.H, cfg.F, cfg.T, cfg.d,
                                                  cfg.window, cfg.ref_frame, args.bq, 0, code))
    if args.row_block:
        fsa.fsa_plan_set_row_block(plan, args.row_block)
    ws = torch.zeros(fsa.fsa_workspace_bytes(plan), dtype=torch.uint8, device="cuda")
    O = torch.empty_like(Q)
    pairs = fsa.fsa_plan_valid_pairs(plan)
    flops = 4.0 * cfg.d * pairs * cfg.B * cfg.H
    stream = torch.cuda.current_stream()

    def step(mode=args.mode):
        fsa.fsa_bounds(plan, Q, K, ws, cfg.scale, stream)
        fsa.fsa_forward(plan, Q, K, V, O, ws, cfg.scale, mode, stream)

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record(stream)
        fsa.fsa_bounds(plan, Q, K, ws, cfg.scale, stream)
        ev[i][1].record(stream)
        fsa.fsa_forward(plan, Q, K, V, O, ws, cfg.scale, args.mode, stream)
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    bnd = [e[0].elapsed_time(e[1]) for e in ev]
    fwd = [e[1].elapsed_time(e[2]) for e in ev]
    bnd_ms = sum(bnd) / args.steps
    fwd_ms = sum(fwd) / args.steps
    sclk = current_sclk_mhz()

    # A/B: the same forward with every head on the online path
    ab = None
    if args.ab_launches > 0 and args.mode != "online":
        e = [torch.cuda.Event(enable_timing=True) for _ in range(args.ab_launches + 1)]
        fsa.fsa_forward(plan, Q, K, V, O, ws, cfg.scale, "online", stream)
        e[0].record(stream)
        for i in range(args.ab_launches):
            fsa.fsa_forward(plan, Q, K, V, O, ws, cfg.scale, "online", stream)
            e[i + 1].record(stream)
        torch.cuda.synchronize()
        on_ms = e[0].elapsed_time(e[-1]) / args.ab_launches
        step()                          # leave O as the benchmarked mode wrote it
        torch.cuda.synchronize()
        ab = {"online_only_forward_ms": round(on_ms, 4),
              "online_only_forward_tflops": round(flops / on_ms / 1e9, 2),
              "fixed_max_speedup": round(on_ms / fwd_ms, 4)}

    elig = float(fsa.fsa_copy_eligibility(plan, ws, stream).mean())
    bf16 = cfg.dtype == "bf16"
    peak = PEAK_BF16_TFLOPS if bf16 else PEAK_FP32_TFLOPS
    achieved = flops / fwd_ms / 1e9
    line = {
        "metric": METRIC,
        "value": round(flops / ms_step / 1e9, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {"workload": workload_name(cfg),
                   "B": cfg.B, "H": cfg.H, "F": cfg.F, "T": cfg.T, "d": cfg.d,
                   **({"M": cfg.M} if cfg.M else {}),
                   "mode": args.mode, "bq": fsa.fsa_plan_shape(plan).bq,
                   "row_block": fsa.fsa_plan_row_block(plan),
                   "valid_pairs_per_head": pairs, "valid_flops_per_step": flops},
        "ms_per_call": round(ms_step, 4),
        "pct_bf16_peak": round(100.0 * flops / ms_step / 1e9 / PEAK_BF16_TFLOPS, 2),
        "forward_ms": round(fwd_ms, 4),
        "forward_ms_median": round(statistics.median(fwd), 4),
        "bounds_ms": round(bnd_ms, 4),
        "bounds_ms_median": round(statistics.median(bnd), 4),
        "sclk_mhz_after_timing": sclk,
        "eligible_head_fraction": round(elig, 4),
        "ab": ab,
        "roofline": {"kernel": "fwd_bf16" if bf16 else "fwd_f32",
                     "bound": "mfma" if bf16 else "alu", "achieved": round(achieved, 2),
                     "peak": peak, "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                     "traffic": measured_traffic(cfg.name)},
        "cpu_baseline": None,
    }
    if args.config == "720p" and args.extra:
        line["workloads"] = {n: extra_workload(n) for n in args.extra.split(",") if n}
    if not args.no_cpu_baseline:
        print("[bench] oracle baseline on the host cores", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(cfg, flops, args.cpu_heads)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
