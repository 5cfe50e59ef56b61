#!/usr/bin/env python3
"""Benchmark of the sparse-MoE FFN layer forward on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload mixtral] [--no-cpu-baseline]
                    [--activation gelu|silu] [--no-expert-bias] [--min-capacity N]
                    [--routing top-k|expert-choice] [--mxfp8] [--packed-weights]

A step is one full layer forward (router, permute -- or scan and selection
under expert choice --, expert phase 1, expert phase 2, combine) over one batch of seeded synthetic tokens already
resident in HBM.  Prints ONE JSON line with tokens/s, the roofline of the
dominant kernel and the CPU oracle timed on a bounded sample of the same
workload.  The timed steps record HIP events only around the two expert
phases (each recorded event costs a few microseconds of the layer), so the
dominant kernel's duration is measured live over the timed region; the
breakdown of the other stages comes from extra steps after it that record
every stage boundary.

Only one GPU is used; --gpus N with N > 1 exits with a message.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE-layer fwd tokens/s + % bf16 MFMA peak, Mixtral-shape E=8 top-2"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0       # MI355X dense fp8 MFMA
PEAK_F32_TFLOPS = 157.3        # MI355X fp32 (matrix and vector)
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
GEMM_SRC = os.path.join(ROOT, "sparse_mixture_experts_28_amd", "csrc", "gemm.hip")
MX_GEMM_SRC = os.path.join(ROOT, "sparse_mixture_experts_28_amd", "csrc", "mxfp8.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_hbm_traffic.json")

# oracle sample per workload: the first N tokens (about 10-30 s of host work)
CPU_SAMPLE_TOKENS = {"tiny": 64, "switch": 4096, "mixtral": 8192, "glam": 16384, "deepseek": 1024}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="mixtral", choices=["tiny", "switch", "mixtral", "glam", "deepseek"])
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=0, help="oracle sample size (0 = workload default)")
    ap.add_argument("--activation", default="gelu", choices=["gelu", "silu"],
                    help="expert activation (silu with --no-expert-bias: the Mixtral expert form)")
    ap.add_argument("--no-expert-bias", action="store_true", help="bias-free expert Linears (NULL b1, b2)")
    ap.add_argument("--min-capacity", type=int, default=0, help="capacity floor (with a capacity factor)")
    ap.add_argument("--packed-weights", action="store_true",
                    help="bf16 expert weights in the tile-packed layout (moe_pack_weights, packed once before timing)")
    ap.add_argument("--mxfp8", action="store_true",
                    help="MXFP8 expert Linears (weights quantized on the GPU before the timed steps)")
    ap.add_argument("--routing", default="top-k", choices=["top-k", "expert-choice"],
                    help="expert-choice: each expert takes C = ceil(k T / E) tokens (the rows top-k routing makes)")
    ap.add_argument("--flush-calls", type=int, default=10,
                    help="after the timed steps, time this many single calls each preceded by a 512 MB write "
                         "that evicts L2 and the Infinity Cache (0 = skip)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (reference for HBM byte counters)")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def gemm_source_sha(mx: bool = False):
    with open(MX_GEMM_SRC if mx else GEMM_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic(workload: str, phase: str, mx: bool = False):
    """HBM bytes per launch of a GEMM phase (read + write, from FETCH_SIZE and
    WRITE_SIZE counter runs scaled by a copy-kernel calibration) as committed
    under profiles/, or None when absent or taken on another version of the
    kernel source (gemm.hip, or mxfp8.hip for the MXFP8 path)."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    entry = t.get(workload + ("_mxfp8" if mx else ""))
    if not entry or entry.get("gemm_source_sha") != gemm_source_sha(mx) or phase not in entry:
        return None
    return entry[phase]["fetch_bytes"] + entry[phase]["write_bytes"]


def host_info():
    """The host the oracle runs on: CPU model, the cores this process may use
    (its affinity mask) and the BLAS library numpy calls."""
    from threadpoolctl import threadpool_info
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = [f"{p.get('internal_api')} {p.get('version')} ({os.path.basename(p.get('filepath', ''))}, "
            f"{p.get('threading_layer', 'n/a')} threading)"
            for p in threadpool_info() if p.get("user_api") == "blas"]
    return {"cpu_model": model, "affinity_cores": len(os.sched_getaffinity(0)), "logical_cpus": os.cpu_count(),
            "blas": "; ".join(blas) or "unknown"}


def cpu_baseline(inp, stacked, ntok: int, ec: bool = False, mx: bool = False):
    from threadpoolctl import threadpool_info, threadpool_limits

    import oracle
    host = host_info()
    # BLAS threads = the cores this process may use (its affinity mask), capped
    # by OMP_NUM_THREADS where the host sets one (the process's CPU share), set explicitly
    nthreads = host["affinity_cores"]
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        nthreads = min(nthreads, int(env))
    limiter = threadpool_limits(limits=nthreads, user_api="blas")
    c = inp.cfg
    ntok = min(ntok, c.T)
    W1, b1, W2, b2 = stacked
    x = inp.x[:ntok]
    get = lambda e: (W1[e], None if b1 is None else b1[e], W2[e], None if b2 is None else b2[e])
    t0 = time.perf_counter()
    if mx:
        from oracle import mxfp8
        ntok = min(ntok, 1024)
        x = inp.x[:ntok]

        def eq(e):   # the oracle quantizes each expert's weights itself (timed: it is oracle work)
            W1q = mxfp8.quantize(oracle.widen(W1[e], "bf16"))
            W2q = mxfp8.quantize(oracle.widen(W2[e], "bf16"))
            return (*W1q, None if b1 is None else b1[e], *W2q, None if b2 is None else b2[e])
        t0 = time.perf_counter()
        mxfp8.moe_forward_mxfp8_ref(x, inp.W_g, eq, c.E, c.k, float(np.float32(c.cf)), c.S, inp.b_g, kind=c.dtype,
                                    activation=c.activation, min_capacity=c.min_capacity)
    elif ec:
        oracle.moe_forward_expert_choice_ref(x, inp.W_g, get, c.E, min(ntok, -(-c.k * ntok // c.E)), c.S, inp.b_g,
                                             kind=c.dtype, activation=c.activation)
    else:
        oracle.moe_forward_ref(x, inp.W_g, get, c.E, c.k, float(np.float32(c.cf)), c.S, inp.b_g, kind=c.dtype,
                               activation=c.activation, min_capacity=c.min_capacity)
    dt = time.perf_counter() - t0
    threads = [p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"]
    limiter.restore_original_limits()
    cores = max(threads) if threads else 1
    return {"value": ntok / dt, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"first {ntok} of {c.T} tokens of the same workload (routing and capacity over the sample), "
                      f"float64 numpy oracle, {dt:.1f} s",
            "cpu_model": host["cpu_model"], "affinity_cores": host["affinity_cores"],
            "logical_cpus": host["logical_cpus"], "blas": host["blas"], "blas_threads": int(cores)}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus > 1 or world > 1:
        print("bench.py runs on exactly one GPU: the layer is measured on one MI355X and no multi-GPU "
              "path is built (expert parallelism is a design note only).", file=sys.stderr)
        sys.exit(2)

    import torch

    import sparse_mixture_experts_28_amd as moe
    from synthetic import make_inputs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inp = make_inputs(args.workload, seed=args.seed, activation=args.activation,
                      expert_bias=not args.no_expert_bias, min_capacity=args.min_capacity)
    c = inp.cfg
    t0 = time.perf_counter()
    stacked = inp.stacked()
    log(f"generated {args.workload} in {time.perf_counter() - t0:.1f} s")

    def up(a):
        if c.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    x, W_g = up(inp.x), up(inp.W_g)
    W1, b1, W2, b2 = (None if a is None else up(a) for a in stacked)
    b_g = None if inp.b_g is None else torch.from_numpy(inp.b_g).to(dev)
    dt_code = moe.MOE_BF16 if c.dtype == "bf16" else moe.MOE_F32
    T, d, h, E, k, S = c.T, c.d, c.h, c.E, c.k, c.S
    ec = args.routing == "expert-choice"
    mx = args.mxfp8
    if mx and (ec or c.dtype != "bf16"):
        raise SystemExit("--mxfp8 runs the bf16 workloads with top-k routing")
    packed = args.packed_weights
    if packed and (mx or c.dtype != "bf16" or d % 256 or h % 256):
        raise SystemExit("--packed-weights needs bf16 expert Linears with d and h multiples of 256 (not --mxfp8)")
    if packed:
        W1, W2 = moe.pack_weights(W1), moe.pack_weights(W2)
        torch.cuda.synchronize()
    C = min(T, -(-k * T // E))
    if mx:
        nbytes = moe.moe_workspace_bytes_mxfp8(T, d, h, E, k, S)
        W1c, W1s = moe.quantize_mxfp8(W1)
        W2c, W2s = moe.quantize_mxfp8(W2)
        torch.cuda.synchronize()
        del W1, W2
    elif ec:
        nbytes = moe.moe_workspace_bytes_expert_choice(T, d, h, E, C, S, dt_code)
        ec_token = torch.empty((E, C), dtype=torch.int32, device=dev)
        ec_w = torch.empty((E, C), dtype=torch.float32, device=dev)
    else:
        nbytes = moe.moe_workspace_bytes(T, d, h, E, k, S, dt_code)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    out = torch.empty((T, d), dtype=x.dtype, device=dev)
    topk_idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    topk_w = torch.empty((T, k), dtype=torch.float32, device=dev)
    aux = torch.empty((1,), dtype=torch.float32, device=dev)
    z_loss = torch.empty((1,), dtype=torch.float32, device=dev)
    counts = torch.empty((E,), dtype=torch.int32, device=dev)
    kept = torch.empty((E,), dtype=torch.int32, device=dev)
    slot_pos = torch.empty((T, k), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)

    launch = moe.MoeLaunch()
    launch.T, launch.d, launch.h, launch.dtype = T, d, h, dt_code
    launch.b_g = b_g.data_ptr() if b_g is not None else None
    launch.expert_counts, launch.expert_kept, launch.slot_pos = counts.data_ptr(), kept.data_ptr(), slot_pos.data_ptr()
    launch.workspace, launch.workspace_bytes = ws.data_ptr(), ws.numel()
    launch.stream = stream.cuda_stream
    launch.z_loss = z_loss.data_ptr()
    launch.activation = moe.ACTIVATIONS[c.activation]
    launch.min_capacity = c.min_capacity
    launch.weights_packed = 1 if packed else 0

    nst = moe.MOE_NUM_STAGE_EVENTS
    # stage boundaries 3, 4, 5: before expert phase 1, after it, after phase 2
    gemm_bounds = (3, 4, 5)
    n_bd = max(3, min(args.steps, 10))   # breakdown steps after the timed region

    def make_events(n, bounds):
        ev = [[torch.cuda.Event(enable_timing=True) if b in bounds else None for b in range(nst)]
              for _ in range(n)]
        for row in ev:
            for e in row:
                if e is not None:
                    e.record(stream)  # creates the handle
        arr = [(ctypes.c_void_p * nst)(*[0 if e is None else int(e.cuda_event) for e in row]) for row in ev]
        return ev, arr

    events, ev_arrays = make_events(args.steps, gemm_bounds)
    bd_events, bd_arrays = make_events(n_bd, range(nst))
    ptr = lambda t: None if t is None else t.data_ptr()
    if mx:
        ptrs = (x.data_ptr(), W_g.data_ptr(), W1c.data_ptr(), W1s.data_ptr(), ptr(b1), W2c.data_ptr(), W2s.data_ptr(),
                ptr(b2))
    else:
        ptrs = (x.data_ptr(), W_g.data_ptr(), W1.data_ptr(), ptr(b1), W2.data_ptr(), ptr(b2))

    def step(ev=None):
        launch.stage_events = None if ev is None else ctypes.cast(ev, ctypes.c_void_p)
        if mx:
            st = moe.moe_forward_mxfp8(*ptrs, E, k, float(c.cf), S, out.data_ptr(), topk_idx.data_ptr(),
                                       topk_w.data_ptr(), aux.data_ptr(), launch)
        elif ec:
            st = moe.moe_forward_expert_choice(*ptrs, E, C, S, out.data_ptr(), ec_token.data_ptr(),
                                               ec_w.data_ptr(), aux.data_ptr(), launch)
        else:
            st = moe.moe_forward(*ptrs, E, k, float(c.cf), S, out.data_ptr(), topk_idx.data_ptr(),
                                 topk_w.data_ptr(), aux.data_ptr(), launch)
        if st != moe.MOE_OK:
            raise RuntimeError(moe.moe_status_string(st))

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} done")

    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        step(ev_arrays[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    log(f"timed {args.steps} steps in {wall * 1e3:.2f} ms")

    # the two expert phases over the timed steps
    gemm_ms_steps = np.array([[events[i][b].elapsed_time(events[i][b + 1]) for b in gemm_bounds[:2]]
                              for i in range(args.steps)])
    # every stage, over n_bd further steps
    for i in range(n_bd):
        step(bd_arrays[i])
    torch.cuda.synchronize()
    per_step_ms = np.array([[bd_events[i][s].elapsed_time(bd_events[i][s + 1]) for s in range(nst - 1)]
                            for i in range(n_bd)])
    stage_ms = per_step_ms.mean(axis=0)

    # Single calls from cold caches: a 512 MB write before each evicts L2 and
    # the 256 MB Infinity Cache, so weights and activations come from HBM.
    # Reported beside the back-to-back figure above, which is `value`.
    flushed = None
    if args.flush_calls > 0:
        scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        e0 = [torch.cuda.Event(enable_timing=True) for _ in range(args.flush_calls)]
        e1 = [torch.cuda.Event(enable_timing=True) for _ in range(args.flush_calls)]
        for i in range(args.flush_calls):
            scratch.fill_(i & 0xff)
            e0[i].record(stream)
            step()
            e1[i].record(stream)
        torch.cuda.synchronize()
        fl = np.array([a.elapsed_time(b) for a, b in zip(e0, e1)])
        unfl = per_step_ms.sum(axis=1)
        flushed = {"calls": args.flush_calls, "median_ms": float(np.median(fl)), "min_ms": float(fl.min()),
                   "tokens_per_s_median": T / (float(np.median(fl)) * 1e-3),
                   "unflushed_median_ms": float(np.median(unfl)), "unflushed_min_ms": float(unfl.min())}
        del scratch
        log(f"flushed calls: median {flushed['median_ms']:.3f} ms (unflushed {flushed['unflushed_median_ms']:.3f})")
    stages = dict(zip(moe.STAGES, stage_ms.tolist()))   # under expert choice "scatter" is the selection
    bd_phase = {"expert_phase1": stages["expert_phase1"], "expert_phase2": stages["expert_phase2"]}
    stages["expert_phase1"], stages["expert_phase2"] = (float(v) for v in gemm_ms_steps.mean(axis=0))

    kept_np = kept.cpu().numpy().astype(np.int64)
    a_kept = int(kept_np.sum())
    rows = a_kept + S * T
    s = 2 if c.dtype == "bf16" else 4
    gemm_flops = 2.0 * d * h * rows                      # per launch (each phase)
    active = int((kept_np > 0).sum()) + S
    bytes_router = T * d * s + E * d * s + 8 * T * k
    # the permute reads each assignment's expert and in-tile rank and the per-tile
    # expert counts, and writes its slot and, for kept ones, the row's token (no
    # token row is copied)
    ntile = -(-T // (32 if (c.dtype == "bf16" and d % 256 == 0 and E <= 64 and -(-T // 64) < 256) else 64))
    bytes_scatter = 12 * T * k + 4 * a_kept + 4 * ntile * E
    bytes_combine = rows * d * s + T * d * s + 8 * T * k
    if ec:
        # router also writes the expert-major float64 logits and each token's max and sum;
        # the selection reads the logits once and writes the [E, T] rank table and, per
        # taken pair, token, row token and weight (reading that token's max and sum);
        # the combine reads the rank table and the weights instead of slot positions
        bytes_router = T * d * s + E * d * s + 8 * E * T + 12 * T
        bytes_scatter = 8 * E * T + 4 * E * T + 24 * E * C
        bytes_combine = rows * d * s + T * d * s + 4 * E * T + 4 * E * C
    # minimal traffic: active expert weights once, x once (phase 1 gathers its
    # rows), H written once / read once, Y written once
    bytes_gemm1 = active * h * d * s + T * d * s + rows * h * s
    bytes_gemm2 = active * h * d * s + rows * (h + d) * s
    if mx:
        # codes 1 byte plus one scale byte per 32 elements for the weights, x and H
        q = 33.0 / 32.0
        bytes_gemm1 = active * h * d * q + T * d * q + rows * h * q
        bytes_gemm2 = active * h * d * q + rows * h * q + rows * d * 2

    def gbs(b, ms):
        return b / (ms * 1e-3) / 1e9

    def tfs(f, ms):
        return f / (ms * 1e-3) / 1e12

    per_stage = {
        "router": {"ms": stages["router"], "GB/s": gbs(bytes_router, stages["router"]), "bytes": bytes_router},
        **({"scan": {"ms": stages["scan"]},
            "select": {"ms": stages["scatter"], "GB/s": gbs(bytes_scatter, stages["scatter"]),
                       "bytes": bytes_scatter}} if ec else
           {"permute": {"ms": stages["scan"] + stages["scatter"],
                        "GB/s": gbs(bytes_scatter, stages["scan"] + stages["scatter"]), "bytes": bytes_scatter}}),
        "expert_phase1": {"ms": stages["expert_phase1"], "TFLOP/s": tfs(gemm_flops, stages["expert_phase1"]),
                          "GB/s": gbs(bytes_gemm1, stages["expert_phase1"]), "flops": gemm_flops},
        "expert_phase2": {"ms": stages["expert_phase2"], "TFLOP/s": tfs(gemm_flops, stages["expert_phase2"]),
                          "GB/s": gbs(bytes_gemm2, stages["expert_phase2"]), "flops": gemm_flops},
        "combine": {"ms": stages["combine"], "GB/s": gbs(bytes_combine, stages["combine"]), "bytes": bytes_combine},
    }
    dom = "expert_phase1" if stages["expert_phase1"] >= stages["expert_phase2"] else "expert_phase2"
    dom_ms = stages[dom]
    dom_bytes = bytes_gemm1 if dom == "expert_phase1" else bytes_gemm2
    traffic = measured_traffic(args.workload + ("_packed" if packed else ""), dom, mx)
    if c.dtype == "f32":
        # float32 layers run the grouped GEMM on the float32 matrix cores
        roof = {"bound": "mfma", "achieved": tfs(gemm_flops, dom_ms), "peak": PEAK_F32_TFLOPS, "unit": "TFLOP/s"}
    elif args.workload == "mixtral":
        roof = {"bound": "mfma", "achieved": tfs(gemm_flops, dom_ms),
                "peak": PEAK_FP8_TFLOPS if mx else PEAK_BF16_TFLOPS, "unit": "TFLOP/s"}
    else:   # fine-grained experts stream their weights: HBM-bound
        roof = {"bound": "hbm", "achieved": gbs(dom_bytes, dom_ms), "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = traffic
    roof["kernel"] = f"gemm ({dom})"
    gemm_ms = stages["expert_phase1"] + stages["expert_phase2"]
    if c.dtype == "f32":
        roof["gemm_both_phases_frac_of_f32_peak"] = tfs(2 * gemm_flops, gemm_ms) / PEAK_F32_TFLOPS
    else:
        roof["gemm_both_phases_frac_of_bf16_peak"] = tfs(2 * gemm_flops, gemm_ms) / PEAK_BF16_TFLOPS
    if mx:
        roof["gemm_both_phases_frac_of_fp8_peak"] = tfs(2 * gemm_flops, gemm_ms) / PEAK_FP8_TFLOPS

    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("copy calibration: 3 x 1 GiB device copies done")

    variant = f", expert-choice routing C={C} tokens per expert" if ec else ""
    if packed:
        variant += ", tile-packed expert weights"
    if mx:
        variant += ", MXFP8 expert Linears (E4M3, E8M0 scale per 32)"
    if c.activation != "gelu" or not c.expert_bias or c.min_capacity:
        variant += (f", {c.activation} experts" + ("" if c.expert_bias else " without bias") +
                    (f", min_capacity={c.min_capacity}" if c.min_capacity else ""))
    result = {
        "metric": METRIC,
        "value": T * args.steps / wall,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp8" if mx else c.dtype,
        "data": "synthetic (seeded normal inputs and random-init weights of the named shapes)",
        "config": {"workload": f"{args.workload}-shaped MoE layer: T={T} d={d} h={h} E={E} k={k} shared={S} "
                               f"capacity_factor={c.cf} {c.dtype}" + variant,
                   "T": T, "d": d, "h": h, "E": E, "k": k, "n_shared": S, "capacity_factor": c.cf,
                   "activation": c.activation, "expert_bias": c.expert_bias, "min_capacity": c.min_capacity,
                   "kept_assignments": a_kept, "routing": args.routing, "weights_packed": packed,
                   **({"tokens_per_expert": C,
                       "untaken_tokens": T - int(torch.unique(ec_token).numel())} if ec else
                      {"dropped_assignments": T * k - a_kept})},
        "roofline": roof,
        "stages": per_stage,
        "layer_ms_events": float(stage_ms.sum()),
        "stage_timing": {"expert_phases": f"HIP events around them in each of the {args.steps} timed steps",
                         "other_stages": f"HIP events at every stage boundary in {n_bd} steps after the timed ones",
                         "expert_phases_in_those_steps_ms": bd_phase},
        "cold_cache": flushed,
    }
    if not args.no_cpu_baseline:
        ntok = args.cpu_tokens or CPU_SAMPLE_TOKENS[args.workload]
        log(f"cpu baseline: oracle on {ntok} tokens")
        result["cpu_baseline"] = cpu_baseline(inp, stacked, ntok, ec, mx)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
