"""Benchmark: Q4_K GEMV weight GB/s and % of HBM roofline at batch 1 on the
Qwen3.5-9B-shaped FFN and untied lm_head (shapes from issue #3346,
size_variants.9b: d = 4096, intermediate = 12288, V = 248320).

One step is one pass of the decode hot path over resident weights:
    h      = silu(W_gate x) * (W_up x)   q4k_fused_swiglu  2 x [12288, 4096]
    y      = W_down h                    q4k_gemv          [4096, 12288]
    logits = W_lm_head y                 q4k_gemv          [248320, 4096]
657 MB of Q4_K weights per step (more than the 256 MB Infinity Cache, so
every step streams its weights from HBM).  Inputs are seeded synthetic data of
the pages' value distributions (q4_dequant_gemv_amd/inputs.py).

Prints ONE JSON line.  `value` is step weight bytes / mean step time.  The K
steps are captured once into a HIP graph; after one untimed replay the graph
is replayed R times back to back (R >= 5, R * K >= 200), each replay -- K
steps -- between its own pair of HIP events on the launch stream, and the step
time is the mean over the R replays (`--eager` times R back-to-back regions of
K plain launches instead; both rates are in the line, with every region's
figure).  Every timed section is preceded by >= 100 ms of the same work,
untimed and back to back (warm_up): after a few milliseconds of idle GPU the
same steps run up to a fifth slower and speed up over tens of milliseconds of
load, so a single short region timed right after a synchronize or a graph
capture measures that ramp, not the kernels.
`roofline` covers the dominant kernel (the lm_head GEMV): algorithmic bytes
per launch / mean launch time over R * K back-to-back launches, again between
two events on the launch stream.  `traffic` comes from the committed rocprofv3
counter summary (profiles/traffic_lm_head_9b.json) when it was taken from the
kernel sources as they are now, else null.  `cpu_baseline` times the CPU
oracle on full steps.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "Q4_K GEMV weight GB/s and % HBM roofline at batch 1 (9B lm_head/FFN)"
KERNEL_SOURCES = ["q4k_device.h", "q4k_int_dot.h", "gemv.hip", "api.hip"]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "q4_dequant_gemv_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_profile(launch_weight_bytes: int):
    path = os.path.join(ROOT, "profiles", "traffic_lm_head_9b.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing")
    ap.add_argument("--no-batched", action="store_true", help="skip the skinny-GEMM timings")
    ap.add_argument("--step-only", action="store_true",
                    help="time only the decode step and its three kernels (no batched, block, Q8_0, f16, prefill, "
                         "small-config or streaming-ceiling timings, no CPU baseline): for kernel traces")
    ap.add_argument("--eager", action="store_true",
                    help="time the steps as eager launches instead of one captured HIP graph")
    ap.add_argument("--sweep", action="store_true",
                    help="also time every kernel at every config shape (table on stderr)")
    ap.add_argument("--case", default=None,
                    help="only run one kernel in a loop, for profilers: gemv:NAME, swiglu:NAME, "
                         "residual:NAME, q8_0:NAME, dequant:NAME, batched:M:NAME or prefill:M:NAME "
                         "with NAME a shape of inputs.SHAPES, or multi:gdn_0p8b")
    return ap.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: this path runs on one GPU; multi-GPU runs are not part of this benchmark "
              "(row shards need no communication between GPUs; only one GPU's share is built and timed)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from q4_dequant_gemv_amd import inputs, q4k

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    q4k.lib()
    if args.case:
        run_case(args.case, args.steps, args.warmup, q4k, inputs, torch, np, dev)
        return

    log("[bench] generating inputs")
    shapes = {nm: inputs.SHAPES[nm] for nm in ("gate_9b", "up_9b", "down_9b", "lm_head_9b")}
    host = {
        "gate_9b": inputs.make_q4k(*shapes["gate_9b"], config_id=2, tensor_id=0),
        "up_9b": inputs.make_q4k(*shapes["up_9b"], config_id=2, tensor_id=1),
        "down_9b": inputs.make_q4k(*shapes["down_9b"], config_id=2, tensor_id=2),
        "lm_head_9b": inputs.make_q4k(*shapes["lm_head_9b"], config_id=3, tensor_id=0),
    }
    x_host = inputs.make_x(1, 4096, config_id=2, tensor_id=100)[0]
    W = {nm: torch.from_numpy(a.reshape(-1)).to(dev) for nm, a in host.items()}
    x = torch.from_numpy(x_host).to(dev)
    h = torch.empty(12288, dtype=torch.float32, device=dev)
    y = torch.empty(4096, dtype=torch.float32, device=dev)
    logits = torch.empty(248320, dtype=torch.float32, device=dev)
    wbytes = {nm: a.nbytes for nm, a in host.items()}
    step_weight_bytes = sum(wbytes.values())
    stream = torch.cuda.current_stream()

    def step(s=stream):
        q4k.fused_swiglu(W["gate_9b"], W["up_9b"], x, h=h, stream=s)
        q4k.gemv(W["down_9b"], h, y=y, stream=s)
        q4k.gemv(W["lm_head_9b"], y, y=logits, stream=s)

    log(f"[bench] warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    replays = max(5, -(-200 // args.steps))

    def time_regions(run_region):
        """Per-step times (us) of `replays` back-to-back regions, each between
        its own pair of events on the launch stream, after >= 100 ms of the
        same regions untimed (see warm_up)."""
        warm_up(run_region, torch, stream)
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(replays + 1)]
        evs[0].record(stream)
        for r in range(replays):
            run_region()
            evs[r + 1].record(stream)
        torch.cuda.synchronize()
        return [evs[r].elapsed_time(evs[r + 1]) * 1e3 / args.steps for r in range(replays)]

    def eager_region():
        for _ in range(args.steps):
            step()

    # Timed region: K whole steps between two events on the launch stream (no
    # events between the kernels), R times.  By default the K steps are
    # captured once into a HIP graph (the way a decode loop is deployed) and
    # each region is one replay of it; the eager rate is reported beside it.
    log(f"[bench] timing {replays} regions of {args.steps} steps")
    torch.cuda.synchronize()
    eager_us = time_regions(eager_region)
    eager_ms = sum(eager_us) / len(eager_us) * 1e-3
    t0 = time.perf_counter()
    if args.eager:
        region_us = eager_us
        launch = f"eager launches, {replays} regions of {args.steps} steps"
    else:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(args.steps):
                step(None)  # the capture stream
        torch.cuda.synchronize()
        region_us = time_regions(graph.replay)
        launch = f"one HIP graph of {args.steps} steps, replayed {replays} times back to back"
        del graph
    ms_per_step = sum(region_us) / len(region_us) * 1e-3
    wall = time.perf_counter() - t0
    value = step_weight_bytes / (ms_per_step * 1e-3) / 1e9

    # Per kernel: R * K launches of that kernel alone, back to back on the
    # launch stream between two events.  The FFN matrices (85 MB
    # together) would stay in the 256 MB Infinity Cache when repeated, so
    # those launches rotate over copies totalling >= 512 MiB, as in the step
    # where the lm_head evicts them; the lm_head (572 MB) streams from HBM.
    kernel_bytes = {
        "fused_swiglu": wbytes["gate_9b"] + wbytes["up_9b"] + 4 * 4096 + 4 * 12288,
        "gemv_down": wbytes["down_9b"] + 4 * 12288 + 4 * 4096,
        "gemv_lm_head": wbytes["lm_head_9b"] + 4 * 4096 + 4 * 248320,
    }

    def rotated(names):
        """The resident weights plus enough copies to total >= 512 MiB."""
        n_copies = max(1, -(-(512 << 20) // sum(wbytes[nm] for nm in names)))
        return [[W[nm] for nm in names]] + [[W[nm].clone() for nm in names] for _ in range(n_copies - 1)]

    sets_sw = rotated(["gate_9b", "up_9b"])
    sets_dn = rotated(["down_9b"])
    launches = {
        "fused_swiglu": lambda i: q4k.fused_swiglu(*sets_sw[i % len(sets_sw)], x, h=h, stream=stream),
        "gemv_down": lambda i: q4k.gemv(sets_dn[i % len(sets_dn)][0], h, y=y, stream=stream),
        "gemv_lm_head": lambda i: q4k.gemv(W["lm_head_9b"], y, y=logits, stream=stream),
    }
    kernels = {}
    n_launch = replays * args.steps
    for nm, fn in launches.items():
        for i in range(args.warmup):
            fn(i)
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        warm_up(lambda: [fn(i) for i in range(args.steps)], torch, stream)
        a.record(stream)
        for i in range(n_launch):
            fn(i)
        b.record(stream)
        torch.cuda.synchronize()
        mean_s = a.elapsed_time(b) / n_launch * 1e-3
        gbs = kernel_bytes[nm] / mean_s / 1e9
        kernels[nm] = {"mean_us": round(mean_s * 1e6, 3), "GB/s": round(gbs, 1),
                       "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4), "calls_per_s": round(1.0 / mean_s, 1),
                       "per_launch_us": _per_launch(fn, torch, stream, 100)}
    del sets_sw, sets_dn
    achieved = kernels["gemv_lm_head"]["GB/s"]
    roofline = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic_from_profile(wbytes["lm_head_9b"]),
                "kernel": "q4k_gemv lm_head 248320x4096", "bytes_per_launch": kernel_bytes["gemv_lm_head"]}

    # The skinny-GEMM workload over the same FFN weights (m tokens): one call
    # per launch, weights rotated over >= 512 MiB of copies.
    batched = {}
    if args.step_only:
        args.no_batched = True
        args.no_cpu_baseline = True
    if not args.no_batched:
        for nm in ("gate_9b", "down_9b"):
            n_, k_ = shapes[nm]
            sets_b = rotated([nm])
            for mtok in (2, 4, 16, 32, 64):
                xs = torch.from_numpy(inputs.make_x(mtok, k_, config_id=4, tensor_id=100 + mtok)).to(dev)
                yb = torch.empty((mtok, n_), dtype=torch.float32, device=dev)
                t = _time_launches(lambda i: q4k.gemv_batched(sets_b[i % len(sets_b)][0], xs, y=yb, stream=stream),
                                   torch, stream, 50, 20)
                # the same work with the caller's workspace: no allocation per call
                ws = torch.empty(max(1, q4k.gemv_batched_workspace_size(mtok, n_, k_)), dtype=torch.uint8,
                                 device=dev)
                t_ws = _time_launches(
                    lambda i: q4k.gemv_batched_ws(sets_b[i % len(sets_b)][0], xs, ws, y=yb, stream=stream), torch,
                    stream, 50, 20)
                batched[f"{nm} m={mtok}"] = {"mean_us": round(t * 1e6, 2),
                                             "weight_GB/s": round(wbytes[nm] / t / 1e9, 1),
                                             "TFLOP/s": round(2.0 * mtok * n_ * k_ / t / 1e12, 2),
                                             "workspace_call_us": round(t_ws * 1e6, 2)}
                del ws
            del sets_b

    blocks = q8 = f16io = prefill = small = shards = {}
    ceiling = None
    if not args.step_only:
        blocks = decode_blocks(q4k, inputs, torch, dev, stream, args.steps, args.warmup)
        q8 = q8_0_kernels(q4k, inputs, torch, dev, stream, args.steps, args.warmup)
        f16io = f16_variants(q4k, inputs, torch, dev, stream, args.steps, args.warmup, not args.no_batched)
        prefill = prefill_kernels(q4k, inputs, torch, dev, stream) if not args.no_batched else {}
        ceiling = stream_read_ceiling(torch, dev, stream, kernels["gemv_lm_head"]["GB/s"])
        small = small_configs(q4k, inputs, torch, dev, stream)
        shards = shard_shapes(q4k, inputs, torch, dev, stream)

    log(f"[bench] {ms_per_step * 1e3:.1f} us/step, {value:.1f} GB/s; per kernel {kernels}; "
        f"batched {batched}; decode blocks {blocks}; q8_0 {q8}; f16 i/o {f16io}; prefill {prefill}; "
        f"host wall {wall:.3f}s")

    cpu = None
    if not args.no_cpu_baseline:
        import oracle

        cores = len(os.sched_getaffinity(0))
        threads = max(1, min(cores, 64))
        log(f"[bench] cpu baseline: oracle on full steps for >= 10 s, {threads} threads")
        t0 = time.perf_counter()
        reps = 0
        while True:
            ref_h = oracle.fused_swiglu(host["gate_9b"], host["up_9b"], x_host, threads=threads)["h"]
            ref_y = oracle.gemv(host["down_9b"], ref_h.astype(np.float32), threads=threads)[0]
            oracle.gemv(host["lm_head_9b"], ref_y.astype(np.float32), threads=threads)
            reps += 1
            cpu_s = time.perf_counter() - t0
            if cpu_s >= 10.0 or reps >= 200:
                break
        cpu = {"value": round(reps * step_weight_bytes / cpu_s / 1e9, 3), "unit": "GB/s", "cores": threads,
               "kind": "oracle",
               "sample": f"{reps} full steps (gate+up SwiGLU, down, lm_head: all rows, 657 MB of Q4_K each), "
                         f"{cpu_s:.1f} s on {threads} host threads"}
        # the same oracle on one thread (one full step)
        t1 = time.perf_counter()
        ref_h = oracle.fused_swiglu(host["gate_9b"], host["up_9b"], x_host, threads=1)["h"]
        ref_y = oracle.gemv(host["down_9b"], ref_h.astype(np.float32), threads=1)[0]
        oracle.gemv(host["lm_head_9b"], ref_y.astype(np.float32), threads=1)
        one_s = time.perf_counter() - t1
        cpu["single_thread"] = {"value": round(step_weight_bytes / one_s / 1e9, 3), "unit": "GB/s",
                                "sample": f"1 full step, {one_s:.1f} s on 1 host thread"}

    if args.sweep:
        sweep(q4k, inputs, torch, np, dev)

    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "qwen3.5-9b-shaped decode FFN + lm_head at batch 1: fused gate+up SwiGLU "
                        "(2 x 12288x4096), down (4096x12288), untied lm_head (248320x4096), Q4_K weights, f32 activations",
            "weight_bytes_per_step": step_weight_bytes,
            "launch": launch,
            "eager_ms_per_step": round(eager_ms, 5),
            "regions_us_per_step": [round(v, 2) for v in region_us],
            "eager_regions_us_per_step": [round(v, 2) for v in eager_us],
            "frac_hbm_peak_step": round(value / HBM_PEAK_GBS, 4),
            "kernels": kernels,
            "batched_9b_ffn": batched,
            "decode_blocks": blocks,
            "q8_0_9b": q8,
            "f16_io_9b": f16io,
            "prefill_9b_ffn": prefill,
            "stream_read_1GiB": ceiling,
            "configs_0_1": small,
            "shard_of_8_9b": shards,
        },
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def small_configs(q4k, inputs, torch, dev, stream):
    """The GEMV and dequant calls at the small config shapes (the 1024 x 1024
    square; the 0.8B q-proj, out-proj and lm_head): see graph_timed_calls."""
    return graph_timed_calls(q4k, inputs, torch, dev, stream,
                             (("gemv", "square_1k"), ("dequant", "square_1k"), ("gemv", "q_proj_0p8b"),
                              ("gemv", "out_proj_0p8b"), ("gemv", "lm_head_0p8b")))


def shard_shapes(q4k, inputs, torch, dev, stream):
    """One GPU's share of the 9B decode matrices split eight ways: a
    vocabulary shard of the lm_head (31,040 rows), a row shard of gate and up
    (SwiGLU over 1536 rows) and a split-K shard of down (K = 1536, a partial
    y that an all-reduce would sum)."""
    return graph_timed_calls(q4k, inputs, torch, dev, stream,
                             (("gemv", "lm_head_9b_shard8"), ("swiglu", "gate_9b_shard8"), ("gemv", "down_9b_kshard8")))


def graph_timed_calls(q4k, inputs, torch, dev, stream, cases):
    """GEMV, SwiGLU or dequant calls, weights rotated over >= 512 MiB of
    copies: the launches captured in a HIP graph (the rate a decode loop sees;
    eager Python calls of small sizes are bound by the host), the same
    launches eager back to back, and single-launch percentiles."""
    out = {}
    for kind, name in cases:
        n, k = inputs.SHAPES[name]
        mats = 2 if kind == "swiglu" else 1
        w0 = torch.from_numpy(inputs.make_q4k(n, k, config_id=7, tensor_id=1).reshape(-1)).to(dev)
        copies = max(1, -(-(512 << 20) // (mats * w0.numel())))
        ws = [w0] + [w0.clone() for _ in range(mats * copies - 1)]
        x = torch.from_numpy(inputs.make_x(1, k, config_id=7)[0]).to(dev)
        if kind == "gemv":
            y = torch.empty(n, dtype=torch.float32, device=dev)

            def fn(i, s=stream):
                q4k.gemv(ws[i % copies], x, y=y, stream=s)

            nbytes = w0.numel() + 4 * (n + k)
        elif kind == "swiglu":
            y = torch.empty(n, dtype=torch.float32, device=dev)

            def fn(i, s=stream):
                c = i % copies
                q4k.fused_swiglu(ws[2 * c], ws[2 * c + 1], x, h=y, stream=s)

            nbytes = 2 * w0.numel() + 4 * (n + k)
        else:
            y = torch.empty((n, k), dtype=torch.float32, device=dev)

            def fn(i, s=stream):
                q4k.dequant(ws[i % copies], k, out=y, stream=s)

            nbytes = w0.numel() + 4 * n * k
        # enough launches to touch every copy: >= 512 MiB, beyond the Infinity Cache
        nl = max(200, copies)
        t = _time_launches(fn, torch, stream, nl, 20)
        # the same launches captured into a HIP graph, timed over one replay
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(nl):
                fn(i, None)  # the capture stream
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        warm_up(graph.replay, torch, stream)
        a.record(stream)
        graph.replay()
        b.record(stream)
        torch.cuda.synchronize()
        tg = a.elapsed_time(b) / nl * 1e-3
        del graph
        out[f"{kind} {name}"] = {"shape": f"{n}x{k}", "bytes": nbytes, "graph_us": round(tg * 1e6, 3),
                                 "graph_GB/s": round(nbytes / tg / 1e9, 1),
                                 "frac_hbm_peak": round(nbytes / tg / HBM_PEAK_GBS / 1e9, 4),
                                 "eager_us": round(t * 1e6, 3), "per_launch_us": _per_launch(fn, torch, stream, 100)}
        del ws, y
    return out


def stream_read_ceiling(torch, dev, stream, lm_head_gbs):
    """The device's achievable HBM read rate, for context: the read-only
    streaming kernel (libq4k_stream.so) over 1 GiB, the best of a few grid
    sizes, load depths and the two cache policies.  None if that library is
    not built."""
    import ctypes

    from q4_dequant_gemv_amd import build as hip_build

    if not os.path.exists(hip_build.STREAM_LIB):
        log("[bench] libq4k_stream.so not built: no streaming ceiling")
        return None
    lib = ctypes.CDLL(hip_build.STREAM_LIB)
    lib.q4k_stream_read.restype = ctypes.c_int
    lib.q4k_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                    ctypes.c_int, ctypes.c_void_p]
    nbytes = 1 << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(7)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    grids = [cus * g for g in (1, 2, 3, 4, 8)]
    out = torch.empty(max(grids) * 256, dtype=torch.int32, device=dev)
    s = ctypes.c_void_p(stream.cuda_stream)
    best = None
    for policy in (0, 2):
        for grid in grids:
            for unroll in (4, 8):
                def call(i):
                    rc = lib.q4k_stream_read(ctypes.c_void_p(buf.data_ptr()), nbytes, ctypes.c_void_p(out.data_ptr()),
                                             grid, unroll, policy, s)
                    if rc != 0:
                        raise RuntimeError(f"q4k_stream_read: hip error {rc}")

                t = _time_launches(call, torch, stream, 20, 3)
                gbs = nbytes / t / 1e9
                if best is None or gbs > best["GB/s"]:
                    best = {"GB/s": round(gbs, 1), "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4), "grid": grid,
                            "loads_in_flight_per_thread": unroll, "cache_policy": "non-temporal" if policy else "default"}
    best["lm_head_gemv_frac_of_it"] = round(lm_head_gbs / best["GB/s"], 4)
    del buf, out
    return best


def _per_launch(fn, torch, stream, reps):
    """p10 / median / p90 of single launches, each between its own pair of
    events on the launch stream (the events add a little to short kernels)."""
    import numpy as np

    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    torch.cuda.synchronize()
    for i, (e0, e1) in enumerate(evs):
        e0.record(stream)
        fn(i)
        e1.record(stream)
    torch.cuda.synchronize()
    t = np.sort(np.array([e0.elapsed_time(e1) * 1e3 for e0, e1 in evs]))
    return {"p10": round(float(np.percentile(t, 10)), 3), "median": round(float(np.median(t)), 3),
            "p90": round(float(np.percentile(t, 90)), 3), "n": reps}


def warm_up(run_region, torch, stream, seconds=0.1):
    """Runs `run_region` back to back for at least `seconds` of GPU time and
    returns without synchronizing, so that the timed work queued next starts
    on a busy GPU.  After the host has kept the GPU idle for a few
    milliseconds (a synchronize, a graph capture) the device runs the same
    work up to a fifth slower at first and speeds up over some tens of
    milliseconds of load (per-step times of back-to-back 20-step replays
    falling from 130 to 109 us); timing starts past that."""
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(stream)
    run_region()
    b.record(stream)
    torch.cuda.synchronize()
    one = max(a.elapsed_time(b) * 1e-3, 1e-6)
    for _ in range(int(seconds / one) + 1):
        run_region()


def _time_graph(fn, count, torch, stream):
    """Mean time of one fn(i, s) when `count` of them are recorded into one HIP
    graph (s: the capture stream) and the graph is replayed after a warm-up."""
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(count):
            fn(i, None)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    warm_up(graph.replay, torch, stream)
    a.record(stream)
    graph.replay()
    b.record(stream)
    torch.cuda.synchronize()
    del graph
    return a.elapsed_time(b) / count * 1e-3


def _time_launches(fn, torch, stream, steps, warmup):
    """Mean time of one fn(i) over `steps` back-to-back calls between two
    events on the launch stream, after a warm-up (warm_up)."""
    for i in range(warmup):
        fn(i)
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    warm_up(lambda: [fn(i) for i in range(steps)], torch, stream)
    a.record(stream)
    for i in range(steps):
        fn(i)
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps * 1e-3


def decode_blocks(q4k, inputs, torch, dev, stream, steps, warmup):
    """The multi-matrix and residual entry points on their decode workloads,
    each beside the separate calls it replaces; weights rotated over
    >= 512 MiB of copies:
      * the four input projections of a 0.8B linear-attention layer (qkv 6144,
        z 2048, a 16, b 16 rows, K = 1024) against one x: one gemv_multi
        launch, and four gemv launches;
      * the 9B down projection (4096 x 12288) with the residual added in its
        epilogue, and the plain GEMV."""
    out = {}
    names = inputs.GDN_PROJECTIONS_0P8B
    k = inputs.SHAPES[names[0]][1]
    ns = [inputs.SHAPES[nm][0] for nm in names]
    mats = [inputs.make_q4k(n, k, config_id=4, tensor_id=i).reshape(-1) for i, n in enumerate(ns)]
    nbytes = sum(m.nbytes for m in mats)
    copies = max(1, -(-(512 << 20) // nbytes))
    sets = [[torch.from_numpy(m).to(dev) for m in mats] for _ in range(copies)]
    x = torch.from_numpy(inputs.make_x(1, k, config_id=4, tensor_id=100)[0]).to(dev)
    ys = [torch.empty(n, dtype=torch.float32, device=dev) for n in ns]
    t_multi = _time_launches(lambda i: q4k.gemv_multi(sets[i % copies], x, ys=ys, ns=ns, stream=stream), torch,
                             stream, steps, warmup)

    def four(i):
        for w, y, n in zip(sets[i % copies], ys, ns):
            q4k.gemv(w, x, y=y, n=n, stream=stream)

    t_four = _time_launches(four, torch, stream, steps, warmup)
    # the same launches recorded into HIP graphs (device time, no host cost
    # per call): one multi node against four gemv nodes per step
    nl = max(200, copies)
    g_multi = _time_graph(lambda i, s: q4k.gemv_multi(sets[i % copies], x, ys=ys, ns=ns, stream=s), nl, torch,
                          stream)

    def four_g(i, s):
        for w, y, n in zip(sets[i % copies], ys, ns):
            q4k.gemv(w, x, y=y, n=n, stream=s)

    g_four = _time_graph(four_g, nl, torch, stream)
    abytes = nbytes + 4 * k + 4 * sum(ns)
    out["gdn_in_proj_0p8b"] = {"weight_bytes": nbytes, "multi_us": round(t_multi * 1e6, 3),
                               "multi_GB/s": round(abytes / t_multi / 1e9, 1),
                               "four_calls_us": round(t_four * 1e6, 3),
                               "four_calls_GB/s": round(abytes / t_four / 1e9, 1),
                               "multi_graph_us": round(g_multi * 1e6, 3),
                               "four_calls_graph_us": round(g_four * 1e6, 3)}
    del sets
    n, k = inputs.SHAPES["down_9b"]
    w0 = inputs.make_q4k(n, k, config_id=6, tensor_id=1).reshape(-1)
    copies = max(1, -(-(512 << 20) // w0.nbytes))
    ws = [torch.from_numpy(w0).to(dev) for _ in range(copies)]
    h = torch.from_numpy(inputs.make_x(1, k, config_id=6, tensor_id=101)[0]).to(dev)
    r = torch.from_numpy(inputs.make_x(1, n, config_id=6, tensor_id=102)[0]).to(dev)
    y = torch.empty(n, dtype=torch.float32, device=dev)
    t_res = _time_launches(lambda i: q4k.gemv_residual(ws[i % copies], h, r, y=y, stream=stream), torch, stream,
                           steps, warmup)
    t_plain = _time_launches(lambda i: q4k.gemv(ws[i % copies], h, y=y, stream=stream), torch, stream, steps,
                             warmup)
    abytes = w0.nbytes + 4 * k + 8 * n
    out["down_residual_9b"] = {"weight_bytes": w0.nbytes, "residual_us": round(t_res * 1e6, 3),
                               "residual_GB/s": round(abytes / t_res / 1e9, 1),
                               "plain_gemv_us": round(t_plain * 1e6, 3)}
    del ws
    return out


def q8_0_kernels(q4k, inputs, torch, dev, stream, steps, warmup):
    """The Q8_0 GEMV on the 9B shapes (34-byte blocks of 32 weights, 1.0625
    bytes per weight), weights rotated over >= 512 MiB of copies."""
    out = {}
    for nm, tid in (("lm_head_9b", 0), ("gate_9b", 1), ("down_9b", 2)):
        n, k = inputs.SHAPES[nm]
        w0 = inputs.make_q8_0(n, k, config_id=52, tensor_id=tid).reshape(-1)
        copies = max(1, -(-(512 << 20) // w0.nbytes))
        ws = [torch.from_numpy(w0).to(dev) for _ in range(copies)]
        x = torch.from_numpy(inputs.make_x(1, k, config_id=52, tensor_id=100 + tid)[0]).to(dev)
        y = torch.empty(n, dtype=torch.float32, device=dev)
        t = _time_launches(lambda i: q4k.q8_0_gemv(ws[i % copies], x, y=y, stream=stream), torch, stream, steps,
                           warmup)
        abytes = w0.nbytes + 4 * k + 4 * n
        out[nm] = {"weight_bytes": w0.nbytes, "mean_us": round(t * 1e6, 3), "GB/s": round(abytes / t / 1e9, 1),
                   "frac_hbm_peak": round(abytes / t / 1e9 / HBM_PEAK_GBS, 4)}
        del ws
    return out


def f16_variants(q4k, inputs, torch, dev, stream, steps, warmup, batched):
    """f16 activations and outputs (q4k_gemv_dt, q4k_gemv_batched_dt) on the
    9B lm_head and gate, beside the f32 calls; weights rotated over >= 512 MiB."""
    out = {}
    n, k = inputs.SHAPES["lm_head_9b"]
    w = torch.from_numpy(inputs.make_q4k(n, k, config_id=61, tensor_id=0).reshape(-1)).to(dev)
    x = torch.from_numpy(inputs.make_x(1, k, config_id=61)[0]).to(dev)
    xh = x.half()
    y = torch.empty(n, dtype=torch.float16, device=dev)
    t = _time_launches(lambda i: q4k.gemv_dt(w, xh, y=y, stream=stream), torch, stream, steps, warmup)
    out["lm_head_9b f16->f16"] = {"mean_us": round(t * 1e6, 3),
                                  "GB/s": round((w.numel() + 2 * k + 2 * n) / t / 1e9, 1)}
    del w
    if batched:
        n, k = inputs.SHAPES["gate_9b"]
        w0 = torch.from_numpy(inputs.make_q4k(n, k, config_id=61, tensor_id=1).reshape(-1)).to(dev)
        copies = max(1, -(-(512 << 20) // w0.numel()))
        ws = [w0] + [w0.clone() for _ in range(copies - 1)]
        for m in (16, 64):
            xs = torch.from_numpy(inputs.make_x(m, k, config_id=61, tensor_id=m)).to(dev)
            for label, xin, yd in (("f32->f32", xs, torch.float32), ("f16->f16", xs.half(), torch.float16)):
                yb = torch.empty((m, n), dtype=yd, device=dev)
                t = _time_launches(lambda i: q4k.gemv_batched_dt(ws[i % copies], xin, y=yb, stream=stream), torch,
                                   stream, min(steps, 50), min(warmup, 5))
                out[f"gate_9b m={m} {label}"] = {"mean_us": round(t * 1e6, 2),
                                                 "TFLOP/s": round(2.0 * m * n * k / t / 1e12, 2)}
        del ws
    return out


F16_DENSE_PEAK_TFLOPS = 2500.0


def prefill_kernels(q4k, inputs, torch, dev, stream):
    """The prefill GEMM (q4k_prefill_gemm, f16 activations, f32 outputs) on
    the 9B gate and down projections at m = 128 .. 2048 tokens, and, for
    comparison, the skinny-GEMM path on the same activations widened to f32
    (an f16 batched call of these sizes runs the prefill GEMM itself)."""
    out = {}
    for nm in ("gate_9b", "down_9b"):
        n, k = inputs.SHAPES[nm]
        w = torch.from_numpy(inputs.make_q4k(n, k, config_id=73, tensor_id=0).reshape(-1)).to(dev)
        for m in (128, 256, 512, 1024, 2048):
            xh = torch.from_numpy(inputs.make_x(m, k, config_id=73, tensor_id=m)).to(dev).half()
            y = torch.empty((m, n), dtype=torch.float32, device=dev)
            t = _time_launches(lambda i: q4k.prefill_gemm(w, xh, y=y, stream=stream), torch, stream, 20, 3)
            tf = 2.0 * m * n * k / t / 1e12
            rec = {"mean_us": round(t * 1e6, 2), "TFLOP/s": round(tf, 1),
                   "frac_f16_peak": round(tf / F16_DENSE_PEAK_TFLOPS, 4)}
            if m <= 512:
                xf = xh.float()
                tb = _time_launches(lambda i: q4k.gemv_batched_dt(w, xf, y=y, stream=stream), torch, stream, 10, 2)
                rec["batched_f32_call_us"] = round(tb * 1e6, 2)
                del xf
            out[f"{nm} m={m}"] = rec
        del w
    return out


def time_call(fn, torch, reps=50, warm=5):
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    s = torch.cuda.current_stream()
    for a, b in evs:
        a.record(s)
        fn()
        b.record(s)
    torch.cuda.synchronize()
    import numpy as np

    return float(np.median([a.elapsed_time(b) for a, b in evs])) * 1e-3


def run_case(case, steps, warmup, q4k, inputs, torch, np, dev):
    """One kernel at one shape, rotated over >= 512 MiB of weight copies.
    `copy` instead runs a plain 512 MiB device-to-device copy (the reference
    kernel that calibrates the profiler's byte counters)."""
    if case == "copy":
        src = torch.empty(512 << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(warmup):
            dst.copy_(src)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(steps):
            dst.copy_(src)
        b.record()
        torch.cuda.synchronize()
        t = a.elapsed_time(b) / steps * 1e-3
        log(f"[case] copy 512 MiB: {t * 1e6:.1f} us per copy, {2 * src.numel() / t / 1e9:.1f} GB/s read+write")
        return
    parts = case.split(":")
    kind, name = parts[0], parts[-1]
    if kind == "prefill":
        m = int(parts[1])
        n, k = inputs.SHAPES[name]
        w = torch.from_numpy(inputs.make_q4k(n, k, config_id=7, tensor_id=1).reshape(-1)).to(dev)
        xh = torch.from_numpy(inputs.make_x(m, k, config_id=7)).to(dev).half()
        y = torch.empty((m, n), dtype=torch.float32, device=dev)
        stream = torch.cuda.current_stream()
        t = _time_launches(lambda i: q4k.prefill_gemm(w, xh, y=y), torch, stream, steps, warmup)
        log(f"[case] {case}: {t * 1e6:.2f} us per call, {2.0 * m * n * k / t / 1e12:.1f} TFLOP/s")
        return
    if kind == "multi":
        if name != "gdn_0p8b":
            raise SystemExit("multi case: only multi:gdn_0p8b")
        names = inputs.GDN_PROJECTIONS_0P8B
        k = inputs.SHAPES[names[0]][1]
        ns = [inputs.SHAPES[nm][0] for nm in names]
        mats = [inputs.make_q4k(n, k, config_id=7, tensor_id=i).reshape(-1) for i, n in enumerate(ns)]
        nbytes = sum(m.nbytes for m in mats)
        copies = max(1, -(-(512 << 20) // nbytes))
        sets = [[torch.from_numpy(m).to(dev) for m in mats] for _ in range(copies)]
        x = torch.from_numpy(inputs.make_x(1, k, config_id=7)[0]).to(dev)
        ys = [torch.empty(n, dtype=torch.float32, device=dev) for n in ns]
        stream = torch.cuda.current_stream()
        t = _time_launches(lambda i: q4k.gemv_multi(sets[i % copies], x, ys=ys, ns=ns), torch, stream, steps,
                           warmup)
        log(f"[case] {case}: {t * 1e6:.2f} us per call (host-enqueued back to back), {nbytes / t / 1e9:.1f} GB/s")
        return
    m = int(parts[1]) if kind == "batched" else 1
    n, k = inputs.SHAPES[name]
    if kind == "q8_0":
        w0 = inputs.make_q8_0(n, k, config_id=7, tensor_id=1).reshape(-1)
    else:
        w0 = inputs.make_q4k(n, k, config_id=7, tensor_id=1).reshape(-1)
    mats = 2 if kind == "swiglu" else 1
    copies = max(1, -(-(512 << 20) // (mats * w0.nbytes)))
    ws = [torch.from_numpy(w0).to(dev) for _ in range(copies * mats)]
    xs = torch.from_numpy(inputs.make_x(m, k, config_id=7)).to(dev)
    out = torch.empty((n, k) if kind == "dequant" else (m, n), dtype=torch.float32, device=dev)
    res = torch.from_numpy(inputs.make_x(1, n, config_id=7, tensor_id=102)[0]).to(dev)

    def call(i):
        c = i % copies
        if kind == "gemv":
            q4k.gemv(ws[c], xs[0], y=out[0])
        elif kind == "swiglu":
            q4k.fused_swiglu(ws[2 * c], ws[2 * c + 1], xs[0], h=out[0])
        elif kind == "batched":
            q4k.gemv_batched(ws[c], xs, y=out)
        elif kind == "dequant":
            q4k.dequant(ws[c], k, out=out)
        elif kind == "residual":
            q4k.gemv_residual(ws[c], xs[0], res, y=out[0])
        elif kind == "q8_0":
            q4k.q8_0_gemv(ws[c], xs[0], y=out[0])
        else:
            raise SystemExit(f"unknown case kind {kind}")

    for i in range(warmup):
        call(i)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(steps):
        call(i)
    b.record()
    torch.cuda.synchronize()
    t = a.elapsed_time(b) / steps * 1e-3
    nbytes = mats * w0.nbytes + (out.numel() * 4 if kind == "dequant" else 0)
    log(f"[case] {case}: {t * 1e6:.2f} us per call (host-enqueued back to back), {nbytes / t / 1e9:.1f} GB/s")


def sweep(q4k, inputs, torch, np, dev):
    """Every kernel at every config shape; weights rotated over >= 512 MiB of
    copies so repeated calls do not hit the Infinity Cache."""
    log("[sweep] kernel  shape  m  us  GB/s(weights)  frac")

    def copies(nbytes):
        return max(1, -(-(512 << 20) // nbytes))

    def gemv_case(name, n, k):
        w0 = inputs.make_q4k(n, k, config_id=7, tensor_id=1).reshape(-1)
        ws = [torch.from_numpy(w0).to(dev) for _ in range(copies(w0.nbytes))]
        x = torch.from_numpy(inputs.make_x(1, k, config_id=7)[0]).to(dev)
        y = torch.empty(n, dtype=torch.float32, device=dev)
        it = iter(range(10 ** 9))
        t = time_call(lambda: q4k.gemv(ws[next(it) % len(ws)], x, y=y), torch)
        log(f"[sweep] gemv {name} {n}x{k} m=1 {t * 1e6:.2f} {w0.nbytes / t / 1e9:.1f} {w0.nbytes / t / 8e12:.3f}")
        del ws

    for name in ("square_1k", "q_proj_0p8b", "out_proj_0p8b", "lm_head_0p8b", "down_9b", "gate_9b", "lm_head_9b"):
        gemv_case(name, *inputs.SHAPES[name])
    n, k = inputs.SHAPES["gate_9b"]
    g0 = inputs.make_q4k(n, k, config_id=7, tensor_id=2).reshape(-1)
    c = copies(2 * g0.nbytes)
    gs = [torch.from_numpy(g0).to(dev) for _ in range(c)]
    us = [torch.from_numpy(g0).to(dev) for _ in range(c)]
    x = torch.from_numpy(inputs.make_x(1, k, config_id=7)[0]).to(dev)
    hh = torch.empty(n, dtype=torch.float32, device=dev)
    it = iter(range(10 ** 9))

    def sw():
        i = next(it) % c
        q4k.fused_swiglu(gs[i], us[i], x, h=hh)

    t = time_call(sw, torch)
    log(f"[sweep] swiglu gate+up {n}x{k} m=1 {t * 1e6:.2f} {2 * g0.nbytes / t / 1e9:.1f} {2 * g0.nbytes / t / 8e12:.3f}")
    del gs, us
    for name in ("gate_9b", "down_9b"):
        n, k = inputs.SHAPES[name]
        w0 = inputs.make_q4k(n, k, config_id=7, tensor_id=3).reshape(-1)
        ws = [torch.from_numpy(w0).to(dev) for _ in range(copies(w0.nbytes))]
        for m in (1, 4, 16, 32, 64):
            xs = torch.from_numpy(inputs.make_x(m, k, config_id=7)).to(dev)
            yy = torch.empty((m, n), dtype=torch.float32, device=dev)
            it2 = iter(range(10 ** 9))
            t = time_call(lambda: q4k.gemv_batched(ws[next(it2) % len(ws)], xs, y=yy), torch)
            tflops = 2.0 * m * n * k / t / 1e12
            log(f"[sweep] batched {name} {n}x{k} m={m} {t * 1e6:.2f} {w0.nbytes / t / 1e9:.1f} "
                f"{w0.nbytes / t / 8e12:.3f} ({tflops:.1f} TFLOP/s)")
        del ws
    n, k = inputs.SHAPES["lm_head_0p8b"]
    w0 = inputs.make_q4k(n, k, config_id=7, tensor_id=4).reshape(-1)
    ws = [torch.from_numpy(w0).to(dev) for _ in range(copies(w0.nbytes))]
    out = torch.empty((n, k), dtype=torch.float32, device=dev)
    it3 = iter(range(10 ** 9))
    t = time_call(lambda: q4k.dequant(ws[next(it3) % len(ws)], k, out=out), torch, reps=20)
    tot = w0.nbytes + out.numel() * 4
    log(f"[sweep] dequant {n}x{k} {t * 1e6:.2f} {tot / t / 1e9:.1f} (read+write) {tot / t / 8e12:.3f}")


if __name__ == "__main__":
    main()
