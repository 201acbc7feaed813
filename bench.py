"""VSA forward benchmark on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

Workload: Wan-1.3B 480p shape -- token grid 16x14x26 (5824 tokens) padded to
16x16x28 (7168 tokens, 112 cubes), 12 heads, d = 128, bf16, top-K = 14 of 112
cubes (87.5% sparse), synthetic seeded q/k/v.  A step is one vsa_forward call
(raster q/k/v in HBM -> O_fine, O_coarse, block indices, LSE); inputs rotate
over 5 independent sets (268 MB) so calls read HBM rather than a warm cache.

Prints one JSON line.  Besides the headline (ms per forward, with the median
and 10th/90th percentile of single calls) it reports the fine kernel alone
(vsa_fine on cube-order inputs), coarse + fine, the in-repo dense flash
attention on the same padded sequence (the faster of the dense kernel
vsa_dense and the fine kernel with every cube selected) and on the 5824 real
tokens, valid x valid ("useful") TFLOPS, the
forward and fine-stage times of every workload of the pages (tiny fp32,
410M DiT, Wan-1.3B, Wan-14B), the fine kernel's MFMA roofline, and the fp64
CPU oracle timed on the host cores.  An "fp8" object reports the same shape
through the FP8 path (E4M3 q/k/v with per-cube scales): the quantization
pass, the FP8 fine kernel with its roofline against the FP8 MFMA peak, and
the whole FP8 forward.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "VSA fwd ms + sparse TFLOPS (% bf16 MFMA peak), 7168 tok, 12 heads, 87.5% sparse"
N_SETS = 5


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    # the GPU clock takes a few hundred calls to settle; untimed
    ap.add_argument("--warmup", type=int, default=400)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-reps", type=int, default=5)
    ap.add_argument("--workload", choices=["wan1.3b", "wan14b"], default="wan1.3b",
                    help="shape of --stage runs (the full bench always uses wan1.3b)")
    ap.add_argument("--stage", choices=["all", "forward", "fine", "fine_raster", "dense", "coarse",
                                        "reorder", "backward",
                                        "fine_fp8", "forward_fp8", "quantize_fp8"],
                    default="all",
                    help="time one stage only (for profiler runs); prints a short JSON line")
    return ap.parse_args()


def timed(fn, steps, warmup, rotate):
    """Average ms per call of fn(i) over `steps` calls, HIP events on the current stream."""
    import torch
    for i in range(warmup):
        fn(i % rotate)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(steps):
        fn(i % rotate)
    stop.record()
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / steps


def per_launch(fn, launches, warmup, rotate):
    """Average duration of single launches, each bracketed by its own HIP events
    on the current stream (launches do not overlap, as under a profiler)."""
    import torch
    for i in range(warmup):
        fn(i % rotate)
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(launches)]
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(pairs):
        a.record()
        fn(i % rotate)
        b.record()
    torch.cuda.synchronize()
    return sum(a.elapsed_time(b) for a, b in pairs) / launches


def per_call(fn, calls, warmup, rotate):
    """Median, 10th and 90th percentile (ms) of single calls, each between its own
    HIP events on the current stream."""
    import torch
    for i in range(warmup):
        fn(i % rotate)
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(calls)]
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(pairs):
        a.record()
        fn(i % rotate)
        b.record()
    torch.cuda.synchronize()
    t = sorted(a.elapsed_time(b) for a, b in pairs)
    pick = lambda f: t[min(len(t) - 1, int(f * len(t)))]
    return pick(0.5), pick(0.1), pick(0.9)


def settle_clock(fn, rotate, seconds=1.0):
    """Untimed calls of fn for at least `seconds` of wall time before any
    measurement: an idle GPU starts at a low clock and needs some hundred
    milliseconds of load to reach its working clock, which a few warm-up
    calls of a 0.1 ms kernel do not give.  Returns the wall time spent (ms)."""
    import torch
    t0 = time.perf_counter()
    i = 0
    while True:
        for _ in range(50):
            fn(i % rotate)
            i += 1
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= seconds:
            return round((time.perf_counter() - t0) * 1e3, 1)


def valid_counts(w):
    """Valid slots n_c of every cube of a workload's grid, cube order."""
    ct, ch, cw = -(-w.T // 4), -(-w.Hh // 4), -(-w.Ww // 4)
    return [min(4, w.T - 4 * t) * min(4, w.Hh - 4 * h) * min(4, w.Ww - 4 * x)
            for t in range(ct) for h in range(ch) for x in range(cw)]


def graph_timed(fn, steps, warmup):
    """ms per call of fn() captured once into a HIP graph and replayed: device
    time without the host cost of each binding call, which dominates for the
    small workloads."""
    import torch
    fn()                                   # allocations and library set-up outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fn()
    return timed(lambda i: graph.replay(), steps, warmup, 1)


def graph_timed_sets(fns, steps, warmup):
    """graph_timed over several input sets: one graph per fns[i], replayed in
    rotation, so that each call reads its own inputs from HBM."""
    import torch
    graphs = []
    for fn in fns:
        fn()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            fn()
        graphs.append(graph)
    return timed(lambda i: graphs[i].replay(), steps, warmup, len(graphs))


def per_config(args, dev):
    """vsa_forward and the fine stage alone (cube-order inputs) for every workload
    of the pages: one seeded input set each, computed-sparse and useful TFLOPS.
    Times are HIP-graph replays (device time per call)."""
    import torch
    import block_sparse_attention_cube_amd as vsa
    from block_sparse_attention_cube_amd import flops
    from synth import configs, inputs
    out = []
    for w in (configs.TINY_F32, configs.DIT_410M, configs.WAN_1_3B, configs.WAN_14B):
        grid = (w.T, w.Hh, w.Ww)
        dtype = torch.float32 if w.dtype == "f32" else torch.bfloat16
        host = inputs.make_inputs(w, seed=0)
        s = {n: inputs.as_torch(host[n], w.dtype, dev) for n in "qkv"}
        del host
        big = w.N * w.H > 1_000_000
        steps, warm = (10, 2) if big else (max(10, args.steps // 2), max(2, args.warmup // 2))
        plan = vsa.ForwardPlan(w.B, w.H, grid, w.d, w.topk, dtype, dev)
        f_ms = graph_timed(lambda: plan.run(s["q"], s["k"], s["v"]), steps, warm)
        cube = {n: vsa.reorder(s[n], grid) for n in "qkv"}
        _, idx = vsa.coarse(cube["q"], cube["k"], cube["v"], grid, w.topk)
        obuf = torch.empty_like(cube["q"])
        fine_ms = graph_timed(lambda: vsa.fine(cube["q"], cube["k"], cube["v"], idx, grid, out=obuf),
                              steps, warm)
        fl = flops.fine_forward_flops(w.B, w.H, w.C, w.topk, w.d)
        useful = flops.useful_fine_flops(w.B, w.H, w.d, valid_counts(w), idx.cpu().numpy())
        rec = {"workload": w.name, "dtype": w.dtype, "B": w.B, "H": w.H, "grid": list(grid),
               "d": w.d, "cubes": w.C, "topk": w.topk,
               "forward_ms": round(f_ms, 5), "fine_ms": round(fine_ms, 5),
               "fine_sparse_tflops": round(fl / (fine_ms * 1e-3) / 1e12, 2),
               "fine_useful_tflops": round(useful / (fine_ms * 1e-3) / 1e12, 2),
               "useful_over_computed": round(useful / fl, 4),
               "executed_over_computed": round(
                   flops.executed_fine_flops(grid, w.d, idx.cpu().numpy()) / fl, 4)
               if w.dtype == "bf16" else 1.0,
               "timing": "hip graph replay"}
        del cube, obuf, plan      # the cube-order copies are not needed below
        if w.dtype == "bf16" and w.d == 128:
            rec.update(fp8_config(w, grid, s, idx, fl, steps, warm, dev))
        out.append(rec)
        del s, idx
        torch.cuda.empty_cache()
    return out


def fp8_config(w, grid, s, idx, fl, steps, warm, dev):
    """The FP8 forward and FP8 fine stage of one d = 128 workload (HIP-graph
    replays; the fine stage uses the bf16 path's block indices)."""
    import torch
    import block_sparse_attention_cube_amd as vsa
    plan = vsa.ForwardFp8Plan(w.B, w.H, grid, w.d, w.topk, dev)
    fwd_ms = graph_timed(lambda: plan.run(s["q"], s["k"], s["v"]), steps, warm)
    del plan
    q8 = vsa.quantize_fp8(s["q"], s["k"], s["v"], grid)
    obuf = torch.empty((w.B, w.H, w.Np, w.d), dtype=torch.bfloat16, device=dev)
    fine_ms = graph_timed(lambda: vsa.fine_fp8(*q8, idx, grid, return_lse=False, out=obuf),
                          steps, warm)
    return {"fp8_forward_ms": round(fwd_ms, 5), "fp8_fine_ms": round(fine_ms, 5),
            "fp8_fine_sparse_tflops": round(fl / (fine_ms * 1e-3) / 1e12, 2)}


def traffic_record(kernel_source, record="fine_fwd_wan1.3b_traffic.json"):
    """HBM bytes per launch from the committed counter record, if it was taken
    on the current kernel source (else None)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", record)
    try:
        rec = json.load(open(path))
        src = open(os.path.join(ROOT, kernel_source), "rb").read()
    except OSError:
        return None
    if rec.get("source_sha256") != hashlib.sha256(src).hexdigest():
        return None
    return rec["traffic_bytes"]


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(w, x, reps):
    from threadpoolctl import threadpool_info, threadpool_limits
    from oracle import vsa_oracle as vo
    host_cpus = os.cpu_count() or 1
    try:
        allowed = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        allowed = host_cpus
    with threadpool_limits(limits=allowed):
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        t0 = time.perf_counter()
        for _ in range(reps):
            vo.forward(x["q"], x["k"], x["v"], w.T, w.Hh, w.Ww, w.topk)
        dt = time.perf_counter() - t0
    return {"value": round(dt / reps * 1e3, 3), "unit": "ms", "cores": threads, "kind": "oracle",
            "host_cpus": host_cpus, "cpus_allowed": allowed, "blas_threads": threads,
            "cpu_model": cpu_model(),
            "sample": f"whole {w.name} forward (all {w.H} heads, {w.C} query cubes), fp64 NumPy, "
                      f"{reps} repetitions, {dt:.1f} s total"}


def sparsity_sweep(args, dev):
    """Forward and backward at top-K ratios 0.2 / 0.1 / 0.03 of the Wan-1.3B shape."""
    import torch
    import block_sparse_attention_cube_amd as vsa
    from block_sparse_attention_cube_amd import flops
    from synth import configs, inputs
    out = []
    steps = max(10, args.steps // 4)
    warm = max(2, args.warmup // 4)
    for w in configs.SWEEP:
        grid = (w.T, w.Hh, w.Ww)
        host = [inputs.make_inputs(w, seed=s, grads=True) for s in range(2)]
        sets = [{n: inputs.as_torch(h[n], w.dtype, dev) for n in h} for h in host]
        # the training pair: the forward keeps its per-cube means for the backward
        fwd = vsa.ForwardPlan(w.B, w.H, grid, w.d, w.topk, torch.bfloat16, dev, keep_means=True)
        bwd = vsa.BackwardPlan(w.B, w.H, grid, w.d, w.topk, torch.bfloat16, dev)
        outs = []
        for s in sets:
            of, oc, idx, lse = fwd.run(s["q"], s["k"], s["v"])
            outs.append((of.clone(), idx.clone(), lse.clone(), fwd.means.clone()))
        # each call timed two ways: back to back from the host (at small top-K
        # the host cost of a binding call exceeds the GPU work of a forward)
        # and as HIP-graph replays (which add ~1 us per kernel node); the
        # faster of the two is reported
        fcall = lambda i: fwd.run(sets[i]["q"], sets[i]["k"], sets[i]["v"])
        bcall = lambda i: bwd.run(sets[i]["q"], sets[i]["k"], sets[i]["v"], outs[i][0],
                                  outs[i][2], outs[i][1], sets[i]["do_fine"],
                                  sets[i]["do_coarse"], means=outs[i][3])
        settle_clock(bcall, 2, 0.5)
        f_eager, b_eager = timed(fcall, steps, warm, 2), timed(bcall, steps, warm, 2)
        f_graph = graph_timed_sets([lambda i=i: fcall(i) for i in range(2)], steps, warm)
        b_graph = graph_timed_sets([lambda i=i: bcall(i) for i in range(2)], steps, warm)
        f_ms, b_ms = min(f_eager, f_graph), min(b_eager, b_graph)
        ff = flops.fine_forward_flops(w.B, w.H, w.C, w.topk, w.d)
        fb = flops.fine_backward_flops(w.B, w.H, w.C, w.topk, w.d)
        out.append({"topk": w.topk, "sparsity": round(1 - w.topk / w.C, 4),
                    "fwd_ms": round(f_ms, 5), "bwd_ms": round(b_ms, 5),
                    "fwd_tflops": round(ff / (f_ms * 1e-3) / 1e12, 2),
                    "bwd_tflops": round(fb / (b_ms * 1e-3) / 1e12, 2),
                    "fwd_eager_ms": round(f_eager, 5), "fwd_graph_ms": round(f_graph, 5),
                    "bwd_eager_ms": round(b_eager, 5), "bwd_graph_ms": round(b_graph, 5),
                    "timing": "faster of back-to-back calls and HIP-graph replays, "
                              "2 input sets rotated"})
    return out


def fp8_section(args, w, grid, sets, idx_sets, dev):
    """The Wan-1.3B shape through the FP8 path: quantization, the FP8 fine
    kernel (cube-order output, the block indices of the bf16 coarse stage)
    and the whole FP8 forward, inputs rotated as for the headline."""
    import torch
    import block_sparse_attention_cube_amd as vsa
    from block_sparse_attention_cube_amd import flops
    n = len(sets)
    q8s = [vsa.quantize_fp8(s["q"], s["k"], s["v"], grid) for s in sets]
    obuf = torch.empty((w.B, w.H, w.Np, w.d), dtype=torch.bfloat16, device=dev)
    quant = lambda i: vsa.quantize_fp8(sets[i]["q"], sets[i]["k"], sets[i]["v"], grid)
    fine8 = lambda i: vsa.fine_fp8(*q8s[i], idx_sets[i], grid, return_lse=False, out=obuf)
    plan = vsa.ForwardFp8Plan(w.B, w.H, grid, w.d, w.topk, dev)
    fwd8 = lambda i: plan.run(sets[i]["q"], sets[i]["k"], sets[i]["v"])
    quant_ms = timed(quant, args.steps, args.warmup, n)
    fine_ms = timed(fine8, args.steps, args.warmup, n)
    launch_ms = per_launch(fine8, args.steps, args.warmup, n)
    fwd_ms = timed(fwd8, args.steps, args.warmup, n)
    fl = flops.fine_forward_flops(w.B, w.H, w.C, w.topk, w.d)
    code_bytes = 3 * w.B * w.H * w.Np * w.d
    raster_bytes = 3 * w.B * w.H * w.N * w.d * 2
    achieved = fl / (launch_ms * 1e-3) / 1e12
    return {
        "scheme": "E4M3 q, k, v with per-cube power-of-two scales; P rounded to E4M3; "
                  "fp32 accumulation; coarse stage and top-K as the bf16 path",
        "quantize_ms": round(quant_ms, 5),
        "quantize_gbps": round((raster_bytes + code_bytes) / (quant_ms * 1e-3) / 1e9, 1),
        "fine_ms": round(fine_ms, 5),
        "fine_launch_ms": round(launch_ms, 5),
        "fine_tflops": round(fl / (fine_ms * 1e-3) / 1e12, 2),
        "forward_ms": round(fwd_ms, 5),
        "speedup_fine_vs_bf16": None,
        "roofline": {"bound": "mfma", "kernel": "fine_fwd_fp8_kernel<false> (vsa_fine_fp8)",
                     "achieved": round(achieved, 2), "peak": flops.PEAK_FP8_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / flops.PEAK_FP8_TFLOPS, 4),
                     "traffic": traffic_record("block_sparse_attention_cube_amd/csrc/fine_fp8.hip",
                                               "fine_fp8_wan1.3b_traffic.json"),
                     "flops_per_launch": fl, "launch_ms": round(launch_ms, 5)},
    }


CAL_BYTES = 256 << 20


def stage_only(args, w, grid, sets, cube_sets, step):
    import torch
    import block_sparse_attention_cube_amd as vsa
    n = len(sets)
    # one plain device copy of known size, so HBM byte counters can be scaled
    src = torch.empty(CAL_BYTES, dtype=torch.uint8, device=sets[0]["q"].device)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    if args.stage == "forward":
        fn = step
    elif args.stage == "backward":
        from synth import configs
        w = configs.SWEEP[0]
        print(json.dumps({"stage": "backward", "sweep": sparsity_sweep(args, sets[0]["q"].device)}),
              flush=True)
        return
    elif args.stage == "reorder":
        fn = lambda i: [vsa.reorder(sets[i][t], grid) for t in "qkv"]
    elif args.stage == "quantize_fp8":
        fn = lambda i: vsa.quantize_fp8(sets[i]["q"], sets[i]["k"], sets[i]["v"], grid)
    elif args.stage == "forward_fp8":
        plan8 = vsa.ForwardFp8Plan(w.B, w.H, grid, w.d, w.topk, sets[0]["q"].device)
        fn = lambda i: plan8.run(sets[i]["q"], sets[i]["k"], sets[i]["v"])
    elif args.stage == "fine_fp8":
        idx = [vsa.coarse(c["q"], c["k"], c["v"], grid, w.topk)[1] for c in cube_sets]
        q8s = [vsa.quantize_fp8(s["q"], s["k"], s["v"], grid) for s in sets]
        out = torch.empty_like(cube_sets[0]["q"])
        fn = lambda i: vsa.fine_fp8(*q8s[i], idx[i], grid, return_lse=False, out=out)
    else:
        idx = [vsa.coarse(c["q"], c["k"], c["v"], grid, w.topk)[1] for c in cube_sets]
        out = torch.empty_like(cube_sets[0]["q"])
        if args.stage == "fine":
            fn = lambda i: vsa.fine(cube_sets[i]["q"], cube_sets[i]["k"], cube_sets[i]["v"],
                                    idx[i], grid, out=out)
        elif args.stage == "fine_raster":
            ocs = [vsa.coarse(c["q"], c["k"], c["v"], grid, w.topk)[0] for c in cube_sets]
            rout = (torch.empty_like(sets[0]["q"]), torch.empty_like(sets[0]["q"]))
            fn = lambda i: vsa.fine_raster(sets[i]["q"], sets[i]["k"], sets[i]["v"], idx[i], grid,
                                           oc=ocs[i], out=rout)
        elif args.stage == "dense":
            fn = lambda i: vsa.dense(cube_sets[i]["q"], cube_sets[i]["k"], cube_sets[i]["v"], grid,
                                     return_lse=False, out=out)
        else:
            fn = lambda i: vsa.coarse(cube_sets[i]["q"], cube_sets[i]["k"], cube_sets[i]["v"],
                                      grid, w.topk)
    ms = timed(fn, args.steps, args.warmup, n)
    launch_ms = per_launch(fn, args.steps, 0, n)
    print(json.dumps({"stage": args.stage, "ms": round(ms, 5), "launch_ms": round(launch_ms, 5),
                      "steps": args.steps}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); "
              "multi-GPU sharding is not part of this library", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import block_sparse_attention_cube_amd as vsa
    from block_sparse_attention_cube_amd import flops
    from synth import configs, inputs

    w = configs.WAN_1_3B
    n_sets = N_SETS
    if args.stage != "all" and args.workload == "wan14b":
        w, n_sets = configs.WAN_14B, 1     # 2.3 GB of q, k, v: beyond every cache already
    grid = (w.T, w.Hh, w.Ww)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    host_sets = [inputs.make_inputs(w, seed=s) for s in range(n_sets)]
    sets = [{n: inputs.as_torch(h[n], w.dtype, dev) for n in "qkv"} for h in host_sets]
    cube_sets = [{n: vsa.reorder(s[n], grid) for n in "qkv"} for s in sets]

    plan = vsa.ForwardPlan(w.B, w.H, grid, w.d, w.topk, torch.bfloat16, dev)
    step = lambda i: plan.run(sets[i]["q"], sets[i]["k"], sets[i]["v"])
    if args.stage != "all":
        stage_only(args, w, grid, sets, cube_sets, step)
        return
    settle_ms = settle_clock(step, N_SETS)
    ms = timed(step, args.steps, args.warmup, N_SETS)
    med_ms, p10_ms, p90_ms = per_call(step, max(20, args.steps // 2), args.warmup, N_SETS)
    warm_ms = timed(lambda i: step(0), args.steps, args.warmup, 1)

    # fine kernel alone and coarse + fine on cube-order inputs
    idx_sets, oc_sets = [], []
    for c in cube_sets:
        oc, idx = vsa.coarse(c["q"], c["k"], c["v"], grid, w.topk)
        idx_sets.append(idx)
        oc_sets.append(oc)
    o_buf = torch.empty_like(cube_sets[0]["q"])
    fine_step = lambda i: vsa.fine(cube_sets[i]["q"], cube_sets[i]["k"], cube_sets[i]["v"],
                                   idx_sets[i], grid, out=o_buf)
    fine_ms = timed(fine_step, args.steps, args.warmup, N_SETS)
    fine_launch_ms = per_launch(fine_step, args.steps, args.warmup, N_SETS)
    # the fine stage exactly as vsa_forward runs it: raster gather, raster
    # O_fine and LSE, O_coarse broadcast (vsa_fine_raster)
    raster_out = (torch.empty_like(sets[0]["q"]), torch.empty_like(sets[0]["q"]))
    raster_step = lambda i: vsa.fine_raster(sets[i]["q"], sets[i]["k"], sets[i]["v"], idx_sets[i],
                                            grid, oc=oc_sets[i], out=raster_out)
    raster_launch_ms = per_launch(raster_step, args.steps, args.warmup, N_SETS)

    def coarse_fine(i):
        c = cube_sets[i]
        _, idx = vsa.coarse(c["q"], c["k"], c["v"], grid, w.topk)
        vsa.fine(c["q"], c["k"], c["v"], idx, grid, out=o_buf)
    cf_ms = timed(coarse_fine, args.steps, args.warmup, N_SETS)

    # dense baseline on the same 7168-token sequence, pad keys masked: the
    # faster of the dedicated dense kernel (vsa_dense, no index list, 128
    # query rows per workgroup) and the sparse kernel with every cube selected
    d_steps, d_warm = max(10, args.steps // 8), max(2, args.warmup // 4)
    all_idx = torch.arange(w.C, dtype=torch.int32, device=dev).expand(w.B, w.H, w.C, w.C).contiguous()
    dense_kc_ms = timed(lambda i: vsa.fine(cube_sets[i]["q"], cube_sets[i]["k"], cube_sets[i]["v"],
                                           all_idx, grid, return_lse=False, out=o_buf),
                        d_steps, d_warm, N_SETS)
    dense_kernel_ms = timed(lambda i: vsa.dense(cube_sets[i]["q"], cube_sets[i]["k"],
                                                cube_sets[i]["v"], grid, return_lse=False,
                                                out=o_buf), d_steps, d_warm, N_SETS)
    dense_ms = min(dense_kc_ms, dense_kernel_ms)
    # dense attention over the 5824 real tokens only: 5824 = 91 x 64, and dense
    # attention does not depend on token order, so the raster rows read as the
    # cube order of a 4 x 4 x 364 grid (91 full cubes)
    real_grid = (4, 4, w.N // 16)
    real_c = w.N // 64
    real_idx = torch.arange(real_c, dtype=torch.int32, device=dev).expand(
        w.B, w.H, real_c, real_c).contiguous()
    o_real = torch.empty_like(sets[0]["q"])
    dense_real_kc_ms = timed(lambda i: vsa.fine(sets[i]["q"], sets[i]["k"], sets[i]["v"], real_idx,
                                                real_grid, return_lse=False, out=o_real),
                             d_steps, d_warm, N_SETS)
    dense_real_kernel_ms = timed(lambda i: vsa.dense(sets[i]["q"], sets[i]["k"], sets[i]["v"],
                                                     real_grid, return_lse=False, out=o_real),
                                 d_steps, d_warm, N_SETS)
    dense_real_ms = min(dense_real_kc_ms, dense_real_kernel_ms)
    useful = flops.useful_fine_flops(w.B, w.H, w.d, valid_counts(w), idx_sets[0].cpu().numpy())
    fp8 = fp8_section(args, w, grid, sets, idx_sets, dev)
    fp8["speedup_fine_vs_bf16"] = round(fine_launch_ms / fp8["fine_launch_ms"], 3)
    configs_out = per_config(args, dev)

    sweep = sparsity_sweep(args, dev)

    fl = flops.fine_forward_flops(w.B, w.H, w.C, w.topk, w.d)
    fl_dense = flops.fine_forward_flops(w.B, w.H, w.C, w.C, w.d)
    fine_tflops = fl / (fine_ms * 1e-3) / 1e12
    launch_tflops = fl / (fine_launch_ms * 1e-3) / 1e12
    raster_tflops = fl / (raster_launch_ms * 1e-3) / 1e12
    traffic = traffic_record("block_sparse_attention_cube_amd/csrc/fine_fwd.hip")
    raster_traffic = traffic_record("block_sparse_attention_cube_amd/csrc/fine_fwd.hip",
                                    "fine_fwd_raster_wan1.3b_traffic.json")
    fwd_tflops = fl / (ms * 1e-3) / 1e12

    result = {
        "metric": METRIC,
        "value": round(ms, 5),
        "unit": "ms",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "wan1.3b-480p: grid 16x14x26 -> 16x16x28 (7168 tok, 112 cubes), "
                               "B=1, H=12, d=128, bf16, top-K 14 (87.5% sparse)",
                   "global_batch": w.B, "seq_len": w.Np, "heads": w.H, "head_dim": w.d,
                   "topk": w.topk, "cubes": w.C, "input_sets_rotated": N_SETS},
        "sparse_tflops": round(fwd_tflops, 2),
        "pct_bf16_peak": round(100 * fwd_tflops / flops.PEAK_BF16_TFLOPS, 2),
        "warm_ms": round(warm_ms, 5),
        "clock_settle_ms": settle_ms,
        "fine_ms": round(fine_ms, 5),
        "fine_tflops": round(fine_tflops, 2),
        "coarse_fine_ms": round(cf_ms, 5),
        "dense_fa_ms": round(dense_ms, 5),
        "dense_fa_kernel_ms": round(dense_kernel_ms, 5),
        "dense_fine_all_cubes_ms": round(dense_kc_ms, 5),
        "speedup_fine_vs_dense": round(dense_ms / fine_ms, 3),
        "speedup_coarse_fine_vs_dense": round(dense_ms / cf_ms, 3),
        "speedup_forward_vs_dense": round(dense_ms / ms, 3),
        "dense_tflops": round(fl_dense / (dense_ms * 1e-3) / 1e12, 2),
        "dense_real_tokens_ms": round(dense_real_ms, 5),
        "dense_real_tokens_kernel_ms": round(dense_real_kernel_ms, 5),
        "dense_real_tokens_fine_all_cubes_ms": round(dense_real_kc_ms, 5),
        "speedup_forward_vs_dense_real_tokens": round(dense_real_ms / ms, 3),
        "value_median_ms": round(med_ms, 5), "value_p10_ms": round(p10_ms, 5),
        "value_p90_ms": round(p90_ms, 5),
        "fine_useful_tflops": round(useful / (fine_ms * 1e-3) / 1e12, 2),
        "per_config": configs_out,
        "fp8": fp8,
        "sweep": sweep,
        "fine_launch_ms": round(fine_launch_ms, 5),
        "fine_raster_launch_ms": round(raster_launch_ms, 5),
        "roofline": {"bound": "mfma",
                     "kernel": "fine_fwd_bf16_kernel<128,true> (vsa_fine_raster: the fine stage "
                               "of vsa_forward)",
                     "achieved": round(raster_tflops, 2), "peak": flops.PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(raster_tflops / flops.PEAK_BF16_TFLOPS, 4),
                     "traffic": raster_traffic,
                     "flops_per_launch": fl, "launch_ms": round(raster_launch_ms, 5)},
        "roofline_cube_order": {"bound": "mfma",
                                "kernel": "fine_fwd_bf16_kernel<128,false> (vsa_fine)",
                                "achieved": round(launch_tflops, 2),
                                "peak": flops.PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                                "frac": round(launch_tflops / flops.PEAK_BF16_TFLOPS, 4),
                                "traffic": traffic, "flops_per_launch": fl,
                                "launch_ms": round(fine_launch_ms, 5)},
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, host_sets[0], args.cpu_reps)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
