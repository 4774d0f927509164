#!/usr/bin/env python3
"""Throughput of the routed mixture-of-experts block on one MI355X.

One step = one pass of the whole block (router logits, top-k, bucketing,
gate/up dequant-GEMV with SwiGLU, down, shared expert, combine) over one
batch of synthetic tokens with every input already resident in HBM.

Default workload (the headline): decode of one token through a
DeepSeek-V4-Flash-shaped layer (n_embd 4096, 256 routed experts, top-6, FFN
width 2048, Q2K routed experts, Q8_0 shared expert, fp32 router), weights
drawn from N(0, 0.02) and encoded, activations N(0, 1).

The same run then measures the other workloads of the metric, each as an
object of the line with its own tokens/s, roofline and CPU baseline:
"prefill_2048" (2048 bf16 token rows through the matrix-core grouped GEMMs)
and "decode_b32" (32 fp32 rows, Zipf-skewed routing) on the same resident
layer, then "stack43_b1" and "stack43_b8" (the 43-block stack, every layer
resident, one and eight token rows).  --clauses picks them.

Cold-cache timing: step i runs on device replica i % R of the layer (R x
2.14 GB, far above the 256 MB last-level cache) with token i % 64, so no
step finds the previous steps' weights in cache and the routing varies.
Steps are timed with HIP events on the stream that replays them.

Prints one JSON line on stdout; progress goes to stderr.
"""
import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s; decode HBM GB/s and prefill MFMA % of MI355X peak"
ALU_PEAK_TOPS = 256 * 64 * 2.4e9 / 1e12  # 32-bit lane operations per second: 256 CUs x 64 lanes x 2.4 GHz
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA, published


# the workloads the default run measures after decode_b1, in this order
CLAUSES = ("prefill_2048", "decode_b32", "stack43_b1", "stack43_b8")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2048)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="decode_b1",
                    choices=["decode_b1", "decode_b32", "prefill_2048", "stack43_b1", "stack43_b8", "hotlist_43x256",
                             "decode_b1_q4k"])
    ap.add_argument("--replicas", type=int, default=16)
    ap.add_argument("--stack-layers", type=int, default=43,
                    help="stack workloads: resident layers (43 = the whole stack; fewer for counter passes)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="budget of the oracle CPU baseline")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="launch every step eagerly (for counter profiling)")
    ap.add_argument("--copy-calib", type=float, default=0.0, metavar="MB",
                    help="only run 20 plain device copies of MB megabytes (scale reference for HBM counters)")
    ap.add_argument("--read-stream", action="store_true",
                    help="only measure the plain read-stream ceiling (moe_read_stream) at several sizes")
    ap.add_argument("--clauses", default=",".join(CLAUSES),
                    help="decode_b1 only: the other workloads the run adds to the line (comma list, empty for none)")
    ap.add_argument("--no-prefill", action="store_true", help="decode_b1 only: the same as --clauses ''")
    ap.add_argument("--prefill-cpu-seconds", type=float, default=10.0,
                    help="budget of the oracle CPU baseline of each added workload")
    return ap.parse_args()


def copy_calib(mb):
    import torch
    n = int(mb * 1e6) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(20):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calib_bytes_read": n * 4, "copy_calib_bytes_written": n * 4, "launches": 20}))


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (--gpus %d, WORLD_SIZE %d). "
              "Run it with --gpus 1." % (args.gpus, world), file=sys.stderr)
        sys.exit(2)

    if args.copy_calib > 0:
        copy_calib(args.copy_calib)
        return
    if args.read_stream:
        read_stream(args)
        return

    if args.workload.startswith("stack43"):
        B = int(args.workload.split("_b")[1])
        st = make_stack(args.stack_layers)
        print(json.dumps(measure_stack(st, B, args.steps, args.warmup, args.no_graph,
                                       None if args.no_cpu else args.cpu_seconds)), flush=True)
        return
    if args.workload == "hotlist_43x256":
        run_hotlist(args)
        return

    import torch

    import synth

    torch.cuda.set_device(0)
    t0 = time.time()
    if args.workload == "decode_b1_q4k":  # the flash shape with Q4_K routed experts
        s = synth.DS4_FLASH
        L = synth.make_layer(synth.WEIGHTS_SEED, 0, D=s["D"], E=s["E"], k=s["k"], F=s["F"], Fs=s["Fs"],
                             gate_fmt=synth.Q4K, down_fmt=synth.Q4K)
    else:
        L = synth.flash_layer()
    log("layer generated in %.1f s" % (time.time() - t0))
    reps = resident_replicas(L, max(1, args.replicas))
    line = measure_layer(args, args.workload, L, reps, args.cpu_seconds)
    line["context"] = PAGES_CONTEXT
    clauses = [] if args.no_prefill or args.workload != "decode_b1" else [c for c in args.clauses.split(",") if c]
    for c in clauses:
        if c not in CLAUSES:
            sys.exit("unknown clause %r (one of %s)" % (c, ", ".join(CLAUSES)))

    def add(name, sub):
        for key in ("metric", "n_gpus", "higher_is_better", "scaling", "vs_baseline", "data", "context"):
            sub.pop(key, None)
        line[name] = sub
        log("%s: %.1f tokens/s, %.4f ms per step" % (name, sub["value"], sub["ms_per_step"]))

    # the metric's other workloads, measured in the same run: the batched
    # ones on the same resident layer, then the stack on layers of its own
    for c in clauses:
        if not c.startswith("stack43"):
            add(c, measure_layer(args, c, L, reps, args.prefill_cpu_seconds))
    if any(c.startswith("stack43") for c in clauses):
        del reps
        import torch
        torch.cuda.empty_cache()
        st = make_stack(43)
        for c in clauses:
            if c.startswith("stack43"):
                B = int(c.split("_b")[1])
                add(c, measure_stack(st, B, 256 if B == 1 else 64, 20 if B == 1 else 8, False,
                                     None if args.no_cpu else args.prefill_cpu_seconds / 2))
    print(json.dumps(line), flush=True)


# The pages' own figure, for context only: the whole model (attention and all
# 43 layers) on another machine ("DwarfStar Native Inference Engine",
# performance table).
PAGES_CONTEXT = {
    "pages_generation_tokens_s": 39.35,
    "pages_prefill_tokens_s": 790.18,
    "pages_hardware": "MacBook Pro M5 Max 128 GB (Metal), whole DeepSeek-V4-Flash with attention, ctx 2048",
    "note": "context only: another machine and the whole model, not this block alone",
}


def resident_replicas(L, R):
    """R device copies of the layer (the bench rotates them so that every
    step reads weights that are not in the 256 MB last-level cache)."""
    import numpy as np
    import torch

    import quantized_routed_moe_router_amd as moe
    dev = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).cuda()
    base = moe.LayerWeights(L.n_embd, L.n_expert, L.n_expert_used, L.n_ff_exp, L.n_ff_shared, L.gate_fmt,
                            L.up_fmt, L.down_fmt, L.shared_fmt, dev(L.router_w), dev(L.gate), dev(L.up),
                            dev(L.down), dev(L.sh_gate), dev(L.sh_up), dev(L.sh_down), None, L.route_scale)
    reps = [base]
    for _ in range(R - 1):
        reps.append(moe.LayerWeights(**{f: (getattr(base, f).clone() if isinstance(getattr(base, f), torch.Tensor)
                                            else getattr(base, f)) for f in base.__dataclass_fields__}))
    torch.cuda.synchronize()
    log("%d replicas resident (%.1f GB)" % (R, R * (base.gate.numel() * 3 + base.sh_gate.numel() * 3) / 1e9))
    return reps


def measure_layer(args, workload, L, reps, cpu_seconds):
    """One workload on the resident replicas: K timed steps of one forward
    each (graph replays, timed with HIP events on the stream), the per-call
    spread, the dominant kernel's launch time, and the CPU oracle beside it."""
    import copy

    import numpy as np
    import torch

    import quantized_routed_moe_router_amd as moe
    import synth

    if workload in ("decode_b1", "decode_b1_q4k"):
        T, n_x = 1, 64
        x_all = synth.activations(1, n_x, L.n_embd)
        mode = moe.F32
        bias = None
    elif workload == "decode_b32":
        T, n_x = 32, 8
        x_all = synth.activations(2, 32 * n_x, L.n_embd)
        bias = synth.zipf_bias(2, L.n_expert)
        mode = moe.F32
    else:
        T, n_x = 2048, 1
        x_all = synth.activations(3, 2048, L.n_embd)
        mode = moe.BF16
        bias = None
    Lw = copy.copy(L)
    Lw.router_bias = bias
    if bias is not None:  # the same weights with the router bias attached
        bd = torch.from_numpy(bias).cuda()
        reps = [copy.copy(W) for W in reps]
        for W in reps:
            W.router_bias = bd
    R = len(reps)
    base = reps[0]
    if mode == moe.BF16:
        xs = torch.from_numpy(synth.to_bf16_bits(x_all).view(np.int16)).cuda().view(torch.bfloat16)
    else:
        xs = torch.from_numpy(np.ascontiguousarray(x_all)).cuda()
    xin = [xs[(i % n_x) * T:(i % n_x) * T + T] for i in range(n_x)]
    ws = moe.alloc_workspace(base, T, mode)
    r = moe.Routing(T, L.n_expert_used, L.n_expert)
    y = torch.zeros((T, L.n_embd), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()

    # One forward of the block.
    def step(i):
        moe.layer_forward(reps[i % R], xin[i % n_x], y, ws, routing=r)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # One graph holds R consecutive steps (one per replica).  Replaying it is
    # how a decode loop issues the block without per-kernel host overhead.
    # The K steps are timed with HIP events on the replay stream (the host
    # clock is kept beside them); --no-graph launches every step eagerly
    # instead (counter profiling).
    K = args.steps
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    graphs, single = [], []
    if args.no_graph:
        torch.cuda.synchronize()
        t_start = time.perf_counter()
        ev0.record()
        for i in range(K):
            step(i)
        ev1.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t_start
        n_replays = 0
    else:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for n in sorted({R, K % R} - {0}, reverse=True):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=side):
                    for i in range(n):
                        step(i)
                graphs.append((n, g))
            for i in range(R):  # one step per graph, for the per-call spread
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=side):
                    step(i)
                single.append(g)
        torch.cuda.current_stream().wait_stream(side)
        full = [g for n, g in graphs if n == R]
        rest = [g for n, g in graphs if n != R]
        plan = full * (K // R) + rest
        for g in (full or rest)[:1] * 2:
            g.replay()
        torch.cuda.synchronize()
        t_start = time.perf_counter()
        ev0.record()
        for g in plan:
            g.replay()
        ev1.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t_start
        n_replays = len(plan)
    ms_step = ev0.elapsed_time(ev1) / K
    # per-call spread: 64 single-step replays queued behind a spin kernel,
    # an event between consecutive calls
    spread = None
    if single:
        n_calls = 64
        evc = [torch.cuda.Event(enable_timing=True) for _ in range(n_calls + 1)]
        torch.cuda._sleep(2000000)
        evc[0].record()
        for j in range(n_calls):
            single[j % R].replay()
            evc[j + 1].record()
        torch.cuda.synchronize()
        per = np.array([evc[j].elapsed_time(evc[j + 1]) * 1000.0 for j in range(n_calls)])
        spread = [round(float(np.percentile(per, q)), 2) for q in (10, 50, 90)]

    # The dominant kernel's launch time: HIP events on the launch stream
    # around a run of R back-to-back launches, one per weight replica (each
    # reads cold weights), on the routing of one input; 8 such runs over
    # different inputs.  Events inside a captured graph do not time, and a
    # pair of events around a single launch also holds its dispatch latency,
    # so the run is long and a bounded spin kernel ahead of it lets the host
    # queue the whole run before the GPU reaches it.
    n_runs = 8
    # the grouped-GEMM path (many rows, Q2K experts): stage 5 is its routed
    # gate/up kernel alone; elsewhere stage 3 is the gate/up kernel
    gemm = T > 16 and L.gate_fmt == synth.Q2K and L.down_fmt == synth.Q2K
    st_gu = moe.STAGE_ROUTED_GATE_UP if gemm else moe.STAGE_GATE_UP
    ev_src = ("HIP events around runs of %d back-to-back stage-%d launches on cold replicas, %d runs, "
              "median per launch" % (R, st_gu, n_runs))
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_runs)]
    for i, e in enumerate(evs):
        x = xin[i % n_x]
        moe.layer_forward_stage(base, x, y, ws, moe.STAGE_ROUTER, routing=r)
        moe.layer_forward_stage(base, x, y, ws, moe.STAGE_ROUTE, routing=r)
        if gemm:  # activation codes and tiles for stage 5
            moe.layer_forward_stage(base, x, y, ws, moe.STAGE_GATE_UP, routing=r)
        torch.cuda._sleep(1000000)
        e[0].record()
        for W in reps:
            moe.layer_forward_stage(W, x, y, ws, st_gu, routing=r)
        e[1].record()
        moe.layer_forward_stage(base, x, y, ws, moe.STAGE_DOWN_COMBINE, routing=r)
    torch.cuda.synchronize()
    times = [a.elapsed_time(b) / R for a, b in evs]
    gateup_ms = float(np.median(times))
    gateup_p10, gateup_p90 = float(np.percentile(times, 10)), float(np.percentile(times, 90))
    log("%s: timed %d steps, %.4f ms per step by HIP events (host clock %.4f ms, %d graph replays); "
        "gate/up avg %.2f us (%s)" % (workload, K, ms_step, 1000.0 * wall / K, n_replays, gateup_ms * 1e3, ev_src))

    # routing of every distinct input, outside the timed region, for the byte counts
    n_unique = []
    for i in range(n_x):
        moe.route(base, xin[i], r, ws)
        torch.cuda.synchronize()
        n_unique.append(int(r.n_active.item()))
    nu = float(np.mean(n_unique))
    D, F, Fs, k = L.n_embd, L.n_ff_exp, L.n_ff_shared, L.n_expert_used
    xb = 2 if mode == moe.BF16 else 4
    gu_expert = 2 * synth.tensor_bytes(L.gate_fmt, F * D)
    dn_expert = synth.tensor_bytes(L.down_fmt, D * F)
    sh_gu = 2 * synth.tensor_bytes(L.shared_fmt, Fs * D)
    sh_dn = synth.tensor_bytes(L.shared_fmt, D * Fs)
    router_b = D * L.n_expert * 4 + (L.n_expert * 4 if bias is not None else 0)
    step_bytes = router_b + nu * (gu_expert + dn_expert) + sh_gu + sh_dn + T * D * xb + T * D * 4
    # the timed launch holds the routed experts' gate/up only: the decode
    # kernel (T <= 16) or the grouped GEMM (stage 5); the other batched
    # kernels' stage 3 also runs the shared expert
    small = T <= 16
    if small:  # the decode gate/up kernel this layer takes
        kernel_name = "dec_k3_q2k4096_kernel" if L.gate_fmt == synth.Q2K and D == 4096 else "dec_k3_kernel"
        gateup_bytes = nu * gu_expert + T * D * xb + T * k * F * 4
    elif gemm:  # x codes (2 bytes per value) in, h out (fp32)
        kernel_name = "pf_gemm_kernel"
        gateup_bytes = nu * gu_expert + T * D * 2 + T * k * F * 4
    else:
        kernel_name = "large_gateup_kernel"
        gateup_bytes = nu * gu_expert + T * D * xb + T * k * F * 4 + sh_gu + T * Fs * 4
    achieved = gateup_bytes / (gateup_ms * 1e-3) / 1e9
    # bf16 rows: the routed gate/up is a dense contraction per expert at the
    # ridge, priced against the dense bf16 matrix-core peak
    gateup_flops = 2.0 * T * k * 2 * F * D
    mfma_bound = gemm and mode == moe.BF16
    tokens_s = T / (ms_step * 1e-3)
    flops = 2.0 * T * (k * 3 * D * F + 3 * D * Fs)

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(Lw, x_all, T, mode, cpu_seconds)

    line = {
        "metric": METRIC,
        "value": round(tokens_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if mode == moe.BF16 else "f32",
        "numerics": ("%s x, fp32 h and y; the exact integer codes of the weights against activations coded "
                     "as int16 (per group of 16 values for a few rows, per row on the matrix cores), int32 "
                     "sums scaled in fp32" % ("bf16" if mode == moe.BF16 else "fp32")),
        "data": "synthetic",
        "config": {
            "workload": workload,
            "tokens_per_step": T,
            "n_embd": D, "n_expert": L.n_expert, "n_expert_used": k, "n_ff_exp": F, "n_ff_shared": Fs,
            "formats": "%s gate/up/down, Q8_0 shared, fp32 router" % ("Q4K" if L.gate_fmt == synth.Q4K else "Q2K"),
            "cache": "cold: %d device replicas rotated, %d distinct inputs" % (R, n_x),
            "launch": "hipGraph of %d steps, replayed" % R,
        },
        "timing": "HIP events on the replay stream around the %d timed steps" % K,
        "wall_ms_per_step": round(1000.0 * wall / K, 5),
        "call_us_p10_p50_p90": spread,
        "call_timing": "64 single-step graph replays queued back to back, an event between consecutive calls",
        "hbm_gbps": round(step_bytes / (ms_step * 1e-3) / 1e9, 1),
        "algorithmic_bytes_per_step": int(step_bytes),
        "tflops": round(flops / (ms_step * 1e-3) / 1e12, 2),
        "unique_experts_per_step": nu,
        "roofline": {
            "kernel": kernel_name,
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(kernel_name, workload),
            "bytes_per_launch": int(gateup_bytes),
            "avg_launch_us": round(gateup_ms * 1e3, 3),
            "launch_us_p10_p90": [round(gateup_p10 * 1e3, 3), round(gateup_p90 * 1e3, 3)],
            "timing": ev_src,
        },
        "cpu_baseline": cpu,
    }
    if mfma_bound:
        tf = gateup_flops / (gateup_ms * 1e-3) / 1e12
        line["roofline"].update({
            "bound": "mfma", "achieved": round(tf, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(tf / BF16_PEAK_TFLOPS, 4), "flops_per_launch": gateup_flops,
            "hbm_gbps": round(achieved, 1),
        })
        line["mfma_pct_of_bf16_peak_whole_step"] = round(100.0 * flops / (ms_step * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
                                                         2)
    del ws, y, xs
    torch.cuda.empty_cache()
    return line


def read_stream(args):
    """The HBM bandwidth one launch of a plain read reaches (moe_read_stream),
    at the sizes of this block's kernels and beyond: back-to-back launches
    over rotating buffers (at least 1 GB in all, so no launch finds its data
    in the 256 MB last-level cache), HIP events around each run of launches,
    median per launch.  Also the cost of an almost empty launch."""
    import numpy as np
    import torch

    import quantized_routed_moe_router_amd as moe
    torch.cuda.set_device(0)
    out = []
    for mb in (4, 9, 18, 33, 80, 256, 1024):
        nbytes = mb * (1 << 20)
        nbuf = max(4, (1 << 30) // nbytes + 1)
        bufs = [torch.ones(nbytes // 4, dtype=torch.float32, device="cuda") for _ in range(nbuf)]
        blocks = max(1, min(4096, nbytes // 16 // (256 * 4)))
        sink = torch.zeros(4 * blocks, dtype=torch.int32, device="cuda")
        for bfr in bufs[:2]:
            moe.read_stream(bfr, sink)
        runs = []
        for _ in range(5):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda._sleep(1000000)
            a.record()
            for bfr in bufs:
                moe.read_stream(bfr, sink)
            b.record()
            torch.cuda.synchronize()
            runs.append(a.elapsed_time(b) * 1000.0 / nbuf)
        us = float(np.median(runs))
        out.append({"mb": mb, "bytes": nbytes, "blocks": blocks, "us_per_launch": round(us, 3),
                    "gbps": round(nbytes / (us * 1e-6) / 1e9, 1)})
        log("read stream %5d MB: %.2f us per launch, %.0f GB/s" % (mb, us, out[-1]["gbps"]))
        del bufs
        torch.cuda.empty_cache()
    # an almost empty launch (16 bytes, one workgroup), 256 of them captured
    # in a graph and replayed, so that the host's launch rate plays no part
    tiny = torch.ones(4, dtype=torch.float32, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            for _ in range(256):
                moe.read_stream(tiny, sink)
    torch.cuda.current_stream().wait_stream(side)
    g.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    g.replay()
    b.record()
    torch.cuda.synchronize()
    print(json.dumps({"read_stream": out, "empty_launch_us": round(a.elapsed_time(b) * 1000.0 / 256, 3),
                      "peak_gbps": HBM_PEAK_GBS}), flush=True)


def measured_traffic(kernel, workload):
    """HBM bytes per launch of the kernel from the committed counter summary
    (profiles/<kernel>_<workload>_hbm_counters.md), or None when there is
    none or it was taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", "%s_%s_hbm_counters.md" % (kernel, workload))
    try:
        with open(path) as f:
            text = f.read()
    except OSError:
        return None
    vals = {}
    for line in text.splitlines():
        if line.startswith("- traffic_bytes_per_launch:"):
            vals["bytes"] = float(line.split(":", 1)[1])
        elif line.startswith("- kernel_source_sha256:"):
            vals["sha"] = line.split(":", 1)[1].strip()
    from quantized_routed_moe_router_amd.profsum import kernel_source_digest
    if "bytes" not in vals or vals.get("sha") != kernel_source_digest(kernel):
        return None
    return vals["bytes"]


def make_stack(n_layer):
    """The 43-block stack's layers, resident: code-sampled weights of the
    stack's formats and shapes per layer (n_layer of them, 43 = the whole
    stack), and layer 0 on the host for the CPU baseline."""
    import numpy as np
    import torch

    import quantized_routed_moe_router_amd as moe
    import synth

    torch.cuda.set_device(0)
    n_layer = max(1, min(43, n_layer))
    cb = synth.codebook(4)
    cbd = torch.from_numpy(np.ascontiguousarray(cb)).cuda()
    dev = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).cuda()
    t0 = time.time()
    Ws, host0 = [], None
    for l in range(n_layer):
        L = synth.stack_layer_sampled(l, cb)
        if l == 0:
            host0 = L
        Ws.append(moe.LayerWeights(L.n_embd, L.n_expert, L.n_expert_used, L.n_ff_exp, L.n_ff_shared, L.gate_fmt,
                                   L.up_fmt, L.down_fmt, L.shared_fmt, dev(L.router_w), dev(L.gate), dev(L.up),
                                   dev(L.down), dev(L.sh_gate), dev(L.sh_up), dev(L.sh_down), None, 1.0,
                                   codebook=cbd, gamma=dev(L.gamma)))
        del L
        if (l + 1) % 8 == 0:
            log("%d of %d layers resident (%.1f s)" % (l + 1, n_layer, time.time() - t0))
    torch.cuda.synchronize()
    log("%d layers generated and resident in %.1f s" % (n_layer, time.time() - t0))
    return Ws, host0


def measure_stack(st, B, K, warmup, no_graph, cpu_seconds):
    """The 43-block stack x <- x + MoE(RMSNorm(x)) at B token rows on the
    resident layers st: one step = the blocks in order (moe_block_forward
    each), captured once in a graph and replayed; K timed steps after
    `warmup`; the CPU oracle for cpu_seconds (None: skipped)."""
    import numpy as np
    import torch

    import quantized_routed_moe_router_amd as moe
    import synth

    Ws, host0 = st
    n_layer = len(Ws)
    W0 = Ws[0]
    D = W0.n_embd
    x0 = synth.stack43(B=B).x
    x = torch.from_numpy(np.ascontiguousarray(x0)).cuda()
    xn = torch.empty_like(x)
    ws = moe.alloc_workspace(W0, B)
    r = moe.Routing(B, W0.n_expert_used, W0.n_expert)

    # eager runs (counter profiling) keep each block's number of active
    # experts, so that the gate/up kernel's bytes per launch can be averaged
    # over exactly the launches the counters see
    seen = [] if no_graph else None

    def step():  # one moe_block_forward per block: x <- x + MoE(RMSNorm(x))
        for W in Ws:
            moe.block_forward(W, x, ws, eps=1e-6, routing=r)
            if seen is not None:
                seen.append(r.n_active.clone())

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    if no_graph:
        t_start = time.perf_counter()
        ev0.record()
        for _ in range(K):
            step()
        ev1.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t_start
    else:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                step()
        torch.cuda.current_stream().wait_stream(side)
        g.replay()
        torch.cuda.synchronize()
        t_start = time.perf_counter()
        ev0.record()
        for _ in range(K):
            g.replay()
        ev1.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t_start
    ms_step = ev0.elapsed_time(ev1) / K

    # the dominant kernel (stage 3: routed gate/up, CB2): events around runs
    # of back-to-back stage-3 launches, one per layer (cold weights), on the
    # routing of layer 0's stages 1-2
    n_runs = 8
    moe.rmsnorm(x, W0.gamma, xn, 1e-6)
    moe.layer_forward_stage(W0, xn, x, ws, moe.STAGE_ROUTER, routing=r, accumulate=True)
    moe.layer_forward_stage(W0, xn, x, ws, moe.STAGE_ROUTE, routing=r, accumulate=True)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_runs)]
    for e in evs:
        torch.cuda._sleep(1000000)
        e[0].record()
        for W in Ws:
            moe.layer_forward_stage(W, xn, x, ws, moe.STAGE_GATE_UP, routing=r, accumulate=True)
        e[1].record()
    torch.cuda.synchronize()
    times = [a.elapsed_time(b) / n_layer for a, b in evs]
    gu_ms = float(np.median(times))
    nu = float(r.n_active.item())
    launch_nu = None
    if seen:  # every block of the warm-up and timed steps, then the timing runs on layer 0's routing
        launch_nu = (float(torch.cat(seen).double().sum().item()) + nu * n_runs * n_layer) / (len(seen) + n_runs * n_layer)
    gu_expert = 2 * synth.tensor_bytes(synth.CB2, W0.n_ff_exp * D)
    dn_expert = synth.tensor_bytes(synth.Q2K, D * W0.n_ff_exp)
    sh = 3 * synth.tensor_bytes(synth.Q8_0, W0.n_ff_shared * D)
    gateup_bytes = nu * gu_expert + B * D * 4 + B * W0.n_expert_used * W0.n_ff_exp * 4
    layer_bytes = D * W0.n_expert * 4 + nu * (gu_expert + dn_expert) + sh + D * 4 + 2 * B * D * 4
    achieved = gateup_bytes / (gu_ms * 1e-3) / 1e9
    tokens_s = B / (ms_step * 1e-3)
    log("timed %d steps in %.3f s; gate/up %.2f us per launch" % (K, wall, gu_ms * 1e3))

    cpu = None
    if cpu_seconds is not None:
        import oracle
        t_start, done = time.perf_counter(), 0
        while True:
            oracle.stack_forward([host0], x0)
            done += 1
            el = time.perf_counter() - t_start
            if el >= cpu_seconds:
                break
        per_layer = el / done
        cpu = {"value": round(B / (n_layer * per_layer), 4), "unit": "tokens/s", "cores": 1, "kind": "oracle",
               "sample": "%d pass(es) of layer 0 at %d token(s) in %.1f s, times %d layers (nproc %d)" % (
                   done, B, el, n_layer, os.cpu_count() or 0)}
    kernel_name = "dec_k3_cb24096_kernel" if D == 4096 else "dec_k3_kernel"
    line = {
        "metric": METRIC,
        "value": round(tokens_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "stack43_b%d" % B, "tokens_per_step": B, "n_layer": n_layer,
            "n_embd": D, "n_expert": W0.n_expert, "n_expert_used": W0.n_expert_used, "n_ff_exp": W0.n_ff_exp,
            "n_ff_shared": W0.n_ff_shared, "formats": "CB2 gate/up, Q2K down, Q8_0 shared, fp32 router",
            "weights": "code-sampled per layer",
            "launch": "hipGraph of one %d-block step (moe_block_forward per block), replayed" % n_layer,
        },
        "timing": "HIP events on the replay stream around the %d timed steps" % K,
        "wall_ms_per_step": round(1000.0 * wall / K, 5),
        "hbm_gbps": round(n_layer * layer_bytes / (ms_step * 1e-3) / 1e9, 1),
        "algorithmic_bytes_per_step": int(n_layer * layer_bytes),
        "unique_experts_layer0": nu,
        "unique_experts_per_gate_up_launch": launch_nu,
        "roofline": {
            "kernel": kernel_name,
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(kernel_name, "stack43_b%d" % B),
            "bytes_per_launch": int(gateup_bytes),
            "avg_launch_us": round(gu_ms * 1e3, 3),
            "timing": "HIP events around runs of %d back-to-back stage-3 launches (one per layer), %d runs, "
                      "median per launch" % (n_layer, n_runs),
        },
        "cpu_baseline": cpu,
    }
    del ws, x, xn
    torch.cuda.empty_cache()
    return line


def run_hotlist(args):
    """Hot-expert profiling over the 43-block stack: per step, the selection
    counts of 43 layers' routings (8 tokens, top-6 of 256, a Zipf-skewed
    choice of experts so that some run far more often) are added into the
    profile, then the 11,008 {layer, expert} entries are sorted by hits."""
    import numpy as np
    import torch

    import quantized_routed_moe_router_amd as moe
    torch.cuda.set_device(0)
    n_layer, E, k, B = 43, 256, 6, 8
    rng = np.random.default_rng(13)
    idx = []
    for l in range(n_layer):
        p = 1.0 / np.arange(1, E + 1) ** 1.1
        p = p[rng.permutation(E)]
        p /= p.sum()
        idx.append(torch.from_numpy(np.stack([rng.choice(E, k, replace=False, p=p) for _ in range(B)])
                                    .astype(np.int32)).cuda())
    n = n_layer * E
    counts = torch.zeros(n, dtype=torch.int64, device="cuda")
    order = torch.empty(n, dtype=torch.int32, device="cuda")
    n_hot = torch.empty(1, dtype=torch.int32, device="cuda")

    def step():
        for l in range(n_layer):
            moe.count_selections(idx[l], E, l, counts)
        moe.hotlist(counts, order, n_hot)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            step()
    torch.cuda.current_stream().wait_stream(side)
    g.replay()
    torch.cuda.synchronize()
    K = args.steps
    t0 = time.perf_counter()
    for _ in range(K):
        g.replay()
    torch.cuda.synchronize()
    ms_step = 1000.0 * (time.perf_counter() - t0) / K
    # the sort's launch time: events around runs of 16 back-to-back launches
    runs = []
    for _ in range(8):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(1000000)
        a.record()
        for _ in range(16):
            moe.hotlist(counts, order, n_hot)
        b.record()
        torch.cuda.synchronize()
        runs.append(a.elapsed_time(b) / 16)
    sort_ms = float(np.median(runs))
    cmps = n * n  # the list by ranks: every key against every key
    achieved = cmps / (sort_ms * 1e-3) / 1e12
    cpu = None
    if not args.no_cpu:
        import oracle
        host = [t.cpu().numpy() for t in idx]
        c = np.zeros(n, np.int64)
        done, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < min(args.cpu_seconds, 5.0):
            for l in range(n_layer):
                oracle.count_selections(host[l], E, l, c)
            oracle.hotlist(c)
            done += 1
        el = time.perf_counter() - t0
        cpu = {"value": round(done / el, 2), "unit": "profile steps/s", "cores": 1, "kind": "oracle",
               "sample": "%d step(s) of 43 layers' counts and one sort of %d entries in %.1f s" % (done, n, el)}
    line = {
        "metric": "hot-expert profile steps/s (43 layers' selection counts + the sorted list)",
        "value": round(1000.0 / ms_step, 1), "unit": "profile steps/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "int64", "data": "synthetic",
        "config": {"workload": args.workload, "n_layer": n_layer, "n_expert": E, "n_expert_used": k,
                   "tokens_per_layer": B, "entries": n, "launch": "hipGraph of one step (44 launches), replayed"},
        "roofline": {
            "kernel": "hotlist_kernel", "bound": "alu", "achieved": round(achieved, 4), "peak": ALU_PEAK_TOPS,
            "unit": "T key compares/s", "frac": round(achieved / ALU_PEAK_TOPS, 5), "traffic": None,
            "avg_launch_us": round(sort_ms * 1e3, 3),
            "note": "each compare is a 64-bit compare and an add (about 3 lane operations); a one-launch "
                    "list of 11,008 entries is mostly launch and LDS staging",
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def cpu_baseline(L, x_all, T, mode, budget_s):
    """The plain C oracle, single-threaded, on a bounded sample of the same
    workload: whole steps of T rows for small T; for larger batches, chunks of
    at most 16 of the workload's rows through the full layer (routing, experts,
    shared expert and combine of those rows) until the time budget is spent."""
    import numpy as np

    import oracle
    import synth
    rows = T if T <= 32 else 16
    done, t_start = 0, time.perf_counter()
    nrow = x_all.shape[0]
    while True:
        i0 = (done * rows) % nrow
        x = x_all[i0:i0 + rows]
        if mode == 1:
            oracle.moe_forward(L, x_bf16=synth.to_bf16_bits(x))
        else:
            oracle.moe_forward(L, x=x)
        done += 1
        el = time.perf_counter() - t_start
        if rows < T:
            log("cpu baseline: %d row(s) in %.1f s" % (done * rows, el))
        if el >= budget_s or (rows > 1 and rows == T and done >= 1):
            break
    cpu = platform.processor() or platform.machine()
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": round(done * rows / el, 3), "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": "%d call(s) of %d token row(s)%s through the full layer in %.1f s (%s, nproc %d)" % (
                done, rows, "" if rows == T else " (chunks of the %d-row batch)" % T, el, cpu,
                os.cpu_count() or 0)}


if __name__ == "__main__":
    main()
