#!/usr/bin/env python3
"""Benchmark of the MXFP4 weight-streaming MoE layer on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload moe_t32_zipf] [--layers L]
    python bench.py --workload dense_t1|dense_t4 [--act8]      (the dense mx_linear)

A step is one MoE layer forward (route + sort, gate_up + SwiGLU, down + combine) over one
batch of T tokens.  Steps cycle over L distinct layers (own weights, own activations and
routing), as a decode step walks a stack of MoE layers, so no step finds its expert
weights in a cache: the 256 MB last-level cache is smaller than the active bytes of L-1
layers.  Inputs are resident in HBM before timing.  The timed region replays one HIP
graph holding the L layer forwards (moe_mxfp4_forward) K/L times, between two device
synchronizations; K is rounded up to a multiple of L.

Printed: one JSON line with the layer time (us), effective weight GB/s, a roofline entry
for the dominant kernel (gate_up) and the CPU oracle's time on a bounded sample of the same
workload.  The kernel's launch time comes from a second pass over the same K steps right
after the timed region, issued as the three stage calls with a HIP event between them on
the stream the kernels run on.  roofline.traffic is the kernel's HBM bytes per launch as
measured by the committed counter summary under profiles/, and null when the workload
differs or the kernel's sources changed since the counters were taken.

Dense workloads (dense_t1, dense_t4): a step is one mx_linear call.  The calls cycle over
enough copies of the weights (own addresses) that their total exceeds the last-level cache
by far; one HIP graph holds one call per copy.  The per-call time of the roofline entry
comes from HIP events around each graph replay of the timed region.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

import numpy as np

METRIC = "µs per MXFP4 MoE layer and effective weight GB/s (% of 8 TB/s) at T=1..128"
DENSE_METRIC = "µs per dense MXFP4 linear call (mx_linear) and effective weight GB/s (% of 8 TB/s)"
# the dense calls cycle over weight copies totalling at least this many bytes
DENSE_CYCLE_BYTES = 1 << 30
HBM_PEAK_GBPS = 8000.0
ROOT = os.path.dirname(os.path.abspath(__file__))
# sources (and build flags) the gate_up kernel is compiled from; the counter summary records
# their hash, so measured traffic is only reported for the kernel it was measured on
GATE_UP_SOURCES = ("mxfp4_weight_moe_amd/build.py", "mxfp4_weight_moe_amd/csrc/mx_device.hpp",
                   "mxfp4_weight_moe_amd/csrc/mx_internal.hpp", "mxfp4_weight_moe_amd/csrc/mx_stream.hpp",
                   "mxfp4_weight_moe_amd/csrc/mx_act8.hpp", "mxfp4_weight_moe_amd/csrc/moe_policies.hpp",
                   "mxfp4_weight_moe_amd/csrc/moe_experts.hip")
GATE_UP_COUNTERS = os.path.join(ROOT, "profiles", "moe_gate_up_kernel.moe_t32_zipf.hbm_counters.txt")


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="moe_t32_zipf",
                    help="moe_t4 | moe_t32_zipf | moe_t128 | moe_sweep_t<T>")
    ap.add_argument("--layers", type=int, default=4, help="distinct layers cycled by the steps")
    ap.add_argument("--eager", action="store_true", help="time eager launches instead of graph replay")
    ap.add_argument("--persistent", action="store_true",
                    help="time the single-launch layer (moe_mxfp4_forward_persistent, T <= 16)")
    ap.add_argument("--act8", action="store_true",
                    help="MXFP8 activations for both expert GEMMs (moe_mxfp4_forward_a8, scaled MFMA)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=32, help="tokens of the oracle's timed sample")
    ap.add_argument("--stage-steps", type=int, default=None, help="steps of the per-kernel event pass (default K)")
    ap.add_argument("--copy-mib", type=int, default=1024,
                    help="size of the untimed reference copy (read + write) that calibrates HBM byte counters")
    return ap.parse_args()


def workload_config(name: str):
    import synthetic
    if name in synthetic.MOE_CONFIGS:
        return synthetic.MOE_CONFIGS[name]
    if name.startswith("moe_sweep_t"):
        return synthetic.sweep_config(int(name[len("moe_sweep_t"):]))
    raise SystemExit(f"unknown workload {name}")


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def gate_up_source_hash() -> str:
    h = hashlib.sha256()
    for rel in GATE_UP_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per gate_up launch from the committed counter summary ("key: value" lines),
    or None when the summary is absent, for another workload, or for other kernel sources."""
    try:
        with open(GATE_UP_COUNTERS) as f:
            kv = dict(line.split(":", 1) for line in f if ":" in line and not line.startswith((" ", "#")))
    except OSError:
        return None
    kv = {a.strip(): b.strip() for a, b in kv.items()}
    if kv.get("workload") != workload or kv.get("kernel_sources_sha256") != gate_up_source_hash():
        return None
    try:
        return int(kv["hbm_read_bytes_per_launch"]) + int(kv["hbm_write_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); this library has no multi-GPU path.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    import mxfp4_weight_moe_amd as mx  # raises if the HIP library is not built
    import synthetic

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.workload in synthetic.LINEAR_CONFIGS:
        return dense_main(args, synthetic.LINEAR_CONFIGS[args.workload], torch, mx, dev)
    cfg = workload_config(args.workload)
    T, H, I, E, k = cfg.T, cfg.H, cfg.I, cfg.E, cfg.k
    ns = cfg.n_shared
    if args.persistent and (T > 16 or T * k > 128 or ns or args.act8):
        raise SystemExit("--persistent takes T <= 16, T * top_k <= 128, no shared experts and bf16 activations")
    # the event pass times each layer as a whole when the stage calls cannot reproduce it
    whole_layer = args.persistent or ns > 0 or args.act8
    L = max(1, args.layers)

    def log(*a):
        print(*a, file=sys.stderr, flush=True)

    # ---------------------------------------------------------------- set-up (all before timing)
    log(f"[bench] workload {cfg.name}: T={T} H={H} I={I} E={E} k={k} routing={cfg.routing} layers={L}")
    layers = []
    for li in range(L):
        w = synthetic.moe_weights_device(cfg, dev, layer=li)
        x_bits, logits = synthetic.moe_activations(cfg, layer=li)
        layers.append(dict(
            w=w,
            x=torch.from_numpy(x_bits.view(np.int16)).to(dev).view(torch.bfloat16),
            logits=torch.from_numpy(logits).to(dev),
            y=torch.empty((T, H), dtype=torch.bfloat16, device=dev),
            x_bits=x_bits, logits_host=logits,
        ))
    ws = mx.workspace(T, H, I, E + ns, k + ns, dev)
    # buffers of the stage-by-stage pass
    ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    gates = torch.empty((T, k), dtype=torch.float32, device=dev)
    srt = dict(counts=torch.empty(E, dtype=torch.int32, device=dev),
               offsets=torch.empty(E + 1, dtype=torch.int32, device=dev),
               sorted_slots=torch.empty(T * k, dtype=torch.int32, device=dev),
               active=torch.empty(E, dtype=torch.int32, device=dev),
               num_active=torch.empty(2, dtype=torch.int32, device=dev))
    h = torch.empty((T * k, I), dtype=torch.bfloat16, device=dev)
    names = ("layer",) if whole_layer else ("route_sort", "gate_up", "down_combine")
    n_active = []
    for lay in layers:
        mx.moe_route_sort(lay["logits"], k, ids=ids, gates=gates, out=srt)
        n_active.append(int(srt["num_active"][0].item()) + ns)  # the shared experts are always read
    log(f"[bench] inputs resident: {torch.cuda.memory_allocated() / 2**30:.1f} GiB; active experts {n_active}")

    def forward(lay):
        w = lay["w"]
        mx.moe_mxfp4_forward(lay["x"], lay["logits"], k, w["wgu"], w["sgu"], w["wd"], w["sd"], out=lay["y"], ws=ws,
                             persistent=args.persistent, n_shared=ns, act8=args.act8)

    def staged(i, e, stream):
        lay = layers[i % L]
        w = lay["w"]
        if whole_layer:  # one kernel per layer (persistent), or the whole layer's launches
            e[0].record(stream)
            forward(lay)
            e[1].record(stream)
            return
        e[0].record(stream)
        mx.moe_route_sort(lay["logits"], k, ids=ids, gates=gates, out=srt)
        e[1].record(stream)
        mx.moe_gate_up_swiglu(lay["x"], w["wgu"], w["sgu"], srt, k, h=h, ws=ws)
        e[2].record(stream)
        mx.moe_down_combine(h, gates, w["wd"], w["sd"], srt, T, k, out=lay["y"], ws=ws)
        e[3].record(stream)

    for lay in layers:
        forward(lay)
    torch.cuda.synchronize()

    # Untimed reference copy of a known size: under a counter profiler its FETCH_SIZE and
    # WRITE_SIZE give the scale between the counters and bytes actually moved.
    if args.copy_mib > 0:
        src = torch.empty(args.copy_mib << 18, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    graph = None
    if not args.eager:
        # one graph holds the L layers back to back, as one decode step's graph would
        side = torch.cuda.Stream(dev)
        side.wait_stream(torch.cuda.current_stream(dev))
        with torch.cuda.stream(side):
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph, stream=side):
                for lay in layers:
                    forward(lay)
        torch.cuda.current_stream(dev).wait_stream(side)
        torch.cuda.synchronize()

    def run_steps(n):  # n is a multiple of L
        for _ in range(n // L):
            if graph is not None:
                graph.replay()
            else:
                for lay in layers:
                    forward(lay)

    # ---------------------------------------------------------------- warm-up and timed region
    # Warm-up long enough for the clocks to settle: kernel times drift down over the
    # first tens of milliseconds of back-to-back work after an idle GPU.
    run_steps(L * max(1, -(-args.warmup // L)))
    reps = max(1, -(-args.steps // L))
    K = reps * L
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run_steps(K)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / K
    log(f"[bench] timed {K} steps: {ms_per_step * 1e3:.1f} us/layer")

    # ---------------------------------------------------------------- per-kernel pass (HIP events)
    # Right after the timed region, the same K layer forwards issued as the three stage calls
    # (the kernels the forward launches), with a HIP event between stages recorded on the
    # stream the kernels are launched on.  Launches are queued far faster than the GPU
    # drains them, so the stream never runs dry and each event pair brackets one kernel.
    stream = torch.cuda.current_stream(dev)
    KS = args.stage_steps or K
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(KS)]
    for i in range(KS):
        staged(i, evs[i], stream)
    torch.cuda.synchronize()
    stage_ms = {n: [] for n in names}
    for e in evs:
        for j, n in enumerate(names):
            stage_ms[n].append(e[j].elapsed_time(e[j + 1]))
    staged_us_per_layer = evs[0][0].elapsed_time(evs[-1][-1]) * 1e3 / KS

    # ---------------------------------------------------------------- bytes and roofline
    gu_expert = 2 * I * H // 2 + 2 * I * H // 32          # gate_up codes + scales per expert
    dn_expert = H * I // 2 + H * I // 32                  # down codes + scales per expert
    act_bytes = T * H * 2 + T * E * 4 + T * H * 2         # x, router logits, y
    layer_bytes = [na * (gu_expert + dn_expert) + act_bytes for na in n_active]
    mean_layer_bytes = float(np.mean([layer_bytes[i % L] for i in range(K)]))
    us_per_layer = ms_per_step * 1e3
    eff_gbps = mean_layer_bytes / (us_per_layer * 1e-6) / 1e9
    if whole_layer:
        # the single kernel (or the layer's launches together) reads the whole layer's bytes
        gu_bytes = [layer_bytes[i % L] for i in range(KS)]
        gu_ms = stage_ms["layer"]
    else:
        # gate_up per launch: its experts' codes + scales, x read once, h written
        gu_bytes = [n_active[i % L] * gu_expert + T * H * 2 + T * k * I * 2 for i in range(KS)]
        gu_ms = stage_ms["gate_up"]
    gu_achieved = float(np.sum(gu_bytes) / (np.sum(gu_ms) * 1e-3) / 1e9)
    roofline = {
        "kernel": ("moe_fused_kernel" if args.persistent else "layer (all launches)") if whole_layer
        else "moe_gate_up_kernel",
        "bound": "hbm",
        "achieved": round(gu_achieved, 1),
        "peak": HBM_PEAK_GBPS,
        "unit": "GB/s",
        "frac": round(gu_achieved / HBM_PEAK_GBPS, 4),
        "traffic": None if whole_layer else measured_traffic(cfg.name),
        "avg_launch_us": round(float(np.mean(gu_ms)) * 1e3, 2),
        "launches": len(gu_ms),
        "timing": "HIP events on the launch stream, one pair per launch, right after the timed region",
        "bytes_per_launch": int(np.mean(gu_bytes)),
    }

    # ---------------------------------------------------------------- CPU oracle baseline
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        lay = layers[0]
        n = max(1, min(args.cpu_tokens, T))
        toks = np.arange(n, dtype=np.int32)
        w_host = {key: lay["w"][key].cpu().numpy() for key in ("wgu", "sgu", "wd", "sd")}
        threads = oracle.default_threads()
        log(f"[bench] oracle on {n} of {T} tokens, {threads} threads")
        c0 = time.perf_counter()
        oracle.moe_tokens(lay["x_bits"], lay["logits_host"], k, w_host["wgu"], w_host["sgu"], w_host["wd"],
                          w_host["sd"], T, H, I, E, tokens=toks, nthreads=threads, n_shared=ns, act8=args.act8)
        c1 = time.perf_counter()
        cpu = {
            "value": round((c1 - c0) * (T / n) * 1e6, 1),
            "unit": "us/layer",
            "cores": threads,
            "kind": "oracle",
            "sample": f"layer 0, tokens 0..{n - 1} of {T} (all {k} routed experts each), full route+gate_up+down+combine; "
                      f"time scaled by {T}/{n}; CPU: {cpu_model()}",
            "seconds": round(c1 - c0, 2),
        }
        del w_host

    out = {
        "metric": METRIC,
        "value": round(us_per_layer, 2),
        "unit": "us/layer",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8 (E4M3) x fp4 (E2M1), fp32 accumulate" if args.act8 else "bf16",
        "data": "synthetic",
        "config": {
            "workload": cfg.name, "T": T, "H": H, "I": I, "E": E, "top_k": k, "n_shared": ns, "routing": cfg.routing,
            "weights": "MXFP4 (E2M1 codes, E8M0 scale per 32)", "accumulate": "fp32",
            "activations": "MXFP8 (E4M3, E8M0 scale per 32), quantized in the GEMM kernels" if args.act8 else "bf16",
            "layers_cycled": L, "timing": "eager launches" if args.eager else "HIP graph replay",
            "path": "one persistent launch" if args.persistent else "route_sort, gate_up, down, combine launches",
        },
        "effective_GBps": round(eff_gbps, 1),
        "pct_of_8TBps": round(100 * eff_gbps / HBM_PEAK_GBPS, 2),
        "active_experts": n_active,
        "algorithmic_bytes_per_layer": int(mean_layer_bytes),
        "stages_us": {n: round(float(np.mean(v)) * 1e3, 2) for n, v in stage_ms.items()},
        "staged_us_per_layer": round(staged_us_per_layer, 2),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "env": {"GPU_MAX_HW_QUEUES": os.environ.get("GPU_MAX_HW_QUEUES"), "torch": torch.__version__,
                "hip": getattr(torch.version, "hip", None)},
    }
    print(json.dumps(out), flush=True)


def dense_main(args, cfg, torch, mx, dev):
    """The dense layer: y[T,N] = bf16(x[T,K] @ W[N,K]^T) with MXFP4 W, one call per step."""
    import synthetic

    def log(*a):
        print(*a, file=sys.stderr, flush=True)

    T, K, N = cfg.T, cfg.K, cfg.N
    x_bits, w, s = synthetic.linear_inputs(cfg)
    w_bytes = w.nbytes + s.nbytes
    copies = max(8, -(-DENSE_CYCLE_BYTES // w_bytes))
    log(f"[bench] workload {cfg.name}: T={T} K={K} N={N}, {copies} weight copies of {w_bytes} B")
    x = torch.from_numpy(x_bits.view(np.int16)).to(dev).view(torch.bfloat16)
    w0, s0 = torch.from_numpy(w).to(dev), torch.from_numpy(s).to(dev)
    ws = [(w0.clone(), s0.clone()) for _ in range(copies)]
    ys = [torch.empty((T, N), dtype=torch.bfloat16, device=dev) for _ in range(copies)]
    del w0, s0

    def call(i):
        mx.mx_linear(x, ws[i][0], ws[i][1], out=ys[i], act8=args.act8)

    for i in range(copies):
        call(i)
    torch.cuda.synchronize()
    side = torch.cuda.Stream(dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=side):
            for i in range(copies):
                call(i)
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()
    for _ in range(max(1, -(-args.warmup // copies))):
        graph.replay()
    reps = max(1, -(-args.steps // copies))
    nsteps = reps * copies
    # HIP events on the replay stream bracket each replay of the graph: a call is shorter than
    # its host-side submission, so eager event pairs would time the host, not the kernel
    stream = torch.cuda.current_stream(dev)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    evs[0].record(stream)
    for r in range(reps):
        graph.replay()
        evs[r + 1].record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    us_per_call = (t1 - t0) * 1e6 / nsteps
    log(f"[bench] timed {nsteps} calls: {us_per_call:.2f} us/call")
    call_ms = [evs[r].elapsed_time(evs[r + 1]) / copies for r in range(reps)]
    call_bytes = w_bytes + T * K * 2 + T * N * 2  # weights, x, y
    achieved = call_bytes / (float(np.mean(call_ms)) * 1e-3) / 1e9
    eff_gbps = call_bytes / (us_per_call * 1e-6) / 1e9

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        threads = oracle.default_threads()
        fn = oracle.mx_linear_a8 if args.act8 else oracle.mx_linear
        reps_cpu = 3
        c0 = time.perf_counter()
        for _ in range(reps_cpu):
            fn(x_bits, w, s, T, K, N, nthreads=threads)
        c1 = time.perf_counter()
        cpu = {"value": round((c1 - c0) / reps_cpu * 1e6, 1), "unit": "us/call", "cores": threads, "kind": "oracle",
               "sample": f"the whole call, {reps_cpu} repetitions averaged; CPU: {cpu_model()}",
               "seconds": round(c1 - c0, 2)}

    out = {
        "metric": DENSE_METRIC,
        "value": round(us_per_call, 3),
        "unit": "us/call",
        "n_gpus": 1,
        "steps": nsteps,
        "warmup": args.warmup,
        "ms_per_step": round(us_per_call * 1e-3, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8 (E4M3) x fp4 (E2M1), fp32 accumulate" if args.act8 else "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "T": T, "K": K, "N": N, "weights": "MXFP4 (E2M1 codes, E8M0 scale per 32)",
                   "activations": "MXFP8, quantized in the kernel" if args.act8 else "bf16", "accumulate": "fp32",
                   "weight_copies_cycled": copies, "timing": "HIP graph replay"},
        "effective_GBps": round(eff_gbps, 1),
        "pct_of_8TBps": round(100 * eff_gbps / HBM_PEAK_GBPS, 2),
        "algorithmic_bytes_per_call": call_bytes,
        "roofline": {"kernel": "mx_linear_kernel", "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": None,
                     "avg_launch_us": round(float(np.mean(call_ms)) * 1e3, 3), "launches": nsteps,
                     "timing": "HIP events on the replay stream around each graph replay of the timed region, "
                               "per call (includes the graph's gaps between kernels)",
                     "bytes_per_launch": call_bytes},
        "cpu_baseline": cpu,
        "env": {"GPU_MAX_HW_QUEUES": os.environ.get("GPU_MAX_HW_QUEUES"), "torch": torch.__version__,
                "hip": getattr(torch.version, "hip", None)},
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
