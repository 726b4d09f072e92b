#!/usr/bin/env python3
"""Benchmark of the MXFP4 weight-streaming MoE layer on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload moe_t32_zipf] [--layers L]
    python bench.py --workload dense_t1|dense_t4 [--act8]      (the dense mx_linear)

A step is one MoE layer forward (route + sort, gate_up + SwiGLU, down + combine) over one
batch of T tokens, in the launches moe_mxfp4_forward makes for that size (config.path).  Steps cycle over L distinct layers (own weights, own activations and
routing), as a decode step walks a stack of MoE layers, so no step finds its expert
weights in a cache: the 256 MB last-level cache is smaller than the active bytes of L-1
layers.  Inputs are resident in HBM before timing.  One HIP graph holds the L layer
forwards (moe_mxfp4_forward); the timed region replays it K/L times between two device
synchronizations (K rounded up to a multiple of L), with a HIP event between replays for
the per-replay statistics.

Before the W warm-up steps, a settle phase replays the same graph for --settle-ms of wall
time.  After an idle spell the GPU's power management takes some 30 ms of sustained load
to reach its steady state, and the first replays run up to a third slower; the settle
phase is the pages' practice of warming the GPU before timed kernels ("Zyphra Inference
Wave 2", Methodology and Limitations, Appendix B) with a length set in time rather than in
steps.  The first replays of the settle phase are reported beside the result.

Printed: one JSON line for the chosen workload -- layer time (us), effective weight GB/s
and its share of 8 TB/s and of this GPU's measured copy and read bandwidth (the library's
HBM reference kernels), a roofline entry for the dominant kernel (the launch of both
expert GEMMs from 6 to 32 tokens where the forward runs them in one, gate_up otherwise), the CPU
oracle's time on a bounded sample of the same workload and the worst parity ratio of that
sample against the GPU's output, and (by default) the other configurations of the
benchmark under "configs".  The kernel's launch time comes from a pass of max(K, 200)
steps right after the timed region (behind a few graph replays, so the GPU does not idle in
between), issued as the stage calls that make the forward's launches, with a HIP event
between them on the stream the kernels run on.  roofline.traffic is the kernel's HBM bytes
per launch as measured by the committed counter summary under profiles/, and null when the
workload differs or the kernel's sources changed since the counters were taken.

Dense workloads (dense_t1, dense_t4): a step is one mx_linear call.  The calls cycle over
enough copies of the weights (own addresses) that their total exceeds the last-level cache
by far; one HIP graph holds one call per copy.  The per-call time of the roofline entry
comes from HIP events around each graph replay of the timed region.
"""
from __future__ import annotations

import argparse
import glob
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
MOE_REL = 1e-2  # the MoE acceptance bound: |gpu - oracle| <= 1e-2 * sum_j g_j sum_i |h_i w_in| + 1 bf16 ulp
ROOT = os.path.dirname(os.path.abspath(__file__))
STAGE_MIN = 200           # launches the per-kernel event pass times at least
STAGE_LEAD_REPLAYS = 8    # graph replays queued right before it
# the other configurations a default run reports beside its headline workload
EXTRA_WORKLOADS = ("dense_t1", "dense_t4", "moe_t4", "moe_t128", "moe_sweep_t1")
# sources (and build flags) the expert GEMM kernels are compiled from; the counter summaries
# record their hash, so measured traffic is only reported for the kernel it was measured on
EXPERT_SOURCES = ("mxfp4_weight_moe_amd/build.py", "mxfp4_weight_moe_amd/csrc/mx_device.hpp",
                   "mxfp4_weight_moe_amd/csrc/mx_internal.hpp", "mxfp4_weight_moe_amd/csrc/mx_stream.hpp",
                   "mxfp4_weight_moe_amd/csrc/mx_act8.hpp", "mxfp4_weight_moe_amd/csrc/moe_policies.hpp",
                   "mxfp4_weight_moe_amd/csrc/moe_experts.hip", "mxfp4_weight_moe_amd/csrc/moe_fused.hip")
HEADLINE_COUNTERS = os.path.join(ROOT, "profiles", "moe_experts_sorted_kernel.moe_t32_zipf.hbm_counters.txt")
MFMA_COUNTERS = os.path.join(ROOT, "profiles", "moe_t128.mfma_counters.txt")


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="wall time of graph replays before the warm-up steps (power-management settle)")
    ap.add_argument("--workload", default="moe_t32_zipf",
                    help="moe_t4 | moe_t32_zipf | moe_t128 | moe_sweep_t<T> | dense_t1 | dense_t4 | ...")
    ap.add_argument("--layers", type=int, default=4, help="distinct layers cycled by the steps")
    ap.add_argument("--eager", action="store_true", help="time eager launches instead of graph replay")
    ap.add_argument("--persistent", action="store_true",
                    help="time the single-launch layer (moe_mxfp4_forward_persistent, T <= 16)")
    ap.add_argument("--act8", action="store_true",
                    help="MXFP8 activations for both expert GEMMs (moe_mxfp4_forward_a8, scaled MFMA)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=32, help="tokens per layer of the oracle's timed sample")
    ap.add_argument("--cpu-layers", type=int, default=2, help="layers of the oracle's timed sample")
    ap.add_argument("--stage-steps", type=int, default=None,
                    help="steps of the per-kernel event pass (default max(K, 200))")
    ap.add_argument("--no-extra", action="store_true", help="time only --workload (no other configurations)")
    ap.add_argument("--extra-steps", type=int, default=80, help="timed steps of each other configuration")
    ap.add_argument("--hbm-mib", type=int, default=4096, help="buffer of the HBM reference kernels (0: skip)")
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


def gpu_clocks() -> dict:
    """The active SCLK / MCLK levels the driver reports (sysfs), where readable."""
    out = {}
    for f in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_[sm]clk")):
        try:
            with open(f) as fh:
                cur = [line.split(":", 1)[1].strip(" *\n") for line in fh if "*" in line]
            if cur:
                out[os.path.basename(f)[len("pp_dpm_"):]] = cur[0]
        except OSError:
            pass
    return out


def forward_path(T: int, k: int, E: int, ns: int, I: int, H: int) -> str:
    """The launches moe_mxfp4_forward makes for these sizes (its dispatch)."""
    if (ns == 0 and T <= 32 and T * k <= 256 and E <= 1024 and I % 1024 == 0 and H % 128 == 0
            and min(T * k, E) * (I // 64) >= 1536):
        return "route, gate_up + down (one launch, sorting in every workgroup), combine launches"
    if ns == 0 and T <= 16 and T * k <= 128:
        return "gate_up (routing and sorting in every workgroup), down, combine launches (combine inside down at the smallest T)"
    if ns == 0 and T <= 32 and T * k <= 256 and E <= 1024:
        return "route, gate_up (sorting in every workgroup), down, combine launches"
    if (16 < T <= 32 and I % 1024 == 0 and H % 128 == 0
            and min(T * (k + ns), E + ns) * (I // 64) >= 1536):
        return "route, sort, gate_up + down (one launch), combine launches"
    return "route_sort, gate_up, down, combine launches"


def source_hash(paths) -> str:
    h = hashlib.sha256()
    for rel in paths:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def expert_source_hash() -> str:
    return source_hash(EXPERT_SOURCES)


def read_summary(path):
    """The "key: value" lines of a committed counter summary, or None."""
    try:
        with open(path) as f:
            kv = dict(line.split(":", 1) for line in f if ":" in line and not line.startswith((" ", "#")))
    except OSError:
        return None
    return {a.strip(): b.strip() for a, b in kv.items()}


def measured_traffic(workload: str, kernel: str):
    """HBM bytes per launch of `kernel` from the committed counter summary, or None when the
    summary is absent, for another workload or kernel, or for other kernel sources."""
    kv = read_summary(HEADLINE_COUNTERS)
    if (not kv or kv.get("workload") != workload or kv.get("kernel") != kernel
            or kv.get("kernel_sources_sha256") != expert_source_hash()):
        return None
    try:
        return int(kv["hbm_read_bytes_per_launch"]) + int(kv["hbm_write_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def measured_mfma():
    """MFMA utilisation of the expert GEMMs at T = 128 from the committed counter summary
    (null when its kernel sources changed since)."""
    kv = read_summary(MFMA_COUNTERS)
    if not kv or kv.get("kernel_sources_sha256") != expert_source_hash():
        return None
    try:
        return {"workload": kv["workload"], "gate_up_mfma_busy_pct": float(kv["gate_up_mfma_busy_pct"]),
                "down_mfma_busy_pct": float(kv["down_mfma_busy_pct"]),
                "gate_up_useful_tflops": float(kv["gate_up_useful_tflops"]),
                "source": os.path.relpath(MFMA_COUNTERS, ROOT)}
    except (KeyError, ValueError):
        return None


def stats_us(v):
    a = np.asarray(v, np.float64)
    return {"n": int(a.size), "mean": round(float(a.mean()), 2), "median": round(float(np.median(a)), 2),
            "p10": round(float(np.percentile(a, 10)), 2), "p90": round(float(np.percentile(a, 90)), 2)}


def moe_bound_ratio(gpu_bits, ora_bits, scale):
    """Worst |gpu - oracle| / (1e-2 * scale + 1 bf16 ulp) over the finite outputs, and the
    number of outputs whose NaN / Inf status differs."""
    def f(b):
        return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    g, o = f(gpu_bits), f(ora_bits)
    fin = np.isfinite(g) & np.isfinite(o)
    mismatch = int(((np.isnan(g) != np.isnan(o)) | ((np.isinf(g) | np.isinf(o)) & ~fin & (g != o))).sum())
    m = np.maximum(np.abs(g[fin]), np.abs(o[fin]))
    small = m < 2.0 ** -126
    ulp = np.where(small, 2.0 ** -133, 2.0 ** (np.floor(np.log2(np.where(small, 1.0, m))) - 7))
    ratio = np.abs(g[fin] - o[fin]) / (MOE_REL * np.asarray(scale, np.float64)[fin] + ulp)
    return (float(ratio.max()) if ratio.size else 0.0), mismatch


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def settle(replay, stream, torch, settle_ms: float, units: int, record: int = 8):
    """Replays back to back for settle_ms of wall time, at most two in flight (so the host
    never queues more work than that); returns (replays, the first `record` replays' us per
    unit: per layer, or per call)."""
    timed = [torch.cuda.Event(enable_timing=True) for _ in range(record + 1)]
    lag = [torch.cuda.Event(), torch.cuda.Event()]
    timed[0].record(stream)
    n = 0
    t0 = time.perf_counter()
    while True:
        if n >= 2:
            lag[n % 2].synchronize()  # replay n - 2 has finished
        replay()
        lag[n % 2].record(stream)
        n += 1
        if n <= record:
            timed[n].record(stream)
        if n >= record and (time.perf_counter() - t0) * 1e3 >= settle_ms:
            break
    torch.cuda.synchronize()
    first = [round(timed[i].elapsed_time(timed[i + 1]) * 1e3 / units, 2) for i in range(record)]
    return n, first


# ------------------------------------------------------------------------------ MoE workloads

def moe_case(cfg, args, torch, mx, dev, *, steps: int, warmup: int, stage_pass: bool, cpu_leg: bool):
    """Times one MoE workload; returns its result dict (the JSON line's fields)."""
    import synthetic
    T, H, I, E, k = cfg.T, cfg.H, cfg.I, cfg.E, cfg.k
    ns = cfg.n_shared
    whole_layer = args.persistent or ns > 0 or args.act8
    L = max(1, args.layers)
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
    ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    gates = torch.empty((T, k), dtype=torch.float32, device=dev)
    srt = dict(counts=torch.empty(E, dtype=torch.int32, device=dev),
               offsets=torch.empty(E + 1, dtype=torch.int32, device=dev),
               sorted_slots=torch.empty(T * k, dtype=torch.int32, device=dev),
               active=torch.empty(E, dtype=torch.int32, device=dev),
               num_active=torch.empty(2, dtype=torch.int32, device=dev))
    h = torch.empty((T * k, I), dtype=torch.bfloat16, device=dev)
    d = torch.empty((T * k, H), dtype=torch.float32, device=dev)
    # From 17 to 32 tokens (no shared experts) the forward routes in a launch of its own, then
    # runs both expert GEMMs in one launch (or, where that does not apply, a gate_up that
    # sorts the slots in every workgroup); the per-kernel pass issues the same calls.
    path = forward_path(T, k, E, ns, I, H)
    single_path = not whole_layer and path.startswith("route, gate_up + down")
    sorted_path = not whole_layer and path.startswith("route, gate_up (")
    names = ("layer",) if whole_layer else (("route", "gate_up_down", "combine") if single_path else
                                           ("route", "gate_up", "down_combine") if sorted_path
                                           else ("route_sort", "gate_up", "down_combine"))
    n_active = []
    for lay in layers:
        mx.moe_route_sort(lay["logits"], k, ids=ids, gates=gates, out=srt)
        n_active.append(int(srt["num_active"][0].item()) + ns)  # the shared experts are always read
    log(f"[bench] inputs resident: {torch.cuda.memory_allocated() / 2**30:.1f} GiB; active experts {n_active}")

    def forward(lay):
        w = lay["w"]
        mx.moe_mxfp4_forward(lay["x"], lay["logits"], k, w["wgu"], w["sgu"], w["wd"], w["sd"], out=lay["y"], ws=ws,
                             persistent=args.persistent, n_shared=ns, act8=args.act8, check=False)

    def staged(i, e, stream):
        lay = layers[i % L]
        w = lay["w"]
        if whole_layer:  # one kernel per layer (persistent), or the whole layer's launches
            e[0].record(stream)
            forward(lay)
            e[1].record(stream)
            return
        if single_path:
            h.view(torch.int16).fill_(-1)  # the expert launch's "not yet written" pattern
            e[0].record(stream)
            mx.moe_route_topk(lay["logits"], k, ids=ids, gates=gates)
            e[1].record(stream)
            mx.moe_expert_gemms_from_ids(lay["x"], ids, w["wgu"], w["sgu"], w["wd"], w["sd"], h=h, d=d, ws=ws,
                                         fill_h=False)
            e[2].record(stream)
            mx.moe_combine(d, gates, out=lay["y"])
            e[3].record(stream)
            return
        e[0].record(stream)
        if sorted_path:
            mx.moe_route_topk(lay["logits"], k, ids=ids, gates=gates)
            e[1].record(stream)
            mx.moe_gate_up_swiglu_from_ids(lay["x"], ids, w["wgu"], w["sgu"], h=h, sort=srt, ws=ws)
        else:
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
    if stage_pass and args.copy_mib > 0:
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

    def replay():
        if graph is not None:
            graph.replay()
        else:
            for lay in layers:
                forward(lay)

    stream = torch.cuda.current_stream(dev)
    # ---------------------------------------------------------------- settle, warm-up, timed region
    clocks_before = gpu_clocks()
    n_settle, first = settle(replay, stream, torch, args.settle_ms, L)
    for _ in range(max(0, -(-warmup // L))):
        replay()
    reps = max(1, -(-steps // L))
    K = reps * L
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    evs[0].record(stream)
    for r in range(reps):
        replay()
        evs[r + 1].record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    clocks_after = gpu_clocks()
    ms_per_step = (t1 - t0) * 1e3 / K
    replay_us = [evs[r].elapsed_time(evs[r + 1]) * 1e3 / L for r in range(reps)]
    log(f"[bench] {cfg.name}: settle {n_settle} replays (first {first}); timed {K} steps: "
        f"{ms_per_step * 1e3:.1f} us/layer")

    gu_expert = 2 * I * H // 2 + 2 * I * H // 32          # gate_up codes + scales per expert
    dn_expert = H * I // 2 + H * I // 32                  # down codes + scales per expert
    act_bytes = T * H * 2 + T * E * 4 + T * H * 2         # x, router logits, y
    layer_bytes = [na * (gu_expert + dn_expert) + act_bytes for na in n_active]
    mean_layer_bytes = float(np.mean([layer_bytes[i % L] for i in range(K)]))
    us_per_layer = ms_per_step * 1e3
    eff_gbps = mean_layer_bytes / (us_per_layer * 1e-6) / 1e9
    res = {
        "value": round(us_per_layer, 2), "K": K, "ms_per_step": round(ms_per_step, 5),
        "effective_GBps": round(eff_gbps, 1), "pct_of_8TBps": round(100 * eff_gbps / HBM_PEAK_GBPS, 2),
        "active_experts": n_active, "algorithmic_bytes_per_layer": int(mean_layer_bytes),
        "replay_us_per_layer": stats_us(replay_us),
        "settle": {"ms": args.settle_ms, "replays": n_settle, "first_replays_us_per_layer": first},
        "clocks": {"before": clocks_before, "after": clocks_after},
        "config": {
            "workload": cfg.name, "T": T, "H": H, "I": I, "E": E, "top_k": k, "n_shared": ns, "routing": cfg.routing,
            "weights": "MXFP4 (E2M1 codes, E8M0 scale per 32)", "accumulate": "fp32",
            "activations": "MXFP8 (E4M3, E8M0 scale per 32), quantized in the GEMM kernels" if args.act8 else "bf16",
            "layers_cycled": L, "timing": "eager launches" if args.eager else "HIP graph replay",
            "path": "one persistent launch" if args.persistent else
            forward_path(T, k, E, ns, I, H),
        },
    }

    # ---------------------------------------------------------------- per-kernel pass (HIP events)
    # Right after the timed region, the layer forwards issued as the three stage calls
    # (the kernels the forward launches), with a HIP event between stages recorded on the
    # stream the kernels are launched on.  Launches are queued far faster than the GPU
    # drains them, so the stream never runs dry and each event pair brackets one kernel.
    if stage_pass:
        # At least STAGE_MIN steps whatever --steps says, and the GPU kept loaded across the
        # hand-over (replays queued with no host synchronization before the pass): after the
        # timed region's synchronization an idle GPU would start the pass in the power
        # manager's transient (measured: 20 launches right after a synchronization averaged
        # 280 us against 254 us).
        KS = args.stage_steps or max(K, STAGE_MIN)
        sev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(KS)]
        for _ in range(STAGE_LEAD_REPLAYS):
            replay()
        for i in range(KS):
            staged(i, sev[i], stream)
        torch.cuda.synchronize()
        stage_ms = {n: [] for n in names}
        for e in sev:
            for j, n in enumerate(names):
                stage_ms[n].append(e[j].elapsed_time(e[j + 1]))
        if whole_layer:
            gu_bytes = [layer_bytes[i % L] for i in range(KS)]
            gu_ms = stage_ms["layer"]
        elif single_path:
            # both expert GEMMs: their experts' codes + scales, x read, h written and read, d written
            gu_bytes = [n_active[i % L] * (gu_expert + dn_expert) + T * H * 2 + 2 * T * k * I * 2 + T * k * H * 4
                        for i in range(KS)]
            gu_ms = stage_ms["gate_up_down"]
        else:
            # gate_up per launch: its experts' codes + scales, x read once, h written
            gu_bytes = [n_active[i % L] * gu_expert + T * H * 2 + T * k * I * 2 for i in range(KS)]
            gu_ms = stage_ms["gate_up"]
        gu_achieved = float(np.sum(gu_bytes) / (np.sum(gu_ms) * 1e-3) / 1e9)
        res["stages_us"] = {n: round(float(np.mean(v)) * 1e3, 2) for n, v in stage_ms.items()}
        res["staged_us_per_layer"] = round(sev[0][0].elapsed_time(sev[-1][-1]) * 1e3 / KS, 2)
        kname = (("moe_fused_kernel" if args.persistent else "layer (all launches)") if whole_layer
                 else ("moe_experts_sorted_kernel" if single_path else
                       "moe_gate_up_sorted_kernel" if sorted_path else "moe_gate_up_kernel"))
        res["roofline"] = {
            "kernel": kname,
            "bound": "hbm", "achieved": round(gu_achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(gu_achieved / HBM_PEAK_GBPS, 4),
            "traffic": None if whole_layer else measured_traffic(cfg.name, kname),
            "avg_launch_us": round(float(np.mean(gu_ms)) * 1e3, 2), "launches": len(gu_ms),
            "timing": "HIP events on the launch stream, one pair per launch, right after the timed region",
            "bytes_per_launch": int(np.mean(gu_bytes)),
        }

    # ---------------------------------------------------------------- CPU oracle: baseline and parity
    # The oracle on the first --cpu-tokens tokens of the first --cpu-layers layers (the whole
    # layer at T <= 32): its time is the baseline, and its outputs are compared with the GPU's
    # output of the same layers under the MoE bound.
    if cpu_leg:
        import oracle
        threads = oracle.default_threads()
        n = max(1, min(args.cpu_tokens, T))
        nl = max(1, min(args.cpu_layers, L))
        toks = np.arange(n, dtype=np.int32)
        log(f"[bench] oracle on {n} of {T} tokens of {nl} layer(s), {threads} threads")
        secs, worst, mismatch = 0.0, 0.0, 0
        for lay in layers[:nl]:
            lay["y"].fill_(float("nan"))
            forward(lay)
            torch.cuda.synchronize()
            y_gpu = lay["y"].view(torch.int16).cpu().numpy().view(np.uint16)
            w_host = {key: lay["w"][key].cpu().numpy() for key in ("wgu", "sgu", "wd", "sd")}
            c0 = time.perf_counter()
            y_ora, scale, _ = oracle.moe_tokens(lay["x_bits"], lay["logits_host"], k, w_host["wgu"], w_host["sgu"],
                                                w_host["wd"], w_host["sd"], T, H, I, E, tokens=toks, nthreads=threads,
                                                n_shared=ns, act8=args.act8)
            secs += time.perf_counter() - c0
            wr, mm = moe_bound_ratio(y_gpu[:n], y_ora, scale)
            worst, mismatch = max(worst, wr), mismatch + mm
            del w_host
        res["cpu_baseline"] = {
            "value": round(secs / nl * (T / n) * 1e6, 1), "unit": "us/layer", "cores": threads, "kind": "oracle",
            "sample": f"layers 0..{nl - 1}, tokens 0..{n - 1} of {T} each (all {k} routed experts per token), full "
                      f"route+gate_up+down+combine; time per layer scaled by {T}/{n}; CPU: {cpu_model()}",
            "seconds": round(secs, 2),
        }
        res["parity"] = {"layers": nl, "tokens": n, "outputs": int(nl * n * H), "worst_ratio": round(worst, 4),
                         "nan_inf_mismatches": mismatch, "ok": bool(worst <= 1.0 and mismatch == 0),
                         "bound": "|gpu - oracle| <= 1e-2 * sum_j gate_j sum_i |h_i w_in| + 1 bf16 ulp, per output; "
                                  "worst_ratio = max |gpu - oracle| / bound over the sample"}
    del layers, ws, h
    torch.cuda.empty_cache()
    return res


# ------------------------------------------------------------------------------ dense workloads

def dense_case(cfg, args, torch, mx, dev, *, steps: int, warmup: int, cpu_leg: bool):
    """y[T,N] = bf16(x[T,K] @ W[N,K]^T) with MXFP4 W, one call per step."""
    import synthetic
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
    stream = torch.cuda.current_stream(dev)
    clocks_before = gpu_clocks()
    n_settle, first = settle(graph.replay, stream, torch, args.settle_ms, copies)
    for _ in range(max(0, -(-warmup // copies))):
        graph.replay()
    reps = max(2, -(-steps // copies))
    nsteps = reps * copies
    # HIP events on the replay stream bracket each replay of the graph: a call is shorter than
    # its host-side submission, so eager event pairs would time the host, not the kernel
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
    log(f"[bench] {cfg.name}: timed {nsteps} calls: {us_per_call:.2f} us/call")
    call_us = [evs[r].elapsed_time(evs[r + 1]) * 1e3 / copies for r in range(reps)]
    call_bytes = w_bytes + T * K * 2 + T * N * 2  # weights, x, y
    achieved = call_bytes / (float(np.mean(call_us)) * 1e-6) / 1e9
    eff_gbps = call_bytes / (us_per_call * 1e-6) / 1e9
    res = {
        "value": round(us_per_call, 3), "K": nsteps, "ms_per_step": round(us_per_call * 1e-3, 6),
        "effective_GBps": round(eff_gbps, 1), "pct_of_8TBps": round(100 * eff_gbps / HBM_PEAK_GBPS, 2),
        "algorithmic_bytes_per_call": call_bytes, "replay_us_per_call": stats_us(call_us),
        "settle": {"ms": args.settle_ms, "replays": n_settle, "first_replays_us_per_call": first},
        "clocks": {"before": clocks_before, "after": gpu_clocks()},
        "config": {"workload": cfg.name, "T": T, "K": K, "N": N, "weights": "MXFP4 (E2M1 codes, E8M0 scale per 32)",
                   "activations": "MXFP8, quantized in the kernel" if args.act8 else "bf16", "accumulate": "fp32",
                   "weight_copies_cycled": copies, "timing": "HIP graph replay"},
        "roofline": {"kernel": "mx_linear_kernel", "bound": "hbm", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": None, "avg_launch_us": round(float(np.mean(call_us)), 3), "launches": nsteps,
                     "timing": "HIP events on the replay stream around each graph replay of the timed region, "
                               "per call (includes the graph's gaps between kernels)",
                     "bytes_per_launch": call_bytes},
    }
    if cpu_leg:
        import oracle
        threads = oracle.default_threads()
        fn = oracle.mx_linear_a8 if args.act8 else oracle.mx_linear
        reps_cpu = 3
        c0 = time.perf_counter()
        for _ in range(reps_cpu):
            fn(x_bits, w, s, T, K, N, nthreads=threads)
        c1 = time.perf_counter()
        res["cpu_baseline"] = {"value": round((c1 - c0) / reps_cpu * 1e6, 1), "unit": "us/call", "cores": threads,
                               "kind": "oracle",
                               "sample": f"the whole call, {reps_cpu} repetitions averaged; CPU: {cpu_model()}",
                               "seconds": round(c1 - c0, 2)}
    del ws, ys, graph
    torch.cuda.empty_cache()
    return res


# ------------------------------------------------------------------------------ HBM yardsticks

def hbm_reference(args, torch, mx, dev, reps: int = 30):
    """This GPU's streaming-read and copy bandwidth with the library's reference kernels
    (mx_hbm_read, mx_hbm_copy) over --hbm-mib MiB, after their own settle; medians."""
    nbytes = args.hbm_mib << 20
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    src.fill_(0x5A)
    dst = torch.empty_like(src)
    xor = torch.zeros(4, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)
    out = {"bytes": nbytes}
    for name, fn, moved in (("read", lambda: mx.hbm_read(src, xor, clear=False), nbytes),
                            ("copy", lambda: mx.hbm_copy(dst, src), 2 * nbytes)):
        settle(fn, stream, torch, min(args.settle_ms, 200.0), 1, record=1)
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        evs[0].record(stream)
        for r in range(reps):
            fn()
            evs[r + 1].record(stream)
        torch.cuda.synchronize()
        us = [evs[r].elapsed_time(evs[r + 1]) * 1e3 for r in range(reps)]
        med = float(np.median(us))
        out[f"{name}_GBps"] = round(moved / (med * 1e-6) / 1e9, 1)
        out[f"{name}_us_median"] = round(med, 2)
    out["kernels"] = ("mx_hbm_read (16-byte nontemporal loads, XOR kept live), mx_hbm_copy (bytes read + written); "
                      "timed right after the headline workload")
    del src, dst
    torch.cuda.empty_cache()
    return out


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
    dense = args.workload in synthetic.LINEAR_CONFIGS
    if dense:
        head = dense_case(synthetic.LINEAR_CONFIGS[args.workload], args, torch, mx, dev, steps=args.steps,
                          warmup=args.warmup, cpu_leg=not args.no_cpu_baseline)
    else:
        if args.persistent:
            c = workload_config(args.workload)
            if c.T > 16 or c.T * c.k > 128 or c.n_shared or args.act8:
                raise SystemExit("--persistent takes T <= 16, T * top_k <= 128, no shared experts and bf16 "
                                 "activations")
        head = moe_case(workload_config(args.workload), args, torch, mx, dev, steps=args.steps, warmup=args.warmup,
                        stage_pass=True, cpu_leg=not args.no_cpu_baseline)

    hbm = hbm_reference(args, torch, mx, dev) if args.hbm_mib > 0 else None

    extras = {}
    if not args.no_extra and not args.persistent:
        for name in EXTRA_WORKLOADS:
            if name == args.workload:
                continue
            if name in synthetic.LINEAR_CONFIGS:
                r = dense_case(synthetic.LINEAR_CONFIGS[name], args, torch, mx, dev, steps=max(args.extra_steps, 1000),
                               warmup=args.warmup, cpu_leg=False)
                extras[name] = {"us_per_call": r["value"], "replay_us_per_call": r["replay_us_per_call"],
                                "effective_GBps": r["effective_GBps"], "pct_of_8TBps": r["pct_of_8TBps"],
                                "bytes": r["algorithmic_bytes_per_call"], "config": r["config"]}
            else:
                r = moe_case(workload_config(name), args, torch, mx, dev, steps=args.extra_steps, warmup=args.warmup,
                             stage_pass=False, cpu_leg=False)
                extras[name] = {"us_per_layer": r["value"], "replay_us_per_layer": r["replay_us_per_layer"],
                                "effective_GBps": r["effective_GBps"], "pct_of_8TBps": r["pct_of_8TBps"],
                                "active_experts": r["active_experts"], "bytes": r["algorithmic_bytes_per_layer"],
                                "config": r["config"]}

    unit = "us/call" if dense else "us/layer"
    out = {
        "metric": DENSE_METRIC if dense else METRIC,
        "value": head["value"],
        "unit": unit,
        "n_gpus": 1,
        "steps": head["K"],
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8 (E4M3) x fp4 (E2M1), fp32 accumulate" if args.act8 else "bf16",
        "data": "synthetic",
        "config": head["config"],
        "effective_GBps": head["effective_GBps"],
        "pct_of_8TBps": head["pct_of_8TBps"],
    }
    if hbm:
        out["pct_of_copy"] = round(100 * head["effective_GBps"] / hbm["copy_GBps"], 2)
        out["pct_of_read"] = round(100 * head["effective_GBps"] / hbm["read_GBps"], 2)
        out["copy_GBps"] = hbm["copy_GBps"]
    for key in ("active_experts", "algorithmic_bytes_per_layer", "algorithmic_bytes_per_call", "stages_us",
                "staged_us_per_layer", "replay_us_per_layer", "replay_us_per_call", "settle", "clocks"):
        if key in head:
            out[key] = head[key]
    out["roofline"] = head["roofline"]
    out["cpu_baseline"] = head.get("cpu_baseline")
    if "parity" in head:
        out["parity"] = head["parity"]
    out["hbm_reference"] = hbm
    if not dense:
        out["mfma_t128"] = measured_mfma()
    out["configs"] = extras
    out["env"] = {"GPU_MAX_HW_QUEUES": os.environ.get("GPU_MAX_HW_QUEUES"), "torch": torch.__version__,
                  "hip": getattr(torch.version, "hip", None), "device": torch.cuda.get_device_name(dev)}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
