"""Benchmark of the low-bit sparse-MoE hot path on one MI355X.

Headline (the line's value): the 48-layer MoE stack (d 2560, 512 experts of
intermediate 640 per layer, top-10 plus a shared expert of 640, 2-bit blocks),
eight tokens per pass (one real token plus seven drafts, as in a verify
pass), RMSNorm between layers.  One step = one pass of the whole stack over
one batch of 8 synthetic tokens, replayed from a HIP graph; all weights
(about 38 GB) are resident in HBM before timing starts.  Consecutive steps
take the next of 16 input batches (so the routing changes from pass to
pass), each step bracketed by its own events; the same is also reported with
the Infinity Cache emptied before every pass, and for the same input
replayed back to back.

The default run also measures, under "configs", the other configurations of
the workload set, each with its own roofline and oracle baseline: the same
2-bit stack at 16 tokens per pass (one pass of 16 hi + lo token rows per
layer), one full-size layer at T = 1 (Infinity Cache emptied before each
forward), the 48-layer 3-bit stack at T = 8 and T = 1, one layer over an
8192-token prefill chunk, and the codebook-block layer and stack.
--workload picks a single one.

Prints one JSON line: tokens/s, plus achieved HBM bandwidth from the
algorithmic bytes of the actual routing, the roofline of the dominant kernel
(durations measured with HIP events on the launch stream) and the CPU oracle
timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def host_cpu():
    """The host CPU the oracle baseline runs on: model name and the number of
    logical CPUs this process may use (the oracle itself uses one thread)."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 0
    return {"host_cpu": model, "host_nproc": n, "threads_used": 1}


def algorithmic_bytes_decode(wl, idx_layers: np.ndarray, T: int):
    """Bytes the method must move per pass, from the routing actually taken:
    router weights and bias, every distinct routed expert once plus the
    shared expert, activations in and out.  Returns (total, per-layer gate/up
    bytes, per-layer down bytes)."""
    eb = wl.expert_bytes()
    gu_per_expert = 2 * wl.I * (wl.d // 32) * wl.block_bytes()
    dn_per_expert = wl.d * (wl.I // 32) * wl.block_bytes()
    sh_gu = 2 * wl.Is * (wl.d // 32) * wl.block_bytes() if wl.Is else 0
    sh_dn = wl.d * (wl.Is // 32) * wl.block_bytes() if wl.Is else 0
    total = 0
    gu, dn = [], []
    for l in range(idx_layers.shape[0]):
        U = len(np.unique(idx_layers[l]))
        gu.append(U * gu_per_expert + sh_gu)
        dn.append(U * dn_per_expert + sh_dn)
        total += wl.E * wl.d * 4 + wl.E * 4 + U * eb + (wl.expert_bytes(wl.Is) if wl.Is else 0) + 2 * T * wl.d * 4
    return total, np.array(gu, dtype=np.float64), np.array(dn, dtype=np.float64)


def measured_traffic(workload: str, kernel: str):
    """HBM bytes per launch of the dominant kernel as the byte counters read
    them (profiles/traffic.json: FETCH_SIZE and WRITE_SIZE per dispatch,
    scaled by the copy calibration), or None when no counters were taken for
    this workload or the kernel's sources changed since."""
    import hashlib

    here = os.path.dirname(os.path.abspath(__file__))
    try:
        with open(os.path.join(here, "profiles", "traffic.json")) as f:
            tab = json.load(f)
    except (OSError, ValueError):
        return None
    ent = tab.get(workload)
    if not ent or ent.get("kernel") != kernel:
        return None
    h = hashlib.sha256()
    for src in ent["sources"]:
        with open(os.path.join(here, src), "rb") as f:
            h.update(f.read())
    if h.hexdigest() != ent.get("sources_sha256"):
        return None
    return 1024.0 * (ent["fetch_kib"] * tab["fetch_scale"] + ent["write_kib"] * tab["write_scale"])


def time_classes(bqe, run_pass, classes, reps, max_launches, before=None):
    """Average duration (seconds per launch) of each kernel class the pass
    launches, from the events its launches record themselves (launches
    serialized); classes the pass does not launch are left out."""
    kdur = {}
    for cls, name in classes:
        tot, n = 0.0, 0
        for i in range(reps):
            if before is not None:
                before(i)
            bqe.moe_timing_start(cls, max_launches)
            run_pass(i)
            ms, cnt = bqe.moe_timing_stop()
            tot += ms
            n += cnt
        if n:
            kdur[name] = (tot / n) * 1e-3
    return kdur


def decode_classes(bqe):
    # the persistent decode pass (one launch per pass) where it applies, else
    # the three kernels per layer
    return ((bqe.TIMING_PERSIST, "decode_pass"), (bqe.TIMING_GATE_UP, "gate_up"), (bqe.TIMING_DOWN, "down"),
            (bqe.TIMING_ROUTER, "router"))


def data_note(wl):
    blocks = ("counter-hash codebook blocks (uniform indices, signs; fp16 scales) over a seeded 512x4 grid of odd "
              "magnitudes" if wl.codebook else "counter-hash codes/scales")
    return f"synthetic ({blocks}, N(0,1) activations, N(0,0.02) router + Zipf(1.1) log bias)"


def cpu_baseline_stack(wl, T, x_np, n_layers_sample):
    """Time the oracle (single-threaded fp64 C) on the first layers of the
    stack; expert generation is excluded from the timed parts."""
    import moe_inputs as mi
    import oracle

    h = x_np
    t_total = 0.0
    for l in range(n_layers_sample):
        W, b = mi.router(wl, l)
        t0 = time.perf_counter()
        if l > 0:
            h = oracle.rmsnorm(h, 1e-6)
        logits = oracle.router_logits(h, W, b)
        idx, w = oracle.topk(logits, wl.k)
        t_total += time.perf_counter() - t0
        ex = {int(e): mi.expert_canon(wl, l, int(e)).numpy() for e in np.unique(idx)}
        sh = mi.expert_canon(wl, l, -1).numpy() if wl.Is else None
        grid = mi.codebook_grid(wl.seed) if wl.codebook else None
        OL = oracle.Layer(wl.d, wl.E, wl.I, wl.Is, wl.k, wl.bits, W, b, ex, sh, grid=grid)
        t0 = time.perf_counter()
        h, _, _, _ = oracle.layer_forward(OL, h, force_idx=idx, force_w=w)
        t_total += time.perf_counter() - t0
    per_layer = t_total / n_layers_sample
    return T / (per_layer * wl.layers), per_layer


def cpu_baseline_prefill(wl, x_np, n_tok):
    """Time the oracle (single-threaded fp64 C) on the first n_tok tokens of
    the prefill chunk: router, top-k and the layer; expert generation untimed."""
    import moe_inputs as mi
    import oracle

    W, b = mi.router(wl, 0)
    h = x_np[:n_tok]
    t0 = time.perf_counter()
    logits = oracle.router_logits(h, W, b)
    idx, w = oracle.topk(logits, wl.k)
    t_total = time.perf_counter() - t0
    ex = {int(e): mi.expert_canon(wl, 0, int(e)).numpy() for e in np.unique(idx)}
    sh = mi.expert_canon(wl, 0, -1).numpy() if wl.Is else None
    OL = oracle.Layer(wl.d, wl.E, wl.I, wl.Is, wl.k, wl.bits, W, b, ex, sh)
    t0 = time.perf_counter()
    oracle.layer_forward(OL, h, force_idx=idx, force_w=w)
    t_total += time.perf_counter() - t0
    return n_tok / t_total, t_total


def bench_prefill(args):
    """One MoE layer over a prompt chunk of T tokens (default 8192)."""
    import torch

    import bit_quantized_experts_amd as bqe
    import moe_inputs as mi
    from moe_inputs.device import activations_device, packed_layer

    wl = mi.WORKLOADS["prefill"]
    T = args.T or wl.T
    dev = "cuda"
    torch.cuda.set_device(0)
    L = packed_layer(wl, 0, dev)
    x_np = mi.activations(wl, T=T, stream=1)
    x = activations_device(x_np, dev)
    y = torch.empty((T, wl.d), dtype=torch.float32, device=dev)
    ws = bqe.new_workspace(L.workspace_bytes(T), dev)
    idx = torch.empty((T, wl.k), dtype=torch.int32, device=dev)
    w = torch.empty((T, wl.k), dtype=torch.float32, device=dev)
    rio = bqe.RouteIO(None, None, None, idx.data_ptr(), w.data_ptr())

    if args.f16act and T > bqe.MAX_TOK_F16ACT:
        raise SystemExit(f"--f16act takes at most {bqe.MAX_TOK_F16ACT} tokens")
    fwd = bqe.moe_layer_forward_f16act if args.f16act else bqe.moe_layer_forward

    def run_pass():
        fwd(L.handle, x, y, ws, rio)

    if args.timing_only:
        bqe.moe_timing_start(bqe.TIMING_PREFILL_ROUTER, 1)
    run_pass()
    if args.timing_only:
        bqe.moe_timing_stop()
    torch.cuda.synchronize()
    idx_np = idx.cpu().numpy()
    kdur = {}
    # a layer of at most 8 tokens runs the decode kernels: time those
    classes = ((bqe.TIMING_GATE_UP, "gate_up"), (bqe.TIMING_DOWN, "down"), (bqe.TIMING_ROUTER, "router")) \
        if T <= bqe.MAX_TOK_DECODE_KERNELS or args.f16act else \
        ((bqe.TIMING_PREFILL_GATE_UP, "gate_up"), (bqe.TIMING_PREFILL_DOWN, "down"), (bqe.TIMING_PREFILL_ROUTER, "router"))
    for cls, name in classes:
        tot, n = 0.0, 0
        for _ in range(5):
            bqe.moe_timing_start(cls, 1)
            run_pass()
            ms, cnt = bqe.moe_timing_stop()
            tot += ms
            n += cnt
        kdur[name] = (tot / n) * 1e-3

    if args.timing_only:
        return {"timing_only": wl.name, "kernels_avg_us": {n: kdur[n] * 1e6 for n in kdur}}

    graph = None
    if not args.no_graph:
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for _ in range(2):
                run_pass()
        torch.cuda.current_stream().wait_stream(s)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            run_pass()
        torch.cuda.synchronize()
    step = graph.replay if graph is not None else run_pass
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # each timed step after a 512 MB write (the Infinity Cache then holds
    # none of the layer's weights), bracketed by its own events
    flush = torch.empty(512 * 1024 * 1024 // 4, dtype=torch.float32, device=dev)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for i in range(args.steps):
        flush.fill_(float(i))
        ev[i][0].record()
        step()
        ev[i][1].record()
    torch.cuda.synchronize()
    times = np.array([a.elapsed_time(b) * 1e-3 for a, b in ev])
    sec_per_step = float(times.mean())
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    sec_b2b = e0.elapsed_time(e1) * 1e-3 / args.steps

    # algorithmic matrix-core work from the routing taken: 2 flops per
    # multiply-add, gate+up (2 d I) and down (d I) per routed pair, the
    # shared expert once per token; the router GEMM is counted apart
    pairs = int((idx_np >= 0).sum())
    gu_flops = 2.0 * pairs * 2 * wl.d * wl.I + 2.0 * T * 2 * wl.d * wl.Is
    dn_flops = 2.0 * pairs * wl.d * wl.I + 2.0 * T * wl.d * wl.Is
    rt_flops = 2.0 * T * wl.E * wl.d
    flops = {"gate_up": gu_flops, "down": dn_flops, "router": rt_flops}
    kernels = {n: {"avg_us": kdur[n] * 1e6, "flops_per_launch": flops[n],
                   "TFLOPs": flops[n] / kdur[n] / 1e12} for n in kdur}
    dom = max(("gate_up", "down"), key=lambda n: kdur[n])
    achieved = flops[dom] / kdur[dom] / 1e12
    gemm_util = (gu_flops + dn_flops) / (kdur["gate_up"] + kdur["down"]) / 1e12 / MFMA_F16_PEAK_TFLOPS
    counts = np.bincount(idx_np.reshape(-1), minlength=wl.E)
    # algorithmic bytes of the routing taken (each touched expert once); a
    # short chunk's grouped GEMMs do too few flops per byte to be bound by the
    # matrix cores (below 2.5 PFLOP/s / 8 TB/s = 312 flop/B): its roofline is
    # then HBM, the dominant kernel's weight bytes over its duration
    total_bytes, gu_b, dn_b = algorithmic_bytes_decode(wl, idx_np[None], T)
    wbytes = {"gate_up": float(gu_b[0]), "down": float(dn_b[0])}
    for n in ("gate_up", "down"):
        kernels[n]["bytes_per_launch"] = wbytes[n]
        kernels[n]["GBps"] = wbytes[n] / kdur[n] / 1e9
    hbm_bound = flops[dom] / wbytes[dom] < MFMA_F16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    if hbm_bound:
        ach = wbytes[dom] / kdur[dom] / 1e9
        roofline = {"bound": "hbm", "kernel": dom, "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": ach / HBM_PEAK_GBS, "traffic": None}
    else:
        roofline = {"bound": "mfma", "kernel": dom, "achieved": achieved, "peak": MFMA_F16_PEAK_TFLOPS,
                    "unit": "TFLOP/s", "frac": achieved / MFMA_F16_PEAK_TFLOPS,
                    "traffic": measured_traffic(wl.name, dom) if T == wl.T else None}

    cpu = None
    if args.cpu_tokens > 0:
        log(f"timing the CPU oracle on {args.cpu_tokens} tokens ...")
        tps, tsec = cpu_baseline_prefill(wl, x_np, args.cpu_tokens)
        cpu = {"value": tps, "unit": "tokens/s", "cores": 1, "kind": "oracle", **host_cpu(),
               "sample": f"first {args.cpu_tokens} of {T} tokens of the chunk ({tsec:.1f} s: router, top-k, "
                         f"layer), single thread; expert generation untimed"}
    out = {
        "metric": "MoE prefill tokens/s (one layer, chunk of T tokens)",
        "value": T / sec_per_step,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": sec_per_step * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16 MFMA operands (weights s*c, activations scaled per row), fp32 accumulate",
        "data": data_note(wl),
        "config": {"workload": wl.name, "layers": 1, "T": T, "f16act": bool(args.f16act), "d": wl.d, "experts": wl.E,
                   "d_ff": wl.I,
                   "shared_d_ff": wl.Is, "top_k": wl.k, "bits": wl.bits, "graph": graph is not None,
                   "parallelism": "none (1 GPU)"},
        "step_ms": {"p10": float(np.percentile(times, 10)) * 1e3, "median": float(np.median(times)) * 1e3,
                    "p90": float(np.percentile(times, 90)) * 1e3,
                    "note": "512 MB written before each step (Infinity Cache emptied)"},
        "back_to_back": {"ms_per_step": sec_b2b * 1e3, "value": T / sec_b2b},
        "grouped_gemm_mfma_util": gemm_util,
        "hbm_GBps": total_bytes / sec_per_step / 1e9,
        "bytes_per_step": float(total_bytes),
        "tokens_per_expert": {"max": int(counts.max()), "empty_experts": int((counts == 0).sum())},
        "roofline": roofline,
        "kernels": kernels,
        "cpu_baseline": cpu,
    }
    return out


def bench_stack_prefill(args):
    """Chunked prefill through the 48-layer 2-bit stack (RMSNorm between
    layers): one step = one chunk of T tokens (default 8192) through every
    layer, replayed from a HIP graph, each step after a 512 MB write and
    bracketed by its own events."""
    import torch

    import bit_quantized_experts_amd as bqe
    import moe_inputs as mi
    from moe_inputs.device import activations_device, packed_layer

    wl = mi.WORKLOADS["stack_prefill"]
    if args.layers:
        wl = mi.small(wl, layers=args.layers)
    T = args.T or wl.T
    dev = "cuda"
    torch.cuda.set_device(0)
    layers = [packed_layer(wl, l, dev) for l in range(wl.layers)]
    handles = [L.handle for L in layers]
    x = activations_device(mi.activations(wl, T=T, stream=1), dev)
    y = torch.empty((T, wl.d), dtype=torch.float32, device=dev)
    ws = bqe.new_workspace(max(L.workspace_bytes(T) for L in layers), dev)
    idx_l = torch.empty((wl.layers, T, wl.k), dtype=torch.int32, device=dev)
    w_l = torch.empty((wl.layers, T, wl.k), dtype=torch.float32, device=dev)

    def run_pass(record_routing=False):
        if record_routing:
            bqe.moe_stack_forward(handles, x, y, ws, 1e-6, None, idx_l, w_l)
        else:
            bqe.moe_stack_forward(handles, x, y, ws, 1e-6)

    run_pass(True)
    torch.cuda.synchronize()
    idx_np = idx_l.cpu().numpy()
    kdur = {}
    for cls, name in ((bqe.TIMING_PREFILL_GATE_UP, "gate_up"), (bqe.TIMING_PREFILL_DOWN, "down"),
                      (bqe.TIMING_PREFILL_ROUTER, "router")):
        bqe.moe_timing_start(cls, wl.layers)
        run_pass()
        ms, cnt = bqe.moe_timing_stop()
        kdur[name] = (ms / cnt) * 1e-3

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run_pass()
    torch.cuda.current_stream().wait_stream(s)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run_pass()
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        graph.replay()
    flush = torch.empty(512 * 1024 * 1024 // 4, dtype=torch.float32, device=dev)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for i in range(args.steps):
        flush.fill_(float(i))
        ev[i][0].record()
        graph.replay()
        ev[i][1].record()
    torch.cuda.synchronize()
    times = np.array([a.elapsed_time(b) * 1e-3 for a, b in ev])
    sec_per_step = float(times.mean())

    # algorithmic matrix-core work from the routing of every layer (as for
    # one layer: gate+up 2 d I and down d I multiply-adds per routed pair,
    # the shared expert once per token)
    pairs = (idx_np >= 0).sum(axis=(1, 2)).astype(np.float64)
    gu_flops = 2.0 * pairs * 2 * wl.d * wl.I + 2.0 * T * 2 * wl.d * wl.Is
    dn_flops = 2.0 * pairs * wl.d * wl.I + 2.0 * T * wl.d * wl.Is
    flops = {"gate_up": float(gu_flops.mean()), "down": float(dn_flops.mean()), "router": 2.0 * T * wl.E * wl.d}
    kernels = {n: {"avg_us": kdur[n] * 1e6, "flops_per_launch": flops[n],
                   "TFLOPs": flops[n] / kdur[n] / 1e12} for n in kdur}
    dom = max(("gate_up", "down"), key=lambda n: kdur[n])
    achieved = flops[dom] / kdur[dom] / 1e12
    total_flops = float(gu_flops.sum() + dn_flops.sum())
    cpu = None
    if args.cpu_tokens > 0 and args.cpu_layers > 0:
        n_tok, n_l = min(args.cpu_tokens, 16), min(args.cpu_layers, 2, wl.layers)  # (a few seconds)
        log(f"timing the CPU oracle on {n_tok} tokens through {n_l} layers ...")
        tps, per_layer = cpu_baseline_stack(wl, n_tok, mi.activations(wl, T=T, stream=1)[:n_tok], n_l)
        cpu = {"value": tps, "unit": "tokens/s", "cores": 1, "kind": "oracle", **host_cpu(),
               "sample": f"first {n_tok} of {T} tokens through the first {n_l} of {wl.layers} layers "
                         f"({per_layer:.2f} s/layer), scaled to the full stack; single thread; expert generation untimed"}
    out = {
        "metric": "MoE-stack prefill tokens/s (48 layers, chunk of T tokens)",
        "value": T / sec_per_step,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": sec_per_step * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16 MFMA operands (weights s*c, activations scaled per row), fp32 accumulate",
        "data": data_note(wl),
        "config": {"workload": wl.name, "layers": wl.layers, "T": T, "d": wl.d, "experts": wl.E, "d_ff": wl.I,
                   "shared_d_ff": wl.Is, "top_k": wl.k, "bits": wl.bits, "graph": True,
                   "parallelism": "none (1 GPU)"},
        "step_ms": {"p10": float(np.percentile(times, 10)) * 1e3, "median": float(np.median(times)) * 1e3,
                    "p90": float(np.percentile(times, 90)) * 1e3,
                    "note": "512 MB written before each step (Infinity Cache emptied)"},
        "expert_gemm_TFLOPs_per_step": total_flops / sec_per_step / 1e12,
        "distinct_experts_per_layer": [int(len(np.unique(idx_np[l]))) for l in range(wl.layers)],
        "max_tokens_per_expert_per_layer": [int(np.bincount(idx_np[l].reshape(-1), minlength=wl.E).max())
                                            for l in range(wl.layers)],
        "roofline": {"bound": "mfma", "kernel": dom, "achieved": achieved, "peak": MFMA_F16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / MFMA_F16_PEAK_TFLOPS, "traffic": None},
        "kernels": kernels,
        "cpu_baseline": cpu,
    }
    return out


def bench_layer_t1(args, name="layer_t1"):
    """One full-size layer, decode T = 1, over a ring of 16 input rows (the
    routing changes from row to row).  Before each timed forward a 512 MB
    buffer is written, so the layer's weights are not served from the 256 MB
    Infinity Cache; each forward is bracketed by events on the stream."""
    import torch

    import bit_quantized_experts_amd as bqe
    import moe_inputs as mi
    from moe_inputs.device import activations_device, packed_layer

    wl = mi.WORKLOADS[name]
    dev = "cuda"
    torch.cuda.set_device(0)
    L = packed_layer(wl, 0, dev)
    ring = 16
    xs = [activations_device(mi.activations(wl, T=1, stream=500 + i), dev) for i in range(ring)]
    y = torch.empty((1, wl.d), dtype=torch.float32, device=dev)
    ws = bqe.new_workspace(L.workspace_bytes(1), dev)
    idx = torch.empty((1, wl.k), dtype=torch.int32, device=dev)
    w = torch.empty((1, wl.k), dtype=torch.float32, device=dev)
    rio = bqe.RouteIO(None, None, None, idx.data_ptr(), w.data_ptr())
    flush = torch.empty(512 * 1024 * 1024 // 4, dtype=torch.float32, device=dev)
    for i in range(ring):
        bqe.moe_layer_forward(L.handle, xs[i], y, ws, rio)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(ring)]
    times = []
    n_rep = max(1, args.steps // ring)
    for rep in range(args.warmup // ring + n_rep):
        for i in range(ring):
            flush.fill_(float(i))
            ev[i][0].record()
            bqe.moe_layer_forward(L.handle, xs[i], y, ws, rio)
            ev[i][1].record()
        torch.cuda.synchronize()
        if rep >= args.warmup // ring:
            times += [a.elapsed_time(b) * 1e-3 for a, b in ev]
    sec = float(np.mean(times))
    # algorithmic bytes: router + bias, the 10 routed experts and the shared
    # expert, x and y
    nbytes = wl.E * wl.d * 4 + wl.E * 4 + wl.k * wl.expert_bytes() + wl.expert_bytes(wl.Is) + 2 * wl.d * 4
    kdur = time_classes(bqe, lambda i: bqe.moe_layer_forward(L.handle, xs[i], y, ws, rio), decode_classes(bqe),
                        ring, 1, before=lambda i: flush.fill_(float(i)))
    gu_bytes = (wl.k + 1) * 2 * wl.I * (wl.d // 32) * wl.block_bytes()
    dn_bytes = (wl.k + 1) * wl.d * (wl.I // 32) * wl.block_bytes()
    per = {"gate_up": gu_bytes, "down": dn_bytes, "router": wl.E * wl.d * 4 + wl.E * 4, "decode_pass": nbytes}
    kernels = {n: {"avg_us": kdur[n] * 1e6, "bytes_per_launch": per[n], "GBps": per[n] / kdur[n] / 1e9} for n in kdur}
    dom = max(kdur, key=lambda n: kdur[n])
    achieved = per[dom] / kdur[dom] / 1e9
    cpu = None
    if args.cpu_layers > 0:
        rows = np.concatenate([mi.activations(wl, T=1, stream=500 + i) for i in range(ring)], axis=0)
        tps, per_layer = cpu_baseline_stack(wl, ring, rows, 1)
        cpu = {"value": tps, "unit": "tokens/s", "cores": 1, "kind": "oracle", **host_cpu(),
               "sample": f"the layer on the {ring} rows of the ring ({per_layer:.2f} s), single thread; "
                         f"expert generation untimed"}
    out = {
        "metric": "MoE layer forwards/s (decode T=1, one full-size layer)",
        "value": 1.0 / sec,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": len(times),
        "warmup": args.warmup,
        "ms_per_step": sec * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16 MFMA operands (codes exact, activations as fp16 hi+lo), fp32 accumulate",
        "data": data_note(wl),
        "config": {"workload": wl.name, "layers": 1, "T": 1, "d": wl.d, "experts": wl.E, "d_ff": wl.I,
                   "shared_d_ff": wl.Is, "top_k": wl.k, "bits": wl.bits, "ring": ring,
                   "infinity_cache": "flushed before each forward", "parallelism": "none (1 GPU)"},
        "hbm_GBps": nbytes / sec / 1e9,
        "bytes_per_step": nbytes,
        "p10_p90_us": [float(np.percentile(times, 10) * 1e6), float(np.percentile(times, 90) * 1e6)],
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None},
        "kernels": kernels,
        "cpu_baseline": cpu,
    }
    return out


def copy_calibration(n_mib: int, reps: int):
    """A plain device-to-device copy of n_mib MiB, reps times: the reference
    for scaling the FETCH_SIZE / WRITE_SIZE counters to bytes (the copy reads
    and writes exactly n_mib MiB per launch)."""
    import torch

    torch.cuda.set_device(0)
    n = n_mib * 1024 * 1024 // 4
    src = torch.arange(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    assert bool((dst[-4:] == src[-4:]).all())
    print(json.dumps({"copy_calibration": {"bytes_read": n * 4, "bytes_written": n * 4, "launches": reps}}))


def build_stack(wl):
    """Generate and pack every layer of a stack on the GPU (untimed)."""
    import torch

    from moe_inputs.device import packed_layer

    t0 = time.time()
    layers = [packed_layer(wl, l, "cuda") for l in range(wl.layers)]
    torch.cuda.synchronize()
    log(f"built {wl.layers} packed layers of {wl.name} in {time.time() - t0:.1f}s "
        f"({sum(L.buffer.numel() for L in layers) / 1e9:.2f} GB resident)")
    return layers


def bench_stack(args, wl, T, layers):
    """The stack over T tokens per pass: one step = one pass of every layer
    over one batch of T synthetic tokens, replayed from a HIP graph."""
    import torch

    import bit_quantized_experts_amd as bqe
    import moe_inputs as mi
    from moe_inputs.device import activations_device

    dev = "cuda"

    # a ring of input batches: consecutive passes route differently, as in
    # decoding, instead of re-reading the same experts every pass
    RING = 16
    ring_np = [mi.activations(wl, T=T, stream=1 + i) for i in range(RING)]
    ring = [activations_device(r, dev) for r in ring_np]
    x_np = ring_np[0]
    x = torch.empty_like(ring[0])
    x.copy_(ring[0])
    y = torch.empty((T, wl.d), dtype=torch.float32, device=dev)
    ws = bqe.new_workspace(max(L.workspace_bytes(T) for L in layers), dev)
    handles = [L.handle for L in layers]
    idx_l = torch.empty((wl.layers, T, wl.k), dtype=torch.int32, device=dev)
    w_l = torch.empty((wl.layers, T, wl.k), dtype=torch.float32, device=dev)

    fwd = bqe.moe_stack_forward_f16act if args.f16act else bqe.moe_stack_forward

    def run_pass(record_routing=False):
        if record_routing:
            fwd(handles, x, y, ws, 1e-6, None, idx_l, w_l)
        else:
            fwd(handles, x, y, ws, 1e-6)

    # eager warm-up (also initialises the library before any capture); with
    # --timing-only it runs with the launches serialized like the timed passes
    if args.timing_only:
        bqe.moe_timing_start(bqe.TIMING_ROUTER, 1)
    run_pass(True)
    if args.timing_only:
        bqe.moe_timing_stop()
    torch.cuda.synchronize()
    idx_np = idx_l.cpu().numpy()

    # per-kernel durations, measured with HIP events bracketing each launch on
    # the launch stream (eager passes, one kernel class at a time)
    kdur = time_classes(bqe, lambda i: run_pass(), decode_classes(bqe), 3, wl.layers)

    if args.timing_only:
        return {"timing_only": wl.name, "T": T, "kernels_avg_us": {n: kdur[n] * 1e6 for n in kdur}}

    graph = None
    if not args.no_graph:
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for _ in range(2):
                run_pass()
        torch.cuda.current_stream().wait_stream(s)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            run_pass()
        torch.cuda.synchronize()

    step = graph.replay if graph is not None else run_pass
    flush = torch.empty(512 * 1024 * 1024 // 4, dtype=torch.float32, device=dev)

    def timed_ring(n, with_flush):
        """n passes over the ring, each bracketed by its own events (the
        input copy, and the 512 MB write that empties the Infinity Cache,
        stay outside); seconds per pass."""
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for i in range(n):
            if with_flush:
                flush.fill_(float(i))
            x.copy_(ring[i % RING])
            ev[i][0].record()
            step()
            ev[i][1].record()
        torch.cuda.synchronize()
        return np.array([a.elapsed_time(b) * 1e-3 for a, b in ev])

    timed_ring(args.warmup, False)
    times = timed_ring(args.steps, False)
    sec_per_step = float(times.mean())
    times_fl = timed_ring(max(10, args.steps // 2), True)
    # the same input every pass, back to back (the experts of the previous pass
    # partly still in the Infinity Cache)
    x.copy_(ring[0])
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    sec_same = e0.elapsed_time(e1) * 1e-3 / args.steps

    # the graph replays the eager pass's routing (same input), and the
    # algorithmic bytes of every ring input from its own routing
    run_pass(True)
    torch.cuda.synchronize()
    assert np.array_equal(idx_l.cpu().numpy(), idx_np), "routing changed between passes"
    ring_bytes = []
    distinct = []
    for i in range(RING):
        x.copy_(ring[i])
        run_pass(True)
        torch.cuda.synchronize()
        ir = idx_l.cpu().numpy()
        ring_bytes.append(algorithmic_bytes_decode(wl, ir, T)[0])
        distinct += [int(len(np.unique(ir[l]))) for l in range(wl.layers)]
    total_bytes = float(np.mean(ring_bytes))
    _, gu_bytes, dn_bytes = algorithmic_bytes_decode(wl, idx_np, T)
    gbs = total_bytes / sec_per_step / 1e9

    # roofline of the dominant kernel (largest share of the pass)
    # (the persistent pass moves the whole pass's bytes in one launch of up
    # to 64 layers)
    per_class_bytes = {"gate_up": gu_bytes.mean(), "down": dn_bytes.mean(),
                       "router": float(wl.E * wl.d * 4 + wl.E * 4),
                       "decode_pass": algorithmic_bytes_decode(wl, idx_np, T)[0] / ((wl.layers + 63) // 64)}
    dom = max(kdur, key=lambda n: kdur[n])
    achieved = per_class_bytes[dom] / kdur[dom] / 1e9
    kernels = {n: {"avg_us": kdur[n] * 1e6, "bytes_per_launch": per_class_bytes[n],
                   "GBps": per_class_bytes[n] / kdur[n] / 1e9} for n in kdur}

    cpu = None
    if args.cpu_layers > 0:
        log(f"timing the CPU oracle on {args.cpu_layers} layers ...")
        tps, per_layer = cpu_baseline_stack(wl, T, x_np, args.cpu_layers)
        cpu = {"value": tps, "unit": "tokens/s", "cores": 1, "kind": "oracle", **host_cpu(),
               "sample": f"first {args.cpu_layers} of {wl.layers} layers at T={T}, "
                         f"{per_layer:.2f} s/layer, scaled to the full stack; expert generation untimed"}

    out = {
        "metric": "MoE-stack tokens/s (decode verify pass)",
        "value": T / sec_per_step,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": sec_per_step * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("fp16 MFMA operands (codes exact, activations rounded to fp16), fp32 accumulate" if args.f16act
                  else "fp16 MFMA operands (codes exact, activations as fp16 hi+lo), fp32 accumulate"),
        "data": data_note(wl),
        "config": {"workload": wl.name, "layers": wl.layers, "T": T, "f16act": bool(args.f16act), "d": wl.d, "experts": wl.E, "d_ff": wl.I,
                   "shared_d_ff": wl.Is, "top_k": wl.k, "bits": wl.bits, "graph": graph is not None,
                   "inputs": f"ring of {RING} batches of {T} rows", "parallelism": "none (1 GPU)"},
        "step_ms": {"p10": float(np.percentile(times, 10)) * 1e3, "median": float(np.median(times)) * 1e3,
                    "p90": float(np.percentile(times, 90)) * 1e3},
        "flushed": {"note": "512 MB written before each pass (Infinity Cache emptied)",
                    "ms_per_step": float(times_fl.mean()) * 1e3, "value": T / float(times_fl.mean()),
                    "p10_ms": float(np.percentile(times_fl, 10)) * 1e3,
                    "p90_ms": float(np.percentile(times_fl, 90)) * 1e3},
        "same_input_back_to_back": {"ms_per_step": sec_same * 1e3, "value": T / sec_same},
        "hbm_GBps": gbs,
        "bytes_per_step": total_bytes,
        "distinct_experts_per_layer": {"min": min(distinct), "mean": float(np.mean(distinct)), "max": max(distinct)},
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": measured_traffic(wl.name, dom) if (T == wl.T and not args.layers) else None},
        "kernels": kernels,
        "cpu_baseline": cpu,
    }
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="all",
                    choices=["all", "stack_t8_2bit", "stack_3bit", "prefill", "layer_t1", "stack_prefill",
                             "layer_t1_cb3", "stack_cb3"],
                    help="all (default): the 2-bit stack at T = 8 as the value, with the one-layer T = 1 "
                         "decode, the 3-bit stack at T = 8 and T = 1, the 8192-token prefill and the "
                         "codebook-block layer and stack under configs")
    ap.add_argument("--T", type=int, default=None, help="tokens per pass (default: the workload's)")
    ap.add_argument("--layers", type=int, default=None, help="override the number of layers (testing only)")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--f16act", action="store_true",
                    help="stacks: the fp16-activation decode entry point (up to 16 tokens per pass)")
    ap.add_argument("--cpu-layers", type=int, default=12,
                    help="oracle sample size in layers (0 = skip; about 10 s of CPU time at T = 8)")
    ap.add_argument("--cpu-tokens", type=int, default=96,
                    help="prefill: oracle sample size in tokens (0 = skip; about 10 s of CPU time)")
    ap.add_argument("--timing-only", action="store_true",
                    help="only the per-kernel timing passes (every launch serialized), for profiler runs")
    ap.add_argument("--copy-calib", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (counter calibration) and exit")
    args = ap.parse_args()

    if args.copy_calib:
        copy_calibration(args.copy_calib, 5)
        return

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for {args.gpus}); this build has no multi-GPU path. "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    if args.workload == "prefill":
        print(json.dumps(bench_prefill(args)))
        return
    if args.workload in ("layer_t1", "layer_t1_cb3"):
        print(json.dumps(bench_layer_t1(args, args.workload)))
        return
    if args.workload == "stack_prefill":
        print(json.dumps(bench_stack_prefill(args)))
        return

    import torch

    import moe_inputs as mi

    torch.cuda.set_device(0)
    if args.workload != "all":
        wl = mi.WORKLOADS[args.workload]
        if args.layers:
            wl = mi.small(wl, layers=args.layers)
        print(json.dumps(bench_stack(args, wl, args.T or wl.T, build_stack(wl))))
        return

    # Default: the headline configuration (the 48-layer 2-bit stack at T = 8)
    # is the line's value; the other configurations of the workload set are
    # measured in the same run and reported under "configs", each with its
    # own roofline and oracle baseline.
    wl = mi.WORKLOADS["stack_t8_2bit"]
    layers = build_stack(wl)
    out = bench_stack(args, wl, wl.T, layers)
    if args.timing_only:
        print(json.dumps(out))
        return
    configs = {}
    # the same stack at 16 tokens per pass: one decode pass of 16 hi + lo
    # token rows per layer (the oracle sample halved: each layer costs twice
    # the CPU time)
    log("stack_t8_2bit T=16 ...")
    args16 = argparse.Namespace(**vars(args))
    args16.cpu_layers = max(1, args.cpu_layers // 2) if args.cpu_layers > 0 else 0
    configs["stack_t8_2bit_T16"] = bench_stack(args16, wl, 16, layers)
    del layers
    torch.cuda.empty_cache()
    log("layer_t1 ...")
    configs["layer_t1"] = bench_layer_t1(args)
    torch.cuda.empty_cache()
    wl3 = mi.WORKLOADS["stack_3bit"]
    layers = build_stack(wl3)
    for T in (wl3.T,) + tuple(wl3.extra_T):
        log(f"stack_3bit T={T} ...")
        configs[f"stack_3bit_T{T}"] = bench_stack(args, wl3, T, layers)
    del layers
    torch.cuda.empty_cache()
    log("prefill ...")
    configs["prefill_T8192"] = bench_prefill(args)
    torch.cuda.empty_cache()
    # short chunks (several conversations decoded together, or a short
    # prompt): the same layer over 32 and 256 tokens
    for Ts in (32, 256):
        log(f"prefill T={Ts} ...")
        a_s = argparse.Namespace(**vars(args))
        a_s.T = Ts
        a_s.cpu_tokens = min(args.cpu_tokens, 16)
        configs[f"prefill_T{Ts}"] = bench_prefill(a_s)
        torch.cuda.empty_cache()
    log("layer_t1_cb3 ...")
    configs["layer_t1_cb3"] = bench_layer_t1(args, "layer_t1_cb3")
    torch.cuda.empty_cache()
    wlc = mi.WORKLOADS["stack_cb3"]
    layers = build_stack(wlc)
    log(f"stack_cb3 T={wlc.T} ...")
    configs[f"stack_cb3_T{wlc.T}"] = bench_stack(args, wlc, wlc.T, layers)
    del layers
    out["configs"] = configs
    print(json.dumps(out))


if __name__ == "__main__":
    main()
