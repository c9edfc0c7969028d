"""Benchmark of the MoE-LoRA hot path on one MI355X.

A step is one pass of the whole path over one batch -- the align outputs and
the fused result -- on seeded synthetic inputs already resident in HBM: one
fused_moe_lora_with_align launch where the batch allows it (at most 64 pairs
and 64 slots; the decode shapes), else moe_lora_align then fused_moe_lora
(``--path`` chooses; the two-launch step is reported beside the one-launch
one).  The
default workload is the gpt-oss-20b-like decode w13 shape (M=16, K=2880,
N=2x2880, E=32, topk=4, L=6 slots all active, r=64, BLOCK_M=16).

Timing:
  * value / ms_per_step: K steps captured in one HIP graph and replayed,
    bracketed by synchronize on both sides.  Every input buffer is rotated
    over enough copies that the touched bytes exceed 4x the 256 MB
    Infinity Cache, so weights are read from HBM (``--warm`` disables this).
  * roofline: the fused kernel's own duration from HIP events on the replay
    stream around replays of one graph of K launches of that kernel alone
    (the eager figure beside it: K back-to-back launches queued behind a
    short GPU sleep), against the algorithmic bytes
    it must move (weights of the active (slice, slot, expert) groups once,
    the X rows it reads, the Y rows it reads and writes, routed weights and
    block metadata).
  * cpu_baseline: the CPU oracle (plain C, fp64) on the same inputs.
  * two_kernel: fused_moe_lora_two_kernel (shrink and expand with the rank
    vectors through memory) on the same inputs, graph-timed with the align
    step and event-timed for its two kernels; one_shot_speedup is the latter
    over the fused kernel's time.
  * layer_chain (decode workloads with a w2 partner): one MoE layer, w13 ->
    activation -> w2, the LoRA side of each projection (align, fused with
    add_inputs = 0 into a zero buffer, moe_lora_accumulate to join) on an
    auxiliary stream with four events beside stand-in base GEMMs that stream
    the base expert weights a decode step reads (and the base MoE align);
    each side alone, serial and overlapped.  dual_stream: the same for one
    projection, for the other decode workloads.
  * align_stress: the align step alone at M = 65536, topk = 8, E = 256, L = 16.
  * prefill: the Qwen3-MoE-like prefill (C4) -- fused kernel time, HBM
    roofline, MFMA rate, and rocprofv3's MFMA counters when recorded for the
    current sources -- so one default run covers both halves of the metric.
  * value's spread: p10 / p50 / p90 over 9 replays of the same graph.
  * align_free (batches of at most 1024 pairs): fused_moe_lora_naive on the
    same inputs -- the decode path with no align launch -- at the workload's
    block_m and at block_m = 1.  ``--path naive`` times it as the step instead.

Prints ONE JSON line on stdout; progress goes to stderr.
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

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = ("fused MoE-LoRA µs/call + achieved HBM TB/s (decode) / MFMA % (prefill)")
HBM_PEAK_GBPS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
# attainable dense bf16 MFMA rates measured on MI355X with loops of eight
# independent products per wavefront on every SIMD: v_mfma_f32_32x32x16_bf16
# reaches 2310 TFLOP/s, v_mfma_f32_16x16x32_bf16 (the instruction the fused
# kernels use) 1260 TFLOP/s
BF16_MEASURED_TFLOPS_32X32X16 = 2310.0
BF16_MEASURED_TFLOPS_16X16X32 = 1260.0
MALL_BYTES = 256 * 2 ** 20
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
COUNTERS_FILE = os.path.join(ROOT, "profiles", "counters.json")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# The sources each fused kernel is built from: its own file, the file that
# sizes and issues its launch, the host entry points, and every header these
# include (followed through the headers' own includes).  Counters recorded for
# a kernel stay valid while these are unchanged.
KERNEL_SOURCES = {
    "fused_stream_kernel": ["fused_stream.hip", "fused_valu.hip"],
    "fused_valu_kernel": ["fused_valu.hip"],
    "fused_mfma_kernel": ["fused_mfma.hip"],
}
SHARED_SOURCES = ["api.hip"]
_INCLUDE = re.compile(r'^\s*#\s*include\s+"([^"]+)"', re.M)


def kernel_source_files(kernel: str) -> list:
    """KERNEL_SOURCES[kernel] + SHARED_SOURCES and their included files,
    as paths relative to the package's csrc directory."""
    csrc = os.path.join(ROOT, "moe_lora_adapter_amd", "csrc")
    todo = list(KERNEL_SOURCES[kernel] + SHARED_SOURCES)
    seen = set()
    while todo:
        f = os.path.normpath(todo.pop())
        if f in seen:
            continue
        seen.add(f)
        with open(os.path.join(csrc, f)) as fh:
            text = fh.read()
        base = os.path.dirname(f)
        todo += [os.path.join(base, inc) for inc in _INCLUDE.findall(text)]
    return sorted(seen)


def kernel_sources_sha(kernel: str) -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "moe_lora_adapter_amd", "csrc")
    for f in kernel_source_files(kernel):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


# ----------------------------------------------------------------- algorithmic work
def algorithmic_work(case):
    """Bytes and flops the fused step must move / compute (see module doc)."""
    s = case.shape
    slot = np.repeat(case.token_lora_mapping, s.topk).astype(np.int64)
    ex = case.topk_ids.reshape(-1).astype(np.int64)
    valid = (slot >= 0) & (slot < s.L) & (ex >= 0) & (ex < s.E)
    P = int(valid.sum())
    keys = np.unique(slot[valid] * s.E + ex[valid])
    groups = len(keys) * s.S
    idx = np.nonzero(valid)[0]
    xrows = len(np.unique(idx if s.x_per_pair else idx // s.topk))
    cnt = np.bincount(slot[valid] * s.E + ex[valid], minlength=s.L * s.E)
    padded = int((-(-cnt // s.block_m) * s.block_m).sum())
    w_bytes = groups * (s.r * s.K + s.Ns * s.r) * 2
    x_bytes = xrows * s.K * 2
    y_bytes = P * s.S * s.Ns * 2 * (2 if s.add else 1)
    meta = padded * 4 + (padded // s.block_m) * 4 + (P * 4 if s.mul else 0)
    fused_bytes = w_bytes + x_bytes + y_bytes + meta
    flops = 2.0 * P * s.S * s.r * (s.K + s.Ns)
    align_bytes = s.numel * 4 + s.M * 4 + padded * 4 + (padded // s.block_m) * 4 + 2 * s.L * 4
    # the align-free path reads the routing (topk_ids, mapping) instead of the
    # align outputs
    naive_bytes = w_bytes + x_bytes + y_bytes + s.numel * 4 + s.M * 4 + (P * 4 if s.mul else 0)
    # fused_moe_lora_with_align: the align-free read plus the align outputs written
    with_align_bytes = naive_bytes + align_bytes - (s.numel * 4 + s.M * 4)
    return dict(valid_pairs=P, active_groups=len(keys), fused_bytes=int(fused_bytes),
                weight_bytes=int(w_bytes), x_bytes=int(x_bytes), y_bytes=int(y_bytes),
                meta_bytes=int(meta), fused_flops=flops, align_bytes=int(align_bytes),
                naive_bytes=int(naive_bytes), with_align_bytes=int(with_align_bytes))


# ----------------------------------------------------------------- device inputs
class DeviceSet:
    """One copy of every buffer a step reads or writes."""

    def __init__(self, case, dev, proto=None):
        import torch
        import moe_lora_adapter_amd as mla
        s = case.shape
        if proto is None:
            t16 = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)  # noqa: E731
            self.topk_ids = torch.from_numpy(case.topk_ids).to(dev)
            self.mapping = torch.from_numpy(case.token_lora_mapping).to(dev)
            self.w = torch.from_numpy(case.topk_weights).to(dev)
            self.x, self.a, self.b, self.y = t16(case.x), t16(case.lora_a), t16(case.lora_b), t16(case.y_in)
        else:
            for k in ("topk_ids", "mapping", "w", "x", "a", "b", "y"):
                setattr(self, k, getattr(proto, k).clone())
        self.align = mla.alloc_align_output(s.M, s.topk, s.E, s.L, s.block_m, dev)
        ws = mla.align_workspace_size(s.M, s.topk, s.E, s.L, s.block_m)
        self.ws = torch.empty(max(ws, 16), dtype=torch.uint8, device=dev)
        self.ws2 = None  # two-kernel workspace, allocated when that path is timed


def run_align(ds, s):
    import moe_lora_adapter_amd as mla
    mla.moe_lora_align(ds.topk_ids, ds.mapping, s.E, s.L, s.block_m, out=ds.align, workspace=ds.ws)


def run_fused(ds, s, variant):
    import moe_lora_adapter_amd as mla
    mla.fused_moe_lora(ds.x, ds.a, ds.b, ds.align, ds.w, ds.y, mul_routed_weight=s.mul,
                       add_inputs=s.add, x_per_pair=s.x_per_pair, variant=variant)


def run_fused_ws(ds, s, variant, workspace):
    """fused_moe_lora_ws: the decode stream kernel with its K split."""
    import moe_lora_adapter_amd as mla
    mla.fused_moe_lora_ws(ds.x, ds.a, ds.b, ds.align, ds.w, ds.y, mul_routed_weight=s.mul,
                          add_inputs=s.add, workspace=workspace, x_per_pair=s.x_per_pair,
                          variant=variant)


def run_naive(ds, s, block_m, variant):
    import moe_lora_adapter_amd as mla
    mla.fused_moe_lora_naive(ds.x, ds.a, ds.b, ds.topk_ids, ds.mapping, ds.w, ds.y,
                             mul_routed_weight=s.mul, add_inputs=s.add, block_m=block_m,
                             x_per_pair=s.x_per_pair, variant=variant)


def resolve_path(requested, s):
    """The step --path names; "auto": one launch (fused_moe_lora_with_align)
    where the batch allows it, else align + fused."""
    if requested != "auto":
        return requested
    wa_ok = s.numel <= 64 and s.L <= 64  # MOE_LORA_WITH_ALIGN_MAX_PAIRS / _SLOTS
    return "with_align" if wa_ok else "sorted"


def run_with_align(ds, s, variant):
    """fused_moe_lora_with_align: the align outputs and the fused result in one launch."""
    import moe_lora_adapter_amd as mla
    mla.fused_moe_lora_with_align(ds.topk_ids, ds.mapping, ds.x, ds.a, ds.b, ds.w, ds.y, E=s.E,
                                  L=s.L, block_m=s.block_m, mul_routed_weight=s.mul,
                                  add_inputs=s.add, out=ds.align, x_per_pair=s.x_per_pair,
                                  variant=variant)


def naive_kernel_name(s, block_m, variant):
    """The kernel of the align-free path: the sorted path's choice for
    block_m >= 16, the vector kernels below that."""
    return _kernel_name(s, variant if block_m >= 16 else "valu")


def run_two_kernel(ds, s):
    import moe_lora_adapter_amd as mla
    mla.fused_moe_lora_two_kernel(ds.x, ds.a, ds.b, ds.align, ds.w, ds.y, mul_routed_weight=s.mul,
                                  add_inputs=s.add, x_per_pair=s.x_per_pair, workspace=ds.ws2)


def step(ds, s, variant):
    run_align(ds, s)
    run_fused(ds, s, variant)


# ----------------------------------------------------------------- measurements
def time_steps_graph(sets, s, variant, steps, fn=None, replays=None, n_replays=9):
    """Capture `steps` steps (rotating over the copies) in one graph; replay.
    `fn(ds)` replaces the align + fused step when given.  Returns the seconds
    per step of the first timed replay; with a list in `replays`, the graph is
    replayed `n_replays` times in all and every replay's seconds per step are
    appended to it (the first included)."""
    import torch
    fn = fn or (lambda ds: step(ds, s, variant))
    g = torch.cuda.CUDAGraph()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        fn(sets[0])  # stream warm-up outside the capture
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for i in range(steps):
            fn(sets[i % len(sets)])
    torch.cuda.synchronize()
    g.replay()  # untimed replay: first-launch costs of the graph
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    g.replay()
    torch.cuda.synchronize()
    first = (time.perf_counter() - t0) / steps
    if replays is not None:
        # more replays of the same graph, each bracketed the same way
        replays.append(first)
        for _ in range(n_replays - 1):
            t0 = time.perf_counter()
            g.replay()
            torch.cuda.synchronize()
            replays.append((time.perf_counter() - t0) / steps)
    return first


def time_kernel_events(sets, s, variant, which, launches):
    """Average duration of one kernel: `launches` back-to-back launches of it
    between one pair of HIP events on its stream, queued behind a short GPU
    sleep so the launches run back to back.  The align outputs of every copy
    are already in place from earlier steps, so fused launches need no align
    in between."""
    import torch
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(int(2.4e9 * 0.05))   # ~50 ms: lets the launches queue up
    e0.record()
    for i in range(launches):
        ds = sets[i % len(sets)]
        if callable(which):
            which(ds)
        elif which == "fused":
            run_fused(ds, s, variant)
        else:
            run_align(ds, s)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / launches


def time_kernel_graph(sets, s, variant, which, launches, windows=5):
    """Per-window average duration of one kernel launched as a graph replay
    runs it: `launches` launches of it (rotating over the copies) captured in
    one HIP graph, each of `windows` replays bracketed by a pair of HIP events
    on the stream the replay runs on.  Returns the list of window averages
    in us.  (Eager launches carry their kernel arguments in host memory,
    which a kernel's first read then waits for; graph-launched kernels do
    not.)"""
    import torch
    fn = which if callable(which) else (
        (lambda ds: run_fused(ds, s, variant)) if which == "fused" else (lambda ds: run_align(ds, s)))
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn(sets[0])
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for i in range(launches):
            fn(sets[i % len(sets)])
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    out = []
    for _ in range(windows):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        out.append(e0.elapsed_time(e1) * 1e3 / launches)
    del g
    return out


def time_kernel_windows(sets, s, variant, which, launches, windows=5, out=None):
    """A kernel's duration over several windows of graph-replayed launches
    (time_kernel_graph): (mean, p10, p90) of the per-window averages, in us;
    with a dict in `out`, also their p50 and the same statistics of eager
    launches (time_kernel_events) there."""
    w = time_kernel_graph(sets, s, variant, which, launches, windows)
    if out is not None:
        out["p50"] = float(np.percentile(w, 50))
        ew = [time_kernel_events(sets, s, variant, which, launches) for _ in range(windows)]
        out["eager_avg"] = float(np.mean(ew))
        out["eager_p50"] = float(np.percentile(ew, 50))
    return float(np.mean(w)), float(np.percentile(w, 10)), float(np.percentile(w, 90))


def spread(us_list):
    a = np.asarray(us_list, dtype=np.float64)
    return {"n": int(a.size), "p10": round(float(np.percentile(a, 10)), 3),
            "p50": round(float(np.percentile(a, 50)), 3),
            "p90": round(float(np.percentile(a, 90)), 3)}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or platform.machine()


def load_counters(kernel, workload):
    """MFMA counters of a kernel and workload (profiles/counters.json), or None
    when the kernel's sources changed since they were taken."""
    try:
        with open(COUNTERS_FILE) as f:
            rec = json.load(f).get(f"{kernel}/{workload}")
    except (OSError, ValueError):
        return None
    if not rec or rec.get("src_sha") != kernel_sources_sha(kernel):
        return None
    return rec


def prefill_line(args, dev, variant):
    """The prefill half of the metric: the Qwen3-MoE-like prefill (M = 8192,
    topk = 8, E = 128, L = 8 with 3 active, r = 128, K = 2048, N = 2 x 768,
    BLOCK_M = 64), cold inputs, the fused kernel event-timed, its HBM
    roofline and its MFMA rate (algorithmic and, when recorded for these
    sources, rocprofv3's MfmaUtil / MfmaFlopsBF16)."""
    import torch
    from moe_lora_adapter_amd import synth
    s = synth.shape("qwen3_prefill")
    log(f"prefill line: drawing {s.name}")
    case = synth.draw(s)
    work = algorithmic_work(case)
    touched = work["fused_bytes"] + work["align_bytes"]
    copies = 1 if args.warm else max(1, min(8, math.ceil(args.cold_bytes / touched)))
    sets = [DeviceSet(case, dev)]
    for _ in range(copies - 1):
        sets.append(DeviceSet(case, dev, proto=sets[0]))
    steps = max(10, args.steps)
    for i in range(max(args.warmup, 3)):
        step(sets[i % copies], s, variant)
    torch.cuda.synchronize()
    reps = []
    time_steps_graph(sets, s, variant, steps, replays=reps, n_replays=5)
    med = {}
    kus, k10, k90 = time_kernel_windows(sets, s, variant, "fused", steps, out=med)
    kname = _kernel_name(s, variant)
    gbps = work["fused_bytes"] / (kus * 1e-6) / 1e9
    tflops = work["fused_flops"] / (kus * 1e-6) / 1e12
    traffic, _ = load_traffic(kname, s.name)
    ctr = load_counters(kname, s.name)
    res = {"workload": s.name, "steps": steps, "step": "moe_lora_align + fused_moe_lora",
           "us_per_call": round(float(np.median(reps)) * 1e6, 3),
           "us_per_call_replays": spread([r * 1e6 for r in reps]),
           "cache": f"cold: {copies} rotated input copies" if not args.warm else "warm",
           "roofline": {"bound": "hbm", "kernel": kname, "achieved": round(gbps, 1),
                        "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                        "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": traffic,
                        "algorithmic_bytes_per_launch": work["fused_bytes"],
                        "kernel_us_avg": round(kus, 3), "kernel_us_p10": round(k10, 3),
                        "kernel_us_p50": round(med["p50"], 3), "kernel_us_p90": round(k90, 3),
                        "kernel_us_eager_avg": round(med["eager_avg"], 3)},
           "mfma": {"algorithmic_tflops": round(tflops, 2), "peak_tflops": BF16_PEAK_TFLOPS,
                    "frac": round(tflops / BF16_PEAK_TFLOPS, 4),
                    "measured_peak_tflops": {"32x32x16": BF16_MEASURED_TFLOPS_32X32X16,
                                             "16x16x32": BF16_MEASURED_TFLOPS_16X16X32},
                    "frac_of_measured_16x16x32": round(tflops / BF16_MEASURED_TFLOPS_16X16X32, 4),
                    "counters": None if ctr is None else
                    {k: ctr[k] for k in ("mfma_util_pct", "mfma_flops_bf16_per_dispatch",
                                         "mfma_issued_tflops", "kernel_trace_avg_us")
                     if k in ctr}},
           "work": {k: work[k] for k in ("valid_pairs", "active_groups", "fused_bytes",
                                         "fused_flops")}}
    del sets
    torch.cuda.empty_cache()
    return res


def align_stress_line(args, dev, workload="align_stress"):
    """The align step alone on its stress case (M = 65536, topk = 8, E = 256,
    L = 16, BLOCK_M = 64; or another align-only workload): graph-timed calls
    and event-timed windows."""
    import torch
    import moe_lora_adapter_amd as mla
    from moe_lora_adapter_amd import synth
    s = synth.shape(workload)
    case = synth.draw(s, with_tensors=False)
    work = algorithmic_work(case)
    steps = max(10, min(args.steps, 200))

    class _Set:
        pass
    sets = []
    for _ in range(4):   # a few copies of the routing, rotated
        d = _Set()
        d.topk_ids = torch.from_numpy(case.topk_ids).to(dev)
        d.mapping = torch.from_numpy(case.token_lora_mapping).to(dev)
        d.align = mla.alloc_align_output(s.M, s.topk, s.E, s.L, s.block_m, dev)
        d.ws = torch.empty(max(16, mla.align_workspace_size(s.M, s.topk, s.E, s.L, s.block_m)),
                           dtype=torch.uint8, device=dev)
        sets.append(d)
    fn = lambda ds: run_align(ds, s)  # noqa: E731
    for i in range(5):
        fn(sets[i % 4])
    torch.cuda.synchronize()
    reps = []
    time_steps_graph(sets, s, None, steps, fn=fn, replays=reps, n_replays=5)
    kus, k10, k90 = time_kernel_windows(sets, s, None, "align", steps)
    gbps = work["align_bytes"] / (kus * 1e-6) / 1e9
    return {"workload": s.name, "M": s.M, "topk": s.topk, "E": s.E, "L": s.L,
            "block_m": s.block_m, "steps": steps,
            "us_per_call": round(float(np.median(reps)) * 1e6, 3),
            "us_per_call_replays": spread([r * 1e6 for r in reps]),
            "kernels_us_avg": round(kus, 3), "kernels_us_p10": round(k10, 3),
            "kernels_us_p90": round(k90, 3),
            "algorithmic_bytes": work["align_bytes"], "achieved_GBps": round(gbps, 1)}


def layer_chain_line(sets, s, case, steps, dev, copies):
    """One MoE layer, w13 -> activation -> w2, with the LoRA side of each
    projection on an auxiliary stream (moe_lora_adapter_amd.streams: four
    events) beside stand-in base GEMMs that stream the base weights of the
    experts the batch routes to (one bf16 GEMM per projection over
    [K, N x distinct experts]; the w13 side also runs the base MoE align, one
    slot, beside the LoRA align).  Graph-timed per layer: base alone, LoRA
    alone, both serial on one stream, and dual-stream."""
    import torch
    import moe_lora_adapter_amd as mla
    from moe_lora_adapter_amd import synth
    from moe_lora_adapter_amd.streams import LoraStreams, W13, W2
    c13, c2 = synth.draw_layer(s.name)
    if not (np.array_equal(c13.topk_ids, case.topk_ids)
            and np.array_equal(c13.token_lora_mapping, case.token_lora_mapping)):
        raise RuntimeError("layer draw does not reproduce the workload's routing")
    s2 = c2.shape
    t16 = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)  # noqa: E731
    for k, d in enumerate(sets):     # the w2 adapters, one copy per rotated set
        d.a2 = t16(c2.lora_a) if k == 0 else sets[0].a2.clone()
        d.b2 = t16(c2.lora_b) if k == 0 else sets[0].b2.clone()
    w2 = torch.from_numpy(c2.topk_weights).to(dev)
    ex = case.topk_ids.reshape(-1)
    n_exp = max(1, len(np.unique(ex[(ex >= 0) & (ex < s.E)])))
    w13cat = torch.empty((s.K, s.N * n_exp), dtype=torch.bfloat16, device=dev).normal_(0, s.K ** -0.5)
    w2cat = torch.empty((s2.K, s2.N * n_exp), dtype=torch.bfloat16, device=dev).normal_(0, s2.K ** -0.5)
    base1 = torch.empty((s.M, s.N * n_exp), dtype=torch.bfloat16, device=dev)
    base2 = torch.empty((s.numel, s2.N * n_exp), dtype=torch.bfloat16, device=dev)
    zero_map = torch.zeros(s.M, dtype=torch.int32, device=dev)
    base_al = mla.alloc_align_output(s.M, s.topk, s.E, 1, s.block_m, dev)
    base_ws = torch.empty(max(16, mla.align_workspace_size(s.M, s.topk, s.E, 1, s.block_m)),
                          dtype=torch.uint8, device=dev)
    d1 = torch.zeros_like(sets[0].y)
    h = torch.empty((s.numel, s2.K), dtype=torch.bfloat16, device=dev)
    y2 = torch.zeros((s.M, s.topk, s2.N), dtype=torch.bfloat16, device=dev)
    d2 = torch.zeros_like(y2)
    st = LoraStreams()

    def base13(d):
        mla.moe_lora_align(d.topk_ids, zero_map, s.E, 1, s.block_m, out=base_al,
                           workspace=base_ws)
        torch.matmul(d.x, w13cat, out=base1)

    def lora13(d):
        d1.zero_()
        run_align(d, s)
        mla.fused_moe_lora(d.x, d.a, d.b, d.align, d.w, d1, mul_routed_weight=s.mul,
                           add_inputs=False)

    def act(d):   # a stand-in SwiGLU over the gate and up slices
        y = d.y.view(s.numel, s.N)
        torch.mul(torch.nn.functional.silu(y[:, :s.Ns]), y[:, s.Ns:], out=h)

    def base2_fn(d):
        torch.matmul(h, w2cat, out=base2)

    def lora2(d):
        d2.zero_()
        mla.fused_moe_lora(h, d.a2, d.b2, d.align, w2, d2, mul_routed_weight=s2.mul,
                           add_inputs=False, x_per_pair=True)

    def serial(d):
        base13(d)
        lora13(d)
        mla.moe_lora_accumulate(d.y, d1)
        act(d)
        base2_fn(d)
        lora2(d)
        mla.moe_lora_accumulate(y2, d2)

    def dual(d):
        st.fork_join(W13, lambda: base13(d), lambda: lora13(d), d.y, d1)
        act(d)
        st.fork_join(W2, lambda: base2_fn(d), lambda: lora2(d), y2, d2)

    def base_only(d):
        base13(d)
        act(d)
        base2_fn(d)

    def lora_only(d):
        lora13(d)
        mla.moe_lora_accumulate(d.y, d1)
        act(d)
        lora2(d)
        mla.moe_lora_accumulate(y2, d2)

    def timed(fn):
        return time_steps_graph(sets, s, None, steps, fn=fn) * 1e6

    def timed_eager(fn):
        for i in range(len(sets)):
            fn(sets[i])
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            fn(sets[i % len(sets)])
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / steps * 1e6

    log("layer chain line")
    res = {"w2_workload": s2.name,
           "base_stand_in": (f"w13: bf16 GEMM [{s.M} x {s.K}] x [{s.K} x {s.N * n_exp}], "
                             f"w2: [{s.numel} x {s2.K}] x [{s2.K} x {s2.N * n_exp}] "
                             f"({n_exp} distinct experts' base weights, "
                             f"{(w13cat.numel() + w2cat.numel()) * 2 / 1e9:.2f} GB), "
                             "plus the base MoE align"),
           "events": 4,
           "base_us": round(timed(base_only), 3),
           "lora_us": round(timed(lora_only), 3),
           "serial_us": round(timed(serial), 3),
           "dual_stream_us": round(timed(dual), 3),
           "eager_serial_us": round(timed_eager(serial), 3),
           "eager_dual_stream_us": round(timed_eager(dual), 3),
           "timing": "graph: one HIP graph of K layers; eager: K layers launched from the "
                     "host, synchronize on both sides"}
    res["overlap_saving_us"] = round(res["serial_us"] - res["dual_stream_us"], 3)
    res["eager_overlap_saving_us"] = round(res["eager_serial_us"] - res["eager_dual_stream_us"], 3)
    for d in sets:
        del d.a2, d.b2
    del w13cat, w2cat, base1, base2
    torch.cuda.empty_cache()
    return res


def dual_stream_line(sets, s, case, steps, dev):
    """The dual-stream path against a stand-in base GEMM (graph-timed per step).

    The base MoE w13 GEMM of a decode batch streams the base weights of every
    expert the batch routes to; the stand-in is one bf16 GEMM of the batch's X
    rows with a [K, N x distinct experts] matrix, the same bytes.  The LoRA side
    is align + fused_moe_lora (add_inputs = 0 into a zero-filled buffer); the
    join is moe_lora_accumulate.  Reported: each alone, both serial on one
    stream, and the LoRA side on an auxiliary stream beside the base."""
    import torch
    import moe_lora_adapter_amd as mla
    slot = np.repeat(case.token_lora_mapping, s.topk)
    ex = case.topk_ids.reshape(-1)
    valid = (slot >= 0) & (slot < s.L) & (ex >= 0) & (ex < s.E)
    n_exp = max(1, len(np.unique(ex[valid])))
    x_rows = sets[0].x.shape[0]
    w = torch.empty((s.K, s.N * n_exp), dtype=torch.bfloat16, device=dev).normal_()
    xb = sets[0].x[: max(1, x_rows)].contiguous()
    base_out = torch.empty((xb.shape[0], s.N * n_exp), dtype=torch.bfloat16, device=dev)
    deltas = [torch.zeros_like(ds.y) for ds in sets]
    aux = torch.cuda.Stream()
    evs = [torch.cuda.Event() for _ in range(steps)]

    def base(i):
        torch.matmul(xb, w, out=base_out)

    def lora(i, stream=None):
        ds, d = sets[i % len(sets)], deltas[i % len(sets)]
        d.zero_()
        mla.moe_lora_align(ds.topk_ids, ds.mapping, s.E, s.L, s.block_m, out=ds.align,
                           workspace=ds.ws)
        mla.fused_moe_lora(ds.x, ds.a, ds.b, ds.align, ds.w, d, mul_routed_weight=s.mul,
                           add_inputs=False, x_per_pair=s.x_per_pair)

    def join(i):
        ds, d = sets[i % len(sets)], deltas[i % len(sets)]
        mla.moe_lora_accumulate(ds.y, d)

    def serial(i):
        base(i)
        lora(i)
        join(i)

    def dual(i):
        main = torch.cuda.current_stream()
        aux.wait_stream(main)
        with torch.cuda.stream(aux):
            lora(i)
            evs[i].record(aux)
        base(i)
        main.wait_event(evs[i])
        join(i)

    def timed(fn):
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn(0)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            for i in range(steps):
                fn(i)
        g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        g.replay()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / steps * 1e6

    log("dual-stream line")
    res = {"base_stand_in": f"bf16 GEMM [{xb.shape[0]} x {s.K}] x [{s.K} x {s.N * n_exp}] "
                            f"({n_exp} distinct experts' base weights, "
                            f"{w.numel() * 2 / 1e9:.2f} GB)",
           "base_us": round(timed(base), 3),
           "lora_us": round(timed(lambda i: (lora(i), join(i))), 3),
           "serial_us": round(timed(serial), 3),
           "dual_stream_us": round(timed(dual), 3)}
    res["overlap_saving_us"] = round(res["serial_us"] - res["dual_stream_us"], 3)
    del w, base_out
    return res


def cpu_baseline(case, budget_s):
    import oracle
    o = oracle.load()
    s = case.shape
    slot = np.repeat(case.token_lora_mapping, s.topk)
    ex = case.topk_ids.reshape(-1)
    valid = np.nonzero((slot >= 0) & (slot < s.L) & (ex >= 0) & (ex < s.E))[0]
    t0 = time.perf_counter()
    o.align(case.topk_ids, case.token_lora_mapping, s.E, s.L, s.block_m)
    t_align = time.perf_counter() - t0
    # time one pair first, then size a sample to the budget
    probe = valid[:1]
    t0 = time.perf_counter()
    o.fused(case.x, case.lora_a, case.lora_b, case.topk_ids, case.token_lora_mapping,
            case.topk_weights, case.y_in, s.mul, s.add, x_per_pair=s.x_per_pair, pairs=probe)
    per_pair = max(time.perf_counter() - t0, 1e-6)
    threads = o.num_threads()
    n_full = len(valid)
    reps, n_sample = 1, n_full
    est_full = per_pair * n_full / max(1, min(threads, n_full))
    if est_full > budget_s:
        n_sample = max(threads, int(n_full * budget_s / est_full))
    else:
        reps = max(1, int(budget_s / max(est_full, 1e-3)))
    sample = valid[np.linspace(0, n_full - 1, n_sample).astype(np.int64)] if n_sample < n_full else None
    times = []
    for _ in range(reps):
        t0 = time.perf_counter()
        o.fused(case.x, case.lora_a, case.lora_b, case.topk_ids, case.token_lora_mapping,
                case.topk_weights, case.y_in, s.mul, s.add, x_per_pair=s.x_per_pair, pairs=sample)
        times.append(time.perf_counter() - t0)
    t_fused = float(np.median(times)) * (n_full / n_sample)
    if sample is None:
        desc = f"whole step (align + fused over all {n_full} valid pairs), median of {reps} runs"
    else:
        desc = (f"align over all pairs + fused over {n_sample} of {n_full} valid pairs "
                f"(evenly spaced), scaled to all pairs")
    return {"value": round((t_align + t_fused) * 1e6, 1), "unit": "us/call", "cores": threads,
            "cpu_model": cpu_model(), "kind": "oracle", "sample": desc,
            "align_us": round(t_align * 1e6, 1), "fused_us": round(t_fused * 1e6, 1)}


def copy_calibration(dev, mib=256, reps=5):
    """Plain device copies of known size, for scaling rocprofv3 byte counters."""
    import torch
    a = torch.empty(mib * 2 ** 20 // 4, dtype=torch.float32, device=dev).fill_(1.0)
    b = torch.empty_like(a)
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    log(f"copy calibration: {reps} copies of {mib} MiB")


def load_traffic(kernel, workload):
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f).get(f"{kernel}/{workload}")
    except (OSError, ValueError):
        return None, None
    if not rec or rec.get("src_sha") != kernel_sources_sha(kernel):
        return None, rec
    return rec.get("traffic_bytes_per_launch"), rec


# ----------------------------------------------------------------- main
def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="oss20b_decode_w13_a6")
    ap.add_argument("--variant", default="auto", choices=["auto", "valu", "mfma"])
    ap.add_argument("--warm", action="store_true", help="no cache-defeating rotation")
    ap.add_argument("--cold-bytes", type=float, default=4 * MALL_BYTES)
    ap.add_argument("--cpu-budget", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run plain 256 MiB device copies (rocprofv3 counter scaling)")
    ap.add_argument("--path", default="auto", choices=["auto", "with_align", "sorted", "naive"],
                    help="the step: with_align = fused_moe_lora_with_align (align outputs "
                         "and fused result in one launch), sorted = moe_lora_align + "
                         "fused_moe_lora, naive = fused_moe_lora_naive (no align outputs); "
                         "auto = with_align where it applies (<= 64 pairs and slots), else "
                         "sorted")
    ap.add_argument("--naive-block-m", type=int, default=None,
                    help="block_m of the align-free path (default: the workload's)")
    ap.add_argument("--no-two-kernel", action="store_true",
                    help="skip the two-kernel comparator line")
    ap.add_argument("--no-dual-stream", action="store_true",
                    help="skip the dual-stream overlap line")
    ap.add_argument("--k-split", action="store_true",
                    help="time align + fused_moe_lora_ws (K split) as the step")
    ap.add_argument("--no-k-split-line", action="store_true",
                    help="skip the line that times the step with the K split")
    ap.add_argument("--no-prefill", action="store_true",
                    help="skip the prefill sub-object (Qwen3-MoE-like prefill)")
    ap.add_argument("--no-align-stress", action="store_true",
                    help="skip the align stress sub-object")
    ap.add_argument("--step-only", action="store_true",
                    help="time the step alone: no comparison lines (profiler runs)")
    args = ap.parse_args(argv)
    if args.step_only:
        args.no_k_split_line = args.no_two_kernel = args.no_dual_stream = True
        args.no_prefill = args.no_align_stress = True

    if args.gpus != 1:
        print("bench.py: this build measures one GPU only (the hot path has no "
              "cross-GPU step); run with --gpus 1", file=sys.stderr)
        return 2
    if int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: one process, one GPU", file=sys.stderr)
        return 2

    import torch
    import moe_lora_adapter_amd as mla
    from moe_lora_adapter_amd import synth

    dev = torch.device("cuda:0")
    mla.lib()
    s = synth.shape(args.workload)
    if s.align_only:
        # an align-only workload: the align step is the whole step
        log(f"workload {s.name}: align only")
        if args.calibrate_copy:
            copy_calibration(dev)
        res = align_stress_line(args, dev, s.name)
        out = {"metric": "moe_lora_align us/call", "value": res["us_per_call"], "unit": "us/call",
               "n_gpus": 1, "steps": res["steps"], "warmup": args.warmup,
               "ms_per_step": round(res["us_per_call"] / 1e3, 6), "higher_is_better": False,
               "scaling": "weak", "vs_baseline": None, "dtype": "int32",
               "data": "synthetic (seeded routing and adapter mapping, no dataset)",
               "config": {"workload": s.name, "M": s.M, "topk": s.topk, "E": s.E, "L": s.L,
                          "block_m": s.block_m, "step": "moe_lora_align"},
               "align": res}
        print(json.dumps(out), flush=True)
        return 0
    log(f"workload {s.name}: drawing inputs")
    case = synth.draw(s)
    work = algorithmic_work(case)
    touched = work["fused_bytes"] + work["align_bytes"]
    copies = 1 if args.warm else max(1, min(64, math.ceil(args.cold_bytes / touched)))
    log(f"{copies} input copies (touched {touched / 1e6:.1f} MB each)")
    sets = [DeviceSet(case, dev)]
    for _ in range(copies - 1):
        sets.append(DeviceSet(case, dev, proto=sets[0]))
    variant = args.variant
    naive_ok = s.numel <= mla.NAIVE_MAX_PAIRS
    wa_ok = s.numel <= mla.WITH_ALIGN_MAX_PAIRS and s.L <= mla.WITH_ALIGN_MAX_SLOTS
    naive_bm = args.naive_block_m or s.block_m
    path = resolve_path(args.path, s)
    if path == "naive" and not naive_ok:
        print(f"bench.py: the align-free path takes at most {mla.NAIVE_MAX_PAIRS} pairs",
              file=sys.stderr)
        return 2
    if path == "with_align" and not wa_ok:
        print(f"bench.py: fused_moe_lora_with_align takes at most {mla.WITH_ALIGN_MAX_PAIRS} "
              f"pairs and {mla.WITH_ALIGN_MAX_SLOTS} slots", file=sys.stderr)
        return 2
    full_path = path in ("with_align", "sorted")  # steps that produce the align outputs
    naive_fn = lambda ds: run_naive(ds, s, naive_bm, variant)  # noqa: E731
    # the sorted path's step: align + fused_moe_lora, or with --k-split align +
    # fused_moe_lora_ws when its kernel uses a workspace (the decode stream
    # kernel's K split); one zero-filled workspace serves every copy (the
    # calls run one after another)
    nbx = mla.fused_moe_lora_workspace_bytes(s.M, s.topk, s.K, s.Ns, s.S, s.E, s.L, s.r,
                                             s.block_m, s.x_per_pair, variant)
    k_split = path == "sorted" and nbx > 0 and args.k_split
    xws = torch.zeros(nbx, dtype=torch.uint8, device=dev) if nbx > 0 else None
    fused_fn = ((lambda ds: run_fused_ws(ds, s, variant, xws)) if k_split  # noqa: E731
                else (lambda ds: run_fused(ds, s, variant)))
    wa_fn = lambda ds: run_with_align(ds, s, variant)  # noqa: E731
    step_fn = {"naive": naive_fn, "with_align": wa_fn}.get(
        path, lambda ds: (run_align(ds, s), fused_fn(ds)))

    log(f"warmup {args.warmup} steps")
    for i in range(args.warmup):
        step_fn(sets[i % copies])
    torch.cuda.synchronize()
    if args.calibrate_copy:
        copy_calibration(dev)

    log(f"timing {args.steps} steps (one graph)")
    replays = []
    sec_per_step = time_steps_graph(sets, s, variant, args.steps, fn=step_fn, replays=replays)
    log("timing kernels with events")
    med = {}
    if path == "naive":
        fused_avg, f10, f90 = time_kernel_windows(sets, s, variant, naive_fn, args.steps, out=med)
        align_avg = None
        kbytes = work["naive_bytes"]
    elif path == "with_align":
        fused_avg, f10, f90 = time_kernel_windows(sets, s, variant, wa_fn, args.steps, out=med)
        align_avg = None
        kbytes = work["with_align_bytes"]
    else:
        fused_avg, f10, f90 = time_kernel_windows(sets, s, variant, fused_fn, args.steps, out=med)
        align_avg = time_kernel_events(sets, s, variant, "align", args.steps)
        kbytes = work["fused_bytes"]

    gbps = kbytes / (fused_avg * 1e-6) / 1e9
    tflops = work["fused_flops"] / (fused_avg * 1e-6) / 1e12
    kname = {"sorted": _kernel_name(s, variant),
             "with_align": naive_kernel_name(s, s.block_m, variant)}.get(
        path, naive_kernel_name(s, naive_bm, variant))
    traffic, _rec = load_traffic(kname, {"sorted": s.name, "with_align": f"{s.name}/with_align"}
                                 .get(path, f"{s.name}/naive_b{naive_bm}"))
    out = {
        "metric": METRIC,
        "value": round(sec_per_step * 1e6, 3),
        "unit": "us/call",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(sec_per_step * 1e3, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; routing, adapter mapping and weights drawn, no dataset)",
        "config": {"workload": s.name, "M": s.M, "K": s.K, "N": s.N, "slices": s.S, "E": s.E,
                   "topk": s.topk, "L": s.L, "active_slots": s.active, "r": s.r,
                   "block_m": s.block_m, "mul_routed_weight": s.mul, "add_inputs": s.add,
                   "x_per_pair": s.x_per_pair,
                   "step": {"sorted": ("moe_lora_align + fused_moe_lora_ws (K split over a "
                                       "block's workgroups)" if k_split else
                                       "moe_lora_align + fused_moe_lora"),
                            "with_align": ("fused_moe_lora_with_align (the align outputs and "
                                           "the fused result in one launch)"),
                            "naive": f"fused_moe_lora_naive (no align outputs), "
                                     f"block_m={naive_bm}"}[path],
                   "timing": "one HIP graph of K steps; value from its first timed replay",
                   "cache": ("warm" if args.warm else
                             f"cold: {copies} rotated input copies, "
                             f"{copies * touched / 2 ** 30:.2f} GiB touched")},
        "roofline": {"bound": "hbm", "kernel": kname,
                     "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": traffic,
                     "algorithmic_bytes_per_launch": kbytes,
                     "kernel_us_avg": round(fused_avg, 3),
                     "kernel_us_p10": round(f10, 3), "kernel_us_p50": round(med["p50"], 3),
                     "kernel_us_p90": round(f90, 3),
                     "kernel_us_eager_avg": round(med["eager_avg"], 3),
                     "kernel_timing": "HIP events on the replay stream around 5 replays of "
                                      "one graph of K launches of the kernel alone; avg over "
                                      "the replays, p10/p50/p90 of the replay averages "
                                      "(kernel_us_eager_avg: the same launches eager)"},
        "us_per_call_replays": spread([r * 1e6 for r in replays]),
        "fused_tflops": round(tflops, 3),
        "mfma_frac_of_bf16_peak": round(tflops / BF16_PEAK_TFLOPS, 5),
        "align_kernel_us_avg": round(align_avg, 3) if align_avg is not None else None,
        "work": work,
    }
    plain_avg = fused_avg if (path == "sorted" and not k_split) else None
    if path == "with_align" and not args.step_only:
        # the same path in two launches: moe_lora_align, then fused_moe_lora
        log("two launches: align + fused")
        fn2l = lambda ds: (run_align(ds, s), run_fused(ds, s, variant))  # noqa: E731
        for i in range(args.warmup):
            fn2l(sets[i % copies])
        us2l = time_steps_graph(sets, s, variant, args.steps, fn=fn2l) * 1e6
        plain_avg = time_kernel_events(sets, s, variant, "fused", args.steps)
        al2l = time_kernel_events(sets, s, variant, "align", args.steps)
        g2l = work["fused_bytes"] / (plain_avg * 1e-6) / 1e9
        out["two_launches"] = {"us_per_call": round(us2l, 3), "kernel": _kernel_name(s, variant),
                               "kernel_us_avg": round(plain_avg, 3),
                               "align_kernel_us_avg": round(al2l, 3),
                               "achieved_GBps": round(g2l, 1),
                               "frac": round(g2l / HBM_PEAK_GBPS, 4),
                               "algorithmic_bytes_per_launch": work["fused_bytes"]}
    if full_path and naive_ok and not args.step_only:
        # the align-free path on the same inputs: no align launch, blocks
        # formed on chip (block_m of the workload, and one pair per block)
        out["align_free"] = []
        for bm in sorted({s.block_m, 1}, reverse=True):
            fn = lambda ds, bm=bm: run_naive(ds, s, bm, variant)  # noqa: E731
            log(f"align-free path, block_m={bm}")
            for i in range(args.warmup):
                fn(sets[i % copies])
            us = time_steps_graph(sets, s, variant, args.steps, fn=fn) * 1e6
            kus = time_kernel_events(sets, s, variant, fn, args.steps)
            g = work["naive_bytes"] / (kus * 1e-6) / 1e9
            out["align_free"].append({
                "block_m": bm, "us_per_call": round(us, 3),
                "kernel": naive_kernel_name(s, bm, variant),
                "kernel_us_avg": round(kus, 3), "achieved_GBps": round(g, 1),
                "frac": round(g / HBM_PEAK_GBPS, 4),
                "algorithmic_bytes_per_launch": work["naive_bytes"]})
    if full_path and nbx > 0 and not args.no_k_split_line:
        # the step the other way: with the K split (fused_moe_lora_ws: the
        # workgroups of a block share A's K range and exchange partial rank
        # vectors) or, when that is the step, without it
        other = not k_split
        log("step with the K split" if other else "step without the K split")
        ofn = ((lambda ds: run_fused_ws(ds, s, variant, xws)) if other  # noqa: E731
               else (lambda ds: run_fused(ds, s, variant)))
        fno = lambda ds: (run_align(ds, s), ofn(ds))  # noqa: E731
        for i in range(args.warmup):
            fno(sets[i % copies])
        uso = time_steps_graph(sets, s, variant, args.steps, fn=fno) * 1e6
        kuso = time_kernel_events(sets, s, variant, ofn, args.steps)
        go = work["fused_bytes"] / (kuso * 1e-6) / 1e9
        kplain, ksplit = (plain_avg, kuso) if other else (kuso, fused_avg)
        out["with_k_split" if other else "without_k_split"] = {
            "us_per_call": round(uso, 3), "kernel": kname, "kernel_us_avg": round(kuso, 3),
            "achieved_GBps": round(go, 1), "frac": round(go / HBM_PEAK_GBPS, 4),
            "workspace_bytes": nbx,
            "k_split_kernel_speedup": round(kplain / ksplit, 3) if kplain else None}
    if full_path and s.r <= mla.TWO_KERNEL_MAX_RANK and not args.no_two_kernel:
        # the two-kernel path on the same inputs (rank vectors through memory):
        # the comparator of the one-shot kernels
        nb = mla.two_kernel_workspace_bytes(s.M, s.topk, s.K, s.Ns, s.S, s.E, s.L, s.r,
                                            s.block_m, s.x_per_pair)
        ws2 = torch.empty(max(nb, 16), dtype=torch.uint8, device=dev)
        for ds in sets:
            ds.ws2 = ws2  # one workspace: its contents are rewritten by every call
        log("two-kernel path")
        fn2 = lambda ds: (run_align(ds, s), run_two_kernel(ds, s))  # noqa: E731
        for i in range(args.warmup):
            fn2(sets[i % copies])
        us2 = time_steps_graph(sets, s, variant, args.steps, fn=fn2) * 1e6
        kus2 = time_kernel_events(sets, s, variant, lambda ds: run_two_kernel(ds, s), args.steps)
        out["two_kernel"] = {"us_per_call": round(us2, 3), "kernels_us_avg": round(kus2, 3),
                             "workspace_bytes": nb,
                             "one_shot_speedup": round(kus2 / (plain_avg or fused_avg), 3)}
    if full_path and naive_ok and not args.no_dual_stream:
        from moe_lora_adapter_amd import synth as _synth
        try:
            _synth.w2_partner(s.name)
            has_w2 = True
        except KeyError:
            has_w2 = False
        if has_w2:
            out["layer_chain"] = layer_chain_line(sets, s, case, args.steps, dev, copies)
        else:
            out["dual_stream"] = dual_stream_line(sets, s, case, args.steps, dev)
    if not args.no_cpu_baseline:
        log(f"cpu baseline (oracle, ~{args.cpu_budget:.0f} s)")
        out["cpu_baseline"] = cpu_baseline(case, args.cpu_budget)
    if not args.no_align_stress:
        log("align stress line")
        out["align_stress"] = align_stress_line(args, dev)
    if not args.no_prefill and s.name != "qwen3_prefill":
        del sets
        torch.cuda.empty_cache()
        out["prefill"] = prefill_line(args, dev, variant)
    print(json.dumps(out), flush=True)
    return 0


def _kernel_name(s, variant):
    import moe_lora_adapter_amd as mla
    return mla.fused_kernel_name(s.M, s.topk, s.K, s.Ns, s.S, s.E, s.L, s.r, s.block_m,
                                 s.x_per_pair, variant)


if __name__ == "__main__":
    sys.exit(main())
