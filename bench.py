#!/usr/bin/env python3
"""Benchmark of the WKV forward on one MI355X.

Default workload (the headline metric): GPT-mode WKV forward at B=8, T=1024,
C=2048, fp32, shaped like one layer of a 24-layer, 2048-wide model at context
1024; 24 independently seeded layers, all resident in HBM (4.8 GB of inputs
and outputs, far above the 256 MB last-level cache), called back to back.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the forward over all 24 layers (24 calls of
wkv_forward).  Prints one JSON line with the lane-token throughput
(tokens x channels / s), the roofline of the forward kernel (algorithmic HBM
bytes per launch over its average launch time, measured with HIP events on the
stream it runs on), and the float64 CPU oracle timed on this host as a baseline.
The same line carries, under "other_configs", the stream, decode and stability
forward and backward figures, each timed as its own --workload run times it
(fewer steps; --headline-only leaves them out).

Other workloads print their own line in the same format; they are parity
workloads with extra measurements, not the headline:
    stream, decode, stability_fwd, stability_bwd   the other operator shapes
    stability_bwd_state       the backward of a chunk with carried states
    stability_bwd_bf16        the backward with bf16 activations and gradients
    stability_fwd_ckpt        the forward that also writes 128-token checkpoints
    stability_bwd_ckpt[_bf16] the backward that starts from those checkpoints
    stability_bwd_gated_ckpt  the same for the gated output (dr written too)
    gpt_gated, decode_gated   the same with the output gate sigmoid(r) fused in
    gpt_bf16, gpt_f16         the GPT forward with 16-bit activations (state fp32)
    token_shift               the token shift at the GPT shape (3 mixes)
    token_shift_bwd           its backward (dx, d_x_prev, dmu)
    copy                      a 1 GiB device copy, the bandwidth reference
"""
from __future__ import annotations

import argparse
import gc
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "WKV fwd tokens·channels/sec + HBM GB/s (% peak), B=8 T=1024 C=2048 fp32"
METRIC_GATED = ("WKV fwd with the sigmoid(r) output gate, tokens·channels/sec, "
                "B=8 T=1024 C=2048 fp32")
PEAK_HBM_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
# The sources each kernel is compiled from (its own file and the shared
# headers): a counter run stays valid while these are unchanged.
_CSRC = "linear_recurrent_attention_amd/csrc/"
_SHARED = [_CSRC + "wkv_device.hpp", _CSRC + "wkv_internal.hpp"]
KERNEL_SOURCES = {
    "fwd_lookback_kernel": [_CSRC + "wkv_lookback.hip"] + _SHARED,
    "fwd_seg_kernel": [_CSRC + "wkv_forward.hip"] + _SHARED,
    "fwd_lane_kernel": [_CSRC + "wkv_forward.hip"] + _SHARED,
    "step_kernel": [_CSRC + "wkv_step.hip"] + _SHARED,
    "bwd_seg_kernel": [_CSRC + "wkv_backward.hip"] + _SHARED,
    "shift_kernel": [_CSRC + "wkv_shift.hip"] + _SHARED,
    "shift_bwd_kernel": [_CSRC + "wkv_shift.hip"] + _SHARED,
}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def source_hash(kernel: str) -> str:
    """Hash of the sources the named kernel (its template name; arguments
    ignored) is built from."""
    h = hashlib.sha256()
    for p in KERNEL_SOURCES[kernel.split("<")[0]]:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter runs, if they
    were taken on the current kernel sources; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    e = rec.get(workload)
    if not e or e.get("kernel") != kernel or e.get("source_hash") != source_hash(kernel):
        return None
    return e.get("bytes_per_launch")


ORACLE_MAX_THREADS = 256


def host_cpus():
    """(cores this job may run on, how that was decided, online CPUs).  The
    job's share is its affinity mask, further limited by OMP_NUM_THREADS
    where the machine sets it (a shared host gives each GPU a share of its
    cores that way, whatever the online count)."""
    online = os.cpu_count() or 1
    try:
        n = len(os.sched_getaffinity(0))
        how = "affinity mask"
    except AttributeError:
        n, how = online, "online CPUs"
    omp = os.environ.get("OMP_NUM_THREADS", "")
    if omp.isdigit() and 0 < int(omp) < n:
        n, how = int(omp), f"OMP_NUM_THREADS (affinity mask holds {n})"
    if n > ORACLE_MAX_THREADS:
        n, how = ORACLE_MAX_THREADS, (how + f" holds {n}; the oracle runs at most "
                                      f"{ORACLE_MAX_THREADS} threads")
    return max(1, n), how, online


def host_cores() -> int:
    return host_cpus()[0]


def host_description() -> dict:
    n, how, online = host_cpus()
    return {"cpu_model": cpu_model(), "cpus_online": online, "cores_used_from": how}


class Timer:
    """HIP events on the stream the kernels are launched on.  Python's cyclic
    garbage collector is paused between start and stop: a full collection in a
    process holding torch takes about 30 ms of host time, during which no
    launch is issued and the GPU drains its queue and idles inside the timed
    region (measured: one such pause tripled a batch of 120 gpt launches)."""

    def __init__(self, torch, stream):
        self.torch = torch
        self.stream = stream
        self.a = torch.cuda.Event(enable_timing=True)
        self.b = torch.cuda.Event(enable_timing=True)
        self.gc_was_enabled = False

    def start(self):
        self.gc_was_enabled = gc.isenabled()
        gc.disable()
        self.a.record(self.stream)

    def stop_ms(self):
        self.b.record(self.stream)
        self.b.synchronize()
        if self.gc_was_enabled:
            gc.enable()
        return self.a.elapsed_time(self.b)


def cpu_model() -> str:
    """The host CPU's model name, with its family/model/stepping numbers where
    the name alone is generic."""
    info = {}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if ":" in line:
                    key, val = (x.strip() for x in line.split(":", 1))
                    info.setdefault(key, val)
                if not line.strip() and info:
                    break
    except OSError:
        return "unknown"
    name = info.get("model name", "unknown")
    ids = [f"{k} {info[k]}" for k in ("cpu family", "model", "stepping") if k in info]
    return name + (f" ({', '.join(ids)})" if ids else "")


def timed_oracle(fn, budget_s: float):
    """Calls fn(i) for i = 0, 1, ... until budget_s seconds of oracle time
    have been spent (at least one call).  fn returns (lane-tokens, seconds of
    oracle compute) for its sample, or None when there is no sample left.
    Returns (lane-tokens, seconds, calls)."""
    done, elapsed, i = 0, 0.0, 0
    while i == 0 or elapsed < budget_s:
        r = fn(i)
        if r is None:
            break
        done += r[0]
        elapsed += r[1]
        i += 1
    return done, elapsed, i


def cpu_baseline_gpt(torch, synth, inputs_fn, budget_s: float):
    """The oracle's O(T) recurrence on whole layers of the same workload."""
    import oracle
    cores = host_cores()
    done = 0
    elapsed = 0.0
    layer = 0
    gated = False
    # whole layers, cycling over the 24 until the budget is spent (at least
    # one pass), so that the figure rests on about budget_s of CPU work
    host = {}  # float64 host copies, made once per layer (not timed)
    while layer < 24 or elapsed < budget_s:
        if layer % 24 not in host:
            d = inputs_fn(layer % 24)
            host[layer % 24] = ([d[n].double().cpu().numpy() for n in ("w", "u", "k", "v")],
                                d["r"].double().cpu().numpy() if "r" in d else None,
                                d["k"].numel())
        a, r, n_lt = host[layer % 24]
        t0 = time.perf_counter()
        y, _ = oracle.forward_scan(*a, nthreads=cores)
        if r is not None:
            gated = True
            oracle.gate(y, r)
        elapsed += time.perf_counter() - t0
        done += n_lt
        layer += 1
    what = "recurrence and gate (the gate single-threaded)" if gated else "recurrence"
    # the same on one thread, on the first layer
    d = inputs_fn(0)
    a = [d[n].double().cpu().numpy() for n in ("w", "u", "k", "v")]
    t0 = time.perf_counter()
    oracle.forward_scan(*a, nthreads=1)
    one = d["k"].numel() / (time.perf_counter() - t0)
    per_tok = 12.0 if not gated else 16.0   # algorithmic fp32 bytes per lane-token
    return {"value": done / elapsed, "unit": "tok·ch/s", "cores": cores, "kind": "oracle",
            "sample": f"{layer} layer calls over the 24 seeded B=8 T=1024 C=2048 layers, "
                      f"whole, float64 O(T) {what} on {cores} threads ({elapsed:.1f} s)",
            "value_1_thread": one, "effective_gbs": done / elapsed * per_tok / 1e9,
            **host_description()}


def bench_gpt(args, torch, wkv, synth, gated: bool = False, io: str = "f32"):
    """GPT-mode forward of 24 seeded layers; gated: with the time-mixing output
    gate y = sigmoid(r) * wkv fused in (r read beside k and v); io: element
    format of k, v, r and y ("f32", "f16" or "bf16"; the state is float32)."""
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[io]
    esz = 4 if io == "f32" else 2
    sh = synth.SHAPES[synth.GPT]
    B, T, C, NL = sh["B"], sh["T"], sh["C"], sh["layers"]
    dev = torch.device("cuda")
    stream = torch.cuda.current_stream()
    log(f"gpt: generating {NL} layers of B={B} T={T} C={C} on the device")
    layers = []
    for l in range(NL):
        d = synth.make(synth.GPT, index=l, device=dev)
        if io != "f32":
            d["k"], d["v"] = d["k"].to(tdt), d["v"].to(tdt)
        d["y"] = torch.empty_like(d["k"])
        d["s"] = torch.empty((3, B, C), device=dev)
        if gated:
            d["r"] = synth.receptance(synth.GPT, l, (B, T, C), device=dev).to(tdt)
        layers.append(d)
    plan = tuple(args.plan) if args.plan else None
    chosen = plan or wkv.wkv_forward_plan_auto(B, T, C)
    if gated and not plan:
        chosen = gated_auto_plan(chosen)

    def call(d):
        if io != "f32":
            wkv.wkv_forward_typed(d["w"], d["u"], d["k"], d["v"], d.get("r"), y=d["y"],
                                  state_out=d["s"], stream=stream, plan=plan)
        elif gated:
            wkv.wkv_forward_gated(d["w"], d["u"], d["k"], d["v"], d["r"], y=d["y"],
                                  state_out=d["s"], stream=stream, plan=plan)
        else:
            wkv.wkv_forward(d["w"], d["u"], d["k"], d["v"], y=d["y"], state_out=d["s"],
                            stream=stream, plan=plan)

    for _ in range(args.warmup):
        for d in layers:
            call(d)
    torch.cuda.synchronize()
    # Isolated launches: each layer alone between two events on an idle
    # stream (median of 5, mean over layers).  Reported beside the metric, not
    # as it: an isolated launch also pays the grid's ramp-up and drain, which
    # back-to-back launches overlap with their neighbours.
    per_layer = []
    tm = Timer(torch, stream)
    for d in layers:
        reps = []
        for _ in range(5):
            tm.start()
            call(d)
            reps.append(tm.stop_ms())
        reps.sort()
        per_layer.append(reps[len(reps) // 2])
    torch.cuda.synchronize()
    log(f"gpt: timing {args.steps} steps x {NL} layers")
    t_wall = time.perf_counter()
    tm.start()
    for _ in range(args.steps):
        for d in layers:
            call(d)
    ms = tm.stop_ms()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t_wall) * 1e3
    launches = args.steps * NL
    ms_launch = ms / launches
    lane_tok = B * T * C
    # k, v (and r) in, y out; w, u; state out
    algo_bytes = (4 if gated else 3) * esz * lane_tok + 8 * C + 12 * B * C
    achieved = algo_bytes / (ms_launch * 1e-3) / 1e9
    kname = kernel_name(chosen, wkv, gated, io)
    wl = ("gpt_gated" if gated else "gpt") + ("" if io == "f32" else "_" + io)
    traffic = measured_traffic(kname, wl)
    metric = METRIC_GATED if gated else METRIC
    if io != "f32":
        metric = metric.replace("fp32", f"{io} activations, fp32 state")
    out = {
        "metric": metric,
        "value": lane_tok * launches / (ms * 1e-3),
        "unit": "tok·ch/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": io,
        "data": "synthetic (seeded; k, v ~ N(0,1) with k x2, decay ~ U(-5,1), u ~ N(0,0.5)"
                + (", r ~ N(0,2))" if gated else ")"),
        "config": {"workload": ("gpt_gated_forward" if gated else "gpt_forward") +
                   ("" if io == "f32" else "_" + io), "B": B, "T": T, "C": C, "layers": NL,
                   "kernel": kname, "plan": list(chosen),
                   "timing": "value, ms_per_step and roofline come from the timed region: "
                             f"{args.steps} steps x {NL} layers launched back to back on one "
                             "stream between two HIP events",
                   "isolated_launch_ms": sum(per_layer) / len(per_layer),
                   "isolated_launch_note": "one layer alone between two events on an idle "
                                           "stream (median of 5, mean over the layers): adds "
                                           "the grid's ramp-up and drain, which back-to-back "
                                           "launches overlap",
                   "hbm_gbs": achieved, "pct_peak_hbm": 100 * achieved / PEAK_HBM_GBS,
                   "wall_ms_timed_region": wall_ms},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS, "traffic": traffic,
                     "algorithmic_bytes_per_launch": algo_bytes,
                     "avg_launch_us": ms_launch * 1e3},
    }
    if not args.no_cpu_baseline:
        log("gpt: timing the CPU oracle")
        names = ("w", "u", "k", "v", "r") if gated else ("w", "u", "k", "v")
        out["cpu_baseline"] = cpu_baseline_gpt(
            torch, synth, lambda l: {n: layers[l][n] for n in names}, args.cpu_seconds)
    return out


IO_NAMES = {"f32": "wkv::IoF32", "f16": "wkv::IoF16", "bf16": "wkv::IoBF16"}


def kernel_name(plan, wkv, gated: bool = False, io: str = "f32") -> str:
    """Kernel symbol (template arguments as in the profiler's kernel names)."""
    kernel, nw, ls = plan[:3]
    cw = plan[3] if len(plan) > 3 and plan[3] else 64
    g = "true" if gated else "false"
    t = IO_NAMES[io]
    if kernel == wkv.WKV_KERNEL_LANE:
        return f"fwd_lane_kernel<{g}, {t}>"
    if kernel == wkv.WKV_KERNEL_SEGMENTED:
        return f"fwd_seg_kernel<{nw * cw // 64}, {ls}, {cw}, {g}, {t}>"
    if kernel == wkv.WKV_KERNEL_LOOKBACK:
        return f"fwd_lookback_kernel<{cw // 64}, {nw}, {ls}, {g}, {t}>"
    return f"kernel{kernel}<{nw}, {ls}>"


def gated_auto_plan(plan):
    """The plan the library's automatic choice takes for the gated forward: a
    look-back block keeps its length, cut into segments of at most 16 tokens
    (the gated look-back kernel is compiled for those only)."""
    kernel, ns, ls = plan[:3]
    if kernel == 3 and ls > 16:
        return (kernel, ns * ls // 16, 16) + tuple(plan[3:])
    return tuple(plan)


def bench_stream(args, torch, wkv, synth):
    """B=1 C=5120, 1024 chunks of 1024 tokens with the state carried; all
    64.6 GB of inputs resident before timing; per-call mean."""
    sh = synth.SHAPES[synth.STREAM]
    C, TC, NCH = sh["C"], sh["T"], sh["chunks"]
    dev = torch.device("cuda")
    stream = torch.cuda.current_stream()
    w, u = synth.channel_params(synth.STREAM, 0, C, device=dev)
    log(f"stream: generating {NCH} chunks")
    k = torch.empty((NCH, 1, TC, C), device=dev)
    v = torch.empty((NCH, 1, TC, C), device=dev)
    for j in range(NCH):
        k[j], v[j] = synth.sequence(synth.STREAM, j, (1, TC, C), device=dev)
    y = torch.empty((NCH, 1, TC, C), device=dev)
    st = torch.empty((3, 1, C), device=dev)
    plan = tuple(args.plan) if args.plan else None

    # the 1024 calls' arguments are marshalled once (as a C caller would hold
    # them), so the loop measures the launches, not Python's per-call checks
    calls = [wkv.bind_forward(w, u, k[j], v[j], y[j], state_in=None if j == 0 else st,
                              state_out=st, stream=stream, plan=plan) for j in range(NCH)]

    def run_all():
        for c in calls:
            c()

    for _ in range(args.warmup):
        run_all()
    torch.cuda.synchronize()
    tm = Timer(torch, stream)
    tm.start()
    for _ in range(args.steps):
        run_all()
    ms = tm.stop_ms()
    per_call = ms / (args.steps * NCH)
    lane_tok = TC * C
    algo = 12 * lane_tok + 8 * C + 24 * C
    chosen = plan or wkv.wkv_forward_plan_auto(1, TC, C)
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        cores = host_cores()
        w64, u64 = w.double().cpu().numpy(), u.double().cpu().numpy()
        carried = [None]

        def chunk(j):
            if j >= NCH:
                return None
            kk, vv = k[j].double().cpu().numpy(), v[j].double().cpu().numpy()
            t0 = time.perf_counter()
            _, carried[0] = oracle.forward_scan(w64, u64, kk, vv, carried[0], nthreads=cores)
            return TC * C, time.perf_counter() - t0

        done, secs, calls = timed_oracle(chunk, args.cpu_seconds)
        cpu = {"value": done / secs, "unit": "tok·ch/s", "cores": cores, "kind": "oracle",
               "sample": f"the first {calls} of the 1024 chunks (B=1 T=1024 C=5120 each), state "
                         f"carried, float64 O(T) recurrence on {cores} threads ({secs:.1f} s)"}
    return {"metric": "WKV streaming fwd tokens·channels/sec, B=1 C=5120, 1024 chunks x 1024",
            "value": lane_tok * NCH * args.steps / (ms * 1e-3), "unit": "tok·ch/s",
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": ms / args.steps, "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "f32", "data": "synthetic",
            "config": {"workload": "stream_forward", "C": C, "chunk": TC, "chunks": NCH,
                       "kernel": kernel_name(chosen, wkv), "per_call_us": per_call * 1e3},
            "roofline": {"bound": "hbm", "achieved": algo / (per_call * 1e-3) / 1e9,
                         "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": algo / (per_call * 1e-3) / 1e9 / PEAK_HBM_GBS,
                         "traffic": measured_traffic(kernel_name(chosen, wkv), "stream"),
                         "algorithmic_bytes_per_launch": algo, "avg_launch_us": per_call * 1e3},
            "cpu_baseline": cpu}


def bench_decode(args, torch, wkv, synth, gated: bool = False):
    """L=24 B=1024 C=4096 batched T=1 steps; state from 256 warm-up tokens;
    inputs from a ring of 32 distinct [24][1024][4096] k, v (and r) sets.
    gated: the step with the output gate y = sigmoid(r) * wkv."""
    sh = synth.SHAPES[synth.DECODE]
    L, B, C, WU, RING = sh["L"], sh["B"], sh["C"], sh["warmup"], sh["ring"]
    dev = torch.device("cuda")
    stream = torch.cuda.current_stream()
    state = torch.empty((L, 3, B, C), device=dev)
    w_all = torch.empty((L, C), device=dev)
    u_all = torch.empty((L, C), device=dev)
    for l in range(L):
        w_all[l], u_all[l] = synth.channel_params(synth.DECODE, l, C, device=dev)
        kk, vv = synth.sequence(synth.DECODE, l, (B, WU, C), device=dev)
        wkv.wkv_forward(w_all[l], u_all[l], kk, vv, state_out=state[l], stream=stream)
        del kk, vv
    log("decode: generating the input ring")
    ring = [synth.sequence(synth.DECODE, 1000 + r, (L, B, C), device=dev) for r in range(RING)]
    if gated:
        ring = [kv + (synth.receptance(synth.DECODE, 1000 + r, (L, B, C), device=dev),)
                for r, kv in enumerate(ring)]
    y = torch.empty((L, B, C), device=dev)
    nsteps = args.steps * 64

    def call(r):
        e = ring[r % RING]
        if gated:
            wkv.wkv_step_gated(w_all, u_all, e[0], e[1], e[2], state, y=y, stream=stream)
        else:
            wkv.wkv_step(w_all, u_all, e[0], e[1], state, y=y, stream=stream)

    for r in range(args.warmup * 8):
        call(r)
    torch.cuda.synchronize()
    tm = Timer(torch, stream)
    tm.start()
    for r in range(nsteps):
        call(r)
    ms = tm.stop_ms()
    per = ms / nsteps
    lanes = L * B * C
    algo = (40 if gated else 36) * lanes + 8 * L * C
    # (four channels per thread, in four 1024-channel chunks; two when gated)
    kname = f"step_kernel<4, {2 if gated else 4}, {'true' if gated else 'false'}, wkv::IoF32>"
    wl = "decode_gated" if gated else "decode"
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        cores = host_cores()
        # one step of layer l (B x C lanes) from the current state, per sample
        def layer(l):
            if l >= L:
                return None
            a = [t.double().cpu().numpy() for t in (w_all[l], u_all[l], ring[0][0][l:l + 1],
                                                     ring[0][1][l:l + 1])]
            kk = a[2].reshape(B, 1, C)
            vv = a[3].reshape(B, 1, C)
            rr = ring[0][2][l].double().cpu().numpy() if gated else None
            s_in = state[l].double().cpu().numpy()
            t0 = time.perf_counter()
            yy, _ = oracle.forward_scan(a[0], a[1], kk, vv, s_in, nthreads=cores)
            if gated:
                oracle.gate(yy[:, 0, :], rr)
            return B * C, time.perf_counter() - t0

        done, secs, calls = timed_oracle(layer, args.cpu_seconds)
        cpu = {"value": done / secs / lanes, "unit": "steps/s", "cores": cores, "kind": "oracle",
               "sample": f"{calls} of the 24 layers (B=1024 C=4096 lanes each) stepped once, "
                         f"float64, on {cores} threads ({secs:.1f} s), extrapolated per lane-step "
                         f"to the whole L=24 step"}
    metric = ("WKV decode steps/sec with the sigmoid(r) output gate, L=24 B=1024 C=4096 fp32"
              if gated else "WKV decode steps/sec, L=24 B=1024 C=4096 fp32")
    return {"metric": metric, "value": 1e3 / per,
            "unit": "steps/s", "n_gpus": 1, "steps": nsteps, "warmup": args.warmup * 8,
            "ms_per_step": per, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "f32", "data": "synthetic",
            "config": {"workload": "decode_gated_step" if gated else "decode_step", "L": L,
                       "B": B, "C": C, "kernel": kname,
                       "state_gbs": 24 * lanes / (per * 1e-3) / 1e9},
            "roofline": {"bound": "hbm", "achieved": algo / (per * 1e-3) / 1e9,
                         "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": algo / (per * 1e-3) / 1e9 / PEAK_HBM_GBS,
                         "traffic": measured_traffic(kname, wl),
                         "algorithmic_bytes_per_launch": algo, "avg_launch_us": per * 1e3},
            "cpu_baseline": cpu}


def bench_stability(args, torch, wkv, synth, backward: bool, carried: bool = False,
                    io: str = "f32", ckpt: bool = False, gated: bool = False):
    """B=8 T=4096 C=2048 with wide exponents; backward: the gradients; carried:
    the backward of a chunk that starts from a carried state and hands one on
    (wkv_backward_state, with the state gradient in and out); ckpt: the forward
    that also writes its 128-token checkpoints, or the backward that starts
    from them (wkv_forward_checkpointed / wkv_backward_checkpointed; the
    checkpoints are written by the forward before the timed region); gated: the
    backward of the gated output sigmoid(r) * wkv from the checkpoints
    (wkv_backward_gated, dr written as well)."""
    sh = synth.SHAPES[synth.STABILITY]
    B, T, C = sh["B"], sh["T"], sh["C"]
    dev = torch.device("cuda")
    stream = torch.cuda.current_stream()
    sets = [synth.make(synth.STABILITY, index=i, device=dev, with_dy=backward) for i in range(4)]
    if io != "f32":   # backward with 16-bit k, v, dy, dk, dv (state and dw, du float32)
        tdt = {"f16": torch.float16, "bf16": torch.bfloat16}[io]
        for st_ in sets:
            for n in ("k", "v", "dy"):
                st_[n] = st_[n].to(tdt)
    lane_tok = B * T * C
    nck = wkv.checkpoint_count(T)
    if gated:
        for i, st_ in enumerate(sets):
            st_["r"] = synth.receptance(synth.STABILITY, i, (B, T, C), device=dev).to(st_["k"].dtype)
    if ckpt:
        for st_ in sets:
            _, _, st_["ck"] = wkv.wkv_forward_checkpointed(st_["w"], st_["u"], st_["k"], st_["v"],
                                                           r=st_.get("r"))
    if backward:
        ws = torch.empty(wkv.wkv_backward_workspace_size(B, T, C), device=dev, dtype=torch.uint8)
        outs = [tuple(torch.empty_like(s["k"]) for _ in range(2)) for s in sets]
        dwu = torch.empty((2, C), device=dev)

        if carried:
            for i, st_ in enumerate(sets):
                # a state from 64 earlier tokens, the state handed on, and an
                # upstream gradient in its coordinates
                kk, vv = synth.sequence(synth.STABILITY, 200 + i, (B, 64, C), device=dev)
                _, st_["s_in"] = wkv.wkv_forward(st_["w"], st_["u"], kk, vv, state_out=True)
                _, st_["s_out"] = wkv.wkv_forward(st_["w"], st_["u"], st_["k"], st_["v"],
                                                  state_in=st_["s_in"], state_out=True)
                st_["g"] = synth.normal((3, B, C), 1.0, synth.seed_of(synth.STABILITY, 300 + i, 0),
                                        device=dev)
            dsi = torch.empty((3, B, C), device=dev)

        if gated:
            drs = [torch.empty_like(s["k"]) for s in sets]

        def call(i):
            s = sets[i]
            if gated:
                wkv.wkv_backward_gated(s["w"], s["u"], s["k"], s["v"], s["r"], s["dy"],
                                       checkpoints=s["ck"], dk=outs[i][0], dv=outs[i][1],
                                       dr=drs[i], dw=dwu[0], du=dwu[1], workspace=ws,
                                       stream=stream)
            elif ckpt:
                wkv.wkv_backward_checkpointed(s["w"], s["u"], s["k"], s["v"], s["dy"], s["ck"],
                                              dk=outs[i][0], dv=outs[i][1], dw=dwu[0],
                                              du=dwu[1], workspace=ws, stream=stream)
            elif io != "f32":
                wkv.wkv_backward_typed(s["w"], s["u"], s["k"], s["v"], s["dy"], dk=outs[i][0],
                                       dv=outs[i][1], dw=dwu[0], du=dwu[1], workspace=ws,
                                       stream=stream)
            elif carried:
                wkv.wkv_backward_state(s["w"], s["u"], s["k"], s["v"], s["dy"],
                                       state_in=s["s_in"], state_out=s["s_out"],
                                       d_state_out=s["g"], dk=outs[i][0], dv=outs[i][1],
                                       dw=dwu[0], du=dwu[1], d_state_in=dsi, workspace=ws,
                                       stream=stream)
            else:
                wkv.wkv_backward(s["w"], s["u"], s["k"], s["v"], s["dy"], dk=outs[i][0],
                                 dv=outs[i][1], dw=dwu[0], du=dwu[1], workspace=ws,
                                 stream=stream)
        # k, v, dy in, dk, dv out; w, u in, dw, du out; with carried states also
        # state_in, state_out's o-plane and the upstream gradient in, d_state_in out
        esz = 4 if io == "f32" else 2
        # (and the checkpoints in: 12 bytes per lane each)
        # (and the checkpoints in: 12 bytes per lane each; gated: r in, dr out)
        algo = ((7 if gated else 5) * esz * lane_tok + 16 * C +
                (40 * B * C if carried else 0) + (12 * B * C * nck if ckpt else 0))
        name = "WKV backward tokens·channels/sec, B=8 T=4096 C=2048 fp32"
        # (the whole-tile variant when T is a multiple of its 128-token tile)
        full = T % 128 == 0
        kname = (f"bwd_seg_kernel<16, 8, {'true' if full else 'false'}, "
                 f"{'true' if ckpt else 'false'}, {'true' if gated else 'false'}, "
                 f"{IO_NAMES[io]}>")
        if io != "f32":
            name = name.replace("fp32", f"{io} activations, fp32 state")
        if carried:
            name = name.replace("backward", "backward with carried states")
        if ckpt:
            name = name.replace("backward", "backward from the forward's checkpoints")
        if gated:
            name = name.replace("backward", "gated backward (dr too)")
    else:
        ys = [torch.empty_like(s["k"]) for s in sets]

        def call(i):
            s = sets[i]
            if ckpt:
                wkv.wkv_forward_checkpointed(s["w"], s["u"], s["k"], s["v"], y=ys[i],
                                             checkpoints=s["ck"], stream=stream)
            else:
                wkv.wkv_forward(s["w"], s["u"], s["k"], s["v"], y=ys[i], stream=stream)
        algo = 12 * lane_tok + 8 * C + (12 * B * C * nck if ckpt else 0)
        name = "WKV fwd tokens·channels/sec, B=8 T=4096 C=2048 fp32 (wide exponents)"
        if ckpt:
            name = name.replace("fwd", "fwd with 128-token checkpoints")
        kname = kernel_name(wkv.wkv_forward_plan_auto(B, T, C), wkv)
    for i in range(args.warmup):
        call(i % 4)
    torch.cuda.synchronize()
    n = args.steps * 4
    tm = Timer(torch, stream)
    tm.start()
    for i in range(n):
        call(i % 4)
    ms = tm.stop_ms()
    per = ms / n
    wl = ("stability_bwd_state" if carried else "stability_bwd") if backward else "stability_fwd"
    if gated:
        wl += "_gated"
    if ckpt:
        wl += "_ckpt"
    if io != "f32":
        wl += "_" + io
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        cores = host_cores()

        def seq(i):  # one sequence (T x C lanes) of the first input set per sample
            if i >= B:
                return None
            st_ = sets[0]
            a = [st_[n].double().cpu().numpy() for n in ("w", "u")]
            kk, vv = (st_[n][i:i + 1].double().cpu().numpy() for n in ("k", "v"))
            if carried:
                # the oracle's stateful backward is the O(T^2) closed form: time one
                # 256-token piece of the sequence, counted as such
                cut = 256
                sub = lambda t, lo, hi: t[i:i + 1, lo:hi].double().cpu().numpy()
                # the carried states are the oracle's own: from tokens 256..319 of
                # the sequence, then over the timed piece
                _, s_in = oracle.forward_scan(a[0], a[1], sub(st_["k"], cut, cut + 64),
                                              sub(st_["v"], cut, cut + 64))
                kp, vp, gp = (sub(st_[n], 0, cut) for n in ("k", "v", "dy"))
                _, s_out = oracle.forward_scan(a[0], a[1], kp, vp, s_in)
                t0 = time.perf_counter()
                oracle.backward_state(a[0], a[1], kp, vp, gp, s_in, s_out,
                                      st_["g"][:, i:i + 1].double().cpu().numpy())
                return cut * C, time.perf_counter() - t0
            dyy = st_["dy"][i:i + 1].double().cpu().numpy() if backward else None
            rr = st_["r"][i:i + 1].double().cpu().numpy() if gated else None
            t0 = time.perf_counter()
            if backward and gated:
                # the oracle's gated backward: wkv, the gate's chain rule, the reverse scan
                yy, _ = oracle.forward_scan(a[0], a[1], kk, vv, nthreads=cores)
                gg, _ = oracle.gate_backward(yy, rr, dyy)
                oracle.backward_scan(a[0], a[1], kk, vv, gg, nthreads=cores)
            elif backward:
                oracle.backward_scan(a[0], a[1], kk, vv, dyy, nthreads=cores)
            else:
                oracle.forward_scan(a[0], a[1], kk, vv, nthreads=cores)
            return T * C, time.perf_counter() - t0

        done, secs, calls = timed_oracle(seq, args.cpu_seconds)
        cpu = {"value": done / secs, "unit": "tok·ch/s", "cores": cores, "kind": "oracle",
               "sample": f"{calls} of the 8 sequences (T=4096 C=2048 each), float64 O(T) "
                         f"{'recurrence, gate chain rule and reverse scan' if gated else ('reverse scan' if backward else 'recurrence')} "
                         f"on {cores} threads ({secs:.1f} s)"}
        if carried:
            cpu["cores"] = 1
            cpu["sample"] = (f"the first 256 tokens of {calls} of the 8 sequences (C=2048), "
                             f"float64 O(T^2) closed-form backward with carried states on one "
                             f"thread ({secs:.1f} s)")
    return {"metric": name, "value": lane_tok / (per * 1e-3), "unit": "tok·ch/s",
            "n_gpus": 1, "steps": n, "warmup": args.warmup, "ms_per_step": per,
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": io,
            "data": "synthetic", "config": {"workload": wl, "B": B, "T": T, "C": C,
                                            "kernel": kname},
            "roofline": {"bound": "hbm", "achieved": algo / (per * 1e-3) / 1e9,
                         "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": algo / (per * 1e-3) / 1e9 / PEAK_HBM_GBS,
                         "traffic": measured_traffic(kname, wl),
                         "algorithmic_bytes_per_launch": algo, "avg_launch_us": per * 1e3},
            "cpu_baseline": cpu}


def bench_shift(args, torch, wkv, synth, backward: bool = False):
    """Token shift at the GPT shape (B=8 T=1024 C=2048) with the three mixes of
    the R, K and V inputs, the carried token updated in place; rotating over
    4 input sets (1 GiB of traffic in all, beyond the 256 MB last-level
    cache).  backward: the shift's backward (dx, d_x_prev, dmu) from seeded
    gradients of the mixes and of the carried token."""
    sh = synth.SHAPES[synth.GPT]
    B, T, C, M, NSET = sh["B"], sh["T"], sh["C"], 3, 4
    dev = torch.device("cuda")
    stream = torch.cuda.current_stream()
    sets = []
    for i in range(NSET):
        mu, x, xp = synth.shift_inputs(synth.GPT, 100 + i, B, T, C, M, device=dev)
        e = dict(mu=mu, x=x, xp=xp)
        if backward:
            e["d"] = synth.normal((M, B, T, C), 1.0, synth.seed_of(synth.GPT, 9800 + i, 0),
                                  device=dev)
            e["dxpo"] = synth.normal((B, C), 1.0, synth.seed_of(synth.GPT, 9900 + i, 0),
                                     device=dev)
            e["dx"], e["dxp"] = torch.empty_like(x), torch.empty((B, C), device=dev)
            e["dmu"] = torch.empty((M, C), device=dev)
        else:
            e["out"] = torch.empty((M, B, T, C), device=dev)
        sets.append(e)
    if backward:
        ws = torch.empty(max(1, int(wkv.load_library().wkv_token_shift_backward_workspace_size(
            B, T, C, M))), device=dev, dtype=torch.uint8)

    def call(i):
        e = sets[i % NSET]
        if backward:
            wkv.wkv_token_shift_backward(e["mu"], e["x"], e["d"], x_prev=e["xp"],
                                         d_x_prev_out=e["dxpo"], dx=e["dx"], d_x_prev=e["dxp"],
                                         dmu=e["dmu"], workspace=ws, stream=stream)
        else:
            wkv.wkv_token_shift(e["mu"], e["x"], e["xp"], out=e["out"], x_prev_out=e["xp"],
                                stream=stream)

    for i in range(args.warmup * NSET):
        call(i)
    torch.cuda.synchronize()
    n = args.steps * 8
    tm = Timer(torch, stream)
    tm.start()
    for i in range(n):
        call(i)
    ms = tm.stop_ms()
    per = ms / n
    elems = B * T * C
    if backward:
        # x and the M mix gradients in, dx out; mu in, dmu out; the carried
        # token's gradient in, d_x_prev out
        algo = (8 + 4 * M) * elems + 8 * M * C + 8 * B * C
        kname = f"shift_bwd_kernel<wkv::IoF32, 4, {M}>"
    else:
        # x in, M outputs out; mu; carried token in and out
        algo = (4 + 4 * M) * elems + 4 * M * C + 8 * B * C
        kname = f"shift_kernel<wkv::IoF32, 4, {M}>"
    wl = "token_shift_bwd" if backward else "token_shift"
    cpu = None
    if not args.no_cpu_baseline:
        import oracle

        def one(i):
            if i >= NSET:
                return None
            e = sets[i]
            a = [e[nm].double().cpu().numpy() for nm in ("mu", "x", "xp")]
            if backward:
                dd, dp = e["d"].double().cpu().numpy(), e["dxpo"].double().cpu().numpy()
                t0 = time.perf_counter()
                oracle.token_shift_backward(*a, dd, dp)
            else:
                t0 = time.perf_counter()
                oracle.token_shift(*a)
            return elems, time.perf_counter() - t0

        done, secs, calls = timed_oracle(one, args.cpu_seconds)
        cpu = {"value": done / secs, "unit": "tok·ch/s", "cores": 1, "kind": "oracle",
               "sample": f"{calls} of the 4 input sets (B=8 T=1024 C=2048, M=3), float64 "
                         f"loop on 1 thread ({secs:.1f} s)"}
    metric = "token shift tokens·channels/sec, B=8 T=1024 C=2048, 3 mixes, fp32"
    if backward:
        metric = metric.replace("token shift", "token shift backward")
    return {"metric": metric,
            "value": elems / (per * 1e-3), "unit": "tok·ch/s", "n_gpus": 1, "steps": n,
            "warmup": args.warmup * NSET, "ms_per_step": per, "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "f32",
            "data": "synthetic (seeded; x, x_prev ~ N(0,1), mu ~ U(0,1))",
            "config": {"workload": wl, "B": B, "T": T, "C": C, "mixes": M,
                       "kernel": kname},
            "roofline": {"bound": "hbm", "achieved": algo / (per * 1e-3) / 1e9,
                         "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": algo / (per * 1e-3) / 1e9 / PEAK_HBM_GBS,
                         "traffic": measured_traffic(kname, wl),
                         "algorithmic_bytes_per_launch": algo, "avg_launch_us": per * 1e3},
            "cpu_baseline": cpu}


def bench_copy(args, torch, wkv, synth):
    """A plain device-to-device copy of 1 GiB (torch's copy kernel): the
    reference for scaling the HBM byte counters (FETCH_SIZE, WRITE_SIZE) read
    by rocprofv3, since its algorithmic traffic is known exactly."""
    n = (1 << 30) // 4
    dev = torch.device("cuda")
    stream = torch.cuda.current_stream()
    x = torch.empty(n, device=dev).uniform_()
    y = torch.empty_like(x)
    for _ in range(args.warmup):
        y.copy_(x)
    torch.cuda.synchronize()
    tm = Timer(torch, stream)
    tm.start()
    for _ in range(args.steps):
        y.copy_(x)
    ms = tm.stop_ms() / args.steps
    algo = 2 * 4 * n
    return {"metric": "device copy GB/s (1 GiB read + 1 GiB written)",
            "value": algo / (ms * 1e-3) / 1e9, "unit": "GB/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
            "data": "synthetic", "config": {"workload": "copy", "bytes_read": 4 * n,
                                            "bytes_written": 4 * n}}


def other_configs(args, torch, wkv, synth):
    """The other workloads' figures beside the headline, each timed the way
    its own --workload run times it (fewer steps, no CPU baseline): the stream
    chunks, the batched decode step, and the stability forward and backward."""
    import copy
    res = {}
    for name, fn, steps in (("stream", bench_stream, 2), ("decode", bench_decode, 4),
                            ("stability_fwd", lambda a, t, w, s: bench_stability(a, t, w, s, False), 5),
                            ("stability_bwd", lambda a, t, w, s: bench_stability(a, t, w, s, True), 5)):
        a = copy.copy(args)
        a.steps, a.warmup, a.no_cpu_baseline = steps, 1, True
        torch.cuda.empty_cache()
        log(f"other configs: {name}")
        r = fn(a, torch, wkv, synth)
        rf = r["roofline"]
        res[name] = {"metric": r["metric"], "value": r["value"], "unit": r["unit"],
                     "kernel": r["config"].get("kernel"),
                     "avg_launch_us": rf["avg_launch_us"], "hbm_gbs": rf["achieved"],
                     "frac": rf["frac"],
                     "traffic_x_algorithmic": (rf["traffic"] / rf["algorithmic_bytes_per_launch"]
                                               if rf.get("traffic") else None),
                     "timed_steps": r["steps"]}
    torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="gpt",
                    choices=["gpt", "gpt_gated", "gpt_bf16", "gpt_f16", "stream", "decode",
                             "decode_gated", "stability_fwd", "stability_bwd",
                             "stability_bwd_state", "stability_bwd_bf16", "stability_fwd_ckpt",
                             "stability_bwd_ckpt", "stability_bwd_ckpt_bf16",
                             "stability_bwd_gated_ckpt", "token_shift", "token_shift_bwd",
                             "copy"])
    ap.add_argument("--plan", type=int, nargs="+", default=None,
                    metavar="N", help="force a forward kernel: KERNEL SEGMENTS SEG_LEN [CHANNELS] "
                    "(wkv_forward_ex plan)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--headline-only", action="store_true",
                    help="gpt workload: skip the other workloads' summary (other_configs)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU (--gpus 1): the WKV lanes are independent, so the "
              "operator shards across GPUs without communication, and libwkv has no multi-GPU "
              "path to measure.", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("no HIP device visible", file=sys.stderr)
        sys.exit(1)
    from linear_recurrent_attention_amd import synth, wkv
    wkv.load_library()
    fn = {"gpt": bench_gpt, "stream": bench_stream, "decode": bench_decode, "copy": bench_copy,
          "gpt_gated": lambda a, t, w, s: bench_gpt(a, t, w, s, True),
          "gpt_bf16": lambda a, t, w, s: bench_gpt(a, t, w, s, False, "bf16"),
          "gpt_f16": lambda a, t, w, s: bench_gpt(a, t, w, s, False, "f16"),
          "decode_gated": lambda a, t, w, s: bench_decode(a, t, w, s, True),
          "token_shift": bench_shift,
          "token_shift_bwd": lambda a, t, w, s: bench_shift(a, t, w, s, True),
          "stability_fwd": lambda a, t, w, s: bench_stability(a, t, w, s, False),
          "stability_bwd": lambda a, t, w, s: bench_stability(a, t, w, s, True),
          "stability_bwd_state": lambda a, t, w, s: bench_stability(a, t, w, s, True, True),
          "stability_bwd_bf16": lambda a, t, w, s: bench_stability(a, t, w, s, True, False,
                                                                   "bf16"),
          "stability_fwd_ckpt": lambda a, t, w, s: bench_stability(a, t, w, s, False,
                                                                   ckpt=True),
          "stability_bwd_ckpt": lambda a, t, w, s: bench_stability(a, t, w, s, True, ckpt=True),
          "stability_bwd_ckpt_bf16": lambda a, t, w, s: bench_stability(a, t, w, s, True, False,
                                                                        "bf16", ckpt=True),
          "stability_bwd_gated_ckpt": lambda a, t, w, s: bench_stability(a, t, w, s, True,
                                                                         ckpt=True, gated=True),
          }[args.workload]
    torch.cuda.synchronize()
    out = fn(args, torch, wkv, synth)
    if args.workload == "gpt" and not args.headline_only:
        out["other_configs"] = other_configs(args, torch, wkv, synth)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
