"""Benchmark of the weight-only block-INT4 MatMul on one MI355X.

Headline workload: the Qwen3-4B-shaped INT4 decode step (M = 1, fp32
activations, block 128, default zero point 8): 36 layers x {fused QKV
2560->6144, o 4096->2560, gate||up 2560->19456, down 9728->2560} + LM head
2560->151936 = 145 launches over 2,136,832,000 bytes of packed weights and
scales.  One step = that whole sequence, replayed as one captured HIP graph on
one stream; inputs are seeded synthetic tensors already resident in HBM (the
step streams 2.1 GB, more than the 256 MB last-level cache, so every step is
cold).  value = packed-weight bytes per step / step time (GB/s).

The timed region is exactly --steps graph replays between two HIP events on
the launch stream, bracketed by device synchronizations; a second pass of at
least 60 replays, each between its own pair of events, gives the p50 / min /
max and the raw samples.  The same protocol times the other workloads in
``extra``: the Qwen3-4B prefill step (2048 bf16 rows, the MFMA bar) with its
own roofline block, the Qwen3-0.6B decode and prefill steps, the single
1024->3072 GEMV cold (rotating over 512 copies, 1 GB) and hot, the plain
streaming read of 1 GB (achievable HBM, the control arm), each distinct
projection of the headline step alone, cold, beside a plain read of its bytes
(``decode_projections``: the per-launch floor of moving those bytes), and
``next_rows``:
small M (4, 8, 16 rows), the tied LM head with greedy ArgMax and the
embedding gather, the QDQ import, and the fused gate||up SiLU GEMV against the
unfused pair.

roofline: every launch of the headline step is the decode GEMV; its
algorithmic bytes per launch (packed weights + scales + zero points, averaged
over the step's launches) are divided by its average launch duration, the
event-timed step over the number of launches.  cpu_baseline: the CPU oracle
(fp64, as it is) timed on the host on a bounded sample of the same step, on
all the cores the process may use and on one core, with the CPU model.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--config C]
"""

from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E peak, GB/s (datasheet)
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA peak, TFLOP/s (datasheet)
METRIC = "INT4 GEMV weight GB/s (% HBM peak) at M=1; prefill TFLOP/s (% MFMA peak)"
MIN_SAMPLES = 60


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def time_runs(run, steps, warmup, samples=MIN_SAMPLES):
    """Exactly `steps` calls of run() between two HIP events on the current
    stream (device synchronized before and after), then `samples` calls each
    between its own pair of events.  Returns ms per call and the samples."""
    import torch
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(steps):
        run()
    e1.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    ms = e0.elapsed_time(e1) / steps
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(samples + 1)]
    ev[0].record()
    for i in range(samples):
        run()
        ev[i + 1].record()
    torch.cuda.synchronize()
    raw = [ev[i].elapsed_time(ev[i + 1]) for i in range(samples)]
    return ms, wall, raw


def sample_stats(raw, digits=5):
    return {"n": len(raw), "p50_ms": round(statistics.median(raw), digits),
            "min_ms": round(min(raw), digits), "max_ms": round(max(raw), digits),
            "raw_ms": [round(x, digits) for x in raw]}


# ---- CPU baseline: the oracle as it stands, timed on the host ----------------

def _oracle_args(w, i, rows):
    import numpy as np
    import torch
    from workloads.generate import projection_inputs
    inp = projection_inputs(w, i, 0, "cpu")
    a = inp.a[:rows] if rows is not None else inp.a
    f32 = w.act_dtype == "f32"
    act = a.numpy() if f32 else a.view(torch.int16).numpy().view(np.uint16)
    sc = inp.scales.numpy() if f32 else inp.scales.view(torch.int16).numpy().view(np.uint16)
    return (act, inp.q.numpy(), None if inp.zp is None else inp.zp.numpy(), sc,
            None if inp.bias is None else inp.bias.numpy())


def cpu_baseline(cfg, budget_s, threads, rows=None):
    """The oracle on `threads` host threads: the step's launches in order,
    repeated until `budget_s` of oracle time is spent (input generation is not
    timed).  Decode steps: full columns, every row.  Prefill steps: `rows` of
    the M rows, the rate extrapolated to all M rows (labelled so)."""
    import oracle
    from workloads import workload

    w = workload(cfg)
    orc = oracle.get()
    r = w.M if rows is None else min(rows, w.M)
    done_bytes = done_flops = 0
    spent = 0.0
    calls = 0
    first = last = None
    cache, cached = {}, 0
    while spent < budget_s:
        for i, L in enumerate(w.launches):
            args = cache.get(i) or _oracle_args(w, i, r)
            if i not in cache and cached + args[1].nbytes < (2 << 30):
                cache[i] = args
                cached += args[1].nbytes
            t0 = time.perf_counter()
            orc.matmul(args[0], args[1], args[2], args[3], w.block_size, bias=args[4], nthreads=threads)
            spent += time.perf_counter() - t0
            done_bytes += w.weight_bytes(L)
            done_flops += 2 * r * L.K * L.N
            calls += 1
            first = first or L.name
            last = L.name
            if spent >= budget_s:
                break
    n = len(w.launches)
    what = f"{calls} launches ({calls / n:.2f} passes over the step's {n}, {first}..{last})"
    if w.M == 1:
        return {"value": done_bytes / spent / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
                "sample": f"{what}, full columns, M=1", "seconds": round(spent, 2)}
    return {"value": done_flops / spent / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{what}, {r} of {w.M} rows, full columns; rate extrapolated to all {w.M} rows "
                      f"(the oracle's cost is linear in rows)", "extrapolated": True,
            "seconds": round(spent, 2)}


def cpu_baselines(cfg, budget_s, rows=None):
    """All cores the process may use, and one core; with the CPU model."""
    cores = len(os.sched_getaffinity(0))
    log(f"[bench] cpu baseline config {cfg}: oracle on {cores} threads, then 1")
    allc = cpu_baseline(cfg, budget_s, cores, rows)
    one = cpu_baseline(cfg, budget_s, 1, rows)
    allc["one_core"] = {k: one[k] for k in ("value", "unit", "sample", "seconds")}
    allc["cpu_model"] = cpu_model()
    allc["host_cpus_visible"] = os.cpu_count()
    return allc


# ---- GPU measurements -------------------------------------------------------

def measure_step(w, steps, warmup, samples=MIN_SAMPLES, persistent=True):
    """Build one step of workload w (weights packed on the GPU), capture it
    as one graph and time its replays; for a decode step also the eager
    (sequence driver) step and the step as one persistent launch.  The
    launch order of a traced run is: one eager step, warmup + steps + samples
    graph replays, then (decode) warmup + steps eager steps and warmup +
    steps persistent launches."""
    import torch
    from weight_only_int4_matmulnbits_amd.step import Step

    log(f"[bench] {w.title} (M={w.M}): building ({len(w.launches)} launches)")
    step = Step(w, "cuda", seed=0)
    step.run()
    torch.cuda.synchronize()
    step.capture()
    ms, wall, raw = time_runs(step.replay, steps, warmup, samples)
    log(f"[bench] {w.title}: {ms:.4f} ms/step graph-replayed (p50 {statistics.median(raw):.4f})")
    out = {"ms_per_step": ms, "wall_ms_per_step": wall, "samples": sample_stats(raw),
           "launches": step.launches, "weight_bytes": step.weight_bytes, "flops": w.step_flops(),
           "pack_ms": step.pack_seconds * 1e3, "workspace_bytes": step.sequence.workspace_bytes}
    if w.M == 1:
        ms_e, _, _ = time_runs(step.run, steps, warmup, 0)
        out["eager_ms_per_step"] = ms_e
    if w.M == 1 and persistent:
        # the same step as one persistent launch (mnb_step_*), for comparison
        step.make_persistent()
        ms_p, _, _ = time_runs(step.launch_persistent, steps, warmup, 0)
        step.persistent.check()
        out["persistent_ms_per_step"] = ms_p
        log(f"[bench] {w.title}: {ms_p:.4f} ms/step as one persistent launch")
    step.close()
    del step
    torch.cuda.empty_cache()
    return out


def trace_persistent(cfg, launches=5):
    """Where the time of the persistent decode step goes: one traced launch
    (after `launches` untraced ones) of the step as a single mnb_step launch,
    from the phase timestamps every workgroup's control wavefront records
    (mnb_step_set_trace).  Per projection kind, means over its projections of
    the median over workgroups of: the wait (from the last workgroup's
    arrival after the previous projection to the poll that sees it), the row
    staging, the compute phase (row staged to the workgroup's sums complete),
    the output store and its acknowledgement, and the projection's span
    (last arrival to last arrival)."""
    import numpy as np
    import torch
    from weight_only_int4_matmulnbits_amd.step import Step
    from workloads import workload

    w = workload(cfg)
    st = Step(w, "cuda", seed=0)
    p = st.make_persistent()
    for _ in range(launches):
        st.launch_persistent()
    tr = p.trace_buffer()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    st.launch_persistent()
    e1.record()
    p.check()
    t = tr.cpu().numpy().astype(np.float64) / 100.0          # microseconds (100 MHz)
    t -= t[:, 0, 0].min()
    arrive = t[:, :, 4].max(axis=0)
    names = [L.name.split(".")[-1] for L in w.launches]
    rows = {}
    for i in range(len(names)):
        wait = t[:, i, 1] - arrive[i - 1] if i else np.zeros(t.shape[0])
        rows.setdefault(names[i], []).append(
            (np.median(wait), np.median(t[:, i, 2] - t[:, i, 1]), np.median(t[:, i, 3] - t[:, i, 2]),
             np.median(t[:, i, 4] - t[:, i, 3]), arrive[i] - (arrive[i - 1] if i else 0.0)))
    out = [f"{w.title}: one persistent launch {e0.elapsed_time(e1) * 1e3:.1f} us (event-timed, traced), "
           f"{t.shape[0]} workgroups, {len(names)} projections; last arrival at {arrive[-1]:.1f} us",
           f"{'projection':10} {'count':>5} {'wait':>7} {'stage':>7} {'compute':>8} {'store':>7} {'span':>7}  (us)"]
    for k, v in rows.items():
        a = np.array(v).mean(axis=0)
        out.append(f"{k:10} {len(v):5d} " + " ".join(f"{x:7.2f}" for x in a))
    st.close()
    return "\n".join(out)


def measured_traffic(cfg, kind):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when there is none for this workload or the kernel sources changed
    since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)[kind]
        h = hashlib.sha256()
        for src in rec["sources"]:
            with open(os.path.join(ROOT, src), "rb") as f:
                h.update(f.read())
        if h.hexdigest() != rec["kernel_sha256"]:
            return None
        return rec[f"config{cfg}"]["traffic_bytes_per_launch"]
    except (OSError, KeyError, ValueError):
        return None


def roofline_for(w, r):
    """Decode: every launch of the step is the decode GEMV, so its average
    launch duration is the event-timed step over the step's launches, and
    its algorithmic bytes per launch are the step's weight bytes over the
    same count.  Prefill: the same with 2*M*K*N flop, a launch being one
    projection (the GEMM and, where K is split, its reduction)."""
    avg_s = r["ms_per_step"] * 1e-3 / r["launches"]
    if w.M == 1:
        per_launch = r["weight_bytes"] / r["launches"]
        achieved = per_launch / avg_s / 1e9
        return {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS, "traffic": measured_traffic(w.cfg, "gemv"),
                "kernel": "gemv_kernel (every launch of the step)",
                "algorithmic_bytes_per_launch": per_launch, "avg_launch_us": avg_s * 1e6}
    per_launch = r["flops"] / r["launches"]
    achieved = per_launch / avg_s / 1e12
    return {"bound": "mfma", "achieved": achieved, "peak": BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": achieved / BF16_PEAK_TFLOPS,
            "traffic": measured_traffic(w.cfg, "gemm"),
            "kernel": ("gemm_bf16_wide_kernel + split-K/tail reductions (every projection of the step)"
                       if w.act_dtype == "bf16" else
                       "gemm_f32_int_kernel + split-K reductions (every projection of the step)"),
            "algorithmic_flops_per_launch": per_launch, "avg_launch_us": avg_s * 1e6}


def summary(w, r, with_samples=True):
    s = {"workload": w.title, "config_index": w.cfg, "M": w.M, "ms_per_step": round(r["ms_per_step"], 5),
         "launches": r["launches"], "workspace_bytes": r["workspace_bytes"]}
    if w.M == 1:
        s["weight_GBps"] = r["weight_bytes"] / (r["ms_per_step"] * 1e-3) / 1e9
        s["hbm_frac"] = s["weight_GBps"] / HBM_PEAK_GBS
        s["eager_ms_per_step"] = round(r["eager_ms_per_step"], 5)
        if "persistent_ms_per_step" in r:
            s["persistent_ms_per_step"] = round(r["persistent_ms_per_step"], 5)
            s["persistent_weight_GBps"] = r["weight_bytes"] / (r["persistent_ms_per_step"] * 1e-3) / 1e9
    else:
        s["TFLOPs"] = r["flops"] / (r["ms_per_step"] * 1e-3) / 1e12
        s["mfma_frac"] = s["TFLOPs"] / BF16_PEAK_TFLOPS
    s["avg_launch_us"] = r["ms_per_step"] * 1e3 / r["launches"]
    if with_samples:
        s["samples"] = r["samples"]
    s["roofline"] = roofline_for(w, r)
    return s


def probe_lib():
    import ctypes
    import torch  # noqa: F401  -- the HIP runtime torch loaded comes first
    path = os.path.join(ROOT, "weight_only_int4_matmulnbits_amd", "libmnb_probe.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build first")
    L = ctypes.CDLL(path)
    L.mnb_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
    L.mnb_probe_stream_read.restype = ctypes.c_int
    return L


def measure_control_read(steps, warmup, nbytes=1 << 30):
    """Achievable HBM: a plain 16-byte non-temporal streaming read of 1 GiB
    (libmnb_probe), the same protocol as the steps."""
    import ctypes
    import torch
    L = probe_lib()
    buf = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    sink = torch.zeros(1024, dtype=torch.int32, device="cuda")
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def run():
        rc = L.mnb_probe_stream_read(ctypes.c_void_p(buf.data_ptr()), nbytes, ctypes.c_void_p(sink.data_ptr()), st)
        if rc != 0:
            raise RuntimeError(f"probe read failed: {rc}")

    ms, _, raw = time_runs(run, steps, warmup)
    del buf, sink
    torch.cuda.empty_cache()
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"workload": "plain streaming read of 1 GiB, 16-byte non-temporal loads (libmnb_probe)",
            "bytes": nbytes, "ms": ms, "GBps": gbs, "frac_of_datasheet_peak": gbs / HBM_PEAK_GBS,
            "samples": {k: v for k, v in sample_stats(raw).items() if k != "raw_ms"}}


def measure_config1(steps, warmup, copies=512):
    """The single 1024->3072 GEMV: cold, one graph of `copies` launches each
    on its own copy of the weights (1 GB in all, more than the last-level
    cache), and hot, the same launches on one copy."""
    import torch
    import weight_only_int4_matmulnbits_amd as mnb
    from workloads import workload
    from workloads.generate import projection_inputs

    w = workload(1)
    inp = projection_inputs(w, 0, 0, "cuda")
    pw = mnb.PackedWeight.from_logical(inp.q, inp.scales, inp.zp, inp.bias, block_size=w.block_size)
    y = torch.empty(1, 3072, device="cuda")
    cold = [mnb.PackedWeight(pw.K, pw.N, pw.block_size, pw.act_dtype, pw.b_packed.clone(), pw.scales.clone())
            for _ in range(copies)]
    out = {"workload": f"{w.title} (fp32, block 32, default zero point)", "weight_bytes": pw.weight_bytes}
    for name, ws in (("cold", cold), ("hot", [pw] * copies)):
        seq = mnb.Sequence([(x, inp.a, y) for x in ws])
        seq.capture()
        ms, _, raw = time_runs(seq.replay, max(3, steps // 10), max(2, warmup // 2), 10)
        us = ms * 1e3 / copies
        out[name] = {"us_per_launch": us, "GBps": pw.weight_bytes / (us * 1e-6) / 1e9,
                     "launches_per_graph": copies,
                     "copies": len({id(x) for x in ws}),
                     "p50_us_per_launch": statistics.median(raw) * 1e3 / copies}
        seq.close()
    out["hbm_frac_cold"] = out["cold"]["GBps"] / HBM_PEAK_GBS
    del cold, pw
    torch.cuda.empty_cache()
    return out


def measure_decode_projections(steps, warmup, cfg=4, min_bytes=600 << 20):
    """Each distinct projection of a decode step alone, cold: a graph of
    back-to-back decode GEMV launches, each on its own copy of the weights
    (together more than the last-level cache), and beside it a graph of plain
    16-byte streaming reads of the same number of bytes from the same number
    of distinct buffers (libmnb_probe).  The read is the floor of a launch
    that only moves the projection's bytes; the GEMV's excess over it is what
    the unpacking, the dot products, the reductions and the stores add."""
    import ctypes
    import math
    import torch
    import weight_only_int4_matmulnbits_amd as mnb
    from workloads import workload
    from workloads.generate import projection_inputs

    L = probe_lib()
    w = workload(cfg)
    first = {}
    for i, launch in enumerate(w.launches):
        first.setdefault(launch.name.split(".")[-1], i)
    out = {"workload": f"{w.title}: each distinct projection alone, cold (one graph of launches on "
                       f"distinct copies, at least {min_bytes >> 20} MiB in all)"}
    sink = torch.zeros(1024, dtype=torch.int32, device="cuda")
    for kind, i in first.items():
        inp = projection_inputs(w, i, 0, "cuda")
        pw = mnb.PackedWeight.from_logical(inp.q, inp.scales, inp.zp, inp.bias, block_size=w.block_size)
        nbytes = pw.weight_bytes
        copies = max(3, math.ceil(min_bytes / nbytes))
        ws = [pw] + [mnb.PackedWeight(pw.K, pw.N, pw.block_size, pw.act_dtype, pw.b_packed.clone(),
                                      pw.scales.clone(), None if pw.zp_packed is None else pw.zp_packed.clone(),
                                      pw.bias) for _ in range(copies - 1)]
        y = torch.empty(1, pw.N, dtype=inp.a.dtype, device="cuda")
        seq = mnb.Sequence([(x, inp.a, y) for x in ws])
        seq.capture()
        ms_g, _, raw_g = time_runs(seq.replay, max(3, steps // 10), max(2, warmup // 2), 10)
        seq.close()
        del seq, ws, y
        torch.cuda.empty_cache()
        # the same bytes read by the probe, each launch from its own buffer
        rb = (nbytes + 255) // 256 * 256
        buf = torch.ones(copies * rb // 4, dtype=torch.float32, device="cuda")
        cs = torch.cuda.Stream()
        cs.wait_stream(torch.cuda.current_stream())
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cs):
            h = ctypes.c_void_p(cs.cuda_stream)
            for c in range(copies):
                rc = L.mnb_probe_stream_read(ctypes.c_void_p(buf.data_ptr() + c * rb), nbytes // 16 * 16,
                                             ctypes.c_void_p(sink.data_ptr()), h)
                if rc != 0:
                    raise RuntimeError(f"probe read failed: {rc}")
        ms_r, _, raw_r = time_runs(g.replay, max(3, steps // 10), max(2, warmup // 2), 10)
        del g, buf
        torch.cuda.empty_cache()
        gemv_us, read_us = ms_g * 1e3 / copies, ms_r * 1e3 / copies
        out[kind] = {"K": pw.K, "N": pw.N, "weight_bytes": nbytes, "copies": copies,
                     "gemv_us": gemv_us, "gemv_GBps": nbytes / (gemv_us * 1e-6) / 1e9,
                     "gemv_p50_us": statistics.median(raw_g) * 1e3 / copies,
                     "read_us": read_us, "read_GBps": (nbytes // 16 * 16) / (read_us * 1e-6) / 1e9,
                     "read_p50_us": statistics.median(raw_r) * 1e3 / copies,
                     "gemv_over_read": gemv_us / read_us}
        log(f"[bench] {kind}: gemv {gemv_us:.2f} us vs read {read_us:.2f} us ({nbytes / 1e6:.2f} MB)")
        del pw, inp
        torch.cuda.empty_cache()
    del sink
    return out


def graph_time_us(fn, steps, warmup, reps=20):
    """Average device time of one fn() call: reps calls captured back to back
    in one graph (a graph of one short kernel is bound by the host's launch
    rate), replayed; HIP events on the replay stream."""
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for _ in range(reps):
            fn()
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / (steps * reps)


def measure_next_rows(steps, warmup, only=None):
    """One measurement per row beyond the decode / prefill step: the small-M
    steps (speculative blocks of 4, 8 and 16 rows), the LM head with greedy
    ArgMax and the tied-embedding gather, the QDQ import, and the fused
    gate||up SiLU GEMV against its unfused pair.  `only`: the names of the
    rows to run (all when None)."""
    import torch
    import weight_only_int4_matmulnbits_amd as mnb
    from workloads import workload
    from workloads.generate import random_inputs

    out = {}

    def want(name):
        return only is None or name in only

    # f1: the 0.6B decode step with 4, 8 and 16 rows per projection, each
    # also as a multiple of the same step at one row (measured here too)
    if want("small_m"):
        sm = {}
        for M in (1, 4, 8, 16):
            wm = workload(2, M=M)
            r = measure_step(wm, steps, warmup, 20)
            gbs = r["weight_bytes"] / (r["ms_per_step"] * 1e-3) / 1e9
            sm[f"M{M}"] = {"workload": f"Qwen3-0.6B-shaped INT4 step, {M} rows (speculative block)",
                           "ms_per_step": r["ms_per_step"], "p50_ms": r["samples"]["p50_ms"],
                           "launches": r["launches"], "weight_GBps": gbs, "hbm_frac": gbs / HBM_PEAK_GBS,
                           "rows_per_s": M / (r["ms_per_step"] * 1e-3)}
            if M > 1:
                sm[f"M{M}"]["x_one_row"] = r["ms_per_step"] / sm["M1"]["ms_per_step"]
        out["small_m"] = sm
    # f2: LM head (tied weight, N = vocabulary) + greedy token, and the gather
    if want("lm_head_argmax"):
        K, N, bs = 1024, 151936, 32
        g = random_inputs(K, N, 1, bs, "f32", True, False, seed=1).to("cuda")
        pw = mnb.PackedWeight.from_logical(g.q, g.scales, g.zp, block_size=bs)
        logits = torch.empty(1, N, device="cuda")
        tok = torch.empty(1, dtype=torch.int64, device="cuda")
        aws = mnb.workspace(mnb.argmax_workspace_bytes(1, N))
        ids1 = torch.tensor([151935], device="cuda")
        ids512 = torch.randint(0, N, (512,), device="cuda", generator=torch.Generator("cuda").manual_seed(2))
        rows1 = torch.empty(1, K, device="cuda")
        rows512 = torch.empty(512, K, device="cuda")
        t_lm = graph_time_us(lambda: pw.matmul(g.a, out=logits), steps, warmup)
        t_lm_arg = graph_time_us(lambda: (pw.matmul(g.a, out=logits), mnb.argmax(logits, out=tok, workspace=aws)),
                                 steps, warmup)
        t_g1 = graph_time_us(lambda: mnb.gather_rows(ids1, pw.b_packed, pw.scales, pw.zp_packed, K=K, N=N,
                                                     block_size=bs, out=rows1), steps, warmup)
        t_g512 = graph_time_us(lambda: mnb.gather_rows(ids512, pw.b_packed, pw.scales, pw.zp_packed, K=K, N=N,
                                                       block_size=bs, out=rows512), steps, warmup)
        row_read = K // 2 + (K // bs) * 4 + (K // bs + 1) // 2
        out["lm_head_argmax"] = {
            "workload": "Qwen3-0.6B tied LM head 1024->151936 (fp32, block 32, zero points) + greedy ArgMax",
            "lm_head_us": t_lm, "lm_head_GBps": pw.weight_bytes / (t_lm * 1e-6) / 1e9,
            "lm_head_plus_argmax_us": t_lm_arg, "argmax_added_us": t_lm_arg - t_lm}
        out["embedding_gather"] = {
            "workload": "rows of the same packed tied weight, fp32 out",
            "rows_1_us": t_g1, "rows_512_us": t_g512,
            "rows_512_GBps": 512 * (row_read + 4 * K) / (t_g512 * 1e-6) / 1e9}
        del pw, logits, rows512, aws
    # f3: QDQ import of the 4B gate||up weight (axis 0 -> N-major)
    if want("qdq_import"):
        K, N, bs = 2560, 19456, 128
        gen = torch.Generator("cuda").manual_seed(3)
        w_q = torch.randint(0, 256, (K * N // 2,), dtype=torch.uint8, device="cuda", generator=gen)
        z_q = torch.randint(0, 256, ((K // bs) * N // 2,), dtype=torch.uint8, device="cuda", generator=gen)
        s_q = torch.rand((K // bs) * N, device="cuda", generator=gen).to(torch.bfloat16)
        mnb.import_qdq(w_q, s_q, z_q, K=K, N=N, block_size=bs, axis=0)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(5):
            mnb.import_qdq(w_q, s_q, z_q, K=K, N=N, block_size=bs, axis=0)
        e1.record()
        torch.cuda.synchronize()
        t_imp = e0.elapsed_time(e1) * 1e3 / 5
        moved = 2 * (w_q.numel() + z_q.numel() + 2 * s_q.numel())
        out["qdq_import"] = {"workload": "Qwen3-4B gate||up 2560x19456 QDQ (axis 0, block 128) -> MatMulNBits",
                             "us": t_imp, "GBps_read_plus_written": moved / (t_imp * 1e-6) / 1e9,
                             "tied_lm_head_copy_avoided": mnb.qdq_is_native(1024, 151936, 32, axis=1)}
        del w_q, z_q, s_q
    # f4: gate||up with silu(gate) * up fused, against the unfused pair
    if want("gate_up_silu"):
        fused = {}
        for name, K, I, bs, dt in (("0.6B", 1024, 3072, 32, "f32"), ("4B", 2560, 9728, 128, "f32")):
            g = random_inputs(K, 2 * I, 1, bs, dt, name == "0.6B", False, seed=4).to("cuda")
            pw = mnb.PackedWeight.from_logical(g.q, g.scales, g.zp, block_size=bs)
            y = torch.empty(1, 2 * I, dtype=g.a.dtype, device="cuda")
            h = torch.empty(1, I, dtype=g.a.dtype, device="cuda")

            def unfused():
                pw.matmul(g.a, out=y)
                torch.mul(torch.nn.functional.silu(y[:, :I]), y[:, I:], out=h)

            t_u = graph_time_us(unfused, steps, warmup)
            t_f = graph_time_us(lambda: mnb.gemv_silu_mul(g.a, pw.b_packed, pw.scales, pw.zp_packed, K=K,
                                                          N=2 * I, block_size=bs, out=h), steps, warmup)
            fused[name] = {"K": K, "I": I, "dtype": dt, "unfused_us": t_u, "fused_us": t_f,
                           "fused_GBps": pw.weight_bytes / (t_f * 1e-6) / 1e9}
            del pw, y, h, g
        out["gate_up_silu"] = fused
    # f4: RMSNorm fused into the decode projection input (Qwen3-4B qkv),
    # against torch's normalization followed by the GEMV
    if want("rmsnorm_gemv"):
        K, N, bs = 2560, 6144, 128
        g = random_inputs(K, N, 1, bs, "f32", False, False, seed=6).to("cuda")
        pw = mnb.PackedWeight.from_logical(g.q, g.scales, block_size=bs)
        gamma = torch.rand(K, device="cuda") + 0.5
        xn = torch.empty_like(g.a)
        y = torch.empty(1, N, device="cuda")

        def unfused_n():
            torch.mul(g.a * torch.rsqrt(g.a.pow(2).mean(-1, keepdim=True) + 1e-6), gamma, out=xn)
            pw.matmul(xn, out=y)

        t_u = graph_time_us(unfused_n, steps, warmup)
        t_f = graph_time_us(lambda: mnb.gemv_rmsnorm(g.a, gamma, 1e-6, pw.b_packed, pw.scales, K=K, N=N,
                                                     block_size=bs, out=y), steps, warmup)
        t_p = graph_time_us(lambda: pw.matmul(g.a, out=y), steps, warmup)
        out["rmsnorm_gemv"] = {"workload": "Qwen3-4B qkv 2560->6144 (fp32, block 128) on an RMS-normalized row",
                               "unfused_us": t_u, "fused_us": t_f, "plain_gemv_us": t_p}
        del pw, g, gamma, xn, y
    # f4 at prefill: the Qwen3-4B gate||up at 2048 bf16 rows, the gated
    # epilogue in the prefill kernel against the product then torch's SiLU and
    # multiply (the unfused graph)
    if want("gate_up_silu_prefill"):
        M, K, I, bs = 2048, 2560, 9728, 128
        g = random_inputs(K, 2 * I, M, bs, "bf16", True, True, seed=5).to("cuda")
        pw = mnb.PackedWeight.from_logical(g.q, g.scales, g.zp, g.bias, block_size=bs)
        y = torch.empty(M, 2 * I, dtype=torch.bfloat16, device="cuda")
        h = torch.empty(M, I, dtype=torch.bfloat16, device="cuda")
        ws_u = mnb.workspace(mnb.workspace_bytes(pw.desc, M))
        ws_f = mnb.workspace(mnb.gemm_silu_workspace_bytes(pw.desc, M))

        def unfused_p():
            pw.matmul(g.a, out=y, workspace=ws_u)
            torch.mul(torch.nn.functional.silu(y[:, :I]), y[:, I:], out=h)

        def fused_p():
            mnb.gemm_silu_mul(g.a, pw.b_packed, pw.scales, pw.zp_packed, pw.bias, K=K, N=2 * I,
                              block_size=bs, out=h, workspace=ws_f)

        t_u = graph_time_us(unfused_p, max(5, steps // 2), warmup, reps=4)
        t_f = graph_time_us(fused_p, max(5, steps // 2), warmup, reps=4)
        fl = 2 * M * K * 2 * I
        out["gate_up_silu_prefill"] = {
            "workload": "Qwen3-4B gate||up 2560->2x9728 at 2048 bf16 rows, block 128, zero points, bias",
            "unfused_us": t_u, "fused_us": t_f, "fused_TFLOPs": fl / (t_f * 1e-6) / 1e12,
            "output_bytes_unfused": M * 2 * I * 2, "output_bytes_fused": M * I * 2}
        del pw, y, h, g, ws_u, ws_f
    torch.cuda.empty_cache()
    return out


# ---- rocprofv3 summaries (run on the CSV output of the commands in
# profiles/; nothing here touches the GPU) ----

def _read_csv(path):
    import csv
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _library_rows(rows):
    # dispatches of this library's per-projection kernels (packing and the
    # persistent step kernel, timed after the steps, excluded)
    return [r for r in rows if "mnb::" in r["Kernel_Name"] and "pack_" not in r["Kernel_Name"]
            and "step_kernel" not in r["Kernel_Name"]]


def _short(name):
    name = name.replace("mnb::(anonymous namespace)::", "").replace("(GemvArgs)", "").replace("(Bf16Args)", "")
    return name.replace("void ", "")


def summarize_trace(trace_dir, cfg, steps, warmup, samples=MIN_SAMPLES, bench_json=None, rows=None):
    """Per-kernel statistics and the timed graph-replayed steps of one
    `bench.py --config cfg --steps steps --warmup warmup --samples samples
    --no-extra` run under `rocprofv3 --kernel-trace --stats` (with `--rows
    rows` when given); with the JSON line that run printed, the tracer's
    overhead against its untraced event-timed step."""
    from workloads import workload
    import statistics
    w = workload(cfg, M=rows) if rows else workload(cfg)
    n = len(w.launches)
    rows = _library_rows(_read_csv(os.path.join(trace_dir, "run_kernel_trace.csv")))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    stats = _read_csv(os.path.join(trace_dir, "run_kernel_stats.csv"))
    out = ["kernel statistics (run_kernel_stats.csv, library matmul kernels):"]
    for r in stats:
        if "mnb::" in r["Name"] and "pack_" not in r["Name"]:
            out.append(f"  {_short(r['Name']):<62} calls {int(r['Calls']):6d}  avg {float(r['AverageNs']) / 1e3:9.3f} us"
                       f"  min {float(r['MinNs']) / 1e3:8.3f}  max {float(r['MaxNs']) / 1e3:8.3f}")
    # the run (measure_step): one eager step, `warmup` + `steps` + `samples`
    # graph replays, then for a decode step `warmup` + `steps` eager steps;
    # kernels per step = dispatches / steps
    total_steps = 1 + warmup + steps + samples + ((warmup + steps) if w.M == 1 else 0)
    per_step = len(rows) // total_steps
    out.append(f"library dispatches in trace: {len(rows)} ({total_steps} steps x {per_step})")
    def span_stats(rng):
        sums, spans, durs = [], [], []
        for k in rng:
            st = rows[k * per_step:(k + 1) * per_step]
            d = [int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in st]
            sums.append(sum(d))
            durs.extend(d)
            spans.append(int(st[-1]["End_Timestamp"]) - int(st[0]["Start_Timestamp"]))
        return statistics.median(sums), statistics.median(spans), statistics.mean(durs) / 1e3
    timed = range(1 + warmup, 1 + warmup + steps)
    s_sum, s_span, avg = span_stats(timed)
    out.append(f"timed graph-replayed steps: median sum of kernel durations {s_sum / 1e3:.1f} us, "
               f"first-start to last-end {s_span / 1e3:.1f} us")
    if w.M == 1:
        # Back to back in a replayed graph, the tracer stamps about half of
        # the kernels as starting exactly when the previous one ends and puts
        # ~3.7 us gaps before the others, so those durations are not a
        # kernel's own.  In the eager steps every kernel runs alone (host
        # launch gaps of several us), which gives its duration undisturbed.
        e_timed = range(1 + 2 * warmup + steps + samples, 1 + 2 * warmup + 2 * steps + samples)
        e_sum, e_span, e_avg = span_stats(e_timed)
        out.append(f"timed eager steps: median sum of kernel durations {e_sum / 1e3:.1f} us "
                   f"(first-start to last-end {e_span / 1e3:.1f} us, host launch gaps included)")
        per = w.step_weight_bytes() / n
        out.append(f"average kernel duration, eager steps: {e_avg:.3f} us over {n} launches per step -> "
                   f"{per / (e_avg * 1e-6) / 1e9:.1f} GB/s of algorithmic bytes per launch")
        out.append(f"average kernel duration, graph-replayed steps (tracer-stamped): {avg:.3f} us")
    else:
        # per projection: the GEMM plus its reduction, medians over the timed steps
        names = [L.name.split(".")[-1] for L in w.launches]
        kinds = sorted(set(names), key=names.index)
        k0 = 1 + warmup
        per = {}
        for k in timed:
            st = rows[k * per_step:(k + 1) * per_step]
            i = 0
            for L, nm in zip(w.launches, names):
                g = int(st[i]["End_Timestamp"]) - int(st[i]["Start_Timestamp"])
                i += 1
                red = 0
                while i < len(st) and "reduce" in st[i]["Kernel_Name"]:
                    red += int(st[i]["End_Timestamp"]) - int(st[i]["Start_Timestamp"])
                    i += 1
                per.setdefault(nm, []).append((g, red, 2 * w.M * L.K * L.N, w.weight_bytes(L)))
        for nm in kinds:
            v = per[nm]
            g = statistics.median(x[0] for x in v) / 1e3
            r = statistics.median(x[1] for x in v) / 1e3
            fl, wb = v[0][2], v[0][3]
            out.append(f"  {nm:<8} GEMM {g:9.2f} us ({fl / (g * 1e-6) / 1e12:7.1f} TFLOP/s, weights "
                       f"{wb / (g * 1e-6) / 1e9:7.1f} GB/s)  reduction {r:6.1f} us")
        out.append(f"average launch (GEMM + reduction) {s_sum / 1e3 / n:.3f} us over {n} launches per step")
    if bench_json:
        with open(bench_json) as f:
            rec = json.loads([l for l in f if l.startswith("{")][-1])
        un = rec["ms_per_step"] * 1e3
        out.append(f"event timing printed by the same run (bench JSON; HIP events, taken while the tracer "
                   f"ran): {un:.1f} us per graph-replayed step; the median sum of traced kernel durations, "
                   f"{s_sum / 1e3:.1f} us, is {'within' if s_sum / 1e3 <= un else 'above'} it "
                   f"({100 * (s_sum / 1e3 / un - 1):+.1f} %)")
    return "\n".join(out)


def traffic_from(fetch_dir, write_dir, cfg, copy_mib, kind="gemv"):
    """HBM bytes per library dispatch from `--pmc FETCH_SIZE` and `--pmc
    WRITE_SIZE` runs of `bench.py --config cfg --copy-calibration copy_mib`:
    each counter is scaled by known bytes / its reading for the plain copy
    kernel of the same run.  Updates profiles/traffic.json (with the hash of
    the kernel sources the counters were taken with) and returns the text."""
    import hashlib
    from workloads import workload
    w = workload(cfg)
    known = copy_mib << 20
    res, lines = {}, []
    for name, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = [r for r in _read_csv(os.path.join(d, "run_counter_collection.csv")) if r["Counter_Name"] == name]
        cal = [float(r["Counter_Value"]) for r in rows if "copyBuffer" in r["Kernel_Name"]]
        lib_rows = _library_rows(rows)
        lib = [float(r["Counter_Value"]) for r in lib_rows]
        factor = known / (max(cal) * 1024.0)
        if w.M == 1:
            # decode: one dispatch per launch of the step
            n_units, unit = len(lib), "dispatch"
        else:
            # prefill: a projection is its product kernel plus any split-K or
            # tail reduction (and gated-row) dispatches; count the products
            n_units = sum(1 for r in lib_rows if "reduce" not in r["Kernel_Name"]
                          and "silu_mul_rows" not in r["Kernel_Name"])
            unit = "projection"
        per = sum(lib) / n_units * 1024.0 * factor
        res[name] = (per, factor)
        over = "" if w.M == 1 else f" over {n_units} {unit}s"
        lines.append(f"{name}: copy of {copy_mib} MiB: counter {max(cal):.1f} KiB -> factor {factor:.3f}; "
                     f"{len(lib)} dispatches{over}, {sum(lib) / n_units:.1f} KiB raw -> "
                     f"{per / 1e6:.4f} MB per {unit}")
    tot = res["FETCH_SIZE"][0] + res["WRITE_SIZE"][0]
    if w.M == 1:
        alg = w.step_weight_bytes() / len(w.launches)
        lines.append(f"HBM traffic per launch {tot / 1e6:.4f} MB vs algorithmic {alg / 1e6:.4f} MB "
                     f"({tot / alg:.3f}x)")
    else:
        # a prefill projection must read A and the packed weight once and write Y once
        esz = 4 if w.act_dtype == "f32" else 2
        alg = sum(w.weight_bytes(L) + esz * w.M * (L.K + L.N) for L in w.launches) / len(w.launches)
        lines.append(f"HBM traffic per projection {tot / 1e6:.4f} MB (reductions included) vs the minimum "
                     f"(A + packed weight read once, Y written once) {alg / 1e6:.4f} MB ({tot / alg:.3f}x)")
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        rec = {}
    srcs = {"gemv": ["weight_only_int4_matmulnbits_amd/csrc/mnb_gemv.hip",
                     "weight_only_int4_matmulnbits_amd/csrc/mnb_gemv_kernel.h",
                     "weight_only_int4_matmulnbits_amd/csrc/mnb_gemv_f32.hip",
                     "weight_only_int4_matmulnbits_amd/csrc/mnb_gemv_bf16.hip",
                     "weight_only_int4_matmulnbits_amd/csrc/mnb_gemv_core.h",
                     "weight_only_int4_matmulnbits_amd/csrc/mnb_internal.h"],
            "gemm": ["weight_only_int4_matmulnbits_amd/csrc/mnb_gemm.hip",
                     "weight_only_int4_matmulnbits_amd/csrc/mnb_internal.h"]}[kind]
    h = hashlib.sha256()
    for src in srcs:
        with open(os.path.join(ROOT, src), "rb") as f:
            h.update(f.read())
    ent = rec.get(kind, {})
    if ent.get("kernel_sha256") != h.hexdigest():
        ent = {}
    ent.update({"kernel_sha256": h.hexdigest(), "sources": srcs})
    ent[f"config{cfg}"] = {"traffic_bytes_per_launch": tot, "fetch_bytes_per_launch": res["FETCH_SIZE"][0],
                           "write_bytes_per_launch": res["WRITE_SIZE"][0], "fetch_factor": res["FETCH_SIZE"][1],
                           "write_factor": res["WRITE_SIZE"][1]}
    rec[kind] = ent
    rec["note"] = ("HBM bytes per launch from rocprofv3 --pmc FETCH_SIZE and --pmc WRITE_SIZE runs (KiB per "
                   "dispatch summed over the run and divided by its decode dispatches, or by its prefill "
                   "projections, whose split-K and tail reductions count with them), each scaled by known "
                   "bytes / the counter's reading for one plain device-to-device copy "
                   "(__amd_rocclr_copyBuffer) in the same run.  Valid only while the kernel sources hash to "
                   "kernel_sha256; written by bench.py --traffic-from.")
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
    return "\n".join(lines)


def counters_from(dirs, cus=256):
    """Per-kernel averages of the counters of one or more rocprofv3 `--pmc`
    runs (run_counter_collection.csv), library kernels and the plain copy of
    --copy-calibration, plus the derived
    fractions that need them.  GRBM_GUI_ACTIVE is summed over the chip's 8
    XCDs, so the kernel's own active cycles are GRBM_GUI_ACTIVE / 8; MFMA busy =
    SQ_VALU_MFMA_BUSY_CYCLES (summed over every SIMD) / (those cycles x CUs x 4
    SIMDs), wait = SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES, LDS bank conflicts per
    LDS instruction."""
    import collections
    per = collections.defaultdict(lambda: collections.defaultdict(list))
    for d in dirs:
        for r in _read_csv(os.path.join(d, "run_counter_collection.csv")):
            name = r["Kernel_Name"]
            if "copyBuffer" in name:
                name = "copy (reference for scaling byte counters)"
            elif "mnb::" not in name or "pack_" in name:
                continue
            else:
                name = _short(name)
            per[name][r["Counter_Name"]].append(float(r["Counter_Value"]))
    out = []
    for k, cs in sorted(per.items(), key=lambda kv: -len(next(iter(kv[1].values())))):
        n = max(len(v) for v in cs.values())
        avg = {c: sum(v) / len(v) for c, v in cs.items()}
        out.append(f"{k}  ({n} dispatches)")
        for c in sorted(avg):
            out.append(f"    {c:<28} {avg[c]:16.1f}")
        if "SQ_VALU_MFMA_BUSY_CYCLES" in avg and "GRBM_GUI_ACTIVE" in avg and avg["GRBM_GUI_ACTIVE"] > 0:
            active = avg["GRBM_GUI_ACTIVE"] / 8
            out.append(f"    -> {active:.0f} active cycles per XCD; MFMA busy "
                       f"{100 * avg['SQ_VALU_MFMA_BUSY_CYCLES'] / (active * cus * 4):.1f} % "
                       f"of {cus} CUs x 4 SIMDs over them")
        if "SQ_WAIT_INST_ANY" in avg and avg.get("SQ_WAVE_CYCLES", 0) > 0:
            out.append(f"    -> waiting on any instruction {100 * avg['SQ_WAIT_INST_ANY'] / avg['SQ_WAVE_CYCLES']:.1f} % "
                       f"of wave cycles")
        if "SQ_LDS_BANK_CONFLICT" in avg and avg.get("SQ_INSTS_LDS", 0) > 0:
            out.append(f"    -> {avg['SQ_LDS_BANK_CONFLICT'] / avg['SQ_INSTS_LDS']:.3f} LDS bank-conflict cycles "
                       f"per LDS instruction")
    return "\n".join(out)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=60)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=4)
    ap.add_argument("--samples", type=int, default=MIN_SAMPLES,
                    help="individually timed replays for p50/min/max (at least 60 by default)")
    ap.add_argument("--no-extra", action="store_true", help="headline config only")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=6.0,
                    help="seconds of oracle time per policy (all cores, one core) for the headline")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="also run one plain device-to-device copy of MIB MiB, the "
                         "reference for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE")
    ap.add_argument("--summarize-trace", metavar="DIR",
                    help="print the summary of a rocprofv3 --kernel-trace --stats run of this "
                         "bench (same --config/--steps/--warmup/--samples) and exit; no GPU is used")
    ap.add_argument("--bench-json", metavar="FILE",
                    help="with --summarize-trace: the JSON line the traced run printed, to state "
                         "the tracer's overhead against the same run's untraced timing")
    ap.add_argument("--next-rows", nargs="+", metavar="ROW",
                    help="run only these rows of extra.next_rows (small_m, lm_head_argmax, "
                         "qdq_import, gate_up_silu, rmsnorm_gemv, gate_up_silu_prefill), print "
                         "them as one JSON line and exit (for profiling one row)")
    ap.add_argument("--decode-projections", action="store_true",
                    help="decode configs: each distinct projection alone, cold, beside a plain read "
                         "of its bytes (extra.decode_projections); print it as one JSON line and exit")
    ap.add_argument("--rows", type=int, metavar="M",
                    help="profiling: the config's step with M rows per projection (implies --no-extra "
                         "and --no-cpu-baseline; also for --summarize-trace)")
    ap.add_argument("--no-persistent", action="store_true",
                    help="decode configs: do not time the step as one persistent launch (profiling "
                         "runs: rocprofv3 can end with a segmentation fault after cooperative launches)")
    ap.add_argument("--trace-step", action="store_true",
                    help="decode configs: print where the time of the persistent step launch goes "
                         "(phase timestamps of every workgroup) and exit")
    ap.add_argument("--counters-from", nargs="+", metavar="DIR",
                    help="per-kernel averages of rocprofv3 --pmc runs of this bench and exit; no GPU")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="derive HBM bytes per launch from rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE "
                         "runs of this bench (same --config, --copy-calibration), update "
                         "profiles/traffic.json and exit; no GPU is used")
    args = ap.parse_args()
    if args.rows:
        args.no_extra = args.no_cpu_baseline = True
    if args.summarize_trace:
        print(summarize_trace(args.summarize_trace, args.config, args.steps, args.warmup, args.samples,
                              args.bench_json, args.rows))
        return
    if args.counters_from:
        print(counters_from(args.counters_from))
        return
    if args.traffic_from:
        from workloads import workload
        kind = "gemv" if workload(args.config).M == 1 else "gemm"
        print(traffic_from(args.traffic_from[0], args.traffic_from[1], args.config,
                           args.copy_calibration or 256, kind))
        return
    if args.gpus != 1:
        print(f"bench.py: this build computes on exactly one GPU; --gpus {args.gpus} is not "
              "supported (the path has no multi-GPU sharding: every box here has one GPU)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    from workloads import workload

    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] copy calibration: {n} bytes read, {n} bytes written")
        del src, dst

    if args.trace_step:
        print(trace_persistent(args.config), flush=True)
        return

    if args.decode_projections:
        print(json.dumps(measure_decode_projections(args.steps, args.warmup, args.config)), flush=True)
        return

    if args.next_rows:
        rows = measure_next_rows(max(10, args.steps // 3), max(2, args.warmup // 2), only=set(args.next_rows))
        print(json.dumps(rows), flush=True)
        return

    w = workload(args.config, M=args.rows) if args.rows else workload(args.config)
    r = measure_step(w, args.steps, args.warmup, args.samples, persistent=not args.no_persistent)
    dec = w.M == 1
    value = (r["weight_bytes"] / (r["ms_per_step"] * 1e-3) / 1e9 if dec
             else r["flops"] / (r["ms_per_step"] * 1e-3) / 1e12)
    line = {
        "metric": METRIC,
        "value": value,
        "unit": "GB/s" if dec else "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if w.act_dtype == "f32" else "bf16",
        "data": "synthetic",
        "config": {"workload": w.title, "config_index": args.config, "M": w.M,
                   "block_size": w.block_size, "launches": r["launches"],
                   "projections": w.n_projections, "weight_bytes": r["weight_bytes"],
                   "flops": r["flops"], "graph_replay": True},
        "roofline": roofline_for(w, r),
        "samples": r["samples"],
        "wall_ms_per_step": r["wall_ms_per_step"],
        "pack_ms": r["pack_ms"],
    }
    if dec:
        line["eager_ms_per_step"] = r["eager_ms_per_step"]
        if "persistent_ms_per_step" in r:
            line["persistent_ms_per_step"] = r["persistent_ms_per_step"]
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baselines(args.config, args.cpu_budget, rows=None if dec else 2)
    if not args.no_extra:
        extra = {}
        for c in (5, 3, 2):
            if c == args.config:
                continue
            wc = workload(c)
            rc = measure_step(wc, args.steps, args.warmup, args.samples, persistent=not args.no_persistent)
            extra[f"config{c}"] = summary(wc, rc)
            if c in (5, 3) and not args.no_cpu_baseline:
                extra[f"config{c}"]["cpu_baseline"] = cpu_baselines(c, 3.0, rows=2)
        log("[bench] config 1 (cold and hot), the 1 GiB streaming-read control arm")
        extra["config1"] = measure_config1(args.steps, args.warmup)
        extra["control_read"] = measure_control_read(args.steps, args.warmup)
        if dec:
            log("[bench] decode projections alone, cold, beside plain reads of their bytes")
            extra["decode_projections"] = measure_decode_projections(args.steps, args.warmup, args.config)
        ach = extra["control_read"]["GBps"]
        line["roofline"]["achievable_GBps_control"] = ach if dec else None
        if dec:
            line["roofline"]["frac_of_achievable"] = line["roofline"]["achieved"] / ach
        log("[bench] next rows: small M, LM head + argmax, gather, QDQ import, gated gate||up")
        extra["next_rows"] = measure_next_rows(max(10, args.steps // 3), max(2, args.warmup // 2))
        line["extra"] = extra
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
