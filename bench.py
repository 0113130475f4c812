"""Benchmark of the weight-only block-INT4 MatMul on one MI355X.

Headline workload: the Qwen3-0.6B-shaped INT4 decode step (M = 1, fp32
activations, block 32, per-block zero points): 28 layers x {fused QKV
1024->4096, o 2048->1024, gate||up 1024->6144, down 3072->1024} + LM head
1024->151936 = 113 launches over 381,802,496 bytes of packed weights, scales
and zero points.  One step = that whole sequence, replayed as one captured HIP
graph on one stream; inputs are seeded synthetic tensors already resident in
HBM.  value = packed-weight bytes per step / step time (GB/s).

Also printed in the same JSON line (``extra``): the Qwen3-4B decode step and
the two prefill steps (TFLOP/s), the eager (non-graph) decode step time, and
``next_rows``: the 0.6B step with 4 rows (small-M kernel), the tied LM head
with greedy ArgMax and the embedding gather, the QDQ import, and the fused
gate||up SiLU GEMV against the unfused pair.

roofline: the only kernel of the headline step is the decode GEMV; its
algorithmic bytes per launch (packed weights + scales + zero points, averaged
over the step's launches) are divided by its average launch duration, the
event-timed step time (HIP events on the launch stream around the timed graph
replays) over the number of launches.  cpu_baseline: the CPU oracle timed on
the host cores on a bounded sample of the same step.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--config C]
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E peak, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA peak, TFLOP/s
METRIC = "INT4 GEMV weight GB/s (% HBM peak) at M=1; prefill TFLOP/s (% MFMA peak)"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def time_steps(step, steps, warmup, graph):
    import torch
    run = step.replay if graph else step.run
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
    return e0.elapsed_time(e1) / steps, wall


def cpu_baseline(cfg, budget_s):
    """The oracle (as it is) on the host cores: launches of the step in order
    until the time budget is used; returns a dict in the metric's unit."""
    import oracle
    from workloads import workload
    from workloads.generate import projection_inputs
    import numpy as np
    import torch

    w = workload(cfg)
    orc = oracle.get()
    cores = len(os.sched_getaffinity(0))
    done_bytes = done_flops = 0
    spent = 0.0
    names = []
    rows = w.M if w.M == 1 else 2
    for i, L in enumerate(w.launches):
        inp = projection_inputs(w, i, 0, "cpu")
        a = inp.a[:rows]
        act = (a.numpy() if w.act_dtype == "f32"
               else a.view(torch.int16).numpy().view(np.uint16))
        sc = (inp.scales.numpy() if w.act_dtype == "f32"
              else inp.scales.view(torch.int16).numpy().view(np.uint16))
        t0 = time.perf_counter()
        orc.matmul(act, inp.q.numpy(), None if inp.zp is None else inp.zp.numpy(), sc,
                   w.block_size, bias=None if inp.bias is None else inp.bias.numpy(),
                   nthreads=cores)
        spent += time.perf_counter() - t0
        done_bytes += w.weight_bytes(L)
        done_flops += 2 * rows * L.K * L.N
        names.append(L.name)
        if spent >= budget_s:
            break
    if w.M == 1:
        val, unit = done_bytes / spent / 1e9, "GB/s"
        sample = (f"{len(names)} of {len(w.launches)} launches of the step "
                  f"({names[0]}..{names[-1]}), full columns, M=1")
    else:
        val, unit = done_flops / spent / 1e12, "TFLOP/s"
        sample = (f"{len(names)} launches ({names[0]}..{names[-1]}), "
                  f"{rows} of {w.M} rows")
    return {"value": val, "unit": unit, "cores": cores, "kind": "oracle",
            "sample": sample, "seconds": round(spent, 2)}


def measure_config(cfg, steps, warmup, graph=True):
    from workloads import workload
    return measure_config_w(workload(cfg), steps, warmup, graph)


def measure_config_w(w, steps, warmup, graph=True):
    import torch
    from weight_only_int4_matmulnbits_amd.step import Step

    cfg = w.cfg
    log(f"[bench] config {cfg}: {w.title} (M={w.M}): building ({len(w.launches)} launches)")
    step = Step(w, "cuda", seed=0)
    step.run()
    torch.cuda.synchronize()
    if graph:
        step.capture()
    ms, wall = time_steps(step, steps, warmup, graph)
    log(f"[bench] config {cfg}: {ms:.4f} ms/step (graph={graph})")
    out = {"ms_per_step": ms, "wall_ms_per_step": wall, "launches": step.launches,
           "weight_bytes": step.weight_bytes, "flops": w.step_flops(),
           "pack_ms": step.pack_seconds * 1e3}
    if w.M == 1:
        ms_eager, _ = time_steps(step, steps, warmup, False)
        out["eager_ms_per_step"] = ms_eager
    step.close()
    del step
    torch.cuda.empty_cache()
    return w, out


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
    # capture on the warm-up stream: the library's per-stream workspace (used
    # by the argmax partials) exists there, and is not allocated in a capture
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


def measure_next_rows(steps, warmup):
    """One measurement per row beyond the decode / prefill step: the small-M
    step (a speculative block of 4 rows), the LM head with greedy ArgMax and
    the tied-embedding gather, the QDQ import, and the fused gate||up SiLU
    GEMV against its unfused pair."""
    import torch
    import weight_only_int4_matmulnbits_amd as mnb
    from workloads import workload
    from workloads.generate import random_inputs

    out = {}
    # f1: the 0.6B decode step with 4 rows per projection
    w4 = workload(2, M=4)
    _, r = measure_config_w(w4, steps, warmup)
    out["small_m"] = {"workload": "Qwen3-0.6B-shaped INT4 step, 4 rows (speculative block)",
                      "M": 4, "ms_per_step": r["ms_per_step"], "launches": r["launches"],
                      "weight_GBps": r["weight_bytes"] / (r["ms_per_step"] * 1e-3) / 1e9,
                      "hbm_frac": r["weight_bytes"] / (r["ms_per_step"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
                      "rows_per_s": 4 / (r["ms_per_step"] * 1e-3)}
    # f2: LM head (tied weight, N = vocabulary) + greedy token, and the gather
    K, N, bs = 1024, 151936, 32
    g = random_inputs(K, N, 1, bs, "f32", True, False, seed=1).to("cuda")
    pw = mnb.PackedWeight.from_logical(g.q, g.scales, g.zp, block_size=bs)
    logits = torch.empty(1, N, device="cuda")
    tok = torch.empty(1, dtype=torch.int64, device="cuda")
    ids1 = torch.tensor([151935], device="cuda")
    ids512 = torch.randint(0, N, (512,), device="cuda", generator=torch.Generator("cuda").manual_seed(2))
    rows1 = torch.empty(1, K, device="cuda")
    rows512 = torch.empty(512, K, device="cuda")
    t_lm = graph_time_us(lambda: pw.matmul(g.a, out=logits), steps, warmup)
    t_lm_arg = graph_time_us(lambda: (pw.matmul(g.a, out=logits), mnb.argmax(logits, out=tok)),
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
    del pw, logits, rows512
    # f3: QDQ import of the 4B gate||up weight (axis 0 -> N-major)
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
    fused = {}
    for name, K, I, bs, dt in (("0.6B", 1024, 3072, 32, "f32"), ("4B", 2560, 9728, 128, "bf16")):
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
        fused[name] = {"K": K, "I": I, "unfused_us": t_u, "fused_us": t_f,
                       "fused_GBps": pw.weight_bytes / (t_f * 1e-6) / 1e9}
        del pw, y, h, g
    out["gate_up_silu"] = fused
    torch.cuda.empty_cache()
    return out


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
    """The step is nothing but launches of one kernel (the decode GEMV, or the
    prefill GEMM), so its average launch duration is the event-timed step time
    over the launches of the step; this includes the gaps between launches
    inside the replayed graph, which rocprofv3's kernel trace of the same
    command shows to be small."""
    avg_s = r["ms_per_step"] * 1e-3 / r["launches"]
    if w.M == 1:
        per_launch = r["weight_bytes"] / r["launches"]
        achieved = per_launch / avg_s / 1e9
        return {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS, "traffic": measured_traffic(w.cfg, "gemv"),
                "kernel": "gemv_kernel (every launch of the step)",
                "algorithmic_bytes_per_launch": per_launch,
                "avg_launch_us": avg_s * 1e6}
    per_launch = r["flops"] / r["launches"]
    achieved = per_launch / avg_s / 1e12
    return {"bound": "mfma", "achieved": achieved, "peak": BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": achieved / BF16_PEAK_TFLOPS,
            "traffic": measured_traffic(w.cfg, "gemm"),
            "kernel": "gemm_kernel (every launch of the step)",
            "algorithmic_flops_per_launch": per_launch,
            "avg_launch_us": avg_s * 1e6}


def summary(w, r):
    s = {"workload": w.title, "ms_per_step": round(r["ms_per_step"], 5),
         "launches": r["launches"]}
    if w.M == 1:
        s["weight_GBps"] = r["weight_bytes"] / (r["ms_per_step"] * 1e-3) / 1e9
        s["hbm_frac"] = s["weight_GBps"] / HBM_PEAK_GBS
        s["eager_ms_per_step"] = round(r["eager_ms_per_step"], 5)
    else:
        s["TFLOPs"] = r["flops"] / (r["ms_per_step"] * 1e-3) / 1e12
        s["mfma_frac"] = s["TFLOPs"] / BF16_PEAK_TFLOPS
    s["avg_launch_us"] = r["ms_per_step"] * 1e3 / r["launches"]
    return s


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=2)
    ap.add_argument("--no-extra", action="store_true", help="headline config only")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="also run one plain device-to-device copy of MIB MiB, the "
                         "reference for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build runs on exactly one GPU; --gpus {args.gpus} is not "
              "supported (the path has no multi-GPU sharding)", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)

    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] copy calibration: {n} bytes read, {n} bytes written")
        del src, dst

    w, r = measure_config(args.config, args.steps, args.warmup)
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
    }
    line["pack_ms"] = r["pack_ms"]
    if dec:
        line["eager_ms_per_step"] = r["eager_ms_per_step"]
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle)")
        line["cpu_baseline"] = cpu_baseline(args.config, args.cpu_budget)
    if not args.no_extra:
        extra = {}
        for c in (4, 3, 5):
            if c == args.config:
                continue
            st = max(3, args.steps // (10 if c == 5 else 2))
            wc, rc = measure_config(c, st, max(2, args.warmup // 2))
            extra[f"config{c}"] = summary(wc, rc)
        log("[bench] next rows: small M, LM head + argmax, gather, QDQ import, gated gate||up")
        extra["next_rows"] = measure_next_rows(max(5, args.steps // 5), max(2, args.warmup // 2))
        line["extra"] = extra
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
