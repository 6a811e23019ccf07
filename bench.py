#!/usr/bin/env python3
"""Benchmark of the looped gated-delta-rule (GDN) mixer on one MI355X.

One step = one gdn_loop_prefill call: T = 4 weight-tied loops, each running the projection GEMM with its
fused epilogue and the gate launch, the chunk prep and the carry (the sequential state chain with the chunk
outputs and the loop residual computed a chunk behind inside the same workgroups), over the 4096-token,
16-head, width-2048 bf16 prompt (B=1, L=4096, H=16, dk=dv=128, T=4, alpha in (0.9, 1)).  Inputs are seeded
synthetic draws (synth.prefill_inputs) resident in HBM before timing starts.

Printed (one JSON line on stdout): prefill tokens/s (tokens of the prompt per second, each token passing all
4 loops), the roofline of the dominant kernel (the projection GEMM, bf16 MFMA) from the HIP start/stop events
carried on its dispatches inside the timed region, the CPU oracle timed on the same workload, and a secondary
measurement of batched decode (64 sequences x 256 generated tokens, 4 loop states each; HBM-bound).

Usage: python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-decode] [--no-cpu-baseline]
       python bench.py --calib-copy          (plain 256 MiB device copy, for HBM counter calibration)
Only one GPU is used: --gpus N with N > 1 exits with a message.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "looped-GDN prefill tokens/s (×T=4) and decode tokens/s; % MFMA / HBM roofline"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E, published
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = ["proj_gemm.hip", "scan_chunk.hip", "decode.hip", "gdn_device.h"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "looped_linear_attention_amd", "csrc", name)) as f:
            text = f.read()
        # code only: comments and blank lines do not change what the counters measured
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        h.update("\n".join(ln.rstrip() for ln in text.splitlines() if ln.strip()).encode())
    return h.hexdigest()[:16]


def proj_flops_per_token(w) -> int:
    """Algorithmic flops of one loop's projection per token: 2 d (H (2 dk + dv) + 2 H)."""
    return 2 * w.d * (w.H * (2 * w.dk + w.dv) + 2 * w.H)


def proj_gemm_kernel(w, tokens):
    """(kernel name, algorithmic flops per token) of the projection GEMM launch in the looped prefill: bf16
    inputs of 1024 or more tokens take k_proj_wide, which also forms the 2H gate pre-activations (as partial
    sums that the chunk preparation adds up) when 2H <= 32, and leaves them to their own launch otherwise."""
    if w.act == "bf16" and tokens >= 1024:
        gate_cols = 2 * w.H if 2 * w.H <= 32 else 0
        return "k_proj_wide", 2 * w.d * (w.H * (2 * w.dk + w.dv) + gate_cols)
    return ("k_proj_bf16" if w.act == "bf16" else "k_proj_f32"), proj_flops_per_token(w)


def proj_weight_bytes(w) -> int:
    """Bytes of the packed bf16 projection weights [d, H (2 dk + dv) + 2 H], read once per loop."""
    return 2 * w.d * (w.H * (2 * w.dk + w.dv) + 2 * w.H)


def scan_flops_per_token(w, C=64) -> int:
    """Algorithmic flops of one loop's chunkwise scan per token (all heads): H (C (3 dk + 2 dv) + 6 dk dv)."""
    return w.H * (C * (3 * w.dk + 2 * w.dv) + 6 * w.dk * w.dv)


def decode_bytes_per_launch(N, H, D, act_bytes=2) -> int:
    """Algorithmic HBM bytes of one decode launch: state read + write, q/k/v, alpha/beta, o."""
    return N * H * (2 * D * D * 4 + 3 * D * act_bytes + 2 * 4 + D * 4)


def traffic_for(kernel: str, workload: str):
    """HBM bytes per launch measured by rocprofv3 counters for this kernel build, or None if stale/absent."""
    try:
        with open(PROFILE_TRAFFIC) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    ent = data.get(f"{kernel}@{workload}")
    if not ent or ent.get("source_hash") != kernel_source_hash():
        return None
    return ent.get("bytes_per_launch")


def bench_prefill(args, w, torch, gl, synth):
    dev = lambda t: t.contiguous().to("cuda")
    x = synth.prefill_inputs(w)
    desc = gl.make_desc(w.B, w.L, w.H, w.dk, w.dv, T=w.T, act=w.act, alpha_lo=w.alpha_lo)
    Wp = torch.empty(gl.gdn_weights_packed_bytes(desc) // (4 if w.act == "f32" else 2),
                     dtype=desc.act_dtype, device="cuda")
    gl.gdn_weights_pack(desc, dev(x["Wq"]), dev(x["Wk"]), dev(x["Wv"]), dev(x["wa"]), dev(x["wb"]), Wp)
    h0, rho = dev(x["h0"]), dev(x["rho"])
    ws = gl.workspace(desc, gl.GDN_OP_LOOP_PREFILL)
    h_out = torch.empty(w.B, w.L, w.d, device="cuda")
    stream = torch.cuda.current_stream()

    def step():
        gl.gdn_loop_prefill(desc, h0, Wp, rho, h_out, None, None, ws, stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    stages = {"project": gl.GDN_STAGE_PROJECT, "gates": gl.GDN_STAGE_GATES, "scan_prep": gl.GDN_STAGE_SCAN_PREP,
              "scan_carry": gl.GDN_STAGE_SCAN_CARRY}

    def timed_pass(names, stride=1):
        """args.steps steps with the dispatch events of the named stages armed on every stride-th launch;
        (ms total, wall s, per-stage)."""
        timers = {k: gl.gdn_timer_create(stages[k], args.steps * w.T) for k in names}
        for t in timers.values():
            gl.gdn_timer_set_stride(t, stride)
            gl.gdn_timer_attach(t)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        wall0 = time.perf_counter()
        e0.record(stream)
        for _ in range(args.steps):
            step()
        e1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - wall0
        gl.gdn_timer_detach()
        ms_total = e0.elapsed_time(e1)
        per_stage = {}
        for k, t in timers.items():
            n, ms = gl.gdn_timer_read(t)
            if n:   # the gate stage has no launch when the GEMM forms the gates
                per_stage[k] = dict(launches=n, avg_ms=ms / n, share=ms / ms_total)
            gl.gdn_timer_destroy(t)
        return ms_total, wall, per_stage

    # The timed region carries dispatch events on every fifth projection GEMM launch only (each armed dispatch
    # costs the GPU a few microseconds; 5 is coprime to the 4 loops, so the sample covers every loop evenly); the
    # per-stage breakdown comes from a second pass with every launch of every stage armed.
    stride = 5 if args.steps * w.T >= 20 else 1
    ms_total, wall, timed_stages = timed_pass(["project"], stride)
    _, _, per_stage = timed_pass(list(stages))
    per_stage["project"] = timed_stages["project"]
    ms_step = ms_total / args.steps
    tokens = w.B * w.L
    for v in per_stage.values():
        v["share"] = v["avg_ms"] * w.T / ms_step
    return dict(ms_step=ms_step, wall_s=wall, tokens=tokens, per_stage=per_stage)


def bench_decode(args, torch, gl, synth):
    w = synth.workload("decode_n64_s256")
    steps = args.decode_steps
    log(f"decode: generating inputs for {w.B} sequences x {steps} steps x {w.T} loops ...")
    states = synth.decode_state_init(w).to("cuda")
    q, k, v, al, be = [], [], [], [], []
    for item in synth.decode_step_inputs(w, steps):
        q.append(item["q"]); k.append(item["k"]); v.append(item["v"])
        al.append(item["alpha"]); be.append(item["beta"])
    Q = torch.stack(q).to("cuda"); K = torch.stack(k).to("cuda"); V = torch.stack(v).to("cuda")
    A = torch.stack(al).to("cuda"); Bt = torch.stack(be).to("cuda")
    del q, k, v, al, be
    desc = gl.make_desc(w.B, 1, w.H, w.dk, w.dv, T=1, act=w.act)
    o = torch.empty(w.B, w.H, w.dv, device="cuda")
    stream = torch.cuda.current_stream()
    S = [states[t].contiguous() for t in range(w.T)]

    # per-launch views made once, outside the timed region
    qs, ks, vs, als, bes = (list(t.unbind(0)) for t in (Q, K, V, A, Bt))

    def run():
        i = 0
        for s in range(steps):
            for tau in range(w.T):
                gl.gdn_scan_decode(desc, qs[i], ks[i], vs[i], als[i], bes[i], S[tau], o, stream)
                i += 1

    run()  # warm-up run
    torch.cuda.synchronize()
    # whole runs without the stage timer (an armed launch costs a few microseconds of its own)
    times = []
    for rep in range(3):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        run()
        e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    # then one run with every k_decode launch timed by the library's dispatch events
    timer = gl.gdn_timer_create(gl.GDN_STAGE_DECODE, steps * w.T)
    gl.gdn_timer_attach(timer)
    run()
    torch.cuda.synchronize()
    gl.gdn_timer_detach()
    n, ms = gl.gdn_timer_read(timer)
    gl.gdn_timer_destroy(timer)
    ms_run = statistics.median(times)
    avg_launch_ms = ms / max(n, 1)
    bpl = decode_bytes_per_launch(w.B, w.H, w.dk)
    gbs = bpl / (avg_launch_ms * 1e-3) / 1e9
    return {
        "workload": "decode_n64_s256", "sequences": w.B, "steps": steps, "loops": w.T,
        "value": w.B * steps / (ms_run * 1e-3), "unit": "tokens/s", "ms_per_run": ms_run,
        "roofline": {"bound": "hbm", "kernel": "k_decode", "achieved": gbs, "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS,
                     "traffic": traffic_for("k_decode", "decode_n64_s256"),
                     "bytes_per_launch": bpl, "avg_launch_us": avg_launch_ms * 1e3},
    }


def cpu_baseline(w, synth):
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # threadpoolctl missing: report OpenMP threads only
        blas_threads = 1
    x = synth.prefill_inputs(w)
    runs, t0 = 0, time.perf_counter()
    while True:   # whole runs of the full workload until at least 10 s of CPU work
        oracle.loop_prefill(x["h0"], x["Wq"], x["Wk"], x["Wv"], x["wa"], x["wb"], x["rho"], w.H, w.dk, w.dv,
                            w.alpha_lo, w.act)
        runs += 1
        dt = time.perf_counter() - t0
        if dt >= 10.0:
            break
    cores = max(oracle.num_threads(), blas_threads)
    return {"value": runs * w.B * w.L / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"the full {w.name} workload ({w.B * w.L} tokens x {w.T} loops), {runs} run(s) in "
                      f"{dt:.1f} s (fp64: numpy/OpenBLAS projections, C/OpenMP recurrence)"}


def calib_copy(torch):
    n = 256 << 20
    a = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"calib_copy_bytes": n, "launches": 5}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="prefill_b1_l4096")
    ap.add_argument("--decode-steps", type=int, default=256)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calib-copy", action="store_true")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus > 1 or world > 1:
        print(f"bench.py measures one GPU only (asked for {max(args.gpus, world)}): the looped GDN path here "
              "runs on a single MI355X; multi-GPU sharding is a design note, not a measured path.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    if args.calib_copy:
        calib_copy(torch)
        return
    import looped_linear_attention_amd as gl
    import synth
    gl.load()
    w = synth.workload(args.workload)
    log(f"prefill: {w.name}, warmup {args.warmup}, steps {args.steps}")
    pf = bench_prefill(args, w, torch, gl, synth)
    proj = pf["per_stage"]["project"]
    kname, kflops = proj_gemm_kernel(w, pf["tokens"])
    flops_launch = kflops * pf["tokens"]
    achieved = flops_launch / (proj["avg_ms"] * 1e-3) / 1e12
    traffic = traffic_for(kname, w.name)
    total_flops = (proj_flops_per_token(w) + scan_flops_per_token(w)) * w.T * pf["tokens"]
    out = {
        "metric": METRIC,
        "value": pf["tokens"] / (pf["ms_step"] * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": pf["ms_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.act,
        "data": "synthetic (seeded Gaussian inputs and random-init weights of the workload's shape)",
        "config": {"workload": w.name, "B": w.B, "L": w.L, "H": w.H, "dk": w.dk, "dv": w.dv, "d": w.d,
                   "T": w.T, "chunk": 64, "alpha_lo": w.alpha_lo},
        "roofline": {"bound": "mfma", "kernel": kname, "achieved": achieved,
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                     "traffic": traffic, "flops_per_launch": flops_launch,
                     "avg_launch_us": proj["avg_ms"] * 1e3},
        "whole_path": {"algorithmic_tflops": total_flops / (pf["ms_step"] * 1e-3) / 1e12,
                       "frac_of_bf16_peak": total_flops / (pf["ms_step"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                       "loop_tokens_per_s": w.T * pf["tokens"] / (pf["ms_step"] * 1e-3),
                       "stages": {k: {"avg_launch_us": v["avg_ms"] * 1e3, "share_of_step": v["share"]}
                                  for k, v in pf["per_stage"].items()}},
    }
    if not args.no_decode:
        out["decode"] = bench_decode(args, torch, gl, synth)
    if not args.no_cpu_baseline:
        log("cpu baseline: running the oracle ...")
        out["cpu_baseline"] = cpu_baseline(w, synth)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out))


if __name__ == "__main__":
    main()
