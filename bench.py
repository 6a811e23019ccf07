#!/usr/bin/env python3
"""Benchmark of the looped gated-delta-rule (GDN) mixer on one MI355X.

One step = one gdn_loop_prefill call: T = 4 weight-tied loops, each running the projection GEMM (which also
forms the gate pre-activations), the chunk prep and the carry (the sequential state chain with the chunk
outputs and the loop residual computed a chunk behind inside the same workgroups).  The headline workload is
the largest single-GPU prompt: 4 sequences of 8192 tokens, 16 heads of 128, width 2048, bf16 inputs with an
fp32 state (B=4, L=8192, T=4).  Inputs are seeded synthetic draws (synth.prefill_inputs) resident in HBM
before timing starts.

Printed (one JSON line on stdout):
  value           prefill tokens/s of the headline workload (tokens of the prompts per second, each token
                  passing all 4 loops), from W warm-up and K timed steps;
  roofline        the dominant kernel (the projection GEMM, bf16 MFMA), from the HIP start/stop events
                  carried on its dispatches inside the timed region;
  roofline_carry  the carry against HBM (algorithmic bytes: q/k/v read, the previous h read, h and its bf16
                  copy written), from a pass with every stage's dispatches timed;
  whole_path      the step's algorithmic flops against the bf16 peak, and the per-stage times;
  extra_workloads the 32768-token prompt and the 4096-token prompt, measured the same way;
  decode          batched decode, 64 sequences x 256 generated tokens, 4 loop states each (the state step
                  alone; HBM-bound);
  loop_decode     the same 64 sequences through whole loops (projection, state step and residual per loop);
  act             the headline workload through gdn_loop_prefill_act (per-token adaptive halting): rate,
                  halting loops, share of position-loops projected;
  scan_backward   gradients of one scan pass at the 4096-token prompt's shape (gdn_scan_backward);
  loop_backward   gradients through the 4 loops of the 4096-token prompt (gdn_loop_backward);
  block           the headline workload through a one-block LT2 stack looped T times (gdn_block_loop_prefill);
  cpu_baseline    the oracle on a bounded sample of the headline workload, on the host's cores.

Usage: python bench.py [--steps K] [--warmup W] [--workload NAME] [--extra NAME,...] [--no-decode] [--only LEG]
                       [--no-act] [--no-block] [--no-backward] [--no-cpu-baseline]
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
PEAK_FP32_TFLOPS = 157.3    # MI355X fp32 vector, published
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "traffic.json")
# the source files each counter-measured kernel is built from: its counters (profiles/traffic.json) stand only
# while these files' code is unchanged
KERNEL_SOURCES = {
    "k_proj_wide": ["proj_gemm.hip", "gdn_device.h"], "k_proj_dpart": ["proj_gemm.hip", "gdn_device.h"],
    "k_scan_prep": ["scan_chunk.hip", "gdn_device.h"], "k_scan_carry": ["scan_chunk.hip", "gdn_device.h"],
    "k_scan_carry_w": ["scan_chunk.hip", "gdn_device.h"], "k_decode": ["decode.hip", "gdn_device.h"],
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash(kernel: str) -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
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


def carry_bytes_per_step(w) -> int:
    """Algorithmic HBM bytes of the T carry launches of one prefill step, per token: q, k, v read; the
    previous loop's h read (loop 1: the bf16 h0, later loops fp32); h written in fp32 and, for loops 1..T-1,
    its bf16 copy for the next loop's projection."""
    ab = 2 if w.act == "bf16" else 4
    qkv = w.H * (2 * w.dk + w.dv) * ab
    total = 0
    for tau in range(w.T):
        h_prev = w.d * (ab if tau == 0 else 4)
        total += qkv + h_prev + w.d * 4 + (w.d * 2 if (w.act == "bf16" and tau < w.T - 1) else 0)
    return total


def carry_kernel(w) -> str:
    """The carry the library launches: 32-column slices (k_scan_carry_w) for bf16 128-wide heads when
    16-column slices would need more than one workgroup per CU, else k_scan_carry."""
    import torch
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    return "k_scan_carry_w" if (w.act == "bf16" and w.dk == 128 and w.B * w.H * (w.dk // 16) > cus) else "k_scan_carry"


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
    if not ent or kernel not in KERNEL_SOURCES or ent.get("source_hash") != kernel_source_hash(kernel):
        return None
    return ent.get("bytes_per_launch")


def bench_prefill(args, w, torch, gl, synth, warmup):
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

    for _ in range(warmup):
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

    # Where gdn_loop_prefill runs this shape as a pipeline over pieces (its automatic setting), the step time is
    # that of the pipelined call, timed with no dispatch events armed; the kernels then share the CUs, so their
    # per-launch times and rooflines come from the same call run loop by loop (gdn_loop_prefill_set_pieces(-1)).
    pipe = None
    piece = gl.gdn_loop_prefill_pieces(desc)
    if piece > 0:
        ms_pipe, wall, _ = timed_pass([])
        gl.gdn_loop_prefill_set_pieces(-1)
        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        per_seq, t0 = 0, 0
        while t0 < w.L:   # the runs gdn_loop_prefill forms: a last run under 1024 tokens joins the one before
            n = min(piece, w.L - t0)
            t0 += n if w.L - (t0 + n) >= 1024 else w.L - t0
            per_seq += 1
        pipe = dict(ms_step=ms_pipe / args.steps, wall_s=wall, piece_tokens=piece, pieces_per_sequence=per_seq)
    try:
        # The timed region carries dispatch events on every fifth projection GEMM launch only (each armed
        # dispatch costs the GPU a few microseconds; 5 is coprime to the 4 loops, so the sample covers every
        # loop evenly); the per-stage breakdown comes from a second pass with every launch of every stage armed.
        stride = 5 if args.steps * w.T >= 20 else 1
        ms_total, wall, timed_stages = timed_pass(["project"], stride)
        _, _, per_stage = timed_pass(list(stages))
    finally:
        gl.gdn_loop_prefill_set_pieces(args.pieces)
    per_stage["project"] = timed_stages["project"]
    ms_step = ms_total / args.steps
    tokens = w.B * w.L
    for v in per_stage.values():
        v["share"] = v["avg_ms"] * w.T / ms_step
    if pipe is None:
        return dict(ms_step=ms_step, wall_s=wall, tokens=tokens, per_stage=per_stage)
    return dict(ms_step=pipe["ms_step"], wall_s=pipe["wall_s"], tokens=tokens, per_stage=per_stage,
                pipeline=dict(piece_tokens=pipe["piece_tokens"], pieces_per_sequence=pipe["pieces_per_sequence"],
                              loop_by_loop_ms_per_step=ms_step))


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


def bench_loop_decode(args, torch, gl, synth, dw):
    """64 sequences through whole loops, one gdn_loop_decode call (T loops: projection, state step, residual)
    per generated token; the token inputs h_t are seeded N(0, 1) draws of width d, resident before timing, and
    the weights those of the 4096-token prompt (same 16 x 128 heads, width 2048)."""
    import numpy as np
    w = synth.workload("prefill_b1_l4096")
    steps = args.decode_steps
    dev = lambda t: t.contiguous().to("cuda")
    x = synth.prefill_inputs(w, L=1)
    desc = gl.make_desc(dw.B, 1, w.H, w.dk, w.dv, T=w.T, act=w.act, alpha_lo=w.alpha_lo)
    Wp = torch.empty(gl.gdn_weights_packed_bytes(desc) // 2, dtype=desc.act_dtype, device="cuda")
    gl.gdn_weights_pack(desc, dev(x["Wq"]), dev(x["Wk"]), dev(x["Wv"]), dev(x["wa"]), dev(x["wb"]), Wp)
    rng = np.random.default_rng(dw.seed + 7)
    hs = torch.from_numpy(rng.standard_normal((steps, dw.B, w.d), dtype=np.float32)).to(torch.bfloat16).to("cuda")
    hts = list(hs.unbind(0))
    rho = dev(x["rho"])
    states = synth.decode_state_init(dw).to("cuda")
    ws = gl.workspace(desc, gl.GDN_OP_LOOP_DECODE)
    h_out = torch.empty(dw.B, w.d, device="cuda")
    stream = torch.cuda.current_stream()

    def run():
        for s in range(steps):
            gl.gdn_loop_decode(desc, hts[s], Wp, rho, states, h_out, ws, stream)

    run()
    torch.cuda.synchronize()
    times = []
    for rep in range(3):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        run()
        e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    ms_run = statistics.median(times)
    tok_s = dw.B * steps / (ms_run * 1e-3)
    # roofline: per generated token, the state traffic of the T loops plus each loop's weight stream shared
    # by the batch
    bytes_tok = decode_bytes_per_launch(dw.B, w.H, w.dk) * w.T / dw.B + w.T * proj_weight_bytes(w) / dw.B
    roof = PEAK_HBM_GBS * 1e9 / bytes_tok
    return {"workload": "decode_n64_s256 with projections", "sequences": dw.B, "steps": steps, "loops": w.T,
            "value": tok_s, "unit": "tokens/s", "ms_per_run": ms_run,
            "roofline": {"bound": "hbm", "bytes_per_token": bytes_tok, "roofline_tokens_per_s": roof,
                         "frac": tok_s / roof}}


def bwd_kernel_flops_per_chunk(D, C=64) -> int:
    """fp32 flops k_bwd_chunk performs per (b, h, chunk): per 16-column block K S, Q S, K dS' (3 C 16 D),
    U = T diag(beta) E and P^T dO (2 C C 16), the dP and dTb sums (2 C C 16), the dQ and dK sums (3 C D 16);
    then T^T dT, dN (2 C^3) and the four (Gam (.) dP / dA) products with K or Q (4 C C D); 2 flops a MAC."""
    blocks = D // 16
    per_block = 3 * C * 16 * D + 2 * C * C * 16 + 2 * C * C * 16 + 3 * C * D * 16
    return 2 * (blocks * per_block + 2 * C ** 3 + 4 * C * C * D)


def bench_backward(args, torch, gl, synth, name="prefill_b1_l4096"):
    """gdn_scan_backward on one scan pass of a prompt workload's shape (q/k/v of unit norm, alpha in
    (alpha_lo, 1), beta in (0, 1), carried initial state, incoming gradients for o and the final state)."""
    w = synth.workload(name)
    B, L, H, D = w.B, w.L, w.H, w.dk
    dev = lambda t: t.contiguous().to("cuda")
    x = synth.scan_inputs(90, B, L, H, D, D, act=w.act, alpha_range=(max(w.alpha_lo, 0.05), 1.0), with_state=True)
    g = synth.grad_inputs(91, B, L, H, D, D)
    desc = gl.make_desc(B, L, H, D, D, T=1, act=w.act)
    ws = gl.workspace(desc, gl.GDN_OP_SCAN_BACKWARD)
    ins = [dev(x[k]) for k in ("q", "k", "v", "alpha", "beta", "s_init")] + [dev(g["d_o"]), dev(g["d_sfinal"])]
    outs = [torch.empty(B, L, H, D, device="cuda") for _ in range(3)] + \
           [torch.empty(B, L, H, device="cuda") for _ in range(2)] + [torch.empty(B, H, D, D, device="cuda")]
    stream = torch.cuda.current_stream()

    def call():
        gl.gdn_scan_backward(desc, *ins, *outs, ws, stream)

    for _ in range(max(args.warmup, 5)):
        call()
    torch.cuda.synchronize()
    n = max(args.steps, 10)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(n):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / n
    stages = {"fwd_prep": gl.GDN_STAGE_SCAN_PREP, "fwd_carry": gl.GDN_STAGE_SCAN_CARRY,
              "bwd_ops": gl.GDN_STAGE_BWD_OPS, "bwd_carry": gl.GDN_STAGE_BWD_CARRY,
              "bwd_chunk": gl.GDN_STAGE_BWD_CHUNK}
    timers = {k: gl.gdn_timer_create(v, n) for k, v in stages.items()}
    for t in timers.values():
        gl.gdn_timer_attach(t)
    for _ in range(n):
        call()
    torch.cuda.synchronize()
    gl.gdn_timer_detach()
    per = {}
    for k, t in timers.items():
        cnt, tot = gl.gdn_timer_read(t)
        per[k] = tot / max(cnt, 1)
        gl.gdn_timer_destroy(t)
    Nc = (L + 63) // 64
    fl = bwd_kernel_flops_per_chunk(D) * B * H * Nc
    ach = fl / (per["bwd_chunk"] * 1e-3) / 1e12
    return {"workload": f"scan backward, {name} shape (B={B}, L={L}, H={H}, dk=dv={D}, {w.act} inputs)",
            "value": B * L / (ms * 1e-3), "unit": "tokens/s", "ms_per_call": ms,
            "stages_us": {k: v * 1e3 for k, v in per.items()},
            "roofline": {"bound": "alu", "kernel": "k_bwd_chunk", "achieved": ach, "peak": PEAK_FP32_TFLOPS,
                         "unit": "TFLOP/s", "frac": ach / PEAK_FP32_TFLOPS, "flops_per_launch": fl,
                         "avg_launch_us": per["bwd_chunk"] * 1e3}}


def bench_act(args, torch, gl, synth, w):
    """gdn_loop_prefill_act on the headline prompt workload: the looped mixer with per-token adaptive halting
    (halting layer from synth.act_inputs).  Reports the throughput, the halting loops and the share of
    position-loops whose projection ran (only positions that ran the previous loop are projected again)."""
    dev = lambda t: t.contiguous().to("cuda")
    x = synth.prefill_inputs(w)
    a = synth.act_inputs(w)
    desc = gl.make_desc(w.B, w.L, w.H, w.dk, w.dv, T=w.T, act=w.act, alpha_lo=w.alpha_lo)
    Wp = torch.empty(gl.gdn_weights_packed_bytes(desc) // (4 if w.act == "f32" else 2),
                     dtype=desc.act_dtype, device="cuda")
    gl.gdn_weights_pack(desc, dev(x["Wq"]), dev(x["Wk"]), dev(x["Wv"]), dev(x["wa"]), dev(x["wb"]), Wp)
    h0, rho, wh = dev(x["h0"]), dev(x["rho"]), dev(a["w_halt"])
    ws = gl.workspace(desc, gl.GDN_OP_LOOP_PREFILL_ACT)
    h_out = torch.empty(w.B, w.L, w.d, device="cuda")
    hl = torch.empty(w.B, w.L, dtype=torch.int32, device="cuda")
    pd = torch.empty(w.B, w.L, device="cuda")
    stream = torch.cuda.current_stream()

    def call():
        gl.gdn_loop_prefill_act(desc, h0, Wp, rho, wh, a["b_halt"], a["eps"], h_out, hl, pd, ws, stream)

    for _ in range(max(args.warmup, 5)):
        call()
    torch.cuda.synchronize()
    n = max(args.steps, 10)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(n):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / n
    loops = hl.cpu().numpy().ravel()
    counts = [int((loops == t).sum()) for t in range(1, w.T + 1)]
    M = w.B * w.L
    # loop 1 projects every position; loop t > 1 those that ran loop t - 1 (not halted before it)
    projected = M + sum(int((loops >= t - 1).sum()) for t in range(2, w.T + 1))
    return {"workload": f"{w.name} with adaptive halting (w_halt ~ N(0, 1/d), b_halt {a['b_halt']}, "
                        f"eps {a['eps']})",
            "value": M / (ms * 1e-3), "unit": "tokens/s", "ms_per_call": ms,
            "halting_loop_counts": counts, "mean_loops": float(loops.mean()),
            "projected_share": projected / (M * w.T)}


def bench_loop_backward(args, torch, gl, synth, name="prefill_b1_l4096"):
    """gdn_loop_backward through the T loops of a prompt workload (the forward's h^(1..T-1) from
    gdn_loop_prefill, a seeded N(0, 1) incoming gradient dL/dh^(T))."""
    w = synth.workload(name)
    B, L, H, D, d, T = w.B, w.L, w.H, w.dk, w.d, w.T
    dev = lambda t: t.contiguous().to("cuda")
    x = synth.prefill_inputs(w)
    desc = gl.make_desc(B, L, H, D, D, T=T, act=w.act, alpha_lo=w.alpha_lo)
    Wp = torch.empty(gl.gdn_weights_packed_bytes(desc) // (4 if w.act == "f32" else 2), dtype=desc.act_dtype,
                     device="cuda")
    gl.gdn_weights_pack(desc, dev(x["Wq"]), dev(x["Wk"]), dev(x["Wv"]), dev(x["wa"]), dev(x["wb"]), Wp)
    h0, rho = dev(x["h0"]), dev(x["rho"])
    h_out = torch.empty(B, L, d, device="cuda")
    h_loops = torch.empty(T, B, L, d, device="cuda")
    gl.gdn_loop_prefill(desc, h0, Wp, rho, h_out, None, h_loops, gl.workspace(desc, gl.GDN_OP_LOOP_PREFILL))
    dh = dev(synth.grad_inputs(92, B, L, H, D, D, with_state_grad=False)["d_o"].reshape(B, L, d))
    ws = gl.workspace(desc, gl.GDN_OP_LOOP_BACKWARD)
    f = dict(device="cuda")
    outs = [torch.empty(B, L, d, **f), torch.empty(d, H * D, **f), torch.empty(d, H * D, **f),
            torch.empty(d, H * D, **f), torch.empty(d, H, **f), torch.empty(d, H, **f), torch.empty(T, d, **f)]
    stream = torch.cuda.current_stream()

    def call():
        gl.gdn_loop_backward(desc, h0, Wp, rho, h_loops, dh, *outs, ws, stream)

    for _ in range(3):
        call()
    torch.cuda.synchronize()
    n = max(min(args.steps, 10), 3)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(n):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / n
    stages = {"gemm": gl.GDN_STAGE_BWD_GEMM, "fwd_prep": gl.GDN_STAGE_SCAN_PREP, "fwd_carry": gl.GDN_STAGE_SCAN_CARRY,
              "bwd_ops": gl.GDN_STAGE_BWD_OPS, "bwd_carry": gl.GDN_STAGE_BWD_CARRY,
              "bwd_chunk": gl.GDN_STAGE_BWD_CHUNK}
    timers = {k: gl.gdn_timer_create(v, 3 * n * T) for k, v in stages.items()}
    for t in timers.values():
        gl.gdn_timer_attach(t)
    for _ in range(n):
        call()
    torch.cuda.synchronize()
    gl.gdn_timer_detach()
    per, tot = {}, {}
    for k, t in timers.items():
        cnt, total = gl.gdn_timer_read(t)
        per[k] = total / max(cnt, 1)
        tot[k] = total / n
        gl.gdn_timer_destroy(t)
    M = B * L
    P = (H * 3 * D + 127) // 128 * 128 + 128
    # per loop: dY W and x^T dY (counted once each), plus the raw projections recomputed where the projection
    # GEMM does not store them itself (it does for bf16 inputs of >= 1024 tokens with 2H <= 32)
    nprod = 2 if (w.act == "bf16" and M >= 1024 and 2 * H <= 32) else 3
    gemm_flops = nprod * 2 * M * P * d
    gemm_ach = gemm_flops * T / (tot["gemm"] * 1e-3) / 1e12
    return {"workload": f"loop backward, {name} (B={B}, L={L}, H={H}, dk=dv={D}, d={d}, T={T}, {w.act} inputs)",
            "value": M / (ms * 1e-3), "unit": "tokens/s", "ms_per_call": ms,
            "stages_ms_per_call": tot, "stages_avg_launch_us": {k: v * 1e3 for k, v in per.items()},
            "gemm": {"bound": "mfma", "kernel": "k_gemm_tile" if w.act == "bf16" else "k_gemm_nt", "achieved": gemm_ach, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": gemm_ach / PEAK_BF16_TFLOPS,
                     "note": "algorithmic 2MNK per product; fp32 operands run 2-3 bf16 passes"}}


def bench_block(args, torch, gl, synth, name="prefill_b4_l8192", layers=1):
    """gdn_block_loop_prefill: T loops of an LT2 block stack (pre-norm, the mixer, the sigmoid-gated output
    projection, the SwiGLU FFN, identity residuals) on a prompt workload's shape."""
    w = synth.workload(name)
    B, L, H, D, d, T = w.B, w.L, w.H, w.dk, w.d, w.T
    F = synth.block_ffn(w)
    dev = lambda t: t.contiguous().to("cuda")
    x = synth.prefill_inputs(w)
    blocks = synth.block_inputs(w, layers)
    desc = gl.make_desc(B, L, H, D, D, T=T, act=w.act, alpha_lo=w.alpha_lo)
    n = gl.gdn_block_packed_bytes(desc, F)
    Wb = torch.empty(layers * n, dtype=torch.uint8, device="cuda")
    keys = ("g1", "Wq", "Wk", "Wv", "wa", "wb", "Wg", "Wo", "g2", "W1", "W3", "W2")
    for i, blk in enumerate(blocks):
        gl.gdn_block_pack(desc, F, *[dev(blk[k]) for k in keys], Wb[i * n:(i + 1) * n])
    ws = gl.block_workspace(desc, F)
    h0, rho = dev(x["h0"]), dev(x["rho"])
    h_out = torch.empty(B, L, d, device="cuda")
    stream = torch.cuda.current_stream()

    def call():
        gl.gdn_block_loop_prefill(desc, F, layers, h0, Wb, rho, h_out, ws, stream)

    for _ in range(3):
        call()
    torch.cuda.synchronize()
    nrep = max(min(args.steps, 10), 3)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(nrep):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / nrep
    stages = {"block_gemm": gl.GDN_STAGE_BLOCK_GEMM, "project": gl.GDN_STAGE_PROJECT,
              "scan_prep": gl.GDN_STAGE_SCAN_PREP, "scan_carry": gl.GDN_STAGE_SCAN_CARRY}
    timers = {k: gl.gdn_timer_create(v, 4 * nrep * T * layers) for k, v in stages.items()}
    for t in timers.values():
        gl.gdn_timer_attach(t)
    for _ in range(nrep):
        call()
    torch.cuda.synchronize()
    gl.gdn_timer_detach()
    per, tot = {}, {}
    for k, t in timers.items():
        cnt, total = gl.gdn_timer_read(t)
        per[k] = total / max(cnt, 1)
        tot[k] = total / nrep
        gl.gdn_timer_destroy(t)
    M, HD = B * L, H * D
    gemm_flops = 2 * M * (d * HD + HD * d + d * 2 * F + F * d)             # per block application
    step_flops = T * layers * (gemm_flops + proj_flops_per_token(w) * M + scan_flops_per_token(w) * M)
    gemm_ach = gemm_flops * T * layers / (tot["block_gemm"] * 1e-3) / 1e12
    return {"workload": f"LT2 block stack, {name} shape (B={B}, L={L}, d={d}, H={H}, ffn={F}, layers={layers}, "
                        f"T={T}, {w.act})",
            "value": M / (ms * 1e-3), "unit": "tokens/s", "ms_per_call": ms,
            "algorithmic_tflops": step_flops / (ms * 1e-3) / 1e12,
            "frac_of_bf16_peak": step_flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
            "stages_ms_per_call": tot, "stages_avg_launch_us": {k: v * 1e3 for k, v in per.items()},
            "gemm": {"bound": "mfma", "kernel": "k_gemm_tile", "achieved": gemm_ach, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": gemm_ach / PEAK_BF16_TFLOPS}}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, synth, sample_tokens=2048):
    """The fp64 oracle on a bounded sample of the workload: the first `sample_tokens` tokens of sequence 0
    through all T loops, repeated until at least 10 s of CPU work; tokens/s of the sample."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # threadpoolctl missing: report OpenMP threads only
        blas_threads = 1
    Ls = min(sample_tokens, w.L)
    x = synth.prefill_inputs(w, L=Ls, B=1)
    runs, t0 = 0, time.perf_counter()
    while True:
        oracle.loop_prefill(x["h0"], x["Wq"], x["Wk"], x["Wv"], x["wa"], x["wb"], x["rho"], w.H, w.dk, w.dv,
                            w.alpha_lo, w.act)
        runs += 1
        dt = time.perf_counter() - t0
        if dt >= 10.0:
            break
    cores = max(oracle.num_threads(), blas_threads)
    return {"value": runs * Ls / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"{w.name}: sequence 0, first {Ls} tokens, all {w.T} loops, {runs} run(s) in {dt:.1f} s "
                      f"(fp64: numpy/OpenBLAS projections, C/OpenMP recurrence)"}


def calib_copy(torch):
    n = 256 << 20
    a = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"calib_copy_bytes": n, "launches": 5}))


def prefill_record(w, pf):
    """Rate, rooflines and per-stage times of one prefill workload."""
    tokens = pf["tokens"]
    st = pf["per_stage"]
    proj = st["project"]
    kname, kflops = proj_gemm_kernel(w, tokens)
    flops_launch = kflops * tokens
    achieved = flops_launch / (proj["avg_ms"] * 1e-3) / 1e12
    total_flops = (proj_flops_per_token(w) + scan_flops_per_token(w)) * w.T * tokens
    step_s = pf["ms_step"] * 1e-3
    rec = {
        "value": tokens / step_s, "unit": "tokens/s", "ms_per_step": pf["ms_step"],
        "config": {"workload": w.name, "B": w.B, "L": w.L, "H": w.H, "dk": w.dk, "dv": w.dv, "d": w.d,
                   "T": w.T, "chunk": 64, "alpha_lo": w.alpha_lo},
        "roofline": {"bound": "mfma", "kernel": kname, "achieved": achieved,
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                     "traffic": traffic_for(kname, w.name), "flops_per_launch": flops_launch,
                     "avg_launch_us": proj["avg_ms"] * 1e3},
        "whole_path": {"algorithmic_tflops": total_flops / step_s / 1e12,
                       "frac_of_bf16_peak": total_flops / step_s / 1e12 / PEAK_BF16_TFLOPS,
                       "loop_tokens_per_s": w.T * tokens / step_s,
                       "stages": {k: {"avg_launch_us": v["avg_ms"] * 1e3, "share_of_step": v["share"]}
                                  for k, v in st.items()}},
    }
    if "pipeline" in pf:
        rec["pipeline"] = dict(pf["pipeline"], note=(
            "the step runs as a pipeline over pieces of each sequence (one stream of projections and chunk preps, "
            "a carry stream per loop); the kernel rooflines and stage times are those of the same call run loop "
            "by loop, and the stage shares are of that call's step"))
    if "scan_carry" in st:
        bpl = carry_bytes_per_step(w) * tokens / w.T
        gbs = bpl / (st["scan_carry"]["avg_ms"] * 1e-3) / 1e9
        cname = carry_kernel(w)
        rec["roofline_carry"] = {"bound": "hbm", "kernel": cname, "achieved": gbs,
                                 "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS,
                                 "traffic": traffic_for(cname, w.name), "bytes_per_launch": bpl,
                                 "avg_launch_us": st["scan_carry"]["avg_ms"] * 1e3}
    return rec


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="prefill_b4_l8192")
    ap.add_argument("--extra", default="prefill_b1_l32768,prefill_b1_l4096",
                    help="comma-separated further prefill workloads reported under extra_workloads ('' for none)")
    ap.add_argument("--decode-steps", type=int, default=256)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-act", action="store_true")
    ap.add_argument("--no-block", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calib-copy", action="store_true")
    ap.add_argument("--pieces", type=int, default=0,
                    help="gdn_loop_prefill_set_pieces for the prefill legs: 0 the library's automatic setting, -1 loop "
                         "by loop (every launch covers the whole prompt; for counter runs), > 0 tokens per piece")
    ap.add_argument("--only", default="", choices=["", "act", "block", "scan_backward", "loop_backward", "decode",
                                                   "loop_decode"],
                    help="run one secondary leg alone and print its record (for profiling; no headline line)")
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
    gl.gdn_loop_prefill_set_pieces(args.pieces)
    w = synth.workload(args.workload)
    if args.only:
        legs = {"act": lambda: bench_act(args, torch, gl, synth, w),
                "block": lambda: bench_block(args, torch, gl, synth, w.name),
                "scan_backward": lambda: bench_backward(args, torch, gl, synth),
                "loop_backward": lambda: bench_loop_backward(args, torch, gl, synth),
                "decode": lambda: bench_decode(args, torch, gl, synth),
                "loop_decode": lambda: bench_loop_decode(args, torch, gl, synth, synth.workload("decode_n64_s256"))}
        log(f"{args.only} alone")
        print(json.dumps({args.only: legs[args.only]()}))
        return
    log(f"prefill: {w.name}, warmup {args.warmup}, steps {args.steps}")
    pf = bench_prefill(args, w, torch, gl, synth, args.warmup)
    head = prefill_record(w, pf)
    out = {
        "metric": METRIC,
        "value": head["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.act,
        "data": "synthetic (seeded Gaussian inputs and random-init weights of the workload's shape)",
        "config": head["config"],
        "roofline": head["roofline"],
    }
    for key in ("roofline_carry", "whole_path"):
        if key in head:
            out[key] = head[key]
    extras = {}
    for name in [n for n in args.extra.split(",") if n and n != w.name]:
        we = synth.workload(name)
        log(f"prefill (extra): {name}, warmup {max(args.warmup, 20)}, steps {args.steps}")
        extras[name] = prefill_record(we, bench_prefill(args, we, torch, gl, synth, max(args.warmup, 20)))
    if extras:
        out["extra_workloads"] = extras
    if not args.no_act:
        log(f"adaptive halting: {w.name} ...")
        out["act"] = bench_act(args, torch, gl, synth, w)
    if not args.no_block:
        log(f"LT2 block stack: {w.name} ...")
        out["block"] = bench_block(args, torch, gl, synth, w.name)
    if not args.no_backward:
        log("scan backward: the 4096-token prompt's shape ...")
        out["scan_backward"] = bench_backward(args, torch, gl, synth)
        log("loop backward: the 4096-token prompt ...")
        out["loop_backward"] = bench_loop_backward(args, torch, gl, synth)
    if not args.no_decode:
        out["decode"] = bench_decode(args, torch, gl, synth)
        log("loop decode: 64 sequences with projections ...")
        out["loop_decode"] = bench_loop_decode(args, torch, gl, synth, synth.workload("decode_n64_s256"))
    if not args.no_cpu_baseline:
        log("cpu baseline: running the oracle ...")
        out["cpu_baseline"] = cpu_baseline(w, synth)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out))


if __name__ == "__main__":
    main()
