"""GPU parity of the projection stage and of the whole looped mixer (prefill and decode) against the oracle.

Workloads are the seeded synthetic ones of ``synth``: the tiny fp32 case, and the 16-head, width-2048 bf16
cases -- the 4096-token prompt in full (every head), the 4x8192 and 32768-token prompts in the launch
configuration of the benchmark (every token of two heads).

Every check is held to a fixed bar (1e-4 for fp32, 3e-3 for bf16 inputs with an fp32 state; the metric of
tests/helpers.py), each on the inputs its stage actually received:

* the fp32 loop free-running, end to end, against the oracle's loop;
* each loop tau of a bf16 loop stage by stage ("stage-forced"): the GPU's own h^(tau-1) (fp32, read from
  h_loops) is the input of loop tau on both sides.
  - Projection: the q/k/v and gates that loop tau of the GPU used (read from the documented workspace regions
    after a call with T = tau; loops 1..tau are computed identically for every T) against
    oracle.project(bf16(h^(tau-1))): q/k/v within the fp32 summation bound plus one bf16 step, the gates
    within 1e-5.
  - Scan and residual: oracle.scan on those same bf16 q/k/v with the oracle's fp64 gates, plus
    rho_tau (.) h^(tau-1), against the GPU's h^(tau) and final state of loop tau.

The free-running bf16 loop is not unique: a value within fp32 summation error of a bf16 rounding boundary
may round either way in any valid implementation, and the next loop's projection amplifies that step.  The
free-running deviation is printed for the 4096-token prompt as a diagnostic and is not a gate.
"""
import dataclasses
import numpy as np
import pytest
import torch

import looped_linear_attention_amd as gl
import oracle
import synth
from helpers import (TOL_BF16, TOL_F32, canary_intact, check_projection, dev, norm_err, padded, poison_, rel_err,
                     say)

pytestmark = pytest.mark.gpu


def _pack(w, x):
    desc = gl.make_desc(w.B, w.L, w.H, w.dk, w.dv, T=w.T, act=w.act, alpha_lo=w.alpha_lo)
    Wp = torch.empty(gl.gdn_weights_packed_bytes(desc) // (4 if w.act == "f32" else 2),
                     dtype=desc.act_dtype, device="cuda")
    gl.gdn_weights_pack(desc, dev(x["Wq"]), dev(x["Wk"]), dev(x["Wv"]), dev(x["wa"]), dev(x["wb"]), Wp)
    return Wp


class LoopRun:
    """One gdn_loop_prefill call with T loops on NaN-poisoned outputs and workspace, canaries past every
    output.  Holds h^(T) and, with keep, every h^(tau) and final state (on the device), and the workspace's
    views of loop T's q/k/v/alpha/beta."""

    def __init__(self, w, x, B, L, T, Wp=None, keep=True):
        desc = gl.make_desc(B, L, w.H, w.dk, w.dv, T=T, act=w.act, alpha_lo=w.alpha_lo)
        Wp = _pack(w, x) if Wp is None else Wp
        ws = poison_(gl.workspace(desc, gl.GDN_OP_LOOP_PREFILL))
        h_out, hb = padded((B, L, w.d))
        states, sb = padded((T, B, w.H, w.dk, w.dv)) if keep else (None, None)
        loops, lb = padded((T, B, L, w.d)) if keep else (None, None)
        gl.gdn_loop_prefill(desc, dev(x["h0"][:B, :L]), Wp, dev(x["rho"][:T]), h_out, states, loops, ws)
        torch.cuda.synchronize()
        for t, buf in ((h_out, hb), (states, sb), (loops, lb)):
            if t is not None:
                assert canary_intact(buf, t.numel()), "a write past the end of an output"
                assert bool(torch.isfinite(t).all()), "an output element was not written (or is not finite)"
        self.desc, self.ws, self.Wp = desc, ws, Wp
        self.h_out, self.states, self.loops = h_out, states, loops

    def operands(self, heads=None):
        """Loop T's q, k, v [M, nh, D], alpha, beta [M, nh] (CPU) for the selected heads (default all)."""
        op = gl.GDN_OP_LOOP_PREFILL
        out = []
        for reg in (gl.GDN_WS_Q, gl.GDN_WS_K, gl.GDN_WS_V, gl.GDN_WS_ALPHA, gl.GDN_WS_BETA):
            t = gl.workspace_view(self.ws, self.desc, op, reg)
            if heads is not None:
                t = t[:, list(heads)]
            out.append(t.cpu())
        return out


def _head_slices(w, heads):
    cq = np.concatenate([np.arange(h * w.dk, (h + 1) * w.dk) for h in heads])
    cv = np.concatenate([np.arange(h * w.dv, (h + 1) * w.dv) for h in heads])
    return cq, cv


def _weights(w, x, heads):
    cq, cv = _head_slices(w, heads)
    hs = list(heads)
    f = lambda t: t.double().numpy()
    return f(x["Wq"])[:, cq], f(x["Wk"])[:, cq], f(x["Wv"])[:, cv], f(x["wa"])[:, hs], f(x["wb"])[:, hs]


def check_forced_loops(w, x, B, L, heads=None, tol=TOL_BF16, full=None, prefix_bitwise=True):
    """Stage-forced parity of every loop (see the module docstring) for the selected heads (default all).

    ``full``: an existing T-loop LoopRun with keep=True of the same inputs, else one is made.
    ``prefix_bitwise``: the call with T = tau reproduces h^(tau) of the full call bit for bit (False where the
    two calls take different carry variants, as a pipelined call against the loop-by-loop T = 1 call)."""
    heads = tuple(range(w.H)) if heads is None else tuple(heads)
    nh = len(heads)
    cq, cv = _head_slices(w, heads)
    full = LoopRun(w, x, B, L, w.T) if full is None else full
    Wq, Wk, Wv, wa, wb = _weights(w, x, heads)
    rho = x["rho"].double().numpy()
    h0 = x["h0"][:B, :L].double().numpy()
    for tau in range(1, w.T + 1):
        run = full if tau == w.T else LoopRun(w, x, B, L, tau, Wp=full.Wp, keep=False)
        if tau < w.T and prefix_bitwise:   # loops 1..tau do not depend on T: the shorter call reproduces h^(tau)
            assert torch.equal(run.h_out, full.loops[tau - 1])
        gq, gk, gv, ga, gb = run.operands(heads)
        del run
        h_prev = h0 if tau == 1 else full.loops[tau - 2].cpu().double().numpy()
        M = B * L
        x_in = h_prev.reshape(M, w.d)
        if w.act == "bf16":
            x_in = oracle.round_bf16(x_in)
        ra, rb = check_projection(gq, gk, gv, ga, gb, x_in, Wq, Wk, Wv, wa, wb, nh, w.dk, w.dv, w.alpha_lo, w.act)
        o, S = oracle.scan(gq.reshape(B, L, nh, w.dk), gk.reshape(B, L, nh, w.dk), gv.reshape(B, L, nh, w.dv),
                           ra.reshape(B, L, nh), rb.reshape(B, L, nh))
        h_ref = o.reshape(B, L, nh * w.dv) + rho[tau - 1][cv] * h_prev[:, :, cv]
        g_h = full.loops[tau - 1][:, :, torch.as_tensor(cv, device="cuda")].cpu()
        g_s = full.states[tau - 1][:, list(heads)].cpu()
        eh, es = rel_err(g_h, h_ref), rel_err(g_s, S)
        say(f"    loop {tau}: h^({tau}) max-rel {eh:.2e} (normwise {norm_err(g_h, h_ref):.1e}), "
            f"state max-rel {es:.2e} (normwise {norm_err(g_s, S):.1e}); bar {tol:.0e}")
        assert eh <= tol and es <= tol
    return full


# ---------------------------------------------------------------------------
# projection stage (gdn_project: the GEMM with the gates in its epilogue or a launch of their own)
# ---------------------------------------------------------------------------
def _proj_workload(name):
    # bf16 with 64-wide heads and an odd head count: a 384-column tile holds two
    # heads' q|k|v, and the last tile only one
    if name == "bf16_d64_h3":
        return dataclasses.replace(synth.workload("prefill_b1_l4096"), name=name, H=3, dk=64, dv=64, d=192)
    return synth.workload(name)


# M >= 1024 bf16 tokens take the wide tiles (k_gates + k_proj_wide), shorter inputs the 256 x 128 tiles
# (at most 64 tokens: only the first two 32-row tiles of each 256-token tile are loaded and multiplied)
@pytest.mark.parametrize("name,M", [("tiny_f32", 256), ("prefill_b1_l4096", 300), ("prefill_b1_l4096", 1),
                                    ("prefill_b1_l4096", 64), ("prefill_b1_l4096", 65), ("bf16_d64_h3", 40),
                                    ("prefill_b1_l4096", 1100), ("bf16_d64_h3", 300), ("bf16_d64_h3", 1100)])
def test_project_parity(name, M):
    w = _proj_workload(name)
    say(f"[project] {name} M={M}")
    x = synth.prefill_inputs(w, L=min(M, w.L))
    xin = x["h0"].reshape(-1, w.d)[:M].contiguous()
    desc = gl.make_desc(M, 1, w.H, w.dk, w.dv, T=1, act=w.act, alpha_lo=w.alpha_lo)
    Wp = _pack(w, x)
    a = desc.act_dtype
    q = poison_(torch.empty(M, w.H, w.dk, dtype=a, device="cuda"))
    k = poison_(torch.empty_like(q))
    v = poison_(torch.empty(M, w.H, w.dv, dtype=a, device="cuda"))
    al = poison_(torch.empty(M, w.H, device="cuda"))
    be = poison_(torch.empty(M, w.H, device="cuda"))
    gl.gdn_project(desc, dev(xin), Wp, q, k, v, al, be)
    torch.cuda.synchronize()
    check_projection(q.cpu(), k.cpu(), v.cpu(), al.cpu(), be.cpu(), xin.double().numpy(),
                     *_weights(w, x, range(w.H)), w.H, w.dk, w.dv, w.alpha_lo, w.act)


# ---------------------------------------------------------------------------
# looped prefill
# ---------------------------------------------------------------------------
def test_loop_prefill_tiny_f32():
    """fp32 throughout: the free-running loop end to end (every h^(tau) and state) at 1e-4."""
    w = synth.workload("tiny_f32")
    say("[loop_prefill] tiny_f32 free-running")
    x = synth.prefill_inputs(w)
    g = LoopRun(w, x, w.B, w.L, w.T)
    r = oracle.loop_prefill(x["h0"], x["Wq"], x["Wk"], x["Wv"], x["wa"], x["wb"], x["rho"], w.H, w.dk, w.dv,
                            w.alpha_lo, w.act, keep_loops=True, keep_states=True)
    el = [rel_err(g.loops[t].cpu(), r["loops"][t]) for t in range(w.T)]
    es = [rel_err(g.states[t].cpu(), r["states"][t]) for t in range(w.T)]
    eh = rel_err(g.h_out.cpu(), r["h"])
    say(f"    h^(T) err {eh:.2e}; per-loop h {[f'{e:.1e}' for e in el]}; states {[f'{e:.1e}' for e in es]}")
    assert eh <= TOL_F32 and max(el) <= TOL_F32 and max(es) <= TOL_F32


def test_loop_prefill_tiny_f32_forced():
    """The same fp32 workload stage-forced (projection at 1e-5, scan and residual at 1e-4)."""
    w = synth.workload("tiny_f32")
    say("[loop_prefill] tiny_f32 stage-forced")
    check_forced_loops(w, synth.prefill_inputs(w), w.B, w.L, tol=TOL_F32)


@pytest.mark.parametrize("L", [1, 63, 65, 200])
def test_loop_prefill_bf16_ragged(L):
    w = synth.workload("prefill_b1_l4096")
    say(f"[loop_prefill] 16 heads bf16 L={L}, stage-forced")
    check_forced_loops(w, synth.prefill_inputs(w, L=L), 1, L)


def test_loop_prefill_b1_l4096_full():
    """The full 4096-token prompt, every head and token, stage-forced at 3e-3; the free-running deviation
    from the oracle's own loop is printed (not a gate, see the module docstring)."""
    w = synth.workload("prefill_b1_l4096")
    say("[loop_prefill] prefill_b1_l4096 full size, every head, stage-forced")
    x = synth.prefill_inputs(w)
    full = check_forced_loops(w, x, w.B, w.L)
    r = oracle.loop_prefill(x["h0"], x["Wq"], x["Wk"], x["Wv"], x["wa"], x["wb"], x["rho"], w.H, w.dk, w.dv,
                            w.alpha_lo, w.act, keep_loops=True, keep_states=True)
    for t in range(w.T):
        g = full.loops[t].cpu()
        say(f"    (diagnostic) free-running loop {t + 1}: h max-rel {rel_err(g, r['loops'][t]):.2e}, "
            f"normwise {norm_err(g, r['loops'][t]):.2e}; state normwise "
            f"{norm_err(full.states[t].cpu(), r['states'][t]):.2e}")


@pytest.mark.parametrize("name,heads", [("prefill_b4_l8192", (0, 9)), ("prefill_b1_l32768", (5, 15))])
def test_loop_prefill_full_size_heads(name, heads):
    """Full-size launch (as benchmarked): every token of two heads (on different XCDs) through all four
    loops, stage-forced at 3e-3, including the projection bound and the gates the chunk preparation forms
    from the GEMM's partial sums."""
    w = synth.workload(name)
    say(f"[loop_prefill] {name} full launch, heads {heads}, every token, stage-forced")
    check_forced_loops(w, synth.prefill_inputs(w), w.B, w.L, heads=heads)


def test_loop_prefill_bf16_d64_h3_wide():
    """1100 tokens of three 64-wide heads: the wide projection, whose two column tiles each leave a partial
    gate pre-activation (the second over the single remaining 64-channel block) for the chunk preparation."""
    w = _proj_workload("bf16_d64_h3")
    say("[loop_prefill] bf16, 3 heads of 64, L=1100, stage-forced")
    check_forced_loops(w, synth.prefill_inputs(w, L=1100), 1, 1100)


def test_loop_prefill_b2_ragged_wide():
    """Two sequences of 700 tokens (1400 >= 1024: the wide projection with gate partials): the second sequence
    starts inside a 256-token GEMM tile and both end in a 60-token partial chunk."""
    w = synth.workload("prefill_b4_l8192")
    say("[loop_prefill] 16 heads bf16 B=2 L=700 (prefill_b4_l8192 rows), stage-forced")
    x = synth.prefill_inputs(w, B=2, L=700)
    assert tuple(x["h0"].shape) == (2, 700, w.d)
    check_forced_loops(w, x, 2, 700)


def test_loop_prefill_b3_ragged_wide_carry():
    """Three sequences of 700 tokens with 16 heads: 384 (sequence, head, 16-column) slices are more than one
    round of workgroups, so the carry takes 32-column slices; both sequences' ends fall in partial chunks."""
    w = synth.workload("prefill_b4_l8192")
    say("[loop_prefill] 16 heads bf16 B=3 L=700 (32-column carry), stage-forced")
    x = synth.prefill_inputs(w, B=3, L=700)
    check_forced_loops(w, x, 3, 700)


@pytest.mark.parametrize("L", [300, 1500])
def test_loop_prefill_no_decay(L):
    """alpha_lo = 1: every gate alpha is exactly 1, the loops run the delta rule without decay (DeltaNet),
    on both projection variants (300 tokens: gates in the GEMM epilogue; 1500: gate partials)."""
    w = dataclasses.replace(synth.workload("prefill_b1_l4096"), alpha_lo=1.0)
    say(f"[loop_prefill] alpha = 1, L={L}, stage-forced")
    check_forced_loops(w, synth.prefill_inputs(w, L=L), w.B, L)


def test_loop_prefill_d64_h16():
    """16 heads of 64 (d = 1024) over 2048 tokens: eight 384-row column tiles of two heads each."""
    w = dataclasses.replace(synth.workload("prefill_b1_l4096"), name="bf16_d64_h16", dk=64, dv=64, d=1024)
    say("[loop_prefill] bf16, 16 heads of 64, L=2048, stage-forced")
    x = synth.prefill_inputs(w, L=2048)
    assert tuple(x["h0"].shape) == (1, 2048, 1024)
    check_forced_loops(w, x, 1, 2048)


def test_loop_prefill_deterministic_and_no_aliasing_effects():
    w = synth.workload("prefill_b1_l4096")
    say("[loop_prefill] determinism, with and without per-loop outputs")
    x = synth.prefill_inputs(w, L=700)
    h1 = LoopRun(w, x, 1, 700, w.T).h_out
    h2 = LoopRun(w, x, 1, 700, w.T, keep=False).h_out
    h3 = LoopRun(w, x, 1, 700, w.T, keep=False).h_out
    assert torch.equal(h1, h2) and torch.equal(h2, h3)


def test_loop_prefill_zero_values_closed_form():
    """Wv = 0 makes every mixer output zero, so h^(T) = (prod rho) (.) h^(0) (up to fp32 products)."""
    w = synth.workload("prefill_b1_l4096")
    say("[loop_prefill] Wv = 0 closed form")
    x = synth.prefill_inputs(w, L=130)
    x["Wv"] = torch.zeros_like(x["Wv"])
    g_h = LoopRun(w, x, 1, 130, w.T, keep=False).h_out.cpu()
    ref = torch.prod(x["rho"].double(), 0)[None, None] * x["h0"].double()
    assert rel_err(g_h, ref) < 1e-6


# ---------------------------------------------------------------------------
# looped decode
# ---------------------------------------------------------------------------
def _decode_call(w, Wp, T, h_t, rho, states, N, ws_short=0):
    """gdn_loop_decode with T loops on poisoned output and workspace (ws_short bytes smaller than
    gdn_workspace_bytes reports); returns (h_out, desc, ws)."""
    desc = gl.make_desc(N, 1, w.H, w.dk, w.dv, T=T, act=w.act, alpha_lo=w.alpha_lo)
    ws = poison_(torch.empty(gl.gdn_workspace_bytes(desc, gl.GDN_OP_LOOP_DECODE) - ws_short, dtype=torch.uint8,
                             device="cuda"))
    ho, hb = padded((N, w.d))
    gl.gdn_loop_decode(desc, h_t, Wp, rho[:T].contiguous(), states, ho, ws)
    torch.cuda.synchronize()
    assert canary_intact(hb, ho.numel()) and bool(torch.isfinite(ho).all())
    return ho, desc, ws


def check_forced_decode_step(w, x, Wp, h_t, rho, states_before, N, tol, ws_short=0):
    """One generated token per sequence, each loop stage-forced: the GPU's h^(tau-1) of the token and its
    loop-tau state before the step are the inputs on both sides (gdn_loop_decode with T = tau on a copy of
    the states gives h^(tau) and leaves loop tau's projections in the workspace).  Returns the GPU's
    h^(T) and states after the step, from a T-loop call on the states themselves."""
    heads = range(w.H)
    Wq, Wk, Wv, wa, wb = _weights(w, x, heads)
    rho64 = x["rho"].double().numpy()
    h_prev = h_t.cpu().double().numpy()
    for tau in range(1, w.T + 1):
        st = states_before[:tau].clone()
        ho, desc, ws = _decode_call(w, Wp, tau, h_t, rho, st, N, ws_short)
        ops = [gl.workspace_view(ws, desc, gl.GDN_OP_LOOP_DECODE, r).cpu()
               for r in (gl.GDN_WS_Q, gl.GDN_WS_K, gl.GDN_WS_V, gl.GDN_WS_ALPHA, gl.GDN_WS_BETA)]
        x_in = oracle.round_bf16(h_prev) if w.act == "bf16" else h_prev
        ra, rb = check_projection(*ops, x_in, Wq, Wk, Wv, wa, wb, w.H, w.dk, w.dv, w.alpha_lo, w.act)
        gq, gk, gv = ops[:3]
        o, S = oracle.scan(gq.reshape(N, 1, w.H, w.dk), gk.reshape(N, 1, w.H, w.dk), gv.reshape(N, 1, w.H, w.dv),
                           ra.reshape(N, 1, w.H), rb.reshape(N, 1, w.H), states_before[tau - 1].cpu())
        h_ref = o.reshape(N, w.d) + rho64[tau - 1] * h_prev
        eh, es = rel_err(ho.cpu(), h_ref), rel_err(st[tau - 1].cpu(), S)
        say(f"      loop {tau}: h max-rel {eh:.2e}, state max-rel {es:.2e}")
        assert eh <= tol and es <= tol
        h_prev = ho.cpu().double().numpy()
    states = states_before.clone()
    ho, _, _ = _decode_call(w, Wp, w.T, h_t, rho, states, N, ws_short)
    assert torch.equal(ho.cpu().double(), torch.from_numpy(h_prev))   # the T-loop call equals its forced loops
    return ho, states


@pytest.mark.parametrize("name,N,L0,steps", [("tiny_f32", 1, 100, 3), ("prefill_b1_l4096", 3, 70, 3)])
def test_loop_decode_after_prefill(name, N, L0, steps):
    """GPU prefill over L0 tokens, then GPU decode of the next tokens.  fp32: free-running against the
    oracle over L0 + steps tokens at 1e-4.  bf16: every step and loop stage-forced at 3e-3."""
    w = synth.workload(name)
    say(f"[loop_decode] {name} N={N} prefill {L0} then {steps} steps")
    xb = synth.prefill_inputs(w)
    # N sequences: reuse the drawn stream's rows as separate sequences
    h0 = xb["h0"].reshape(-1, w.d)[: N * (L0 + steps)].reshape(N, L0 + steps, w.d).contiguous()
    x = dict(xb)
    x["h0"] = h0
    pre = LoopRun(w, x, N, L0, w.T)
    states = pre.states.clone()
    rho = dev(x["rho"])
    if w.act == "f32":
        outs = []
        for s in range(steps):
            ho, _, _ = _decode_call(w, pre.Wp, w.T, dev(h0[:, L0 + s]), rho, states, N)
            outs.append(ho)
        r = oracle.loop_prefill(h0, x["Wq"], x["Wk"], x["Wv"], x["wa"], x["wb"], x["rho"], w.H, w.dk, w.dv,
                                w.alpha_lo, w.act)
        for s in range(steps):
            e = rel_err(outs[s].cpu(), r["h"][:, L0 + s])
            say(f"    step {s}: err {e:.2e}")
            assert e <= TOL_F32
        return
    for s in range(steps):
        say(f"    step {s}")
        _, states = check_forced_decode_step(w, x, pre.Wp, dev(h0[:, L0 + s]), rho, states, N, TOL_BF16)


def test_loop_decode_n64_forced():
    """The benchmark's loop-decode shape: 64 sequences of 16 heads of 128 at width 2048, decode states drawn
    as the decode workload draws them, four generated tokens, every step and loop stage-forced at 3e-3."""
    w = synth.workload("prefill_b1_l4096")
    wd = synth.workload("decode_n64_s256")
    N, steps = wd.B, 4
    say(f"[loop_decode] N={N}, {steps} steps, stage-forced")
    x = synth.prefill_inputs(w, L=N * steps)
    hs = x["h0"].reshape(N * steps, w.d).reshape(steps, N, w.d)
    states = dev(synth.decode_state_init(wd))
    Wp = _pack(w, x)
    rho = dev(x["rho"])
    for s in range(steps):
        say(f"    step {s}")
        _, states = check_forced_decode_step(w, x, Wp, dev(hs[s]), rho, states, N, TOL_BF16)


@pytest.mark.parametrize("name", ["prefill_b1_l4096", "tiny_f32"])
def test_loop_decode_batch_independent(name):
    """Each sequence's projection, state step and residual do not depend on the batch around it: a call
    on 64 sequences gives the same bits, in h_out and in every state, as four calls of 16."""
    w = synth.workload(name)
    N, part = 64, 16
    say(f"[loop_decode] {name}: N={N} against {N // part} calls of {part}")
    x = synth.prefill_inputs(w, L=N)
    h_t = dev(x["h0"].reshape(-1, w.d)[:N].contiguous())
    Wp = _pack(w, x)
    rho = dev(x["rho"])
    g = torch.Generator().manual_seed(5)
    states0 = (0.05 * torch.randn(w.T, N, w.H, w.dk, w.dv, generator=g)).to("cuda")
    s_all = states0.clone()
    h_all, _, _ = _decode_call(w, Wp, w.T, h_t, rho, s_all, N)
    h_part = torch.empty_like(h_all)
    s_part = states0.clone()
    for p0 in range(0, N, part):
        st = s_part[:, p0:p0 + part].contiguous()
        ho, _, _ = _decode_call(w, Wp, w.T, h_t[p0:p0 + part].contiguous(), rho, st, part)
        h_part[p0:p0 + part] = ho
        s_part[:, p0:p0 + part] = st
    torch.cuda.synchronize()
    assert torch.equal(h_all, h_part)
    assert torch.equal(s_all, s_part)


@pytest.mark.parametrize("H,D,N", [(1, 128, 5), (20, 64, 7), (16, 128, 1)])
def test_loop_decode_split_projection_shapes(H, D, N):
    """The decode projection split over the channels on other shapes: d = 128 (two channel ranges), twenty
    heads of 64 (d = 1280, four ranges, 40 gate columns: a gate tile wider than 32), one sequence at d = 2048;
    one generated token, every loop stage-forced at 3e-3."""
    w = dataclasses.replace(synth.workload("prefill_b1_l4096"), name=f"bf16_h{H}_d{D}", H=H, dk=D, dv=D, d=H * D)
    say(f"[loop_decode] split projection H={H} D={D} N={N}, stage-forced")
    x = synth.prefill_inputs(w, L=N)
    g = torch.Generator().manual_seed(7)
    states = dev(torch.randn(w.T, N, H, D, D, generator=g) * 0.02)
    Wp = _pack(w, x)
    check_forced_decode_step(w, x, Wp, dev(x["h0"][0]), dev(x["rho"]), states, N, TOL_BF16)


def test_loop_decode_workspace_without_partials():
    """A decode workspace without the projection's partials region (the last one) runs the projection unsplit:
    one step stage-forced at 3e-3 (64 sequences, 16 heads of 128); a workspace one region smaller still is
    refused.  gdn_loop_decode_noalloc at a width whose partials would not fit its 8 MiB scratch (32 heads of 128,
    64 sequences) runs unsplit too and gives the same bits as gdn_loop_decode on the smaller workspace."""
    up = lambda n: (n + 255) // 256 * 256
    for H, N in [(16, 64), (32, 64)]:
        w = dataclasses.replace(synth.workload("prefill_b1_l4096"), name=f"bf16_h{H}", H=H, d=H * 128)
        say(f"[loop_decode] H={H} N={N}, workspace without the partials region")
        x = synth.prefill_inputs(w, L=N)
        Wp = _pack(w, x)
        desc = gl.make_desc(N, 1, H, 128, 128, T=w.T, act=w.act, alpha_lo=w.alpha_lo)
        full = gl.gdn_workspace_bytes(desc, gl.GDN_OP_LOOP_DECODE)
        short = up(4 * N * ((H * 3 * 128 + 127) // 128 * 128 + 128) * 4)
        g = torch.Generator().manual_seed(5)
        st0 = dev(torch.randn(w.T, N, H, 128, 128, generator=g) * 0.02)
        h_t, rho = dev(x["h0"][0]), dev(x["rho"])
        with pytest.raises(gl.GdnError):
            gl.gdn_loop_decode(desc, h_t, Wp, rho, st0.clone(), torch.empty(N, w.d, device="cuda"),
                               torch.empty(full - short - 256, dtype=torch.uint8, device="cuda"))
        if H == 16:
            check_forced_decode_step(w, x, Wp, h_t, rho, st0, N, TOL_BF16, ws_short=short)
            continue
        assert full > 8 << 20 >= full - short
        ho_ws, _, _ = _decode_call(w, Wp, w.T, h_t, rho, st_ws := st0.clone(), N, short)
        st = st0.clone()
        ho = torch.empty(N, w.d, device="cuda")
        gl.gdn_loop_decode_noalloc(desc, h_t, Wp, rho, st, ho)
        torch.cuda.synchronize()
        assert torch.equal(ho, ho_ws) and torch.equal(st, st_ws)
