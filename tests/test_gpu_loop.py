"""GPU parity of the projection stage and of the whole looped mixer (prefill and decode) against the oracle.

Workloads are the seeded synthetic ones of ``synth``: the tiny fp32 case (1e-4 bar), and the 16-head,
width-2048 bf16 cases (3e-3 bar) -- in full for the 4096-token prompt, and for the 8192x4 and 32768-token
prompts in the same launch configuration as the benchmark with the oracle on prefixes (every loop is causal,
so the first tokens of a full-size run must equal a run over just those tokens).

What is unique is gated at the bar: each stage on identical inputs (the scans in test_gpu_scan.py; the
projection here, whose bf16 outputs may differ from the oracle's only by the fp32 summation error bound
plus one bf16 step), and the fp32 loop end to end.  The bf16 loop end to end is not unique: bf16 rounding
decisions of values within fp32 summation error of a boundary go either way in any valid implementation
and propagate through the loops.  Its bars are the fixed ones or a multiple of the oracle's own spread when
it is recomputed as other valid fp32 implementations would (tests/helpers.py, loop_envelope), whichever is
larger: 2x for normwise errors, 4x for the heavy-tailed max-relative statistic.  Where the decay is strong
(alpha_lo = 0) a final state rests on the last few tokens, and two valid free-running implementations can
drift apart further than the envelope's few re-runs show; there each loop is checked teacher-forced: rerun by
the oracle from the GPU's own h^(t-1) and held to that one loop's envelope (_check_forced).
"""
import dataclasses
import numpy as np
import pytest
import torch

import looped_linear_attention_amd as gl
import oracle
import synth
from helpers import (ENV_MAX, ENV_NORM, TOL_BF16, TOL_F32, bf16_ulp, dev, envelope_bar, fp32_blocked,
                     loop_envelope, norm_err, rel_err, say)

pytestmark = pytest.mark.gpu


def _pack(w, x):
    desc = gl.make_desc(w.B, w.L, w.H, w.dk, w.dv, T=w.T, act=w.act, alpha_lo=w.alpha_lo)
    Wp = torch.empty(gl.gdn_weights_packed_bytes(desc) // (4 if w.act == "f32" else 2),
                     dtype=desc.act_dtype, device="cuda")
    gl.gdn_weights_pack(desc, dev(x["Wq"]), dev(x["Wk"]), dev(x["Wv"]), dev(x["wa"]), dev(x["wb"]), Wp)
    return Wp


def _loop_gpu(w, x, B, L, keep=True):
    desc = gl.make_desc(B, L, w.H, w.dk, w.dv, T=w.T, act=w.act, alpha_lo=w.alpha_lo)
    Wp = _pack(w, x)
    ws = gl.workspace(desc, gl.GDN_OP_LOOP_PREFILL)
    h_out = torch.empty(B, L, w.d, device="cuda")
    states = torch.empty(w.T, B, w.H, w.dk, w.dv, device="cuda") if keep else None
    loops = torch.empty(w.T, B, L, w.d, device="cuda") if keep else None
    gl.gdn_loop_prefill(desc, dev(x["h0"][:B, :L]), Wp, dev(x["rho"]), h_out, states, loops, ws)
    torch.cuda.synchronize()
    return h_out.cpu(), (states.cpu() if keep else None), (loops.cpu() if keep else None)


def _oracle_loop(w, x, B, L, keep=True):
    return oracle.loop_prefill(x["h0"][:B, :L], x["Wq"], x["Wk"], x["Wv"], x["wa"], x["wb"], x["rho"],
                               w.H, w.dk, w.dv, w.alpha_lo, w.act, keep_loops=keep, keep_states=keep)


# ---------------------------------------------------------------------------
# projection stage
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
    q = torch.empty(M, w.H, w.dk, dtype=a, device="cuda")
    k = torch.empty_like(q)
    v = torch.empty(M, w.H, w.dv, dtype=a, device="cuda")
    al = torch.empty(M, w.H, device="cuda")
    be = torch.empty(M, w.H, device="cuda")
    gl.gdn_project(desc, dev(xin), Wp, q, k, v, al, be)
    torch.cuda.synchronize()
    rq, rk, rv, ra, rb = oracle.project(xin, x["Wq"], x["Wk"], x["Wv"], x["wa"], x["wb"], w.H, w.dk, w.dv,
                                        w.alpha_lo, w.act)
    if w.act == "f32":
        for g, r in ((q, rq), (k, rk), (v, rv), (al, ra), (be, rb)):
            assert rel_err(g.cpu(), r) < 1e-5
    else:
        # bf16-stored values: the GPU's fp32 dot products differ from the exact ones by at most the standard
        # recursive-summation bound gamma_K * sum|x||w| (K = d terms, u = 2^-24); after rounding to bf16 the
        # two results may additionally sit one bf16 step apart.  q and k carry their norm's error as well.
        K = w.d
        gam = K * 2.0 ** -24 / (1 - K * 2.0 ** -24)
        xa = np.abs(xin.double().numpy())
        for g, r, W, normed in ((q, rq, x["Wq"], True), (k, rk, x["Wk"], True), (v, rv, x["Wv"], False)):
            Wd = W.double().numpy()
            p = (xin.double().numpy() @ Wd).reshape(M, w.H, -1)
            mag = (xa @ np.abs(Wd)).reshape(M, w.H, -1)
            if normed:
                nrm = np.sqrt(np.sum(p * p, -1, keepdims=True) + 1e-6)
                bound = 2 * gam * (mag + np.abs(p)) / nrm
            else:
                bound = 2 * gam * mag
            gg = g.cpu().double().numpy()
            diff = np.abs(gg - r)
            step = bf16_ulp(np.maximum(np.abs(r), np.abs(gg)))
            assert np.all(diff <= bound + step * 1.0001), float((diff - bound - step).max())
            assert np.mean(diff > 0) < 0.01
        assert rel_err(al.cpu(), ra) < 1e-5 and rel_err(be.cpu(), rb) < 1e-5


# ---------------------------------------------------------------------------
# looped prefill
# ---------------------------------------------------------------------------
def _check_loop(w, x, B, L, tol, gpu=None, Lcmp=None, forced=False):
    """Compare GPU loop outputs (first Lcmp tokens) with the oracle; bf16 uses the spread envelope.

    ``forced`` (bf16, whole sequences): the states are checked loop by loop from the GPU's own h^(t-1)
    (_check_forced) instead of against the free-running oracle, whose final states can drift further apart
    than the envelope's few re-runs show when the decay is strong."""
    g_h, g_s, g_l = gpu if gpu is not None else _loop_gpu(w, x, B, L)
    Lc = L if Lcmp is None else Lcmp
    if w.act == "f32":
        r = _oracle_loop(w, x, B, Lc)
        el = [rel_err(g_l[t][:, :Lc], r["loops"][t]) for t in range(w.T)]
        eh = rel_err(g_h[:, :Lc], r["h"])
        say(f"    h^(T) err {eh:.2e}; per-loop {[f'{e:.1e}' for e in el]}")
        assert eh <= tol and max(el) <= tol
        if g_s is not None and Lc == L:
            assert max(rel_err(g_s[t], r["states"][t]) for t in range(w.T)) <= tol
        return g_h, g_s, r
    r, sp = loop_envelope(w, x, B, Lc)
    for t in range(w.T):
        em, en = rel_err(g_l[t][:, :Lc], r["loops"][t]), norm_err(g_l[t][:, :Lc], r["loops"][t])
        bm, bn = envelope_bar(sp["h_max"][t], tol, ENV_MAX), envelope_bar(sp["h_norm"][t], 1e-4, ENV_NORM)
        say(f"    loop {t + 1}: h max-rel {em:.2e} (spread {sp['h_max'][t]:.2e}, bar {bm:.2e}); "
            f"normwise {en:.2e} (spread {sp['h_norm'][t]:.2e}, bar {bn:.2e})")
        assert em <= bm and en <= bn
        if g_s is not None and Lc == L and not forced:
            _check_state(g_s[t], r["states"][t], sp, t, tol)
    if forced:
        assert g_s is not None and Lc == L
        _check_forced(w, x, B, L, tol, g_s, g_l)
    return g_h, g_s, r


def _check_state(g, r, sp, t, tol):
    es, esn = rel_err(g, r), norm_err(g, r)
    bs, bsn = envelope_bar(sp["s_max"][t], tol, ENV_MAX), envelope_bar(sp["s_norm"][t], 1e-4, ENV_NORM)
    say(f"       state max-rel {es:.2e} (spread {sp['s_max'][t]:.2e}, bar {bs:.2e}); "
        f"normwise {esn:.2e} (spread {sp['s_norm'][t]:.2e}, bar {bsn:.2e})")
    assert es <= bs and esn <= bsn


def _check_forced(w, x, B, L, tol, g_s, g_l):
    """Teacher-forced check: loop t is rerun by the oracle (with its envelope, including eight variants whose
    q/k/v sums accumulate as an MFMA k-loop does) from the GPU's own fp32 h^(t-1), and the GPU's h^(t) and
    final state of loop t are held to that one loop's bars.

    This gates what each loop computes, which is unique up to the one loop's bf16 rounding decisions; the
    free-running comparison also carries every earlier loop's valid rounding decisions, amplified."""
    for t in range(w.T):
        h_in = x["h0"][:B, :L] if t == 0 else g_l[t - 1].double().numpy()
        r, sp = loop_envelope(w, x, B, L, h_in=h_in, loops=slice(t, t + 1), perms=8)
        em, en = rel_err(g_l[t], r["loops"][0]), norm_err(g_l[t], r["loops"][0])
        bm, bn = envelope_bar(sp["h_max"][0], tol, ENV_MAX), envelope_bar(sp["h_norm"][0], 1e-4, ENV_NORM)
        say(f"    loop {t + 1} from the GPU's h^({t}): h max-rel {em:.2e} (bar {bm:.2e}); "
            f"normwise {en:.2e} (bar {bn:.2e})")
        assert em <= bm and en <= bn
        _check_state(g_s[t], r["states"][0], sp, 0, tol)


def test_loop_prefill_tiny_f32():
    w = synth.workload("tiny_f32")
    say("[loop_prefill] tiny_f32 full")
    x = synth.prefill_inputs(w)
    _check_loop(w, x, w.B, w.L, TOL_F32)


@pytest.mark.parametrize("L", [1, 63, 65, 200])
def test_loop_prefill_bf16_ragged(L):
    w = synth.workload("prefill_b1_l4096")
    say(f"[loop_prefill] 16 heads bf16 L={L}")
    x = synth.prefill_inputs(w, L=L)
    _check_loop(w, x, 1, L, TOL_BF16)


def test_loop_prefill_b1_l4096_full():
    w = synth.workload("prefill_b1_l4096")
    say("[loop_prefill] prefill_b1_l4096 full size (three oracle runs, ~1 min)")
    x = synth.prefill_inputs(w)
    _check_loop(w, x, w.B, w.L, TOL_BF16)


@pytest.mark.parametrize("name,prefix", [("prefill_b4_l8192", 512), ("prefill_b1_l32768", 1024)])
def test_loop_prefill_full_size_prefix(name, prefix):
    """Full-size launch (as benchmarked); the oracle checks every batch row's first `prefix` tokens."""
    w = synth.workload(name)
    say(f"[loop_prefill] {name} full launch, oracle on {prefix}-token prefix")
    x = synth.prefill_inputs(w)
    g_h, g_s, g_l = _loop_gpu(w, x, w.B, w.L, keep=True)
    assert np.isfinite(g_h.numpy()).all() and np.isfinite(g_s.numpy()).all()
    _check_loop(w, x, w.B, w.L, TOL_BF16, gpu=(g_h, None, g_l), Lcmp=prefix)


def _forced_head(w, x, B, L, t, head, h_prev, x_in, rot=None, **kw):
    """Oracle loop t of one head from a given h^(t-1) (fp64 [B, L, d]) and its bf16 rounding x_in: the head's
    q/k/v and gate columns only, its scan, its residual (``rot``: q/k/v summed as an MFMA k-loop does, see
    helpers.fp32_blocked).  Returns (h^(t) columns [B, L, dv], S_final [B, dk, dv])."""
    cq, cv = slice(head * w.dk, (head + 1) * w.dk), slice(head * w.dv, (head + 1) * w.dv)
    Wq, Wk, Wv = (x[n][:, c].double().numpy() for n, c in (("Wq", cq), ("Wk", cq), ("Wv", cv)))
    q, k, v, al, be = oracle.project(x_in, Wq, Wk, Wv, x["wa"][:, head:head + 1],
                                     x["wb"][:, head:head + 1], 1, w.dk, w.dv, w.alpha_lo, w.act, **kw)
    if rot is not None:
        f32 = np.float32
        qf, kf = fp32_blocked(x_in, Wq, rot), fp32_blocked(x_in, Wk, rot)
        v = oracle.round_bf16(fp32_blocked(x_in, Wv, rot))
        q = oracle.round_bf16(qf / np.sqrt(np.sum(qf * qf, axis=-1, keepdims=True, dtype=f32) + f32(1e-6)))
        k = oracle.round_bf16(kf / np.sqrt(np.sum(kf * kf, axis=-1, keepdims=True, dtype=f32) + f32(1e-6)))
    o, st = oracle.scan(q.reshape(B, L, 1, w.dk), k.reshape(B, L, 1, w.dk), v.reshape(B, L, 1, w.dv),
                        al.reshape(B, L, 1), be.reshape(B, L, 1))
    rho = x["rho"][t].double().numpy()[cv]
    return o.reshape(B, L, w.dv) + rho * h_prev[:, :, cv], st[:, 0]


@pytest.mark.parametrize("name,head", [("prefill_b4_l8192", 0), ("prefill_b1_l32768", 15)])
def test_loop_prefill_full_size_heads(name, head):
    """Full-size launch (as benchmarked), every token of one head through all four loops, teacher-forced: loop t
    of the head is rerun by the oracle from the GPU's own h^(t-1) (only that head's projection columns and scan
    are needed) and the GPU's h^(t) columns and final states are held to that one loop's envelope (a library
    fp32 matmul, a one-ulp jitter of every bf16 rounding and two MFMA-order sums; bars as in _check_forced)."""
    w = synth.workload(name)
    say(f"[loop_prefill] {name} full launch, head {head} teacher-forced over all {w.L} tokens")
    x = synth.prefill_inputs(w)
    B, L = w.B, w.L
    _, g_s, g_l = _loop_gpu(w, x, B, L, keep=True)
    cv = slice(head * w.dv, (head + 1) * w.dv)
    for t in range(w.T):
        h_prev = x["h0"].double().numpy() if t == 0 else g_l[t - 1].double().numpy()
        flat = h_prev.reshape(B * L, w.d)
        rh, rs = _forced_head(w, x, B, L, t, head, h_prev, oracle.round_bf16(flat))
        runs = [_forced_head(w, x, B, L, t, head, h_prev, oracle.round_bf16(flat), fp32_sum=True),
                _forced_head(w, x, B, L, t, head, h_prev, oracle.round_bf16(flat, np.random.default_rng(9100 + t)),
                             jitter=np.random.default_rng(9200 + t))]
        x_ref = oracle.round_bf16(flat)
        runs += [_forced_head(w, x, B, L, t, head, h_prev, x_ref, rot=r) for r in (0, w.d // 32)]
        sp = dict(h_max=max(rel_err(a, rh) for a, _ in runs), h_norm=max(norm_err(a, rh) for a, _ in runs),
                  s_max=max(rel_err(b, rs) for _, b in runs), s_norm=max(norm_err(b, rs) for _, b in runs))
        gh, gs = g_l[t].double().numpy()[:, :, cv], g_s[t].double().numpy()[:, head]
        em, en = rel_err(gh, rh), norm_err(gh, rh)
        es, esn = rel_err(gs, rs), norm_err(gs, rs)
        bm, bn = envelope_bar(sp["h_max"], TOL_BF16, ENV_MAX), envelope_bar(sp["h_norm"], 1e-4, ENV_NORM)
        bs, bsn = envelope_bar(sp["s_max"], TOL_BF16, ENV_MAX), envelope_bar(sp["s_norm"], 1e-4, ENV_NORM)
        say(f"    loop {t + 1}: h max-rel {em:.2e} (bar {bm:.2e}) normwise {en:.2e} (bar {bn:.2e}); "
            f"state max-rel {es:.2e} (bar {bs:.2e}) normwise {esn:.2e} (bar {bsn:.2e})")
        assert em <= bm and en <= bn and es <= bs and esn <= bsn


def test_loop_prefill_bf16_d64_h3_wide():
    """1100 tokens of three 64-wide heads: the wide projection, whose two column tiles each leave a partial
    gate pre-activation (the second over the single remaining 64-channel block) for the chunk preparation."""
    w = _proj_workload("bf16_d64_h3")
    say("[loop_prefill] bf16, 3 heads of 64, L=1100")
    x = synth.prefill_inputs(w, L=1100)
    _check_loop(w, x, 1, 1100, TOL_BF16)


def test_loop_prefill_b2_ragged_wide():
    """Two sequences of 700 tokens (1400 >= 1024: the wide projection with gate partials): the second sequence
    starts inside a 256-token GEMM tile and both end in a 60-token partial chunk.  The states are checked
    teacher-forced: with alpha_lo = 0 the free-running loop-2 state drifts 3.7e-4 (normwise) from the oracle's
    while the oracle rerun from the GPU's own h^(1) lands within 1e-5 of the GPU's."""
    w = synth.workload("prefill_b4_l8192")
    say("[loop_prefill] 16 heads bf16 B=2 L=700 (prefill_b4_l8192 rows)")
    x = synth.prefill_inputs(w, B=2, L=700)
    assert tuple(x["h0"].shape) == (2, 700, w.d)
    _check_loop(w, x, 2, 700, TOL_BF16, forced=True)


@pytest.mark.parametrize("name,L", [("prefill_b1_l4096", 300)])
def test_loop_prefill_no_decay(name, L):
    """alpha_lo = 1: every gate alpha is exactly 1, the loops run the delta rule without decay (DeltaNet).

    bf16 only at the loop level: with fp32 inputs one scan without decay lands about 3e-5 from the oracle (the
    split-bf16 products carry ~16 bits and no decay damps them; the fp32 scan-level cases with alpha = 1 pass the
    1e-4 bar), and four loops compound that to 1.1e-4 on the 256-token fp32 workload."""
    w = dataclasses.replace(synth.workload(name), alpha_lo=1.0)
    say(f"[loop_prefill] {name} with alpha = 1, L={L}")
    x = synth.prefill_inputs(w, L=L)
    _check_loop(w, x, w.B, L, TOL_F32 if w.act == "f32" else TOL_BF16)


def test_loop_prefill_d64_h16():
    """16 heads of 64 (d = 1024) over 2048 tokens: eight 384-row column tiles of two heads each, so every XCD
    takes one column tile and the gate block pairs stay in tile order.  States teacher-forced: already at loop 1
    (identical inputs) the final states differ from the oracle's by the q/k/v roundings that the GEMM's fp32
    sums flip, more than the free-running envelope's library-matmul variants flip."""
    w = dataclasses.replace(synth.workload("prefill_b1_l4096"), name="bf16_d64_h16", dk=64, dv=64, d=1024)
    say("[loop_prefill] bf16, 16 heads of 64, L=2048")
    x = synth.prefill_inputs(w, L=2048)
    assert tuple(x["h0"].shape) == (1, 2048, 1024)
    _check_loop(w, x, 1, 2048, TOL_BF16, forced=True)


def test_loop_prefill_deterministic_and_no_aliasing_effects():
    w = synth.workload("prefill_b1_l4096")
    say("[loop_prefill] determinism, with and without per-loop outputs")
    x = synth.prefill_inputs(w, L=700)
    h1, _, _ = _loop_gpu(w, x, 1, 700, keep=True)
    h2, _, _ = _loop_gpu(w, x, 1, 700, keep=False)
    h3, _, _ = _loop_gpu(w, x, 1, 700, keep=False)
    assert torch.equal(h1, h2) and torch.equal(h2, h3)


def test_loop_prefill_zero_values_closed_form():
    """Wv = 0 makes every mixer output zero, so h^(T) = (prod rho) (.) h^(0) (up to fp32 products)."""
    w = synth.workload("prefill_b1_l4096")
    say("[loop_prefill] Wv = 0 closed form")
    x = synth.prefill_inputs(w, L=130)
    x["Wv"] = torch.zeros_like(x["Wv"])
    g_h, _, _ = _loop_gpu(w, x, 1, 130, keep=False)
    ref = torch.prod(x["rho"].double(), 0)[None, None] * x["h0"].double()
    assert rel_err(g_h, ref) < 1e-6


# ---------------------------------------------------------------------------
# looped decode
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("name,N,L0,steps", [("tiny_f32", 1, 100, 3), ("prefill_b1_l4096", 3, 70, 3)])
def test_loop_decode_after_prefill(name, N, L0, steps):
    """GPU prefill over L0 tokens, then GPU decode of the next tokens, equals the oracle over L0+steps."""
    w = synth.workload(name)
    say(f"[loop_decode] {name} N={N} prefill {L0} then {steps} steps")
    xb = synth.prefill_inputs(w)
    # N sequences: reuse the drawn stream's rows as separate sequences
    h0 = xb["h0"].reshape(-1, w.d)[: N * (L0 + steps)].reshape(N, L0 + steps, w.d).contiguous()
    x = dict(xb)
    x["h0"] = h0
    desc_p = gl.make_desc(N, L0, w.H, w.dk, w.dv, T=w.T, act=w.act, alpha_lo=w.alpha_lo)
    Wp = _pack(w, x)
    ws = gl.workspace(desc_p, gl.GDN_OP_LOOP_PREFILL)
    h_out = torch.empty(N, L0, w.d, device="cuda")
    states = torch.empty(w.T, N, w.H, w.dk, w.dv, device="cuda")
    gl.gdn_loop_prefill(desc_p, dev(h0[:, :L0]), Wp, dev(x["rho"]), h_out, states, None, ws)
    desc_d = gl.make_desc(N, 1, w.H, w.dk, w.dv, T=w.T, act=w.act, alpha_lo=w.alpha_lo)
    wsd = gl.workspace(desc_d, gl.GDN_OP_LOOP_DECODE)
    outs = []
    for s in range(steps):
        ho = torch.empty(N, w.d, device="cuda")
        gl.gdn_loop_decode(desc_d, dev(h0[:, L0 + s]), Wp, dev(x["rho"]), states, ho, wsd)
        outs.append(ho)
    torch.cuda.synchronize()
    if w.act == "f32":
        r = _oracle_loop(w, x, N, L0 + steps, keep=False)
        for s in range(steps):
            e = rel_err(outs[s].cpu(), r["h"][:, L0 + s])
            say(f"    step {s}: err {e:.2e}")
            assert e <= TOL_F32
        return
    r, sp = loop_envelope(w, x, N, L0 + steps)
    for s in range(steps):
        g, rr = outs[s].cpu(), r["h"][:, L0 + s]
        em, en = rel_err(g, rr), norm_err(g, rr)
        say(f"    step {s}: max-rel {em:.2e} normwise {en:.2e} "
            f"(loop-{w.T} spread {sp['h_max'][-1]:.2e}/{sp['h_norm'][-1]:.2e})")
        assert em <= envelope_bar(sp["h_max"][-1], TOL_BF16, ENV_MAX)
        assert en <= envelope_bar(sp["h_norm"][-1], 1e-4, ENV_NORM)
