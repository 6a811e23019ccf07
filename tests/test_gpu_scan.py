"""GPU parity of the single-pass scans (chunkwise prefill and recurrent decode) against the oracle.

Inputs are the seeded draws of ``synth.scan_inputs``; q, k, v are identical on both sides (bf16 or fp32),
so any difference comes from the kernels' arithmetic.  Bars: 1e-4 (fp32 inputs), 3e-3 (bf16 inputs), with
the metric of tests/helpers.py.
"""
import numpy as np
import pytest
import torch

import looped_linear_attention_amd as gl
import oracle
import synth
from helpers import TOL_BF16, TOL_F32, canary_intact, dev, padded, poison_, rel_err, say

pytestmark = pytest.mark.gpu


def _scan_gpu(x, act, s_init=None, want_state=True):
    """gdn_scan_prefill on NaN-poisoned outputs and workspace, with canaries past the outputs."""
    q = x["q"]
    B, L, H, D = q.shape
    desc = gl.make_desc(B, L, H, D, D, T=1, act=act)
    ws = poison_(gl.workspace(desc, gl.GDN_OP_SCAN_PREFILL))
    o, ob = padded((B, L, H, D))
    sf, sb = padded((B, H, D, D)) if want_state else (None, None)
    gl.gdn_scan_prefill(desc, dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(x["alpha"]), dev(x["beta"]),
                        None if s_init is None else dev(s_init), o, sf, ws)
    torch.cuda.synchronize()
    assert canary_intact(ob, o.numel()) and (sf is None or canary_intact(sb, sf.numel()))
    return o.cpu(), (sf.cpu() if sf is not None else None)


CASES = [
    # (B, L, H, D, act, alpha_range, beta_range, with_state)
    (1, 64, 1, 128, "bf16", (0.0, 1.0), (0.0, 1.0), False),
    (1, 1, 1, 128, "bf16", (0.0, 1.0), (0.0, 1.0), True),
    (1, 63, 2, 128, "bf16", (0.9, 1.0), (0.0, 1.0), True),
    (2, 65, 2, 128, "bf16", (0.0, 1.0), (0.0, 1.0), True),
    (1, 257, 3, 128, "bf16", (0.95, 1.0), (0.0, 1.0), False),
    (1, 200, 2, 64, "bf16", (0.0, 1.0), (0.0, 1.0), True),
    (1, 130, 1, 64, "f32", (0.0, 1.0), (0.0, 1.0), True),
    (2, 96, 2, 128, "f32", (0.5, 1.0), (0.0, 1.0), True),
    (1, 300, 2, 128, "bf16", (0.0, 1.0), (0.0, 2.0), True),   # negative eigenvalues (beta up to 2)
    (1, 300, 2, 128, "bf16", (1.0, 1.0), (0.0, 1.0), True),   # no decay (alpha = 1: DeltaNet)
    (1, 200, 2, 64, "f32", (1.0, 1.0), (0.0, 2.0), True),     # no decay, beta up to 2
    # more (sequence, head) pairs than one round of 16-column workgroups: the 32-column carry
    (3, 1000, 16, 128, "bf16", (0.0, 1.0), (0.0, 1.0), True),  # ragged: 15 chunks + 40 tokens
    (5, 130, 16, 128, "bf16", (0.9, 1.0), (0.0, 2.0), True),   # 2 chunks + 2 tokens, beta up to 2
]


@pytest.mark.parametrize("B,L,H,D,act,ar,br,ws", CASES)
def test_scan_prefill_parity(B, L, H, D, act, ar, br, ws):
    say(f"[scan_prefill] B={B} L={L} H={H} D={D} act={act} alpha={ar} beta={br} s_init={ws}")
    x = synth.scan_inputs(100 + L + D, B, L, H, D, D, act=act, alpha_range=ar, beta_range=br,
                          with_state=ws)
    o, sf = _scan_gpu(x, act, x.get("s_init"))
    ro, rs = oracle.scan(x["q"], x["k"], x["v"], x["alpha"], x["beta"], x.get("s_init"))
    eo, es = rel_err(o, ro), rel_err(sf, rs)
    say(f"    o err {eo:.2e}  S err {es:.2e}")
    tol = TOL_F32 if act == "f32" else TOL_BF16
    assert np.isfinite(o.numpy()).all()
    assert eo <= tol and es <= tol


@pytest.mark.parametrize("B,L,H,ar", [(1, 4096, 16, (0.9, 1.0)), (4, 8192, 16, (0.0, 1.0)),
                                      (1, 32768, 16, (0.95, 1.0))])
def test_scan_prefill_long_full_size(B, L, H, ar):
    """Scan-level parity at the prompts' full lengths and head counts (identical bf16 inputs on both sides), so
    any error the carry accumulates over hundreds of chunks is measured against the 3e-3 bar."""
    say(f"[scan_prefill] long: B={B} L={L} H={H} alpha={ar}")
    x = synth.scan_inputs(40 + B, B, L, H, 128, 128, act="bf16", alpha_range=ar)
    o, sf = _scan_gpu(x, "bf16")
    ro, rs = oracle.scan(x["q"], x["k"], x["v"], x["alpha"], x["beta"])
    eo, es = rel_err(o, ro), rel_err(sf, rs)
    say(f"    o err {eo:.2e}  S err {es:.2e}")
    assert eo <= TOL_BF16 and es <= TOL_BF16


def test_scan_prefill_identity_and_decay():
    """alpha = 1, beta = 0 keeps S_0 (o_t = S_0^T q_t); beta = 0 alone gives pure decay of S_0."""
    say("[scan_prefill] invariants alpha=1,beta=0 and beta=0")
    x = synth.scan_inputs(7, 1, 150, 2, 128, 128, act="bf16", with_state=True)
    x["alpha"][:] = 1.0
    x["beta"][:] = 0.0
    o, sf = _scan_gpu(x, "bf16", x["s_init"])
    assert torch.equal(sf, x["s_init"])
    ro, _ = oracle.scan(x["q"], x["k"], x["v"], x["alpha"], x["beta"], x["s_init"])
    assert rel_err(o, ro) < 1e-4
    x = synth.scan_inputs(8, 1, 150, 2, 128, 128, act="bf16", alpha_range=(0.9, 1.0), with_state=True)
    x["beta"][:] = 0.0
    o, sf = _scan_gpu(x, "bf16", x["s_init"])
    g = torch.prod(x["alpha"].double(), dim=1)
    assert rel_err(sf, g[:, :, None, None] * x["s_init"].double()) < 1e-4


def test_scan_prefill_split_resume():
    """Scanning [0, m) then [m, L) from the GPU's own carried state equals the oracle's single pass."""
    say("[scan_prefill] split/resume")
    x = synth.scan_inputs(9, 1, 300, 2, 128, 128, act="bf16", with_state=True)
    ro, rs = oracle.scan(x["q"], x["k"], x["v"], x["alpha"], x["beta"], x["s_init"])
    for m in (64, 100):
        a = {k: v[:, :m].contiguous() for k, v in x.items() if k != "s_init"}
        b = {k: v[:, m:].contiguous() for k, v in x.items() if k != "s_init"}
        o1, s1 = _scan_gpu(a, "bf16", x["s_init"])
        o2, s2 = _scan_gpu(b, "bf16", s1)
        assert rel_err(torch.cat([o1, o2], 1), ro) <= TOL_BF16
        assert rel_err(s2, rs) <= TOL_BF16


def test_scan_prefill_deterministic():
    say("[scan_prefill] determinism")
    x = synth.scan_inputs(10, 2, 333, 4, 128, 128, act="bf16", with_state=True)
    o1, s1 = _scan_gpu(x, "bf16", x["s_init"])
    o2, s2 = _scan_gpu(x, "bf16", x["s_init"])
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


@pytest.mark.parametrize("N,H,D,act,steps", [(4, 2, 128, "bf16", 5), (3, 2, 64, "f32", 4), (64, 16, 128, "bf16", 2)])
def test_scan_decode_parity(N, H, D, act, steps):
    say(f"[scan_decode] N={N} H={H} D={D} act={act} steps={steps}")
    x = synth.scan_inputs(20 + D, N, steps, H, D, D, act=act, with_state=True)
    desc = gl.make_desc(N, 1, H, D, D, T=1, act=act)
    states = dev(x["s_init"])
    rs = x["s_init"]
    tol = TOL_F32 if act == "f32" else TOL_BF16
    for t in range(steps):
        sl = {k: v[:, t].contiguous() for k, v in x.items() if k != "s_init"}
        o = torch.empty(N, H, D, device="cuda")
        gl.gdn_scan_decode(desc, dev(sl["q"]), dev(sl["k"]), dev(sl["v"]), dev(sl["alpha"]),
                           dev(sl["beta"]), states, o)
        torch.cuda.synchronize()
        ro, rs = oracle.scan(x["q"][:, t:t + 1], x["k"][:, t:t + 1], x["v"][:, t:t + 1],
                             x["alpha"][:, t:t + 1], x["beta"][:, t:t + 1], rs)
        eo, es = rel_err(o.cpu(), ro[:, 0]), rel_err(states.cpu(), rs)
        say(f"    step {t}: o err {eo:.2e} S err {es:.2e}")
        assert eo <= tol and es <= tol


def test_scan_decode_full_generation():
    """The batched-decode workload in full: 64 sequences x 16 heads of 128, 256 generated tokens, each token
    advancing all 4 loop states (1,024 launches), inputs drawn by the workload's own generators.  Every o of
    every (step, loop) and the final states are held to 3e-3 against the oracle run over the 256 tokens of
    each loop state (the decode recurrence is the scan taken one token at a time)."""
    w = synth.workload("decode_n64_s256")
    N, H, D, T, steps = w.B, w.H, w.dk, w.T, w.steps
    say(f"[scan_decode] {N} sequences x {steps} steps x {T} loop states")
    S0 = synth.decode_state_init(w)
    items = list(synth.decode_step_inputs(w, steps))
    stack = lambda key, tau: torch.stack([items[s * T + tau][key] for s in range(steps)], 1)   # [N, steps, ...]
    desc = gl.make_desc(N, 1, H, D, D, T=1, act=w.act)
    states = dev(S0)
    o_all = poison_(torch.empty(steps, T, N, H, D, device="cuda"))
    dq = dev(torch.stack([it["q"] for it in items]))
    dk = dev(torch.stack([it["k"] for it in items]))
    dvv = dev(torch.stack([it["v"] for it in items]))
    da = dev(torch.stack([it["alpha"] for it in items]))
    db = dev(torch.stack([it["beta"] for it in items]))
    for s in range(steps):
        for tau in range(T):
            i = s * T + tau
            gl.gdn_scan_decode(desc, dq[i], dk[i], dvv[i], da[i], db[i], states[tau], o_all[s, tau])
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o_all).all())
    worst_o = worst_s = 0.0
    for tau in range(T):
        ro, rs = oracle.scan(stack("q", tau), stack("k", tau), stack("v", tau), stack("alpha", tau),
                             stack("beta", tau), S0[tau])
        g_o = o_all[:, tau].permute(1, 0, 2, 3).cpu()     # [N, steps, H, D]
        eo = max(rel_err(g_o[:, s], ro[:, s]) for s in range(steps))
        es = rel_err(states[tau].cpu(), rs)
        say(f"    loop state {tau + 1}: worst per-step o err {eo:.2e}, final S err {es:.2e}")
        worst_o, worst_s = max(worst_o, eo), max(worst_s, es)
    assert worst_o <= TOL_BF16 and worst_s <= TOL_BF16


def test_prefill_state_then_decode_matches_longer_prefill():
    """GPU prefill over L tokens, then one GPU decode step, equals the oracle over L+1 tokens."""
    say("[scan] prefill -> decode handoff")
    x = synth.scan_inputs(30, 2, 129, 2, 128, 128, act="bf16")
    pre = {k: v[:, :128].contiguous() for k, v in x.items()}
    _, s = _scan_gpu(pre, "bf16")
    desc = gl.make_desc(2, 1, 2, 128, 128, T=1, act="bf16")
    states = dev(s)
    o = torch.empty(2, 2, 128, device="cuda")
    last = {k: v[:, 128].contiguous() for k, v in x.items()}
    gl.gdn_scan_decode(desc, dev(last["q"]), dev(last["k"]), dev(last["v"]), dev(last["alpha"]),
                       dev(last["beta"]), states, o)
    torch.cuda.synchronize()
    ro, _ = oracle.scan(x["q"], x["k"], x["v"], x["alpha"], x["beta"])
    assert rel_err(o.cpu(), ro[:, 128]) <= TOL_BF16


def test_stage_timer_stride():
    """A timer with stride 3 arms the 3rd and 6th of six launches of its stage, and only those."""
    say("[timer] stride 3 over six decode launches")
    N, H, D = 2, 2, 64
    desc = gl.make_desc(N, 1, H, D, D, T=1, act="f32")
    g = torch.Generator().manual_seed(7)
    q, k, v = (torch.randn(N, H, D, generator=g).cuda() for _ in range(3))
    al, be = torch.full((N, H), 0.9).cuda(), torch.full((N, H), 0.5).cuda()
    S = torch.zeros(N, H, D, D).cuda()
    o = torch.empty(N, H, D).cuda()
    t = gl.gdn_timer_create(gl.GDN_STAGE_DECODE, 8)
    try:
        gl.gdn_timer_set_stride(t, 3)
        gl.gdn_timer_attach(t)
        for _ in range(6):
            gl.gdn_scan_decode(desc, q, k, v, al, be, S, o)
        torch.cuda.synchronize()
        gl.gdn_timer_detach()
        n, ms = gl.gdn_timer_read(t)
        assert n == 2 and ms > 0
        gl.gdn_timer_reset(t)
        assert gl.gdn_timer_read(t)[0] == 0
    finally:
        gl.gdn_timer_detach()
        gl.gdn_timer_destroy(t)
