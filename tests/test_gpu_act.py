"""GPU parity of the looped mixer with per-token adaptive halting (gdn_loop_prefill_act, LT2 Appendix A).

fp32: free-running against oracle.loop_prefill_act at 1e-4, with the same halting loops.  bf16: stage-forced
per loop as in test_gpu_loop.py: loop tau is checked from the GPU's own h^(tau-1) and halting state (read from a
call with T = tau - 1): the projection (fp32 summation bound plus one bf16 step), the scan with the residual
withheld from halted positions (3e-3; halted rows unchanged bit for bit), and the halting sums (1e-5) and
decisions.  The decision is an integer taken in fp32 on both sides, with the dot product summed in different
orders, so a decision may differ only where the oracle's running sum lies within 1e-5 of the threshold.
"""
import numpy as np
import pytest
import torch

import looped_linear_attention_amd as gl
import oracle
import synth
from helpers import TOL_BF16, TOL_F32, check_projection, dev, padded, poison_, rel_err, say

pytestmark = pytest.mark.gpu


def _pack(w, x):
    desc = gl.make_desc(w.B, w.L, w.H, w.dk, w.dv, T=w.T, act=w.act, alpha_lo=w.alpha_lo)
    Wp = torch.empty(gl.gdn_weights_packed_bytes(desc) // (4 if w.act == "f32" else 2), dtype=desc.act_dtype,
                     device="cuda")
    gl.gdn_weights_pack(desc, dev(x["Wq"]), dev(x["Wk"]), dev(x["Wv"]), dev(x["wa"]), dev(x["wb"]), Wp)
    return Wp


def _act_gpu(w, x, a, B, L, T, Wp):
    desc = gl.make_desc(B, L, w.H, w.dk, w.dv, T=T, act=w.act, alpha_lo=w.alpha_lo)
    ws = poison_(gl.workspace(desc, gl.GDN_OP_LOOP_PREFILL_ACT))
    h_out, _ = padded((B, L, w.d))
    hl = torch.full((B, L), -7, dtype=torch.int32, device="cuda")
    pd, _ = padded((B, L))
    gl.gdn_loop_prefill_act(desc, dev(x["h0"][:B, :L]), Wp, dev(x["rho"][:T]), dev(a["w_halt"]), a["b_halt"],
                            a["eps"], h_out, hl, pd, ws)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(h_out).all()) and bool((hl >= 1).all()) and bool((hl <= T).all())
    ops = [gl.workspace_view(ws, desc, gl.GDN_OP_LOOP_PREFILL_ACT, r).cpu()
           for r in (gl.GDN_WS_Q, gl.GDN_WS_K, gl.GDN_WS_V, gl.GDN_WS_ALPHA, gl.GDN_WS_BETA)]
    return h_out.cpu(), hl.cpu().numpy(), pd.cpu().numpy(), ops


def test_act_tiny_f32_free_running():
    w = synth.workload("tiny_f32")
    say("[act] tiny_f32 free-running")
    x = synth.prefill_inputs(w)
    a = synth.act_inputs(w)
    g_h, g_hl, g_pd, _ = _act_gpu(w, x, a, w.B, w.L, w.T, _pack(w, x))
    r = oracle.loop_prefill_act(x["h0"], x["Wq"], x["Wk"], x["Wv"], x["wa"], x["wb"], x["rho"], a["w_halt"],
                                a["b_halt"], a["eps"], w.H, w.dk, w.dv, w.alpha_lo, w.act)
    counts = np.bincount(g_hl.ravel(), minlength=w.T + 1)[1:]
    say(f"    halting loops 1..{w.T}: {counts.tolist()}; h err {rel_err(g_h, r['h']):.2e}")
    assert len(set(g_hl.ravel().tolist())) > 1   # the positions halt at different loops
    assert np.array_equal(g_hl, r["halt_loop"])
    assert np.max(np.abs(g_pd - r["ponder"])) <= 1e-5
    assert rel_err(g_h, r["h"]) <= TOL_F32


@pytest.mark.parametrize("name,B,L", [("prefill_b1_l4096", 1, 4096), ("prefill_b4_l8192", 2, 700),
                                      ("prefill_b4_l8192", 3, 700), ("prefill_b1_l4096", 1, 65)])
def test_act_bf16_forced(name, B, L):
    w = synth.workload(name)
    say(f"[act] {name} B={B} L={L}, stage-forced")
    x = synth.prefill_inputs(w, B=B, L=L)
    a = synth.act_inputs(w)
    Wp = _pack(w, x)
    thr = np.float32(1.0) - np.float32(a["eps"])
    wh = a["w_halt"].numpy().astype(np.float32)
    f = lambda t: t.double().numpy()
    mats = (f(x["Wq"]), f(x["Wk"]), f(x["Wv"]), f(x["wa"]), f(x["wb"]))
    rho = x["rho"].double().numpy()
    h_prev = x["h0"][:B, :L].double().numpy()
    R_prev = np.zeros((B, L), dtype=np.float32)
    hl_prev = None
    M = B * L
    for tau in range(1, w.T + 1):
        g_h, g_hl, g_pd, (gq, gk, gv, ga, gb) = _act_gpu(w, x, a, B, L, tau, Wp)
        halted = R_prev >= thr
        xin = oracle.round_bf16(h_prev.reshape(M, w.d))
        ra, rb = check_projection(gq, gk, gv, ga, gb, xin, *mats, w.H, w.dk, w.dv, w.alpha_lo, w.act)
        o, _ = oracle.scan(gq.reshape(B, L, w.H, w.dk), gk.reshape(B, L, w.H, w.dk), gv.reshape(B, L, w.H, w.dv),
                           ra.reshape(B, L, w.H), rb.reshape(B, L, w.H), want_state=False)
        h_ref = np.where(halted[..., None], h_prev, o.reshape(B, L, w.d) + rho[tau - 1] * h_prev)
        gh = g_h.double().numpy()
        eh = rel_err(gh, h_ref)
        assert np.array_equal(gh[halted], h_prev[halted])    # halted positions frozen bit for bit
        z = g_h.numpy().astype(np.float32) @ wh + np.float32(a["b_halt"])
        p = (np.float32(1.0) / (np.float32(1.0) + np.exp(-z, dtype=np.float32))).astype(np.float32)
        R_ref = np.where(halted, R_prev, (R_prev + p).astype(np.float32))
        ep = float(np.max(np.abs(g_pd - R_ref)))
        flips = (g_pd >= thr) != (R_ref >= thr)
        near = np.abs(R_ref - thr) <= 1e-5
        newly = (g_pd >= thr) & ~halted
        say(f"    loop {tau}: h max-rel {eh:.2e} (bar {TOL_BF16:.0e}), halting sums {ep:.1e}, "
            f"halted before {int(halted.sum())}, newly {int(newly.sum())}, decision flips {int(flips.sum())}")
        assert eh <= TOL_BF16 and ep <= 1e-5 and not np.any(flips & ~near)
        # halting loops so far: earlier halts keep their loop, the rest read tau
        if hl_prev is not None:
            assert np.array_equal(g_hl[halted], hl_prev[halted])
        assert np.all(g_hl[~halted] == tau)
        h_prev, R_prev, hl_prev = gh, g_pd.astype(np.float32), g_hl
    assert 0 < int((hl_prev < w.T).sum()) < M   # some positions halted before loop T, some did not
