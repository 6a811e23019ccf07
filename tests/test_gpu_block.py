"""GPU parity of the LT2 block around the mixer (gdn_block_forward, gdn_block_loop_prefill) against the oracle.

fp32: the T-loop stack of two blocks free-running against oracle.block_loop_prefill at 1e-4 (nothing is rounded
to bf16, so the result is unique up to fp32 rounding).

bf16: one block, stage-forced: each stage is checked on the inputs it actually received, read from the
documented workspace regions (x1, the mixer's q/k/v/gates, o, z, h1, x2, u) -- a value within summation error
of a bf16 boundary may round either way in a valid implementation, so each bf16 store is held to one bf16 step
plus the fp32 summation bound of the products that fed it:
  x1 = bf16(RMSNorm(h; g1))             one bf16 step plus the norm's fp32 error
  q, k, v, gates                        the projection bound of tests/helpers.py (as in the loop tests)
  o = scan(GPU q, k, v; oracle gates)   3e-3 (the scan's bar)
  z = bf16(o (.) sigmoid(x1 Wg))        one bf16 step plus |o| sigma' gamma_K sum|x1||Wg|
  h1 = h + z Wo                         gamma_K sum|z||Wo| plus fp32 rounding
  x2 = bf16(RMSNorm(h1; g2))            one bf16 step plus the norm's fp32 error
  u = bf16(silu(x2 W1) (.) (x2 W3))     one bf16 step plus the products' fp32 summation bounds
  out = h1 + u W2                       gamma_K sum|u||W2| plus fp32 rounding
(gamma_K = K 2^-24 / (1 - K 2^-24), the recursive-summation bound for K terms in fp32, any order.)
The bf16 loop stack is checked against the composition of gdn_block_forward calls on the GPU.
"""
import numpy as np
import pytest
import torch

import looped_linear_attention_amd as gl
import oracle
import synth
from helpers import TOL_BF16, TOL_F32, _np64, bf16_ulp, canary_intact, check_projection, dev, padded, poison_, \
    rel_err, say

pytestmark = pytest.mark.gpu

_KEYS = ("g1", "Wq", "Wk", "Wv", "wa", "wb", "Wg", "Wo", "g2", "W1", "W3", "W2")


def _pack(desc, F, blocks):
    n = gl.gdn_block_packed_bytes(desc, F)
    buf = torch.empty(len(blocks) * n, dtype=torch.uint8, device="cuda")
    for i, b in enumerate(blocks):
        gl.gdn_block_pack(desc, F, *[dev(b[k]) for k in _KEYS], buf[i * n:(i + 1) * n])
    return buf


def _gamma(K):
    u = K * 2.0 ** -24
    return u / (1 - u)


def _check_rounded(name, g, r, bound):
    """g is a bf16 store of a value whose exact form is r: against r rounded to bf16, |g - bf16(r)| <= bound +
    one bf16 step at max(|g|, |r|) (the two may round to neighbours where r lies within the bound of a
    rounding boundary), and few elements differ at all."""
    g, r = _np64(g), oracle.round_bf16(_np64(r))
    diff = np.abs(g - r)
    step = bf16_ulp(np.maximum(np.abs(r), np.abs(g)))
    excess = float((diff - bound - step * 1.0001).max())
    frac = float(np.mean(diff > 0))
    say(f"    {name}: max excess over bound {excess:.2e}, elements differing {frac:.1e}")
    assert excess <= 0, name
    assert frac < 0.01, name


def _check_fp32(name, g, r, bound):
    g, r = _np64(g), _np64(r)
    diff = np.abs(g - r)
    excess = float((diff - bound - 2.0 ** -23 * np.abs(r)).max())
    say(f"    {name}: max excess over bound {excess:.2e}, max-rel {rel_err(g, r):.1e}")
    assert excess <= 0, name


def test_block_loop_tiny_f32():
    w = synth.workload("tiny_f32")
    F = synth.block_ffn(w)
    say(f"[block] tiny_f32, 2 blocks, T={w.T}, ffn={F}")
    x = synth.prefill_inputs(w)
    blocks = synth.block_inputs(w, 2)
    desc = gl.make_desc(w.B, w.L, w.H, w.dk, w.dv, T=w.T, act=w.act, alpha_lo=w.alpha_lo)
    Wb = _pack(desc, F, blocks)
    ws = poison_(gl.block_workspace(desc, F))
    h_out, hb = padded((w.B, w.L, w.d))
    gl.gdn_block_loop_prefill(desc, F, 2, dev(x["h0"]), Wb, dev(x["rho"]), h_out, ws)
    torch.cuda.synchronize()
    assert canary_intact(hb, h_out.numel()) and bool(torch.isfinite(h_out).all())
    ref = oracle.block_loop_prefill(x["h0"], blocks, x["rho"], w.H, w.dk, w.dv, w.alpha_lo, w.act)["h"]
    e = rel_err(h_out.cpu(), ref)
    say(f"    h^(T) max-rel {e:.2e} (bar {TOL_F32:.0e})")
    assert e <= TOL_F32


def _block_forward_gpu(w, F, blk, h):
    B, L, d = h.shape
    desc = gl.make_desc(B, L, w.H, w.dk, w.dv, T=1, act=w.act, alpha_lo=w.alpha_lo)
    Wb = _pack(desc, F, [blk])
    ws = poison_(gl.block_workspace(desc, F))
    out, ob = padded((B, L, d))
    gl.gdn_block_forward(desc, F, dev(h), Wb, out, ws)
    torch.cuda.synchronize()
    assert canary_intact(ob, out.numel()) and bool(torch.isfinite(out).all())
    reg = {r: gl.block_workspace_view(ws, desc, F, r).cpu()
           for r in (gl.GDN_BWS_X1, gl.GDN_WS_Q, gl.GDN_WS_K, gl.GDN_WS_V, gl.GDN_WS_ALPHA, gl.GDN_WS_BETA,
                     gl.GDN_BWS_O, gl.GDN_BWS_Z, gl.GDN_BWS_H1, gl.GDN_BWS_X2, gl.GDN_BWS_U)}
    return out.cpu(), reg, desc, Wb


def _norm_ref(h, g, eps=1e-6):
    """RMSNorm in fp64 and a bound on the fp32 computation's error (sum of squares, 1/sqrt, two products)."""
    r = oracle.rms_norm(h, g, eps)
    return r, np.abs(r) * (_gamma(h.shape[-1]) + 4 * 2.0 ** -24)


def _stage_forced(w, B, L, seed=0):
    F = synth.block_ffn(w)
    blk = synth.block_inputs(w, 1, seed=11 + seed)[0]
    rng = np.random.default_rng(500 + seed)
    h = torch.from_numpy(rng.standard_normal((B, L, w.d), dtype=np.float32))
    out, reg, desc, _ = _block_forward_gpu(w, F, blk, h)
    M, d, HD = B * L, w.d, w.H * w.dv
    W = {k: _np64(v) for k, v in blk.items()}
    hh = _np64(h).reshape(M, d)
    # x1
    x1 = _np64(reg[gl.GDN_BWS_X1])
    r, b = _norm_ref(hh, W["g1"])
    _check_rounded("x1", x1, r, b)
    # the mixer: projections of the GPU's x1, then the scan on the GPU's q/k/v
    gq, gk, gv, ga, gb = (reg[k] for k in (gl.GDN_WS_Q, gl.GDN_WS_K, gl.GDN_WS_V, gl.GDN_WS_ALPHA, gl.GDN_WS_BETA))
    ra, rb = check_projection(gq, gk, gv, ga, gb, x1, W["Wq"], W["Wk"], W["Wv"], W["wa"], W["wb"], w.H, w.dk, w.dv,
                              w.alpha_lo, w.act)
    o_ref, _ = oracle.scan(gq.reshape(B, L, w.H, w.dk), gk.reshape(B, L, w.H, w.dk), gv.reshape(B, L, w.H, w.dv),
                           ra.reshape(B, L, w.H), rb.reshape(B, L, w.H), want_state=False)
    o = _np64(reg[gl.GDN_BWS_O])
    eo = rel_err(o, o_ref.reshape(M, HD))
    say(f"    o: max-rel {eo:.2e} (bar {TOL_BF16:.0e})")
    assert eo <= TOL_BF16
    # z = o (.) sigmoid(x1 Wg) on the GPU's o and x1
    a = x1 @ W["Wg"]
    sg = 1.0 / (1.0 + np.exp(-a))
    _check_rounded("z", _np64(reg[gl.GDN_BWS_Z]), o * sg,
                   np.abs(o) * 0.25 * _gamma(d) * (np.abs(x1) @ np.abs(W["Wg"])) + np.abs(o * sg) * 2.0 ** -22)
    # h1 = h + z Wo
    z = _np64(reg[gl.GDN_BWS_Z])
    h1_ref = hh + z @ W["Wo"]
    h1 = _np64(reg[gl.GDN_BWS_H1])
    _check_fp32("h1", h1, h1_ref, _gamma(HD + 1) * (np.abs(hh) + np.abs(z) @ np.abs(W["Wo"])))
    # x2
    x2 = _np64(reg[gl.GDN_BWS_X2])
    r, b = _norm_ref(h1, W["g2"])
    _check_rounded("x2", x2, r, b)
    # u = silu(x2 W1) (.) (x2 W3)
    p1, p3 = x2 @ W["W1"], x2 @ W["W3"]
    e1 = _gamma(d) * (np.abs(x2) @ np.abs(W["W1"]))
    e3 = _gamma(d) * (np.abs(x2) @ np.abs(W["W3"]))
    s1 = 1.0 / (1.0 + np.exp(-p1))
    silu = p1 * s1
    u_ref = silu * p3
    dsilu = 1.1   # |d silu / da| <= 1.1 everywhere
    _check_rounded("u", _np64(reg[gl.GDN_BWS_U]), u_ref,
                   dsilu * e1 * (np.abs(p3) + e3) + np.abs(silu) * e3 + np.abs(u_ref) * 2.0 ** -21)
    # out = h1 + u W2
    u = _np64(reg[gl.GDN_BWS_U])
    out_ref = h1 + u @ W["W2"]
    F_ = u.shape[1]
    _check_fp32("out", _np64(out).reshape(M, d), out_ref, _gamma(F_ + 1) * (np.abs(h1) + np.abs(u) @ np.abs(W["W2"])))


@pytest.mark.parametrize("name,B,L", [("prefill_b1_l4096", 1, 300), ("prefill_b4_l8192", 2, 130),
                                      ("prefill_b1_l32768", 1, 1100)])
def test_block_forward_bf16_stage_forced(name, B, L):
    w = synth.workload(name)
    say(f"[block] {name} B={B} L={L}, stage-forced")
    _stage_forced(w, B, L)


def test_block_forward_bf16_full_b1_l4096():
    w = synth.workload("prefill_b1_l4096")
    say("[block] prefill_b1_l4096 full size, stage-forced")
    _stage_forced(w, 1, 4096, seed=1)


def test_block_loop_bf16_is_the_composition_of_blocks():
    """gdn_block_loop_prefill with T = 1 and two blocks equals gdn_block_forward twice plus rho (.) h0 (the
    loop fuses the residual into the last product's epilogue: fp32 rounding apart)."""
    w = synth.workload("prefill_b1_l4096")
    F = synth.block_ffn(w)
    B, L = 1, 500
    x = synth.prefill_inputs(w, B=B, L=L)
    blocks = synth.block_inputs(w, 2, seed=21)
    desc = gl.make_desc(B, L, w.H, w.dk, w.dv, T=1, act=w.act, alpha_lo=w.alpha_lo)
    Wb = _pack(desc, F, blocks)
    ws = poison_(gl.block_workspace(desc, F))
    h_out = torch.empty(B, L, w.d, device="cuda")
    h0 = dev(x["h0"])
    rho = dev(x["rho"][:1])
    gl.gdn_block_loop_prefill(desc, F, 2, h0, Wb, rho, h_out, ws)
    n = gl.gdn_block_packed_bytes(desc, F)
    h0f = h0.float()
    y1 = torch.empty_like(h0f)
    y2 = torch.empty_like(h0f)
    gl.gdn_block_forward(desc, F, h0f, Wb[:n], y1, ws)
    gl.gdn_block_forward(desc, F, y1, Wb[n:], y2, ws)
    ref = y2 + rho[0] * h0f
    torch.cuda.synchronize()
    e = rel_err(h_out.cpu(), ref.cpu())
    say(f"    loop vs composition: max-rel {e:.1e}")
    assert e <= 1e-6
