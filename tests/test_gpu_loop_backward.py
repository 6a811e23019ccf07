"""GPU parity of the backward through the T loops (gdn_loop_backward) against oracle.loop_backward.

The forward activations h^(1..T-1) are an input of the backward: the GPU's own loop prefill writes them
(h_loops) and both sides take that same array, so the comparison starts from identical loop inputs.  For
bf16 workloads the comparison is also stage-forced at the forward's rounding points: the oracle's scan
backward takes, for each loop tau, the bf16 q, k, v that the GPU forward computed in loop tau (read from the
documented workspace regions after a call with T = tau), since a value within summation error of a bf16
boundary may round either way in a valid forward and the gradient depends on the side it fell (summing the
raw projections in fp32 instead of fp64 alone moves the oracle's own bf16 dWq by 3.4e-3 on two 130-token
sequences).  Everything else -- the normalisation's and the gates' gradients, the products, rho's gradient --
is the oracle's own fp64 arithmetic.  The GPU backward recomputes each loop with the forward's own kernels,
so its q, k, v are those same values.  The incoming gradient dh = dL/dh^(T) is a seeded N(0, 1) draw.  Every
output (dh0, dWq, dWk, dWv, dwa, dwb, drho) is held to its workload's bar with the metric of
tests/helpers.py: 1e-4 for the fp32 workload (free-running from the same h_loops: nothing is rounded to
bf16), 3e-3 for the bf16 ones.  The oracle is pinned by finite differences of the forward loop
(tests/test_oracle_pins.py).  Outputs and workspace are NaN-poisoned, with canaries past every output.
"""
import numpy as np
import pytest
import torch

import looped_linear_attention_amd as gl
import oracle
import synth
from helpers import TOL_BF16, TOL_F32, canary_intact, dev, padded, poison_, rel_err, say

pytestmark = pytest.mark.gpu

_OUTS = ("dh0", "dWq", "dWk", "dWv", "dwa", "dwb", "drho")


def _run(w, B, L, seed=90):
    x = synth.prefill_inputs(w, B=B, L=L)
    desc = gl.make_desc(B, L, w.H, w.dk, w.dv, T=w.T, act=w.act, alpha_lo=w.alpha_lo)
    Wp = torch.empty(gl.gdn_weights_packed_bytes(desc) // (4 if w.act == "f32" else 2), dtype=desc.act_dtype,
                     device="cuda")
    gl.gdn_weights_pack(desc, dev(x["Wq"]), dev(x["Wk"]), dev(x["Wv"]), dev(x["wa"]), dev(x["wb"]), Wp)
    h0, rho = dev(x["h0"][:B, :L]), dev(x["rho"])
    h_out = torch.empty(B, L, w.d, device="cuda")
    h_loops = torch.empty(w.T, B, L, w.d, device="cuda")
    gl.gdn_loop_prefill(desc, h0, Wp, rho, h_out, None, h_loops, gl.workspace(desc, gl.GDN_OP_LOOP_PREFILL))
    dh = synth.grad_inputs(seed, B, L, w.H, w.dk, w.dv, with_state_grad=False)["d_o"].reshape(B, L, w.d)
    ws = poison_(gl.workspace(desc, gl.GDN_OP_LOOP_BACKWARD))
    shapes = dict(dh0=(B, L, w.d), dWq=(w.d, w.H * w.dk), dWk=(w.d, w.H * w.dk), dWv=(w.d, w.H * w.dv),
                  dwa=(w.d, w.H), dwb=(w.d, w.H), drho=(w.T, w.d))
    outs, bufs = {}, {}
    for k, sh in shapes.items():
        outs[k], bufs[k] = padded(sh)
    dh_dev = dev(dh)
    gl.gdn_loop_backward(desc, h0, Wp, rho, h_loops, dh_dev, *[outs[k] for k in _OUTS], ws)
    torch.cuda.synchronize()
    for k, t in outs.items():
        assert canary_intact(bufs[k], t.numel()), k
        assert bool(torch.isfinite(t).all()), k
    assert torch.equal(dh_dev.cpu(), dh)   # the incoming gradient is read only
    loops = [h_loops[i].cpu() for i in range(w.T)]
    qkv = _forward_operands(w, h0, Wp, rho, B, L) if w.act == "bf16" else None
    ref = oracle.loop_backward(x["h0"][:B, :L], x["Wq"], x["Wk"], x["Wv"], x["wa"], x["wb"], x["rho"], loops, dh,
                               w.H, w.dk, w.dv, w.alpha_lo, w.act, qkv=qkv)
    return {k: v.cpu() for k, v in outs.items()}, ref


def _forward_operands(w, h0, Wp, rho, B, L):
    """Loop tau's bf16 q, k, v as the GPU forward computed them, for tau = 1..T."""
    op = gl.GDN_OP_LOOP_PREFILL
    out = []
    for tau in range(1, w.T + 1):
        desc = gl.make_desc(B, L, w.H, w.dk, w.dv, T=tau, act=w.act, alpha_lo=w.alpha_lo)
        ws = poison_(gl.workspace(desc, op))
        gl.gdn_loop_prefill(desc, h0, Wp, rho[:tau].contiguous(), torch.empty(B, L, w.d, device="cuda"), None,
                            None, ws)
        out.append(tuple(gl.workspace_view(ws, desc, op, r).cpu() for r in (gl.GDN_WS_Q, gl.GDN_WS_K, gl.GDN_WS_V)))
    return out


def _check(name, got, ref, tol):
    errs = {k: rel_err(got[k], ref[k]) for k in _OUTS}
    say(f"    {name}: " + ", ".join(f"{k} {e:.1e}" for k, e in errs.items()) + f" (bar {tol:.0e})")
    for k, e in errs.items():
        assert e <= tol, (k, e)


def test_loop_backward_tiny_f32():
    w = synth.workload("tiny_f32")
    say("[loop_backward] tiny_f32")
    got, ref = _run(w, w.B, w.L)
    _check("tiny_f32", got, ref, TOL_F32)


@pytest.mark.parametrize("name,B,L", [("prefill_b1_l4096", 1, 300), ("prefill_b4_l8192", 2, 130),
                                      ("prefill_b1_l32768", 1, 65)])
def test_loop_backward_bf16(name, B, L):
    w = synth.workload(name)
    say(f"[loop_backward] {name} B={B} L={L}")
    got, ref = _run(w, B, L)
    _check(f"{name} B={B} L={L}", got, ref, TOL_BF16)


def test_loop_backward_full_size_b1_l4096():
    """The 4096-token prompt in full (16 heads of 128, d = 2048, T = 4): the shape the bench times."""
    w = synth.workload("prefill_b1_l4096")
    say("[loop_backward] prefill_b1_l4096 full size")
    got, ref = _run(w, w.B, w.L)
    _check("prefill_b1_l4096", got, ref, TOL_BF16)


def test_loop_backward_deterministic():
    w = synth.workload("prefill_b1_l4096")
    a, _ = _run(w, 1, 200, seed=91)
    b, _ = _run(w, 1, 200, seed=91)
    for k in _OUTS:
        assert torch.equal(a[k], b[k]), k
