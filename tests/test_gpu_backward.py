"""GPU parity of the scan's backward pass (gdn_scan_backward) against the oracle's reverse recurrence.

Inputs are the seeded draws of ``synth.scan_inputs`` and ``synth.grad_inputs`` (identical on both sides);
the loss is <d_o, o> + <d_sfinal, S_final>.  Every gradient (dq, dk, dv, dalpha, dbeta, ds_init) is held to
the bar of its workload with the metric of tests/helpers.py: 1e-4 for fp32 inputs, 3e-3 for bf16 inputs.
The oracle itself is pinned by finite differences of the forward oracle (tests/test_oracle_pins.py).
Outputs and workspace are NaN-poisoned, with canaries past every output.
"""
import numpy as np
import pytest
import torch

import looped_linear_attention_amd as gl
import oracle
import synth
from helpers import TOL_BF16, TOL_F32, canary_intact, dev, padded, poison_, rel_err, say

pytestmark = pytest.mark.gpu


def _backward_gpu(x, g, act):
    B, L, H, D = x["q"].shape
    desc = gl.make_desc(B, L, H, D, D, T=1, act=act)
    ws = poison_(gl.workspace(desc, gl.GDN_OP_SCAN_BACKWARD))
    outs = {}
    bufs = {}
    for name, shape in (("dq", (B, L, H, D)), ("dk", (B, L, H, D)), ("dv", (B, L, H, D)), ("dalpha", (B, L, H)),
                        ("dbeta", (B, L, H)), ("ds_init", (B, H, D, D))):
        outs[name], bufs[name] = padded(shape)
    si = x.get("s_init")
    gl.gdn_scan_backward(desc, dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(x["alpha"]), dev(x["beta"]),
                         None if si is None else dev(si), dev(g["d_o"]),
                         None if g.get("d_sfinal") is None else dev(g["d_sfinal"]),
                         outs["dq"], outs["dk"], outs["dv"], outs["dalpha"], outs["dbeta"], outs["ds_init"], ws)
    torch.cuda.synchronize()
    for name, t in outs.items():
        assert canary_intact(bufs[name], t.numel()), name
        assert bool(torch.isfinite(t).all()), name
    return {k: v.cpu() for k, v in outs.items()}


CASES = [
    # (B, L, H, D, act, alpha_range, beta_range, with_state, with_state_grad)
    (1, 64, 1, 128, "bf16", (0.0, 1.0), (0.0, 1.0), False, False),
    (1, 1, 1, 128, "bf16", (0.0, 1.0), (0.0, 1.0), True, True),
    (2, 65, 2, 128, "bf16", (0.0, 1.0), (0.0, 1.0), True, True),
    (1, 200, 2, 64, "bf16", (0.5, 1.0), (0.0, 1.0), True, True),
    (1, 130, 1, 64, "f32", (0.5, 1.0), (0.0, 1.0), True, True),
    (2, 96, 2, 64, "f32", (0.0, 1.0), (0.0, 1.0), False, True),
    (1, 300, 2, 128, "bf16", (0.3, 1.0), (0.0, 2.0), True, True),   # negative eigenvalues (beta up to 2)
    (1, 300, 2, 128, "bf16", (1.0, 1.0), (0.0, 1.0), True, True),   # no decay (alpha = 1)
    (3, 1000, 16, 128, "bf16", (0.5, 1.0), (0.0, 1.0), True, True),  # forward recomputation on 32-column slices
]


@pytest.mark.parametrize("B,L,H,D,act,ar,br,ws,wg", CASES)
def test_scan_backward_parity(B, L, H, D, act, ar, br, ws, wg):
    say(f"[scan_backward] B={B} L={L} H={H} D={D} act={act} alpha={ar} beta={br} s_init={ws} d_sfinal={wg}")
    x = synth.scan_inputs(500 + L + D, B, L, H, D, D, act=act, alpha_range=ar, beta_range=br, with_state=ws)
    g = synth.grad_inputs(600 + L, B, L, H, D, D, with_state_grad=wg)
    got = _backward_gpu(x, g, act)
    ref = oracle.scan_backward(x["q"], x["k"], x["v"], x["alpha"], x["beta"], g["d_o"], x.get("s_init"),
                               g.get("d_sfinal"))
    tol = TOL_F32 if act == "f32" else TOL_BF16
    errs = {name: rel_err(got[name], ref[name]) for name in ("dq", "dk", "dv", "dalpha", "dbeta", "ds_init")}
    say("    " + "  ".join(f"{k} {v:.2e}" for k, v in errs.items()))
    assert max(errs.values()) <= tol, errs


def test_scan_backward_full_size_b1_l4096():
    """The 4096-token, 16-head shape of the prompt workloads (alpha in (0.9, 1))."""
    say("[scan_backward] B=1 L=4096 H=16 D=128 bf16")
    x = synth.scan_inputs(77, 1, 4096, 16, 128, 128, act="bf16", alpha_range=(0.9, 1.0), with_state=True)
    g = synth.grad_inputs(78, 1, 4096, 16, 128, 128)
    got = _backward_gpu(x, g, "bf16")
    ref = oracle.scan_backward(x["q"], x["k"], x["v"], x["alpha"], x["beta"], g["d_o"], x["s_init"], g["d_sfinal"])
    errs = {name: rel_err(got[name], ref[name]) for name in ("dq", "dk", "dv", "dalpha", "dbeta", "ds_init")}
    say("    " + "  ".join(f"{k} {v:.2e}" for k, v in errs.items()))
    assert max(errs.values()) <= TOL_BF16, errs


def test_scan_backward_deterministic():
    x = synth.scan_inputs(5, 2, 333, 4, 128, 128, act="bf16", with_state=True)
    g = synth.grad_inputs(6, 2, 333, 4, 128, 128)
    a, b = _backward_gpu(x, g, "bf16"), _backward_gpu(x, g, "bf16")
    assert all(torch.equal(a[k], b[k]) for k in a)
