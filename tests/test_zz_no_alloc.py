"""gdn_loop_decode_noalloc: the looped decode step on the library's own device scratch array.

GPU: two calls in a row (64 sequences, then 16: a smaller input over the same scratch, which still holds the
first call's contents) must equal gdn_loop_decode with a caller workspace on the same inputs.  They run the
same kernels, so the results are expected bitwise equal; the gate is the 3e-3 bar of the bf16 workloads.
CPU: a step whose workspace exceeds the scratch array is refused on the host, before any device call.
"""
import ctypes

import numpy as np
import pytest
import torch

import looped_linear_attention_amd as gl
import synth
from helpers import TOL_BF16, dev, rel_err, say


def _inputs(w, N, seed):
    rng = np.random.default_rng(seed)
    h_t = torch.from_numpy(rng.standard_normal((N, w.d), dtype=np.float32)).to(torch.bfloat16)
    st = torch.from_numpy(rng.standard_normal((w.T, N, w.H, w.dk, w.dv), dtype=np.float32) * np.float32(0.02 ** 0.5))
    return h_t, st


@pytest.mark.gpu
def test_noalloc_decode_matches_workspace_decode():
    w = synth.workload("prefill_b1_l4096")
    x = synth.prefill_inputs(w, L=1)
    for N, seed in ((64, 1), (16, 2)):
        say(f"[noalloc] {N} sequences")
        desc = gl.make_desc(N, 1, w.H, w.dk, w.dv, T=w.T, act=w.act, alpha_lo=w.alpha_lo)
        Wp = torch.empty(gl.gdn_weights_packed_bytes(desc) // 2, dtype=torch.bfloat16, device="cuda")
        gl.gdn_weights_pack(desc, dev(x["Wq"]), dev(x["Wk"]), dev(x["Wv"]), dev(x["wa"]), dev(x["wb"]), Wp)
        h_t, st0 = _inputs(w, N, seed)
        h_t, rho = dev(h_t), dev(x["rho"])
        s_ref, s_new = dev(st0), dev(st0)
        h_ref = torch.empty(N, w.d, device="cuda")
        h_new = torch.full((N, w.d), float("nan"), device="cuda")
        ws = gl.workspace(desc, gl.GDN_OP_LOOP_DECODE)
        gl.gdn_loop_decode(desc, h_t, Wp, rho, s_ref, h_ref, ws)
        gl.gdn_loop_decode_noalloc(desc, h_t, Wp, rho, s_new, h_new)
        torch.cuda.synchronize()
        eh, es = rel_err(h_new.cpu(), h_ref.cpu()), rel_err(s_new.cpu(), s_ref.cpu())
        same = torch.equal(h_new, h_ref) and torch.equal(s_new, s_ref)
        say(f"    h err {eh:.1e}, states err {es:.1e}, bitwise equal: {same}")
        assert eh <= TOL_BF16 and es <= TOL_BF16


def test_noalloc_rejects_oversized_step():
    """bf16 at width 2048 needs 16,512 B of scratch per sequence (q/k/v, gates, the bf16 operand): 509
    sequences exceed the 8 MiB array and are refused before any device call (fake device addresses)."""
    lib = gl.load()
    ok = gl.make_desc(508, 1, 16, 128, 128, T=4)
    assert gl.gdn_workspace_bytes(ok, gl.GDN_OP_LOOP_DECODE) <= 8 << 20
    big = gl.make_desc(509, 1, 16, 128, 128, T=4)
    assert gl.gdn_workspace_bytes(big, gl.GDN_OP_LOOP_DECODE) > 8 << 20
    fake = ctypes.c_void_p(0x100000)
    st = lib.gdn_loop_decode_noalloc(ctypes.byref(big), fake, fake, fake, fake, ctypes.c_void_p(0x200000), None)
    assert st == -4 and "GDN_NOALLOC_SCRATCH_BYTES" in gl.gdn_last_error()
