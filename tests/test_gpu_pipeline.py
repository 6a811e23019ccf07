"""The loop prefill run as a pipeline over pieces (gdn_loop_prefill_set_pieces) against the same call run loop
by loop.

Every row's arithmetic is the same in both orders (the projection, the chunk preparation and the carry of a
chunk see the same operands; the state crosses a piece boundary through fp32 memory unchanged), so where both
orders take the same carry variant the outputs must agree bit for bit: h^(T), every h^(tau) and every loop's
final state.  Where the whole call takes the 32-column carry and the pieces the 16-column one, the pipelined
call is held to the oracle stage by stage at the fixed bf16 bar instead (check_forced_loops).
"""
import numpy as np
import pytest
import torch

import looped_linear_attention_amd as gl
import synth
from helpers import say
from test_gpu_loop import LoopRun, _pack, check_forced_loops

pytestmark = pytest.mark.gpu


@pytest.fixture
def pieces():
    """Sets the piece length for one test and restores the automatic setting afterwards."""
    yield gl.gdn_loop_prefill_set_pieces
    gl.gdn_loop_prefill_set_pieces(0)


def _both(w, x, B, L, piece, set_pieces):
    Wp = _pack(w, x)
    set_pieces(-1)
    ref = LoopRun(w, x, B, L, w.T, Wp=Wp)
    set_pieces(piece)
    assert gl.gdn_loop_prefill_pieces(ref.desc) > 0
    run = LoopRun(w, x, B, L, w.T, Wp=Wp)
    return ref, run


@pytest.mark.parametrize("B,L,piece", [(1, 3772, 1024), (2, 1100, 1024), (1, 4096, 2048), (2, 2500, 1024)])
def test_pieces_match_loop_by_loop(B, L, piece, pieces):
    """16 heads of 128 (the 16-column carry in both orders): pieces of one sequence with a ragged last piece
    (3772 = 1024 + 1024 + 1724 tokens, ending in a 60-token chunk), one piece per sequence, the automatic piece
    length, and two sequences of two pieces each."""
    w = synth.workload("prefill_b4_l8192")
    say(f"[pipeline] B={B} L={L} pieces of {piece} against loop by loop")
    x = synth.prefill_inputs(w, B=B, L=L)
    ref, run = _both(w, x, B, L, piece, pieces)
    assert torch.equal(run.h_out, ref.h_out)
    assert torch.equal(run.loops, ref.loops)
    assert torch.equal(run.states, ref.states)
    # the documented regions hold loop T's operands in both orders
    for a, b in zip(run.operands(), ref.operands()):
        assert torch.equal(a, b)


def test_pieces_repeat_bitwise(pieces):
    """Back-to-back pipelined calls on one stream (the second reuses the streams and events of the first) give
    the same bits."""
    w = synth.workload("prefill_b1_l4096")
    say("[pipeline] prefill_b1_l4096, three pipelined calls in a row")
    x = synth.prefill_inputs(w)
    pieces(1024)
    Wp = _pack(w, x)
    desc = gl.make_desc(w.B, w.L, w.H, w.dk, w.dv, T=w.T, act=w.act, alpha_lo=w.alpha_lo)
    ws = gl.workspace(desc, gl.GDN_OP_LOOP_PREFILL)
    h0, rho = x["h0"].to("cuda"), x["rho"].to("cuda")
    outs = []
    for _ in range(3):
        h = torch.empty(w.B, w.L, w.d, device="cuda")
        gl.gdn_loop_prefill(desc, h0, Wp, rho, h, None, None, ws)
        outs.append(h)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[1], outs[2])
    assert bool(torch.isfinite(outs[0]).all())


def test_pieces_on_side_stream(pieces):
    """A pipelined call on a non-default torch stream orders against that stream: work queued after it sees
    its outputs (here a copy of h_out made on the same stream), and it starts after what was queued before
    (h0 filled on that stream just before the call)."""
    w = synth.workload("prefill_b1_l4096")
    say("[pipeline] prefill_b1_l4096 on a side stream")
    x = synth.prefill_inputs(w)
    Wp = _pack(w, x)
    desc = gl.make_desc(w.B, w.L, w.H, w.dk, w.dv, T=w.T, act=w.act, alpha_lo=w.alpha_lo)
    pieces(-1)
    ref = LoopRun(w, x, w.B, w.L, w.T, Wp=Wp, keep=False).h_out
    pieces(1024)
    ws = gl.workspace(desc, gl.GDN_OP_LOOP_PREFILL)
    rho = x["rho"].to("cuda")
    h0_src = x["h0"].to("cuda")
    h0 = torch.zeros_like(h0_src)
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        h0.copy_(h0_src)
        h = torch.empty(w.B, w.L, w.d, device="cuda")
        gl.gdn_loop_prefill(desc, h0, Wp, rho, h, None, None, ws, stream=s)
        h_copy = h.clone()
    s.synchronize()
    assert torch.equal(h_copy, ref)


def test_pieces_headline_shape_stage_forced(pieces):
    """4 x 8192 tokens in pieces of 2048: the whole call takes the 32-column carry, the pieces the 16-column
    one, so the pipelined call is checked against the oracle, stage by stage at 3e-3, on every token of two
    heads (on different XCDs)."""
    w = synth.workload("prefill_b4_l8192")
    say("[pipeline] prefill_b4_l8192 in pieces of 2048, heads (3, 12), stage-forced")
    pieces(2048)
    # (the call with T = 1 runs loop by loop, on the 32-column carry: its h^(1) may differ in the last bits)
    check_forced_loops(w, synth.prefill_inputs(w), w.B, w.L, heads=(3, 12), prefix_bitwise=False)


@pytest.mark.parametrize("T,H,D,L,piece", [(5, 16, 128, 2500, 1024), (2, 16, 128, 4096, 2048), (4, 16, 64, 3000, 1024),
                                           (3, 8, 128, 2100, 1024)])
def test_pieces_other_loop_counts_and_heads(T, H, D, L, piece, pieces):
    """More loops than carry streams (T = 5: loops 1 and 4 share one), two loops, heads of 64 and eight heads: the
    pipelined call against the same call loop by loop, bit for bit (both take the 16-column carry)."""
    import dataclasses
    w = dataclasses.replace(synth.workload("prefill_b1_l4096"), name=f"bf16_t{T}_h{H}_d{D}", T=T, H=H, dk=D, dv=D,
                            d=H * D)
    say(f"[pipeline] T={T} H={H} D={D} L={L} pieces of {piece} against loop by loop")
    x = synth.prefill_inputs(w, L=L)
    ref, run = _both(w, x, 1, L, piece, pieces)
    assert torch.equal(run.h_out, ref.h_out)
    assert torch.equal(run.loops, ref.loops)
    assert torch.equal(run.states, ref.states)


def test_pieces_two_host_threads(pieces):
    """Two host threads issue pipelined calls at the same time, each on its own stream with its own workspace and
    outputs (the library's shared streams and events are taken in turn while a call enqueues): both results equal
    the same call run alone, bit for bit."""
    import threading
    w = synth.workload("prefill_b1_l4096")
    say("[pipeline] two host threads, pieces of 1024")
    x = synth.prefill_inputs(w)
    Wp = _pack(w, x)
    desc = gl.make_desc(w.B, w.L, w.H, w.dk, w.dv, T=w.T, act=w.act, alpha_lo=w.alpha_lo)
    pieces(1024)
    h0, rho = x["h0"].to("cuda"), x["rho"].to("cuda")
    ref = torch.empty(w.B, w.L, w.d, device="cuda")
    gl.gdn_loop_prefill(desc, h0, Wp, rho, ref, None, None, gl.workspace(desc, gl.GDN_OP_LOOP_PREFILL))
    torch.cuda.synchronize()
    outs, errors = [None, None], []
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    wss = [gl.workspace(desc, gl.GDN_OP_LOOP_PREFILL) for _ in range(2)]
    hs = [torch.empty(w.B, w.L, w.d, device="cuda") for _ in range(2)]
    torch.cuda.synchronize()

    def work(i):
        try:
            torch.cuda.set_device(0)
            for _ in range(3):
                gl.gdn_loop_prefill(desc, h0, Wp, rho, hs[i], None, None, wss[i], stream=streams[i])
            streams[i].synchronize()
            outs[i] = hs[i].clone()
        except Exception as e:   # reported below
            errors.append(e)

    th = [threading.Thread(target=work, args=(i,)) for i in range(2)]
    for t in th:
        t.start()
    for t in th:
        t.join(timeout=120)
    assert not errors, errors
    torch.cuda.synchronize()
    assert torch.equal(outs[0], ref) and torch.equal(outs[1], ref)


def test_pieces_stage_timers(pieces):
    """The stage timers record the pipelined call's launches (on the library's own streams): one projection, prep
    and carry per loop and piece."""
    w = synth.workload("prefill_b1_l4096")
    say("[pipeline] stage timers on a pipelined call")
    x = synth.prefill_inputs(w)
    Wp = _pack(w, x)
    desc = gl.make_desc(w.B, w.L, w.H, w.dk, w.dv, T=w.T, act=w.act, alpha_lo=w.alpha_lo)
    pieces(1024)
    ws = gl.workspace(desc, gl.GDN_OP_LOOP_PREFILL)
    h = torch.empty(w.B, w.L, w.d, device="cuda")
    h0, rho = x["h0"].to("cuda"), x["rho"].to("cuda")
    stages = (gl.GDN_STAGE_PROJECT, gl.GDN_STAGE_SCAN_PREP, gl.GDN_STAGE_SCAN_CARRY)
    timers = [gl.gdn_timer_create(s, 64) for s in stages]
    for t in timers:
        gl.gdn_timer_attach(t)
    gl.gdn_loop_prefill(desc, h0, Wp, rho, h, None, None, ws)
    torch.cuda.synchronize()
    gl.gdn_timer_detach()
    for t in timers:
        n, ms = gl.gdn_timer_read(t)
        gl.gdn_timer_destroy(t)
        assert n == w.T * 4 and ms > 0   # four pieces of 1024 tokens per loop
