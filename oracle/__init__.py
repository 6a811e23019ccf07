"""CPU oracle for the looped gated-delta-rule (GDN) token mixer.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  It shares no code
with the HIP library (``looped_linear_attention_amd``) and never imports it;
the two meet only through the seeded inputs of ``synth``.

Everything is computed in IEEE double precision.  Where the bf16 workloads
store a value in a narrower type, the oracle rounds at the same point
(fp64 -> fp32 -> bf16, round to nearest even), so both sides see the same
operands at each storage boundary.

Sources (LT2: Linear-Time Looped Transformers):
  * Section 2, "Looped Transformer (LT)" paragraph: h in R^{L x d}, N shared
    blocks reused for T iterations (weight tying, so the same projection
    weights in every loop).
  * Section 2, "LT2" paragraph: q_t, k_t in R^{dk}, v_t in R^{dv} are
    projections of h_t; S_t in R^{dk x dv}; the per-loop residual gate
    h^(tau) = h~^(tau) + rho_tau (.) h^(tau-1) with rho_tau in R^d per channel.
  * Appendix C: the mixer is Gated DeltaNet; T = 4; use_residual = true.
  * Appendix B.1 and Fig. 6 caption: rank-1 (diagonal-plus-low-rank) state
    update, data-dependent gating plus the delta rule, operator norm <= 1.
The recurrence itself (not printed on the pages) is read as the gated delta
rule of the GDN reference the pages cite; see ``gdn_scan_ref.c``.

Readings where the pages are silent (each also listed in the design notes):
  * h~^(tau) is the mixer output o itself (one mixer per loop, H*dv == d).
  * o_t = S_t^T q_t from the post-update state, no 1/sqrt(dk) factor.
  * every loop restarts its scan from S = 0 (one state per loop).
  * q, k are L2-normalised per head: x / sqrt(sum x^2 + eps), eps = 1e-6.
  * alpha = alpha_lo + (1 - alpha_lo) * sigmoid(-a), a = h . wa  (alpha_lo = 0
    gives exp(-softplus(a))); beta = sigmoid(h . wb); one gate pair per
    (token, head).
  * bf16 workloads round h (per-loop GEMM operand), the weights and q/k/v to
    bf16; alpha, beta, the state, o and the residual stream stay fp32.

Functions whose parity is pinned, and by what, are listed in
``tests/test_oracle_pins.py``; every oracle function here is pinned there.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_scan_ref.c")
_LIB_PATH = os.path.join(_HERE, "libgdn_oracle.so")
_lib = None

__all__ = [
    "build", "num_threads", "round_bf16", "round_f32", "scan", "scan_backward", "project",
    "loop_prefill", "loop_prefill_act", "loop_backward", "loop_decode_step", "scan_chunkwise",
    "ffn_width", "rms_norm", "block_forward", "block_loop_prefill",
]


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc: -O3 for x86-64-v3 (AVX2; the library built here also runs on
    other hosts, so not -march=native), no FMA contraction and no reassociation, so every product and sum
    is the IEEE double operation the source writes."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O3", "-march=x86-64-v3", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared",
               "-std=c99", "-o", tmp, _SRC]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=True)
        lib = ctypes.CDLL(_LIB_PATH)
        dp = ctypes.POINTER(ctypes.c_double)
        lib.oracle_scan.argtypes = [ctypes.c_int] * 5 + [dp] * 8
        lib.oracle_scan.restype = ctypes.c_int
        lib.oracle_scan_backward.argtypes = [ctypes.c_int] * 5 + [dp] * 14
        lib.oracle_scan_backward.restype = ctypes.c_int
        lib.oracle_num_threads.argtypes = []
        lib.oracle_num_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def num_threads() -> int:
    """Threads the C recurrence runs on (OpenMP)."""
    return int(_load().oracle_num_threads())


def _f64(x) -> np.ndarray:
    if hasattr(x, "detach"):  # torch tensor (bf16/fp32) -> exact fp64 values
        x = x.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a: Optional[np.ndarray]):
    if a is None:
        return ctypes.POINTER(ctypes.c_double)()
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


# ---------------------------------------------------------------------------
# storage rounding (the two sides round at the same points)
# ---------------------------------------------------------------------------
def round_f32(x) -> np.ndarray:
    """Round to the nearest fp32 (numpy's IEEE conversion), returned as fp64."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def round_bf16(x) -> np.ndarray:
    """fp64 -> fp32 -> bf16 with round-to-nearest-even, returned as fp64.

    bf16 keeps the upper 16 bits of the fp32 bit pattern.  Rounding to
    nearest even adds 0x7FFF plus the lowest kept bit before truncating
    (finite inputs; overflow correctly rounds to infinity).
    """
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    keep_lsb = (u >> np.uint64(16)) & np.uint64(1)
    u = (u + np.uint64(0x7FFF) + keep_lsb) & np.uint64(0xFFFF0000)
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


# ---------------------------------------------------------------------------
# the gated delta rule, token by token (C, fp64)
# ---------------------------------------------------------------------------
def scan(q, k, v, alpha, beta, s_init=None, want_state: bool = True):
    """One scan pass of the gated delta rule on given q, k, v, alpha, beta.

    q, k [B,L,H,dk]; v [B,L,H,dv]; alpha, beta [B,L,H]; s_init [B,H,dk,dv] or
    None (= zeros).  Returns (o [B,L,H,dv], s_final [B,H,dk,dv]) in fp64.
    No normalisation is applied here: q and k are used as given.
    """
    q, k, v, alpha, beta = map(_f64, (q, k, v, alpha, beta))
    B, L, H, dk = q.shape
    dv = v.shape[-1]
    assert k.shape == q.shape and v.shape[:3] == (B, L, H)
    assert alpha.shape == (B, L, H) and beta.shape == (B, L, H)
    si = None if s_init is None else _f64(s_init)
    if si is not None:
        assert si.shape == (B, H, dk, dv)
    o = np.zeros((B, L, H, dv), dtype=np.float64)
    sf = np.zeros((B, H, dk, dv), dtype=np.float64) if want_state else None
    rc = _load().oracle_scan(B, L, H, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
                             _ptr(beta), _ptr(si), _ptr(o), _ptr(sf))
    if rc != 0:
        raise MemoryError("oracle_scan could not allocate its state")
    return o, sf


def scan_backward(q, k, v, alpha, beta, d_o, s_init=None, d_sfinal=None):
    """Gradients of one scan pass (fp64, token by token in reverse; see gdn_scan_ref.c).

    Given d_o = dL/do [B,L,H,dv] and d_sfinal = dL/dS_final [B,H,dk,dv] (None: zero) for the scan of
    ``scan(q, k, v, alpha, beta, s_init)``, returns dict(dq, dk [B,L,H,dk], dv [B,L,H,dv], dalpha, dbeta
    [B,L,H], ds_init [B,H,dk,dv]).  q and k are treated as given (no normalisation).
    """
    q, k, v, alpha, beta, d_o = map(_f64, (q, k, v, alpha, beta, d_o))
    B, L, H, dk = q.shape
    dv = v.shape[-1]
    si = None if s_init is None else _f64(s_init)
    dsf = None if d_sfinal is None else _f64(d_sfinal)
    out = dict(dq=np.zeros((B, L, H, dk)), dk=np.zeros((B, L, H, dk)), dv=np.zeros((B, L, H, dv)),
               dalpha=np.zeros((B, L, H)), dbeta=np.zeros((B, L, H)), ds_init=np.zeros((B, H, dk, dv)))
    rc = _load().oracle_scan_backward(B, L, H, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                      _ptr(si), _ptr(d_o), _ptr(dsf), _ptr(out["dq"]), _ptr(out["dk"]),
                                      _ptr(out["dv"]), _ptr(out["dalpha"]), _ptr(out["dbeta"]),
                                      _ptr(out["ds_init"]))
    if rc != 0:
        raise MemoryError("oracle_scan_backward could not allocate its scratch")
    return out


# ---------------------------------------------------------------------------
# per-loop projections, normalisation and gates (numpy fp64)
# ---------------------------------------------------------------------------
def project(x, Wq, Wk, Wv, wa, wb, H: int, dk: int, dv: int, alpha_lo: float,
            act: str, eps: float = 1e-6):
    """Projections of one loop for token rows x [M, d] (already at operand precision).

    q = x Wq, k = x Wk, v = x Wv (head j owns columns [j*dk, (j+1)*dk)),
    a = x wa, b = x wb (one column per head).  q and k are L2-normalised per
    head; alpha = alpha_lo + (1 - alpha_lo) / (1 + e^a); beta = 1 / (1 + e^-b).
    For act == "bf16", q/k/v are then rounded fp64->fp32->bf16 and alpha, beta
    to fp32 (the precision they are stored in).
    """
    x = _f64(x)
    M = x.shape[0]
    Wq, Wk, Wv, wa, wb = map(_f64, (Wq, Wk, Wv, wa, wb))
    a = x @ wa
    b = x @ wb
    q = (x @ Wq).reshape(M, H, dk)
    k = (x @ Wk).reshape(M, H, dk)
    v = (x @ Wv).reshape(M, H, dv)
    q = q / np.sqrt(np.sum(q * q, axis=-1, keepdims=True) + eps)
    k = k / np.sqrt(np.sum(k * k, axis=-1, keepdims=True) + eps)
    alpha = alpha_lo + (1.0 - alpha_lo) / (1.0 + np.exp(a))
    beta = 1.0 / (1.0 + np.exp(-b))
    if act == "bf16":
        q, k, v = round_bf16(q), round_bf16(k), round_bf16(v)
        alpha, beta = round_f32(alpha), round_f32(beta)
    return q, k, v, alpha, beta


def loop_prefill(h0, Wq, Wk, Wv, wa, wb, rho, H: int, dk: int, dv: int,
                 alpha_lo: float, act: str, eps: float = 1e-6,
                 keep_loops: bool = False, keep_states: bool = False):
    """T weight-tied loops of the GDN mixer with the per-loop residual gate.

    h^(0) = h0 [B, L, d]; for tau = 1..T:
        x      = h^(tau-1)            (f32 workloads)
               = bf16(fp32(h^(tau-1))) (bf16 workloads: the GEMM operand)
        q,k,v,alpha,beta = project(x)
        o      = scan(q, k, v, alpha, beta) from S = 0
        h^(tau) = o.reshape(B, L, H*dv) + rho[tau-1] (.) h^(tau-1)
    Returns dict(h=h^(T) [B,L,d], loops=[h^(1..T)] or None,
    states=[S_final per loop, each [B,H,dk,dv]] or None).  fp64.
    """
    h = _f64(h0)
    rho = _f64(rho)
    B, L, d = h.shape
    T = rho.shape[0]
    assert H * dv == d, "the mixer output must have the width of the residual stream"
    loops, states = [], []
    for tau in range(T):
        x = round_bf16(h) if act == "bf16" else h
        q, k, v, al, be = project(x.reshape(B * L, d), Wq, Wk, Wv, wa, wb, H, dk, dv,
                                  alpha_lo, act, eps)
        o, s = scan(q.reshape(B, L, H, dk), k.reshape(B, L, H, dk), v.reshape(B, L, H, dv),
                    al.reshape(B, L, H), be.reshape(B, L, H), None, want_state=keep_states)
        h = o.reshape(B, L, d) + rho[tau][None, None, :] * h
        if keep_loops:
            loops.append(h.copy())
        if keep_states:
            states.append(s)
    return dict(h=h, loops=loops if keep_loops else None,
                states=states if keep_states else None)


def loop_backward(h0, Wq, Wk, Wv, wa, wb, rho, loops, dh, H: int, dk: int, dv: int, alpha_lo: float, act: str,
                  eps: float = 1e-6, qkv=None):
    """Gradients of ``loop_prefill`` (T weight-tied loops, LT2 Section 2; trained through, Appendix C) for an
    incoming gradient dh = dL/dh^(T) [B, L, d].

    ``loops`` holds the forward's h^(1..T) (``keep_loops``; only h^(1..T-1), the inputs of loops 2..T, are
    read).  Each loop tau = T..1 is recomputed from its input h^(tau-1) and then taken in reverse:
        x                     = h^(tau-1), or bf16(fp32(h^(tau-1))) for bf16 workloads
        qr, kr, v, a, b       = x Wq, x Wk, x Wv, x wa, x wb          (raw projections, per head)
        q = qr / r_q, k = kr / r_k with r = sqrt(|raw|^2 + eps) per (token, head)
        alpha = alpha_lo + (1 - alpha_lo) s, s = 1 / (1 + e^a);  beta = 1 / (1 + e^-b)
        dq, dk, dv, dalpha, dbeta = scan_backward(q, k, v, alpha, beta, d_o = dh)   (from S = 0; the loop's
                                    final state is not an output of the loss, so dS_final = 0)
        dqr = (dq - q (q . dq)) / r_q, likewise dkr          (through the L2 normalisation)
        da  = -dalpha (1 - alpha_lo) s (1 - s),  db = dbeta beta (1 - beta)
        dW* += x^T d*r  (q, k, v, a, b)
        drho_tau = sum over (b, l) of dh (.) h^(tau-1)
        dh <- rho_tau (.) dh + dqr Wq^T + dkr Wk^T + dv Wv^T + da wa^T + db wb^T
    For bf16 workloads the roundings of the forward (x, and q, k, v after normalisation) pass the gradient
    through unchanged: the scan backward is evaluated at the rounded q, k, v, everything else at the unrounded
    values.  ``qkv``, if given, holds for each loop 1..T the rounded (q, k, v) ([B*L, H, dk] / [.., dv]) to use
    there instead of this function's own roundings: a value within summation error of a bf16 rounding boundary
    may round either way in a valid forward, and the gradient depends on the side it fell.  Returns
    dict(dh0 [B,L,d], dWq, dWk [d,H*dk], dWv [d,H*dv], dwa, dwb [d,H], drho [T,d]).  fp64.
    """
    h0 = _f64(h0)
    rho = _f64(rho)
    B, L, d = h0.shape
    T = rho.shape[0]
    M = B * L
    Wq, Wk, Wv, wa, wb = map(_f64, (Wq, Wk, Wv, wa, wb))
    ins = [h0] + [_f64(h) for h in loops[:T - 1]]
    g = _f64(dh).reshape(M, d)
    out = dict(dWq=np.zeros_like(Wq), dWk=np.zeros_like(Wk), dWv=np.zeros_like(Wv), dwa=np.zeros_like(wa),
               dwb=np.zeros_like(wb), drho=np.zeros((T, d)))
    for tau in range(T - 1, -1, -1):
        hp = ins[tau].reshape(M, d)
        x = round_bf16(hp) if act == "bf16" else hp
        qr = (x @ Wq).reshape(M, H, dk)
        kr = (x @ Wk).reshape(M, H, dk)
        vr = (x @ Wv).reshape(M, H, dv)
        a, b = x @ wa, x @ wb
        rq = np.sqrt(np.sum(qr * qr, axis=-1, keepdims=True) + eps)
        rk = np.sqrt(np.sum(kr * kr, axis=-1, keepdims=True) + eps)
        qn, kn = qr / rq, kr / rk
        sg = 1.0 / (1.0 + np.exp(a))
        alpha = alpha_lo + (1.0 - alpha_lo) * sg
        beta = 1.0 / (1.0 + np.exp(-b))
        if act == "bf16":
            qs, ks, vs = round_bf16(qn), round_bf16(kn), round_bf16(vr)
            als, bes = round_f32(alpha), round_f32(beta)
        else:
            qs, ks, vs, als, bes = qn, kn, vr, alpha, beta
        if qkv is not None:
            qs, ks, vs = (_f64(t).reshape(M, H, -1) for t in qkv[tau])
        gs = scan_backward(qs.reshape(B, L, H, dk), ks.reshape(B, L, H, dk), vs.reshape(B, L, H, dv),
                           als.reshape(B, L, H), bes.reshape(B, L, H), g.reshape(B, L, H, dv))
        dq = gs["dq"].reshape(M, H, dk)
        dkn = gs["dk"].reshape(M, H, dk)
        dqr = (dq - qn * np.sum(qn * dq, axis=-1, keepdims=True)) / rq
        dkr = (dkn - kn * np.sum(kn * dkn, axis=-1, keepdims=True)) / rk
        dvr = gs["dv"].reshape(M, H * dv)
        da = -gs["dalpha"].reshape(M, H) * (1.0 - alpha_lo) * sg * (1.0 - sg)
        db = gs["dbeta"].reshape(M, H) * beta * (1.0 - beta)
        dqr, dkr = dqr.reshape(M, H * dk), dkr.reshape(M, H * dk)
        out["dWq"] += x.T @ dqr
        out["dWk"] += x.T @ dkr
        out["dWv"] += x.T @ dvr
        out["dwa"] += x.T @ da
        out["dwb"] += x.T @ db
        out["drho"][tau] = np.sum(g * hp, axis=0)
        g = rho[tau][None, :] * g + dqr @ Wq.T + dkr @ Wk.T + dvr @ Wv.T + da @ wa.T + db @ wb.T
    out["dh0"] = g.reshape(B, L, d)
    return out


# ---------------------------------------------------------------------------
# the LT2 block around the mixer
# ---------------------------------------------------------------------------
def ffn_width(d: int, multiple: int = 256) -> int:
    """Hidden width of the gated FFN: 8d/3 rounded up to a multiple of 256 (the training setup's "FFN
    multiple-of 256", read as the usual SwiGLU sizing; 5632 at d = 2048, 2816 at d = 1024)."""
    return multiple * ((8 * d // 3 + multiple - 1) // multiple)


def rms_norm(x, g, eps: float = 1e-6):
    """x / sqrt(mean(x^2) + eps) * g over the last axis (the pre-norm of each sub-layer)."""
    x = _f64(x)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * _f64(g)


def block_forward(h, wts: dict, H: int, dk: int, dv: int, alpha_lo: float, act: str, eps: float = 1e-6,
                  keep: bool = False):
    """One LT2 block F(h) (LT2 Section 2, "LT2" paragraph: the Transformer block of its Eq. (1) with the
    attention sub-layer replaced by the linear mixer; pre-norm per sub-layer; the head-specific sigmoid
    output gate of Gated Attention applied to the mixer output, as the attention-sink paragraph of Section 3
    adds it inside the looped block):
        x1 = rms_norm(h, g1)
        q, k, v, alpha, beta = project(x1)             (the mixer's projections, as in loop_prefill)
        o  = scan(q, k, v, alpha, beta) from S = 0
        z  = o (.) sigmoid(x1 Wg)                       (Wg [d, H dv]: one gate per head channel)
        h1 = h + z Wo                                   (Wo [H dv, d]; identity residual)
        x2 = rms_norm(h1, g2)
        u  = silu(x2 W1) (.) (x2 W3)                    (W1, W3 [d, F])
        F(h) = h1 + u W2                                (W2 [F, d]; identity residual)
    wts holds g1, Wq, Wk, Wv, wa, wb, Wg, Wo, g2, W1, W3, W2.  For bf16 workloads x1, q/k/v, z, x2 and u are
    rounded to bf16 (the operands of the products), h, h1, o, the statistics and the gates stay fp32.
    Returns F(h) [B, L, d] (fp64), or with keep a dict of every intermediate."""
    h = _f64(h)
    B, L, d = h.shape
    M = B * L
    rb = round_bf16 if act == "bf16" else (lambda t: t)
    W = {k_: _f64(v_) for k_, v_ in wts.items()}
    x1 = rb(rms_norm(h, W["g1"], eps)).reshape(M, d)
    q, k, v, al, be = project(x1, W["Wq"], W["Wk"], W["Wv"], W["wa"], W["wb"], H, dk, dv, alpha_lo, act, eps)
    o, _ = scan(q.reshape(B, L, H, dk), k.reshape(B, L, H, dk), v.reshape(B, L, H, dv), al.reshape(B, L, H),
                be.reshape(B, L, H), None, want_state=False)
    o = o.reshape(M, H * dv)
    gate = 1.0 / (1.0 + np.exp(-(x1 @ W["Wg"])))
    z = rb(o * gate)
    h1 = h.reshape(M, d) + z @ W["Wo"]
    x2 = rb(rms_norm(h1, W["g2"], eps))
    a, b = x2 @ W["W1"], x2 @ W["W3"]
    u = rb(a / (1.0 + np.exp(-a)) * b)
    out = (h1 + u @ W["W2"]).reshape(B, L, d)
    if keep:
        return dict(out=out, x1=x1, q=q, k=k, v=v, alpha=al, beta=be, o=o, z=z, h1=h1, x2=x2, u=u)
    return out


def block_loop_prefill(h0, layers, rho, H: int, dk: int, dv: int, alpha_lo: float, act: str, eps: float = 1e-6,
                       keep_loops: bool = False):
    """T loops of an N-block LT2 stack (LT2 Section 2): h^(tau) = (F_N o ... o F_1)(h^(tau-1)) + rho_tau (.)
    h^(tau-1), with the same N blocks (``layers``, a list of weight dicts) in every loop.  fp64."""
    h = _f64(h0)
    rho = _f64(rho)
    loops = []
    for tau in range(rho.shape[0]):
        x = h
        for wts in layers:
            x = block_forward(x, wts, H, dk, dv, alpha_lo, act, eps)
        h = x + rho[tau][None, None, :] * h
        if keep_loops:
            loops.append(h.copy())
    return dict(h=h, loops=loops if keep_loops else None)


def loop_prefill_act(h0, Wq, Wk, Wv, wa, wb, rho, w_halt, b_halt: float, eps: float, H: int, dk: int, dv: int,
                     alpha_lo: float, act: str, norm_eps: float = 1e-6, keep_loops: bool = False):
    """T weight-tied loops with per-token adaptive halting (LT2 Appendix A, adaptive computation time).

    As ``loop_prefill``, except that after each loop tau every position t that is still running draws a
    halting probability p_t = sigmoid(w_halt . h_t^(tau) + b_halt) and adds it to its running sum R_t; once
    R_t >= 1 - eps the position halts: its hidden state is frozen at h_t^(tau) and takes no further update.
    Every position is still projected and scanned in later loops (its frozen state remains context for the
    positions after it); only the residual update h = o + rho (.) h is withheld from halted positions.

    The halting decision is an integer decided by floating point; it is taken here as the library takes it,
    in fp32: the dot product w_halt . h_t is summed in fp32 (numpy, from the fp32 value of h), the sigmoid
    and the running sum in fp32.  Returns dict(h [B,L,d] fp64, halt_loop [B,L] int (tau_t, or T if the sum
    never reached the threshold), ponder [B,L] fp32 (R_t), loops [h^(1..T)] or None).
    """
    h = _f64(h0)
    rho = _f64(rho)
    B, L, d = h.shape
    T = rho.shape[0]
    w32 = np.asarray(_f64(w_halt), dtype=np.float32)
    R = np.zeros((B, L), dtype=np.float32)
    halt = np.zeros((B, L), dtype=np.int64)          # loop after which the position halted (0: running)
    loops = []
    thr = np.float32(1.0) - np.float32(eps)
    for tau in range(T):
        x = round_bf16(h) if act == "bf16" else h
        q, k, v, al, be = project(x.reshape(B * L, d), Wq, Wk, Wv, wa, wb, H, dk, dv, alpha_lo, act, norm_eps)
        o, _ = scan(q.reshape(B, L, H, dk), k.reshape(B, L, H, dk), v.reshape(B, L, H, dv),
                    al.reshape(B, L, H), be.reshape(B, L, H), None, want_state=False)
        running = halt == 0
        h = np.where(running[..., None], o.reshape(B, L, d) + rho[tau][None, None, :] * h, h)
        if keep_loops:
            loops.append(h.copy())
        z = (h.astype(np.float32) @ w32) + np.float32(b_halt)
        p = (np.float32(1.0) / (np.float32(1.0) + np.exp(-z, dtype=np.float32))).astype(np.float32)
        R = np.where(running, (R + p).astype(np.float32), R)
        newly = running & (R >= thr)
        halt = np.where(newly, tau + 1, halt)
    halt_loop = np.where(halt == 0, T, halt)
    return dict(h=h, halt_loop=halt_loop, ponder=R, loops=loops if keep_loops else None)


def loop_decode_step(h_t, Wq, Wk, Wv, wa, wb, rho, states, H: int, dk: int, dv: int,
                     alpha_lo: float, act: str, eps: float = 1e-6):
    """One generated token per sequence through T loops (recurrent form).

    h_t [N, d] is the token's input; states [T, N, H, dk, dv] holds each loop's
    state after the prefix.  Loop tau projects h^(tau-1), advances its own
    state by one token and applies the residual gate.  Returns
    (h^(T) [N, d], new states [T, N, H, dk, dv]).  fp64.
    """
    h = _f64(h_t)
    rho = _f64(rho)
    st = _f64(states).copy()
    N, d = h.shape
    T = rho.shape[0]
    for tau in range(T):
        x = round_bf16(h) if act == "bf16" else h
        q, k, v, al, be = project(x, Wq, Wk, Wv, wa, wb, H, dk, dv, alpha_lo, act, eps)
        o, s = scan(q.reshape(N, 1, H, dk), k.reshape(N, 1, H, dk), v.reshape(N, 1, H, dv),
                    al.reshape(N, 1, H), be.reshape(N, 1, H), st[tau])
        st[tau] = s
        h = o.reshape(N, d) + rho[tau][None, :] * h
    return h, st


# ---------------------------------------------------------------------------
# second, independent form: the chunkwise (UT-transform) rewrite, numpy/scipy
# ---------------------------------------------------------------------------
def scan_chunkwise(q, k, v, alpha, beta, s_init=None, chunk: int = 64):
    """The same scan computed chunk by chunk (fp64, numpy + scipy).

    Used only to cross-check ``scan``.  Within a chunk with start state S0,
    gamma_r = prod_{i<=r} alpha_i, Gamma_ri = gamma_r / gamma_i (r >= i), and
    A = strict_lower(Gamma (.) K K^T).  With u_t = beta_t (v_t - alpha_t S_{t-1}^T k_t)
    the recurrence reads S_t = alpha_t S_{t-1} + k_t u_t^T, and stacking u:
        (I + diag(beta) A) U = diag(beta) V - diag(beta gamma) K S0
        O      = diag(gamma) Q S0 + lower_incl(Gamma (.) Q K^T) U
        S_next = gamma_C S0 + (diag(gamma_C / gamma) K)^T U
    The unit lower-triangular system is solved with a library routine.
    """
    from scipy.linalg import solve_triangular

    q, k, v, alpha, beta = map(_f64, (q, k, v, alpha, beta))
    B, L, H, dk = q.shape
    dv = v.shape[-1]
    o = np.zeros((B, L, H, dv))
    sf = np.zeros((B, H, dk, dv))
    for b in range(B):
        for h in range(H):
            S = np.zeros((dk, dv)) if s_init is None else _f64(s_init)[b, h].copy()
            for c0 in range(0, L, chunk):
                c1 = min(c0 + chunk, L)
                Q, K, V = q[b, c0:c1, h], k[b, c0:c1, h], v[b, c0:c1, h]
                al, be = alpha[b, c0:c1, h], beta[b, c0:c1, h]
                gam = np.cumprod(al)
                ratio = gam[:, None] / gam[None, :]
                A = np.tril(ratio * (K @ K.T), -1)
                P = np.tril(ratio * (Q @ K.T), 0)
                rhs = be[:, None] * V - (be * gam)[:, None] * (K @ S)
                U = solve_triangular(np.eye(c1 - c0) + be[:, None] * A, rhs,
                                     lower=True, unit_diagonal=True)
                o[b, c0:c1, h] = gam[:, None] * (Q @ S) + P @ U
                S = gam[-1] * S + ((gam[-1] / gam)[:, None] * K).T @ U
            sf[b, h] = S
    return o, sf
