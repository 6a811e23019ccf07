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
    "build", "num_threads", "round_bf16", "round_f32", "scan", "project",
    "loop_prefill", "loop_decode_step", "scan_chunkwise",
]


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (plain -O2, no FMA contraction)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared",
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


def round_bf16(x, jitter=None) -> np.ndarray:
    """fp64 -> fp32 -> bf16 with round-to-nearest-even, returned as fp64.

    bf16 keeps the upper 16 bits of the fp32 bit pattern.  Rounding to
    nearest even adds 0x7FFF plus the lowest kept bit before truncating
    (finite inputs; overflow correctly rounds to infinity).

    ``jitter`` (a numpy Generator, default None) first moves every fp32 value
    one fp32 ulp up or down at random.  It models an implementation whose
    fp32 arithmetic summed in another order: its bf16 rounding decisions are
    equally valid, and the spread of results under jitter measures how far
    two valid bf16 implementations can drift apart.
    """
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    if jitter is not None:
        up = jitter.random(f.shape) < 0.5
        f = np.where(up, np.nextafter(f, np.float32(np.inf)),
                     np.nextafter(f, np.float32(-np.inf))).astype(np.float32)
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


# ---------------------------------------------------------------------------
# per-loop projections, normalisation and gates (numpy fp64)
# ---------------------------------------------------------------------------
def project(x, Wq, Wk, Wv, wa, wb, H: int, dk: int, dv: int, alpha_lo: float,
            act: str, eps: float = 1e-6, jitter=None, fp32_sum: bool = False):
    """Projections of one loop for token rows x [M, d] (already at operand precision).

    q = x Wq, k = x Wk, v = x Wv (head j owns columns [j*dk, (j+1)*dk)),
    a = x wa, b = x wb (one column per head).  q and k are L2-normalised per
    head; alpha = alpha_lo + (1 - alpha_lo) / (1 + e^a); beta = 1 / (1 + e^-b).
    For act == "bf16", q/k/v are then rounded fp64->fp32->bf16 and alpha, beta
    to fp32 (the precision they are stored in).  ``jitter``: see round_bf16.
    ``fp32_sum`` forms the q/k/v dot products with a float32 library matmul
    and normalises q/k in float32 (another valid fp32 implementation of the
    same values; the gates stay fp64).
    """
    x = _f64(x)
    M = x.shape[0]
    Wq, Wk, Wv, wa, wb = map(_f64, (Wq, Wk, Wv, wa, wb))
    a = x @ wa
    b = x @ wb
    if fp32_sum:
        f32 = np.float32
        xf = x.astype(f32)
        q = (xf @ Wq.astype(f32)).reshape(M, H, dk)
        k = (xf @ Wk.astype(f32)).reshape(M, H, dk)
        v = (xf @ Wv.astype(f32)).reshape(M, H, dv).astype(np.float64)
        q = (q / np.sqrt(np.sum(q * q, axis=-1, keepdims=True, dtype=f32) + f32(eps))).astype(np.float64)
        k = (k / np.sqrt(np.sum(k * k, axis=-1, keepdims=True, dtype=f32) + f32(eps))).astype(np.float64)
    else:
        q = (x @ Wq).reshape(M, H, dk)
        k = (x @ Wk).reshape(M, H, dk)
        v = (x @ Wv).reshape(M, H, dv)
        q = q / np.sqrt(np.sum(q * q, axis=-1, keepdims=True) + eps)
        k = k / np.sqrt(np.sum(k * k, axis=-1, keepdims=True) + eps)
    alpha = alpha_lo + (1.0 - alpha_lo) / (1.0 + np.exp(a))
    beta = 1.0 / (1.0 + np.exp(-b))
    if act == "bf16":
        q, k, v = round_bf16(q, jitter), round_bf16(k, jitter), round_bf16(v, jitter)
        alpha, beta = round_f32(alpha), round_f32(beta)
    return q, k, v, alpha, beta


def loop_prefill(h0, Wq, Wk, Wv, wa, wb, rho, H: int, dk: int, dv: int,
                 alpha_lo: float, act: str, eps: float = 1e-6,
                 keep_loops: bool = False, keep_states: bool = False, jitter=None,
                 fp32_sum: bool = False):
    """T weight-tied loops of the GDN mixer with the per-loop residual gate.

    h^(0) = h0 [B, L, d]; for tau = 1..T:
        x      = h^(tau-1)            (f32 workloads)
               = bf16(fp32(h^(tau-1))) (bf16 workloads: the GEMM operand)
        q,k,v,alpha,beta = project(x)
        o      = scan(q, k, v, alpha, beta) from S = 0
        h^(tau) = o.reshape(B, L, H*dv) + rho[tau-1] (.) h^(tau-1)
    Returns dict(h=h^(T) [B,L,d], loops=[h^(1..T)] or None,
    states=[S_final per loop, each [B,H,dk,dv]] or None).  fp64.
    ``jitter``: see round_bf16 (applies to every bf16 rounding point);
    ``fp32_sum``: see project.
    """
    h = _f64(h0)
    rho = _f64(rho)
    B, L, d = h.shape
    T = rho.shape[0]
    assert H * dv == d, "the mixer output must have the width of the residual stream"
    loops, states = [], []
    for tau in range(T):
        x = round_bf16(h, jitter) if act == "bf16" else h
        q, k, v, al, be = project(x.reshape(B * L, d), Wq, Wk, Wv, wa, wb, H, dk, dv,
                                  alpha_lo, act, eps, jitter, fp32_sum)
        o, s = scan(q.reshape(B, L, H, dk), k.reshape(B, L, H, dk), v.reshape(B, L, H, dv),
                    al.reshape(B, L, H), be.reshape(B, L, H), None, want_state=keep_states)
        h = o.reshape(B, L, d) + rho[tau][None, None, :] * h
        if keep_loops:
            loops.append(h.copy())
        if keep_states:
            states.append(s)
    return dict(h=h, loops=loops if keep_loops else None,
                states=states if keep_states else None)


def loop_decode_step(h_t, Wq, Wk, Wv, wa, wb, rho, states, H: int, dk: int, dv: int,
                     alpha_lo: float, act: str, eps: float = 1e-6, jitter=None):
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
        x = round_bf16(h, jitter) if act == "bf16" else h
        q, k, v, al, be = project(x, Wq, Wk, Wv, wa, wb, H, dk, dv, alpha_lo, act, eps, jitter)
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
