"""Shared helpers of the test suite: error metric and GPU call wrappers.

The error metric for floating-point parity is the maximum over elements of
|g - r| / max(|r|, rms(r)) (a relative error floored by the tensor's RMS, so
that elements near zero do not dominate).  Bars: 1e-4 for fp32 workloads and
3e-3 for bf16-input / fp32-state workloads.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

TOL_F32 = 1e-4
TOL_BF16 = 3e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rel_err(g, r) -> float:
    g = np.asarray(g.detach().cpu().double().numpy() if hasattr(g, "detach") else g, dtype=np.float64)
    r = np.asarray(r.detach().cpu().double().numpy() if hasattr(r, "detach") else r, dtype=np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    if r.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(r * r)))
    den = np.maximum(np.abs(r), rms)
    den = np.where(den == 0, 1.0, den)
    return float(np.max(np.abs(g - r) / den))


def norm_err(g, r) -> float:
    """Normwise relative error ||g - r||_2 / ||r||_2."""
    g = np.asarray(g.detach().cpu().double().numpy() if hasattr(g, "detach") else g, dtype=np.float64)
    r = np.asarray(r.detach().cpu().double().numpy() if hasattr(r, "detach") else r, dtype=np.float64)
    nr = np.linalg.norm(r)
    return float(np.linalg.norm(g - r) / (nr if nr > 0 else 1.0))


def fp32_blocked(xin, W, rot, kb=16):
    """x W with fp32 accumulation over kb-channel blocks taken in order from block `rot` (wrapping around):
    each block's products summed by a float32 library matmul, the block sums added one at a time in fp32.
    This is how an MFMA k-loop accumulates; its rounding is tens of fp32 ulps from the exact value where a
    library matmul's is one or two."""
    xf, Wf = xin.astype(np.float32), W.astype(np.float32)
    nb = xf.shape[1] // kb
    acc = np.zeros((xf.shape[0], Wf.shape[1]), dtype=np.float32)
    for i in range(nb):
        b = (rot + i) % nb
        acc += xf[:, b * kb:(b + 1) * kb] @ Wf[b * kb:(b + 1) * kb]
    return acc


def one_loop(w, x, B, L, t, h_in, rot=None, **kw):
    """Oracle loop t (residual gate rho[t]) from h_in [B, L, d], through the oracle's own project and scan.

    ``rot`` replaces the q/k/v dot products by fp32_blocked ones starting at block rot (normalised in fp32,
    then rounded as the oracle rounds them); the gates stay the oracle's.  kw goes to oracle.project.
    Returns (h^(t), S_final)."""
    import oracle
    h_in = h_in.double().numpy() if hasattr(h_in, "double") else np.asarray(h_in, dtype=np.float64)
    xin = oracle.round_bf16(h_in.reshape(B * L, w.d))
    mats = [x[n].double().numpy() for n in ("Wq", "Wk", "Wv", "wa", "wb")]
    q, k, v, al, be = oracle.project(xin, *mats, w.H, w.dk, w.dv, w.alpha_lo, w.act, **kw)
    if rot is not None:
        M, f32 = B * L, np.float32
        qf = fp32_blocked(xin, mats[0], rot).reshape(M, w.H, w.dk)
        kf = fp32_blocked(xin, mats[1], rot).reshape(M, w.H, w.dk)
        v = oracle.round_bf16(fp32_blocked(xin, mats[2], rot).reshape(M, w.H, w.dv))
        q = oracle.round_bf16(qf / np.sqrt(np.sum(qf * qf, axis=-1, keepdims=True, dtype=f32) + f32(1e-6)))
        k = oracle.round_bf16(kf / np.sqrt(np.sum(kf * kf, axis=-1, keepdims=True, dtype=f32) + f32(1e-6)))
    o, st = oracle.scan(q.reshape(B, L, w.H, w.dk), k.reshape(B, L, w.H, w.dk), v.reshape(B, L, w.H, w.dv),
                        al.reshape(B, L, w.H), be.reshape(B, L, w.H))
    return o.reshape(B, L, w.d) + x["rho"][t].double().numpy() * h_in, st


def loop_envelope(w, x, B, L, runs: int = 3, h_in=None, loops=None, perms: int = 0):
    """Oracle loop run plus the spread of valid bf16 implementations around it.

    For bf16 workloads the looped result is not unique: every bf16 rounding of an fp32 intermediate that
    lies within fp32 summation error of a rounding boundary may go either way, and the loops propagate those
    decisions.  The oracle is re-run as other valid implementations would compute it -- once with the q/k/v
    dot products summed and normalised in fp32 by a library matmul, and with its rounding inputs moved by
    one fp32 ulp (seeded) -- and the largest per-loop deviation from the reference run is the spread.
    ``h_in`` (default: the workload's h0 rows) is the loop input and ``loops`` (default: all) a slice of
    the loops whose residual gates are used, so that one loop can be run from a given h^(t-1).  For one
    loop, ``perms`` more re-runs form the q/k/v dot products as an MFMA k-loop does (fp32_blocked, from
    evenly spaced starting blocks): such sums sit tens of fp32 ulps from the exact value and flip bf16
    roundings that one-ulp moves and a library matmul rarely do.
    Returns (reference dict, spread dict) with per-loop lists "h_max", "h_norm", "s_max", "s_norm".
    """
    import oracle
    rho = x["rho"] if loops is None else x["rho"][loops]
    h = x["h0"][:B, :L] if h_in is None else h_in
    T = rho.shape[0]
    args = (h, x["Wq"], x["Wk"], x["Wv"], x["wa"], x["wb"], rho, w.H, w.dk, w.dv, w.alpha_lo, w.act)
    ref = oracle.loop_prefill(*args, keep_loops=True, keep_states=True)
    sp = {k: [0.0] * T for k in ("h_max", "h_norm", "s_max", "s_norm")}

    def take(t, hh, ss):
        sp["h_max"][t] = max(sp["h_max"][t], rel_err(hh, ref["loops"][t]))
        sp["h_norm"][t] = max(sp["h_norm"][t], norm_err(hh, ref["loops"][t]))
        sp["s_max"][t] = max(sp["s_max"][t], rel_err(ss, ref["states"][t]))
        sp["s_norm"][t] = max(sp["s_norm"][t], norm_err(ss, ref["states"][t]))

    variants = [dict(fp32_sum=True)] + [dict(jitter=np.random.default_rng(9000 + i)) for i in range(runs - 1)]
    for kw in variants:
        j = oracle.loop_prefill(*args, keep_loops=True, keep_states=True, **kw)
        for t in range(T):
            take(t, j["loops"][t], j["states"][t])
    if perms:
        assert T == 1 and loops is not None, "channel-order variants are one-loop runs"
        t0 = range(x["rho"].shape[0])[loops][0]
        hin = x["h0"][:B, :L] if h_in is None else h_in
        nb = w.d // 16
        for i in range(perms):
            hh, ss = one_loop(w, x, B, L, t0, hin, rot=(i * nb) // perms)
            take(0, hh, ss)
    return ref, sp


# Envelope factors: normwise deviations are stable across valid implementations (2x); the max-relative
# statistic is decided by a handful of flipped elements and is heavy-tailed (4x).
ENV_NORM, ENV_MAX = 2.0, 4.0


def envelope_bar(spread: float, floor: float, factor: float) -> float:
    """Bar for a non-unique bf16 loop result: the fixed bar, or `factor` times the spread if larger."""
    return max(floor, factor * spread)


def bf16_ulp(r: np.ndarray) -> np.ndarray:
    """Spacing of the bf16 grid at |r| (8 significant bits)."""
    a = np.abs(np.asarray(r, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(a, 1e-38)))
    return np.exp2(e - 7)


def dev(t: torch.Tensor) -> torch.Tensor:
    return t.contiguous().to("cuda")
