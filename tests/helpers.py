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


def loop_envelope(w, x, B, L, runs: int = 3, h_in=None, loops=None):
    """Oracle loop run plus the spread of valid bf16 implementations around it.

    For bf16 workloads the looped result is not unique: every bf16 rounding of an fp32 intermediate that
    lies within fp32 summation error of a rounding boundary may go either way, and the loops propagate those
    decisions.  The oracle is re-run as other valid implementations would compute it -- once with the q/k/v
    dot products summed and normalised in fp32 by a library matmul, and with its rounding inputs moved by
    one fp32 ulp (seeded) -- and the largest per-loop deviation from the reference run is the spread.
    ``h_in`` (default: the workload's h0 rows) is the loop input and ``loops`` (default: all) a slice of
    the loops whose residual gates are used, so that one loop can be run from a given h^(t-1).
    Returns (reference dict, spread dict) with per-loop lists "h_max", "h_norm", "s_max", "s_norm".
    """
    import oracle
    rho = x["rho"] if loops is None else x["rho"][loops]
    h = x["h0"][:B, :L] if h_in is None else h_in
    T = rho.shape[0]
    args = (h, x["Wq"], x["Wk"], x["Wv"], x["wa"], x["wb"], rho, w.H, w.dk, w.dv, w.alpha_lo, w.act)
    ref = oracle.loop_prefill(*args, keep_loops=True, keep_states=True)
    sp = {k: [0.0] * T for k in ("h_max", "h_norm", "s_max", "s_norm")}
    variants = [dict(fp32_sum=True)] + [dict(jitter=np.random.default_rng(9000 + i)) for i in range(runs - 1)]
    for kw in variants:
        j = oracle.loop_prefill(*args, keep_loops=True, keep_states=True, **kw)
        for t in range(T):
            sp["h_max"][t] = max(sp["h_max"][t], rel_err(j["loops"][t], ref["loops"][t]))
            sp["h_norm"][t] = max(sp["h_norm"][t], norm_err(j["loops"][t], ref["loops"][t]))
            sp["s_max"][t] = max(sp["s_max"][t], rel_err(j["states"][t], ref["states"][t]))
            sp["s_norm"][t] = max(sp["s_norm"][t], norm_err(j["states"][t], ref["states"][t]))
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
