"""Shared helpers of the test suite: error metrics, the projection bound, NaN poisoning and GPU call wrappers.

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


def _np64(x) -> np.ndarray:
    if hasattr(x, "detach"):
        x = x.detach().cpu().double().numpy()
    return np.asarray(x, dtype=np.float64)


def rel_err(g, r) -> float:
    g, r = _np64(g), _np64(r)
    assert g.shape == r.shape, (g.shape, r.shape)
    if r.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(r * r)))
    den = np.maximum(np.abs(r), rms)
    den = np.where(den == 0, 1.0, den)
    return float(np.max(np.abs(g - r) / den))


def norm_err(g, r) -> float:
    """Normwise relative error ||g - r||_2 / ||r||_2."""
    g, r = _np64(g), _np64(r)
    nr = np.linalg.norm(r)
    return float(np.linalg.norm(g - r) / (nr if nr > 0 else 1.0))


def bf16_ulp(r: np.ndarray) -> np.ndarray:
    """Spacing of the bf16 grid at |r| (8 significant bits)."""
    a = np.abs(np.asarray(r, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(a, 1e-38)))
    return np.exp2(e - 7)


def check_projection(gq, gk, gv, ga, gb, x_in, Wq, Wk, Wv, wa, wb, H, dk, dv, alpha_lo, act, eps=1e-6):
    """Holds one loop's GPU projections of the token rows x_in [M, d] (already at operand precision) to the
    oracle's, and returns the oracle's gates (alpha, beta) [M, H].

    fp32 workloads: every output within 1e-5 (metric above).  bf16 workloads: q, k, v are stored in bf16, so
    the two sides agree up to where each fp32 dot product rounds.  The GPU's fp32 dot product differs from
    the exact one by at most the recursive-summation bound gamma_K * sum|x||w| (K = d terms, unit roundoff
    2^-24), whatever the summation order; after rounding to bf16 the two results may then sit one bf16 step
    apart, and q and k also carry their norm's error.  The gates are stored in fp32: within 1e-5."""
    import oracle
    x_in = _np64(x_in)
    M = x_in.shape[0]
    Wq, Wk, Wv = _np64(Wq), _np64(Wk), _np64(Wv)
    rq, rk, rv, ra, rb = oracle.project(x_in, Wq, Wk, Wv, _np64(wa), _np64(wb), H, dk, dv, alpha_lo, act, eps)
    gq, gk, gv = (_np64(t).reshape(M, H, -1) for t in (gq, gk, gv))
    if act == "f32":
        for g, r in ((gq, rq), (gk, rk), (gv, rv)):
            assert rel_err(g, r) < 1e-5
    else:
        K = x_in.shape[1]
        gam = K * 2.0 ** -24 / (1 - K * 2.0 ** -24)
        xa = np.abs(x_in)
        for g, r, W, normed in ((gq, rq, Wq, True), (gk, rk, Wk, True), (gv, rv, Wv, False)):
            p = (x_in @ W).reshape(M, H, -1)
            mag = (xa @ np.abs(W)).reshape(M, H, -1)
            if normed:
                nrm = np.sqrt(np.sum(p * p, -1, keepdims=True) + eps)
                bound = 2 * gam * (mag + np.abs(p)) / nrm
            else:
                bound = 2 * gam * mag
            diff = np.abs(g - r)
            step = bf16_ulp(np.maximum(np.abs(r), np.abs(g)))
            assert np.all(diff <= bound + step * 1.0001), float((diff - bound - step).max())
            assert np.mean(diff > 0) < 0.01
    ga, gb = _np64(ga).reshape(M, H), _np64(gb).reshape(M, H)
    ea, eb = rel_err(ga, ra), rel_err(gb, rb)
    assert ea < 1e-5 and eb < 1e-5, (ea, eb)
    return ra, rb


def poison_(t: torch.Tensor) -> torch.Tensor:
    """Fill a device buffer with all-ones bytes: NaN for fp32 and bf16 alike."""
    t.view(torch.uint8).fill_(0xFF)
    return t


def padded(shape, dtype=torch.float32, pad=64, fill=float("nan")):
    """A device buffer of `shape` followed by `pad` canary elements (value 1234.5).

    Returns (the leading view, the whole buffer); the view is poisoned with `fill`."""
    n = int(np.prod(shape))
    buf = torch.full((n + pad,), 1234.5, dtype=dtype, device="cuda")
    buf[:n] = fill
    return buf[:n].view(*shape), buf


def canary_intact(buf: torch.Tensor, n: int) -> bool:
    return bool(torch.all(buf[n:] == 1234.5).item())


def dev(t: torch.Tensor) -> torch.Tensor:
    return t.contiguous().to("cuda")
