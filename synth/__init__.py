"""Seeded synthetic inputs for the looped gated-delta-rule (GDN) token mixer.

This module is shared by the CPU oracle (``oracle/``) and the HIP path
(``looped_linear_attention_amd``).  It only draws random numbers and stores
them in the dtypes the workloads use; it holds none of the method's
arithmetic (no projection, no normalisation of hidden states, no gates, no
recurrence).

Workload shapes follow the LT2 paper ("LT2: Linear-Time Looped
Transformers"): hidden width 2048 with 16 heads (Appendix C, 1.3B scale),
T = 4 loops (Section 3), 1k-32k tokens at batch 1-8 (Section 3.2 efficiency
study).  Values are seeded Gaussians; no dataset or trained weight is
involved, since throughput does not depend on the values.

Generator: ``numpy.random.default_rng(seed)`` (PCG64), fp32 draws in the
fixed order listed per workload.  bf16 tensors are produced from those fp32
draws with round-to-nearest-even (``torch.Tensor.to(torch.bfloat16)``).

Notation for variances: ``N(0, s)`` means variance ``s``; weights use
standard deviation ``1/sqrt(d)``.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Iterator, Optional

import numpy as np
import torch

__all__ = [
    "Workload", "WORKLOADS", "workload", "prefill_inputs", "scan_inputs",
    "decode_state_init", "decode_step_inputs", "unit_rows", "grad_inputs", "act_inputs", "ACT_BIAS", "ACT_EPS",
    "block_ffn", "block_inputs",
]

# The halting layer of the adaptive-halting workloads: w ~ N(0, 1/d) and this bias, so that
# sigmoid(w . h + b) spreads the positions' halting loops over 1..T; eps as on the pages (LT2 Appendix A).
ACT_BIAS = -0.5
ACT_EPS = 0.01


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    L: int
    H: int
    dk: int
    dv: int
    d: int
    T: int
    act: str            # "f32" or "bf16": dtype of h0, weights and q/k/v
    alpha_lo: float     # alpha = alpha_lo + (1 - alpha_lo) * sigmoid(-a)
    seed: int
    steps: int = 0      # decode workloads: generated tokens per sequence


WORKLOADS = {
    # tiny fp32 case the oracle finishes in well under a second
    "tiny_f32": Workload("tiny_f32", B=1, L=256, H=1, dk=64, dv=64, d=64, T=4,
                         act="f32", alpha_lo=0.0, seed=0),
    # 16 heads of 128 at width 2048, one 4096-token sequence
    "prefill_b1_l4096": Workload("prefill_b1_l4096", B=1, L=4096, H=16, dk=128, dv=128,
                                 d=2048, T=4, act="bf16", alpha_lo=0.9, seed=0),
    "prefill_b4_l8192": Workload("prefill_b4_l8192", B=4, L=8192, H=16, dk=128, dv=128,
                                 d=2048, T=4, act="bf16", alpha_lo=0.0, seed=1),
    "prefill_b1_l32768": Workload("prefill_b1_l32768", B=1, L=32768, H=16, dk=128, dv=128,
                                  d=2048, T=4, act="bf16", alpha_lo=0.95, seed=0),
    # 64 sequences x 256 generated tokens, 4 loop states per sequence
    "decode_n64_s256": Workload("decode_n64_s256", B=64, L=1, H=16, dk=128, dv=128,
                                d=2048, T=4, act="bf16", alpha_lo=0.0, seed=0, steps=256),
}


def workload(name: str) -> Workload:
    return WORKLOADS[name]


def _to_act(x: np.ndarray, act: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16) if act == "bf16" else t


def prefill_inputs(w: Workload, L: Optional[int] = None, B: Optional[int] = None) -> dict:
    """Inputs of a looped prefill, drawn in this order:

    h0 ~ N(0,1) [B,L,d]; Wq, Wk ~ N(0,1/d) [d,H*dk]; Wv ~ N(0,1/d) [d,H*dv];
    wa, wb ~ N(0,1/d) [d,H]; rho ~ U(0,0.5) [T,d].

    h0 and the weights are returned in the workload's activation dtype; rho is
    fp32.  ``L``/``B`` select a leading prefix / leading batch rows of the
    full-size draw (the draw itself is always full size, so prefixes agree).
    """
    rng = np.random.default_rng(w.seed)
    d, H, dk, dv = w.d, w.H, w.dk, w.dv
    std = 1.0 / math.sqrt(d)
    h0 = rng.standard_normal((w.B, w.L, d), dtype=np.float32)
    Wq = rng.standard_normal((d, H * dk), dtype=np.float32) * np.float32(std)
    Wk = rng.standard_normal((d, H * dk), dtype=np.float32) * np.float32(std)
    Wv = rng.standard_normal((d, H * dv), dtype=np.float32) * np.float32(std)
    wa = rng.standard_normal((d, H), dtype=np.float32) * np.float32(std)
    wb = rng.standard_normal((d, H), dtype=np.float32) * np.float32(std)
    rho = rng.random((w.T, d), dtype=np.float32) * np.float32(0.5)
    Lp = w.L if L is None else L
    Bp = w.B if B is None else B
    return dict(
        h0=_to_act(h0[:Bp, :Lp], w.act),
        Wq=_to_act(Wq, w.act), Wk=_to_act(Wk, w.act), Wv=_to_act(Wv, w.act),
        wa=_to_act(wa, w.act), wb=_to_act(wb, w.act),
        rho=torch.from_numpy(rho),
    )


def unit_rows(x: np.ndarray) -> np.ndarray:
    """Scale each last-axis row of a fp32 draw to unit Euclidean length (fp32).

    Used to make synthetic unit-norm query/key vectors for scan-level inputs,
    whose contract requires normalised q and k.
    """
    x = x.astype(np.float32)
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True, dtype=np.float32))
    return (x / n).astype(np.float32)


def scan_inputs(seed: int, B: int, L: int, H: int, dk: int, dv: int, act: str = "bf16",
                alpha_range=(0.0, 1.0), beta_range=(0.0, 1.0), with_state: bool = False,
                state_std: float = 0.1) -> dict:
    """Inputs of a single scan pass, drawn in this order:

    q ~ N(0,1) [B,L,H,dk] (rows scaled to unit length); k likewise;
    v ~ N(0,1) [B,L,H,dv]; alpha ~ U(alpha_range) [B,L,H];
    beta ~ U(beta_range) [B,L,H]; optionally s_init ~ N(0, state_std^2) [B,H,dk,dv].

    q/k/v come back in ``act`` (bf16 rounding after scaling to unit length);
    alpha, beta, s_init are fp32.  alpha is clamped away from 0 by the draw
    itself (U(lo,1) with lo >= 0 can return lo exactly only with probability 0;
    a drawn 0 is replaced by the smallest positive fp32).
    """
    rng = np.random.default_rng(seed)
    q = unit_rows(rng.standard_normal((B, L, H, dk), dtype=np.float32))
    k = unit_rows(rng.standard_normal((B, L, H, dk), dtype=np.float32))
    v = rng.standard_normal((B, L, H, dv), dtype=np.float32)
    a0, a1 = alpha_range
    b0, b1 = beta_range
    alpha = (np.float32(a0) + rng.random((B, L, H), dtype=np.float32) * np.float32(a1 - a0))
    alpha = np.maximum(alpha, np.float32(np.finfo(np.float32).tiny)).astype(np.float32)
    beta = (np.float32(b0) + rng.random((B, L, H), dtype=np.float32) * np.float32(b1 - b0)).astype(np.float32)
    out = dict(q=_to_act(q, act), k=_to_act(k, act), v=_to_act(v, act),
               alpha=torch.from_numpy(alpha), beta=torch.from_numpy(beta))
    if with_state:
        s = rng.standard_normal((B, H, dk, dv), dtype=np.float32) * np.float32(state_std)
        out["s_init"] = torch.from_numpy(s)
    return out


def decode_state_init(w: Workload) -> torch.Tensor:
    """Pre-filled decode states S ~ N(0, 0.02) [T, N, H, dk, dv] fp32 (variance 0.02)."""
    rng = np.random.default_rng(w.seed)
    s = rng.standard_normal((w.T, w.B, w.H, w.dk, w.dv), dtype=np.float32)
    s *= np.float32(math.sqrt(0.02))
    return torch.from_numpy(s)


def decode_step_inputs(w: Workload, steps: Optional[int] = None) -> Iterator[dict]:
    """Per (step, loop) scan-level decode inputs, in generation order.

    The state draw comes first from the same seeded stream (see
    ``decode_state_init``, which re-draws it); then for each step s and each
    loop tau: q, k, v ~ N(0,1) [N,H,dk|dv] (q, k scaled to unit length in
    fp32), rounded to bf16; z_a, z_b ~ N(0,1) [N,H] -> alpha = 1/(1+e^{z_a}),
    beta = 1/(1+e^{-z_b}) (fp32).
    """
    rng = np.random.default_rng(w.seed)
    # skip the state draw so the step stream is the one that follows it
    rng.standard_normal((w.T, w.B, w.H, w.dk, w.dv), dtype=np.float32)
    n_steps = w.steps if steps is None else steps
    N, H, dk, dv = w.B, w.H, w.dk, w.dv
    for s in range(n_steps):
        for tau in range(w.T):
            q = unit_rows(rng.standard_normal((N, H, dk), dtype=np.float32))
            k = unit_rows(rng.standard_normal((N, H, dk), dtype=np.float32))
            v = rng.standard_normal((N, H, dv), dtype=np.float32)
            za = rng.standard_normal((N, H), dtype=np.float32)
            zb = rng.standard_normal((N, H), dtype=np.float32)
            alpha = (1.0 / (1.0 + np.exp(za.astype(np.float64)))).astype(np.float32)
            beta = (1.0 / (1.0 + np.exp(-zb.astype(np.float64)))).astype(np.float32)
            yield dict(step=s, tau=tau, q=_to_act(q, "bf16"), k=_to_act(k, "bf16"),
                       v=_to_act(v, "bf16"), alpha=torch.from_numpy(alpha),
                       beta=torch.from_numpy(beta))


def grad_inputs(seed: int, B: int, L: int, H: int, dk: int, dv: int, with_state_grad: bool = True) -> dict:
    """Incoming gradients for a backward pass, drawn in this order: d_o ~ N(0,1) [B,L,H,dv]; optionally
    d_sfinal ~ N(0,1) [B,H,dk,dv]; both fp32 (the loss is taken as <d_o, o> + <d_sfinal, S_final>)."""
    rng = np.random.default_rng(seed)
    out = dict(d_o=torch.from_numpy(rng.standard_normal((B, L, H, dv), dtype=np.float32)))
    if with_state_grad:
        out["d_sfinal"] = torch.from_numpy(rng.standard_normal((B, H, dk, dv), dtype=np.float32))
    return out


def act_inputs(w: Workload, seed: int = 7) -> dict:
    """Halting layer of an adaptive-halting loop: w_halt ~ N(0, 1/d) [d] fp32 (seeded), b_halt = ACT_BIAS,
    eps = ACT_EPS."""
    rng = np.random.default_rng(seed)
    wh = rng.standard_normal(w.d, dtype=np.float32) * np.float32(1.0 / math.sqrt(w.d))
    return dict(w_halt=torch.from_numpy(wh), b_halt=ACT_BIAS, eps=ACT_EPS)


def block_ffn(w: Workload) -> int:
    """Hidden width of a block's gated FFN at the workload's width: 8d/3 rounded up to a multiple of 256
    (5632 at d = 2048, 256 at d = 64)."""
    return 256 * ((8 * w.d // 3 + 255) // 256)


def block_inputs(w: Workload, layers: int, seed: int = 11) -> list:
    """Weights of `layers` LT2 blocks, drawn per block in this order: g1 = 1 + 0.1 N(0,1) [d] fp32; Wq, Wk
    ~ N(0,1/d) [d,H*dk]; Wv ~ N(0,1/d) [d,H*dv]; wa, wb ~ N(0,1/d) [d,H]; Wg ~ N(0,1/d) [d,H*dv]; Wo ~
    N(0,1/(H dv)) [H*dv,d]; g2 as g1; W1, W3 ~ N(0,1/d) [d,F]; W2 ~ N(0,1/F) [F,d] (F = block_ffn).  Matrices
    in the workload's activation dtype."""
    rng = np.random.default_rng(seed)
    d, HK, HV, F = w.d, w.H * w.dk, w.H * w.dv, block_ffn(w)
    n = lambda rows, cols: _to_act(rng.standard_normal((rows, cols), dtype=np.float32)
                                   * np.float32(1.0 / math.sqrt(rows)), w.act)
    out = []
    for _ in range(layers):
        blk = dict(g1=torch.from_numpy(1.0 + 0.1 * rng.standard_normal(d, dtype=np.float32)))
        blk.update(Wq=n(d, HK), Wk=n(d, HK), Wv=n(d, HV), wa=n(d, w.H), wb=n(d, w.H), Wg=n(d, HV), Wo=n(HV, d))
        blk["g2"] = torch.from_numpy(1.0 + 0.1 * rng.standard_normal(d, dtype=np.float32))
        blk.update(W1=n(d, F), W3=n(d, F), W2=n(F, d))
        out.append(blk)
    return out
