"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test names the plausible oracle mistake it would catch.  Sources are the
LT2 pages ("LT2: Linear-Time Looped Transformers"): Section 2 (loop, residual
gate, q/k/v/S shapes), Appendix B.1 (rank-1 DPLR update; reflections realise
permutations; operator spectral norm <= 1), Fig. 6 caption (gating plus the
delta rule).  The pages print no numeric worked example, so the numeric pin is
a hand-derived one (tests/golden/gdn_three_token_hand.json).
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_scan(seed, B, L, H, dk, dv, alpha_range=(0.0, 1.0), beta_range=(0.0, 1.0), state=True):
    x = synth.scan_inputs(seed, B, L, H, dk, dv, act="f32", alpha_range=alpha_range,
                          beta_range=beta_range, with_state=state)
    return {k: v.double().numpy() for k, v in x.items()}


# ---------------------------------------------------------------------------
# bf16 rounding: against torch's conversion (a library routine)
# ---------------------------------------------------------------------------
def test_round_bf16_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(200000) * 10.0 ** rng.integers(-30, 30, 200000),
        # exact ties and neighbours of ties in the bf16 grid
        (np.arange(1, 4096, dtype=np.uint32) << 15).astype(np.uint32).view(np.float32).astype(np.float64),
        np.array([0.0, -0.0, 1.0, -1.0, 3.0e38, -3.0e38, 1e-40, -1e-40]),
    ])
    mine = oracle.round_bf16(x)
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).double().numpy()
    assert np.array_equal(mine, ref)


# ---------------------------------------------------------------------------
# the recurrence: hand-worked example, invariants and closed forms
# ---------------------------------------------------------------------------
def test_scan_hand_worked_example():
    """Catches: pre- vs post-update read-out, S vs S^T, alpha on the write term, sign of the delta term."""
    g = json.load(open(os.path.join(GOLDEN, "gdn_three_token_hand.json")))
    q = np.array(g["q"], float)[None, :, None, :]
    k = np.array(g["k"], float)[None, :, None, :]
    v = np.array(g["v"], float)[None, :, None, :]
    a = np.array(g["alpha"], float)[None, :, None]
    b = np.array(g["beta"], float)[None, :, None]
    o, s = oracle.scan(q, k, v, a, b)
    assert np.abs(o[0, :, 0] - np.array(g["o"])).max() <= g["tol_abs"]
    assert np.abs(s[0, 0] - np.array(g["S_final"])).max() <= g["tol_abs"]


def test_scan_first_token_closed_form():
    """From S_0 = 0 the first state is beta k v^T, so o_1 = beta (k.q) v for any alpha."""
    x = _rand_scan(1, 2, 1, 3, 16, 8, state=False)
    o, s = oracle.scan(x["q"], x["k"], x["v"], x["alpha"], x["beta"])
    kq = np.sum(x["k"] * x["q"], -1)
    ref = (x["beta"] * kq)[..., None] * x["v"]
    assert np.abs(o - ref).max() < 1e-14
    ref_s = x["beta"][:, 0, :, None, None] * x["k"][:, 0, :, :, None] * x["v"][:, 0, :, None, :]
    assert np.abs(s - ref_s).max() < 1e-14


def test_scan_identity_transition():
    """alpha = 1, beta = 0: the state never changes and o_t = S_0^T q_t."""
    x = _rand_scan(2, 2, 33, 2, 16, 8)
    x["alpha"][:] = 1.0
    x["beta"][:] = 0.0
    o, s = oracle.scan(x["q"], x["k"], x["v"], x["alpha"], x["beta"], x["s_init"])
    assert np.array_equal(s, x["s_init"])
    ref = np.einsum("bhij,blhi->blhj", x["s_init"], x["q"])
    assert np.abs(o - ref).max() < 1e-13


def test_scan_delta_write_recalls_value():
    """alpha = 1, beta = 1, unit k: after the update S_t^T k_t = v_t (the delta rule writes v at key k)."""
    x = _rand_scan(3, 1, 20, 2, 16, 8)
    x["k"] /= np.linalg.norm(x["k"], axis=-1, keepdims=True)  # unit length in fp64
    x["alpha"][:] = 1.0
    x["beta"][:] = 1.0
    S = x["s_init"]
    for t in range(20):
        sl = lambda a: a[:, t:t + 1]
        _, S = oracle.scan(sl(x["q"]), sl(x["k"]), sl(x["v"]), sl(x["alpha"]), sl(x["beta"]), S)
        recall = np.einsum("bhij,bhi->bhj", S, x["k"][:, t])
        assert np.abs(recall - x["v"][:, t]).max() < 1e-12


def test_scan_pure_decay():
    """beta = 0: S_t = (prod_{i<=t} alpha_i) S_0."""
    x = _rand_scan(4, 1, 40, 2, 8, 8, alpha_range=(0.5, 1.0))
    x["beta"][:] = 0.0
    o, s = oracle.scan(x["q"], x["k"], x["v"], x["alpha"], x["beta"], x["s_init"])
    g = np.prod(x["alpha"], axis=1)  # [B, H]
    assert np.abs(s - g[:, :, None, None] * x["s_init"]).max() < 1e-14
    gt = np.cumprod(x["alpha"], axis=1)  # [B, L, H]
    ref = gt[..., None] * np.einsum("bhij,blhi->blhj", x["s_init"], x["q"])
    assert np.abs(o - ref).max() < 1e-13


def test_scan_householder_permutation():
    """alpha = 1, beta = 2, k = (e_i - e_j)/sqrt 2, v = 0: I - 2kk^T swaps rows i and j of S.

    A sequence of such reflections realises any permutation (Appendix B.1 (iii)),
    so the final state is the closed-form row permutation of S_0.
    """
    dk, dv, L = 6, 5, 25
    rng = np.random.default_rng(5)
    S0 = rng.standard_normal((1, 1, dk, dv))
    k = np.zeros((1, L, 1, dk))
    perm = np.arange(dk)
    for t in range(L):
        i, j = rng.choice(dk, 2, replace=False)
        k[0, t, 0, i] = 1 / math.sqrt(2)
        k[0, t, 0, j] = -1 / math.sqrt(2)
        perm[[i, j]] = perm[[j, i]]
    q = rng.standard_normal((1, L, 1, dk))
    v = np.zeros((1, L, 1, dv))
    o, s = oracle.scan(q, k, v, np.ones((1, L, 1)), np.full((1, L, 1), 2.0), S0)
    assert np.abs(s[0, 0] - S0[0, 0][perm]).max() < 1e-13


def test_scan_contraction():
    """v = 0, alpha in (0,1], beta in [0,2], |k| = 1: the transition has spectral norm <= 1 (Appendix B.1),
    so the Frobenius norm of S never grows."""
    x = _rand_scan(6, 1, 64, 3, 16, 8, beta_range=(0.0, 2.0))
    x["k"] /= np.linalg.norm(x["k"], axis=-1, keepdims=True)  # unit length in fp64
    x["v"][:] = 0.0
    S = x["s_init"]
    prev = np.linalg.norm(S, axis=(2, 3))
    for t in range(64):
        sl = lambda a: a[:, t:t + 1]
        _, S = oracle.scan(sl(x["q"]), sl(x["k"]), sl(x["v"]), sl(x["alpha"]), sl(x["beta"]), S)
        cur = np.linalg.norm(S, axis=(2, 3))
        assert np.all(cur <= prev * (1 + 1e-14))
        prev = cur


@pytest.mark.parametrize("B,L,H,dk,dv,chunk", [
    (1, 37, 2, 8, 5, 1), (1, 37, 2, 8, 5, 4), (1, 37, 2, 8, 5, 37), (1, 37, 2, 8, 5, 64),
    (2, 130, 2, 16, 8, 64), (1, 65, 1, 64, 64, 64), (1, 200, 1, 128, 128, 64), (1, 1, 1, 4, 4, 64),
])
def test_scan_equals_chunkwise_form(B, L, H, dk, dv, chunk):
    """Brute force: the token recurrence (C) equals the independently written chunkwise UT form (numpy + a
    library triangular solve) for several chunk sizes, including ragged last chunks."""
    x = _rand_scan(7 + L, B, L, H, dk, dv, alpha_range=(0.05, 1.0))
    oa, sa = oracle.scan(x["q"], x["k"], x["v"], x["alpha"], x["beta"], x["s_init"])
    ob, sb = oracle.scan_chunkwise(x["q"], x["k"], x["v"], x["alpha"], x["beta"], x["s_init"], chunk=chunk)
    scale = max(1.0, np.abs(oa).max())
    assert np.abs(oa - ob).max() < 1e-12 * scale
    assert np.abs(sa - sb).max() < 1e-12 * max(1.0, np.abs(sa).max())


def test_scan_split_resume():
    """Scanning [0,m) then [m,L) from the carried state equals one pass (m on and off chunk boundaries)."""
    x = _rand_scan(8, 2, 150, 2, 16, 8)
    o, s = oracle.scan(x["q"], x["k"], x["v"], x["alpha"], x["beta"], x["s_init"])
    for m in (1, 64, 77, 149):
        a = {k: (v[:, :m] if v.ndim >= 3 and k != "s_init" else v) for k, v in x.items()}
        b = {k: (v[:, m:] if v.ndim >= 3 and k != "s_init" else v) for k, v in x.items()}
        o1, s1 = oracle.scan(a["q"], a["k"], a["v"], a["alpha"], a["beta"], x["s_init"])
        o2, s2 = oracle.scan(b["q"], b["k"], b["v"], b["alpha"], b["beta"], s1)
        assert np.abs(np.concatenate([o1, o2], 1) - o).max() < 1e-13
        assert np.abs(s2 - s).max() < 1e-13


def test_scan_value_columns_independent_and_linear():
    """Columns of S never mix (dv can be split), and from S_0 = 0 the output is linear in V."""
    x = _rand_scan(9, 1, 50, 2, 8, 6, state=False)
    o, _ = oracle.scan(x["q"], x["k"], x["v"], x["alpha"], x["beta"])
    o1, _ = oracle.scan(x["q"], x["k"], x["v"][..., :2], x["alpha"], x["beta"])
    o2, _ = oracle.scan(x["q"], x["k"], x["v"][..., 2:], x["alpha"], x["beta"])
    assert np.abs(np.concatenate([o1, o2], -1) - o).max() < 1e-14
    v2 = np.random.default_rng(1).standard_normal(x["v"].shape)
    oa, _ = oracle.scan(x["q"], x["k"], x["v"] * 2.5 + v2, x["alpha"], x["beta"])
    ob, _ = oracle.scan(x["q"], x["k"], v2, x["alpha"], x["beta"])
    assert np.abs(oa - (2.5 * o + ob)).max() < 1e-13


def test_scan_batch_head_equivariance():
    """Permuting (batch, head) slots permutes the results and nothing else."""
    x = _rand_scan(10, 3, 20, 4, 8, 8)
    o, s = oracle.scan(x["q"], x["k"], x["v"], x["alpha"], x["beta"], x["s_init"])
    pb, ph = [2, 0, 1], [3, 1, 0, 2]
    p = lambda a: a[pb][:, :, ph] if a.ndim >= 3 else a[pb][:, ph]
    ps = x["s_init"][pb][:, ph]
    o2, s2 = oracle.scan(p(x["q"]), p(x["k"]), p(x["v"]), p(x["alpha"]), p(x["beta"]), ps)
    assert np.array_equal(o2, p(o)) and np.array_equal(s2, s[pb][:, ph])


# ---------------------------------------------------------------------------
# projections, normalisation and gates
# ---------------------------------------------------------------------------
def test_project_one_hot_rows_select_weight_rows():
    """x = e_m picks row m of each weight: q_j = Wq[m, head j] / sqrt(|.|^2 + eps), v_j = Wv[m, head j].
    Catches transposed weights and wrong head slicing."""
    d, H, dk, dv = 12, 3, 4, 4
    rng = np.random.default_rng(11)
    Wq, Wk, Wv = (rng.standard_normal((d, H * n)) for n in (dk, dk, dv))
    wa, wb = rng.standard_normal((d, H)), rng.standard_normal((d, H))
    x = np.eye(d)
    q, k, v, al, be = oracle.project(x, Wq, Wk, Wv, wa, wb, H, dk, dv, 0.0, "f32")
    for m in range(d):
        for j in range(H):
            rq = Wq[m, j * dk:(j + 1) * dk]
            assert np.allclose(q[m, j], rq / math.sqrt(rq @ rq + 1e-6), rtol=0, atol=1e-15)
            rk = Wk[m, j * dk:(j + 1) * dk]
            assert np.allclose(k[m, j], rk / math.sqrt(rk @ rk + 1e-6), rtol=0, atol=1e-15)
            assert np.array_equal(v[m, j], Wv[m, j * dv:(j + 1) * dv])


def test_gates_closed_forms():
    """alpha_lo = 0 gives alpha = exp(-softplus(a)); alpha in (alpha_lo, 1); a = 0 gives the midpoint;
    beta = sigmoid(b) with beta(0) = 1/2."""
    d, H = 4, 2
    x = np.eye(d) * np.array([[-30.0], [-1.0], [0.0], [2.5]])
    wa = np.ones((d, H))
    wb = np.ones((d, H))
    Z = np.zeros((d, H * 2))
    for lo in (0.0, 0.9, 0.95):
        _, _, _, al, be = oracle.project(x, Z, Z, Z, wa, wb, H, 2, 2, lo, "f32")
        a = np.diag(x)[:, None] * np.ones((1, H))
        ref = lo + (1 - lo) * np.exp(-np.logaddexp(0.0, a))
        assert np.abs(al - ref).max() < 1e-15
        assert np.all(al > lo) and np.all(al < 1.0)
        assert abs(al[2, 0] - (lo + (1 - lo) / 2)) < 1e-15
        assert abs(be[2, 0] - 0.5) < 1e-15
        assert np.abs(be - 1 / (1 + np.exp(-a))).max() < 1e-15
        assert np.abs((be + 1 / (1 + np.exp(a))) - 1).max() < 1e-15


def test_project_bf16_rounding_points():
    """bf16 workloads store q/k/v as bf16 and alpha/beta as fp32: every stored value is on that grid."""
    rng = np.random.default_rng(12)
    d, H, dk, dv = 64, 2, 32, 32
    W = [rng.standard_normal((d, H * n)) / 8 for n in (dk, dk, dv)]
    wa, wb = rng.standard_normal((d, H)), rng.standard_normal((d, H))
    x = oracle.round_bf16(rng.standard_normal((10, d)))
    q, k, v, al, be = oracle.project(x, *W, wa, wb, H, dk, dv, 0.9, "bf16")
    for t in (q, k, v):
        assert np.array_equal(t, oracle.round_bf16(t))
    for t in (al, be):
        assert np.array_equal(t, oracle.round_f32(t))
    # unit norm up to the bf16 grid
    assert np.abs(np.linalg.norm(q, axis=-1) - 1).max() < 2e-2


# ---------------------------------------------------------------------------
# the loop driver
# ---------------------------------------------------------------------------
def _tiny_loop_inputs(seed=0, B=2, L=40, H=2, dk=8, dv=8, T=3):
    rng = np.random.default_rng(seed)
    d = H * dv
    return dict(h0=rng.standard_normal((B, L, d)),
                Wq=rng.standard_normal((d, H * dk)) / math.sqrt(d),
                Wk=rng.standard_normal((d, H * dk)) / math.sqrt(d),
                Wv=rng.standard_normal((d, H * dv)) / math.sqrt(d),
                wa=rng.standard_normal((d, H)) / math.sqrt(d),
                wb=rng.standard_normal((d, H)) / math.sqrt(d),
                rho=rng.random((T, d)) * 0.5), dict(H=H, dk=dk, dv=dv)


def test_loop_zero_values_closed_form():
    """Wv = 0 makes every v and o zero, so h^(T) = (prod_tau rho_tau) (.) h^(0) exactly."""
    x, s = _tiny_loop_inputs(1)
    x["Wv"] = np.zeros_like(x["Wv"])
    r = oracle.loop_prefill(**x, **s, alpha_lo=0.0, act="f32")
    ref = np.prod(x["rho"], axis=0)[None, None] * x["h0"]
    assert np.abs(r["h"] - ref).max() < 1e-15


def test_loop_single_iteration_is_one_pass_plus_gate():
    """T = 1: h^(1) = scan(project(h0)) + rho_1 (.) h0."""
    x, s = _tiny_loop_inputs(2, T=1)
    r = oracle.loop_prefill(**x, **s, alpha_lo=0.0, act="f32")
    B, L, d = x["h0"].shape
    q, k, v, a, b = oracle.project(x["h0"].reshape(B * L, d), x["Wq"], x["Wk"], x["Wv"], x["wa"], x["wb"],
                                   s["H"], s["dk"], s["dv"], 0.0, "f32")
    o, _ = oracle.scan(q.reshape(B, L, s["H"], -1), k.reshape(B, L, s["H"], -1), v.reshape(B, L, s["H"], -1),
                       a.reshape(B, L, s["H"]), b.reshape(B, L, s["H"]))
    assert np.abs(r["h"] - (o.reshape(B, L, d) + x["rho"][0] * x["h0"])).max() < 1e-15


def test_loop_gate_order_and_zero_rho():
    """rho = 0 leaves only the last loop's mixer output; with rho_1 = 0 and rho_2 = 1 (T = 2),
    h^(2) = o^(2) + o^(1) -- which fails if the gates were applied in the wrong order."""
    x, s = _tiny_loop_inputs(3, T=2)
    B, L, d = x["h0"].shape
    x["rho"] = np.zeros((2, d))
    r0 = oracle.loop_prefill(**x, **s, alpha_lo=0.0, act="f32", keep_loops=True)
    x["rho"][1] = 1.0
    r1 = oracle.loop_prefill(**x, **s, alpha_lo=0.0, act="f32", keep_loops=True)
    o1 = r0["loops"][0]
    assert np.abs(r1["loops"][0] - o1).max() == 0.0
    assert np.abs(r1["h"] - (r0["h"] + o1)).max() < 1e-14


def test_loop_causal_prefix():
    """Token t of every loop depends on tokens <= t only: a prefix run equals the prefix of a full run."""
    x, s = _tiny_loop_inputs(4, L=70)
    full = oracle.loop_prefill(**x, **s, alpha_lo=0.9, act="bf16")
    y = dict(x)
    y["h0"] = x["h0"][:, :33]
    pre = oracle.loop_prefill(**y, **s, alpha_lo=0.9, act="bf16")
    assert np.array_equal(pre["h"], full["h"][:, :33])


def test_prefill_then_decode_equals_longer_prefill():
    """States of a prefill over L tokens plus one recurrent decode step equal a prefill over L+1 tokens
    (one state per loop, each loop continuing its own scan)."""
    for act in ("f32", "bf16"):
        x, s = _tiny_loop_inputs(5, L=41)
        full = oracle.loop_prefill(**x, **s, alpha_lo=0.0, act=act)
        y = dict(x)
        y["h0"] = x["h0"][:, :40]
        pre = oracle.loop_prefill(**y, **s, alpha_lo=0.0, act=act, keep_states=True)
        states = np.stack(pre["states"])
        kw = {k: v for k, v in x.items() if k != "h0"}
        h, _ = oracle.loop_decode_step(x["h0"][:, 40], states=states, **kw, **s, alpha_lo=0.0, act=act)
        assert np.abs(h - full["h"][:, 40]).max() < 1e-13


def test_loop_sequences_independent():
    x, s = _tiny_loop_inputs(6, B=3)
    r = oracle.loop_prefill(**x, **s, alpha_lo=0.0, act="f32")
    y = dict(x)
    y["h0"] = x["h0"][1:2]
    r1 = oracle.loop_prefill(**y, **s, alpha_lo=0.0, act="f32")
    assert np.array_equal(r1["h"][0], r["h"][1])


# ---------------------------------------------------------------------------
# seeded generators are deterministic
# ---------------------------------------------------------------------------
def test_generators_deterministic():
    w = synth.workload("tiny_f32")
    a, b = synth.prefill_inputs(w), synth.prefill_inputs(w)
    for key in a:
        assert torch.equal(a[key], b[key])
    assert a["h0"].shape == (1, 256, 64) and a["h0"].dtype == torch.float32
    x1 = synth.scan_inputs(3, 1, 10, 2, 8, 8)
    x2 = synth.scan_inputs(3, 1, 10, 2, 8, 8)
    assert all(torch.equal(x1[k], x2[k]) for k in x1)
    assert torch.allclose(x1["q"].float().norm(dim=-1), torch.ones(1, 10, 2), atol=1e-2)


def test_round_bf16_jitter_moves_one_fp32_ulp():
    """With a jitter generator, each result is the bf16 rounding of the fp32 value one ulp above or below."""
    rng = np.random.default_rng(3)
    x = rng.standard_normal(50000) * 10.0 ** rng.integers(-6, 6, 50000)
    f = x.astype(np.float32)
    up = oracle.round_bf16(np.nextafter(f, np.float32(np.inf)).astype(np.float64))
    dn = oracle.round_bf16(np.nextafter(f, np.float32(-np.inf)).astype(np.float64))
    j = oracle.round_bf16(x, np.random.default_rng(4))
    assert np.all((j == up) | (j == dn))
    assert np.mean(j != oracle.round_bf16(x)) < 0.01
    # exact midpoints of the bf16 grid: the one-ulp move decides the rounding either way
    ties = ((np.arange(1, 20001, dtype=np.uint32) << 16) | np.uint32(0x8000)).view(np.float32).astype(np.float64)
    jt = oracle.round_bf16(ties, np.random.default_rng(5))
    assert 0.3 < np.mean(jt != oracle.round_bf16(ties)) < 0.7
    # fp32 workloads have no bf16 rounding point: jitter leaves the loop unchanged
    xx, s = _tiny_loop_inputs(7)
    a = oracle.loop_prefill(**xx, **s, alpha_lo=0.0, act="f32")
    b = oracle.loop_prefill(**xx, **s, alpha_lo=0.0, act="f32", jitter=np.random.default_rng(0))
    assert np.array_equal(a["h"], b["h"])


def test_project_fp32_sum_is_a_float32_summation():
    """fp32_sum forms the dot products in float32: v equals a float32 matmul; all within fp32 error of fp64."""
    rng = np.random.default_rng(13)
    d, H, D = 256, 2, 32
    W = [rng.standard_normal((d, H * D)) / 16 for _ in range(3)]
    wa, wb = rng.standard_normal((d, H)), rng.standard_normal((d, H))
    x = rng.standard_normal((20, d))
    a = oracle.project(x, *W, wa, wb, H, D, D, 0.0, "f32")
    b = oracle.project(x, *W, wa, wb, H, D, D, 0.0, "f32", fp32_sum=True)
    ref_v = (x.astype(np.float32) @ W[2].astype(np.float32)).astype(np.float64).reshape(20, H, D)
    assert np.array_equal(b[2], ref_v)
    assert np.abs(b[2] - a[2]).max() < 1e-4 and np.abs(b[2] - a[2]).max() > 0
    assert np.abs(b[0] - a[0]).max() < 1e-5 and np.abs(b[1] - a[1]).max() < 1e-5
    assert np.array_equal(b[3], a[3]) and np.array_equal(b[4], a[4])  # gates stay fp64
