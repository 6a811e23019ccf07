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


# ---------------------------------------------------------------------------
# backward of the scan: pinned by finite differences of the (pinned) forward
# ---------------------------------------------------------------------------
def _bwd_case(seed, B, L, H, dk, dv, beta_hi=1.0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, L, H, dk)); q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k = rng.standard_normal((B, L, H, dk)); k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, L, H, dv))
    al = rng.uniform(0.3, 1.0, (B, L, H))
    be = rng.uniform(0.0, beta_hi, (B, L, H))
    s0 = rng.standard_normal((B, H, dk, dv)) * 0.3
    do = rng.standard_normal((B, L, H, dv))
    dsf = rng.standard_normal((B, H, dk, dv))
    return dict(q=q, k=k, v=v, alpha=al, beta=be, s_init=s0), do, dsf


def _loss(x, do, dsf):
    o, s = oracle.scan(x["q"], x["k"], x["v"], x["alpha"], x["beta"], x["s_init"])
    return float(np.sum(o * do) + np.sum(s * dsf))


@pytest.mark.parametrize("B,L,H,dk,dv,beta_hi", [(2, 7, 2, 4, 3, 1.0), (1, 9, 1, 5, 5, 2.0)])
def test_scan_backward_equals_central_differences(B, L, H, dk, dv, beta_hi):
    """Every gradient element against (L(x + e) - L(x - e)) / 2e of the forward oracle, L = <d_o, o> +
    <d_S, S_final>; fp64 central differences are exact to O(e^2) (e = 1e-5 here, error ~1e-9)."""
    x, do, dsf = _bwd_case(11 + L, B, L, H, dk, dv, beta_hi)
    g = oracle.scan_backward(x["q"], x["k"], x["v"], x["alpha"], x["beta"], do, x["s_init"], dsf)
    names = {"q": "dq", "k": "dk", "v": "dv", "alpha": "dalpha", "beta": "dbeta", "s_init": "ds_init"}
    eps = 1e-5
    for key, gk in names.items():
        base = x[key]
        fd = np.zeros_like(base)
        for idx in np.ndindex(base.shape):
            xp, xm = dict(x), dict(x)
            xp[key] = base.copy(); xp[key][idx] += eps
            xm[key] = base.copy(); xm[key][idx] -= eps
            fd[idx] = (_loss(xp, do, dsf) - _loss(xm, do, dsf)) / (2 * eps)
        err = np.max(np.abs(fd - g[gk])) / max(np.max(np.abs(fd)), 1e-12)
        assert err < 1e-7, (key, err)


def test_scan_backward_directional_long():
    """Past the 64-token checkpoint blocks (L = 150): directional derivatives along random directions of
    every input at once agree with central differences."""
    x, do, dsf = _bwd_case(5, 1, 150, 2, 8, 6)
    g = oracle.scan_backward(x["q"], x["k"], x["v"], x["alpha"], x["beta"], do, x["s_init"], dsf)
    rng = np.random.default_rng(6)
    names = {"q": "dq", "k": "dk", "v": "dv", "alpha": "dalpha", "beta": "dbeta", "s_init": "ds_init"}
    for trial in range(3):
        dirs = {key: rng.standard_normal(x[key].shape) for key in names}
        eps = 1e-6
        xp = {key: x[key] + eps * dirs[key] for key in names}
        xm = {key: x[key] - eps * dirs[key] for key in names}
        fd = (_loss(xp, do, dsf) - _loss(xm, do, dsf)) / (2 * eps)
        an = sum(float(np.sum(g[gk] * dirs[key])) for key, gk in names.items())
        assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (fd, an)


def test_scan_backward_pure_decay_closed_form():
    """beta = 0: S_t = gamma_t S_0 and o_t = gamma_t S_0^T q_t, so dq_t = gamma_t S_0 d_o_t, dk = dv = 0 and
    dS_0 = sum_t gamma_t q_t d_o_t^T + gamma_L d_S (gamma_t the product of alpha up to t)."""
    x, do, dsf = _bwd_case(21, 1, 70, 1, 6, 5)
    x["beta"][:] = 0.0
    g = oracle.scan_backward(x["q"], x["k"], x["v"], x["alpha"], x["beta"], do, x["s_init"], dsf)
    gam = np.cumprod(x["alpha"][0, :, 0])
    S0 = x["s_init"][0, 0]
    dq = gam[:, None] * (do[0, :, 0] @ S0.T)
    assert np.allclose(g["dq"][0, :, 0], dq, rtol=1e-12, atol=1e-12)
    assert np.all(g["dk"] == 0) and np.all(g["dv"] == 0)
    ds0 = np.einsum("t,ti,tj->ij", gam, x["q"][0, :, 0], do[0, :, 0]) + gam[-1] * dsf[0, 0]
    assert np.allclose(g["ds_init"][0, 0], ds0, rtol=1e-12, atol=1e-12)


def test_scan_backward_split_chain_rule():
    """Gradients through [0, m) then [m, L) (the second half's ds_init fed to the first half as dS_final)
    equal the single pass's."""
    x, do, dsf = _bwd_case(31, 1, 100, 2, 6, 4)
    g = oracle.scan_backward(x["q"], x["k"], x["v"], x["alpha"], x["beta"], do, x["s_init"], dsf)
    m = 37
    a = {key: (val[:, :m] if key != "s_init" else val) for key, val in x.items()}
    _, s_m = oracle.scan(a["q"], a["k"], a["v"], a["alpha"], a["beta"], a["s_init"])
    b = {key: (val[:, m:] if key != "s_init" else s_m) for key, val in x.items()}
    g2 = oracle.scan_backward(b["q"], b["k"], b["v"], b["alpha"], b["beta"], do[:, m:], b["s_init"], dsf)
    g1 = oracle.scan_backward(a["q"], a["k"], a["v"], a["alpha"], a["beta"], do[:, :m], a["s_init"], g2["ds_init"])
    for key in ("dq", "dk", "dv", "dalpha", "dbeta"):
        assert np.allclose(np.concatenate([g1[key], g2[key]], 1), g[key], rtol=1e-11, atol=1e-12), key
    assert np.allclose(g1["ds_init"], g["ds_init"], rtol=1e-11, atol=1e-12)


# ---------------------------------------------------------------------------
# adaptive halting (ACT) in the loop driver
# ---------------------------------------------------------------------------
def _act_inputs(seed, B=2, L=40, H=2, D=8):
    x, s = _tiny_loop_inputs(seed, B=B, L=L, H=H, dk=D, dv=D, T=4)
    rng = np.random.default_rng(seed + 100)
    w = rng.standard_normal(H * D) / np.sqrt(H * D)
    return x, s, w


def test_act_extremes_equal_plain_loops():
    """b = +inf: every position halts after loop 1 (h = h^(1)); b = -inf: none halts (the plain T loops)."""
    x, s, w = _act_inputs(41)
    plain = oracle.loop_prefill(**x, **s, alpha_lo=0.0, act="f32", keep_loops=True)
    r = oracle.loop_prefill_act(**x, w_halt=w, b_halt=60.0, eps=0.01, **s, alpha_lo=0.0, act="f32")
    assert np.array_equal(r["h"], plain["loops"][0]) and np.all(r["halt_loop"] == 1)
    r = oracle.loop_prefill_act(**x, w_halt=w, b_halt=-60.0, eps=0.01, **s, alpha_lo=0.0, act="f32")
    assert np.array_equal(r["h"], plain["h"]) and np.all(r["halt_loop"] == x["rho"].shape[0])


@pytest.mark.parametrize("pval,tau", [(0.5, 2), (0.3, 4), (0.995, 1)])
def test_act_constant_probability_halts_at_the_threshold_loop(pval, tau):
    """w = 0 gives every position p = sigmoid(b): the running sum first reaches 1 - 0.01 after
    ceil(0.99 / p) loops (0.5 -> 2, 0.3 -> 4, 0.995 -> 1), and h equals that loop's h of the plain run."""
    x, s, w = _act_inputs(42)
    b = float(np.log(pval / (1 - pval)))
    plain = oracle.loop_prefill(**x, **s, alpha_lo=0.0, act="f32", keep_loops=True)
    r = oracle.loop_prefill_act(**x, w_halt=np.zeros_like(w), b_halt=b, eps=0.01, **s, alpha_lo=0.0, act="f32")
    assert np.all(r["halt_loop"] == tau)
    assert np.array_equal(r["h"], plain["loops"][tau - 1])
    assert np.allclose(r["ponder"], tau * pval, rtol=1e-6)


def test_act_frozen_position_is_context_but_not_updated():
    """Only the last position can halt (its halting logit is raised by a large feature only it carries):
    every earlier position is causally unaffected and equals the plain loop, and the last position stays at
    its h^(tau_t) of the plain loop once halted."""
    x, s, w = _act_inputs(43, B=1, L=30)
    h0 = x["h0"].copy()
    h0[0, -1, 0] = 1000.0                     # a feature only the last position carries,
    x["h0"] = h0
    x["rho"] = x["rho"].copy()
    x["rho"][:, 0] = 0.5                      # kept by the residual gate of every loop
    w = np.zeros_like(w)
    w[0] = 1.0                                # logit = h[0] + b: very large only for the last position
    plain = oracle.loop_prefill(**x, **s, alpha_lo=0.0, act="f32", keep_loops=True)
    r = oracle.loop_prefill_act(**x, w_halt=w, b_halt=-20.0, eps=0.01, **s, alpha_lo=0.0, act="f32",
                                keep_loops=True)
    assert r["halt_loop"][0, -1] == 1 and np.all(r["halt_loop"][0, :-1] == x["rho"].shape[0])
    assert np.array_equal(r["h"][0, :-1], plain["h"][0, :-1])
    assert np.array_equal(r["h"][0, -1], plain["loops"][0][0, -1])


# ---------------------------------------------------------------------------
# backward through the T loops
# ---------------------------------------------------------------------------
_LB_KEYS = ("h0", "Wq", "Wk", "Wv", "wa", "wb", "rho")
_LB_GRADS = {"h0": "dh0", "Wq": "dWq", "Wk": "dWk", "Wv": "dWv", "wa": "dwa", "wb": "dwb", "rho": "drho"}


def _loop_loss(x, s, dh, alpha_lo):
    return float(np.sum(oracle.loop_prefill(**x, **s, alpha_lo=alpha_lo, act="f32")["h"] * dh))


def _loop_grads(x, s, dh, alpha_lo, act="f32"):
    fwd = oracle.loop_prefill(**x, **s, alpha_lo=alpha_lo, act=act, keep_loops=True)
    return oracle.loop_backward(**x, loops=fwd["loops"], dh=dh, **s, alpha_lo=alpha_lo, act=act)


@pytest.mark.parametrize("alpha_lo,T", [(0.0, 3), (0.6, 2)])
def test_loop_backward_equals_central_differences(alpha_lo, T):
    """Every element of dh0, dWq, dWk, dWv, dwa, dwb and drho against central differences of L = <dh, h^(T)>
    through the fp64 forward loop (e = 1e-6; exact to O(e^2))."""
    x, s = _tiny_loop_inputs(51 + T, B=2, L=6, H=2, dk=3, dv=3, T=T)
    dh = np.random.default_rng(7).standard_normal(x["h0"].shape)
    g = _loop_grads(x, s, dh, alpha_lo)
    eps = 1e-6
    for key in _LB_KEYS:
        base = x[key]
        fd = np.zeros_like(base)
        for idx in np.ndindex(base.shape):
            xp, xm = dict(x), dict(x)
            xp[key] = base.copy(); xp[key][idx] += eps
            xm[key] = base.copy(); xm[key][idx] -= eps
            fd[idx] = (_loop_loss(xp, s, dh, alpha_lo) - _loop_loss(xm, s, dh, alpha_lo)) / (2 * eps)
        err = np.max(np.abs(fd - g[_LB_GRADS[key]])) / max(np.max(np.abs(fd)), 1e-12)
        assert err < 1e-6, (key, err)


def test_loop_backward_directional_long():
    """Past the scan's 64-token checkpoint blocks (L = 100, 2 sequences, 4 loops): directional derivatives along
    random directions of every input at once agree with central differences."""
    x, s = _tiny_loop_inputs(61, B=2, L=100, H=2, dk=4, dv=4, T=4)
    rng = np.random.default_rng(62)
    dh = rng.standard_normal(x["h0"].shape)
    g = _loop_grads(x, s, dh, 0.3)
    for trial in range(2):
        dirs = {key: rng.standard_normal(x[key].shape) for key in _LB_KEYS}
        eps = 1e-6
        xp = {key: x[key] + eps * dirs[key] for key in _LB_KEYS}
        xm = {key: x[key] - eps * dirs[key] for key in _LB_KEYS}
        fd = (_loop_loss(xp, s, dh, 0.3) - _loop_loss(xm, s, dh, 0.3)) / (2 * eps)
        an = sum(float(np.sum(g[_LB_GRADS[key]] * dirs[key])) for key in _LB_KEYS)
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (fd, an)


@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_loop_backward_zero_values_closed_form(act):
    """Wv = 0: h^(T) = (prod rho) (.) h0 whatever q, k and the gates are, so dh0 = (prod rho) (.) dh,
    drho_tau = sum over positions of dh (.) h0 (.) prod_{sigma != tau} rho_sigma, and the gradients of Wq, Wk,
    wa, wb vanish exactly (the state stays zero, so nothing downstream depends on them)."""
    x, s = _tiny_loop_inputs(71, B=2, L=30, H=2, dk=4, dv=4, T=3)
    x["Wv"] = np.zeros_like(x["Wv"])
    if act == "bf16":
        x["h0"] = oracle.round_bf16(x["h0"])
    dh = np.random.default_rng(72).standard_normal(x["h0"].shape)
    g = _loop_grads(x, s, dh, 0.2, act)
    rho = x["rho"]
    assert np.allclose(g["dh0"], np.prod(rho, 0)[None, None] * dh, rtol=1e-13, atol=1e-15)
    for t in range(rho.shape[0]):
        others = np.prod(np.delete(rho, t, axis=0), 0)
        ref = np.sum(dh * x["h0"], axis=(0, 1)) * others
        assert np.allclose(g["drho"][t], ref, rtol=1e-12, atol=1e-14)
    for key in ("dWq", "dWk", "dwa", "dwb"):
        assert np.all(g[key] == 0), key


def test_loop_backward_given_operands_are_used_for_the_scan():
    """The rounded q, k, v handed in (per loop) replace the oracle's own: handing in its own roundings gives the
    same gradients bit for bit, and handing in q, k, v moved by one bf16 step at one position changes them."""
    x, s = _tiny_loop_inputs(81, B=1, L=20, H=2, dk=4, dv=4, T=2)
    x["h0"] = oracle.round_bf16(x["h0"])
    dh = np.random.default_rng(82).standard_normal(x["h0"].shape)
    fwd = oracle.loop_prefill(**x, **s, alpha_lo=0.1, act="bf16", keep_loops=True)
    ins = [x["h0"]] + fwd["loops"][:-1]
    own = []
    for h in ins:
        q, k, v, _, _ = oracle.project(oracle.round_bf16(h.reshape(20, 8)), x["Wq"], x["Wk"], x["Wv"], x["wa"],
                                       x["wb"], 2, 4, 4, 0.1, "bf16")
        own.append((q, k, v))
    base = oracle.loop_backward(**x, loops=fwd["loops"], dh=dh, **s, alpha_lo=0.1, act="bf16")
    same = oracle.loop_backward(**x, loops=fwd["loops"], dh=dh, **s, alpha_lo=0.1, act="bf16", qkv=own)
    for key in base:
        assert np.array_equal(base[key], same[key]), key
    moved = [tuple(t.copy() for t in o) for o in own]
    moved[1][1][5, 0, 2] = moved[1][1][5, 0, 2] * (1 + 2.0 ** -7)   # k of loop 2, one element, one bf16 step
    diff = oracle.loop_backward(**x, loops=fwd["loops"], dh=dh, **s, alpha_lo=0.1, act="bf16", qkv=moved)
    assert not np.array_equal(diff["dWk"], base["dWk"])


# ---------------------------------------------------------------------------
# the LT2 block around the mixer
# ---------------------------------------------------------------------------
def _block_weights(seed, d, H, dk, dv, F):
    rng = np.random.default_rng(seed)
    n = lambda *shape: rng.standard_normal(shape) / math.sqrt(shape[0])
    return dict(g1=1.0 + 0.1 * rng.standard_normal(d), Wq=n(d, H * dk), Wk=n(d, H * dk), Wv=n(d, H * dv),
                wa=n(d, H), wb=n(d, H), Wg=n(d, H * dv), Wo=n(H * dv, d), g2=1.0 + 0.1 * rng.standard_normal(d),
                W1=n(d, F), W3=n(d, F), W2=n(F, d))


def test_ffn_width_and_rms_norm_hand_values():
    """8d/3 rounded up to 256: 2048 -> 5461.3 -> 5632, 1024 -> 2730.7 -> 2816; rms_norm([3, 4]) =
    [3, 4] / sqrt(12.5) (hand-computed 0.848528.., 1.131370..) times the weight."""
    assert oracle.ffn_width(2048) == 5632 and oracle.ffn_width(1024) == 2816 and oracle.ffn_width(96) == 256
    r = oracle.rms_norm(np.array([3.0, 4.0]), np.array([1.0, 2.0]), eps=0.0)
    assert np.allclose(r, [0.8485281374238570, 2 * 1.1313708498984760], rtol=1e-14)


@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_block_zero_projections_is_identity(act):
    """Wo = W2 = 0: both sub-layers add nothing, F(h) = h exactly; so T loops give prod(1 + rho_tau) (.) h0."""
    d, H, D = 16, 2, 8
    w = _block_weights(91, d, H, D, D, 256)
    w["Wo"][:] = 0.0
    w["W2"][:] = 0.0
    h = oracle.round_bf16(np.random.default_rng(92).standard_normal((2, 20, d)))
    assert np.array_equal(oracle.block_forward(h, w, H, D, D, 0.0, act), h)
    rho = np.random.default_rng(93).random((3, d)) * 0.5
    r = oracle.block_loop_prefill(h, [w, w], rho, H, D, D, 0.0, act)
    assert np.allclose(r["h"], np.prod(1.0 + rho, 0)[None, None] * h, rtol=1e-14)


def test_block_ffn_matches_library_rms_norm_and_silu():
    """Wv = 0 makes the mixer output zero (F(h) = h + FFN(h)); the FFN sub-layer then equals torch's
    rms_norm and silu composed by hand: (silu(x2 W1) * (x2 W3)) W2 with x2 = rms_norm(h; g2)."""
    d, H, D, F = 24, 3, 8, 256
    w = _block_weights(94, d, H, D, D, F)
    w["Wv"][:] = 0.0
    h = np.random.default_rng(95).standard_normal((1, 9, d))
    got = oracle.block_forward(h, w, H, D, D, 0.2, "f32") - h
    t = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float64))
    x2 = torch.nn.functional.rms_norm(t(h), (d,), weight=t(w["g2"]), eps=1e-6)
    ref = (torch.nn.functional.silu(x2 @ t(w["W1"])) * (x2 @ t(w["W3"]))) @ t(w["W2"])
    assert np.allclose(got, ref.numpy(), rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("zero_gate", [True, False])
def test_block_mixer_sublayer_is_the_pinned_loop_through_the_gate(zero_gate):
    """W2 = 0: F(h) = h + (o (.) sigmoid(x1 Wg)) Wo, where x1 = rms_norm(h; g1) (torch's routine) and o is the
    mixer output of x1, i.e. one loop of the pinned loop_prefill with rho = 0 applied to x1.  With Wg = 0
    every gate is sigmoid(0) = 1/2."""
    d, H, D = 16, 2, 8
    w = _block_weights(96, d, H, D, D, 256)
    w["W2"][:] = 0.0
    if zero_gate:
        w["Wg"][:] = 0.0
    h = np.random.default_rng(97).standard_normal((2, 70, d))
    t = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float64))
    x1 = torch.nn.functional.rms_norm(t(h), (d,), weight=t(w["g1"]), eps=1e-6)
    o = oracle.loop_prefill(x1.numpy(), w["Wq"], w["Wk"], w["Wv"], w["wa"], w["wb"], np.zeros((1, d)), H, D, D,
                            0.3, "f32")["h"]
    gate = torch.sigmoid(x1 @ t(w["Wg"])).numpy()
    if zero_gate:
        assert np.all(gate == 0.5)
    got = oracle.block_forward(h, w, H, D, D, 0.3, "f32")
    assert np.allclose(got, h + (o * gate) @ w["Wo"], rtol=1e-12, atol=1e-13)


def test_block_loop_composes_blocks_and_the_loop_residual():
    """h^(1) = F_2(F_1(h0)) + rho_1 (.) h0 and h^(2) = F_2(F_1(h^(1))) + rho_2 (.) h^(1), block by block."""
    d, H, D = 16, 2, 8
    w1, w2 = _block_weights(100, d, H, D, D, 256), _block_weights(101, d, H, D, D, 256)
    h0 = np.random.default_rng(102).standard_normal((1, 40, d))
    rho = np.random.default_rng(103).random((2, d)) * 0.5
    f = lambda x: oracle.block_forward(oracle.block_forward(x, w1, H, D, D, 0.0, "f32"), w2, H, D, D, 0.0, "f32")
    h1 = f(h0) + rho[0] * h0
    h2 = f(h1) + rho[1] * h1
    r = oracle.block_loop_prefill(h0, [w1, w2], rho, H, D, D, 0.0, "f32", keep_loops=True)
    assert np.array_equal(r["loops"][0], h1) and np.array_equal(r["h"], h2)


def test_block_is_causal_and_sequences_independent():
    d, H, D = 16, 2, 8
    w = _block_weights(98, d, H, D, D, 256)
    h = np.random.default_rng(99).standard_normal((2, 30, d))
    base = oracle.block_forward(h, w, H, D, D, 0.1, "f32")
    h2 = h.copy()
    h2[0, 20:] += 1.0
    moved = oracle.block_forward(h2, w, H, D, D, 0.1, "f32")
    assert np.array_equal(moved[0, :20], base[0, :20]) and np.array_equal(moved[1], base[1])
    assert not np.allclose(moved[0, 20:], base[0, 20:])
