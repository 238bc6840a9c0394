"""Pins of the CPU oracle against closed forms, invariants and independent forms.

Each test computes what the mathematics fixes by a route that differs from the
oracle's token-by-token loop (a matmul of stacked records, a per-column scalar
recurrence, an explicit projector matrix, an identity between two of its
outputs), so that a dropped term, a wrong sign, an off-by-one decay index or a
transposed operand in the oracle fails at least one of them.
"""
import numpy as np
import pytest

import oracle
from synth import WORKLOADS, host_step, host_initial_state

RNG = np.random.default_rng(1234)


def _run_tokens_mamba2(S0, alpha, k, v, q):
    """All T tokens of each head through the oracle; returns outputs and final state."""
    S = S0.astype(np.float64).copy()
    nh, T = alpha.shape
    out = oracle.mamba2_round(S, alpha, k, v, q, np.full(nh, T, np.int32))
    return out, S


def _run_tokens_gdn(S0, alpha, beta, k, v, q):
    S = S0.astype(np.float64).copy()
    nh, T = alpha.shape
    out, u = oracle.gdn_round(S, alpha, beta, k, v, q, np.full(nh, T, np.int32))
    return out, u, S


def _rand(nh=3, T=7, P=5, N=6, unit_k=False):
    k = RNG.standard_normal((nh, T, N)).astype(np.float32)
    if unit_k:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    return dict(
        S0=RNG.standard_normal((nh, P, N)).astype(np.float32),
        k=k,
        v=RNG.standard_normal((nh, T, P)).astype(np.float32),
        q=RNG.standard_normal((nh, T, N)).astype(np.float32),
        alpha=RNG.uniform(0.3, 1.0, (nh, T)).astype(np.float32),
        beta=RNG.uniform(0.1, 1.0, (nh, T)).astype(np.float32),
    )


# ---------------------------------------------------------------- Mamba-2 --

def test_p1_alpha_one_is_sum_of_outer_products():
    """alpha = 1: S_t = S_0 + V_{1:t}^T K_{1:t}, one matmul over the stacked records."""
    d = _rand()
    nh, T = d["alpha"].shape
    out, S = _run_tokens_mamba2(d["S0"], np.ones_like(d["alpha"]), d["k"], d["v"], d["q"])
    for hd in range(nh):
        for t in range(T):
            V = d["v"][hd, : t + 1].astype(np.float64)
            K = d["k"][hd, : t + 1].astype(np.float64)
            St = d["S0"][hd].astype(np.float64) + V.T @ K
            np.testing.assert_allclose(out[hd, t], St @ d["q"][hd, t].astype(np.float64), rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(S[hd], St, rtol=1e-12, atol=1e-12)


def test_p2_alpha_zero_is_last_outer_product():
    """alpha = 0: the empty history; o_t = v_t (k_t . q_t), whatever S_0 holds."""
    d = _rand()
    out, S = _run_tokens_mamba2(d["S0"], np.zeros_like(d["alpha"]), d["k"], d["v"], d["q"])
    kq = np.einsum("htn,htn->ht", d["k"].astype(np.float64), d["q"].astype(np.float64))
    np.testing.assert_allclose(out, d["v"] * kq[..., None], rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("c", [0.5, 0.9, 1.3])
def test_p3_constant_decay_closed_form(c):
    """alpha = c: S_t = c^t S_0 + sum_j c^(t-j) v_j k_j^T (decay index pinned)."""
    d = _rand()
    nh, T = d["alpha"].shape
    alpha = np.full_like(d["alpha"], c)
    out, _ = _run_tokens_mamba2(d["S0"], alpha, d["k"], d["v"], d["q"])
    c64 = float(np.float32(c))
    for hd in range(nh):
        for t in range(1, T + 1):
            w = c64 ** (t - np.arange(1, t + 1))  # weights of records 1..t
            V = d["v"][hd, :t].astype(np.float64) * w[:, None]
            St = c64 ** t * d["S0"][hd].astype(np.float64) + V.T @ d["k"][hd, :t].astype(np.float64)
            np.testing.assert_allclose(out[hd, t - 1], St @ d["q"][hd, t - 1], rtol=1e-11, atol=1e-11)


def test_unrolled_form_equals_recurrence():
    """Random alpha: the unrolled sum Gamma_t S_0 q + sum_j gamma_{j,t} v_j (k_j . q).

    This is the identity the pages rest the method on (the state is a decayed
    checkpoint plus a sum over the buffered inputs), written with cumulative
    products and no state at all.
    """
    d = _rand(T=9)
    nh, T = d["alpha"].shape
    out, _ = _run_tokens_mamba2(d["S0"], d["alpha"], d["k"], d["v"], d["q"])
    a = d["alpha"].astype(np.float64)
    for hd in range(nh):
        for t in range(T):
            Gam = np.prod(a[hd, : t + 1])
            gam = np.array([np.prod(a[hd, j + 1 : t + 1]) for j in range(t + 1)])  # empty product = 1
            qt = d["q"][hd, t].astype(np.float64)
            kq = d["k"][hd, : t + 1].astype(np.float64) @ qt
            o = Gam * (d["S0"][hd].astype(np.float64) @ qt) + (d["v"][hd, : t + 1].T.astype(np.float64) @ (gam * kq))
            np.testing.assert_allclose(out[hd, t], o, rtol=1e-11, atol=1e-11)


def test_output_is_row_contraction_not_transposed():
    """P != N and a non-symmetric S_0: o = S q has P entries, contracted over N."""
    d = _rand(nh=1, T=1, P=3, N=8)
    out, _ = _run_tokens_mamba2(d["S0"], np.zeros((1, 1), np.float32) + 0.5, d["k"], d["v"], d["q"])
    S1 = 0.5 * d["S0"][0].astype(np.float64) + np.outer(d["v"][0, 0].astype(np.float64), d["k"][0, 0].astype(np.float64))
    assert out.shape == (1, 1, 3)
    np.testing.assert_allclose(out[0, 0], S1 @ d["q"][0, 0], rtol=1e-12)


# ------------------------------------------------------- Gated DeltaNet --

def test_p4_gdn_beta_one_writes_value_at_key():
    """beta = 1, ||k_t|| = 1, any alpha: S_t k_t = v_t exactly, so q_t = k_t reads v_t."""
    d = _rand()
    nh, T, N = d["k"].shape
    # keys with exactly unit norm in float: four entries of +-1/2, the rest zero
    k = np.zeros((nh, T, N), np.float32)
    for hd in range(nh):
        for t in range(T):
            idx = RNG.choice(N, 4, replace=False)
            k[hd, t, idx] = RNG.choice([-0.5, 0.5], 4)
    out, u, _ = _run_tokens_gdn(d["S0"], d["alpha"], np.ones_like(d["beta"]), k, d["v"], k)
    np.testing.assert_allclose(out, d["v"], rtol=1e-12, atol=1e-12)


def test_p5_gdn_beta_zero_only_decays():
    """beta = 0: S_t = Gamma_t S_0 and the correction records are zero."""
    d = _rand()
    out, u, S = _run_tokens_gdn(d["S0"], d["alpha"], np.zeros_like(d["beta"]), d["k"], d["v"], d["q"])
    G = np.cumprod(d["alpha"].astype(np.float64), axis=1)
    ref = G[..., None] * np.einsum("hpn,htn->htp", d["S0"].astype(np.float64), d["q"].astype(np.float64))
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)
    assert np.all(u == 0.0)


def test_p6_gdn_orthonormal_keys_column_recurrence():
    """k_t = e_{t mod d}: every column of S follows its own scalar recurrence.

    Written column by column: the keyed column becomes alpha (1 - beta) S e + beta v,
    every other column is scaled by alpha.
    """
    nh, T, P, N = 2, 11, 4, 4
    d = _rand(nh=nh, T=T, P=P, N=N)
    k = np.zeros((nh, T, N), np.float32)
    for t in range(T):
        k[:, t, t % N] = 1.0
    out, u, S = _run_tokens_gdn(d["S0"], d["alpha"], d["beta"], k, d["v"], d["q"])
    for hd in range(nh):
        cols = [d["S0"][hd, :, m].astype(np.float64) for m in range(N)]
        for t in range(T):
            a, b = float(d["alpha"][hd, t]), float(d["beta"][hd, t])
            for m in range(N):
                if m == t % N:
                    cols[m] = a * (1.0 - b) * cols[m] + b * d["v"][hd, t].astype(np.float64)
                else:
                    cols[m] = a * cols[m]
            St = np.stack(cols, axis=1)
            np.testing.assert_allclose(out[hd, t], St @ d["q"][hd, t].astype(np.float64), rtol=1e-11, atol=1e-11)
        np.testing.assert_allclose(S[hd], St, rtol=1e-11, atol=1e-11)


def test_gdn_projector_matrix_form():
    """S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T with explicit matrices."""
    d = _rand(unit_k=False)
    nh, T = d["alpha"].shape
    N = d["k"].shape[-1]
    out, u, S = _run_tokens_gdn(d["S0"], d["alpha"], d["beta"], d["k"], d["v"], d["q"])
    for hd in range(nh):
        St = d["S0"][hd].astype(np.float64)
        for t in range(T):
            a, b = float(d["alpha"][hd, t]), float(d["beta"][hd, t])
            kt = d["k"][hd, t].astype(np.float64)
            St = a * St @ (np.eye(N) - b * np.outer(kt, kt)) + b * np.outer(d["v"][hd, t].astype(np.float64), kt)
            np.testing.assert_allclose(out[hd, t], St @ d["q"][hd, t], rtol=1e-11, atol=1e-11)


def test_p7_gdn_correction_rewrite():
    """The page's rewrite: S_t = alpha_t S_{t-1} + u_t k_t^T with u_t = beta_t (v_t - alpha_t S_{t-1} k_t)."""
    d = _rand(T=6)
    nh, T = d["alpha"].shape
    S = d["S0"].astype(np.float64).copy()
    for t in range(T):
        prev = S.copy()
        sl = slice(t, t + 1)
        _, u = oracle.gdn_round(S, d["alpha"][:, sl], d["beta"][:, sl], d["k"][:, sl], d["v"][:, sl],
                                d["q"][:, sl], np.ones(nh, np.int32))
        rebuilt = d["alpha"][:, t, None, None] * prev + np.einsum("hp,hn->hpn", u[:, 0], d["k"][:, t].astype(np.float64))
        np.testing.assert_allclose(S, rebuilt, rtol=1e-12, atol=1e-13)
        w = np.einsum("hpn,hn->hp", prev, d["k"][:, t].astype(np.float64))
        np.testing.assert_allclose(u[:, 0], d["beta"][:, t, None] * (d["v"][:, t] - d["alpha"][:, t, None] * w),
                                   rtol=1e-12, atol=1e-13)


# ----------------------------------------------------------------- KDA --

def _run_tokens_kda(S0, alpha, beta, k, v, q):
    S = S0.astype(np.float64).copy()
    nh, T = beta.shape
    out, u = oracle.kda_round(S, alpha, beta, k, v, q, np.full(nh, T, np.int32))
    return out, u, S


def _alpha_vec(nh, T, N, lo=0.3):
    return RNG.uniform(lo, 1.0, (nh, T, N)).astype(np.float32)


def test_kda_uniform_gate_is_gdn():
    """A gate equal on every key channel reduces Kimi Delta Attention to Gated DeltaNet."""
    d = _rand(unit_k=True)
    nh, T, N = d["k"].shape
    av = np.repeat(d["alpha"][:, :, None], N, axis=2)
    o_kda, u_kda, S_kda = _run_tokens_kda(d["S0"], av, d["beta"], d["k"], d["v"], d["q"])
    o_gdn, u_gdn, S_gdn = _run_tokens_gdn(d["S0"], d["alpha"], d["beta"], d["k"], d["v"], d["q"])
    np.testing.assert_allclose(o_kda, o_gdn, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(u_kda, u_gdn, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(S_kda, S_gdn, rtol=1e-12, atol=1e-12)


def test_kda_beta_zero_decays_each_channel():
    """beta = 0: S_t = S_0 Diag(prod of the gates up to t), so o_t = S_0 (Gamma_t * q_t), per channel."""
    d = _rand()
    nh, T, N = d["k"].shape
    av = _alpha_vec(nh, T, N)
    out, u, S = _run_tokens_kda(d["S0"], av, np.zeros_like(d["beta"]), d["k"], d["v"], d["q"])
    G = np.cumprod(av.astype(np.float64), axis=1)  # [nh, T, N], includes token t's own gate
    ref = np.einsum("hpn,htn->htp", d["S0"].astype(np.float64), G * d["q"].astype(np.float64))
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)
    assert np.all(u == 0.0)


def test_kda_beta_one_writes_value_at_key_when_gates_open():
    """Gates all one, beta = 1, ||k_t|| = 1 exactly: S_t k_t = v_t, so q_t = k_t reads v_t."""
    d = _rand()
    nh, T, N = d["k"].shape
    k = np.zeros((nh, T, N), np.float32)
    for hd in range(nh):
        for t in range(T):
            idx = RNG.choice(N, 4, replace=False)
            k[hd, t, idx] = RNG.choice([-0.5, 0.5], 4)
    out, _, _ = _run_tokens_kda(d["S0"], np.ones((nh, T, N), np.float32), np.ones_like(d["beta"]), k, d["v"], k)
    np.testing.assert_allclose(out, d["v"], rtol=1e-12, atol=1e-12)


def test_kda_orthonormal_keys_column_recurrence():
    """k_t = e_{t mod d}: column m follows a_m (1 - beta) S e_m + beta v when keyed, a_m S e_m otherwise."""
    nh, T, P, N = 2, 11, 4, 4
    d = _rand(nh=nh, T=T, P=P, N=N)
    av = _alpha_vec(nh, T, N)
    k = np.zeros((nh, T, N), np.float32)
    for t in range(T):
        k[:, t, t % N] = 1.0
    out, u, S = _run_tokens_kda(d["S0"], av, d["beta"], k, d["v"], d["q"])
    for hd in range(nh):
        cols = [d["S0"][hd, :, m].astype(np.float64) for m in range(N)]
        for t in range(T):
            b = float(d["beta"][hd, t])
            for m in range(N):
                a = float(av[hd, t, m])
                cols[m] = a * (1.0 - b) * cols[m] + b * d["v"][hd, t].astype(np.float64) if m == t % N else a * cols[m]
            St = np.stack(cols, axis=1)
            np.testing.assert_allclose(out[hd, t], St @ d["q"][hd, t].astype(np.float64), rtol=1e-11, atol=1e-11)
        np.testing.assert_allclose(S[hd], St, rtol=1e-11, atol=1e-11)


def test_kda_projector_matrix_form_and_correction():
    """S_t = S_{t-1} Diag(a_t) (I - beta_t k_t k_t^T) + beta_t v_t k_t^T with explicit matrices, and
    S_t = S_{t-1} Diag(a_t) + u_t k_t^T with u_t = beta_t (v_t - S_{t-1} (a_t * k_t))."""
    d = _rand(T=6)
    nh, T, N = d["k"].shape
    av = _alpha_vec(nh, T, N)
    out, u, _ = _run_tokens_kda(d["S0"], av, d["beta"], d["k"], d["v"], d["q"])
    for hd in range(nh):
        St = d["S0"][hd].astype(np.float64)
        for t in range(T):
            b = float(d["beta"][hd, t])
            kt, vt = d["k"][hd, t].astype(np.float64), d["v"][hd, t].astype(np.float64)
            Da = np.diag(av[hd, t].astype(np.float64))
            ut = b * (vt - St @ (av[hd, t].astype(np.float64) * kt))
            np.testing.assert_allclose(u[hd, t], ut, rtol=1e-11, atol=1e-12)
            nxt = St @ Da @ (np.eye(N) - b * np.outer(kt, kt)) + b * np.outer(vt, kt)
            np.testing.assert_allclose(nxt, St @ Da + np.outer(ut, kt), rtol=1e-11, atol=1e-12)
            St = nxt
            np.testing.assert_allclose(out[hd, t], St @ d["q"][hd, t], rtol=1e-11, atol=1e-11)


# ------------------------------------------------ speculative semantics --

@pytest.mark.parametrize("kind", ["mamba2", "gdn", "kda"])
def test_round_accepts_prefix_only(kind):
    """A round's draft outputs equal step-by-step decoding, and the state advances by acc only."""
    d = _rand(nh=4, T=5, unit_k=(kind != "mamba2"))
    nh, T = d["alpha"].shape
    if kind == "kda":
        d["alpha"] = _alpha_vec(nh, T, d["k"].shape[-1])
    acc = np.array([0, 2, 5, 1], np.int32)
    S = d["S0"].astype(np.float64).copy()
    if kind == "mamba2":
        out = oracle.mamba2_round(S, d["alpha"], d["k"], d["v"], d["q"], acc)
    elif kind == "kda":
        out, _ = oracle.kda_round(S, d["alpha"], d["beta"], d["k"], d["v"], d["q"], acc)
    else:
        out, _ = oracle.gdn_round(S, d["alpha"], d["beta"], d["k"], d["v"], d["q"], acc)
    for hd in range(nh):
        Sx = d["S0"][hd : hd + 1].astype(np.float64).copy()
        for t in range(T):
            sl = (slice(hd, hd + 1), slice(t, t + 1))
            if kind == "mamba2":
                o = oracle.mamba2_round(Sx, d["alpha"][sl], d["k"][sl], d["v"][sl], d["q"][sl], np.ones(1, np.int32))
            elif kind == "kda":
                o, _ = oracle.kda_round(Sx, d["alpha"][sl], d["beta"][sl], d["k"][sl], d["v"][sl], d["q"][sl],
                                        np.ones(1, np.int32))
            else:
                o, _ = oracle.gdn_round(Sx, d["alpha"][sl], d["beta"][sl], d["k"][sl], d["v"][sl], d["q"][sl],
                                        np.ones(1, np.int32))
            np.testing.assert_array_equal(o[0, 0], out[hd, t])
            if t + 1 == acc[hd]:
                np.testing.assert_array_equal(Sx[0], S[hd])
        if acc[hd] == 0:
            np.testing.assert_array_equal(S[hd], d["S0"][hd].astype(np.float64))


# ------------------------------------------------------ oracle rounding --

def test_p11_fp32_oracle_close_to_fp64_on_tiny_workload():
    """The tiny Mamba-2 workload in float and double stays within float rounding."""
    w = WORKLOADS["mamba2_tiny"]
    sh = w.shape
    S64 = host_initial_state(0, w.wid, sh, w.s0_sigma).reshape(-1, sh.P, sh.N).astype(np.float64)
    S32 = S64.astype(np.float32)
    worst = 0.0
    for t in range(w.steps):
        x = host_step(0, w.wid, t, sh, 1)
        args = [x[f].transpose(0, 2, 1, *range(3, x[f].ndim)).reshape(sh.B * sh.H, 1, *x[f].shape[3:])
                for f in ("alpha", "k", "v", "q")]
        args[0] = args[0].reshape(-1, 1)
        o64 = oracle.mamba2_round(S64, *args, np.ones(sh.B * sh.H, np.int32), "f64")
        o32 = oracle.mamba2_round(S32, *args, np.ones(sh.B * sh.H, np.int32), "f32")
        err = np.abs(o32 - o64).max(axis=-1) / np.maximum(np.abs(o64).max(axis=-1), 1e-30)
        worst = max(worst, float(err.max()))
    assert worst < 1e-5, worst
