"""CPU checks of the harness's magnitude denominators (tests/harness.py, Magnitudes).

The bf16-read parity tests divide each head's output error by
max_p (Gamma_t sum_n |S_ck[p,n] q_n| + sum_j gamma_{j,t} |v_j[p]| |k_j . q_t|),
the sizes of the terms the output sums ("ReplaySSM: Cache SSM Inputs, Not
State", How it works: Standard decoding, the decayed checkpoint times q plus
the buffered records). Two facts pin that bookkeeping (which records, which
decays, when the checkpoint moves) without a GPU:

- when every term is non-negative (S_0, k, q, v >= 0, Mamba-2) the sum of
  magnitudes is the output itself, so the denominator equals max_p o_t[p] of the
  oracle exactly;
- otherwise it is never below max_p |o_t[p]| (triangle inequality).
"""
import numpy as np
import pytest

from harness import Magnitudes
from oracle.session import OracleSession

P, N = 6, 5


def _drive(kind, nonneg, rounds=30, seed=3, expanded=False):
    rng = np.random.default_rng(seed)
    B, H, L, T_max = 2, 3, 5, 4
    nh = B * H
    S0 = rng.standard_normal((nh, P, N))
    if nonneg:
        S0 = np.abs(S0)
    s = OracleSession(kind, B, H, P, N, L, T_max, S0.astype(np.float32))
    mag = Magnitudes(nh, L + T_max, P, N, expanded=expanded)
    seq = np.repeat(np.arange(B), H)
    worst_ratio = np.inf
    for rnd in range(rounds):
        T = int(rng.integers(1, T_max + 1))
        f = np.abs if nonneg else (lambda x: x)
        k = f(rng.standard_normal((nh, T, N))).astype(np.float32)
        if kind == "gdn":
            k /= np.linalg.norm(k, axis=-1, keepdims=True)
        q = f(rng.standard_normal((nh, T, N))).astype(np.float32)
        v = f(rng.standard_normal((nh, T, P))).astype(np.float32)
        alpha = rng.uniform(0.3, 1.0, (nh, T)).astype(np.float32)
        beta = rng.uniform(0.1, 1.0, (nh, T)).astype(np.float32) if kind == "gdn" else None
        s.append(alpha, k, v, beta)
        if rnd % 9 == 8:
            folds = s.flush()
            mag.fold(np.array([folds[b] for b in seq]))
        out, u, folds = s.verify(q)
        mag.fold(np.array([folds[b] for b in seq]))
        bound, U = mag.bounds(s.ckpt, alpha, k, v, q, beta)
        if u is not None:  # the correction never exceeds its terms' magnitude
            assert np.all(np.abs(u) <= U * (1 + 1e-12))
        omax = np.abs(out).max(axis=-1)
        if nonneg:
            np.testing.assert_allclose(bound, out.max(axis=-1), rtol=1e-12)
        else:
            assert np.all(bound >= omax * (1 - 1e-12))
            worst_ratio = min(worst_ratio, float((bound / omax).min()))
        a = rng.integers(0, T + 1, B)
        s.accept(a)
        mag.commit(a[seq], alpha, k, U)
    return worst_ratio


@pytest.mark.parametrize("expanded", [False, True])
def test_nonnegative_terms_give_the_output_itself(expanded):
    _drive("mamba2", nonneg=True, expanded=expanded)


@pytest.mark.parametrize("expanded", [False, True])
@pytest.mark.parametrize("kind", ["mamba2", "gdn"])
def test_bound_never_below_output(kind, expanded):
    assert _drive(kind, nonneg=False, expanded=expanded) >= 1.0 - 1e-12


def test_expanded_form_is_the_larger():
    """sum_n |k_n x_n| >= |k . x|: the expanded denominators are never below the others."""
    a = _drive("gdn", nonneg=False, expanded=False, seed=9)
    b = _drive("gdn", nonneg=False, expanded=True, seed=9)
    assert b >= a
