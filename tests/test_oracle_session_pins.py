"""Pins of the oracle's session logic (oracle/session.py) on the CPU.

OracleSession is what every speculative GPU parity test compares against: it
keeps the committed state, takes the checkpoint when the pointer rules fold, and
turns appends, verifies and accepts into rounds of the eager recurrence
("ReplaySSM: Cache SSM Inputs, Not State", How it works: Speculative decoding
and the flowchart under it). These tests drive it with random rounds and check
every result against a reference built a different way:

- the test keeps its own history of committed tokens per head and its own count
  of committed, unfolded records (a fold happens when h + T > L, or on flush);
- the state after n committed tokens is formed without any recurrence for
  Mamba-2 (the unrolled sum Gamma S_0 + sum_j gamma_j v_j k_j^T, with the
  decays as explicit products) and, for the delta rules, as a product of the
  explicit transition matrices Diag(a)(I - beta k k^T) (GDN: alpha I in place of
  Diag(a)) plus the written outer products;
- a draft's output is that state, extended by the drafts up to it, times q;
- the checkpoint must equal the state after the first `folded` committed tokens.

So a checkpoint taken after the round instead of before it, an accepted prefix
taken from the wrong row, a lost or doubled draft when several appends precede
one verify, or a rejected draft leaking into the state fails here.
"""
import numpy as np
import pytest

import oracle
from oracle.session import OracleSession

P, N = 5, 6


def _inputs(rng, kind, nh, T, unit_alpha=False):
    k = rng.standard_normal((nh, T, N)).astype(np.float32)
    if kind != "mamba2":
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    if kind == "kda":
        alpha = rng.uniform(0.4, 1.0, (nh, T, N)).astype(np.float32)
    else:
        alpha = rng.uniform(0.4, 1.0, (nh, T)).astype(np.float32)
    if unit_alpha:
        alpha = np.ones_like(alpha)
    return dict(
        alpha=alpha,
        k=k,
        v=rng.standard_normal((nh, T, P)).astype(np.float32),
        q=rng.standard_normal((nh, T, N)).astype(np.float32),
        beta=rng.uniform(0.1, 1.0, (nh, T)).astype(np.float32) if kind != "mamba2" else None,
    )


def _token(d, hd, t):
    """Record t of head hd as float64 arrays."""
    tok = {f: np.asarray(d[f][hd, t], np.float64) for f in ("alpha", "k", "v", "q")}
    tok["beta"] = float(d["beta"][hd, t]) if d["beta"] is not None else None
    return tok


def _state_after(kind, S0, toks):
    """Reference state after the tokens `toks`, in the forms described above."""
    S0 = np.asarray(S0, np.float64)
    if kind == "mamba2":
        n = len(toks)
        al = np.array([float(t["alpha"]) for t in toks])
        S = np.prod(al) * S0
        for j, t in enumerate(toks):
            S = S + np.prod(al[j + 1:]) * np.outer(t["v"], t["k"])  # empty product = 1
        return S if n else S0.copy()
    S = S0.copy()
    for t in toks:
        gate = np.diag(t["alpha"]) if kind == "kda" else float(t["alpha"]) * np.eye(N)
        M = gate @ (np.eye(N) - t["beta"] * np.outer(t["k"], t["k"]))
        S = S @ M + t["beta"] * np.outer(t["v"], t["k"])
    return S


def _u_of(kind, S_prev, t):
    """The stored correction of a delta-rule token: u = beta (v - S_{t-1} (gate k))."""
    gk = t["alpha"] * t["k"] if kind == "kda" else float(t["alpha"]) * t["k"]
    return t["beta"] * (t["v"] - S_prev @ gk)


class Tracker:
    """The test's own model of one session: committed history and pointer counts."""

    def __init__(self, kind, S0, B, H, L):
        self.kind, self.S0, self.B, self.H, self.L = kind, S0, B, H, L
        self.hist = [[] for _ in range(B * H)]
        self.h = [0] * B
        self.folded = [0] * B

    def state(self, hd, n=None):
        toks = self.hist[hd] if n is None else self.hist[hd][:n]
        return _state_after(self.kind, self.S0[hd], toks)

    def fold_if(self, T):
        folds = []
        for b in range(self.B):
            f = self.h[b] + T > self.L if T > 0 else self.h[b] > 0
            if f:
                self.folded[b] += self.h[b]
                self.h[b] = 0
            folds.append(f)
        return folds

    def round_outputs(self, d):
        """Outputs (and corrections) of every draft of every head from the committed state."""
        nh, T = d["q"].shape[:2]
        out = np.zeros((nh, T, P))
        u = np.zeros((nh, T, P))
        for hd in range(nh):
            base = list(self.hist[hd])
            for i in range(T):
                toks = base + [_token(d, hd, j) for j in range(i + 1)]
                if self.kind != "mamba2":
                    u[hd, i] = _u_of(self.kind, _state_after(self.kind, self.S0[hd], toks[:-1]), toks[-1])
                out[hd, i] = _state_after(self.kind, self.S0[hd], toks) @ toks[-1]["q"]
        return out, u

    def accept(self, d, a_seq):
        nh = d["q"].shape[0]
        for hd in range(nh):
            b = hd // self.H
            self.hist[hd] += [_token(d, hd, j) for j in range(int(a_seq[b]))]
        for b in range(self.B):
            self.h[b] += int(a_seq[b])

    def check_session(self, s):
        nh = self.B * self.H
        for hd in range(nh):
            b = hd // self.H
            np.testing.assert_allclose(s.S[hd], self.state(hd), rtol=1e-10, atol=1e-10)
            np.testing.assert_allclose(s.ckpt[hd], self.state(hd, self.folded[b]), rtol=1e-10, atol=1e-10)
        assert s.pm.h == self.h
        assert s.pm.folded == self.folded


def _session(kind, B, H, L, T_max, rng):
    S0 = rng.standard_normal((B * H, P, N)).astype(np.float32)
    return OracleSession(kind, B, H, P, N, L, T_max, S0), Tracker(kind, S0, B, H, L)


def _append(s, d, split=None):
    """One append of all drafts, or two appends split at `split`."""
    args = lambda sl: (d["alpha"][:, sl], d["k"][:, sl], d["v"][:, sl], None if d["beta"] is None else d["beta"][:, sl])
    if split is None:
        return s.append(*args(slice(None)))
    first = s.append(*args(slice(0, split)))
    second = s.append(*args(slice(split, None)))
    return [a + b for a, b in zip(first, second)]


KINDS = ["mamba2", "gdn", "kda"]


@pytest.mark.parametrize("kind", KINDS)
def test_speculative_rounds_match_history_reference(kind):
    """Random T, random accepted prefixes (0..T, 0 included), some rounds appended in two parts."""
    rng = np.random.default_rng(11)
    B, H, L, T_max = 3, 2, 5, 4
    s, ref = _session(kind, B, H, L, T_max, rng)
    for rnd in range(24):
        T = int(rng.integers(1, T_max + 1))
        d = _inputs(rng, kind, B * H, T)
        split = int(rng.integers(1, T)) if (T > 1 and rnd % 3 == 0) else None
        _append(s, d, split)
        out, u, folds = s.verify(d["q"])
        assert folds == ref.fold_if(T)
        # the checkpoint is the committed state at the fold, i.e. before this round's drafts
        ref.check_session(s)
        exp_out, exp_u = ref.round_outputs(d)
        np.testing.assert_allclose(out, exp_out, rtol=1e-10, atol=1e-10)
        if kind != "mamba2":
            np.testing.assert_allclose(u, exp_u, rtol=1e-10, atol=1e-10)
        a_seq = rng.integers(0, T + 1, B)
        s.accept(a_seq)
        ref.accept(d, a_seq)
        ref.check_session(s)
        if rnd % 7 == 6:
            assert s.flush() == ref.fold_if(0)
            ref.check_session(s)


@pytest.mark.parametrize("kind", KINDS)
def test_standard_decode_matches_history_reference(kind):
    """decode = verify(1) + accept(1): outputs, state and the checkpoint at every fold."""
    rng = np.random.default_rng(12)
    B, H, L = 2, 2, 4
    s, ref = _session(kind, B, H, L, 1, rng)
    for step in range(14):
        d = _inputs(rng, kind, B * H, 1)
        s.append(d["alpha"], d["k"], d["v"], d["beta"])
        out, u, folds = s.decode(d["q"])
        assert folds == ref.fold_if(1)
        exp_out, exp_u = ref.round_outputs(d)
        np.testing.assert_allclose(out, exp_out, rtol=1e-10, atol=1e-10)
        if kind != "mamba2":
            np.testing.assert_allclose(u, exp_u, rtol=1e-10, atol=1e-10)
        ref.accept(d, [1] * B)
        ref.check_session(s)
    assert s.pm.folded == [12, 12] and s.pm.h == [2, 2]


@pytest.mark.parametrize("decode", [True, False])
def test_checkpoint_at_every_fold_is_sum_of_committed_outer_products(decode):
    """alpha = 1: after every fold the checkpoint is S_0 + V^T K over the first `folded`
    committed records, formed as one matmul of the stacked records."""
    rng = np.random.default_rng(13)
    B, H, L, T_max = 2, 2, 6, 4
    S0 = rng.standard_normal((B * H, P, N)).astype(np.float32)
    s = OracleSession("mamba2", B, H, P, N, L, T_max if not decode else 1, S0)
    V = [[] for _ in range(B * H)]
    K = [[] for _ in range(B * H)]
    n_checked = 0
    for rnd in range(30):
        T = 1 if decode else int(rng.integers(1, T_max + 1))
        d = _inputs(rng, "mamba2", B * H, T, unit_alpha=True)
        s.append(d["alpha"], d["k"], d["v"])
        if decode:
            _, _, folds = s.decode(d["q"])
            a_seq = [1] * B
        else:
            _, _, folds = s.verify(d["q"])
        for hd in range(B * H):
            b = hd // H
            if folds[b]:
                n = s.pm.folded[b]
                Vm = np.array(V[hd][:n], np.float64).reshape(n, P)
                Km = np.array(K[hd][:n], np.float64).reshape(n, N)
                np.testing.assert_allclose(s.ckpt[hd], S0[hd].astype(np.float64) + Vm.T @ Km, rtol=1e-12, atol=1e-12)
                n_checked += 1
        if not decode:
            a_seq = rng.integers(0, T + 1, B)
            s.accept(a_seq)
        for hd in range(B * H):
            a = int(a_seq[hd // H])
            V[hd] += list(d["v"][hd, :a])
            K[hd] += list(d["k"][hd, :a])
    assert n_checked >= 8


@pytest.mark.parametrize("kind", KINDS)
def test_two_appends_equal_one_append(kind):
    """Appending T1 then T2 drafts before one verify is appending the T1 + T2 drafts at once."""
    rng = np.random.default_rng(14)
    B, H, L, T_max = 2, 3, 8, 6
    S0 = rng.standard_normal((B * H, P, N)).astype(np.float32)
    s1 = OracleSession(kind, B, H, P, N, L, T_max, S0)
    s2 = OracleSession(kind, B, H, P, N, L, T_max, S0)
    for rnd in range(6):
        T = int(rng.integers(2, T_max + 1))
        d = _inputs(rng, kind, B * H, T)
        slots1 = _append(s1, d, split=int(rng.integers(1, T)))
        slots2 = _append(s2, d)
        assert slots1 == slots2
        o1, u1, f1 = s1.verify(d["q"])
        o2, u2, f2 = s2.verify(d["q"])
        assert f1 == f2
        np.testing.assert_array_equal(o1, o2)
        if kind != "mamba2":
            np.testing.assert_array_equal(u1, u2)
        a_seq = rng.integers(0, T + 1, B)
        s1.accept(a_seq)
        s2.accept(a_seq)
        np.testing.assert_array_equal(s1.S, s2.S)
        np.testing.assert_array_equal(s1.ckpt, s2.ckpt)
        assert s1.pm.snapshot() == s2.pm.snapshot()


@pytest.mark.parametrize("kind", KINDS)
def test_rejected_round_leaves_no_trace(kind):
    """A round accepted with a = 0 and then re-appended gives the outputs and state of a
    session that never saw the rejected drafts (the checkpoint may be taken earlier, at
    the same committed position)."""
    rng = np.random.default_rng(15)
    B, H, L, T_max = 2, 2, 6, 4
    S0 = rng.standard_normal((B * H, P, N)).astype(np.float32)
    sa = OracleSession(kind, B, H, P, N, L, T_max, S0)
    sb = OracleSession(kind, B, H, P, N, L, T_max, S0)
    for rnd in range(10):
        T = int(rng.integers(1, T_max + 1))
        if rnd % 2 == 0:
            junk = _inputs(rng, kind, B * H, T)
            _append(sa, junk)
            sa.verify(junk["q"])
            sa.accept(np.zeros(B, np.int64))
            np.testing.assert_array_equal(sa.S, sb.S)
        d = _inputs(rng, kind, B * H, T)
        _append(sa, d)
        _append(sb, d)
        oa, ua, _ = sa.verify(d["q"])
        ob, ub, _ = sb.verify(d["q"])
        np.testing.assert_array_equal(oa, ob)
        if kind != "mamba2":
            np.testing.assert_array_equal(ua, ub)
        a_seq = rng.integers(0, T + 1, B)
        sa.accept(a_seq)
        sb.accept(a_seq)
        np.testing.assert_array_equal(sa.S, sb.S)
        assert sa.pm.h[0] + sa.pm.folded[0] == sb.pm.h[0] + sb.pm.folded[0]
        for b in range(B):
            if sa.pm.folded[b] == sb.pm.folded[b]:
                np.testing.assert_array_equal(sa.ckpt[b * H:(b + 1) * H], sb.ckpt[b * H:(b + 1) * H])


@pytest.mark.parametrize("kind", KINDS)
def test_accepted_prefix_equals_token_by_token_decoding(kind):
    """The committed state and the accepted drafts' outputs of speculative rounds equal a
    second session that decodes only the accepted tokens, one per step."""
    rng = np.random.default_rng(16)
    B, H, L, T_max = 1, 3, 5, 4
    S0 = rng.standard_normal((B * H, P, N)).astype(np.float32)
    spec = OracleSession(kind, B, H, P, N, L, T_max, S0)
    std = OracleSession(kind, B, H, P, N, L, 1, S0)
    for rnd in range(12):
        T = int(rng.integers(1, T_max + 1))
        d = _inputs(rng, kind, B * H, T)
        _append(spec, d)
        out, u, _ = spec.verify(d["q"])
        a = int(rng.integers(0, T + 1))
        spec.accept([a])
        for i in range(a):
            sl = slice(i, i + 1)
            std.append(d["alpha"][:, sl], d["k"][:, sl], d["v"][:, sl], None if d["beta"] is None else d["beta"][:, sl])
            o1, u1, _ = std.decode(d["q"][:, sl])
            np.testing.assert_allclose(o1[:, 0], out[:, i], rtol=1e-12, atol=1e-12)
            if kind != "mamba2":
                np.testing.assert_allclose(u1[:, 0], u[:, i], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(spec.S, std.S, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("kind", ["gdn", "kda"])
def test_fp32_delta_rule_oracle_close_to_fp64(kind):
    """The float forms of the delta-rule oracles stay within float rounding of the double
    forms (which the closed-form pins fix) over 64 tokens of the workloads' distributions:
    keys and queries L2-normalised, beta = sigmoid(N(0,1)), gates exp(-softplus(N(0,1)))."""
    rng = np.random.default_rng(17)
    nh, T, Pd, Nd = 6, 64, 32, 32
    k = rng.standard_normal((nh, T, Nd))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    q = rng.standard_normal((nh, T, Nd))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    gshape = (nh, T, Nd) if kind == "kda" else (nh, T)
    alpha = np.exp(-np.logaddexp(0.0, rng.standard_normal(gshape)))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((nh, T))))
    v = rng.standard_normal((nh, T, Pd))
    S0 = 0.1 * rng.standard_normal((nh, Pd, Nd))
    args = [a.astype(np.float32) for a in (alpha, beta, k, v, q)]
    fn = oracle.kda_round if kind == "kda" else oracle.gdn_round
    acc = np.full(nh, T, np.int32)
    S64 = S0.astype(np.float32).astype(np.float64)
    S32 = S0.astype(np.float32)
    o64, u64 = fn(S64, *args, acc, "f64")
    o32, u32 = fn(S32, *args, acc, "f32")
    assert o32.dtype == np.float32 and not np.array_equal(o32.astype(np.float64), o64)
    rel = np.abs(o32 - o64).max(axis=-1) / np.abs(o64).max(axis=-1)
    relu = np.abs(u32 - u64).max(axis=-1) / np.abs(u64).max(axis=-1)
    relS = np.abs(S32 - S64).max(axis=(1, 2)) / np.abs(S64).max(axis=(1, 2))
    assert rel.max() < 2e-5 and relu.max() < 2e-5 and relS.max() < 2e-5, (rel.max(), relu.max(), relS.max())
