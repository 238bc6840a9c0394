"""Lock-step runner of the GPU path (through the C ABI) and the CPU oracle.

The GPU runs the whole layer; the oracle follows every head, or a sample of
heads of a full-size layer (heads are independent, so a sample is followed
exactly). Inputs come from synth/ (host numpy for small cases, torch on the GPU
for full-size ones, in which case the sampled heads' slices are copied back),
so both sides see identical numbers.

Error metric, per output vector o (one draft of one head):
    rel = max|o_gpu - o_ref| / max(max|o_ref|, 1e-30)
and a run reports the maximum over all compared vectors. When whole sequences
are followed, the same metric is also taken per (sequence, draft) over the
token's whole layer output (all heads).

With a checkpoint copy read in bf16, each head's output is also measured against
the magnitudes of the terms it sums ("How it works": Standard decoding, the
output is the decayed checkpoint times q plus the buffered records' sum;
Two precisions):
    mag = max|o_gpu - o_ref| / max_p (Gamma_t sum_n |S_ck[p,n] q_t[n]|
                                      + sum_j gamma_{j,t} |v_j[p]| |k_j . q_t|)
with S_ck the oracle's checkpoint (its state at position `folded`), j over the
records since that position up to draft t, and for the delta rule the magnitude
of each correction's own terms in place of |v_j| (class Magnitudes). The bf16
rounding of the checkpoint changes each term by at most 2^-8 of its magnitude,
so this ratio stays bounded where terms cancel and the plain ratio above does
not. For the fp32 checkpoint the dot products are taken as sum_n |k[n] q[n]|
(what bounds an fp32 dot product's rounding) and the guarded ratio
    err / max(max|o_ref|, 1e-2 * mag)
is the plain metric except on outputs more than 100 times smaller than their
terms.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np
import torch

import ssm_decode_amd as rs
from oracle.session import OracleSession
from synth import LayerShape, device_accept, device_initial_state, device_step, host_accept, host_initial_state, host_step


def rel_err(gpu: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """Normwise relative error over the last axis."""
    num = np.abs(gpu.astype(np.float64) - ref.astype(np.float64)).max(axis=-1)
    den = np.maximum(np.abs(ref).max(axis=-1), 1e-30)
    return num / den


@dataclass
class Report:
    max_rel: float = 0.0
    max_rel_token: float = 0.0  # per (sequence, draft): the layer output over every followed head
    max_rel_u: float = 0.0
    max_rel_ckpt: float = 0.0
    max_rel_mag: float = 0.0  # per head, against the term magnitudes (when they are formed)
    mag_vectors: int = 0  # vectors measured against the term magnitudes
    # per head, err / max(max|o_ref|, 1e-2 * term magnitude): the plain metric unless the output
    # is more than 100 times smaller than the terms it sums
    max_rel_guarded: float = 0.0
    # the vector with the largest plain per-head error: that error, its error against the term
    # magnitudes, and its cancellation factor (term magnitude / max|o_ref|)
    worst_rel_vector: Optional[dict] = None
    rels: List[float] = field(default_factory=list)
    # every compared vector's figures, kept when a drift summary is asked for
    all_rel: List[np.ndarray] = field(default_factory=list)
    all_token: List[np.ndarray] = field(default_factory=list)
    all_mag: List[np.ndarray] = field(default_factory=list)
    pointer_mismatch: int = 0
    ring_mismatch: int = 0
    folds: int = 0
    calls: int = 0
    err_word: int = 0
    final_pointers: Optional[dict] = None
    oracle_pointers: Optional[dict] = None

    def update(self, r: np.ndarray) -> None:
        if r.size:
            self.max_rel = max(self.max_rel, float(r.max()))
            self.rels.append(float(np.percentile(r, 99.9)))

    def update_token(self, r: np.ndarray) -> None:
        if r.size:
            self.max_rel_token = max(self.max_rel_token, float(r.max()))

    def update_mag(self, r: np.ndarray) -> None:
        if r.size:
            self.max_rel_mag = max(self.max_rel_mag, float(r.max()))
            self.mag_vectors += int(r.size)

    def drift_summary(self) -> dict:
        """Max and 99.9th percentile of every kept figure."""
        out = {}
        for name, xs in (("per_head", self.all_rel), ("per_token", self.all_token), ("per_head_magnitude", self.all_mag)):
            if xs:
                x = np.concatenate([a.ravel() for a in xs])
                out[name] = {"max": float(x.max()), "p99_9": float(np.percentile(x, 99.9)), "vectors": int(x.size)}
        if self.worst_rel_vector is not None:
            out["worst_per_head_vector"] = self.worst_rel_vector
        return out


class Magnitudes:
    """Per followed head, the records since its checkpoint position, to form the magnitude
    denominator of each output: committed records since the last fold, then the drafts.

    Each record keeps U_j, the magnitude of the value vector it carries: |v_j| for Mamba-2;
    for the delta rule the magnitude of the terms of its correction
        U_j = beta_j |v_j| + beta_j alpha_j (Gamma_{j-1} sum_n |S_ck[p,n] k_j[n]|
                                             + sum_{i<j} gamma_{i,j-1} U_i |k_i . k_j|),
    the bound that |u_j| and its bf16-read error obey (the rebuilt S_{j-1} k_j; "How it
    works": Gated DeltaNet)."""

    def __init__(self, nh: int, C: int, P: int, N: int, expanded: bool = False):
        # expanded: every dot product k . x taken as sum_n |k[n] x[n]| (the size of what a
        # floating-point dot product sums, which bounds its rounding error), else as |k . x|
        self.expanded = expanded
        self.n = np.zeros(nh, np.int64)
        self.a = np.ones((nh, C))
        self.k = np.zeros((nh, C, N))
        self.U = np.zeros((nh, C, P))

    def fold(self, folded_heads: np.ndarray) -> None:
        self.n[folded_heads] = 0
        self.a[folded_heads] = 1.0
        self.k[folded_heads] = 0.0
        self.U[folded_heads] = 0.0

    def _terms(self, Sx, A, K, U, live_end, x):
        """Magnitude vectors [nh, P] of S_{end} x from the checkpoint and records 0..end, with
        Sx = sum_n |S_ck[p,n] x[n]| given."""
        pos = np.arange(A.shape[1])
        live = pos[None, :] <= live_end[:, None]
        Ai = np.where(live, A, 1.0)
        # suffix products: rev[j] = prod of alpha over records j..end; gamma_j = rev[j + 1]
        rev = np.flip(np.cumprod(np.flip(Ai, axis=1), axis=1), axis=1)
        gam = np.concatenate([rev[:, 1:], np.ones_like(rev[:, :1])], axis=1)
        t1 = rev[:, 0][:, None] * Sx
        if self.expanded:
            kx = np.matmul(np.abs(K), np.abs(x)[:, :, None])[:, :, 0]
        else:
            kx = np.abs(np.matmul(K, x[:, :, None])[:, :, 0])
        t2 = np.einsum("hj,hjp->hp", np.where(live, gam * kx, 0.0), U)
        # an empty record set (end = -1) leaves the checkpoint term with Gamma = 1
        return t1 + t2

    def bounds(self, ckpt, alpha, k, v, q, beta=None):
        """[nh, T] denominators for drafts with inputs alpha, k, v (raw), beta (delta rule), q;
        also the drafts' U [nh, T, P] for the accept that follows."""
        nh, T = q.shape[:2]
        R = int(self.n.max()) + T
        A, K, U = self.a[:, :R].copy(), self.k[:, :R].copy(), self.U[:, :R].copy()
        rows = np.arange(nh)
        absS = np.abs(ckpt)
        q = q.astype(np.float64)
        # sum_n |S_ck[p,n] x[n]| for every draft's q (and k), one batched product each
        Sq = np.matmul(absS, np.abs(q).transpose(0, 2, 1)).transpose(0, 2, 1)
        Sk = None if beta is None else np.matmul(absS, np.abs(k.astype(np.float64)).transpose(0, 2, 1)).transpose(0, 2, 1)
        Ud = np.empty((nh, T, v.shape[-1]))
        out = np.empty((nh, T))
        for i in range(T):
            A[rows, self.n + i] = alpha[:, i]
            K[rows, self.n + i] = k[:, i]
            if beta is None:
                Ud[:, i] = np.abs(v[:, i])
            else:  # the correction's terms, from the state before draft i (records up to n + i - 1)
                W = self._terms(Sk[:, i], A, K, U, self.n + i - 1, k[:, i].astype(np.float64))
                b = np.asarray(beta[:, i], np.float64)[:, None]
                Ud[:, i] = b * (np.abs(v[:, i]) + np.asarray(alpha[:, i], np.float64)[:, None] * W)
            U[rows, self.n + i] = Ud[:, i]
            out[:, i] = self._terms(Sq[:, i], A, K, U, self.n + i, q[:, i]).max(axis=1)
        return out, Ud

    def commit(self, acc: np.ndarray, alpha, k, U) -> None:
        rows = np.arange(len(acc))
        for i in range(int(acc.max()) if acc.size else 0):
            m = acc > i
            r = rows[m]
            self.a[r, self.n[m]] = alpha[m, i]
            self.k[r, self.n[m]] = k[m, i]
            self.U[r, self.n[m]] = U[m, i]
            self.n[m] += 1


def whole_sequences(B: int, H: int, seqs: Sequence[int]) -> List[Tuple[int, int]]:
    """Every head of the listed sequences (so that a token's whole layer output is followed)."""
    return [(b, h) for b in sorted(set(seqs)) if 0 <= b < B for h in range(H)]


def sample_heads(B: int, H: int, n: int, seed: int = 0) -> List[Tuple[int, int]]:
    if n >= B * H:
        return [(b, h) for b in range(B) for h in range(H)]
    rng = np.random.default_rng(seed + 17)
    idx = rng.choice(B * H, size=n, replace=False)
    # always include the first and last head of the layer
    idx = np.unique(np.concatenate([idx, [0, B * H - 1]]))
    return [(int(i) // H, int(i) % H) for i in idx]


class Runner:
    """One layer on the GPU plus the oracle on `heads`."""

    def __init__(self, shape: LayerShape, L: int, T_max: int, precision: str = "fp32", seed: int = 0,
                 wid: int = 99, heads: Optional[Sequence[Tuple[int, int]]] = None, gen: str = "host",
                 s0_sigma: float = 0.1, decay: str = "recipe", check_ring: bool = True,
                 keep_all: bool = False, magnitudes: Optional[bool] = None):
        self.shape, self.L, self.T_max, self.seed, self.wid = shape, L, T_max, seed, wid
        self.keep_all = keep_all
        self.gen, self.decay, self.check_ring = gen, decay, check_ring
        self.cfg = rs.make_config(shape.kind, precision, shape.B, shape.H, shape.P, shape.N, L, T_max)
        self.layer = rs.LayerState(self.cfg)
        self.heads = heads if heads is not None else sample_heads(shape.B, shape.H, shape.B * shape.H)
        self.bs = torch.tensor([b for b, _ in self.heads], device="cuda")
        self.hs = torch.tensor([h for _, h in self.heads], device="cuda")
        if gen == "host":
            S0 = torch.from_numpy(host_initial_state(seed, wid, shape, s0_sigma)).cuda()
        else:
            S0 = device_initial_state(seed, wid, shape, s0_sigma, "cuda")
        self.layer.import_state(S0)
        S0h = S0[self.bs, self.hs].cpu().numpy()
        self.oracle = OracleSession(shape.kind, shape.B, shape.H, shape.P, shape.N, L, T_max, S0h, self.heads)
        self.report = Report()
        self.step_id = 0
        # token metric only when whole sequences are followed, in (b, h) order
        seqs = sorted({b for b, _ in self.heads})
        self.token_groups = (len(self.heads) == len(seqs) * shape.H and
                             self.heads == [(b, h) for b in seqs for h in range(shape.H)])
        # magnitude bounds of the outputs whenever a bf16 checkpoint copy is read (or when asked)
        if magnitudes is None:
            magnitudes = precision != "fp32"
        self.mag = (Magnitudes(len(self.heads), L + T_max, shape.P, shape.N, expanded=precision == "fp32")
                    if magnitudes else None)
        self._mag_pending = None

    # -- inputs --------------------------------------------------------------
    def inputs(self, T: int) -> Dict[str, torch.Tensor]:
        sh = self.shape
        if self.gen == "host":
            x = host_step(self.seed, self.wid, self.step_id, sh, T, self.decay)
            out = {k: torch.from_numpy(v).cuda() for k, v in x.items()}
        else:
            out = device_step(self.seed, self.wid, self.step_id, sh, T, "cuda", self.decay)
        self.step_id += 1
        return out

    def _sel(self, t: torch.Tensor) -> np.ndarray:
        """[B, T, H, ...] device tensor -> [nh, T, ...] host array of the followed heads."""
        return t[self.bs, :, self.hs].cpu().numpy()

    # -- calls ---------------------------------------------------------------
    def append(self, x: Dict[str, torch.Tensor], T: int) -> None:
        beta = x.get("beta")
        rs.append(self.cfg, self.layer.struct, T, x["alpha"], x["k"], x["v"], beta)
        slots = self.oracle.append(self._sel(x["alpha"]), self._sel(x["k"]), self._sel(x["v"]),
                                   None if beta is None else self._sel(beta))
        self._slots = slots
        if self.check_ring:
            self._check_ring(x, slots, T)

    def step(self, x: Dict[str, torch.Tensor]) -> np.ndarray:
        """Fused append + decode (replayssm_decode_step); the oracle does append + decode."""
        sh = self.shape
        beta = x.get("beta")
        out = torch.empty((sh.B, 1, sh.H, sh.P), dtype=torch.float32, device="cuda")
        rs.decode_step(self.cfg, self.layer.struct, x["alpha"], x["k"], x["v"], beta, x["q"], out)
        slots = self.oracle.append(self._sel(x["alpha"]), self._sel(x["k"]), self._sel(x["v"]),
                                   None if beta is None else self._sel(beta))
        self._slots = slots
        if self.check_ring:
            self._check_ring(x, slots, 1, check_v=beta is None)
        pd = self.oracle.pending
        q = self._sel(x["q"])
        ref, u, folds = self.oracle.decode(q)
        got = self._sel(out)
        self._score(got, ref, self._bounds(pd, q, u, folds))
        self._commit_mag(np.ones(len(self.heads), np.int64))
        self.report.calls += 1
        self.report.folds += sum(folds)
        if u is not None:
            self._check_u(u, 1)
        return got

    def verify_step(self, x: Dict[str, torch.Tensor], T: int) -> np.ndarray:
        """Fused append + verify (replayssm_verify_step)."""
        sh = self.shape
        beta = x.get("beta")
        out = torch.empty((sh.B, T, sh.H, sh.P), dtype=torch.float32, device="cuda")
        rs.verify_step(self.cfg, self.layer.struct, T, x["alpha"], x["k"], x["v"], beta, x["q"], out)
        slots = self.oracle.append(self._sel(x["alpha"]), self._sel(x["k"]), self._sel(x["v"]),
                                   None if beta is None else self._sel(beta))
        self._slots = slots
        if self.check_ring:
            self._check_ring(x, slots, T, check_v=beta is None)
        pd = self.oracle.pending
        q = self._sel(x["q"])
        ref, u, folds = self.oracle.verify(q)
        got = self._sel(out)
        self._score(got, ref, self._bounds(pd, q, u, folds))
        self.report.calls += 1
        self.report.folds += sum(folds)
        if u is not None:
            self._check_u(u, T)
        return got

    # -- magnitude bounds (bf16-read modes) ------------------------------------
    def _bounds(self, pd, q, u, folds):
        """Denominators of the drafts' outputs; records the drafts for the accept that follows."""
        if self.mag is None:
            return None
        folded = np.array([folds[b] for b, _ in self.heads], dtype=bool)
        self.mag.fold(folded)
        bound, U = self.mag.bounds(self.oracle.ckpt, pd["alpha"], pd["k"], pd["v"], q, pd.get("beta"))
        self._mag_pending = (pd["alpha"], pd["k"], U)
        return bound

    def _commit_mag(self, acc_heads: np.ndarray) -> None:
        if self.mag is not None and self._mag_pending is not None:
            self.mag.commit(np.asarray(acc_heads, np.int64), *self._mag_pending)
            self._mag_pending = None

    def _check_ring(self, x, slots, T, check_v=True) -> None:
        # committed-record copies are bit-exact copies of the inputs (k and alpha always, v for Mamba-2
        # until the record is consumed, where GDN replaces it by u)
        sl = torch.tensor([[slots[b][i] for i in range(T)] for b, _ in self.heads], device="cuda")
        for i in range(T):
            ring_k = self.layer.ring_k[self.bs, self.hs, sl[:, i]]
            ring_a = self.layer.ring_alpha[self.bs, self.hs, sl[:, i]]
            ring_v = self.layer.ring_v[self.bs, self.hs, sl[:, i]]
            ok = torch.equal(ring_k, x["k"][self.bs, i, self.hs]) and torch.equal(ring_a, x["alpha"][self.bs, i, self.hs])
            if check_v:
                ok = ok and torch.equal(ring_v, x["v"][self.bs, i, self.hs])
            if "beta" in x:
                ok = ok and torch.equal(self.layer.ring_beta[self.bs, self.hs, sl[:, i]], x["beta"][self.bs, i, self.hs])
            if not ok:
                self.report.ring_mismatch += 1

    def decode(self, x: Dict[str, torch.Tensor]) -> np.ndarray:
        sh = self.shape
        out = torch.empty((sh.B, 1, sh.H, sh.P), dtype=torch.float32, device="cuda")
        rs.decode(self.cfg, self.layer.struct, x["q"], out)
        pd = self.oracle.pending
        q = self._sel(x["q"])
        ref, u, folds = self.oracle.decode(q)
        got = self._sel(out)
        self._score(got, ref, self._bounds(pd, q, u, folds))
        self._commit_mag(np.ones(len(self.heads), np.int64))
        self.report.calls += 1
        self.report.folds += sum(folds)
        if u is not None:
            self._check_u(u, 1)
        return got

    def _score(self, got: np.ndarray, ref: np.ndarray, bound: Optional[np.ndarray] = None) -> None:
        rel = rel_err(got, ref)
        self.report.update(rel.ravel())
        if self.keep_all:
            self.report.all_rel.append(rel.astype(np.float32))
        if bound is not None:
            err = np.abs(got.astype(np.float64) - ref.astype(np.float64)).max(axis=-1)
            mag = err / np.maximum(bound, 1e-30)
            self.report.update_mag(mag.ravel())
            guard = err / np.maximum(np.maximum(np.abs(ref).max(axis=-1), 1e-2 * bound), 1e-30)
            self.report.max_rel_guarded = max(self.report.max_rel_guarded, float(guard.max()))
            if self.keep_all:
                self.report.all_mag.append(mag.astype(np.float32))
            i = int(np.argmax(rel))
            w = self.report.worst_rel_vector
            if rel.size and (w is None or float(rel.flat[i]) > w["rel"]):
                omax = float(np.abs(ref.reshape(-1, ref.shape[-1])[i]).max())
                self.report.worst_rel_vector = {"rel": float(rel.flat[i]), "rel_magnitude": float(mag.flat[i]),
                                                "cancellation": float(bound.flat[i]) / max(omax, 1e-30)}
        if self.token_groups:
            H, P = self.shape.H, self.shape.P
            T = got.shape[1]
            g = got.reshape(-1, H, T, P).transpose(0, 2, 1, 3).reshape(-1, T, H * P)
            r = ref.reshape(-1, H, T, P).transpose(0, 2, 1, 3).reshape(-1, T, H * P)
            tok = rel_err(g, r)
            self.report.update_token(tok.ravel())
            if self.keep_all:
                self.report.all_token.append(tok.astype(np.float32))

    def verify(self, x: Dict[str, torch.Tensor], T: int) -> np.ndarray:
        sh = self.shape
        out = torch.empty((sh.B, T, sh.H, sh.P), dtype=torch.float32, device="cuda")
        rs.verify(self.cfg, self.layer.struct, T, x["q"], out)
        pd = self.oracle.pending
        q = self._sel(x["q"])
        ref, u, folds = self.oracle.verify(q)
        got = self._sel(out)
        self._score(got, ref, self._bounds(pd, q, u, folds))
        self.report.calls += 1
        self.report.folds += sum(folds)
        if u is not None:
            self._check_u(u, T)
        return got

    def _check_u(self, u_ref: np.ndarray, T: int) -> None:
        """GDN: the drafts' corrections u were written in place of v, in the slots they were appended to."""
        sl = torch.tensor([[self._slots[b][i] for i in range(T)] for b, _ in self.heads], device="cuda")
        got = torch.stack([self.layer.ring_v[self.bs, self.hs, sl[:, i]] for i in range(T)], dim=1).cpu().numpy()
        self.report.max_rel_u = max(self.report.max_rel_u, float(rel_err(got, u_ref).max()))

    def accept(self, a: torch.Tensor) -> None:
        rs.accept(self.cfg, self.layer.struct, a)
        ah = a.cpu().numpy()
        self.oracle.accept(ah)
        self._commit_mag(ah[[b for b, _ in self.heads]])

    def flush(self) -> None:
        rs.flush(self.cfg, self.layer.struct)
        folds = self.oracle.flush()
        self.report.folds += sum(folds)
        if self.mag is not None:
            self.mag.fold(np.array([folds[b] for b, _ in self.heads], dtype=bool))

    # -- checks --------------------------------------------------------------
    def check_pointers(self) -> bool:
        got = self.layer.pointers()
        want = self.oracle.pm.snapshot()
        ok = got == want
        if not ok:
            self.report.pointer_mismatch += 1
        self.report.final_pointers, self.report.oracle_pointers = got, want
        return ok

    def check_checkpoint(self, which: str = "hp") -> float:
        """Relative error of the checkpoint vs the oracle's state at position `folded`, per row."""
        S = self.layer.export_state(which)[self.bs, self.hs].cpu().numpy()
        r = float(rel_err(S, self.oracle.ckpt).max())
        self.report.max_rel_ckpt = max(self.report.max_rel_ckpt, r)
        return r

    def error_word(self) -> int:
        self.report.err_word = rs.read_error(self.layer.struct)
        return self.report.err_word


def run_standard(runner: Runner, steps: int, check_every: int = 1, fused: bool = False) -> Report:
    for t in range(steps):
        x = runner.inputs(1)
        if fused:
            runner.step(x)
        else:
            runner.append(x, 1)
            runner.decode(x)
        if (t + 1) % check_every == 0 or t == steps - 1:
            runner.check_pointers()
    runner.check_checkpoint("hp" if runner.cfg.precision != rs.BF16_SHARED else "lp")
    runner.error_word()
    torch.cuda.synchronize()
    return runner.report


def run_spec(runner: Runner, T: int, rounds: int, check_every: int = 1, accept_mode: str = "uniform",
             fused: bool = False) -> Report:
    sh = runner.shape
    for rnd in range(rounds):
        x = runner.inputs(T)
        if fused:
            runner.verify_step(x, T)
        else:
            runner.append(x, T)
            runner.verify(x, T)
        if accept_mode == "all":
            a = torch.full((sh.B,), T, dtype=torch.int32, device="cuda")
        elif runner.gen == "host":
            a = torch.from_numpy(host_accept(runner.seed, runner.wid, rnd, sh.B, T)).cuda()
        else:
            a = device_accept(runner.seed, runner.wid, rnd, sh.B, T, "cuda")
        runner.accept(a)
        if (rnd + 1) % check_every == 0 or rnd == rounds - 1:
            runner.check_pointers()
    runner.check_checkpoint("hp" if runner.cfg.precision != rs.BF16_SHARED else "lp")
    runner.error_word()
    torch.cuda.synchronize()
    return runner.report
