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
token's whole layer output (all heads), the vector the bf16-read bar applies to.
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
    rels: List[float] = field(default_factory=list)
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
                 s0_sigma: float = 0.1, decay: str = "recipe", check_ring: bool = True):
        self.shape, self.L, self.T_max, self.seed, self.wid = shape, L, T_max, seed, wid
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
        ref, u, folds = self.oracle.decode(self._sel(x["q"]))
        got = self._sel(out)
        self._score(got, ref)
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
        ref, u, folds = self.oracle.verify(self._sel(x["q"]))
        got = self._sel(out)
        self._score(got, ref)
        self.report.calls += 1
        self.report.folds += sum(folds)
        if u is not None:
            self._check_u(u, T)
        return got

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
        ref, u, folds = self.oracle.decode(self._sel(x["q"]))
        got = self._sel(out)
        self._score(got, ref)
        self.report.calls += 1
        self.report.folds += sum(folds)
        if u is not None:
            self._check_u(u, 1)
        return got

    def _score(self, got: np.ndarray, ref: np.ndarray) -> None:
        self.report.update(rel_err(got, ref).ravel())
        if self.token_groups:
            H, P = self.shape.H, self.shape.P
            T = got.shape[1]
            g = got.reshape(-1, H, T, P).transpose(0, 2, 1, 3).reshape(-1, T, H * P)
            r = ref.reshape(-1, H, T, P).transpose(0, 2, 1, 3).reshape(-1, T, H * P)
            self.report.update_token(rel_err(g, r).ravel())

    def verify(self, x: Dict[str, torch.Tensor], T: int) -> np.ndarray:
        sh = self.shape
        out = torch.empty((sh.B, T, sh.H, sh.P), dtype=torch.float32, device="cuda")
        rs.verify(self.cfg, self.layer.struct, T, x["q"], out)
        ref, u, folds = self.oracle.verify(self._sel(x["q"]))
        got = self._sel(out)
        self._score(got, ref)
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
        self.oracle.accept(a.cpu().numpy())

    def flush(self) -> None:
        rs.flush(self.cfg, self.layer.struct)
        self.report.folds += sum(self.oracle.flush())

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
