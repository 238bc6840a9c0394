"""Drives the oracle through a sequence of ReplaySSM calls -- TEST INFRASTRUCTURE ONLY.

For a chosen set of heads (all, or a sample of a full-size layer: heads are
independent, so any subset can be followed exactly) it keeps the eager state
after every committed token, the integer pointer model for every sequence, and
the value the checkpoint must hold: the committed state at the moment the
pointer model folds ("ReplaySSM: Cache SSM Inputs, Not State", How it works:
the checkpoint is the state at the last fold; its value is what the
recurrence gives after `folded` tokens).
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

from . import gdn_round, kda_round, mamba2_round
from .pointer_model import PointerModel


def select_heads(arr: np.ndarray, heads: Sequence[Tuple[int, int]]) -> np.ndarray:
    """[B, T, H, ...] -> [nh, T, ...] for the listed (b, h) pairs."""
    bs = np.array([b for b, _ in heads])
    hs = np.array([h for _, h in heads])
    return np.ascontiguousarray(arr[bs, :, hs])


class OracleSession:
    def __init__(self, kind: str, B: int, H: int, P: int, N: int, L: int, T_max: int,
                 S0_heads: np.ndarray, heads: Optional[Sequence[Tuple[int, int]]] = None,
                 precision: str = "f64"):
        self.kind, self.B, self.H, self.P, self.N = kind, B, H, P, N
        self.heads: List[Tuple[int, int]] = (
            [(b, h) for b in range(B) for h in range(H)] if heads is None else list(heads))
        self.seq_of_head = np.array([b for b, _ in self.heads], dtype=np.int64)
        self.precision = precision
        dt = np.float64 if precision == "f64" else np.float32
        assert S0_heads.shape == (len(self.heads), P, N)
        self.S = np.ascontiguousarray(S0_heads, dtype=dt).copy()
        self.ckpt = self.S.copy()
        self.pm = PointerModel(B, L, T_max)
        self.pending: Optional[Dict[str, np.ndarray]] = None

    # -- calls ---------------------------------------------------------------
    def append(self, alpha, k, v, beta=None) -> List[List[int]]:
        """Per-head draft inputs: alpha [nh,T], k [nh,T,N], v [nh,T,P], beta [nh,T]."""
        T = alpha.shape[1]
        slots = self.pm.append(T)
        new = {"alpha": np.asarray(alpha, np.float32), "k": np.asarray(k, np.float32),
               "v": np.asarray(v, np.float32)}
        if self.kind in ("gdn", "kda"):
            new["beta"] = np.asarray(beta, np.float32)
        if self.pending is None:
            self.pending = new
        else:  # several appends before one verify
            self.pending = {key: np.concatenate([self.pending[key], new[key]], axis=1) for key in new}
        return slots

    def _round(self, q, acc_heads):
        pd = self.pending
        if self.kind == "mamba2":
            return mamba2_round(self.S, pd["alpha"], pd["k"], pd["v"], q, acc_heads, self.precision), None
        if self.kind == "kda":
            return kda_round(self.S, pd["alpha"], pd["beta"], pd["k"], pd["v"], q, acc_heads, self.precision)
        return gdn_round(self.S, pd["alpha"], pd["beta"], pd["k"], pd["v"], q, acc_heads, self.precision)

    def _take_checkpoint(self, folds: Sequence[bool]) -> None:
        sel = np.array([folds[b] for b in self.seq_of_head], dtype=bool)
        self.ckpt[sel] = self.S[sel]

    def verify(self, q):
        """q [nh,T,N] -> out [nh,T,P] (and u [nh,T,P] for GDN). The state is not advanced."""
        T = self.pending["alpha"].shape[1]
        folds = self.pm.verify(T)
        self._take_checkpoint(folds)
        out, u = self._round(np.asarray(q, np.float32), np.zeros(len(self.heads), np.int32))
        return out, u, folds

    def accept(self, a_seq) -> None:
        acc = np.asarray(a_seq, np.int32)[self.seq_of_head]
        T = self.pending["alpha"].shape[1]
        if np.any(acc > 0):
            dummy_q = np.zeros((len(self.heads), T, self.N), np.float32)
            self._round(dummy_q, acc)
        self.pm.accept(a_seq)
        self.pending = None

    def decode(self, q):
        """Standard step: verify(1) + accept(1) in one pass of the recurrence."""
        folds = self.pm.verify(1)
        self._take_checkpoint(folds)
        out, u = self._round(np.asarray(q, np.float32), np.ones(len(self.heads), np.int32))
        self.pm.accept([1] * self.B)
        self.pending = None
        return out, u, folds

    def flush(self) -> List[bool]:
        folds = self.pm.flush()
        self._take_checkpoint(folds)
        return folds
