"""The short causal convolution on the input side, in fp64 -- TEST INFRASTRUCTURE ONLY.

The plain definition over each sequence's whole committed history (no ring, no
window pointer): per channel c and token t,

    y_t[c] = act(bias[c] + sum_{j<W} w[c][j] x_{t-W+1+j}[c]),  x_s = 0 for s < 0,

act = SiLU (z * sigmoid(z)) or the identity. A step with T drafts computes each
draft's output as if the drafts before it had been appended; accepting a keeps the
first a of them in the history (the semantics of speculative decoding in
"ReplaySSM: Cache SSM Inputs, Not State", How it works).
"""
from __future__ import annotations

import numpy as np


def silu(z):
    z = np.asarray(z, np.float64)
    return z / (1.0 + np.exp(-z))


class ConvOracle:
    def __init__(self, B: int, D: int, W: int):
        self.B, self.D, self.W = B, D, W
        self.history = [np.zeros((0, D)) for _ in range(B)]  # committed inputs, oldest first
        self.pending = None

    def step(self, x, w, bias=None, act_silu=True, commit=False):
        """x [B, T, D]; w [D, W]; bias [D] or None -> y [B, T, D] (fp64)."""
        x = np.asarray(x, np.float64)
        w = np.asarray(w, np.float64)
        B, T, D = x.shape
        y = np.empty((B, T, D))
        for b in range(B):
            seq = np.concatenate([self.history[b], x[b]], axis=0)
            t0 = len(self.history[b])
            for i in range(T):
                t = t0 + i
                acc = np.zeros(D) if bias is None else np.asarray(bias, np.float64).copy()
                for j in range(self.W):
                    s = t - self.W + 1 + j
                    if s >= 0:
                        acc += w[:, j] * seq[s]
                y[b, i] = silu(acc) if act_silu else acc
        if commit:
            for b in range(B):
                self.history[b] = np.concatenate([self.history[b], x[b]], axis=0)
            self.pending = None
        else:
            self.pending = x
        return y

    def accept(self, a):
        for b in range(self.B):
            n = int(a[b])
            self.history[b] = np.concatenate([self.history[b], self.pending[b, :n]], axis=0)
        self.pending = None

    def window(self, b: int) -> np.ndarray:
        """The last W - 1 committed inputs of sequence b, zero-padded in front, oldest first."""
        h = self.history[b][-(self.W - 1):] if self.W > 1 else self.history[b][:0]
        pad = np.zeros((self.W - 1 - len(h), self.D))
        return np.concatenate([pad, h], axis=0)
