"""Integer model of the ReplaySSM buffer pointers -- TEST INFRASTRUCTURE ONLY.

Per sequence b:
  head    ring slot of the oldest committed record that is not folded yet
  h       number of committed, not yet folded records
  p       number of pending (appended, not yet accepted) draft records
  folded  number of tokens folded into the checkpoint

Rules, from "ReplaySSM: Cache SSM Inputs, Not State" (How it works: Speculative
decoding, and the flowchart under it):
  append(T)  the T draft records go to ring slots (head + h + p + i) mod C,
             C = L + T_max (the buffer is circular with capacity L + T); p += T
  verify(T)  if h + T > L the committed records are folded into the checkpoint
             first (head += h mod C, folded += h, h = 0): the flush takes only
             already-committed records, so it can run before acceptance is known
  accept(a)  the accepted prefix only advances the pointer: h += a, p = 0;
             rejected records stay in their slots until the next append
             overwrites them
  decode     standard decoding is verify(1) followed by accept(1); it folds
             exactly L records every L tokens (one checkpoint write per window,
             "How it works": Standard decoding)
  flush      unconditional fold of the committed records

The model keeps T_max <= L, which bounds h by L and so keeps h + p <= C.
Plain Python integers, no vectorisation: it is meant to be read.
"""
from __future__ import annotations

from typing import List


class ContractError(ValueError):
    pass


class PointerModel:
    def __init__(self, B: int, L: int, T_max: int):
        if not (1 <= T_max <= L):
            raise ContractError("need 1 <= T_max <= L")
        self.B, self.L, self.T_max = B, L, T_max
        self.C = L + T_max
        self.head: List[int] = [0] * B
        self.h: List[int] = [0] * B
        self.p: List[int] = [0] * B
        self.folded: List[int] = [0] * B
        self.n_folds: List[int] = [0] * B

    def append(self, T: int) -> List[List[int]]:
        """Slots the T new records go to, per sequence."""
        if not (1 <= T <= self.T_max):
            raise ContractError("bad T")
        slots = []
        for b in range(self.B):
            if self.p[b] + T > self.T_max:
                raise ContractError(f"append overflow at b={b}")
            slots.append([(self.head[b] + self.h[b] + self.p[b] + i) % self.C for i in range(T)])
            self.p[b] += T
        return slots

    def _fold(self, b: int) -> None:
        self.head[b] = (self.head[b] + self.h[b]) % self.C
        self.folded[b] += self.h[b]
        self.h[b] = 0
        self.n_folds[b] += 1

    def verify(self, T: int) -> List[bool]:
        """Returns, per sequence, whether this call folds the committed records."""
        folds = []
        for b in range(self.B):
            if self.p[b] != T:
                raise ContractError(f"verify({T}) with p={self.p[b]} at b={b}")
            f = self.h[b] + T > self.L
            if f:
                self._fold(b)
            folds.append(f)
        return folds

    def accept(self, a) -> None:
        for b in range(self.B):
            ab = int(a[b])
            if not (0 <= ab <= self.p[b]):
                raise ContractError(f"accept {ab} > pending {self.p[b]} at b={b}")
            self.h[b] += ab
            self.p[b] = 0

    def decode(self) -> List[bool]:
        folds = self.verify(1)
        self.accept([1] * self.B)
        return folds

    def flush(self) -> List[bool]:
        folds = []
        for b in range(self.B):
            f = self.h[b] > 0
            if f:
                self._fold(b)
            folds.append(f)
        return folds

    def committed_slots(self, b: int) -> List[int]:
        return [(self.head[b] + i) % self.C for i in range(self.h[b])]

    def snapshot(self):
        return {"head": list(self.head), "h": list(self.h), "p": list(self.p),
                "folded": list(self.folded)}
