"""Pins of the oracle's integer pointer model.

Standard decoding folds exactly L records at tokens L+1, 2L+1, ... (one
checkpoint write per window of L tokens), so after s steps the closed form is
n_folds = floor((s-1)/L), folded = L*n_folds, h = s - folded,
head = folded mod C with C = L + 1.
"""
import numpy as np
import pytest

from oracle.pointer_model import ContractError, PointerModel


@pytest.mark.parametrize("L,steps", [(4, 64), (16, 512), (1, 10), (3, 7), (16, 16)])
def test_standard_decode_closed_form(L, steps):
    pm = PointerModel(2, L, 1)
    for _ in range(steps):
        slots = pm.append(1)
        assert slots[0][0] == (pm.head[0] + pm.h[0]) % pm.C
        pm.decode()
    nf = (steps - 1) // L
    assert pm.n_folds[0] == nf
    assert pm.folded[0] == L * nf
    assert pm.h[0] == steps - L * nf
    assert pm.head[0] == (L * nf) % (L + 1)
    assert pm.p[0] == 0


def test_tiny_and_b256_workload_traces():
    """The two standard-decoding workloads: L=4 over 64 steps, L=16 over 512 steps."""
    pm = PointerModel(1, 4, 1)
    for _ in range(64):
        pm.append(1)
        pm.decode()
    assert (pm.n_folds[0], pm.folded[0], pm.h[0], pm.head[0]) == (15, 60, 4, 0)
    pm = PointerModel(1, 16, 1)
    for _ in range(512):
        pm.append(1)
        pm.decode()
    assert (pm.n_folds[0], pm.folded[0], pm.h[0], pm.head[0]) == (31, 496, 16, 3)


def test_hand_trace_speculative():
    """L=4, T=2, C=6, one sequence, accept 2, 1, 0, 2, 2: traced by hand."""
    pm = PointerModel(1, 4, 2)
    trace = []
    for a in [2, 1, 0, 2, 2]:
        s = pm.append(2)[0]
        f = pm.verify(2)[0]
        pm.accept([a])
        trace.append((s, f, pm.head[0], pm.h[0], pm.folded[0]))
    assert trace == [
        ([0, 1], False, 0, 2, 0),   # h=0: 0+2<=4, no fold; h=2
        ([2, 3], False, 0, 3, 0),   # h+T=4<=4; accept 1 -> h=3
        ([3, 4], True, 3, 0, 3),    # slots from head+h=3; 3+2>4 fold 3 -> head=3, folded=3; accept 0
        ([3, 4], False, 3, 2, 3),   # rejected slots 3,4 are overwritten; accept 2 -> h=2
        ([5, 0], False, 3, 4, 3),   # 2+2<=4; wraps around C=6; h=4
    ]


def test_speculative_invariants_random():
    rng = np.random.default_rng(7)
    B, L, T = 16, 16, 4
    pm = PointerModel(B, L, T)
    for _ in range(300):
        slots = pm.append(T)
        for b in range(B):
            committed = set(pm.committed_slots(b))
            assert committed.isdisjoint(slots[b])  # drafts never overwrite committed records
            assert len(set(slots[b])) == T
        folds = pm.verify(T)
        for b in range(B):
            assert pm.h[b] + T <= L  # after the route decision the drafts fit the window
            if folds[b]:
                assert pm.h[b] == 0
        a = rng.integers(0, T + 1, size=B)
        pm.accept(a)
        for b in range(B):
            assert pm.h[b] <= L and pm.p[b] == 0
            assert pm.folded[b] + pm.h[b] >= 0


def test_accept_all_equals_standard_decoding_with_T1():
    a = PointerModel(3, 5, 1)
    b = PointerModel(3, 5, 1)
    for _ in range(40):
        a.append(1)
        a.verify(1)
        a.accept([1, 1, 1])
        b.append(1)
        b.decode()
    assert a.snapshot() == b.snapshot()


def test_contract_errors():
    pm = PointerModel(1, 4, 2)
    pm.append(2)
    with pytest.raises(ContractError):
        pm.append(1)  # p + T > T_max
    with pytest.raises(ContractError):
        pm.verify(1)  # p != T
    pm.verify(2)
    with pytest.raises(ContractError):
        pm.accept([3])
    with pytest.raises(ContractError):
        PointerModel(1, 2, 3)  # T_max > L


def test_flush_folds_committed_only():
    pm = PointerModel(1, 8, 4)
    pm.append(4)
    pm.verify(4)
    pm.accept([3])
    pm.append(2)
    folds = pm.flush()
    assert folds == [True] and pm.folded[0] == 3 and pm.h[0] == 0 and pm.p[0] == 2 and pm.head[0] == 3
    assert pm.flush() == [False]
