"""Kimi Delta Attention heads (a gate per key channel) against the oracle.

The kernel carries the per-channel gate products on the staged keys and
queries instead of in per-record decay tables; these cases aim at that part:
gates that are exactly zero in some channels (no division anywhere, so the
result stays exact), open gates, the standard and speculative routes at the
layer's full size with sampled heads, and the fused calls.
Bar: outputs and the corrections u within 1e-4 relative of the fp64 oracle;
pointers and ring copies bit-exact.
"""
import pytest
import torch

from synth import LayerShape, WORKLOADS, host_accept

from harness import Runner, run_spec, run_standard, sample_heads

pytestmark = pytest.mark.gpu

TOL = 1e-4


def _clean(rep, tol=TOL):
    assert rep.pointer_mismatch == 0, (rep.final_pointers, rep.oracle_pointers)
    assert rep.ring_mismatch == 0
    assert rep.err_word == 0
    assert rep.max_rel <= tol, rep.max_rel
    assert rep.max_rel_ckpt <= tol, rep.max_rel_ckpt
    assert rep.max_rel_u <= tol, rep.max_rel_u


@pytest.mark.parametrize("P,N", [(128, 128), (64, 128), (32, 64), (16, 16), (256, 32)])
@pytest.mark.parametrize("L", [1, 4, 16])
def test_kda_standard_shapes(P, N, L):
    sh = LayerShape("kda", 2, 3, P, N)
    r = Runner(sh, L, 1, wid=300 + L, decay="slow")
    rep = run_standard(r, 2 * L + 5)
    _clean(rep)


@pytest.mark.parametrize("T,L", [(4, 16), (3, 5), (8, 8)])
def test_kda_zero_and_open_gates(T, L):
    """Channels whose gate is exactly 0 (they forget the state and every earlier record) and
    exactly 1 (they keep it), mixed in the same record."""
    sh = LayerShape("kda", 3, 2, 64, 128)
    r = Runner(sh, L, T, wid=310 + T, decay="slow")
    for rnd in range(24):
        x = r.inputs(T)
        a = x["alpha"]
        a[..., 5::11] = 0.0
        a[..., 7::13] = 1.0
        if rnd % 3 == 0:
            a[:, :, :, :] = torch.where(torch.arange(sh.N, device="cuda") < sh.N // 2, a, torch.zeros_like(a))
        r.append(x, T)
        r.verify(x, T)
        r.accept(torch.from_numpy(host_accept(0, 310 + T, rnd, sh.B, T)).cuda())
        r.check_pointers()
    r.check_checkpoint()
    r.error_word()
    _clean(r.report)


def test_kda_b256_standard_512_steps():
    """B=256, H=32, P=N=128, L=16: 512 fused decode steps (the benchmarked launch), sampled heads."""
    w = WORKLOADS["kda_decode_b256"]
    sh = w.shape
    r = Runner(sh, w.L, 1, wid=w.wid, heads=sample_heads(sh.B, sh.H, 32), gen="device", s0_sigma=w.s0_sigma)
    rep = run_standard(r, w.steps, check_every=16, fused=True)
    _clean(rep)
    assert rep.final_pointers["folded"] == [496] * sh.B and rep.final_pointers["h"] == [16] * sh.B


def test_kda_b256_verify_T4():
    w = WORKLOADS["kda_decode_b256"]
    sh = w.shape
    T = w.extra["spec_T"]
    r = Runner(sh, w.L, T, wid=w.wid + 100, heads=sample_heads(sh.B, sh.H, 32), gen="device",
               s0_sigma=w.s0_sigma)
    rep = run_spec(r, T, 128, check_every=8)
    _clean(rep)
    assert rep.folds > 0
