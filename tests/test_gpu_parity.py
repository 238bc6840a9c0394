"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bar: outputs within max relative error 1e-4 (fp32 checkpoint); the checkpoint
after folds within 1e-4 of the oracle's state at position `folded`; pointer
arrays and ring copies bit-exact; no device error bits.
"""
import numpy as np
import pytest
import torch

import ssm_decode_amd as rs
from synth import LayerShape, WORKLOADS, host_initial_state, host_step

from harness import Runner, run_spec, run_standard, sample_heads

pytestmark = pytest.mark.gpu

TOL = 1e-4


def _assert_clean(rep, tol=TOL, tol_ckpt=TOL):
    assert rep.pointer_mismatch == 0, (rep.final_pointers, rep.oracle_pointers)
    assert rep.ring_mismatch == 0
    assert rep.err_word == 0
    assert rep.max_rel <= tol, rep.max_rel
    assert rep.max_rel_ckpt <= tol_ckpt, rep.max_rel_ckpt
    assert rep.max_rel_u <= tol, rep.max_rel_u


def test_tiny_workload_every_output():
    """B=1, H=2, P=N=16, L=4: 64 decode steps, every output, 15 folds."""
    w = WORKLOADS["mamba2_tiny"]
    r = Runner(w.shape, w.L, w.T, wid=w.wid, s0_sigma=w.s0_sigma)
    rep = run_standard(r, w.steps)
    _assert_clean(rep)
    assert rep.final_pointers == {"head": [0], "h": [4], "p": [0], "folded": [60]}
    assert rep.folds == 15


@pytest.mark.parametrize("P,N", [(16, 16), (32, 32), (64, 64), (64, 128), (128, 128), (48, 64), (256, 32)])
@pytest.mark.parametrize("L", [1, 3, 16])
def test_mamba2_shapes_standard(P, N, L):
    sh = LayerShape("mamba2", 3, 5, P, N)  # 15 heads: no multiple of anything
    r = Runner(sh, L, 1, wid=10 + L)
    rep = run_standard(r, 2 * L + 5)
    _assert_clean(rep)


@pytest.mark.parametrize("decay", ["recipe", "slow"])
def test_mamba2_long_run_slow_decay(decay):
    """Slow decay (alpha in [0.9, 1)) keeps the checkpoint visible in every output."""
    sh = LayerShape("mamba2", 2, 3, 64, 128)
    r = Runner(sh, 16, 1, wid=21, decay=decay)
    rep = run_standard(r, 120)
    _assert_clean(rep)
    assert rep.folds == 2 * 7


@pytest.mark.parametrize("P,N", [(128, 128), (32, 64), (16, 16), (256, 32), (256, 128)])
@pytest.mark.parametrize("decay", ["recipe", "slow"])
def test_gdn_standard(P, N, decay):
    sh = LayerShape("gdn", 2, 3, P, N)
    r = Runner(sh, 4, 1, wid=30, decay=decay)
    rep = run_standard(r, 23)
    _assert_clean(rep)


@pytest.mark.parametrize("kind", ["mamba2", "gdn", "kda"])
@pytest.mark.parametrize("T,L", [(1, 4), (2, 5), (3, 8), (4, 16), (8, 8), (5, 13)])
def test_spec_rounds(kind, T, L):
    """Random accepted prefixes (0..T) including rejected drafts that get overwritten."""
    sh = LayerShape(kind, 4, 3, 64, 128)
    r = Runner(sh, L, T, wid=40 + T)
    rep = run_spec(r, T, 30)
    _assert_clean(rep)


@pytest.mark.parametrize("kind", ["mamba2", "gdn", "kda"])
def test_explicit_flush_mid_run(kind):
    sh = LayerShape(kind, 3, 2, 64, 64)
    r = Runner(sh, 8, 4, wid=50, decay="slow")
    sh = r.shape
    for rnd in range(6):
        x = r.inputs(4)
        r.append(x, 4)
        r.verify(x, 4)
        r.accept(torch.tensor([rnd % 5, 4, 2][: sh.B], dtype=torch.int32, device="cuda"))
    x = r.inputs(3)
    r.append(x, 3)  # pending drafts survive the flush
    r.flush()
    assert r.check_pointers()
    assert r.check_checkpoint() <= TOL
    r.verify(x, 3)
    r.accept(torch.full((sh.B,), 3, dtype=torch.int32, device="cuda"))
    r.flush()
    r.flush()  # second flush is a no-op
    assert r.check_pointers()
    assert r.check_checkpoint() <= TOL
    assert r.error_word() == 0
    assert r.report.max_rel <= TOL and r.report.max_rel_u <= TOL


@pytest.mark.parametrize("kind", ["mamba2", "gdn", "kda"])
def test_wide_window_standard(kind):
    """L = 64 with one wavefront per workgroup: more records than lanes (serial decay path,
    staging tail loop, alpha tail)."""
    sh = LayerShape(kind, 2, 3, 16, 32)
    r = Runner(sh, 64, 1, wid=60, decay="slow")
    rep = run_standard(r, 140)
    _assert_clean(rep)
    assert rep.folds == 2 * 2


@pytest.mark.parametrize("kind", ["mamba2", "gdn", "kda"])
def test_wide_window_spec(kind):
    sh = LayerShape(kind, 3, 2, 32, 32)
    r = Runner(sh, 56, 8, wid=61, decay="slow")
    rep = run_spec(r, 8, 24)
    _assert_clean(rep)


@pytest.mark.parametrize("kind,P,N,L", [("mamba2", 64, 128, 16), ("mamba2", 16, 16, 4), ("gdn", 128, 128, 5),
                                        ("gdn", 32, 64, 64), ("kda", 128, 128, 5), ("kda", 32, 64, 64)])
def test_fused_decode_step(kind, P, N, L):
    """replayssm_decode_step = append + decode in one launch: same oracle bar, ring written by it."""
    sh = LayerShape(kind, 3, 5, P, N)
    r = Runner(sh, L, 1, wid=110, decay="slow")
    rep = run_standard(r, 2 * L + 7, fused=True)
    _assert_clean(rep)


@pytest.mark.parametrize("kind", ["mamba2", "gdn", "kda"])
@pytest.mark.parametrize("T,L", [(4, 16), (3, 5), (8, 8)])
def test_fused_verify_step(kind, T, L):
    sh = LayerShape(kind, 4, 3, 64, 128)
    r = Runner(sh, L, T, wid=111 + T)
    rep = run_spec(r, T, 30, fused=True)
    _assert_clean(rep)


@pytest.mark.parametrize("kind", ["mamba2", "gdn", "kda"])
def test_fused_equals_unfused_bitwise(kind):
    """Same inputs through append+decode and through decode_step: identical bits everywhere."""
    sh = LayerShape(kind, 5, 4, 64, 128)
    S0 = torch.from_numpy(host_initial_state(0, 112, sh, 0.1)).cuda()
    cfg = rs.make_config(kind, "fp32", sh.B, sh.H, sh.P, sh.N, 6, 1)
    la, lb = rs.LayerState(cfg), rs.LayerState(cfg)
    la.import_state(S0)
    lb.import_state(S0)
    oa = torch.empty((sh.B, sh.H, sh.P), device="cuda")
    ob = torch.empty_like(oa)
    for t in range(20):
        x = {k: torch.from_numpy(v).cuda() for k, v in host_step(0, 112, t, sh, 1).items()}
        rs.append(cfg, la.struct, 1, x["alpha"], x["k"], x["v"], x.get("beta"))
        rs.decode(cfg, la.struct, x["q"], oa)
        rs.decode_step(cfg, lb.struct, x["alpha"], x["k"], x["v"], x.get("beta"), x["q"], ob)
        assert torch.equal(oa, ob), t
    assert torch.equal(la.hp, lb.hp) and torch.equal(la.ring_k, lb.ring_k) and torch.equal(la.ring_v, lb.ring_v)
    assert torch.equal(la.ring_alpha, lb.ring_alpha) and la.pointers() == lb.pointers()


@pytest.mark.parametrize("kind", ["mamba2", "gdn", "kda"])
@pytest.mark.parametrize("P,N,T,L", [(256, 128, 4, 12), (256, 64, 8, 8), (48, 128, 3, 7)])
def test_spec_rounds_wide_and_odd_heads(kind, P, N, T, L):
    """16 wavefronts per workgroup (dv = 256) and an odd tile count (dv = 48), speculative rounds
    with random accepted prefixes and folds."""
    sh = LayerShape(kind, 3, 2, P, N)
    r = Runner(sh, L, T, wid=130 + T, decay="slow")
    rep = run_spec(r, T, 20)
    _assert_clean(rep)
    assert rep.folds > 0


@pytest.fixture
def two_tiles():
    rs.set_tiling(rs.TILES_TWO)
    yield
    rs.set_tiling(rs.TILES_AUTO)


@pytest.mark.parametrize("kind", ["mamba2", "gdn", "kda"])
@pytest.mark.parametrize("P", [32, 96, 160])
@pytest.mark.parametrize("T,L,fused", [(1, 4, False), (1, 6, True), (4, 9, False), (3, 5, True)])
def test_two_tiles_per_wavefront(kind, P, T, L, fused, two_tiles):
    """dk = 128 with at most four drafts, two 16-row tiles per wavefront forced (the automatic
    choice takes them only for large batches): one wavefront (dv = 32), an odd wavefront count
    (dv = 96, 160), decode and speculative rounds, fused and from the ring, with folds."""
    sh = LayerShape(kind, 3, 3, P, 128)
    r = Runner(sh, L, T, wid=170 + T, decay="slow")
    rep = run_standard(r, 2 * L + 5, fused=fused) if T == 1 else run_spec(r, T, 20, fused=fused)
    _assert_clean(rep)
    assert rep.folds > 0
