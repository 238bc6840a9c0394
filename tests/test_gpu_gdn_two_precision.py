"""Gated DeltaNet with the two-precision checkpoint.

Non-fold steps read the bf16 copy, so the correction u_t = beta_t (v_t - alpha_t S_{t-1} k_t)
stored with a record carries the copy's rounding. A fold recomputes every folded record's u
from the fp32 checkpoint and the record's raw v before folding, so the fp32 checkpoint stays
the exact recurrence ("ReplaySSM: Cache SSM Inputs, Not State", How it works: Gated DeltaNet
and Two precisions). Checked here:

  * the fp32 checkpoint after every fold against the oracle at 1e-4, with slow decay so that
    the checkpoint dominates the outputs; token outputs at the 2e-2 bar;
  * the fp32 checkpoint against the FP32 mode's on the same inputs (two exact computations in
    different orders: agreement at fp32 rounding level, far below the bf16 step);
  * the bf16 copy equals round-to-nearest-even of the fp32 checkpoint, bit for bit;
  * the fused calls, and the full-size layer (B=256, H=32, 128 x 128) on whole sequences.
"""
import numpy as np
import pytest
import torch

import ssm_decode_amd as rs
from synth import LayerShape, WORKLOADS, host_accept, host_initial_state, host_step

from harness import Runner, rel_err, run_spec, run_standard, whole_sequences

pytestmark = pytest.mark.gpu

TOL = 1e-4
TOL_LP = 2e-2
PREC = "fp32_hp_bf16_lp"


def _lp_clean(rep):
    assert rep.pointer_mismatch == 0, (rep.final_pointers, rep.oracle_pointers)
    assert rep.err_word == 0
    assert rep.max_rel_token <= TOL_LP, rep.max_rel_token
    assert rep.mag_vectors > 0 and rep.max_rel_mag <= TOL_LP, rep.max_rel_mag  # per head, against the terms' magnitudes
    assert rep.max_rel_ckpt <= TOL, rep.max_rel_ckpt


@pytest.mark.parametrize("P,N,L", [(128, 128, 8), (64, 64, 16), (32, 64, 5)])
def test_gdn_two_precision_standard(P, N, L):
    sh = LayerShape("gdn", 3, 4, P, N)
    r = Runner(sh, L, 1, precision=PREC, wid=500 + L, decay="slow", s0_sigma=0.5, check_ring=False)
    rep = run_standard(r, 4 * L + 3, check_every=L)
    _lp_clean(rep)
    # the stored corrections carry the bf16 copy's rounding; the checkpoint does not
    print(f"stored u vs exact: {rep.max_rel_u:.2e}; fp32 checkpoint: {rep.max_rel_ckpt:.2e}")
    assert rep.max_rel_u > 10 * rep.max_rel_ckpt
    assert rep.folds >= 3 * sh.B  # folds are counted per sequence


@pytest.mark.parametrize("T,L", [(4, 16), (3, 5), (8, 8)])
def test_gdn_two_precision_spec(T, L):
    sh = LayerShape("gdn", 4, 3, 128, 128)
    r = Runner(sh, L, T, precision=PREC, wid=510 + T, decay="slow", s0_sigma=0.5, check_ring=False)
    rep = run_spec(r, T, 60, check_every=10)
    _lp_clean(rep)
    assert rep.folds > 0


@pytest.mark.parametrize("fused_T", [1, 4])
def test_gdn_two_precision_fused(fused_T):
    sh = LayerShape("gdn", 3, 4, 128, 128)
    r = Runner(sh, 8, fused_T, precision=PREC, wid=520 + fused_T, decay="slow", s0_sigma=0.5, check_ring=False)
    rep = run_standard(r, 30, fused=True) if fused_T == 1 else run_spec(r, fused_T, 40, fused=True)
    _lp_clean(rep)


def _layer(precision, sh, L, T, S0):
    cfg = rs.make_config("gdn", precision, sh.B, sh.H, sh.P, sh.N, L, T)
    lay = rs.LayerState(cfg)
    lay.import_state(S0)
    return cfg, lay


def test_gdn_two_precision_matches_fp32_mode_and_rounds_exactly():
    """Same inputs through FP32 and two-precision layers: after every fold the two fp32
    checkpoints agree to fp32 rounding (max relative difference 1e-5, against bf16's 4e-3 step),
    and the bf16 copy is RNE of the fp32 one bit for bit."""
    sh = LayerShape("gdn", 3, 4, 128, 128)
    L, T = 8, 4
    S0 = torch.from_numpy(host_initial_state(7, 530, sh, 0.5)).cuda()
    c32, l32 = _layer("fp32", sh, L, T, S0)
    c2p, l2p = _layer(PREC, sh, L, T, S0)
    worst, folds = 0.0, 0
    for rnd in range(48):
        x = {k: torch.from_numpy(v).cuda() for k, v in host_step(7, 530, rnd, sh, T, decay="slow").items()}
        out = torch.empty((sh.B, T, sh.H, sh.P), device="cuda")
        h_before = l32.h.clone()
        for cfg, lay in ((c32, l32), (c2p, l2p)):
            rs.append(cfg, lay.struct, T, x["alpha"], x["k"], x["v"], x["beta"])
            rs.verify(cfg, lay.struct, T, x["q"], out)
        a = torch.from_numpy(host_accept(7, 530, rnd, sh.B, T)).cuda()
        rs.accept(c32, l32.struct, a)
        rs.accept(c2p, l2p.struct, a)
        if bool((h_before + T > L).any()):
            folds += 1
            hp32 = l32.export_state("hp").cpu().numpy().reshape(-1, sh.P * sh.N)
            hp2p = l2p.export_state("hp").cpu().numpy().reshape(-1, sh.P * sh.N)
            worst = max(worst, float(rel_err(hp2p, hp32).max()))
        lp = l2p.export_state("lp")
        assert torch.equal(lp, l2p.export_state("hp").to(torch.bfloat16).to(torch.float32)), rnd
        assert l32.pointers() == l2p.pointers()
    assert folds >= 8
    print(f"two-precision vs FP32-mode checkpoint: max rel diff {worst:.2e} over {folds} fold rounds")
    assert worst <= 1e-5, worst
    assert rs.read_error(l2p.struct) == 0


def test_gdn_two_precision_b256_verify():
    """Full size: B=256, H=32, 128 x 128, L=16, T=4, 128 rounds; three whole sequences followed."""
    w = WORKLOADS["gdn_decode_b256"]
    sh = w.shape
    r = Runner(sh, w.L, 4, precision=PREC, wid=w.wid + 600, heads=whole_sequences(sh.B, sh.H, [0, 131, sh.B - 1]),
               gen="device", s0_sigma=w.s0_sigma, check_ring=False)
    rep = run_spec(r, 4, 128, check_every=16)
    print(f"GDN two-precision B=256: token drift {rep.max_rel_token:.3e}, ckpt {rep.max_rel_ckpt:.3e}")
    _lp_clean(rep)
    assert rep.folds > 0
