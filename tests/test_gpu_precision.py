"""The two-precision checkpoint: low-precision rounding never feeds the recurrence.

("ReplaySSM: Cache SSM Inputs, Not State", How it works: Two precisions — non-fold
steps read a low-precision checkpoint, fold steps read the high-precision one and
write both.) Checked GPU against GPU, bit for bit, on identical inputs:

  * the fp32 checkpoint of the two-precision mode equals the FP32 mode's after
    every round (same folds, same arithmetic);
  * the bf16 copy equals the round-to-nearest-even of the fp32 one;
  * outputs of rounds that fold equal the FP32 mode's (they read fp32);
and, against the oracle with slow decay (so the checkpoint matters in every
output), the two-precision drift stays below the shared-bf16 drift.
"""
import numpy as np
import pytest
import torch

import ssm_decode_amd as rs
from synth import LayerShape, host_accept, host_initial_state, host_step

from harness import Runner, run_spec

pytestmark = pytest.mark.gpu


def _layer(precision, sh, L, T, S0):
    cfg = rs.make_config("mamba2", precision, sh.B, sh.H, sh.P, sh.N, L, T)
    lay = rs.LayerState(cfg)
    lay.import_state(S0)
    return cfg, lay


def test_two_precision_bitwise_invariants():
    sh = LayerShape("mamba2", 4, 6, 64, 128)
    L, T = 8, 4
    S0 = torch.from_numpy(host_initial_state(3, 70, sh, 0.1)).cuda()
    c32, l32 = _layer("fp32", sh, L, T, S0)
    c2p, l2p = _layer("fp32_hp_bf16_lp", sh, L, T, S0)
    folds_seen = 0
    for rnd in range(40):
        x = {k: torch.from_numpy(v).cuda() for k, v in host_step(3, 70, rnd, sh, T, decay="slow").items()}
        o32 = torch.empty((sh.B, T, sh.H, sh.P), device="cuda")
        o2p = torch.empty_like(o32)
        h_before = l32.h.clone()
        for cfg, lay, out in ((c32, l32, o32), (c2p, l2p, o2p)):
            rs.append(cfg, lay.struct, T, x["alpha"], x["k"], x["v"])
            rs.verify(cfg, lay.struct, T, x["q"], out)
        folded = (h_before + T > L)
        if folded.any():
            folds_seen += int(folded.sum())
            assert torch.equal(o32[folded], o2p[folded])  # fold rounds read fp32 in both modes
        a = torch.from_numpy(host_accept(3, 70, rnd, sh.B, T)).cuda()
        rs.accept(c32, l32.struct, a)
        rs.accept(c2p, l2p.struct, a)
        hp32 = l32.export_state("hp")
        hp2p = l2p.export_state("hp")
        assert torch.equal(hp32, hp2p), rnd
        lp = l2p.export_state("lp")
        assert torch.equal(lp, hp2p.to(torch.bfloat16).to(torch.float32)), rnd
        assert l32.pointers() == l2p.pointers()
    assert folds_seen > 0
    assert rs.read_error(l32.struct) == 0 and rs.read_error(l2p.struct) == 0


def test_two_precision_drifts_less_than_shared_bf16():
    """Slow decay keeps the checkpoint in every output: shared-bf16 rounding accumulates in the
    recurrence, two-precision rounding does not."""
    sh = LayerShape("mamba2", 4, 8, 64, 128)
    drift = {}
    for prec in ("fp32_hp_bf16_lp", "bf16_shared", "fp32"):
        r = Runner(sh, 8, 4, precision=prec, wid=71, decay="slow", s0_sigma=0.5, check_ring=False)
        rep = run_spec(r, 4, 160, check_every=40)
        assert rep.pointer_mismatch == 0 and rep.err_word == 0
        drift[prec] = rep.max_rel_token
        if prec == "fp32_hp_bf16_lp":  # per head, against the magnitudes of the terms it sums
            assert rep.mag_vectors > 0 and rep.max_rel_mag <= 2e-2, rep.max_rel_mag
    assert drift["fp32"] <= 1e-4
    assert drift["fp32_hp_bf16_lp"] <= 2e-2
    assert drift["fp32_hp_bf16_lp"] < drift["bf16_shared"], drift
    print("max drift vs oracle:", drift)


def test_non_fold_steps_leave_checkpoints_bitwise_untouched():
    """Writes drop from L to 1 per window: between folds the stored checkpoints do not change."""
    sh = LayerShape("mamba2", 3, 4, 64, 128)
    L = 6
    S0 = torch.from_numpy(host_initial_state(5, 72, sh, 0.1)).cuda()
    cfg, lay = _layer("fp32_hp_bf16_lp", sh, L, 1, S0)
    out = torch.empty((sh.B, sh.H, sh.P), device="cuda")
    changes = 0
    for t in range(3 * L + 2):
        hp0, lp0 = lay.hp.clone(), lay.lp.clone()
        fold = int(lay.h[0].item()) + 1 > L
        x = {k: torch.from_numpy(v).cuda() for k, v in host_step(5, 72, t, sh, 1).items()}
        rs.append(cfg, lay.struct, 1, x["alpha"], x["k"], x["v"])
        rs.decode(cfg, lay.struct, x["q"], out)
        same = torch.equal(hp0, lay.hp) and torch.equal(lp0, lay.lp)
        assert same != fold, (t, fold)
        changes += fold
    assert changes == 3  # steps L+1, 2L+1, 3L+1
