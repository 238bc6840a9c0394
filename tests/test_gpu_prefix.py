"""Prefix states: selective flush, snapshot and restore.

The checkpoint alone is a sequence's state only once its committed records are folded; before
that it trails them (the staleness raised about prefix caching in the replies of the thread on
"ReplaySSM"). A cached prefix is therefore taken by folding (replayssm_flush_selected), copied
out (replayssm_snapshot) and used to start other sequences (replayssm_restore).
"""
import numpy as np
import pytest
import torch

import ssm_decode_amd as rs
from synth import LayerShape, host_initial_state, host_step

from harness import Runner, rel_err, run_standard

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("kind,precision", [("mamba2", "fp32"), ("mamba2", "fp32_hp_bf16_lp"),
                                            ("gdn", "fp32"), ("gdn", "fp32_hp_bf16_lp"), ("kda", "fp32")])
def test_snapshot_after_selective_flush_is_the_exact_state(kind, precision):
    """After 11 standard steps (L = 8: 3 records unfolded) a selective flush of sequences 0 and 2
    makes their checkpoints the state after all 11 tokens: the snapshot equals the oracle's
    eager state at 1e-4. Sequence 1 keeps its pointers and its checkpoint bits."""
    sh = LayerShape(kind, 3, 4, 64, 128)
    r = Runner(sh, 8, 1, precision=precision, wid=700, decay="slow", s0_sigma=0.5, check_ring=False)
    run_standard(r, 11)
    lay, cfg = r.layer, r.cfg
    before = lay.pointers()
    hp1 = lay.export_state("hp" if precision != "bf16_shared" else "lp")[1].clone()
    sel = torch.tensor([1, 0, 1], dtype=torch.int32, device="cuda")
    rs.flush_selected(cfg, lay.struct, sel)
    after = lay.pointers()
    assert after["h"] == [0, before["h"][1], 0] and after["folded"][1] == before["folded"][1]
    assert after["folded"][0] == before["folded"][0] + before["h"][0]
    assert torch.equal(lay.export_state("hp" if precision != "bf16_shared" else "lp")[1], hp1)
    seqs = torch.tensor([0, 2], dtype=torch.int32, device="cuda")
    dst = torch.empty((2, sh.H, sh.P, sh.N), device="cuda")
    rs.snapshot(cfg, lay.struct, seqs, dst)
    torch.cuda.synchronize()
    assert rs.read_error(lay.struct) == 0
    ref = r.oracle.S.reshape(sh.B, sh.H, sh.P, sh.N)[[0, 2]]
    err = rel_err(dst.cpu().numpy().reshape(-1, sh.P * sh.N), ref.reshape(-1, sh.P * sh.N)).max()
    assert err <= 1e-4, err


def test_snapshot_of_a_stale_sequence_is_flagged():
    sh = LayerShape("mamba2", 2, 2, 32, 32)
    r = Runner(sh, 8, 1, wid=701)
    run_standard(r, 5)
    dst = torch.empty((1, sh.H, sh.P, sh.N), device="cuda")
    rs.snapshot(r.cfg, r.layer.struct, torch.tensor([1], dtype=torch.int32, device="cuda"), dst)
    assert rs.read_error(r.layer.struct) & rs.DEVERR_STALE


@pytest.mark.parametrize("kind,precision", [("mamba2", "fp32"), ("mamba2", "fp32_hp_bf16_lp"), ("gdn", "fp32"),
                                            ("gdn", "fp32_hp_bf16_lp"), ("kda", "fp32")])
def test_restored_sequences_continue_like_their_source(kind, precision):
    """Sequence 0 is flushed and snapshot; sequences 2 and 3 are restored from it. Fed the same
    tokens as sequence 0 from then on, they give bit-identical outputs and checkpoints."""
    sh = LayerShape(kind, 4, 3, 64, 128)
    L, steps0, steps1 = 6, 9, 20
    cfg = rs.make_config(kind, precision, sh.B, sh.H, sh.P, sh.N, L, 1)
    lay = rs.LayerState(cfg)
    lay.import_state(torch.from_numpy(host_initial_state(4, 702, sh, 0.3)).cuda())
    out = torch.empty((sh.B, sh.H, sh.P), device="cuda")
    for t in range(steps0):
        x = {k: torch.from_numpy(v).cuda() for k, v in host_step(4, 702, t, sh, 1, decay="slow").items()}
        rs.decode_step(cfg, lay.struct, x["alpha"], x["k"], x["v"], x.get("beta"), x["q"], out)
    rs.flush_selected(cfg, lay.struct, torch.tensor([1, 0, 0, 0], dtype=torch.int32, device="cuda"))
    snap = torch.empty((1, sh.H, sh.P, sh.N), device="cuda")
    rs.snapshot(cfg, lay.struct, torch.tensor([0], dtype=torch.int32, device="cuda"), snap)
    rs.restore(cfg, lay.struct, torch.tensor([2, 3], dtype=torch.int32, device="cuda"),
               torch.cat([snap, snap]).contiguous())
    p = lay.pointers()
    assert p["h"][2] == p["h"][3] == 0 and p["folded"][2] == p["folded"][3] == 0
    for t in range(steps1):
        x = {k: torch.from_numpy(v).cuda() for k, v in host_step(4, 703, t, sh, 1, decay="slow").items()}
        for key in x:  # sequences 2 and 3 see sequence 0's tokens
            x[key][2] = x[key][0]
            x[key][3] = x[key][0]
        rs.decode_step(cfg, lay.struct, x["alpha"], x["k"], x["v"], x.get("beta"), x["q"], out)
        assert torch.equal(out[2], out[0]) and torch.equal(out[3], out[0]), t
    which = "hp" if precision != "bf16_shared" else "lp"
    S = lay.export_state(which)
    assert torch.equal(S[2], S[0]) and torch.equal(S[3], S[0])
    if precision == "fp32_hp_bf16_lp":
        lp = lay.export_state("lp")
        assert torch.equal(lp[2], lp[0])
    assert rs.read_error(lay.struct) == 0


def test_out_of_range_indices_are_skipped_and_flagged():
    sh = LayerShape("mamba2", 2, 2, 32, 32)
    cfg = rs.make_config("mamba2", "fp32", sh.B, sh.H, sh.P, sh.N, 4, 1)
    lay = rs.LayerState(cfg)
    S0 = torch.from_numpy(host_initial_state(5, 704, sh, 0.3)).cuda()
    lay.import_state(S0)
    dst = torch.full((3, sh.H, sh.P, sh.N), 7.0, device="cuda")
    rs.snapshot(cfg, lay.struct, torch.tensor([1, -1, 2], dtype=torch.int32, device="cuda"), dst)
    assert rs.read_error(lay.struct) & rs.DEVERR_INDEX
    assert torch.equal(dst[0], S0[1]) and bool((dst[1:] == 7.0).all())
    before = lay.export_state("hp").clone()
    rs.restore(cfg, lay.struct, torch.tensor([5], dtype=torch.int32, device="cuda"), dst[:1].contiguous())
    assert torch.equal(lay.export_state("hp"), before)
