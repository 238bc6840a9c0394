"""Device-side contract violations: flagged in the sticky error word, never faulting.

Each violation is forced from the host with ordinary calls (or by writing a
pointer out of its range through torch); the kernels check the pointers before
they address anything, skip (or clamp) the offending sequence, and leave the
others untouched.
"""
import pytest
import torch

import ssm_decode_amd as rs
from synth import LayerShape, host_initial_state, host_step

pytestmark = pytest.mark.gpu


def _setup(T_max=1, B=3, kind="mamba2"):
    sh = LayerShape(kind, B, 2, 32, 32)
    cfg = rs.make_config(kind, "fp32", B, 2, 32, 32, 4, T_max)
    lay = rs.LayerState(cfg)
    lay.import_state(torch.from_numpy(host_initial_state(0, 95, sh, 0.1)).cuda())
    return sh, cfg, lay


def _x(sh, T, step=0):
    return {k: torch.from_numpy(v).cuda() for k, v in host_step(0, 95, step, sh, T).items()}


def test_decode_without_append_is_flagged_and_skipped():
    sh, cfg, lay = _setup()
    out = torch.full((sh.B, sh.H, sh.P), float("nan"), device="cuda")
    before = lay.pointers()
    rs.decode(cfg, lay.struct, _x(sh, 1)["q"], out)
    assert rs.read_error(lay.struct) == rs.DEVERR_PENDING
    assert lay.pointers() == before
    assert torch.isnan(out).all()  # nothing written for skipped sequences


def test_append_overflow_is_flagged():
    sh, cfg, lay = _setup()
    x = _x(sh, 1)
    rs.append(cfg, lay.struct, 1, x["alpha"], x["k"], x["v"])
    ring = lay.ring_k.clone()
    rs.append(cfg, lay.struct, 1, x["alpha"], x["k"], x["v"])  # p would become 2 > T_max
    assert rs.read_error(lay.struct) == rs.DEVERR_APPEND_OVERFLOW
    assert lay.p.tolist() == [1] * sh.B
    assert torch.equal(ring, lay.ring_k)


def test_accept_more_than_pending_is_clamped():
    sh, cfg, lay = _setup(T_max=4)
    x = _x(sh, 3)
    rs.append(cfg, lay.struct, 3, x["alpha"], x["k"], x["v"])
    out = torch.empty((sh.B, 3, sh.H, sh.P), device="cuda")
    rs.verify(cfg, lay.struct, 3, x["q"], out)
    rs.accept(cfg, lay.struct, torch.tensor([1, 7, -2], dtype=torch.int32, device="cuda"))
    assert rs.read_error(lay.struct) == rs.DEVERR_ACCEPT
    assert lay.h.tolist() == [1, 3, 0] and lay.p.tolist() == [0, 0, 0]


def test_corrupt_pointer_is_skipped_and_others_proceed():
    sh, cfg, lay = _setup()
    x = _x(sh, 1)
    rs.append(cfg, lay.struct, 1, x["alpha"], x["k"], x["v"])
    lay.head[1] = cfg.L + cfg.T_max  # = C: out of range
    out = torch.full((sh.B, sh.H, sh.P), float("nan"), device="cuda")
    rs.decode(cfg, lay.struct, x["q"], out)
    err = rs.read_error(lay.struct)
    assert err & rs.DEVERR_CORRUPT
    assert torch.isnan(out[1]).all()
    assert torch.isfinite(out[0]).all() and torch.isfinite(out[2]).all()
    assert lay.h.tolist() == [1, 0, 1] and lay.head.tolist() == [0, 5, 0]
    rs.flush(cfg, lay.struct)  # the flush kernel skips it too
    rs.append(cfg, lay.struct, 1, x["alpha"], x["k"], x["v"])  # and the append kernel
    assert rs.read_error(lay.struct) & rs.DEVERR_CORRUPT


def test_verify_with_wrong_pending_count_is_flagged():
    sh, cfg, lay = _setup(T_max=4)
    x = _x(sh, 2)
    rs.append(cfg, lay.struct, 2, x["alpha"], x["k"], x["v"])
    out = torch.empty((sh.B, 3, sh.H, sh.P), device="cuda")
    q3 = _x(sh, 3)["q"]
    rs.verify(cfg, lay.struct, 3, q3, out)  # p = 2 != 3
    assert rs.read_error(lay.struct) == rs.DEVERR_PENDING
    assert lay.p.tolist() == [2] * sh.B


def test_host_validation_errors_raise():
    sh, cfg, lay = _setup(T_max=4)
    x = _x(sh, 1)
    with pytest.raises(rs.ReplaySSMError):
        rs.append(cfg, lay.struct, 5, x["alpha"], x["k"], x["v"])
    with pytest.raises(rs.ReplaySSMError):
        rs.verify(cfg, lay.struct, 0, x["q"], x["q"])
