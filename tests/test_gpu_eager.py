"""The eager comparison kernels against the oracle, and replay against eager.

replayssm_eager_step is the conventional step (load the state, update it, read
the output, store it); replayssm_eager_verify keeps one stored state per draft
and replayssm_eager_accept selects the accepted one.
"""
import numpy as np
import pytest
import torch

import ssm_decode_amd as rs
from oracle.session import OracleSession, select_heads
from synth import LayerShape, host_accept, host_initial_state, host_step

from harness import Runner, rel_err, run_standard

pytestmark = pytest.mark.gpu


def _packed(cfg, S0, nslots=1):
    sh = (cfg.B, cfg.H, cfg.dv * cfg.dk)
    packed = torch.empty(sh, device="cuda")
    rs.pack_state(cfg, S0, packed, None)
    if nslots == 1:
        return packed
    pool = torch.zeros((cfg.B, cfg.H, nslots, cfg.dv * cfg.dk), device="cuda")
    pool[:, :, 0].copy_(packed)
    return pool


@pytest.mark.parametrize("kind,P,N", [("mamba2", 64, 128), ("gdn", 128, 128), ("mamba2", 16, 16), ("gdn", 32, 64),
                                       ("kda", 128, 128), ("kda", 32, 64)])
def test_eager_step_matches_oracle(kind, P, N):
    sh = LayerShape(kind, 3, 5, P, N)
    cfg = rs.make_config(kind, "fp32", sh.B, sh.H, P, N, 16, 1)
    S0 = torch.from_numpy(host_initial_state(0, 80, sh, 0.1)).cuda()
    S = _packed(cfg, S0)
    heads = [(b, h) for b in range(sh.B) for h in range(sh.H)]
    ses = OracleSession(kind, sh.B, sh.H, P, N, 16, 1, S0.cpu().numpy().reshape(-1, P, N), heads)
    out = torch.empty((sh.B, sh.H, P), device="cuda")
    worst = 0.0
    for t in range(20):
        x = host_step(0, 80, t, sh, 1, decay="slow")
        xd = {k: torch.from_numpy(v).cuda() for k, v in x.items()}
        rs.eager_step(cfg, S, xd["alpha"], xd["k"], xd["v"], xd.get("beta"), xd["q"], out)
        ses.append(select_heads(x["alpha"], heads), select_heads(x["k"], heads), select_heads(x["v"], heads),
                   select_heads(x["beta"], heads) if "beta" in x else None)
        ref, _, _ = ses.decode(select_heads(x["q"], heads))
        got = out.cpu().numpy().reshape(-1, 1, P)
        worst = max(worst, float(rel_err(got, ref).max()))
    assert worst <= 1e-4, worst
    logical = torch.empty((sh.B, sh.H, P, N), device="cuda")
    rs.unpack_state(cfg, S, None, logical)
    assert float(rel_err(logical.cpu().numpy().reshape(-1, P, N), ses.S).max()) <= 1e-4


@pytest.mark.parametrize("kind", ["mamba2", "gdn", "kda"])
def test_eager_snapshot_verify_matches_oracle(kind):
    sh = LayerShape(kind, 4, 3, 64, 128)
    T = 4
    cfg = rs.make_config(kind, "fp32", sh.B, sh.H, sh.P, sh.N, 16, T)
    S0 = torch.from_numpy(host_initial_state(1, 81, sh, 0.1)).cuda()
    pool = _packed(cfg, S0, T + 1)
    slot = torch.zeros(sh.B, dtype=torch.int32, device="cuda")
    heads = [(b, h) for b in range(sh.B) for h in range(sh.H)]
    ses = OracleSession(kind, sh.B, sh.H, sh.P, sh.N, 16, T, S0.cpu().numpy().reshape(-1, sh.P, sh.N), heads)
    out = torch.empty((sh.B, T, sh.H, sh.P), device="cuda")
    worst = 0.0
    for rnd in range(24):
        x = host_step(1, 81, rnd, sh, T)
        xd = {k: torch.from_numpy(v).cuda() for k, v in x.items()}
        rs.eager_verify(cfg, pool, slot, T, xd["alpha"], xd["k"], xd["v"], xd.get("beta"), xd["q"], out)
        ses.append(select_heads(x["alpha"], heads), select_heads(x["k"], heads), select_heads(x["v"], heads),
                   select_heads(x["beta"], heads) if "beta" in x else None)
        ref, _, _ = ses.verify(select_heads(x["q"], heads))
        worst = max(worst, float(rel_err(out.permute(0, 2, 1, 3).cpu().numpy().reshape(-1, T, sh.P), ref).max()))
        a = host_accept(1, 81, rnd, sh.B, T)
        rs.eager_accept(cfg, slot, torch.from_numpy(a).cuda(), T)
        ses.accept(a)
    assert worst <= 1e-4, worst
    committed = torch.stack([pool[b, :, int(slot[b])] for b in range(sh.B)]).contiguous()
    logical = torch.empty((sh.B, sh.H, sh.P, sh.N), device="cuda")
    rs.unpack_state(cfg, committed, None, logical)
    assert float(rel_err(logical.cpu().numpy().reshape(-1, sh.P, sh.N), ses.S).max()) <= 1e-4


@pytest.mark.parametrize("kind", ["mamba2", "gdn", "kda"])
def test_replay_with_window_one_equals_eager(kind):
    """L = 1 folds every token (state written every step): replay and eager give the same outputs."""
    sh = LayerShape(kind, 2, 4, 64, 128)
    cfg_e = rs.make_config(kind, "fp32", sh.B, sh.H, sh.P, sh.N, 1, 1)
    S0 = torch.from_numpy(host_initial_state(2, 82, sh, 0.1)).cuda()
    S = _packed(cfg_e, S0)
    lay = rs.LayerState(cfg_e)
    lay.import_state(S0)
    oe = torch.empty((sh.B, sh.H, sh.P), device="cuda")
    orp = torch.empty_like(oe)
    for t in range(16):
        xd = {k: torch.from_numpy(v).cuda() for k, v in host_step(2, 82, t, sh, 1, decay="slow").items()}
        rs.eager_step(cfg_e, S, xd["alpha"], xd["k"], xd["v"], xd.get("beta"), xd["q"], oe)
        rs.append(cfg_e, lay.struct, 1, xd["alpha"], xd["k"], xd["v"], xd.get("beta"))
        rs.decode(cfg_e, lay.struct, xd["q"], orp)
        r = rel_err(orp.cpu().numpy(), oe.cpu().numpy())
        assert r.max() <= 1e-5, (t, r.max())
    # the checkpoint after its last fold is the eager state one token earlier; fold it now
    rs.flush(cfg_e, lay.struct)
    logical_e = torch.empty((sh.B, sh.H, sh.P, sh.N), device="cuda")
    rs.unpack_state(cfg_e, S, None, logical_e)
    assert float(rel_err(lay.export_state("hp").cpu().numpy(), logical_e.cpu().numpy()).max()) <= 1e-5
