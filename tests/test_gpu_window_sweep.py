"""Window-size sweep: every (L, T) cell the library supports, at the real head shape, to the
same oracle bar as the headline configuration.

("ReplaySSM: Cache SSM Inputs, Not State", How it works: Window size — a longer window writes
the checkpoint less often and replays more records per token.) The cells are L in {4, 8, 16,
32, 64} and T in {1, 4, 8} with T <= L; L = 64 with T = 8 does not fit the LDS budget and is
rejected (ENOTSUP). Each run covers at least two folds.
"""
import pytest

import ssm_decode_amd as rs
from synth import LayerShape

from harness import Runner, run_spec, run_standard

pytestmark = pytest.mark.gpu

TOL = 1e-4
TOL_LP = 2e-2
CELLS = [(L, T) for L in (4, 8, 16, 32, 64) for T in (1, 4, 8) if T <= L and (L, T) != (64, 8)]


def _rounds(L, T):
    # accepted prefix ~ U{0..T}: h grows by T/2 per round on average; a fold when h + T > L
    return 2 * L + 5 if T == 1 else 2 * (2 * (L - T) // T + 2) + 6


@pytest.mark.parametrize("L,T", CELLS)
def test_window_cell_fp32(L, T):
    sh = LayerShape("mamba2", 3, 4, 64, 128)
    r = Runner(sh, L, T, wid=300 + 10 * L + T, decay="slow")
    rep = run_standard(r, _rounds(L, T)) if T == 1 else run_spec(r, T, _rounds(L, T))
    assert rep.pointer_mismatch == 0, (rep.final_pointers, rep.oracle_pointers)
    assert rep.ring_mismatch == 0 and rep.err_word == 0
    assert rep.max_rel <= TOL and rep.max_rel_ckpt <= TOL, (rep.max_rel, rep.max_rel_ckpt)
    assert rep.folds >= 2 * sh.B, rep.folds


@pytest.mark.parametrize("L,T", [(4, 4), (32, 4), (64, 4)])
def test_window_cell_two_precision(L, T):
    sh = LayerShape("mamba2", 3, 4, 64, 128)
    r = Runner(sh, L, T, precision="fp32_hp_bf16_lp", wid=400 + L, decay="slow", check_ring=False)
    rep = run_spec(r, T, _rounds(L, T))
    assert rep.pointer_mismatch == 0 and rep.err_word == 0
    assert rep.max_rel_token <= TOL_LP and rep.max_rel_ckpt <= TOL, (rep.max_rel_token, rep.max_rel_ckpt)


@pytest.mark.parametrize("kind", ["mamba2", "gdn"])
def test_window_64_fused_verify(kind):
    """The unpadded-row layout (L = 64, T = 4) through the fused verify call, both kinds."""
    sh = LayerShape(kind, 2, 3, 64, 128)
    r = Runner(sh, 64, 4, wid=420, decay="slow")
    rep = run_spec(r, 4, _rounds(64, 4), fused=True)
    assert rep.pointer_mismatch == 0 and rep.ring_mismatch == 0 and rep.err_word == 0
    assert rep.max_rel <= TOL and rep.max_rel_ckpt <= TOL and rep.max_rel_u <= TOL


def test_window_64_drafts_8_is_rejected():
    cfg = rs.make_config("mamba2", "fp32", 3, 4, 64, 128, 64, 8)
    with pytest.raises(rs.ReplaySSMError) as e:
        rs.get_sizes(cfg)
    assert e.value.status == rs.ENOTSUP
