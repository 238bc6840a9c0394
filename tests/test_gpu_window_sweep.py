"""Window-size sweep: every (L, T) cell the library supports, at the real head shape, to the
same oracle bar as the headline configuration.

("ReplaySSM: Cache SSM Inputs, Not State", How it works: Window size — a longer window writes
the checkpoint less often and replays more records per token.) The cells are L in {4, 8, 16,
32, 64} and T in {1, 4, 8} with T <= L; L = 64 with T = 8 stages 69 KiB of records per
workgroup, past the 64 KiB that fits padded rows. Each run covers at least two folds. The long
windows also run with two checkpoint tiles per wavefront forced (the form the benchmark's
batch takes), whose record staging, wide decay scans and unpadded rows differ.
"""
import re

import pytest
import torch

import ssm_decode_amd as rs
from synth import LayerShape

from harness import Runner, run_spec, run_standard

pytestmark = pytest.mark.gpu

TOL = 1e-4
TOL_LP = 2e-2
CELLS = [(L, T) for L in (4, 8, 16, 32, 64) for T in (1, 4, 8) if T <= L]


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


@pytest.fixture
def two_tiles():
    rs.set_tiling(rs.TILES_TWO)
    yield
    rs.set_tiling(rs.TILES_AUTO)


@pytest.mark.parametrize("L,T", [(32, 1), (32, 4), (64, 1), (64, 4)])
def test_window_cell_two_tiles(two_tiles, L, T):
    sh = LayerShape("mamba2", 3, 4, 64, 128)
    r = Runner(sh, L, T, wid=350 + 10 * L + T, decay="slow")
    rep = run_standard(r, _rounds(L, T)) if T == 1 else run_spec(r, T, _rounds(L, T))
    assert rep.pointer_mismatch == 0 and rep.ring_mismatch == 0 and rep.err_word == 0
    assert rep.max_rel <= TOL and rep.max_rel_ckpt <= TOL, (rep.max_rel, rep.max_rel_ckpt)
    assert rep.folds >= 2 * sh.B, rep.folds


@pytest.mark.parametrize("kind", ["mamba2", "gdn"])
def test_window_64_fused_verify_two_tiles(two_tiles, kind):
    sh = LayerShape(kind, 2, 3, 64, 128)
    r = Runner(sh, 64, 4, wid=430, decay="slow")
    rep = run_spec(r, 4, _rounds(64, 4), fused=True)
    assert rep.pointer_mismatch == 0 and rep.ring_mismatch == 0 and rep.err_word == 0
    assert rep.max_rel <= TOL and rep.max_rel_ckpt <= TOL and rep.max_rel_u <= TOL


def test_gdn_two_precision_exact_fold_window_32_two_tiles(two_tiles):
    sh = LayerShape("gdn", 3, 2, 128, 128)
    r = Runner(sh, 32, 4, precision="fp32_hp_bf16_lp", wid=440, decay="slow", s0_sigma=0.5, check_ring=False)
    rep = run_spec(r, 4, _rounds(32, 4))
    assert rep.pointer_mismatch == 0 and rep.err_word == 0
    assert rep.max_rel_token <= TOL_LP and rep.mag_vectors > 0 and rep.max_rel_mag <= TOL_LP
    assert rep.max_rel_ckpt <= TOL, rep.max_rel_ckpt
    assert rep.folds > 0


def test_window_past_the_device_lds_is_rejected():
    """KDA with dv = 256 at L = 64, T = 8 would stage about 165 KB of records per workgroup:
    more than a gfx950 workgroup's 160 KiB (the device's own figure), so the configuration is
    refused before anything runs."""
    limit = torch.cuda.get_device_properties(0).shared_memory_per_block
    assert limit == 160 * 1024, limit
    cfg = rs.make_config("kda", "fp32", 3, 4, 256, 128, 64, 8)
    with pytest.raises(rs.ReplaySSMError) as e:
        rs.get_sizes(cfg)
    assert e.value.status == rs.ENOTSUP
    need = int(re.search(r"need (\d+) bytes of LDS", str(e.value)).group(1))
    assert limit < need < limit + 4096, need
    ok = rs.make_config("kda", "fp32", 3, 4, 128, 128, 64, 8)  # about 128 KB: runs
    assert rs.get_sizes(ok).C == 72


@pytest.mark.parametrize("kind,precision,dv,L,T", [
    ("kda", "fp32", 128, 64, 8),                 # 128,288 bytes of LDS per workgroup
    ("gdn", "fp32_hp_bf16_lp", 128, 64, 4),      # 95,104 bytes (the exact-correction fold's Gram block)
    ("mamba2", "fp32", 256, 64, 8),              # 124,544 bytes
])
def test_long_windows_past_64k_of_lds(kind, precision, dv, L, T):
    """Kernels whose record staging needs more than 64 KiB of LDS, each against the oracle."""
    sh = LayerShape(kind, 2, 2, dv, 128)
    r = Runner(sh, L, T, precision=precision, wid=460 + T, decay="slow", check_ring=precision == "fp32")
    rep = run_spec(r, T, _rounds(L, T))
    assert rep.pointer_mismatch == 0 and rep.ring_mismatch == 0 and rep.err_word == 0
    if precision == "fp32":
        assert rep.max_rel <= TOL and rep.max_rel_u <= TOL, (rep.max_rel, rep.max_rel_u)
    else:
        assert rep.max_rel_token <= TOL_LP and rep.max_rel_mag <= TOL_LP
    assert rep.max_rel_ckpt <= TOL, rep.max_rel_ckpt
    assert rep.folds >= 2 * sh.B, rep.folds
