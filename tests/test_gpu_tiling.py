"""The replay kernel's two tilings (one or two 16-row state tiles per wavefront, chosen by
replayssm_set_tiling or automatically by batch size) give the same bits everywhere: outputs,
both checkpoint copies, rings, pointers. Exercised on decode steps, speculative rounds with
random accepted prefixes, folds and an explicit flush, for every kind and both precisions."""
import pytest
import torch

import ssm_decode_amd as rs
from synth import LayerShape, host_accept, host_initial_state, host_step

pytestmark = pytest.mark.gpu


@pytest.fixture
def restore_tiling():
    yield
    rs.set_tiling(rs.TILES_AUTO)


def _run(kind, precision, sh, L, T, fused, policy, wid, rounds):
    rs.set_tiling(policy)
    S0 = torch.from_numpy(host_initial_state(0, wid, sh, 0.1)).cuda()
    cfg = rs.make_config(kind, precision, sh.B, sh.H, sh.P, sh.N, L, T)
    lay = rs.LayerState(cfg)
    lay.import_state(S0)
    outs = []
    for r in range(rounds):
        x = {k: torch.from_numpy(v).cuda() for k, v in host_step(0, wid, r, sh, T, decay="slow").items()}
        o = torch.empty((sh.B, T, sh.H, sh.P), device="cuda")
        if T == 1:
            if fused:
                rs.decode_step(cfg, lay.struct, x["alpha"], x["k"], x["v"], x.get("beta"), x["q"], o)
            else:
                rs.append(cfg, lay.struct, 1, x["alpha"], x["k"], x["v"], x.get("beta"))
                rs.decode(cfg, lay.struct, x["q"], o)
        else:
            if fused:
                rs.verify_step(cfg, lay.struct, T, x["alpha"], x["k"], x["v"], x.get("beta"), x["q"], o)
            else:
                rs.append(cfg, lay.struct, T, x["alpha"], x["k"], x["v"], x.get("beta"))
                rs.verify(cfg, lay.struct, T, x["q"], o)
            rs.accept(cfg, lay.struct, torch.from_numpy(host_accept(0, wid, r, sh.B, T)).cuda())
        if r == rounds // 2:
            rs.flush(cfg, lay.struct)
        outs.append(o)
    torch.cuda.synchronize()
    assert rs.read_error(lay.struct) == 0
    return torch.stack(outs), lay


# (KDA layers keep an fp32 checkpoint only)
@pytest.mark.parametrize("kind,precision", [("mamba2", "fp32"), ("mamba2", "fp32_hp_bf16_lp"), ("gdn", "fp32"),
                                            ("gdn", "fp32_hp_bf16_lp"), ("kda", "fp32")])
@pytest.mark.parametrize("T,fused", [(1, False), (1, True), (4, True), (3, False)])
def test_one_and_two_tiles_bit_identical(kind, precision, T, fused, restore_tiling):
    P = 64 if kind == "mamba2" else 128
    sh = LayerShape(kind, 3, 5, P, 128)
    L = 5
    wid = 190 + T
    oa, la = _run(kind, precision, sh, L, T, fused, rs.TILES_ONE, wid, 14)
    ob, lb = _run(kind, precision, sh, L, T, fused, rs.TILES_TWO, wid, 14)
    assert torch.equal(oa, ob)
    for name in ("hp", "lp", "ring_alpha", "ring_beta", "ring_k", "ring_v", "ring_vraw", "head", "h", "p",
                 "folded", "err"):
        ta, tb = getattr(la, name), getattr(lb, name)
        assert (ta is None) == (tb is None), name
        if ta is not None:
            assert torch.equal(ta, tb), name
    assert la.pointers() == lb.pointers()
    assert la.pointers()["folded"][0] > 0


def test_auto_policy_switches_by_batch(restore_tiling):
    """Automatic tiling on both sides of the switch point (6 items per compute unit at
    dv = 128) gives the bits of the forced tilings."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for B in (2, -(-8 * cus // 4)):
        sh = LayerShape("gdn", B, 4, 128, 128)
        oa, _ = _run("gdn", "fp32", sh, 4, 1, True, rs.TILES_AUTO, 199, 6)
        ob, _ = _run("gdn", "fp32", sh, 4, 1, True, rs.TILES_ONE, 199, 6)
        oc, _ = _run("gdn", "fp32", sh, 4, 1, True, rs.TILES_TWO, 199, 6)
        assert torch.equal(oa, ob) and torch.equal(oa, oc)


def _run_device(w, precision, T, policy, rounds):
    """The full-size workload's layer on device-drawn inputs: decode steps (T = 1) or
    speculative rounds (fused verify, then a drawn accept), with folds."""
    import synth

    rs.set_tiling(policy)
    sh = w.shape
    cfg = rs.make_config(sh.kind, precision, sh.B, sh.H, sh.P, sh.N, w.L, T)
    lay = rs.LayerState(cfg)
    lay.import_state(synth.device_initial_state(0, w.wid, sh, w.s0_sigma, "cuda"))
    outs = torch.empty((rounds, sh.B, T, sh.H, sh.P), device="cuda")
    for r in range(rounds):
        x = synth.device_step(0, w.wid, 500 + r, sh, T, "cuda")
        if T == 1:
            rs.decode_step(cfg, lay.struct, x["alpha"], x["k"], x["v"], x.get("beta"), x["q"], outs[r])
        else:
            rs.verify_step(cfg, lay.struct, T, x["alpha"], x["k"], x["v"], x.get("beta"), x["q"], outs[r])
            rs.accept(cfg, lay.struct, synth.device_accept(0, w.wid, 500 + r, sh.B, T, "cuda"))
    torch.cuda.synchronize()
    assert rs.read_error(lay.struct) == 0
    return outs, lay


@pytest.mark.parametrize("wname,precision,T", [("mamba2_decode_b256", "fp32", 1),
                                                ("mamba2_decode_b256", "fp32_hp_bf16_lp", 4),
                                                ("gdn_decode_b256", "fp32_hp_bf16_lp", 4),
                                                ("kda_decode_b256", "fp32", 4)])
def test_full_size_layers_bit_identical(wname, precision, T, restore_tiling):
    """At the benchmark's B = 256 shapes (where the automatic choice is two tiles) the forced
    one-tile kernels give the same bits: outputs of every round, both checkpoint copies after
    the folds, rings and pointers."""
    import synth

    w = synth.WORKLOADS[wname]
    rounds = 20 if T == 1 else 12
    oa, la = _run_device(w, precision, T, rs.TILES_ONE, rounds)
    ob, lb = _run_device(w, precision, T, rs.TILES_AUTO, rounds)
    assert torch.equal(oa, ob)
    for name in ("hp", "lp", "ring_alpha", "ring_beta", "ring_k", "ring_v", "ring_vraw", "head", "h", "p", "folded"):
        ta, tb = getattr(la, name), getattr(lb, name)
        if ta is not None:
            assert torch.equal(ta, tb), name
    assert la.pointers() == lb.pointers()
    assert max(la.pointers()["folded"]) > 0
