"""Parity at the full sizes of the workloads, in the launch configuration bench.py times.

The GPU runs every head of the layer; the oracle follows a sample of heads
exactly (heads are independent), including the first and the last head of the
layer. Every step's sampled outputs are compared; the pointer arrays of all
sequences are compared bit for bit every few steps; the ring copies of the
sampled heads after every append; the checkpoint at the end.
"""
import pytest
import torch

from synth import LayerShape, WORKLOADS

from harness import Runner, run_spec, run_standard, sample_heads, whole_sequences

pytestmark = pytest.mark.gpu

TOL = 1e-4
TOL_LP = 2e-2


def _clean(rep, tol=TOL, tol_ckpt=TOL):
    assert rep.pointer_mismatch == 0, (rep.final_pointers, rep.oracle_pointers)
    assert rep.ring_mismatch == 0
    assert rep.err_word == 0
    assert rep.max_rel <= tol, rep.max_rel
    assert rep.max_rel_ckpt <= tol_ckpt, rep.max_rel_ckpt
    assert rep.max_rel_u <= tol, rep.max_rel_u


def test_mamba2_decode_b256_512_steps():
    """B=256, H=128, P=64, N=128, L=16: 512 standard steps, 31 folds per sequence."""
    w = WORKLOADS["mamba2_decode_b256"]
    sh = w.shape
    r = Runner(sh, w.L, 1, wid=w.wid, heads=sample_heads(sh.B, sh.H, 48), gen="device", s0_sigma=w.s0_sigma)
    rep = run_standard(r, w.steps, check_every=16)
    _clean(rep)
    assert rep.final_pointers["folded"] == [496] * sh.B and rep.final_pointers["h"] == [16] * sh.B
    assert rep.final_pointers["head"] == [3] * sh.B


def test_mamba2_decode_step_b256_512_steps():
    """The fused append + decode launch the benchmark times, at full size."""
    w = WORKLOADS["mamba2_decode_b256"]
    sh = w.shape
    r = Runner(sh, w.L, 1, wid=w.wid + 200, heads=sample_heads(sh.B, sh.H, 48), gen="device", s0_sigma=w.s0_sigma)
    rep = run_standard(r, w.steps, check_every=16, fused=True)
    _clean(rep)
    assert rep.final_pointers["folded"] == [496] * sh.B and rep.final_pointers["h"] == [16] * sh.B


def test_mamba2_spec_b256_256_rounds():
    """Same layer, T=4 drafts, C=20, accepted prefix uniform in 0..4, 256 rounds."""
    w = WORKLOADS["mamba2_spec_b256"]
    sh = w.shape
    r = Runner(sh, w.L, w.T, wid=w.wid, heads=sample_heads(sh.B, sh.H, 48), gen="device", s0_sigma=w.s0_sigma)
    rep = run_spec(r, w.T, w.steps, check_every=8)
    _clean(rep)
    assert rep.folds > 0


def test_gdn_b256_standard_512_steps():
    w = WORKLOADS["gdn_decode_b256"]
    sh = w.shape
    r = Runner(sh, w.L, 1, wid=w.wid, heads=sample_heads(sh.B, sh.H, 32), gen="device", s0_sigma=w.s0_sigma)
    rep = run_standard(r, w.steps, check_every=16)
    _clean(rep)


def test_gdn_b256_verify_T4():
    w = WORKLOADS["gdn_decode_b256"]
    sh = w.shape
    r = Runner(sh, w.L, 4, wid=w.wid + 100, heads=sample_heads(sh.B, sh.H, 32), gen="device", s0_sigma=w.s0_sigma)
    rep = run_spec(r, 4, 128, check_every=8)
    _clean(rep)


def test_mamba2_two_precision_b256_1024_rounds():
    """T=4, 1024 speculative rounds of the two-precision layer, next to the shared-bf16 comparison.

    Two-precision: each token's layer output within 2e-2 of the fp32 oracle (every head of the
    followed sequences), and the fp32 checkpoint still the exact recurrence (1e-4). Shared bf16:
    its drift is reported; it must exceed the two-precision drift (its rounding enters the
    recurrence at every fold) and stay sane."""
    w = WORKLOADS["mamba2_2prec_b256"]
    sh = w.shape
    heads = whole_sequences(sh.B, sh.H, [0, 97, sh.B - 1])
    drift = {}
    for precision in ("fp32_hp_bf16_lp", "bf16_shared"):
        r = Runner(sh, w.L, w.T, precision=precision, wid=w.wid, heads=heads, gen="device",
                   s0_sigma=w.s0_sigma, check_ring=False)
        rep = run_spec(r, w.T, w.steps, check_every=32)
        assert rep.pointer_mismatch == 0 and rep.err_word == 0
        drift[precision] = {"token": rep.max_rel_token, "per_head": rep.max_rel, "ckpt": rep.max_rel_ckpt}
    print("max drift vs the fp32 oracle:", drift)
    assert drift["fp32_hp_bf16_lp"]["token"] <= TOL_LP, drift
    assert drift["fp32_hp_bf16_lp"]["ckpt"] <= TOL, drift
    assert drift["bf16_shared"]["token"] < 0.1, drift
    assert drift["bf16_shared"]["token"] > drift["fp32_hp_bf16_lp"]["token"], drift


@pytest.mark.parametrize("B", [1, 32, 512])
def test_two_precision_batch_sweep(B):
    w = WORKLOADS["mamba2_2prec_b256"]
    sh = LayerShape("mamba2", B, 128, 64, 128)
    r = Runner(sh, w.L, w.T, precision="fp32_hp_bf16_lp", wid=w.wid + B, heads=whole_sequences(B, 128, [0, B - 1]),
               gen="device", s0_sigma=w.s0_sigma, check_ring=False)
    rep = run_spec(r, w.T, 64, check_every=8)
    print(f"B={B}: token drift {rep.max_rel_token:.3e}, per-head max {rep.max_rel:.3e}")
    assert rep.pointer_mismatch == 0 and rep.err_word == 0
    assert rep.max_rel_token <= TOL_LP
    assert rep.max_rel_ckpt <= TOL
