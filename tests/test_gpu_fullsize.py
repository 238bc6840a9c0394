"""Parity at the full sizes of the workloads, in the launch configuration bench.py times.

The GPU runs every head of the layer; the oracle follows a sample of heads
exactly (heads are independent), including the first and the last head of the
layer. Every step's sampled outputs are compared; the pointer arrays of all
sequences are compared bit for bit every few steps; the ring copies of the
sampled heads after every append; the checkpoint at the end.
"""
import json
import os

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


def _drift_out(name, data):
    """Writes a drift summary as JSON when REPLAYSSM_DRIFT_OUT names a directory."""
    d = os.environ.get("REPLAYSSM_DRIFT_OUT")
    if d:
        os.makedirs(d, exist_ok=True)
        with open(os.path.join(d, f"{name}.json"), "w") as f:
            json.dump(data, f, indent=1)


def test_mamba2_two_precision_b256_1024_rounds():
    """T=4, 1024 speculative rounds of the two-precision layer, beside the shared-bf16 and fp32
    checkpoints on the same inputs ("How it works": Two precisions).

    Every head's output of every draft of three whole sequences is compared with the fp64 oracle:
    with a bf16 copy read (both bf16 modes) the error stays within 2e-2 of the magnitudes of the
    terms the output sums, per head; the two-precision token outputs within 2e-2 of the token's
    size, and its fp32 checkpoint remains the exact recurrence (1e-4); the fp32 mode within 1e-4
    per head. The shared-bf16 drift must exceed the two-precision drift (its rounding enters the
    recurrence at every fold)."""
    w = WORKLOADS["mamba2_2prec_b256"]
    sh = w.shape
    heads = whole_sequences(sh.B, sh.H, [0, 97, sh.B - 1])
    drift = {}
    for precision in ("fp32_hp_bf16_lp", "bf16_shared", "fp32"):
        r = Runner(sh, w.L, w.T, precision=precision, wid=w.wid, heads=heads, gen="device",
                   s0_sigma=w.s0_sigma, check_ring=False, keep_all=True, magnitudes=True)
        rep = run_spec(r, w.T, w.steps, check_every=32)
        assert rep.pointer_mismatch == 0 and rep.err_word == 0
        assert rep.mag_vectors == len(heads) * w.T * w.steps
        drift[precision] = {**rep.drift_summary(), "checkpoint_max": rep.max_rel_ckpt, "folds": rep.folds,
                            "max_per_head_magnitude": rep.max_rel_mag, "max_per_head_guarded": rep.max_rel_guarded}
    print("drift vs the fp64 oracle:", json.dumps(drift))
    _drift_out("mamba2_b256_1024_rounds", {"B": sh.B, "rounds": w.steps, "T": w.T, "L": w.L,
                                           "followed_sequences": [0, 97, sh.B - 1], "modes": drift})
    two, shared, f32 = drift["fp32_hp_bf16_lp"], drift["bf16_shared"], drift["fp32"]
    # per head, against the magnitudes of the terms each output sums, in both bf16 modes
    assert two["max_per_head_magnitude"] <= TOL_LP and shared["max_per_head_magnitude"] <= TOL_LP, drift
    assert two["per_token"]["max"] <= TOL_LP, drift
    assert two["checkpoint_max"] <= TOL, drift
    # fp32: the plain per-head metric, guarded only on outputs 100x smaller than their terms
    assert f32["max_per_head_guarded"] <= TOL and f32["per_head"]["p99_9"] <= TOL / 10, drift
    assert f32["checkpoint_max"] <= TOL, drift
    assert shared["per_token"]["max"] < 0.1, drift
    assert shared["per_token"]["max"] > two["per_token"]["max"], drift


@pytest.mark.parametrize("B", [1, 32, 512])
def test_two_precision_batch_sweep(B):
    """The batch sweep of the two-precision layer (1024 rounds each, both bf16 modes): the kernel
    variant changes with the batch (one or two checkpoint tiles per wavefront), the bound does not."""
    w = WORKLOADS["mamba2_2prec_b256"]
    sh = LayerShape("mamba2", B, 128, 64, 128)
    seqs = [0, B - 1]
    drift = {}
    for precision in ("fp32_hp_bf16_lp", "bf16_shared"):
        r = Runner(sh, w.L, w.T, precision=precision, wid=w.wid + B, heads=whole_sequences(B, 128, seqs),
                   gen="device", s0_sigma=w.s0_sigma, check_ring=False, keep_all=True)
        rep = run_spec(r, w.T, w.steps, check_every=64)
        assert rep.pointer_mismatch == 0 and rep.err_word == 0
        assert rep.mag_vectors > 0 and rep.max_rel_mag <= TOL_LP, (precision, rep.max_rel_mag)
        drift[precision] = {**rep.drift_summary(), "checkpoint_max": rep.max_rel_ckpt,
                            "max_per_head_magnitude": rep.max_rel_mag}
    print(f"B={B}:", json.dumps(drift))
    _drift_out(f"mamba2_b{B}_1024_rounds", {"B": B, "rounds": w.steps, "T": w.T, "L": w.L,
                                            "followed_sequences": sorted(set(seqs)), "modes": drift})
    assert drift["fp32_hp_bf16_lp"]["per_token"]["max"] <= TOL_LP
    assert drift["fp32_hp_bf16_lp"]["checkpoint_max"] <= TOL
