"""The benchmark's byte model (the numerator of every roofline figure), pinned to the
per-head figures worked out by hand from the layouts:

  Mamba-2 record (alpha, k, v) = 4 + 4N + 4P = 772 B at P = 64, N = 128; q in 512 B, out 256 B;
  a plain decode step with h committed records reads the 32 KiB checkpoint, h + 1 records and
  q, and writes the output: 32,768 + 772 (h + 1) + 768; a fold step adds the 32 KiB write.
  Eager: state load + store (65,536) + record, q and output (1,540) = 67,076 per token.
"""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

P, N = 64, 128


def test_record_sizes():
    assert bench.record_bytes("mamba2", P, N) == 772
    assert bench.record_bytes("gdn", 128, 128) == 4 + 512 + 512 + 4
    assert bench.record_bytes("kda", 128, 128) == 512 + 512 + 512 + 4


@pytest.mark.parametrize("h", [0, 1, 7, 15])
def test_mamba2_plain_decode_step(h):
    assert bench.replay_launch_bytes("mamba2", "fp32", P, N, h, 1, False) == 32768 + 772 * (h + 1) + 768


def test_mamba2_fold_step_and_window_average():
    fold = bench.replay_launch_bytes("mamba2", "fp32", P, N, 16, 1, True)
    assert fold == 32768 + 772 * 17 + 768 + 32768
    # steady state: h before the step cycles 16 (fold), 1, ..., 15
    cycle = [fold] + [bench.replay_launch_bytes("mamba2", "fp32", P, N, h, 1, False) for h in range(1, 16)]
    assert sum(cycle) / 16 == 32768 + 768 + 772 * (sum(range(2, 17)) + 17) / 16 + 32768 / 16
    # one B=256 H=128 launch averages 1.37-1.41 GB over the cycle
    assert 1.37e9 < sum(cycle) / 16 * 256 * 128 < 1.41e9


def test_two_precision_reads_the_bf16_copy_off_fold():
    plain = bench.replay_launch_bytes("mamba2", "fp32_hp_bf16_lp", P, N, 5, 1, False)
    assert plain == 16384 + 772 * 6 + 768
    fold = bench.replay_launch_bytes("mamba2", "fp32_hp_bf16_lp", P, N, 16, 1, True)
    assert fold == 32768 + 772 * 17 + 768 + 32768 + 16384  # fp32 read, both copies written


def test_verify_round_counts_the_drafts():
    # T = 4 drafts: 4 records beyond the h committed ones, 4 q rows in, 4 outputs out
    assert bench.replay_launch_bytes("mamba2", "fp32", P, N, 3, 4, False) == 32768 + 772 * 7 + 4 * 512 + 4 * 256
    # GDN also writes each draft's correction u back into the ring
    g = bench.replay_launch_bytes("gdn", "fp32", 128, 128, 3, 4, False)
    assert g == 65536 + 1032 * 7 + 4 * 512 + 4 * 512 + 4 * 512


def test_eager_and_flush():
    assert bench.eager_bytes("mamba2", P, N, 1, False) == 67076
    assert bench.eager_bytes("gdn", 128, 128, 1, False) == 133128
    # a standalone flush of 16 records: checkpoint read, the records, checkpoint write
    assert bench.flush_launch_bytes("mamba2", "fp32", P, N, 16) == 32768 + 16 * 772 + 32768
    assert bench.flush_launch_bytes("mamba2", "fp32", P, N, 16) * 256 * 128 == 2552233984
    # GDN folds stage no beta; with the two-precision checkpoint they stage raw v and beta
    assert bench.flush_launch_bytes("gdn", "fp32", 128, 128, 16) == 65536 + 16 * 1028 + 65536
    assert bench.flush_launch_bytes("gdn", "fp32_hp_bf16_lp", 128, 128, 16) == 65536 + 16 * 1032 + 65536 + 32768


def test_state_byte_ratio_against_eager():
    # checkpoint read every step plus one write per 16-token window, against a load and a store per token
    replay_state = 4 * P * N * (1 + 1 / 16)
    assert round(2 * 4 * P * N / replay_state, 2) == 1.88


def test_conv_ring_bytes():
    # window of W - 1 inputs read, T inputs read and written to the ring, T outputs written
    assert bench.conv_launch_bytes(40960, 4, 1) == 4 * 40960 * 6
    assert bench.conv_launch_bytes(40960, 4, 4) == 4 * 40960 * 15
