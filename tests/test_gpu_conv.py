"""The input-side convolution kept as an input ring, on the GPU, against the oracle.

replayssm_conv_step / replayssm_conv_accept (through the C ABI) against oracle/conv.py,
which convolves each sequence's whole committed history in fp64. Checked every step:
the outputs (normwise relative error per (sequence, input) vector <= 1e-5: at most
four fp32 products, a bias and SiLU), the window the ring holds (bit-exact copies of
the committed inputs, zeros before the first token), and the start / pending
pointers (exact, from the rule start += accepted, mod W - 1 + T_max).
"""
import numpy as np
import pytest
import torch

import ssm_decode_amd as rs
from oracle.conv import ConvOracle
from synth import host_accept, host_conv_inputs, host_conv_params

pytestmark = pytest.mark.gpu

TOL = 1e-5


def _rel(got, ref):
    num = np.abs(got.astype(np.float64) - ref).max(axis=-1)
    return num / np.maximum(np.abs(ref).max(axis=-1), 1e-30)


class ConvRun:
    def __init__(self, B, D, W, T_max, wid, silu=True, bias=True):
        self.cfg = rs.make_conv_config(B, D, W, T_max)
        self.layer = rs.ConvLayer(self.cfg)
        self.oracle = ConvOracle(B, D, W)
        w, b = host_conv_params(0, wid, D, W)
        self.w_host, self.b_host = w, (b if bias else None)
        self.w = torch.from_numpy(w).cuda()
        self.b = torch.from_numpy(b).cuda() if bias else None
        self.silu, self.wid, self.step_id = silu, wid, 0
        self.start = np.zeros(B, np.int64)
        self.Cc = W - 1 + T_max
        self.max_rel = 0.0

    def step(self, T, commit):
        cfg = self.cfg
        x_host = host_conv_inputs(0, self.wid, self.step_id, cfg.B, T, cfg.D)
        self.step_id += 1
        x = torch.from_numpy(x_host).cuda()
        y = torch.empty_like(x)
        rs.conv_step(cfg, self.layer.struct, T, x, self.w, self.b, self.silu, commit, y)
        ref = self.oracle.step(x_host, self.w_host, self.b_host, self.silu, commit=commit)
        self.max_rel = max(self.max_rel, float(_rel(y.cpu().numpy(), ref).max()))
        if commit:
            self.start = (self.start + T) % self.Cc
        self.check(pend=0 if commit else T)

    def accept(self, a_host):
        rs.conv_accept(self.cfg, self.layer.struct, torch.from_numpy(a_host).cuda())
        self.oracle.accept(a_host)
        self.start = (self.start + a_host) % self.Cc
        self.check(pend=0)

    def check(self, pend):
        cfg = self.cfg
        torch.cuda.synchronize()
        np.testing.assert_array_equal(self.layer.start.cpu().numpy(), self.start)
        np.testing.assert_array_equal(self.layer.pend.cpu().numpy(), np.full(cfg.B, pend))
        ring = self.layer.ring.cpu().numpy()
        for b in range(cfg.B):
            win = np.stack([ring[b, (self.start[b] + j) % self.Cc] for j in range(cfg.W - 1)]) if cfg.W > 1 \
                else np.zeros((0, cfg.D), np.float32)
            np.testing.assert_array_equal(win, self.oracle.window(b).astype(np.float32))


@pytest.mark.parametrize("W", [1, 2, 3, 4])
def test_standard_decoding(W):
    r = ConvRun(3, 64, W, 1, wid=80 + W)
    for _ in range(12):
        r.step(1, commit=True)
    assert r.max_rel <= TOL, r.max_rel
    assert int(r.layer.err[0].item()) == 0


@pytest.mark.parametrize("W,T_max,T", [(4, 4, 4), (4, 4, 2), (2, 8, 8), (3, 8, 5), (1, 4, 3)])
@pytest.mark.parametrize("silu", [True, False])
def test_speculative_rounds(W, T_max, T, silu):
    r = ConvRun(4, 128, W, T_max, wid=90 + W, silu=silu)
    for rnd in range(15):
        r.step(T, commit=False)
        r.accept(host_accept(0, 90 + W, rnd, 4, T))
    assert r.max_rel <= TOL, r.max_rel
    assert int(r.layer.err[0].item()) == 0


def test_layer_width_channels_and_no_bias():
    """A Mamba-2 layer's channel count (x plus B and C: 8192 + 2 x 128 x 128), many channel blocks."""
    r = ConvRun(2, 40960, 4, 4, wid=97, bias=False)
    for rnd in range(5):
        r.step(4, commit=False)
        r.accept(host_accept(0, 97, rnd, 2, 4))
    r.step(1, commit=True)
    assert r.max_rel <= TOL, r.max_rel


def test_contract_violations_are_flagged_and_skipped():
    r = ConvRun(2, 32, 4, 4, wid=98)
    r.step(2, commit=False)
    ring_before = r.layer.ring.clone()
    # a second step while inputs are pending: every sequence is skipped and flagged
    x = torch.ones((2, 2, 32), device="cuda")
    y = torch.zeros_like(x)
    rs.conv_step(r.cfg, r.layer.struct, 2, x, r.w, r.b, True, False, y)
    torch.cuda.synchronize()
    assert torch.equal(r.layer.ring, ring_before)
    assert torch.count_nonzero(y) == 0
    assert int(r.layer.err[0].item()) & rs.DEVERR_PENDING
    # accepting more than is pending is clamped to the pending count
    rs.conv_accept(r.cfg, r.layer.struct, torch.tensor([5, 1], dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert int(r.layer.err[0].item()) & rs.DEVERR_ACCEPT
    np.testing.assert_array_equal(r.layer.start.cpu().numpy(), [2, 1])
    np.testing.assert_array_equal(r.layer.pend.cpu().numpy(), [0, 0])


def test_committing_several_inputs_at_once():
    """commit with T > 1 (several tokens in one call, e.g. a prompt's tail), mixed with rounds."""
    r = ConvRun(3, 96, 4, 4, wid=99)
    for rnd in range(8):
        r.step(4 if rnd % 2 == 0 else 3, commit=True)
        r.step(4, commit=False)
        r.accept(host_accept(0, 99, rnd, 3, 4))
    assert r.max_rel <= TOL, r.max_rel
    assert int(r.layer.err[0].item()) == 0
