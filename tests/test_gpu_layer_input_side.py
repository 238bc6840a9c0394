"""The input side and the path together, as a Mamba-2 layer's decode step calls them.

GPU: replayssm_conv_step on the input-projection channels -> the channels split per head
into x (the record's v), B (k) and C (q) -> replayssm_append_dt (each record's decay from
its raw time step) -> replayssm_decode / replayssm_verify -> acceptance applied to both the
SSM ring and the convolution ring. Oracle: the convolution over the whole history (fp64)
-> the same split -> the decay from the time step (fp64) -> the eager recurrence. The two
chains share only the seeded inputs; outputs are compared per head vector at 1e-4 (the
GPU's convolution outputs differ from the oracle's by ~1e-6 relative, far inside it),
pointers of both rings exactly.
"""
import numpy as np
import pytest
import torch

import ssm_decode_amd as rs
from oracle.conv import ConvOracle
from oracle.decay import alpha_from_dt
from oracle.session import OracleSession, select_heads
from synth import (LayerShape, host_accept, host_conv_inputs, host_conv_params, host_decay_params,
                   host_initial_state, host_time_steps)

pytestmark = pytest.mark.gpu


def _rel(got, ref):
    return np.abs(got.astype(np.float64) - ref).max(axis=-1) / np.maximum(np.abs(ref).max(axis=-1), 1e-30)


class LayerStep:
    def __init__(self, B, H, P, N, W, L, T_max, wid):
        self.B, self.H, self.P, self.N, self.W, self.wid = B, H, P, N, W, wid
        self.D = H * P + 2 * H * N
        shape = LayerShape("mamba2", B, H, P, N)
        self.cfg = rs.make_config("mamba2", "fp32", B, H, P, N, L, T_max)
        self.layer = rs.LayerState(self.cfg)
        S0 = host_initial_state(0, wid, shape, 0.1)
        self.layer.import_state(torch.from_numpy(S0).cuda())
        self.ccfg = rs.make_conv_config(B, self.D, W, T_max)
        self.conv = rs.ConvLayer(self.ccfg)
        self.heads = [(b, h) for b in range(B) for h in range(H)]
        self.ssm_oracle = OracleSession("mamba2", B, H, P, N, L, T_max, S0.reshape(B * H, P, N), self.heads)
        self.conv_oracle = ConvOracle(B, self.D, W)
        w, b = host_conv_params(0, wid, self.D, W)
        self.w_h, self.b_h = w, b
        self.w, self.b = torch.from_numpy(w).cuda(), torch.from_numpy(b).cuda()
        A, bias = host_decay_params(0, wid, shape)
        self.A_h, self.bias_h = A, bias
        self.A, self.bias = torch.from_numpy(A).cuda(), torch.from_numpy(bias).cuda()
        self.step_id = 0
        self.max_rel = 0.0

    def _split(self, y, T, lib):
        H, P, N, B = self.H, self.P, self.N, self.B
        v = y[..., :H * P].reshape(B, T, H, P)
        k = y[..., H * P:H * P + H * N].reshape(B, T, H, N)
        q = y[..., H * P + H * N:].reshape(B, T, H, N)
        if lib == "torch":
            return v.contiguous(), k.contiguous(), q.contiguous()
        return v, k, q

    def round(self, T, spec):
        B, H = self.B, self.H
        x_h = host_conv_inputs(0, self.wid, self.step_id, B, T, self.D)
        dt_h = host_time_steps(0, self.wid, self.step_id, LayerShape("mamba2", B, H, self.P, self.N), T)
        self.step_id += 1
        # GPU chain
        y = torch.empty((B, T, self.D), device="cuda")
        rs.conv_step(self.ccfg, self.conv.struct, T, torch.from_numpy(x_h).cuda(), self.w, self.b, True, not spec, y)
        v, k, q = self._split(y, T, "torch")
        rs.append_dt(self.cfg, self.layer.struct, T, torch.from_numpy(dt_h).cuda(), self.A, self.bias, k, v)
        out = torch.empty((B, T, H, self.P), device="cuda")
        if spec:
            rs.verify(self.cfg, self.layer.struct, T, q, out)
        else:
            rs.decode(self.cfg, self.layer.struct, q, out)
        # oracle chain
        y_o = self.conv_oracle.step(x_h, self.w_h, self.b_h, True, commit=not spec).astype(np.float32)
        v_o, k_o, q_o = self._split(y_o, T, "numpy")
        alpha_o = alpha_from_dt(dt_h, self.A_h, self.bias_h).astype(np.float32)  # [B, T, H]
        self.ssm_oracle.append(select_heads(alpha_o, self.heads), select_heads(k_o, self.heads),
                               select_heads(v_o, self.heads))
        if spec:
            ref, _, _ = self.ssm_oracle.verify(select_heads(q_o, self.heads))
        else:
            ref, _, _ = self.ssm_oracle.decode(select_heads(q_o, self.heads))
        got = select_heads(out.cpu().numpy(), self.heads)
        self.max_rel = max(self.max_rel, float(_rel(got, ref).max()))

    def accept(self, a_h):
        a = torch.from_numpy(a_h).cuda()
        rs.accept(self.cfg, self.layer.struct, a)
        rs.conv_accept(self.ccfg, self.conv.struct, a)
        self.ssm_oracle.accept(a_h)
        self.conv_oracle.accept(a_h)

    def check(self):
        assert self.layer.pointers() == self.ssm_oracle.pm.snapshot()
        assert rs.read_error(self.layer.struct) == 0 and int(self.conv.err[0].item()) == 0
        assert int(self.conv.pend.abs().sum().item()) == 0


def test_standard_decoding_through_the_input_side():
    s = LayerStep(2, 3, 16, 16, 4, 4, 1, wid=110)
    for _ in range(20):
        s.round(1, spec=False)
    s.check()
    assert s.max_rel <= 1e-4, s.max_rel


@pytest.mark.parametrize("T", [2, 4])
def test_speculative_rounds_through_the_input_side(T):
    s = LayerStep(3, 2, 32, 16, 4, 8, 4, wid=111 + T)
    for rnd in range(14):
        s.round(T, spec=True)
        s.accept(host_accept(0, 111 + T, rnd, 3, T))
    s.check()
    assert s.max_rel <= 1e-4, s.max_rel
