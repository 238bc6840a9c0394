"""replayssm_append_dt: the records' decay computed on the GPU from the raw time step.

Each run appends through replayssm_append_dt (alpha = exp(-softplus(dt + dt_bias) A)
per record, fp32 on the GPU) while the oracle appends the decay it computes itself
from the same dt, A and dt_bias (oracle/decay.py, fp64, rounded to fp32 as the
oracle's records are). Checked: the decay written to every ring slot against the
oracle's, k and v copied bit for bit, pointers exact, and every output against
the oracle at 1e-4.

Decay tolerance: the GPU forms y = softplus(x) A and exp(-y) in fp32, each step
within a few ulp (2^-23 ~ 1.2e-7); the relative error of exp(-y) is about y times
the relative error of y, with y <= 12 for these inputs, so |da| / a <= 12 * 3 ulp
+ 2 ulp < 5e-6; the bar is 1e-5.
"""
import numpy as np
import pytest
import torch

import ssm_decode_amd as rs
from harness import Runner, rel_err
from oracle.decay import alpha_from_dt
from synth import LayerShape, host_accept, host_decay_params, host_time_steps

pytestmark = pytest.mark.gpu

ALPHA_RTOL = 1e-5


class DtRunner(Runner):
    """A Runner whose appends go through replayssm_append_dt."""

    def __init__(self, *args, bias=True, **kw):
        super().__init__(*args, **kw)
        A, b = host_decay_params(self.seed, self.wid, self.shape)
        self.A_host, self.bias_host = A, (b if bias else None)
        self.A = torch.from_numpy(A).cuda()
        self.bias = torch.from_numpy(b).cuda() if bias else None
        self.max_alpha_rel = 0.0

    def append_dt(self, x, T):
        dt_host = host_time_steps(self.seed, self.wid, self.step_id - 1, self.shape, T)
        dt = torch.from_numpy(dt_host).cuda()
        beta = x.get("beta")
        rs.append_dt(self.cfg, self.layer.struct, T, dt, self.A, self.bias, x["k"], x["v"], beta)
        hs = np.array([h for _, h in self.heads])
        alpha_ref = alpha_from_dt(self._sel(dt), self.A_host[hs][:, None],
                                  None if self.bias_host is None else self.bias_host[hs][:, None])  # [nh, T]
        slots = self.oracle.append(alpha_ref.astype(np.float32), self._sel(x["k"]), self._sel(x["v"]),
                                   None if beta is None else self._sel(beta))
        self._slots = slots
        sl = torch.tensor([[slots[b][i] for i in range(T)] for b, _ in self.heads], device="cuda")
        for i in range(T):
            got_a = self.layer.ring_alpha[self.bs, self.hs, sl[:, i]].cpu().numpy().astype(np.float64)
            self.max_alpha_rel = max(self.max_alpha_rel,
                                     float(np.max(np.abs(got_a - alpha_ref[:, i]) / alpha_ref[:, i])))
            ok = torch.equal(self.layer.ring_k[self.bs, self.hs, sl[:, i]], x["k"][self.bs, i, self.hs])
            if beta is None:
                ok = ok and torch.equal(self.layer.ring_v[self.bs, self.hs, sl[:, i]], x["v"][self.bs, i, self.hs])
            else:
                ok = ok and torch.equal(self.layer.ring_beta[self.bs, self.hs, sl[:, i]], beta[self.bs, i, self.hs])
            if not ok:
                self.report.ring_mismatch += 1


def run_dt_standard(r: DtRunner, steps: int):
    for _ in range(steps):
        x = r.inputs(1)
        r.append_dt(x, 1)
        r.decode(x)
        r.check_pointers()
    r.check_checkpoint("hp")
    r.error_word()
    return r.report


def run_dt_spec(r: DtRunner, T: int, rounds: int):
    for rnd in range(rounds):
        x = r.inputs(T)
        r.append_dt(x, T)
        r.verify(x, T)
        r.accept(torch.from_numpy(host_accept(r.seed, r.wid, rnd, r.shape.B, T)).cuda())
        r.check_pointers()
    r.check_checkpoint("hp")
    r.error_word()
    return r.report


def _ok(r, rep):
    assert rep.pointer_mismatch == 0 and rep.ring_mismatch == 0 and rep.err_word == 0, rep
    assert r.max_alpha_rel <= ALPHA_RTOL, r.max_alpha_rel
    assert rep.max_rel <= 1e-4 and rep.max_rel_ckpt <= 1e-4, rep


@pytest.mark.parametrize("bias", [True, False])
def test_mamba2_tiny_standard(bias):
    r = DtRunner(LayerShape("mamba2", 1, 2, 16, 16), 4, 1, wid=40, bias=bias)
    rep = run_dt_standard(r, 24)
    _ok(r, rep)
    assert rep.folds >= 4


def test_mamba2_layer_standard_with_folds():
    r = DtRunner(LayerShape("mamba2", 8, 16, 64, 128), 16, 1, wid=41)
    rep = run_dt_standard(r, 40)
    _ok(r, rep)
    assert rep.folds > 0


def test_mamba2_two_precision_spec():
    r = DtRunner(LayerShape("mamba2", 4, 8, 64, 128), 16, 4, precision="fp32_hp_bf16_lp", wid=42)
    rep = run_dt_spec(r, 4, 24)
    assert rep.pointer_mismatch == 0 and rep.ring_mismatch == 0 and rep.err_word == 0, rep
    assert r.max_alpha_rel <= ALPHA_RTOL
    assert rep.max_rel_ckpt <= 1e-4  # the fp32 checkpoint carries the exact recurrence
    assert rep.max_rel_token <= 2e-2, rep  # token outputs with the bf16 copy read off-fold
    assert rep.mag_vectors > 0 and rep.max_rel_mag <= 2e-2, rep  # every head, against its terms' magnitudes


@pytest.mark.parametrize("precision", ["fp32", "fp32_hp_bf16_lp"])
def test_gdn_spec(precision):
    r = DtRunner(LayerShape("gdn", 4, 4, 128, 128), 16, 4, precision=precision, wid=43)
    rep = run_dt_spec(r, 4, 24)
    assert r.max_alpha_rel <= ALPHA_RTOL
    assert rep.pointer_mismatch == 0 and rep.ring_mismatch == 0 and rep.err_word == 0, rep
    assert rep.max_rel_ckpt <= 1e-4, rep
    if precision == "fp32":
        assert rep.max_rel <= 1e-4 and rep.max_rel_u <= 1e-4, rep
    else:
        assert rep.max_rel_token <= 2e-2 and rep.mag_vectors > 0 and rep.max_rel_mag <= 2e-2, rep


def test_extreme_time_steps():
    """dt far below zero gives alpha = 1 exactly (softplus underflows to 0); far above, alpha = 0
    exactly (exp of a huge negative number); the ring holds exactly the oracle's fp32 values and
    the outputs stay within the bar."""
    sh = LayerShape("mamba2", 2, 4, 16, 32)
    r = DtRunner(sh, 4, 1, wid=44, bias=False)
    hs = [h for _, h in r.heads]
    for t in range(10):
        x = r.inputs(1)
        dt = torch.full((sh.B, 1, sh.H), -200.0 if t % 2 else 1.0e4, device="cuda")
        rs.append_dt(r.cfg, r.layer.struct, 1, dt, r.A, None, x["k"], x["v"])
        alpha_ref = alpha_from_dt(r._sel(dt), r.A_host[hs][:, None]).astype(np.float32)
        assert np.all(alpha_ref == (1.0 if t % 2 else 0.0))
        slots = r.oracle.append(alpha_ref, r._sel(x["k"]), r._sel(x["v"]), None)
        sl = torch.tensor([slots[b][0] for b, _ in r.heads], device="cuda")
        got = r.layer.ring_alpha[r.bs, r.hs, sl].cpu().numpy()
        np.testing.assert_array_equal(got, alpha_ref[:, 0])
        r.decode(x)
    r.check_pointers()
    r.error_word()
    assert r.report.pointer_mismatch == 0 and r.report.err_word == 0
    assert r.report.max_rel <= 1e-4, r.report
