"""replayssm_append_static (the append whose arrival counters live in the library's
own device array, for callers that cannot allocate) against replayssm_append.

Two layers start from the same state; one is fed through replayssm_append with its
state's scratch array, the other through replayssm_append_static with st->arrive set
to NULL. After every append the rings and pointers must be bit-identical, and the
outputs of the verify that follows (the same kernel on identical state) too. Two
calls in a row of the static variant, the second on a smaller layer, check that the
counters the first call left behind do not leak into the next.
"""
import pytest
import torch

import ssm_decode_amd as rs
from synth import LayerShape, host_accept, host_initial_state, host_step

pytestmark = pytest.mark.gpu


def _without_scratch(st):
    s = rs.State(*[getattr(st, name) for name, _ in rs.State._fields_])
    s.arrive = None
    return s


def _rings(lay):
    xs = [lay.ring_alpha, lay.ring_k, lay.ring_v, lay.h, lay.p, lay.head, lay.folded, lay.err]
    if lay.ring_beta is not None:
        xs.append(lay.ring_beta)
    return xs


def _run_pair(kind, B, T, rounds, wid):
    sh = LayerShape(kind, B, 6, 64, 128)
    L = 8
    cfg = rs.make_config(kind, "fp32", B, sh.H, sh.P, sh.N, L, T)
    ref, sta = rs.LayerState(cfg), rs.LayerState(cfg)
    S0 = torch.from_numpy(host_initial_state(3, wid, sh, 0.1)).cuda()
    ref.import_state(S0)
    sta.import_state(S0)
    st_static = _without_scratch(sta.struct)
    assert st_static.arrive is None
    out_r = torch.empty((B, T, sh.H, sh.P), device="cuda")
    out_s = torch.empty_like(out_r)
    for rnd in range(rounds):
        x = {k: torch.from_numpy(v).cuda() for k, v in host_step(3, wid, rnd, sh, T).items()}
        rs.append(cfg, ref.struct, T, x["alpha"], x["k"], x["v"], x.get("beta"))
        rs.append_static(cfg, st_static, T, x["alpha"], x["k"], x["v"], x.get("beta"))
        torch.cuda.synchronize()
        for a, b in zip(_rings(ref), _rings(sta)):
            assert torch.equal(a, b), (kind, B, rnd)
        assert int(sta.p[0].item()) == T
        rs.verify(cfg, ref.struct, T, x["q"], out_r)
        rs.verify(cfg, sta.struct, T, x["q"], out_s)
        assert torch.equal(out_r, out_s), (kind, B, rnd)
        acc = torch.from_numpy(host_accept(3, wid, rnd, B, T)).cuda()
        rs.accept(cfg, ref.struct, acc)
        rs.accept(cfg, sta.struct, acc)
    torch.cuda.synchronize()
    assert rs.read_error(ref.struct) == 0 and rs.read_error(sta.struct) == 0
    # the caller's own scratch array of the static layer was never touched
    assert int(sta.arrive.abs().sum().item()) == 0


@pytest.mark.parametrize("kind", ["mamba2", "gdn", "kda"])
def test_static_append_equals_append_on_two_calls_in_a_row(kind):
    _run_pair(kind, 48, 4, 6, 901)   # a larger layer first
    _run_pair(kind, 5, 2, 6, 902)    # then a smaller one on the same device array
