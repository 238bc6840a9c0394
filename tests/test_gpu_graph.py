"""Speculative rounds captured once in a HIP graph and replayed.

Small batches are launch-bound (a B=1 round is three launches of a few microseconds),
so a serving loop captures its rounds (torch.cuda.CUDAGraph around the library's calls
on the capture stream) and replays them. Every replay must leave the layer exactly as
the same calls made eagerly leave a twin layer: outputs, both checkpoint copies, the
rings and the pointers, bit for bit. Replays are interleaved with the twin's eager work
and with synchronisations, and each one is checked.
"""
import pytest
import torch

import ssm_decode_amd as rs
from synth import LayerShape, device_accept, device_initial_state, device_step

pytestmark = pytest.mark.gpu


def _layer(cfg, shape, seed, wid):
    lay = rs.LayerState(cfg)
    lay.import_state(device_initial_state(seed, wid, shape, 0.1, "cuda"))
    return lay


@pytest.mark.parametrize("kind,precision,B,H,P,N", [
    ("mamba2", "fp32", 1, 8, 64, 128),
    ("mamba2", "fp32_hp_bf16_lp", 32, 8, 64, 128),
    ("gdn", "fp32", 2, 4, 128, 128),
    ("gdn", "fp32_hp_bf16_lp", 2, 4, 128, 128),
    ("kda", "fp32", 2, 4, 128, 128),
])
def test_graph_replays_equal_eager_rounds(kind, precision, B, H, P, N):
    shape = LayerShape(kind, B, H, P, N)
    L, T, K, wid = 16, 4, 6, 61
    cfg = rs.make_config(kind, precision, B, H, P, N, L, T)
    g_lay, e_lay, warm = (_layer(cfg, shape, 0, wid) for _ in range(3))
    xs = [device_step(0, wid, 700 + r, shape, T, "cuda") for r in range(K)]
    accs = [device_accept(0, wid, r, B, T, "cuda") for r in range(K)]
    outs_g = [torch.zeros((B, T, H, P), device="cuda") for _ in range(K)]
    outs_e = [torch.zeros_like(o) for o in outs_g]

    def rounds(lay, outs):
        for r in range(K):
            x = xs[r]
            rs.verify_step(cfg, lay.struct, T, x["alpha"], x["k"], x["v"], x.get("beta"), x["q"], outs[r])
            rs.accept(cfg, lay.struct, accs[r])

    # first launches outside the capture (the library caches its occupancy queries then)
    rounds(warm, [torch.zeros_like(o) for o in outs_g])
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(graph, stream=side):
        rounds(g_lay, outs_g)
    torch.cuda.synchronize()
    assert int(g_lay.p.abs().sum().item()) == 0 and int(g_lay.h.abs().sum().item()) == 0  # capture ran nothing

    for rep in range(4):
        graph.replay()
        rounds(e_lay, outs_e)
        torch.cuda.synchronize()
        for r in range(K):
            assert torch.equal(outs_g[r], outs_e[r]), (rep, r)
        for name in ("hp", "lp", "ring_alpha", "ring_beta", "ring_k", "ring_v", "ring_vraw", "head", "h", "p",
                     "folded", "err"):
            a, b = getattr(g_lay, name), getattr(e_lay, name)
            if a is not None:
                assert torch.equal(a, b), (rep, name)
        torch.zeros(1024, device="cuda").add_(1.0)  # unrelated eager work between replays
    assert rs.read_error(g_lay.struct) == 0
    assert int(g_lay.folded.sum().item()) > 0  # the replays crossed folds
