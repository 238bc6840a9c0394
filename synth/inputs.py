"""Seeded synthetic layer inputs.

Distributions (per sequence b, token t, head h), as the ReplaySSM workloads state
them for Mamba-2 and Gated DeltaNet layers:

Mamba-2
  dt ~ N(0, 1), a ~ U(0.5, 2), alpha = exp(-softplus(dt) * a)
  k, q ~ N(0, 1) / sqrt(N) (i.i.d. components), v ~ N(0, 1)
Gated DeltaNet
  k, q = g / ||g||_2 with g ~ N(0, I)  (independently for k and q)
  v ~ N(0, 1), beta = sigmoid(N(0, 1)), alpha = exp(-softplus(N(0, 1)))
Kimi Delta Attention
  as Gated DeltaNet, with one gate per key channel: alpha [.., N], each entry
  exp(-softplus(N(0, 1))) independently
Initial checkpoint: zero, or N(0, sigma^2) entries.
Acceptance lengths (speculative rounds): uniform on {0, ..., T} per sequence.
Supplementary "slow" decay: alpha ~ U[0.9, 1) instead of the recipe above.

Array layouts (all float32, C-contiguous):
  alpha, beta : [B, T, H]            (KDA: alpha [B, T, H, N])
  k, q        : [B, T, H, N]       (N = d_state for Mamba-2, d_k for GDN)
  v           : [B, T, H, P]       (P = head dim for Mamba-2, d_v for GDN)
  S0          : [B, H, P, N]       (logical state layout, row p, column n)
  accept      : [B] int32

Host arrays come from numpy PCG64 streams keyed by
SeedSequence([seed, workload_id, step, field]); device arrays come from a torch
generator on the GPU seeded from the same key (same distributions, different
draws). Nothing here is timed.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, Optional

import numpy as np

# field ids of the per-step streams
_F_ALPHA_DT, _F_ALPHA_A, _F_K, _F_V, _F_Q, _F_BETA, _F_S0, _F_ACC, _F_DT_RAW, _F_A_HEAD, _F_DT_BIAS, \
    _F_CONV_X, _F_CONV_W, _F_CONV_B = range(14)


@dataclass(frozen=True)
class LayerShape:
    kind: str  # "mamba2" | "gdn" | "kda"
    B: int
    H: int
    P: int  # Mamba-2 head dim / GDN d_v
    N: int  # Mamba-2 d_state / GDN d_k

    @property
    def state_bytes_per_head(self) -> int:
        return 4 * self.P * self.N


@dataclass(frozen=True)
class Workload:
    """One synthetic workload: layer shape, window, drafts and run length."""

    wid: int
    name: str
    shape: LayerShape
    L: int
    T: int
    steps: int
    s0_sigma: float
    precision: str = "fp32"
    extra: Dict[str, object] = field(default_factory=dict)

    @property
    def C(self) -> int:
        """Ring capacity: window plus the largest number of pending drafts."""
        return self.L + self.T


WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in [
        Workload(0, "mamba2_tiny", LayerShape("mamba2", 1, 2, 16, 16), L=4, T=1,
                 steps=64, s0_sigma=0.0),
        Workload(1, "mamba2_decode_b256", LayerShape("mamba2", 256, 128, 64, 128),
                 L=16, T=1, steps=512, s0_sigma=0.1),
        Workload(2, "mamba2_spec_b256", LayerShape("mamba2", 256, 128, 64, 128),
                 L=16, T=4, steps=256, s0_sigma=0.1),
        Workload(3, "gdn_decode_b256", LayerShape("gdn", 256, 32, 128, 128),
                 L=16, T=1, steps=512, s0_sigma=0.1, extra={"spec_T": 4}),
        Workload(4, "mamba2_2prec_b256", LayerShape("mamba2", 256, 128, 64, 128),
                 L=16, T=4, steps=1024, s0_sigma=0.1, precision="fp32_hp_bf16_lp",
                 extra={"batch_sweep": (1, 32, 256, 512)}),
        Workload(5, "kda_decode_b256", LayerShape("kda", 256, 32, 128, 128),
                 L=16, T=1, steps=512, s0_sigma=0.1, extra={"spec_T": 4}),
    ]
}


def _rng(seed: int, wid: int, step: int, fid: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, wid, step, fid])))


def _torch_seed(seed: int, wid: int, step: int, fid: int) -> int:
    s = np.random.SeedSequence([seed, wid, step, fid, 0x9E3779B9]).generate_state(2, np.uint32)
    return (int(s[0]) << 31) ^ int(s[1])


def _softplus(x):
    return np.logaddexp(0.0, x)


def host_step(seed: int, wid: int, step: int, shape: LayerShape, T: int,
              decay: str = "recipe") -> Dict[str, np.ndarray]:
    """Inputs of T tokens (or T drafts) for every (sequence, head) of one step."""
    B, H, P, N = shape.B, shape.H, shape.P, shape.N
    out: Dict[str, np.ndarray] = {}
    ashape = (B, T, H, N) if shape.kind == "kda" else (B, T, H)
    if decay == "slow":
        out["alpha"] = _rng(seed, wid, step, _F_ALPHA_DT).uniform(0.9, 1.0, ashape).astype(np.float32)
    elif shape.kind == "mamba2":
        dt = _rng(seed, wid, step, _F_ALPHA_DT).standard_normal((B, T, H))
        a = _rng(seed, wid, step, _F_ALPHA_A).uniform(0.5, 2.0, (B, T, H))
        out["alpha"] = np.exp(-_softplus(dt) * a).astype(np.float32)
    else:
        g = _rng(seed, wid, step, _F_ALPHA_DT).standard_normal(ashape)
        out["alpha"] = np.exp(-_softplus(g)).astype(np.float32)
    if shape.kind == "mamba2":
        sc = 1.0 / np.sqrt(N)
        out["k"] = (_rng(seed, wid, step, _F_K).standard_normal((B, T, H, N)) * sc).astype(np.float32)
        out["q"] = (_rng(seed, wid, step, _F_Q).standard_normal((B, T, H, N)) * sc).astype(np.float32)
    else:
        for name, fid in (("k", _F_K), ("q", _F_Q)):
            g = _rng(seed, wid, step, fid).standard_normal((B, T, H, N))
            out[name] = (g / np.linalg.norm(g, axis=-1, keepdims=True)).astype(np.float32)
        bz = _rng(seed, wid, step, _F_BETA).standard_normal((B, T, H))
        out["beta"] = (1.0 / (1.0 + np.exp(-bz))).astype(np.float32)
    out["v"] = _rng(seed, wid, step, _F_V).standard_normal((B, T, H, P)).astype(np.float32)
    return out


def host_time_steps(seed: int, wid: int, step: int, shape: LayerShape, T: int) -> np.ndarray:
    """Raw time-step inputs dt ~ N(0, 1), [B, T, H] float32 (for the decay-from-dt append)."""
    return _rng(seed, wid, step, _F_DT_RAW).standard_normal((shape.B, T, shape.H)).astype(np.float32)


def host_decay_params(seed: int, wid: int, shape: LayerShape):
    """Per-head decay rate A ~ U(0.5, 2) and time-step bias dt_bias ~ N(0, 0.5^2), each [H] float32
    (the per-head form of the Mamba-2 recipe's a ~ U(0.5, 2))."""
    A = _rng(seed, wid, 0, _F_A_HEAD).uniform(0.5, 2.0, shape.H).astype(np.float32)
    bias = (_rng(seed, wid, 0, _F_DT_BIAS).standard_normal(shape.H) * 0.5).astype(np.float32)
    return A, bias


def host_conv_inputs(seed: int, wid: int, step: int, B: int, T: int, D: int) -> np.ndarray:
    """Input-projection channels entering the short convolution: x ~ N(0, 1), [B, T, D] float32."""
    return _rng(seed, wid, step, _F_CONV_X).standard_normal((B, T, D)).astype(np.float32)


def host_conv_params(seed: int, wid: int, D: int, W: int):
    """Convolution weights w ~ N(0, 1/W) [D, W] and bias ~ N(0, 0.1^2) [D], float32."""
    w = (_rng(seed, wid, 0, _F_CONV_W).standard_normal((D, W)) / np.sqrt(W)).astype(np.float32)
    b = (_rng(seed, wid, 0, _F_CONV_B).standard_normal(D) * 0.1).astype(np.float32)
    return w, b


def host_initial_state(seed: int, wid: int, shape: LayerShape, sigma: float) -> np.ndarray:
    """Initial checkpoint in the logical [B, H, P, N] layout."""
    if sigma == 0.0:
        return np.zeros((shape.B, shape.H, shape.P, shape.N), np.float32)
    g = _rng(seed, wid, 0, _F_S0).standard_normal((shape.B, shape.H, shape.P, shape.N))
    return (g * sigma).astype(np.float32)


def host_accept(seed: int, wid: int, rnd: int, B: int, T: int) -> np.ndarray:
    """Accepted prefix length per sequence, uniform on {0..T}."""
    return _rng(seed, wid, rnd, _F_ACC).integers(0, T + 1, size=B).astype(np.int32)


# ----------------------------------------------------------------------------
# Device-side generation (torch on the GPU) for full-size workloads, where host
# generation of every step would dominate the run. Same distributions.
# ----------------------------------------------------------------------------

def _gen(device, seed, wid, step, fid):
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(_torch_seed(seed, wid, step, fid))
    return g


def device_step(seed: int, wid: int, step: int, shape: LayerShape, T: int, device,
                decay: str = "recipe", out: Optional[dict] = None) -> dict:
    """As host_step, drawn on `device` with torch (fills `out` in place if given)."""
    import torch

    B, H, P, N = shape.B, shape.H, shape.P, shape.N
    f32 = torch.float32
    ashape = (B, T, H, N) if shape.kind == "kda" else (B, T, H)
    if out is None:
        out = {
            "alpha": torch.empty(ashape, dtype=f32, device=device),
            "k": torch.empty((B, T, H, N), dtype=f32, device=device),
            "q": torch.empty((B, T, H, N), dtype=f32, device=device),
            "v": torch.empty((B, T, H, P), dtype=f32, device=device),
        }
        if shape.kind in ("gdn", "kda"):
            out["beta"] = torch.empty((B, T, H), dtype=f32, device=device)
    if decay == "slow":
        out["alpha"].uniform_(0.9, 1.0, generator=_gen(device, seed, wid, step, _F_ALPHA_DT))
    elif shape.kind == "mamba2":
        dt = torch.randn((B, T, H), dtype=torch.float64, device=device,
                         generator=_gen(device, seed, wid, step, _F_ALPHA_DT))
        a = torch.empty((B, T, H), dtype=torch.float64, device=device).uniform_(
            0.5, 2.0, generator=_gen(device, seed, wid, step, _F_ALPHA_A))
        out["alpha"].copy_(torch.exp(-torch.nn.functional.softplus(dt) * a))
    else:
        g = torch.randn(ashape, dtype=torch.float64, device=device,
                        generator=_gen(device, seed, wid, step, _F_ALPHA_DT))
        out["alpha"].copy_(torch.exp(-torch.nn.functional.softplus(g)))
    if shape.kind == "mamba2":
        sc = 1.0 / float(np.sqrt(N))
        out["k"].normal_(0.0, sc, generator=_gen(device, seed, wid, step, _F_K))
        out["q"].normal_(0.0, sc, generator=_gen(device, seed, wid, step, _F_Q))
    else:
        for name, fid in (("k", _F_K), ("q", _F_Q)):
            t = out[name]
            t.normal_(0.0, 1.0, generator=_gen(device, seed, wid, step, fid))
            t.div_(torch.linalg.vector_norm(t, dim=-1, keepdim=True))
        out["beta"].normal_(0.0, 1.0, generator=_gen(device, seed, wid, step, _F_BETA))
        out["beta"].sigmoid_()
    out["v"].normal_(0.0, 1.0, generator=_gen(device, seed, wid, step, _F_V))
    return out


def device_time_steps(seed: int, wid: int, step: int, shape: LayerShape, T: int, device):
    """As host_time_steps, drawn on `device`."""
    import torch

    return torch.randn((shape.B, T, shape.H), dtype=torch.float32, device=device,
                       generator=_gen(device, seed, wid, step, _F_DT_RAW))


def device_decay_params(seed: int, wid: int, shape: LayerShape, device):
    """As host_decay_params, drawn on `device`."""
    import torch

    A = torch.empty(shape.H, dtype=torch.float32, device=device).uniform_(
        0.5, 2.0, generator=_gen(device, seed, wid, 0, _F_A_HEAD))
    bias = torch.empty(shape.H, dtype=torch.float32, device=device).normal_(
        0.0, 0.5, generator=_gen(device, seed, wid, 0, _F_DT_BIAS))
    return A, bias


def device_conv_inputs(seed: int, wid: int, step: int, B: int, T: int, D: int, device):
    """As host_conv_inputs, drawn on `device`."""
    import torch

    return torch.randn((B, T, D), dtype=torch.float32, device=device, generator=_gen(device, seed, wid, step, _F_CONV_X))


def device_initial_state(seed: int, wid: int, shape: LayerShape, sigma: float, device):
    import torch

    S = torch.zeros((shape.B, shape.H, shape.P, shape.N), dtype=torch.float32, device=device)
    if sigma != 0.0:
        S.normal_(0.0, sigma, generator=_gen(device, seed, wid, 0, _F_S0))
    return S


def device_accept(seed: int, wid: int, rnd: int, B: int, T: int, device):
    import torch

    return torch.randint(0, T + 1, (B,), dtype=torch.int32, device=device,
                         generator=_gen(device, seed, wid, rnd, _F_ACC))
