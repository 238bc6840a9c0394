"""ctypes binding of libreplayssm (argument marshalling only).

Every function here has the name of a C entry point of include/replayssm.h
without the `replayssm_` prefix, takes torch tensors that already live on the
GPU, passes their data pointers and the current HIP stream, and raises
ReplaySSMError on a non-zero status. No computation happens in Python and there
is no fallback: if the library is missing, loading fails loudly.

torch is imported first on purpose: the library then binds to the HIP runtime
that torch already loaded (same SONAME), so torch's device pointers and
streams are valid in it.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libreplayssm.so")

MAMBA2, GDN, KDA = 0, 1, 2
FP32, FP32_HP_BF16_LP, BF16_SHARED = 0, 1, 2
PRECISIONS = {"fp32": FP32, "fp32_hp_bf16_lp": FP32_HP_BF16_LP, "bf16_shared": BF16_SHARED}
KINDS = {"mamba2": MAMBA2, "gdn": GDN, "kda": KDA}

OK, EINVAL, ENOTSUP, EHIP = 0, -1, -2, -3
TILES_AUTO, TILES_ONE, TILES_TWO = 0, 1, 2
DEVERR_APPEND_OVERFLOW, DEVERR_PENDING, DEVERR_ACCEPT, DEVERR_CORRUPT, DEVERR_STALE, DEVERR_INDEX = 1, 2, 4, 8, 16, 32

_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_vp = ctypes.c_void_p


class Config(ctypes.Structure):
    _fields_ = [("kind", _i32), ("precision", _i32), ("B", _i32), ("H", _i32), ("dv", _i32),
                ("dk", _i32), ("L", _i32), ("T_max", _i32)]


class State(ctypes.Structure):
    _fields_ = [("hp", _vp), ("lp", _vp), ("ring_alpha", _vp), ("ring_beta", _vp), ("ring_k", _vp),
                ("ring_v", _vp), ("head", _vp), ("h", _vp), ("p", _vp), ("folded", _vp),
                ("arrive", _vp), ("err", _vp), ("ring_vraw", _vp)]


class Sizes(ctypes.Structure):
    _fields_ = [("C", _i32), ("alignment", _i32), ("hp_bytes", _i64), ("lp_bytes", _i64),
                ("ring_alpha_bytes", _i64), ("ring_beta_bytes", _i64), ("ring_k_bytes", _i64),
                ("ring_v_bytes", _i64), ("ptr_bytes", _i64), ("folded_bytes", _i64),
                ("err_bytes", _i64), ("ring_vraw_bytes", _i64)]


class ConvConfig(ctypes.Structure):
    _fields_ = [("B", _i32), ("D", _i32), ("W", _i32), ("T_max", _i32)]


class ConvState(ctypes.Structure):
    _fields_ = [("ring", _vp), ("start", _vp), ("pend", _vp), ("arrive", _vp), ("err", _vp)]


class ReplaySSMError(RuntimeError):
    def __init__(self, status: int, where: str, text: str):
        super().__init__(f"{where}: status {status} ({text})")
        self.status = status


# entry point name -> argument types (all return int, except the two string functions)
SIGNATURES = {
    "replayssm_get_sizes": [ctypes.POINTER(Config), ctypes.POINTER(Sizes)],
    "replayssm_init": [ctypes.POINTER(Config), ctypes.POINTER(State), _vp],
    "replayssm_pack_state": [ctypes.POINTER(Config), _vp, _vp, _vp, _vp],
    "replayssm_unpack_state": [ctypes.POINTER(Config), _vp, _vp, _vp, _vp],
    "replayssm_read_error": [ctypes.POINTER(State), ctypes.POINTER(_i32), _vp],
    "replayssm_append": [ctypes.POINTER(Config), ctypes.POINTER(State), ctypes.c_int, _vp, _vp, _vp, _vp, _vp],
    "replayssm_append_static": [ctypes.POINTER(Config), ctypes.POINTER(State), ctypes.c_int, _vp, _vp, _vp, _vp,
                                _vp],
    "replayssm_append_dt": [ctypes.POINTER(Config), ctypes.POINTER(State), ctypes.c_int, _vp, _vp, _vp, _vp, _vp,
                            _vp, _vp],
    "replayssm_decode": [ctypes.POINTER(Config), ctypes.POINTER(State), _vp, _vp, _vp],
    "replayssm_conv_sizes": [ctypes.POINTER(ConvConfig), ctypes.POINTER(_i64), ctypes.POINTER(_i64)],
    "replayssm_conv_init": [ctypes.POINTER(ConvConfig), ctypes.POINTER(ConvState), _vp],
    "replayssm_conv_step": [ctypes.POINTER(ConvConfig), ctypes.POINTER(ConvState), ctypes.c_int, _vp, _vp, _vp,
                            ctypes.c_int, ctypes.c_int, _vp, _vp],
    "replayssm_conv_accept": [ctypes.POINTER(ConvConfig), ctypes.POINTER(ConvState), _vp, _vp],
    "replayssm_verify": [ctypes.POINTER(Config), ctypes.POINTER(State), ctypes.c_int, _vp, _vp, _vp],
    "replayssm_decode_step": [ctypes.POINTER(Config), ctypes.POINTER(State), _vp, _vp, _vp, _vp, _vp, _vp, _vp],
    "replayssm_verify_step": [ctypes.POINTER(Config), ctypes.POINTER(State), ctypes.c_int, _vp, _vp, _vp, _vp, _vp,
                              _vp, _vp],
    "replayssm_accept": [ctypes.POINTER(Config), ctypes.POINTER(State), _vp, _vp],
    "replayssm_flush": [ctypes.POINTER(Config), ctypes.POINTER(State), _vp],
    "replayssm_eager_step": [ctypes.POINTER(Config), _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp],
    "replayssm_eager_verify": [ctypes.POINTER(Config), _vp, _vp, ctypes.c_int, _vp, _vp, _vp, _vp, _vp, _vp, _vp],
    "replayssm_eager_accept": [ctypes.POINTER(Config), _vp, _vp, ctypes.c_int, _vp],
    "replayssm_probe_read": [_vp, ctypes.c_int64, _vp, _vp],
    "replayssm_set_tiling": [ctypes.c_int],
    "replayssm_get_tiling": [],
    "replayssm_flush_selected": [ctypes.POINTER(Config), ctypes.POINTER(State), _vp, _vp],
    "replayssm_snapshot": [ctypes.POINTER(Config), ctypes.POINTER(State), ctypes.c_int, _vp, _vp, _vp],
    "replayssm_restore": [ctypes.POINTER(Config), ctypes.POINTER(State), ctypes.c_int, _vp, _vp, _vp],
}
STRING_FUNCTIONS = {"replayssm_status_string": [ctypes.c_int], "replayssm_last_error": []}

_lib = None


def lib():
    """The loaded library; raises if it was not built (there is no fallback)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m ssm_decode_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, args in SIGNATURES.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        for name, args in STRING_FUNCTIONS.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _check(status: int, where: str) -> None:
    if status != OK:
        raise ReplaySSMError(status, where, lib().replayssm_last_error().decode())


def _p(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _s(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def _f32(t):
    if t is not None and t.dtype != torch.float32:
        raise TypeError("float32 tensor expected")
    return _p(t)


def _i32t(t):
    if t.dtype != torch.int32:
        raise TypeError("int32 tensor expected")
    return _p(t)


def make_config(kind="mamba2", precision="fp32", B=1, H=1, dv=64, dk=128, L=16, T_max=1) -> Config:
    return Config(KINDS.get(kind, kind), PRECISIONS.get(precision, precision), B, H, dv, dk, L, T_max)


def get_sizes(cfg: Config) -> Sizes:
    out = Sizes()
    _check(lib().replayssm_get_sizes(ctypes.byref(cfg), ctypes.byref(out)), "get_sizes")
    return out


def status_string(status: int) -> str:
    return lib().replayssm_status_string(status).decode()


def last_error() -> str:
    return lib().replayssm_last_error().decode()


def init(cfg, st, stream=None):
    _check(lib().replayssm_init(ctypes.byref(cfg), ctypes.byref(st), _s(stream)), "init")


def pack_state(cfg, src, hp=None, lp=None, stream=None):
    _check(lib().replayssm_pack_state(ctypes.byref(cfg), _f32(src), _p(hp), _p(lp), _s(stream)), "pack_state")


def unpack_state(cfg, hp, lp, dst, stream=None):
    _check(lib().replayssm_unpack_state(ctypes.byref(cfg), _p(hp), _p(lp), _f32(dst), _s(stream)), "unpack_state")


def read_error(st, stream=None) -> int:
    v = _i32(0)
    _check(lib().replayssm_read_error(ctypes.byref(st), ctypes.byref(v), _s(stream)), "read_error")
    return int(v.value)


def append(cfg, st, T, alpha, k, v, beta=None, stream=None):
    _check(lib().replayssm_append(ctypes.byref(cfg), ctypes.byref(st), int(T), _f32(alpha), _f32(k),
                                  _f32(v), _f32(beta), _s(stream)), "append")


def append_static(cfg, st, T, alpha, k, v, beta=None, stream=None):
    _check(lib().replayssm_append_static(ctypes.byref(cfg), ctypes.byref(st), int(T), _f32(alpha), _f32(k),
                                         _f32(v), _f32(beta), _s(stream)), "append_static")


def append_dt(cfg, st, T, dt, A, dt_bias, k, v, beta=None, stream=None):
    _check(lib().replayssm_append_dt(ctypes.byref(cfg), ctypes.byref(st), int(T), _f32(dt), _f32(A), _f32(dt_bias),
                                     _f32(k), _f32(v), _f32(beta), _s(stream)), "append_dt")


def decode(cfg, st, q, out, stream=None):
    _check(lib().replayssm_decode(ctypes.byref(cfg), ctypes.byref(st), _f32(q), _f32(out), _s(stream)), "decode")


def verify(cfg, st, T, q, out, stream=None):
    _check(lib().replayssm_verify(ctypes.byref(cfg), ctypes.byref(st), int(T), _f32(q), _f32(out),
                                  _s(stream)), "verify")


def decode_step(cfg, st, alpha, k, v, beta, q, out, stream=None):
    _check(lib().replayssm_decode_step(ctypes.byref(cfg), ctypes.byref(st), _f32(alpha), _f32(k), _f32(v),
                                       _f32(beta), _f32(q), _f32(out), _s(stream)), "decode_step")


def verify_step(cfg, st, T, alpha, k, v, beta, q, out, stream=None):
    _check(lib().replayssm_verify_step(ctypes.byref(cfg), ctypes.byref(st), int(T), _f32(alpha), _f32(k),
                                       _f32(v), _f32(beta), _f32(q), _f32(out), _s(stream)), "verify_step")


def accept(cfg, st, accepted, stream=None):
    _check(lib().replayssm_accept(ctypes.byref(cfg), ctypes.byref(st), _i32t(accepted), _s(stream)), "accept")


def flush(cfg, st, stream=None):
    _check(lib().replayssm_flush(ctypes.byref(cfg), ctypes.byref(st), _s(stream)), "flush")


def eager_step(cfg, S, alpha, k, v, beta, q, out, stream=None):
    _check(lib().replayssm_eager_step(ctypes.byref(cfg), _f32(S), _f32(alpha), _f32(k), _f32(v),
                                      _f32(beta), _f32(q), _f32(out), _s(stream)), "eager_step")


def eager_verify(cfg, pool, slot, T, alpha, k, v, beta, q, out, stream=None):
    _check(lib().replayssm_eager_verify(ctypes.byref(cfg), _f32(pool), _i32t(slot), int(T), _f32(alpha),
                                        _f32(k), _f32(v), _f32(beta), _f32(q), _f32(out), _s(stream)),
           "eager_verify")


def eager_accept(cfg, slot, accepted, T, stream=None):
    _check(lib().replayssm_eager_accept(ctypes.byref(cfg), _i32t(slot), _i32t(accepted), int(T), _s(stream)),
           "eager_accept")


def flush_selected(cfg, st, select, stream=None):
    _check(lib().replayssm_flush_selected(ctypes.byref(cfg), ctypes.byref(st), _i32t(select), _s(stream)),
           "flush_selected")


def snapshot(cfg, st, seqs, dst, stream=None):
    _check(lib().replayssm_snapshot(ctypes.byref(cfg), ctypes.byref(st), int(seqs.numel()), _i32t(seqs), _f32(dst),
                                    _s(stream)), "snapshot")


def restore(cfg, st, seqs, src, stream=None):
    _check(lib().replayssm_restore(ctypes.byref(cfg), ctypes.byref(st), int(seqs.numel()), _i32t(seqs), _f32(src),
                                   _s(stream)), "restore")


def set_tiling(policy):
    """replayssm_set_tiling: TILES_AUTO, TILES_ONE or TILES_TWO (process-wide; results unchanged)."""
    _check(lib().replayssm_set_tiling(int(policy)), "set_tiling")


def get_tiling():
    return int(lib().replayssm_get_tiling())


def probe_read(src, sink, stream=None):
    """Enqueue one pass of the read-ceiling probe over `src` (a CUDA tensor); `sink` is one float32."""
    _check(lib().replayssm_probe_read(_p(src), ctypes.c_int64(src.numel() * src.element_size()), _f32(sink),
                                      _s(stream)), "probe_read")


class LayerState:
    """Device memory (torch tensors) for one layer's ReplaySSM state, plus the C struct.

    Memory plumbing only: sizes come from replayssm_get_sizes, and replayssm_init
    is called once on construction.
    """

    def __init__(self, cfg: Config, device="cuda", stream=None):
        self.cfg = cfg
        sz = get_sizes(cfg)
        self.C = sz.C
        B, H, dv, dk, C = cfg.B, cfg.H, cfg.dv, cfg.dk, sz.C
        f32, i32 = torch.float32, torch.int32
        self.hp = torch.zeros((B, H, dv * dk), dtype=f32, device=device) if sz.hp_bytes else None
        self.lp = torch.zeros((B, H, dv * dk), dtype=torch.int16, device=device) if sz.lp_bytes else None
        # a scalar gate per record, or (KDA) a gate row of dk channels
        self.ring_alpha = torch.zeros((B, H, C, dk) if cfg.kind == KDA else (B, H, C), dtype=f32, device=device)
        self.ring_beta = torch.zeros((B, H, C), dtype=f32, device=device) if sz.ring_beta_bytes else None
        self.ring_k = torch.zeros((B, H, C, dk), dtype=f32, device=device)
        self.ring_v = torch.zeros((B, H, C, dv), dtype=f32, device=device)
        self.head = torch.zeros(B, dtype=i32, device=device)
        self.h = torch.zeros(B, dtype=i32, device=device)
        self.p = torch.zeros(B, dtype=i32, device=device)
        self.folded = torch.zeros(B, dtype=torch.int64, device=device)
        self.arrive = torch.zeros(B, dtype=i32, device=device)
        self.err = torch.zeros(4, dtype=i32, device=device)
        self.ring_vraw = torch.zeros((B, H, C, dv), dtype=f32, device=device) if sz.ring_vraw_bytes else None
        self.struct = State(*[None if t is None else t.data_ptr() for t in (
            self.hp, self.lp, self.ring_alpha, self.ring_beta, self.ring_k, self.ring_v, self.head,
            self.h, self.p, self.folded, self.arrive, self.err, self.ring_vraw)])
        init(cfg, self.struct, stream)

    def import_state(self, S_logical: torch.Tensor, stream=None):
        """Set the checkpoint from logical [B, H, dv, dk] fp32 values (both copies as the mode needs)."""
        pack_state(self.cfg, S_logical.contiguous(), self.hp, self.lp, stream)

    def export_state(self, which: str = "hp", stream=None) -> torch.Tensor:
        """Logical [B, H, dv, dk] fp32 view of the fp32 ("hp") or bf16 ("lp") checkpoint."""
        cfg = self.cfg
        dst = torch.empty((cfg.B, cfg.H, cfg.dv, cfg.dk), dtype=torch.float32, device=self.ring_k.device)
        if which == "hp":
            unpack_state(cfg, self.hp, None, dst, stream)
        else:
            unpack_state(cfg, None, self.lp, dst, stream)
        return dst

    def tensors(self):
        """Every device tensor the layer's state holds."""
        return [t for t in (self.hp, self.lp, self.ring_alpha, self.ring_beta, self.ring_k, self.ring_v, self.head,
                            self.h, self.p, self.folded, self.arrive, self.err, self.ring_vraw) if t is not None]

    def pointers(self):
        return {"head": self.head.tolist(), "h": self.h.tolist(), "p": self.p.tolist(),
                "folded": self.folded.tolist()}


# ---- convolution input ring -------------------------------------------------

def make_conv_config(B, D, W=4, T_max=1) -> ConvConfig:
    return ConvConfig(int(B), int(D), int(W), int(T_max))


def conv_sizes(cfg: ConvConfig):
    ring, ptr = _i64(0), _i64(0)
    _check(lib().replayssm_conv_sizes(ctypes.byref(cfg), ctypes.byref(ring), ctypes.byref(ptr)), "conv_sizes")
    return int(ring.value), int(ptr.value)


def conv_init(cfg, st, stream=None):
    _check(lib().replayssm_conv_init(ctypes.byref(cfg), ctypes.byref(st), _s(stream)), "conv_init")


def conv_step(cfg, st, T, x, w, bias, silu, commit, y, stream=None):
    _check(lib().replayssm_conv_step(ctypes.byref(cfg), ctypes.byref(st), int(T), _f32(x), _f32(w), _f32(bias),
                                     int(bool(silu)), int(bool(commit)), _f32(y), _s(stream)), "conv_step")


def conv_accept(cfg, st, accepted, stream=None):
    _check(lib().replayssm_conv_accept(ctypes.byref(cfg), ctypes.byref(st), _i32t(accepted), _s(stream)),
           "conv_accept")


class ConvLayer:
    """Device memory (torch tensors) for one layer's convolution input ring, plus the C struct;
    replayssm_conv_init is called once on construction."""

    def __init__(self, cfg: ConvConfig, device="cuda", stream=None):
        self.cfg = cfg
        conv_sizes(cfg)  # validates
        self.Cc = cfg.W - 1 + cfg.T_max
        self.ring = torch.empty((cfg.B, self.Cc, cfg.D), dtype=torch.float32, device=device)
        self.start = torch.empty(cfg.B, dtype=torch.int32, device=device)
        self.pend = torch.empty(cfg.B, dtype=torch.int32, device=device)
        self.arrive = torch.empty(cfg.B, dtype=torch.int32, device=device)
        self.err = torch.empty(4, dtype=torch.int32, device=device)
        self.struct = ConvState(*[t.data_ptr() for t in (self.ring, self.start, self.pend, self.arrive, self.err)])
        conv_init(cfg, self.struct, stream)
