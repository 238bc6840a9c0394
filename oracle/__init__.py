"""CPU oracle for the ReplaySSM decode path -- TEST INFRASTRUCTURE ONLY.

Only tests/, the smoke check in __graft_entry__ and the CPU-baseline leg of
bench.py may import this package. The GPU library never uses it and shares no
code with it.

  liboracle.so (oracle.c)  the eager per-token recurrences in fp64 / fp32
  pointer_model.py         the integer buffer-pointer rules
  session.py               drives both through a sequence of calls
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
SRC_PATH = os.path.join(_HERE, "oracle.c")

_lib = None


def build(verbose: bool = False) -> str:
    """Compile oracle.c with gcc (-O2, OpenMP) into liboracle.so."""
    cmd = ["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-Wall", "-o", LIB_PATH + ".tmp", SRC_PATH]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB_PATH + ".tmp", LIB_PATH)
    return LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH) or os.path.getmtime(LIB_PATH) < os.path.getmtime(SRC_PATH):
            build()
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        i64, i32 = ctypes.c_int64, ctypes.c_int
        L.oracle_mamba2_round_f64.argtypes = [i64, i32, i32, i32, P, P, P, P, P, P, P]
        L.oracle_mamba2_round_f32.argtypes = [i64, i32, i32, i32, P, P, P, P, P, P, P]
        L.oracle_gdn_round_f64.argtypes = [i64, i32, i32, i32, P, P, P, P, P, P, P, P, P]
        L.oracle_gdn_round_f32.argtypes = [i64, i32, i32, i32, P, P, P, P, P, P, P, P, P]
        L.oracle_kda_round_f64.argtypes = [i64, i32, i32, i32, P, P, P, P, P, P, P, P, P]
        L.oracle_kda_round_f32.argtypes = [i64, i32, i32, i32, P, P, P, P, P, P, P, P, P]
        L.oracle_num_threads.restype = ctypes.c_int
        L.oracle_set_num_threads.argtypes = [ctypes.c_int]
        _lib = L
    return _lib


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a, a.ctypes.data


def num_threads() -> int:
    return int(lib().oracle_num_threads())


def set_num_threads(n: int) -> None:
    lib().oracle_set_num_threads(int(n))


def mamba2_round(S, alpha, k, v, q, acc, precision: str = "f64"):
    """One round over nh independent heads (the eager Mamba-2 recurrence).

    S [nh,P,N] is updated in place to the state after the accepted prefix;
    alpha [nh,T]; k,q [nh,T,N]; v [nh,T,P]; acc [nh] int. Returns out [nh,T,P].
    """
    dt = np.float64 if precision == "f64" else np.float32
    assert S.dtype == dt and S.flags.c_contiguous
    nh, P, N = S.shape
    T = alpha.shape[1]
    al, pal = _c(alpha, np.float32)
    kk, pk = _c(k, np.float32)
    vv, pv = _c(v, np.float32)
    qq, pq = _c(q, np.float32)
    ac, pac = _c(acc, np.int32)
    assert kk.shape == (nh, T, N) and qq.shape == (nh, T, N) and vv.shape == (nh, T, P)
    out = np.empty((nh, T, P), dt)
    fn = lib().oracle_mamba2_round_f64 if precision == "f64" else lib().oracle_mamba2_round_f32
    fn(nh, P, N, T, S.ctypes.data, pal, pk, pv, pq, pac, out.ctypes.data)
    return out


def gdn_round(S, alpha, beta, k, v, q, acc, precision: str = "f64"):
    """One round over nh heads of the gated delta rule. Returns (out, u), each [nh,T,P]."""
    dt = np.float64 if precision == "f64" else np.float32
    assert S.dtype == dt and S.flags.c_contiguous
    nh, P, N = S.shape
    T = alpha.shape[1]
    al, pal = _c(alpha, np.float32)
    be, pbe = _c(beta, np.float32)
    kk, pk = _c(k, np.float32)
    vv, pv = _c(v, np.float32)
    qq, pq = _c(q, np.float32)
    ac, pac = _c(acc, np.int32)
    assert kk.shape == (nh, T, N) and qq.shape == (nh, T, N) and vv.shape == (nh, T, P)
    out = np.empty((nh, T, P), dt)
    u = np.empty((nh, T, P), dt)
    fn = lib().oracle_gdn_round_f64 if precision == "f64" else lib().oracle_gdn_round_f32
    fn(nh, P, N, T, S.ctypes.data, pal, pbe, pk, pv, pq, pac, out.ctypes.data, u.ctypes.data)
    return out, u


def kda_round(S, alpha, beta, k, v, q, acc, precision: str = "f64"):
    """One round over nh heads of Kimi Delta Attention (per-channel gate alpha [nh,T,N]).
    Returns (out, u), each [nh,T,P]; u_t = beta_t (v_t - S_{t-1} (alpha_t * k_t))."""
    dt = np.float64 if precision == "f64" else np.float32
    assert S.dtype == dt and S.flags.c_contiguous
    nh, P, N = S.shape
    T = beta.shape[1]
    al, pal = _c(alpha, np.float32)
    be, pbe = _c(beta, np.float32)
    kk, pk = _c(k, np.float32)
    vv, pv = _c(v, np.float32)
    qq, pq = _c(q, np.float32)
    ac, pac = _c(acc, np.int32)
    assert al.shape == (nh, T, N) and kk.shape == (nh, T, N) and qq.shape == (nh, T, N) and vv.shape == (nh, T, P)
    out = np.empty((nh, T, P), dt)
    u = np.empty((nh, T, P), dt)
    fn = lib().oracle_kda_round_f64 if precision == "f64" else lib().oracle_kda_round_f32
    fn(nh, P, N, T, S.ctypes.data, pal, pbe, pk, pv, pq, pac, out.ctypes.data, u.ctypes.data)
    return out, u
