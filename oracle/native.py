"""ctypes wrapper of kda_oracle.c (test infrastructure only).

`build()` compiles the plain C oracle with gcc into oracle/libkda_oracle.so; the
wrappers load the built library and build it only when it is absent.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB = os.path.join(_HERE, "libkda_oracle.so")
_lib = None


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", _SRC, "-o", _LIB + ".tmp", "-lm"]
    subprocess.run(cmd, check=True, capture_output=not verbose)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = C.CDLL(_LIB)
        vp, ip, dp = C.c_void_p, C.c_int, C.c_void_p
        lib.kda_oracle_prefill.argtypes = [ip, ip, ip, ip, ip, ip, vp, vp, vp, vp, vp, vp, dp, dp,
                                           ip, dp, ip]
        lib.kda_oracle_prefill.restype = ip
        lib.kda_oracle_decode_step.argtypes = [ip, ip, ip, ip, ip, vp, vp, vp, vp, vp, dp, dp, ip]
        lib.kda_oracle_decode_step.restype = ip
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _threads(n):
    if n:
        return int(n)
    try:
        return max(1, min(16, len(os.sched_getaffinity(0))))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def prefill(q, k, v, g, beta, S0=None, *, bf16: bool, ckpt_every: int = 0, want_o: bool = True,
            nthreads: int = 0):
    """Sequential fp64 recurrence on stored input bytes.  q/k/v: [B,T,H,d] uint16 (bf16)
    or float32; g [B,T,H,d_k] f32; beta [B,T,H] f32; S0 [B,H,d_k,d_v] f32 or None.
    Returns (o fp64 or None, S_T fp64, ckpts fp64 [B, T/ckpt_every, H, d_k, d_v] or None)."""
    lib = _load()
    q = np.ascontiguousarray(q)
    k = np.ascontiguousarray(k)
    v = np.ascontiguousarray(v)
    g = np.ascontiguousarray(g, dtype=np.float32)
    beta = np.ascontiguousarray(beta, dtype=np.float32)
    if S0 is not None:
        S0 = np.ascontiguousarray(S0, dtype=np.float32)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    o = np.empty((B, T, H, dv)) if want_o else None
    S = np.empty((B, H, dk, dv))
    ck = None
    if ckpt_every:
        ck = np.empty((B, T // ckpt_every, H, dk, dv))
    rc = lib.kda_oracle_prefill(B, T, H, dk, dv, int(bf16), _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                _ptr(beta), _ptr(S0), _ptr(o), _ptr(S), int(ckpt_every), _ptr(ck),
                                _threads(nthreads))
    if rc != 0:
        raise ValueError("kda_oracle_prefill: bad arguments")
    return o, S, ck


def decode_step(state, q, k, v, g, beta, *, bf16: bool, nthreads: int = 0):
    """One step in place on a fp64 state [N,H,d_k,d_v]; returns o fp64 [N,H,d_v]."""
    lib = _load()
    assert state.dtype == np.float64 and state.flags.c_contiguous
    q = np.ascontiguousarray(q)
    k = np.ascontiguousarray(k)
    v = np.ascontiguousarray(v)
    g = np.ascontiguousarray(g, dtype=np.float32)
    beta = np.ascontiguousarray(beta, dtype=np.float32)
    N, H, dk = q.shape
    dv = v.shape[-1]
    o = np.empty((N, H, dv))
    rc = lib.kda_oracle_decode_step(N, H, dk, dv, int(bf16), _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                    _ptr(beta), _ptr(state), _ptr(o), _threads(nthreads))
    if rc != 0:
        raise ValueError("kda_oracle_decode_step: bad arguments")
    return o
