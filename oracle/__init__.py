"""fp64 CPU oracle for the decayed linear recurrence (TEST INFRASTRUCTURE).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The product path (``state_passing_amd``) never does:
it shares no code with the oracle and fails loudly when its own HIP library
is missing.

The arithmetic lives in ``linrec_oracle.c`` (plain C, double precision,
OpenMP over heads).  This module only builds it with gcc and marshals numpy
arrays into it.  ``twin.py`` is a second, numpy-only statement of the same
definition for tiny shapes.

Recurrence (per head): S_0 = S_in, S_t = a_t S_{t-1} + k_t^T v_t,
o_t = q_t S_t, S_out = S_T -- the d x d memory state accumulated over
sub-sequences (Sequence Accumulation and Beyond, "Approach") with boundary
states and their gradients carried across pieces (StateFlow, Abstract).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRCS = [os.path.join(_HERE, "linrec_oracle.c"), os.path.join(_HERE, "deltarule_oracle.c")]
_LIB = os.path.join(_HERE, "liblinrec_oracle.so")

_lib = None


def build(force: bool = True) -> str:
    """Compile the C oracles with gcc (-O2, OpenMP).  Returns the .so path."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
               "-Wall", "-Wextra", "-o", tmp, *_SRCS]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < max(map(os.path.getmtime, _SRCS)):
        build(force=True)
    lib = ctypes.CDLL(_LIB)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    I = ctypes.c_int
    lib.oracle_fwd.restype = I
    lib.oracle_fwd.argtypes = ([I, I, I64, I, I]
                               + [P, I64, I64, I64] * 3
                               + [P, I64, I64, I64]
                               + [P, P, I64, I64, I64, P, I])
    lib.oracle_bwd.restype = I
    lib.oracle_bwd.argtypes = ([I, I, I64, I, I]
                               + [P, I64, I64, I64] * 3
                               + [P, I64, I64, I64]
                               + [P]
                               + [P, I64, I64, I64]
                               + [P]
                               + [P, I64, I64, I64] * 3
                               + [P]
                               + [P, I64, I64, I64]
                               + [I])
    lib.delta_fwd.restype = I
    lib.delta_fwd.argtypes = ([I, I, I64, I, I]
                              + [P, I64, I64, I64] * 5
                              + [P, P, I64, I64, I64, P, I])
    lib.delta_bwd.restype = I
    lib.delta_bwd.argtypes = ([I, I, I64, I, I]
                              + [P, I64, I64, I64] * 5
                              + [P]
                              + [P, I64, I64, I64]
                              + [P]
                              + [P, I64, I64, I64] * 3
                              + [P]
                              + [P, I64, I64, I64] * 2
                              + [I])
    lib.oracle_max_threads.restype = I
    lib.oracle_max_threads.argtypes = []
    _lib = lib
    return lib


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def _act(x, name, B, H, T, d):
    """Check a [B,H,T,d] float64 array (any strides, last dim contiguous)."""
    if x.dtype != np.float64:
        raise TypeError(f"{name}: oracle takes float64, got {x.dtype}")
    if x.shape != (B, H, T, d):
        raise ValueError(f"{name}: shape {x.shape} != {(B, H, T, d)}")
    if T > 0 and d > 1 and x.strides[3] != 8:
        raise ValueError(f"{name}: feature dim must be contiguous")
    s = [st // 8 for st in x.strides[:3]]
    return x.ctypes.data, s[0], s[1], s[2]


def _decay(a, B, H, T):
    """a: None (a_t = 1), shape [H] (per head) or [B,H,T] (per token), float64."""
    if a is None:
        return None, 0, 0, 0
    if a.dtype != np.float64:
        raise TypeError("decay: oracle takes float64")
    if a.shape == (H,):
        return a.ctypes.data, 0, a.strides[0] // 8, 0
    if a.shape == (B, H, T):
        return a.ctypes.data, a.strides[0] // 8, a.strides[1] // 8, a.strides[2] // 8
    raise ValueError(f"decay: shape {a.shape} is neither [H] nor [B,H,T]")


def _state(x, name, B, H, dk, dv):
    if x is None:
        return None
    if x.dtype != np.float64 or x.shape != (B, H, dk, dv) or not x.flags.c_contiguous:
        raise ValueError(f"{name}: need contiguous float64 [B,H,dk,dv]")
    return x.ctypes.data


def fwd(q, k, v, a=None, S_in=None, nthreads: int | None = None, want_o: bool = True):
    """Forward over one (sub-)sequence.  q,k: [B,H,T,dk]; v: [B,H,T,dv].

    Returns (o [B,H,T,dv] or None, S_out [B,H,dk,dv]), all float64.
    """
    lib = _load()
    B, H, T, dk = k.shape
    dv = v.shape[3]
    S_in = None if S_in is None else np.ascontiguousarray(S_in, dtype=np.float64)
    o = np.empty((B, H, T, dv), np.float64) if want_o else None
    S_out = np.empty((B, H, dk, dv), np.float64)
    qa = _act(q, "q", B, H, T, dk) if want_o else (None, 0, 0, 0)
    ka = _act(k, "k", B, H, T, dk)
    va = _act(v, "v", B, H, T, dv)
    aa = _decay(a, B, H, T)
    oa = _act(o, "o", B, H, T, dv) if want_o else (None, 0, 0, 0)
    nt = nthreads or min(B * H, max_threads()) or 1
    rc = lib.oracle_fwd(B, H, T, dk, dv, *qa, *ka, *va, *aa,
                        _state(S_in, "S_in", B, H, dk, dv), *oa,
                        S_out.ctypes.data, nt)
    if rc != 0:
        raise RuntimeError("oracle_fwd: bad arguments")
    return o, S_out


def bwd(q, k, v, a, S_in, dO, dS_out=None, want_da: bool = False,
        nthreads: int | None = None):
    """Backward of L = <dO, o> + <dS_out, S_out>.

    Returns (dq, dk, dv, dS_in) -- plus da [B,H,T] when want_da -- float64.
    """
    lib = _load()
    B, H, T, dk = k.shape
    dv = v.shape[3]
    S_in = None if S_in is None else np.ascontiguousarray(S_in, dtype=np.float64)
    dS_out = None if dS_out is None else np.ascontiguousarray(dS_out, dtype=np.float64)
    dq = np.empty((B, H, T, dk), np.float64)
    dkk = np.empty((B, H, T, dk), np.float64)
    dvv = np.empty((B, H, T, dv), np.float64)
    dS_in = np.empty((B, H, dk, dv), np.float64)
    da = None
    if want_da:
        if a is None:
            raise ValueError("da needs a decay tensor")
        da = np.empty((B, H, T), np.float64)
        daa = (da.ctypes.data, T * H, T, 1)
    else:
        daa = (None, 0, 0, 0)
    nt = nthreads or min(B * H, max_threads()) or 1
    rc = lib.oracle_bwd(B, H, T, dk, dv,
                        *_act(q, "q", B, H, T, dk), *_act(k, "k", B, H, T, dk),
                        *_act(v, "v", B, H, T, dv), *_decay(a, B, H, T),
                        _state(S_in, "S_in", B, H, dk, dv),
                        *(_act(dO, "dO", B, H, T, dv) if dO is not None else (None, 0, 0, 0)),
                        _state(dS_out, "dS_out", B, H, dk, dv),
                        *_act(dq, "dq", B, H, T, dk), *_act(dkk, "dk", B, H, T, dk),
                        *_act(dvv, "dv", B, H, T, dv), dS_in.ctypes.data,
                        *daa, nt)
    if rc != 0:
        raise RuntimeError("oracle_bwd: bad arguments")
    if want_da:
        return dq, dkk, dvv, dS_in, da
    return dq, dkk, dvv, dS_in


# ------------------------------------------------------------ delta rule
#
# Gated delta rule (deltarule_oracle.c): S_t = a_t (I - beta_t k_t^T k_t)
# S_{t-1} + beta_t k_t^T v_t, o_t = q_t S_t -- the recurrence of the Gated
# DeltaNet models StateFlow trains (the gptget summary, "Experimental
# design"), in the layer's d_k x d_v state orientation.


def _beta(x, B, H, T):
    if x.dtype != np.float64 or x.shape != (B, H, T):
        raise ValueError(f"beta: need float64 [B,H,T], got {x.dtype} {x.shape}")
    return x.ctypes.data, x.strides[0] // 8, x.strides[1] // 8, x.strides[2] // 8


def delta_fwd(q, k, v, beta, a=None, S_in=None, nthreads: int | None = None,
              want_o: bool = True):
    """Delta-rule forward over one (sub-)sequence.  beta: [B,H,T].

    Returns (o [B,H,T,dv] or None, S_out [B,H,dk,dv]), float64."""
    lib = _load()
    B, H, T, dk = k.shape
    dv = v.shape[3]
    S_in = None if S_in is None else np.ascontiguousarray(S_in, dtype=np.float64)
    o = np.empty((B, H, T, dv), np.float64) if want_o else None
    S_out = np.empty((B, H, dk, dv), np.float64)
    qa = _act(q, "q", B, H, T, dk) if want_o else (None, 0, 0, 0)
    oa = _act(o, "o", B, H, T, dv) if want_o else (None, 0, 0, 0)
    nt = nthreads or min(B * H, max_threads()) or 1
    rc = lib.delta_fwd(B, H, T, dk, dv, *qa, *_act(k, "k", B, H, T, dk),
                       *_act(v, "v", B, H, T, dv), *_beta(beta, B, H, T), *_decay(a, B, H, T),
                       _state(S_in, "S_in", B, H, dk, dv), *oa, S_out.ctypes.data, nt)
    if rc != 0:
        raise RuntimeError("delta_fwd: bad arguments")
    return o, S_out


def delta_bwd(q, k, v, beta, a, S_in, dO, dS_out=None, want_da: bool = False,
              nthreads: int | None = None):
    """Backward of L = <dO, o> + <dS_out, S_out> through the delta rule.

    Returns (dq, dk, dv, dbeta, dS_in) -- plus da [B,H,T] when want_da."""
    lib = _load()
    B, H, T, dk = k.shape
    dv = v.shape[3]
    S_in = None if S_in is None else np.ascontiguousarray(S_in, dtype=np.float64)
    dS_out = None if dS_out is None else np.ascontiguousarray(dS_out, dtype=np.float64)
    dq = np.empty((B, H, T, dk), np.float64)
    dkk = np.empty((B, H, T, dk), np.float64)
    dvv = np.empty((B, H, T, dv), np.float64)
    dbeta = np.empty((B, H, T), np.float64)
    dS_in = np.empty((B, H, dk, dv), np.float64)
    da = None
    daa = (None, 0, 0, 0)
    if want_da:
        if a is None:
            raise ValueError("da needs a decay tensor")
        da = np.empty((B, H, T), np.float64)
        daa = (da.ctypes.data, T * H, T, 1)
    nt = nthreads or min(B * H, max_threads()) or 1
    rc = lib.delta_bwd(B, H, T, dk, dv,
                       *_act(q, "q", B, H, T, dk), *_act(k, "k", B, H, T, dk),
                       *_act(v, "v", B, H, T, dv), *_beta(beta, B, H, T), *_decay(a, B, H, T),
                       _state(S_in, "S_in", B, H, dk, dv),
                       *(_act(dO, "dO", B, H, T, dv) if dO is not None else (None, 0, 0, 0)),
                       _state(dS_out, "dS_out", B, H, dk, dv),
                       *_act(dq, "dq", B, H, T, dk), *_act(dkk, "dk", B, H, T, dk),
                       *_act(dvv, "dv", B, H, T, dv), dS_in.ctypes.data,
                       dbeta.ctypes.data, T * H, T, 1, *daa, nt)
    if rc != 0:
        raise RuntimeError("delta_bwd: bad arguments")
    if want_da:
        return dq, dkk, dvv, dbeta, dS_in, da
    return dq, dkk, dvv, dbeta, dS_in
