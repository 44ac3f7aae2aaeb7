"""Numpy twin of the C oracle, for tiny shapes (TEST INFRASTRUCTURE).

A second, independent statement of the same token-by-token definition,
written with whole-matrix numpy operations instead of the C loops, so the two
can be checked against each other.  Python loops over tokens only: use it for
T up to a few hundred.

Recurrence (Sequence Accumulation and Beyond, "Approach": a d x d memory
state accumulated token by token; StateFlow, Abstract: boundary state and
gradient carried across pieces):
    S_t = a_t S_{t-1} + k_t^T v_t,  o_t = q_t S_t.
"""
from __future__ import annotations

import numpy as np


def _decay_bh(a, b, h, T):
    if a is None:
        return np.ones(T)
    a = np.asarray(a, np.float64)
    if a.ndim == 1:
        return np.full(T, a[h])
    return a[b, h]


def fwd(q, k, v, a=None, S_in=None):
    B, H, T, dk = k.shape
    dv = v.shape[3]
    o = np.zeros((B, H, T, dv))
    S_out = np.zeros((B, H, dk, dv))
    for b in range(B):
        for h in range(H):
            ab = _decay_bh(a, b, h, T)
            S = np.zeros((dk, dv)) if S_in is None else np.array(S_in[b, h], np.float64)
            for t in range(T):
                S = ab[t] * S + np.outer(k[b, h, t], v[b, h, t])
                o[b, h, t] = q[b, h, t] @ S
            S_out[b, h] = S
    return o, S_out


def bwd(q, k, v, a, S_in, dO, dS_out=None):
    """Adjoint of fwd for L = <dO, o> + <dS_out, S_out>; stores all S_t."""
    B, H, T, dk = k.shape
    dv = v.shape[3]
    dq = np.zeros((B, H, T, dk))
    dkk = np.zeros((B, H, T, dk))
    dvv = np.zeros((B, H, T, dv))
    dS_in = np.zeros((B, H, dk, dv))
    for b in range(B):
        for h in range(H):
            ab = _decay_bh(a, b, h, T)
            S = np.zeros((dk, dv)) if S_in is None else np.array(S_in[b, h], np.float64)
            states = []
            for t in range(T):
                S = ab[t] * S + np.outer(k[b, h, t], v[b, h, t])
                states.append(S)
                dq[b, h, t] = states[t] @ dO[b, h, t]
            G = np.zeros((dk, dv)) if dS_out is None else np.array(dS_out[b, h], np.float64)
            for t in range(T - 1, -1, -1):
                G = G + np.outer(q[b, h, t], dO[b, h, t])
                dkk[b, h, t] = G @ v[b, h, t]
                dvv[b, h, t] = k[b, h, t] @ G
                G = ab[t] * G
            dS_in[b, h] = G
    return dq, dkk, dvv, dS_in
