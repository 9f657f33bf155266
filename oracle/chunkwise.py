"""Chunkwise reformulation of the KDA recurrence, fp64 (test infrastructure only).

The chunkwise-form entry of the "xhh.club" tag page 结构 splits the sequence into
chunks that are linked by a state recurrence and computed inside with matrix
products.  This is that form written out from the definition, using one reference
point per chunk (the chunk start).  With the -5 floor a chunk of C tokens spans at
most 5C in log-decay, so exp(+-G) stays finite in fp64 for C <= 128 (5*128 < 709).

Per chunk, with S the state entering it, G the inclusive cumulative sum of the
floored log-decay over the chunk (per key channel) and rows indexed by token:
  Kt = K*exp(G), Kh = K*exp(-G), Qt = Q*exp(G)
  A  = StrictLower(diag(beta) Kt Kh^T)
  U  = (I + A)^-1 diag(beta) (V - Kt S)      (the per-token "u" of the recurrence)
  O  = Qt S + Lower(Qt Kh^T) U
  S <- diag(exp(G_last)) S + (K*exp(G_last - G))^T U
"""
from __future__ import annotations

import numpy as np

from .sequential import clamp_decay


def chunkwise(q, k, v, g, beta, S0=None, chunk: int = 64):
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    g = np.asarray(g, np.float64)
    beta = np.asarray(beta, np.float64)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if chunk < 1 or chunk > 128:
        raise ValueError("chunk must be in [1, 128] for the fp64 full-chunk factorisation")
    # [B,H,T,*] views for batched matrix products
    qh = q.transpose(0, 2, 1, 3)
    kh = k.transpose(0, 2, 1, 3)
    vh = v.transpose(0, 2, 1, 3)
    gh = clamp_decay(g).transpose(0, 2, 1, 3)
    bh = beta.transpose(0, 2, 1)
    S = np.zeros((B, H, dk, dv)) if S0 is None else np.array(S0, dtype=np.float64)
    o = np.empty((B, H, T, dv))
    for t0 in range(0, T, chunk):
        t1 = min(T, t0 + chunk)
        C = t1 - t0
        Q, K, V, bt = qh[:, :, t0:t1], kh[:, :, t0:t1], vh[:, :, t0:t1], bh[:, :, t0:t1]
        G = np.cumsum(gh[:, :, t0:t1], axis=2)              # [B,H,C,dk]
        Kt = K * np.exp(G)
        Khat = K * np.exp(-G)
        Qt = Q * np.exp(G)
        strict = np.tril(np.ones((C, C)), -1)
        incl = np.tril(np.ones((C, C)))
        A = bt[..., :, None] * (Kt @ np.swapaxes(Khat, -1, -2)) * strict
        rhs = bt[..., :, None] * (V - Kt @ S)
        U = np.linalg.solve(np.eye(C) + A, rhs)
        P = (Qt @ np.swapaxes(Khat, -1, -2)) * incl
        o[:, :, t0:t1] = Qt @ S + P @ U
        GC = G[:, :, -1]                                     # [B,H,dk]
        Kdec = K * np.exp(GC[:, :, None, :] - G)
        S = np.exp(GC)[..., :, None] * S + np.swapaxes(Kdec, -1, -2) @ U
    return o.transpose(0, 2, 1, 3), S
