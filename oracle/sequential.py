"""KDA recurrence, the plain definition, in fp64 (test infrastructure only).

Follows the recurrent-form entry of the "xhh.club" tag page 结构 (per-channel
decay, then erase-and-write into a per-head d_k x d_v state) with the -5 floor on
each step's log-decay from the chunkwise-form entry of the same page.  Shapes:
q, k, g [B,T,H,d_k]; v [B,T,H,d_v]; beta [B,T,H]; S [B,H,d_k,d_v].  Inputs are
fp64 arrays holding the exact values the device receives.
"""
from __future__ import annotations

import numpy as np

FLOOR = -5.0


def clamp_decay(g: np.ndarray) -> np.ndarray:
    """Per-step log-decay after the floor: min(0, max(-5, g))."""
    return np.minimum(0.0, np.maximum(FLOOR, g))


def _step(S, q_t, k_t, v_t, g_t, b_t):
    """One token for every (batch, head): returns (o_t, S_t)."""
    alpha = np.exp(clamp_decay(g_t))                    # [B,H,dk]
    Sp = alpha[..., :, None] * S                        # decay the key rows
    e = np.einsum("bhi,bhij->bhj", k_t, Sp)             # S'^T k
    u = b_t[..., None] * (v_t - e)                      # beta (v - S'^T k)
    S = Sp + k_t[..., :, None] * u[..., None, :]        # write k u^T
    o = np.einsum("bhi,bhij->bhj", q_t, S)              # read S^T q after the write
    return o, S


def recurrent(q, k, v, g, beta, S0=None, ckpt_every: int = 0):
    """Run the recurrence over all T tokens.

    Returns (o [B,T,H,d_v], S_T [B,H,d_k,d_v], ckpts) where ckpts[m-1] is the state
    after the first m*ckpt_every tokens (m = 1 .. T // ckpt_every).
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    g = np.asarray(g, np.float64)
    beta = np.asarray(beta, np.float64)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    S = np.zeros((B, H, dk, dv)) if S0 is None else np.array(S0, dtype=np.float64)
    o = np.empty((B, T, H, dv))
    ckpts = []
    for t in range(T):
        o[:, t], S = _step(S, q[:, t], k[:, t], v[:, t], g[:, t], beta[:, t])
        if ckpt_every and (t + 1) % ckpt_every == 0:
            ckpts.append(S.copy())
    return o, S, ckpts


def decode_step(S, q, k, v, g, beta):
    """One recurrent decode step for N independent sequences: S [N,H,d_k,d_v],
    q/k/g [N,H,d_k], v [N,H,d_v], beta [N,H].  Returns (o [N,H,d_v], S_new)."""
    return _step(np.asarray(S, np.float64), np.asarray(q, np.float64), np.asarray(k, np.float64),
                 np.asarray(v, np.float64), np.asarray(g, np.float64),
                 np.asarray(beta, np.float64))


def norm_gate(o, gate=None, eps: float = 1e-6, weight=None):
    """Per-head RMSNorm over the value axis, then the sigmoid output gate
    (recurrent-form entry of the "xhh.club" tag page 结构: per-head RMSNorm and a
    full-rank sigmoid output gate).  gate=None returns o unchanged."""
    if gate is None:
        return np.asarray(o, np.float64)
    o = np.asarray(o, np.float64)
    y = o / np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + eps)
    if weight is not None:
        y = y * np.asarray(weight, np.float64)
    return y / (1.0 + np.exp(-np.asarray(gate, np.float64)))
