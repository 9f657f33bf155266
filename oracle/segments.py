"""Segment state maps and their associative scan, fp64 (test infrastructure only).

The structure-implications entry of the "xhh.club" tag page 结构 says context
parallelism for KDA decomposes by an associative prefix scan rather than by adding
states; the "nlpx.cn" K3 reading guide, section 6, names the exchanged object a
segment transition and asks why per-rank states cannot simply be summed.

Every token acts on the state as an affine map  S -> M_t S + N_t  with
  M_t = (I - beta_t k_t k_t^T) Diag(exp(gt_t)),   N_t = beta_t k_t v_t^T,
which is the one-step update of the recurrence rewritten (S' = Diag(a) S,
S' + k beta (v - S'^T k)^T = (I - beta k k^T) S' + beta k v^T).  A segment's map is
the composition of its tokens' maps:  (A, B)  with  S_out = A S_in + B.
Composition (later after earlier):  (A2, B2) o (A1, B1) = (A2 A1, A2 B1 + B2).
"""
from __future__ import annotations

import numpy as np

from .sequential import clamp_decay


def segment_map(k, v, g, beta):
    """Map of one token range for every (batch, head): k/g [B,L,H,d_k], v [B,L,H,d_v],
    beta [B,L,H].  Returns (A [B,H,d_k,d_k], B [B,H,d_k,d_v]) by explicit products of
    the per-token matrices."""
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    g = np.asarray(g, np.float64)
    beta = np.asarray(beta, np.float64)
    Bn, L, H, dk = k.shape
    dv = v.shape[-1]
    A = np.broadcast_to(np.eye(dk), (Bn, H, dk, dk)).copy()
    Bm = np.zeros((Bn, H, dk, dv))
    eye = np.eye(dk)
    for t in range(L):
        kt = k[:, t]
        bt = beta[:, t][..., None, None]
        M = (eye - bt * (kt[..., :, None] * kt[..., None, :])) * np.exp(clamp_decay(g[:, t]))[..., None, :]
        N = bt * (kt[..., :, None] * v[:, t][..., None, :])
        A = M @ A
        Bm = M @ Bm + N
    return A, Bm


def compose(later, earlier):
    """(A2, B2) o (A1, B1) = (A2 A1, A2 B1 + B2): apply `earlier`, then `later`."""
    A2, B2 = later
    A1, B1 = earlier
    return A2 @ A1, A2 @ B1 + B2


def apply_map(m, S):
    A, B = m
    return A @ S + B


def fold(maps):
    """Compose a list of maps in sequence order (maps[0] first)."""
    acc = maps[0]
    for m in maps[1:]:
        acc = compose(m, acc)
    return acc


def exclusive_scan(maps, S0):
    """States entering each segment: S_in[0] = S0, S_in[s+1] = map_s(S_in[s])."""
    out = [np.asarray(S0, np.float64)]
    for m in maps[:-1]:
        out.append(apply_map(m, out[-1]))
    return out
