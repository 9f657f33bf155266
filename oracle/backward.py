"""Gradients of the KDA recurrence, fp64 (test infrastructure only).

The pages give no backward pass; they say the chunkwise form is used for training too
("xhh.club" tag page 结构, entry on the chunkwise algorithm).  The gradient of a scalar
loss L follows from the forward definition (sequential.py): given dL/do for the raw
outputs o (before any norm or gate) and dL/dS_T for the final state, return dL/dq,
dL/dk, dL/dv, dL/dg, dL/dbeta and dL/dS0.

Computed by reverse-mode differentiation (torch autograd, CPU, float64) of the plain
recurrence.  To bound memory, the forward is run once storing the state at every
`block`-token boundary, then each block is re-run under autograd from its stored
entering state, in reverse order, receiving the gradient of the state after it.

Reading: the floor and clamp gt = min(0, max(-5, g)) pass the gradient where
-5 <= g <= 0 (torch.clamp's convention at the two kinks).
"""
from __future__ import annotations

import numpy as np


def _torch():
    import torch
    return torch


def _block(S, q, k, v, g, beta):
    """Run tokens t of one block (torch tensors, [B,t,H,*]) from state S; returns (o, S)."""
    torch = _torch()
    outs = []
    for t in range(q.shape[1]):
        gt = torch.clamp(g[:, t], -5.0, 0.0)
        Sp = torch.exp(gt)[..., :, None] * S                         # decay the key rows
        e = torch.einsum("bhi,bhij->bhj", k[:, t], Sp)               # S'^T k
        u = beta[:, t, :, None] * (v[:, t] - e)
        S = Sp + k[:, t, :, :, None] * u[..., None, :]               # write k u^T
        outs.append(torch.einsum("bhi,bhij->bhj", q[:, t], S))       # read after the write
    return torch.stack(outs, 1), S


def backward(q, k, v, g, beta, S0, do, dS_T=None, block: int = 64):
    """Gradients for inputs given as arrays holding the exact values the device receives
    (q/k/v [B,T,H,d], g [B,T,H,d_k], beta [B,T,H], S0 [B,H,d_k,d_v] or None, do
    [B,T,H,d_v], dS_T [B,H,d_k,d_v] or None).  Returns a dict of float64 arrays:
    dq, dk, dv, dg, dbeta, dS0 (and o, S_T of the forward)."""
    torch = _torch()
    f64 = torch.float64
    T_ = lambda a: torch.as_tensor(np.asarray(a, np.float64))   # noqa: E731
    q, k, v, g, beta, do = T_(q), T_(k), T_(v), T_(g), T_(beta), T_(do)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    S = torch.zeros((B, H, dk, dv), dtype=f64) if S0 is None else T_(S0).clone()
    # forward with stored block-entry states
    starts = list(range(0, T, block))
    entry = []
    o_all = torch.empty((B, T, H, dv), dtype=f64)
    with torch.no_grad():
        for t0 in starts:
            entry.append(S.clone())
            sl = slice(t0, min(T, t0 + block))
            o_all[:, sl], S = _block(S, q[:, sl], k[:, sl], v[:, sl], g[:, sl], beta[:, sl])
    S_T = S.clone()
    dS = torch.zeros((B, H, dk, dv), dtype=f64) if dS_T is None else T_(dS_T).clone()
    grads = {n: torch.zeros_like(x) for n, x in (("dq", q), ("dk", k), ("dv", v), ("dg", g),
                                                  ("dbeta", beta))}
    for t0, S_in in reversed(list(zip(starts, entry))):
        sl = slice(t0, min(T, t0 + block))
        leaves = [x[:, sl].clone().requires_grad_(True) for x in (q, k, v, g, beta)]
        Sl = S_in.clone().requires_grad_(True)
        o, S_out = _block(Sl, *leaves)
        L = (o * do[:, sl]).sum() + (S_out * dS).sum()
        gr = torch.autograd.grad(L, leaves + [Sl])
        for n, gx in zip(("dq", "dk", "dv", "dg", "dbeta"), gr[:5]):
            grads[n][:, sl] = gx
        dS = gr[5]
    out = {n: x.numpy() for n, x in grads.items()}
    out["dS0"] = dS.numpy()
    out["o"] = o_all.numpy()
    out["S_T"] = S_T.numpy()
    return out
