"""Exact rational brute force for tiny KDA cases (test infrastructure only).

Runs the state map of each token, S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1}
+ beta_t k_t v_t^T, and the read-out o_t = S_t^T q_t in exact rational arithmetic
(fractions.Fraction) with explicit matrices.  Decays are given directly as
rationals alpha_t (no logarithm), so nothing is rounded.  This is the matrix form of
the recurrent-form entry of the "xhh.club" tag page 结构 (decay, then erase the
old value along k and write the new one), written independently of sequential.py.
"""
from __future__ import annotations

from fractions import Fraction as Fr


def _matmul(a, b):
    n, m, p = len(a), len(b), len(b[0])
    return [[sum((a[i][x] * b[x][j] for x in range(m)), Fr(0)) for j in range(p)] for i in range(n)]


def brute_force(q, k, v, alpha, beta, S0=None):
    """q, k, alpha: T x d_k nested lists; v: T x d_v; beta: T.  All entries are
    converted to Fraction exactly (floats included).  Returns (o, S) as Fractions."""
    T = len(q)
    dk = len(k[0])
    dv = len(v[0])
    S = [[Fr(0)] * dv for _ in range(dk)] if S0 is None else [[Fr(x) for x in r] for r in S0]
    out = []
    for t in range(T):
        kt = [Fr(x) for x in k[t]]
        bt = Fr(beta[t])
        at = [Fr(x) for x in alpha[t]]
        M = [[(Fr(1) if i == j else Fr(0)) - bt * kt[i] * kt[j] for j in range(dk)] for i in range(dk)]
        M = [[M[i][j] * at[j] for j in range(dk)] for i in range(dk)]   # right-multiply by Diag(alpha)
        S = _matmul(M, S)
        vt = [Fr(x) for x in v[t]]
        S = [[S[i][j] + bt * kt[i] * vt[j] for j in range(dv)] for i in range(dk)]
        qt = [Fr(x) for x in q[t]]
        out.append([sum((S[i][j] * qt[i] for i in range(dk)), Fr(0)) for j in range(dv)])
    return out, S
