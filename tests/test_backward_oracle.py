"""Pins of the backward oracle (CPU): central finite differences of the forward oracle
on tiny cases, and the closed form with beta = 0, where the state only decays:
S_t = Diag(e^{G_t}) S0 and o_t = S_t^T q_t, with G_t the cumulative floored log-decay."""
import numpy as np
import pytest

from oracle import recurrent
from oracle.backward import backward


def _case(seed, B=1, T=7, H=1, dk=4, dv=3, beta_zero=False):
    r = np.random.default_rng(seed)
    q = r.standard_normal((B, T, H, dk))
    k = r.standard_normal((B, T, H, dk)) * 0.7
    v = r.standard_normal((B, T, H, dv))
    # log-decays away from the kinks at -5 and 0 (finite differences straddle no kink),
    # including clamped ones below -5 and above 0
    g = r.uniform(-6.0, 0.5, (B, T, H, dk))
    g = np.where(np.abs(g + 5.0) < 0.05, g - 0.1, g)
    g = np.where(np.abs(g) < 0.05, g - 0.1, g)
    beta = np.zeros((B, T, H)) if beta_zero else r.uniform(0.05, 0.95, (B, T, H))
    S0 = r.standard_normal((B, H, dk, dv)) * 0.5
    do = r.standard_normal((B, T, H, dv))
    dS = r.standard_normal((B, H, dk, dv))
    return q, k, v, g, beta, S0, do, dS


def _loss(q, k, v, g, beta, S0, do, dS):
    o, S, _ = recurrent(q, k, v, g, beta, S0)
    return float(np.sum(o * do) + np.sum(S * dS))


@pytest.mark.parametrize("seed,block", [(0, 64), (1, 3), (2, 2)])
def test_backward_matches_finite_differences(seed, block):
    """Every input of a 7-token, d_k=4, d_v=3 case; blocks of 2 and 3 exercise the
    block-wise re-run of the oracle."""
    q, k, v, g, beta, S0, do, dS = _case(seed)
    gr = backward(q, k, v, g, beta, S0, do, dS, block=block)
    args = [q, k, v, g, beta, S0]
    names = ["dq", "dk", "dv", "dg", "dbeta", "dS0"]
    eps = 1e-6
    for ai, name in enumerate(names):
        x = args[ai]
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            a_p = list(args); a_p[ai] = xp
            a_m = list(args); a_m[ai] = xm
            fd[idx] = (_loss(*a_p, do, dS) - _loss(*a_m, do, dS)) / (2 * eps)
        scale = np.max(np.abs(fd)) + 1e-12
        assert np.max(np.abs(gr[name] - fd)) <= 1e-6 * scale + 1e-9, name


def test_backward_beta_zero_closed_form():
    """beta = 0: no writes.  dq_t = e^{G_t} (S0 do_t); dk = dv = 0;
    dS0 = sum_t (e^{G_t} q_t) do_t^T + e^{G_T} dS_T;
    dG_t = e^{G_t} q_t (S0 do_t) for t < T plus e^{G_T} rowsum(S0 dS_T) at t = T,
    dg_u = sum_{t >= u} dG_t where -5 <= g_u <= 0, else 0."""
    q, k, v, g, beta, S0, do, dS = _case(3, T=9, dk=5, dv=4, beta_zero=True)
    gr = backward(q, k, v, g, beta, S0, do, dS, block=4)
    gt = np.minimum(0.0, np.maximum(-5.0, g))
    G = np.cumsum(gt, axis=1)                                   # [B,T,H,dk]
    E = np.exp(G)
    Sd = np.einsum("bhij,bthj->bthi", S0, do)                   # S0 do_t
    assert np.allclose(gr["dq"], E * Sd, rtol=1e-12, atol=1e-12)
    assert np.allclose(gr["dk"], 0.0, atol=1e-12) and np.allclose(gr["dv"], 0.0, atol=1e-12)
    dS0 = np.einsum("bthi,bthj->bhij", E * q, do) + E[:, -1, :, :, None] * dS
    assert np.allclose(gr["dS0"], dS0, rtol=1e-12, atol=1e-12)
    dG = E * q * Sd
    dG[:, -1] += E[:, -1] * np.einsum("bhij,bhij->bhi", S0, dS)
    dg = np.flip(np.cumsum(np.flip(dG, 1), 1), 1) * ((g >= -5.0) & (g <= 0.0))
    assert np.allclose(gr["dg"], dg, rtol=1e-10, atol=1e-12)
