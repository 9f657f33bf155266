"""Pins of the CPU oracle against facts fixed outside it (CPU only).

The pages print no formula and no worked example, so the oracle is pinned by
exact arithmetic, closed forms, library routines and invariants of the recurrence:
  * exact rational brute force of the explicit transition matrices (T <= 8, d = 4)
    and a stored exact fixture (tests/golden/exact_tiny.json);
  * beta = 0: the state only decays, S_T = Diag(exp(sum gt)) S_0, o_t = S_0^T (exp(G_t) q_t);
  * exact recall: beta = 1, unit keys, q = k  =>  o_t = v_t for any decay;
  * d_k = 1 with constant coefficients is a first-order IIR filter (scipy.signal.lfilter);
  * standard-basis keys: every key row follows its own scalar recurrence;
  * chunkwise reformulation == recurrence for several chunk sizes and ragged tails;
  * segment maps: associativity, fold == sequential state, scan == checkpoints,
    and summing per-segment states is wrong;
  * 512-token-style checkpoints and resume; floor and upper clamp of the log-decay;
  * norm/gate identities.
test_oracle_mutants.py checks that plausible mistakes planted in the oracle fail
at least one of these pins.
"""
import json
import math
import os
from fractions import Fraction as Fr

import numpy as np
import pytest
import scipy.signal

import oracle
from oracle import chunkwise, recurrent, norm_gate, segment_map, compose, fold, exclusive_scan
from oracle import apply_map
from oracle import native
from oracle.exact import brute_force
from kda_inputs import make_prefill, to_f64, BF16, F32, make_decode_step, make_decode_state

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _rel(a, b):
    return float(np.max(np.abs(np.asarray(a) - np.asarray(b))) / max(1e-300, np.max(np.abs(b))))


# ---------------------------------------------------------------------------
# pin helpers (also used by the mutant test)
# ---------------------------------------------------------------------------
def pin_exact_error(seed=0, T=8, dk=4, dv=3):
    """Max relative error of recurrent() against the exact rational brute force."""
    rng = np.random.default_rng(seed)
    alpha = rng.choice([1.0, 0.9375, 0.875, 0.75, 0.625, 0.5, 0.25, 0.125], size=(T, dk))
    q = rng.standard_normal((T, dk))
    k = rng.standard_normal((T, dk))
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = rng.standard_normal((T, dv))
    beta = rng.uniform(0.05, 1.0, size=T)
    S0 = rng.standard_normal((dk, dv)) * 0.3
    o_ex, S_ex = brute_force(q.tolist(), k.tolist(), v.tolist(), alpha.tolist(), beta.tolist(),
                             S0.tolist())
    o_ex = np.array([[float(x) for x in r] for r in o_ex])
    S_ex = np.array([[float(x) for x in r] for r in S_ex])
    g = np.log(alpha)
    o, S, _ = recurrent(q[None, :, None], k[None, :, None], v[None, :, None], g[None, :, None],
                        beta[None, :, None], S0[None, None])
    return max(_rel(o[0, :, 0], o_ex), _rel(S[0, 0], S_ex))


def pin_beta_zero_error(seed=1):
    rng = np.random.default_rng(seed)
    B, T, H, dk, dv = 2, 37, 2, 6, 5
    q = rng.standard_normal((B, T, H, dk))
    k = rng.standard_normal((B, T, H, dk))
    v = rng.standard_normal((B, T, H, dv))
    g = rng.uniform(-8.0, 1.0, size=(B, T, H, dk))       # crosses the floor and zero
    beta = np.zeros((B, T, H))
    S0 = rng.standard_normal((B, H, dk, dv))
    o, S, _ = recurrent(q, k, v, g, beta, S0)
    gt = np.clip(g, -5.0, 0.0)
    G = np.cumsum(gt, axis=1)                              # [B,T,H,dk]
    S_exp = np.exp(G[:, -1])[..., None] * S0
    o_exp = np.einsum("bthi,bhij->bthj", np.exp(G) * q, S0)
    return max(_rel(o, o_exp), _rel(S, S_exp))


def pin_recall_error(seed=2):
    rng = np.random.default_rng(seed)
    B, T, H, dk, dv = 1, 50, 3, 8, 4
    k = rng.standard_normal((B, T, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, dv))
    g = rng.uniform(-6.0, 0.0, size=(B, T, H, dk))
    beta = np.ones((B, T, H))
    S0 = rng.standard_normal((B, H, dk, dv))
    o, _, _ = recurrent(k, k, v, g, beta, S0)
    return _rel(o, v)


def pin_iir_error(seed=3):
    rng = np.random.default_rng(seed)
    T, dv = 200, 3
    kappa, b, gam = 0.8, 0.6, -0.3
    a = (1.0 - b * kappa * kappa) * math.exp(gam)
    v = rng.standard_normal((T, dv))
    q = rng.standard_normal(T)
    s0 = rng.standard_normal(dv)
    exp_s = np.stack([scipy.signal.lfilter([b * kappa], [1.0, -a], v[:, j], zi=[a * s0[j]])[0]
                      for j in range(dv)], axis=1)
    o, S, _ = recurrent(q[None, :, None, None], np.full((1, T, 1, 1), kappa), v[None, :, None],
                        np.full((1, T, 1, 1), gam), np.full((1, T, 1), b), s0[None, None, None])
    return max(_rel(o[0, :, 0], q[:, None] * exp_s), _rel(S[0, 0, 0], exp_s[-1]))


def pin_basis_error(seed=4):
    rng = np.random.default_rng(seed)
    T, dk, dv = 40, 8, 5
    pi = rng.integers(0, dk, size=T)
    k = np.eye(dk)[pi]
    q = rng.standard_normal((T, dk))
    v = rng.standard_normal((T, dv))
    g = rng.uniform(-7.0, 0.5, size=(T, dk))
    beta = rng.uniform(0.0, 1.0, size=T)
    S0 = rng.standard_normal((dk, dv))
    rows = [S0[i].copy() for i in range(dk)]
    o_exp = np.zeros((T, dv))
    for t in range(T):
        a = np.exp(np.clip(g[t], -5.0, 0.0))
        rows = [a[i] * rows[i] for i in range(dk)]
        i = pi[t]
        rows[i] = (1.0 - beta[t]) * rows[i] + beta[t] * v[t]
        o_exp[t] = sum(q[t, i] * rows[i] for i in range(dk))
    o, S, _ = recurrent(q[None, :, None], k[None, :, None], v[None, :, None], g[None, :, None],
                        beta[None, :, None], S0[None, None])
    return max(_rel(o[0, :, 0], o_exp), _rel(S[0, 0], np.stack(rows)))


def pin_golden_error():
    with open(os.path.join(os.path.dirname(__file__), "golden", "exact_tiny.json")) as f:
        G = json.load(f)
    q, k, v = (np.array(G[x]) for x in ("q", "k", "v"))
    alpha, beta, S0 = np.array(G["alpha"]), np.array(G["beta"]), np.array(G["S0"])
    o_ex = np.array([[float(Fr(x)) for x in r] for r in G["o"]])
    S_ex = np.array([[float(Fr(x)) for x in r] for r in G["S"]])
    o, S, _ = recurrent(q[None, :, None], k[None, :, None], v[None, :, None],
                        np.log(alpha)[None, :, None], beta[None, :, None], S0[None, None])
    return max(_rel(o[0, :, 0], o_ex), _rel(S[0, 0], S_ex))


def pin_deltanet_error(seed=3, T=12, dk=6, dv=5):
    """alpha == 1 (g = 0) is plain DeltaNet: every token takes one gradient-descent step of
    size beta_t on the regression loss 1/2 ||S^T k_t - v_t||^2.  The gradient comes from
    torch autograd in fp64, not from a hand-written update."""
    import torch
    rng = np.random.default_rng(seed)
    q, k = rng.standard_normal((T, dk)), rng.standard_normal((T, dk))
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = rng.standard_normal((T, dv))
    beta = rng.uniform(0.1, 0.9, T)
    S0 = rng.standard_normal((dk, dv))
    S = torch.tensor(S0, dtype=torch.float64)
    o_exp = np.zeros((T, dv))
    for t in range(T):
        Sv = S.clone().requires_grad_(True)
        kt, vt = torch.tensor(k[t]), torch.tensor(v[t])
        loss = 0.5 * torch.sum((Sv.T @ kt - vt) ** 2)
        (grad,) = torch.autograd.grad(loss, Sv)
        S = (S - beta[t] * grad).detach()
        o_exp[t] = (S.T @ torch.tensor(q[t])).numpy()
    g = np.zeros((T, dk))
    o, Sr, _ = recurrent(q[None, :, None], k[None, :, None], v[None, :, None], g[None, :, None],
                         beta[None, :, None], S0[None, None])
    return max(_rel(o[0, :, 0], o_exp), _rel(Sr[0, 0], S.numpy()))


PINS = {
    "deltanet": (pin_deltanet_error, 1e-12),
    "exact": (pin_exact_error, 1e-12),
    "beta0": (pin_beta_zero_error, 1e-12),
    "recall": (pin_recall_error, 1e-10),
    "iir": (pin_iir_error, 1e-10),
    "basis": (pin_basis_error, 1e-12),
    "golden": (pin_golden_error, 1e-12),
}


@pytest.mark.parametrize("name", sorted(PINS))
def test_pin(name):
    fn, tol = PINS[name]
    assert fn() <= tol


@pytest.mark.parametrize("seed", [10, 11, 12])
def test_exact_bruteforce_seeds(seed):
    assert pin_exact_error(seed=seed, T=7, dk=4, dv=2) <= 1e-12


# ---------------------------------------------------------------------------
# chunkwise == recurrent
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("chunk", [1, 3, 16, 64])
def test_chunkwise_matches_recurrent(chunk):
    c = make_prefill(2, 150, 2, 32, seed=5, in_dtype=F32, s0_std=0.1, g_mode="raw")
    q, k, v = (to_f64(x, F32) for x in (c.q, c.k, c.v))
    o1, S1, _ = recurrent(q, k, v, c.g, c.beta, c.S0)
    o2, S2 = chunkwise(q, k, v, c.g, c.beta, c.S0, chunk=chunk)
    assert _rel(o2, o1) <= 1e-11
    assert _rel(S2, S1) <= 1e-12


def test_chunkwise_full_width_bf16():
    c = make_prefill(1, 130, 2, 128, seed=6, in_dtype=BF16, s0_std=0.01)
    q, k, v = (to_f64(x, BF16) for x in (c.q, c.k, c.v))
    o1, S1, _ = recurrent(q, k, v, c.g, c.beta, c.S0)
    o2, S2 = chunkwise(q, k, v, c.g, c.beta, c.S0, chunk=64)
    assert _rel(o2, o1) <= 1e-11 and _rel(S2, S1) <= 1e-12


# ---------------------------------------------------------------------------
# C oracle == numpy oracle
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", [F32, BF16])
def test_native_matches_numpy(dtype):
    c = make_prefill(2, 96, 3, 128, 40, seed=7, in_dtype=dtype, s0_std=0.05, g_mode="raw")
    o1, S1, ck1 = recurrent(to_f64(c.q, dtype), to_f64(c.k, dtype), to_f64(c.v, dtype), c.g,
                            c.beta, c.S0, ckpt_every=32)
    o2, S2, ck2 = native.prefill(c.q, c.k, c.v, c.g, c.beta, c.S0, bf16=(dtype == BF16),
                                 ckpt_every=32, nthreads=3)
    assert _rel(o2, o1) <= 1e-13 and _rel(S2, S1) <= 1e-13
    for m in range(3):
        assert _rel(ck2[:, m], ck1[m]) <= 1e-13


def test_native_golden():
    with open(os.path.join(os.path.dirname(__file__), "golden", "exact_tiny.json")) as f:
        G = json.load(f)
    q, k, v = (np.array(G[x], np.float32)[None, :, None] for x in ("q", "k", "v"))
    g = np.log(np.array(G["alpha"])).astype(np.float32)[None, :, None]
    beta = np.array(G["beta"], np.float32)[None, :, None]
    S0 = np.array(G["S0"], np.float32)[None, None]
    o, S, _ = native.prefill(q, k, v, g, beta, S0, bf16=False)
    o_ex = np.array([[float(Fr(x)) for x in r] for r in G["o"]])
    S_ex = np.array([[float(Fr(x)) for x in r] for r in G["S"]])
    # g is stored in fp32, so alpha carries ~6e-8 relative error
    assert _rel(o[0, :, 0], o_ex) <= 1e-6 and _rel(S[0, 0], S_ex) <= 1e-6


def test_native_decode_matches_numpy():
    N, H, d = 5, 3, 128
    S = make_decode_state(N, H, d, seed=1).astype(np.float64)
    S_np = S.copy()
    for step in range(3):
        st = make_decode_step(N, H, d, seed=1, step=step)
        o_c = native.decode_step(S, st.q, st.k, st.v, st.g, st.beta, bf16=True)
        o_n, S_np = oracle.decode_step(S_np, to_f64(st.q, BF16), to_f64(st.k, BF16),
                                       to_f64(st.v, BF16), st.g, st.beta)
        assert _rel(o_c, o_n) <= 1e-13
    assert _rel(S, S_np) <= 1e-13


def test_decode_step_is_one_prefill_token():
    c = make_prefill(3, 1, 2, 16, seed=8, in_dtype=F32, s0_std=0.2)
    o1, S1, _ = recurrent(c.q, c.k, c.v, c.g, c.beta, c.S0)
    o2, S2 = oracle.decode_step(c.S0, c.q[:, 0], c.k[:, 0], c.v[:, 0], c.g[:, 0], c.beta[:, 0])
    assert _rel(o2, o1[:, 0]) == 0.0 and _rel(S2, S1) == 0.0


# ---------------------------------------------------------------------------
# decay floor and clamp
# ---------------------------------------------------------------------------
def test_floor_clamps_below_minus_five():
    a = make_prefill(1, 40, 2, 16, seed=9, in_dtype=F32, g_mode="floor", s0_std=0.1)
    b = make_prefill(1, 40, 2, 16, seed=9, in_dtype=F32, g_mode="below_floor", s0_std=0.1)
    assert np.all(b.g < -5.0)
    oa, Sa, _ = recurrent(a.q, a.k, a.v, a.g, a.beta, a.S0)
    ob, Sb, _ = recurrent(b.q, b.k, b.v, b.g, b.beta, b.S0)
    assert np.array_equal(oa, ob) and np.array_equal(Sa, Sb)


def test_positive_log_decay_clamps_to_zero():
    a = make_prefill(1, 20, 1, 8, seed=10, in_dtype=F32, g_mode="zero", s0_std=0.1)
    g_pos = np.full_like(a.g, 0.7)
    o1, S1, _ = recurrent(a.q, a.k, a.v, a.g, a.beta, a.S0)
    o2, S2, _ = recurrent(a.q, a.k, a.v, g_pos, a.beta, a.S0)
    assert np.array_equal(o1, o2) and np.array_equal(S1, S2)


# ---------------------------------------------------------------------------
# segments, scan, checkpoints
# ---------------------------------------------------------------------------
def _small_case(T=96, dk=8, dv=6, seed=11):
    c = make_prefill(1, T, 2, dk, dv, seed=seed, in_dtype=F32, s0_std=0.3, g_mode="raw")
    return c, to_f64(c.q, F32), to_f64(c.k, F32), to_f64(c.v, F32)


def test_scan_associative():
    c, q, k, v = _small_case()
    m = [segment_map(k[:, s:s + 32], v[:, s:s + 32], c.g[:, s:s + 32], c.beta[:, s:s + 32])
         for s in (0, 32, 64)]
    left = compose(m[2], compose(m[1], m[0]))
    right = compose(compose(m[2], m[1]), m[0])
    assert _rel(left[0], right[0]) <= 1e-12 and _rel(left[1], right[1]) <= 1e-12


def test_segment_map_is_affine_in_state():
    c, q, k, v = _small_case()
    A, Bm = segment_map(k, v, c.g, c.beta)
    _, S1, _ = recurrent(q, k, v, c.g, c.beta, c.S0)
    _, S0run, _ = recurrent(q, k, v, c.g, c.beta, None)
    assert _rel(Bm, S0run) <= 1e-12
    assert _rel(A @ c.S0 + Bm, S1) <= 1e-12


def test_fold_scan_checkpoints_and_negative_sum():
    c, q, k, v = _small_case(T=128)
    L = 32
    maps = [segment_map(k[:, s:s + L], v[:, s:s + L], c.g[:, s:s + L], c.beta[:, s:s + L])
            for s in range(0, 128, L)]
    _, S_T, ck = recurrent(q, k, v, c.g, c.beta, c.S0, ckpt_every=L)
    assert _rel(apply_map(fold(maps), c.S0), S_T) <= 1e-12
    S_in = exclusive_scan(maps, c.S0)
    assert _rel(S_in[0], c.S0) == 0.0
    for s in range(1, 4):
        assert _rel(S_in[s], ck[s - 1]) <= 1e-12
    # Context parallelism cannot add the per-segment states: that answer is far off.
    summed = sum(m[1] for m in maps) + c.S0
    assert _rel(summed, S_T) > 0.1


def test_checkpoints_and_resume():
    c, q, k, v = _small_case(T=160)
    _, S_T, ck = recurrent(q, k, v, c.g, c.beta, c.S0, ckpt_every=64)
    assert len(ck) == 2
    for m in range(2):
        n = 64 * (m + 1)
        _, S_pref, _ = recurrent(q[:, :n], k[:, :n], v[:, :n], c.g[:, :n], c.beta[:, :n], c.S0)
        assert np.array_equal(ck[m], S_pref)
    o_full, _, _ = recurrent(q, k, v, c.g, c.beta, c.S0)
    o_res, S_res, _ = recurrent(q[:, 128:], k[:, 128:], v[:, 128:], c.g[:, 128:],
                                c.beta[:, 128:], ck[1])
    assert np.array_equal(S_res, S_T) and np.array_equal(o_res, o_full[:, 128:])


def test_state_size_independent_of_T():
    shapes = set()
    for T in (0, 1, 17, 300):
        c = make_prefill(1, T, 2, 16, 8, seed=12, in_dtype=F32)
        _, S, _ = recurrent(c.q, c.k, c.v, c.g, c.beta, None)
        shapes.add(S.shape)
    assert shapes == {(1, 2, 16, 8)}


# ---------------------------------------------------------------------------
# norm and gate
# ---------------------------------------------------------------------------
def test_norm_gate_identities():
    rng = np.random.default_rng(13)
    o = rng.standard_normal((3, 7, 2, 128)) * 0.1
    eps = 1e-6
    y = norm_gate(o, np.zeros_like(o), eps) * 2.0             # gate 0 multiplies by exactly 0.5
    ms = np.mean(o * o, axis=-1)
    assert np.allclose(np.mean(y * y, axis=-1), ms / (ms + eps), rtol=1e-12, atol=0)
    big = norm_gate(o, np.full_like(o, 800.0), eps)           # sigmoid -> 1
    assert np.allclose(big, y, rtol=1e-15, atol=0)
    assert np.array_equal(norm_gate(o, None), o)
    w = rng.standard_normal(128)
    assert np.allclose(norm_gate(o, np.zeros_like(o), eps, weight=w) * 2.0, y * w, rtol=1e-13)
