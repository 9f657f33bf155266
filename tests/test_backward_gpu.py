"""GPU parity of the backward pass (kda_prefill_backward), through the C ABI, against the
fp64 autograd oracle (oracle.backward) on the same seeded input bytes.

The GPU path computes in fp32 (fp32 MFMA); the oracle in fp64.  Tolerance per gradient:
err = max|x - x_ref| / rms(x_ref) <= 2e-3 (dS0: Frobenius relative error <= 1e-4).  The
bound covers fp32 rounding through the chunk's triangular solve, the 64-token reverse
cumulative sum of the decay gradient and the sweep over up to a few hundred chunks.
"""
import sys

import numpy as np
import pytest
import torch

import linear_attention_sequence_kda_amd as kda
from kda_inputs import BF16, F32, make_output_grads, make_prefill, make_workload, to_f64
from oracle import native
from oracle.backward import backward
from gpu_util import up, down, err_o, err_S, dev

pytestmark = pytest.mark.gpu

TOL = 2e-3
TOL_S = 1e-4
NAMES = ("dq", "dk", "dv", "dg", "dbeta")


def _say(*a):
    print(*a, flush=True, file=sys.stderr)


def run_gpu_t(c, dO, dS, *, S0=True):
    """Gradients as device tensors."""
    B, T, H = c.B, c.T, c.H
    nan = float("nan")
    out = {n: torch.full((B, T, H, 128), nan, device=dev()) for n in ("dq", "dk", "dv", "dg")}
    out["dbeta"] = torch.full((B, T, H), nan, device=dev())
    out["dS0"] = torch.full((B, H, 128, 128), nan, device=dev())
    kda.kda_prefill_backward(up(c.q), up(c.k), up(c.v), up(c.g), up(c.beta), up(dO),
                             S0=up(c.S0) if S0 else None, dS_final=up(dS), **out)
    torch.cuda.synchronize()
    return out


def run_gpu(c, dO, dS, *, S0=True):
    return {n: down(t) for n, t in run_gpu_t(c, dO, dS, S0=S0).items()}


def run_oracle(c, dO, dS, *, S0=True):
    f = lambda x: to_f64(x, c.in_dtype)  # noqa: E731
    return backward(f(c.q), f(c.k), f(c.v), c.g.astype(np.float64), c.beta.astype(np.float64),
                    c.S0.astype(np.float64) if (S0 and c.S0 is not None) else None,
                    dO.astype(np.float64), None if dS is None else dS.astype(np.float64))


def check(c, dO, dS, label, *, S0=True):
    _say(f"backward {label}: B={c.B} T={c.T} H={c.H} {c.in_dtype}")
    got = run_gpu(c, dO, dS, S0=S0)
    ref = run_oracle(c, dO, dS, S0=S0)
    for n in NAMES:
        assert np.isfinite(got[n]).all(), n
        if not np.any(ref[n]):       # an all-zero gradient (e.g. dg with every g below -5)
            assert not np.any(got[n]), n
            _say(f"  {n}: zero, as the reference")
            continue
        e = err_o(got[n], ref[n])
        _say(f"  {n}: err={e:.3e}")
        assert e <= TOL, n
    e = err_S(got["dS0"], ref["dS0"])
    _say(f"  dS0: err={e:.3e}")
    assert e <= TOL_S


def test_backward_bf16_ragged_with_state():
    """Four chunks with an 8-token tail, two heads, an initial state and a final-state
    gradient."""
    c = make_prefill(1, 200, 2, 128, seed=31, in_dtype=BF16, s0_std=0.05)
    dO, dS = make_output_grads(1, 200, 2, seed=31)
    check(c, dO, dS, "bf16 T=200")


def test_backward_f32_short_no_state():
    """fp32 inputs, two sequences of one partial chunk, no S0 and no dS_T."""
    c = make_prefill(2, 37, 1, 128, seed=32, in_dtype=F32)
    dO, _ = make_output_grads(2, 37, 1, seed=32)
    check(c, dO, None, "f32 T=37", S0=False)


def test_backward_clamp_crossing_decays():
    """Raw log-decays that cross the -5 floor and sit above 0 in places: the clamp's
    zero gradient outside [-5, 0]."""
    c = make_prefill(1, 130, 1, 128, seed=33, in_dtype=BF16, s0_std=0.05, g_mode="raw")
    g = c.g.copy()
    g[0, ::7, 0, ::5] = 0.3           # above 0: clamped to 0
    c.g = g
    dO, dS = make_output_grads(1, 130, 1, seed=33)
    check(c, dO, dS, "raw decays T=130")


def test_backward_full_chunks_beta_one():
    c = make_prefill(1, 128, 2, 128, seed=34, in_dtype=BF16, s0_std=0.05, beta_mode="one")
    dO, dS = make_output_grads(1, 128, 2, seed=34)
    check(c, dO, dS, "beta=1 T=128")


def test_backward_floor_decays_many_chunks():
    """Every decay at the floor (the steepest within-block factors, e^75) over 9 chunks."""
    c = make_prefill(1, 576, 1, 128, seed=35, in_dtype=BF16, s0_std=0.05, g_mode="floor")
    dO, dS = make_output_grads(1, 576, 1, seed=35)
    check(c, dO, dS, "floor T=576")


def test_backward_empty_sequence():
    """T = 0: dS0 = dS_T."""
    c = make_prefill(2, 0, 3, 128, seed=36, in_dtype=BF16)
    _, dS = make_output_grads(2, 0, 3, seed=36)
    dS0 = torch.full((2, 3, 128, 128), float("nan"), device=dev())
    e = torch.empty((2, 0, 3, 128), device=dev())
    kda.kda_prefill_backward(up(c.q), up(c.k), up(c.v), up(c.g), up(c.beta), e, dq=e, dk=e, dv=e,
                             dg=e, dbeta=torch.empty((2, 0, 3), device=dev()), dS_final=up(dS),
                             dS0=dS0)
    torch.cuda.synchronize()
    assert torch.equal(dS0.cpu(), torch.from_numpy(dS))


def test_backward_one_head_2k_of_the_prefill_workload():
    """A whole head of the prefill workload's distributions over 2048 tokens (32 chunks),
    every gradient against the oracle."""
    c = make_workload("prefill_8k", seed=5, T=2048, B=1, H=1, in_dtype=BF16)
    dO, dS = make_output_grads(1, 2048, 1, seed=5)
    check(c, dO, dS, "prefill workload, one head, T=2048")


def test_backward_full_size_sampled_dq():
    """The full prefill workload (B=4, T=8192, H=16, S0): o_t = S_t^T q_t and S_t does not
    depend on q_t, so dq_t = S_t dO_t exactly, with S_t the state after token t.  S_t from
    the fp64 oracle over the prefix, at sampled (b, t, h) on chunk edges, inside chunks
    and at the last token; every gradient finite."""
    c = make_workload("prefill_8k", seed=0)
    B, T, H = c.B, c.T, c.H
    dO, dS = make_output_grads(B, T, H, seed=0)
    _say(f"backward full size: B={B} T={T} H={H}")
    got = run_gpu_t(c, dO, dS)
    for n, t in got.items():
        assert bool(torch.isfinite(t).all()), n
    dq = got["dq"]
    samples = [(0, 0, 0), (1, 63, 5), (2, 64, 11), (3, 4095, 15), (0, 8191, 7), (2, 5000, 3),
               (3, 8191, 0), (1, 2047, 9)]
    err = []
    for b, t, h in samples:
        sl = (slice(b, b + 1), slice(0, t + 1), slice(h, h + 1))
        _, St, _ = native.prefill(c.q[sl], c.k[sl], c.v[sl], c.g[sl], c.beta[sl],
                                  c.S0[b:b + 1, h:h + 1], bf16=True, want_o=False)
        ref = St[0, 0] @ dO[b, t, h].astype(np.float64)
        e = err_o(down(dq[b, t, h]), ref)
        _say(f"  dq at (b={b}, t={t}, h={h}): err={e:.3e}")
        err.append(e)
    assert max(err) <= TOL


def test_backward_f32_multi_chunk_heads():
    """fp32 inputs over five chunks (ragged), three sequences of two heads."""
    c = make_prefill(3, 300, 2, 128, seed=37, in_dtype=F32, s0_std=0.05)
    dO, dS = make_output_grads(3, 300, 2, seed=37)
    check(c, dO, dS, "f32 T=300")


@pytest.mark.parametrize("g_mode", ["zero", "below_floor"])
def test_backward_decay_modes(g_mode):
    """No decay at all (g = 0: every factor 1, the pairwise sums undamped) and g = -7
    (below the floor: behaves as -5 and passes no gradient)."""
    c = make_prefill(1, 160, 2, 128, seed=38, in_dtype=BF16, s0_std=0.05, g_mode=g_mode)
    dO, dS = make_output_grads(1, 160, 2, seed=38)
    check(c, dO, dS, f"g={g_mode} T=160")


def test_backward_beta_zero_many_sequences():
    """beta = 0 (no writes: dk = dv = 0 exactly in the closed form) over 4 x 3 heads."""
    c = make_prefill(4, 90, 3, 128, seed=39, in_dtype=BF16, s0_std=0.05, beta_mode="zero")
    dO, dS = make_output_grads(4, 90, 3, seed=39)
    got = run_gpu(c, dO, dS)
    assert np.abs(got["dv"]).max() == 0.0
    ref = run_oracle(c, dO, dS)
    for n in ("dq", "dg", "dbeta"):
        e = err_o(got[n], ref[n])
        _say(f"  beta=0 {n}: err={e:.3e}")
        assert e <= TOL, n
    assert err_S(got["dS0"], ref["dS0"]) <= TOL_S
    assert np.abs(got["dk"]).max() <= 1e-6 * np.abs(ref["dq"]).max()


def test_backward_wide_sweep_units():
    """64 (sequence, head) pairs: enough for the sweeps' 32-column units (the smaller cases
    above run 16-column units); every gradient against the oracle, ragged tail."""
    c = make_prefill(4, 130, 16, 128, seed=40, in_dtype=BF16, s0_std=0.05)
    dO, dS = make_output_grads(4, 130, 16, seed=40)
    check(c, dO, dS, "64 heads x sequences, T=130")
