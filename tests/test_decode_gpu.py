"""GPU parity of the recurrent decode step and of checkpoint/rollback, through the
C ABI, against the fp64 CPU oracle on the same seeded input bytes.

Tolerance (fp32 decode): err_o = max|o - o_ref| / rms(o_ref) <= 1e-4 over all steps.
"""
import sys

import numpy as np
import pytest
import torch

import linear_attention_sequence_kda_amd as kda
from kda_inputs import (BF16, F32, f32_to_bf16, make_decode_state, make_decode_step,
                        make_decode_steps, to_f64)
from oracle import native, norm_gate
from gpu_util import up, down, err_o, err_S, bf16_out_tol, dev

pytestmark = pytest.mark.gpu

TOL_DECODE = 1e-4


def _say(*a):
    print(*a, flush=True, file=sys.stderr)


def _run_steps(N, H, steps, seed, in_dtype=BF16, out_dtype=torch.float32, gate=False,
               norm_weight=None):
    S_np = make_decode_state(N, H, 128, seed=seed)
    S_dev = up(S_np)
    S_ref = S_np.astype(np.float64)
    os_gpu, os_ref = [], []
    gen = np.random.default_rng([seed, 77])
    for s in range(steps):
        st = make_decode_step(N, H, 128, seed=seed, step=s, in_dtype=in_dtype)
        gt = None
        if gate:
            gt = gen.standard_normal((N, H, 128)).astype(np.float32)
            gt_store = gt if in_dtype == F32 else f32_to_bf16(gt)
        o = torch.empty((N, H, 128), dtype=out_dtype, device=dev())
        kda.kda_decode_step(up(st.q), up(st.k), up(st.v), up(st.g), up(st.beta), S_dev, o=o,
                            gate=up(gt_store) if gate else None,
                            norm_weight=None if norm_weight is None else up(norm_weight))
        o_ref = native.decode_step(S_ref, st.q, st.k, st.v, st.g, st.beta,
                                   bf16=(in_dtype == BF16))
        if gate:
            o_ref = norm_gate(o_ref, to_f64(gt_store, in_dtype), 1e-6, norm_weight)
        os_gpu.append(down(o))
        os_ref.append(o_ref)
    torch.cuda.synchronize()
    return np.stack(os_gpu), np.stack(os_ref), down(S_dev), S_ref


def test_decode_small_bf16_inputs():
    _say("decode small N=8 H=4 steps=64 bf16 in, f32 out")
    o, o_ref, S, S_ref = _run_steps(8, 4, 64, seed=3)
    e = err_o(o, o_ref)
    _say(f"err_o={e:.3e} err_S={err_S(S, S_ref):.3e}")
    assert e <= TOL_DECODE
    assert err_S(S, S_ref) <= 1e-5


def test_decode_f32_inputs():
    o, o_ref, S, S_ref = _run_steps(3, 5, 32, seed=4, in_dtype=F32)
    assert err_o(o, o_ref) <= TOL_DECODE and err_S(S, S_ref) <= 1e-5


def test_decode_gate_norm_f32_out():
    w = np.random.default_rng(5).uniform(0.5, 1.5, 128).astype(np.float32)
    o, o_ref, S, S_ref = _run_steps(4, 3, 16, seed=5, gate=True, norm_weight=w)
    assert err_o(o, o_ref) <= TOL_DECODE


def test_decode_bf16_out():
    o, o_ref, S, S_ref = _run_steps(4, 3, 16, seed=6, out_dtype=torch.bfloat16)
    assert err_o(o, o_ref) <= bf16_out_tol(o_ref, TOL_DECODE)
    assert err_S(S, S_ref) <= 1e-5


@pytest.mark.parametrize("N,H", [(1, 8), (17, 15), (16, 16), (9, 29)])
def test_decode_whole_and_split_states(N, H):
    """Below 256 states an ungated step splits each state into four 32-column slices,
    from 256 on a workgroup takes a whole state: both sides of the threshold, state counts
    that are not a multiple of eight, and the one-sequence x 8-head step of the long
    prefill's decode tail."""
    path = "split" if N * H < 256 else "whole"
    _say(f"decode N={N} H={H} ({N * H} states, {path} path), 8 steps")
    o, o_ref, S, S_ref = _run_steps(N, H, 8, seed=N * 100 + H)
    e, es = err_o(o, o_ref), err_S(S, S_ref)
    _say(f"err_o={e:.3e} err_S={es:.3e}")
    assert e <= TOL_DECODE and es <= 1e-5


def test_decode_workload_shape_sampled():
    """256 sequences x 16 heads, 1000 steps, state N(0, 0.05): all states run on the GPU,
    the oracle follows 64 sampled (sequence, head) pairs through every step."""
    N, H, steps, seed = 256, 16, 1000, 0
    _say("decode workload: generating inputs")
    S_np = make_decode_state(N, H, 128, seed=seed)
    X = make_decode_steps(N, H, 128, seed=seed, steps=steps)
    Xd = {k: up(v) for k, v in X.items()}
    S_dev = up(S_np)
    rng = np.random.default_rng(123)
    pairs = rng.choice(N * H, size=64, replace=False)
    n_idx, h_idx = pairs // H, pairs % H
    S_ref = S_np[n_idx, h_idx].astype(np.float64)[:, None]          # [64,1,d,d]
    o_all = torch.empty((steps, 64, 128), dtype=torch.float32, device=dev())
    o = torch.empty((N, H, 128), dtype=torch.float32, device=dev())
    idx_n = torch.as_tensor(n_idx, device=dev())
    idx_h = torch.as_tensor(h_idx, device=dev())
    _say("decode workload: running 1000 steps")
    for s in range(steps):
        kda.kda_decode_step(Xd["q"][s], Xd["k"][s], Xd["v"][s], Xd["g"][s], Xd["beta"][s], S_dev,
                            o=o)
        o_all[s] = o[idx_n, idx_h]
    torch.cuda.synchronize()
    o_gpu = down(o_all)
    o_ref = np.empty((steps, 64, 128))
    for s in range(steps):
        sl = lambda a: np.ascontiguousarray(a[s][n_idx, h_idx][:, None])  # noqa: E731
        o_ref[s] = native.decode_step(S_ref, sl(X["q"]), sl(X["k"]), sl(X["v"]), sl(X["g"]),
                                      sl(X["beta"]), bf16=True)[:, 0]
    e = err_o(o_gpu, o_ref)
    eS = err_S(down(S_dev)[n_idx, h_idx], S_ref[:, 0])
    _say(f"decode workload err_o={e:.3e} err_S={eS:.3e}")
    assert e <= TOL_DECODE
    assert eS <= 1e-5
    assert torch.isfinite(S_dev).all()


def test_decode_workload_all_states():
    """The whole decode workload (256 sequences x 16 heads, state N(0, 0.05)) for its first
    24 steps: every output of every step and every final state against the oracle."""
    N, H, steps, seed = 256, 16, 24, 0
    _say("decode workload, all states: generating inputs")
    S_np = make_decode_state(N, H, 128, seed=seed)
    X = make_decode_steps(N, H, 128, seed=seed, steps=steps)
    Xd = {k: up(v) for k, v in X.items()}
    S_dev = up(S_np)
    o_all = torch.empty((steps, N, H, 128), dtype=torch.float32, device=dev())
    for s in range(steps):
        kda.kda_decode_step(Xd["q"][s], Xd["k"][s], Xd["v"][s], Xd["g"][s], Xd["beta"][s], S_dev,
                            o=o_all[s])
    torch.cuda.synchronize()
    _say("decode workload, all states: oracle")
    S_ref = S_np.astype(np.float64)
    o_ref = np.stack([native.decode_step(S_ref, X["q"][s], X["k"][s], X["v"][s], X["g"][s],
                                         X["beta"][s], bf16=True) for s in range(steps)])
    e, eS = err_o(down(o_all), o_ref), err_S(down(S_dev), S_ref)
    _say(f"decode workload, all states: err_o={e:.3e} err_S={eS:.3e}")
    assert e <= TOL_DECODE
    assert eS <= 1e-5


def test_speculative_rollback_bit_exact():
    """60 steps, checkpoint, 4 speculative steps, rollback: the restored state equals the
    checkpoint bit for bit and the oracle state after step 60; 4 replacement steps with
    fresh draws then match the oracle."""
    N, H, seed = 2, 8, 9
    S_np = make_decode_state(N, H, 128, seed=seed)
    S_dev = up(S_np)
    S_ref = S_np.astype(np.float64)
    o = torch.empty((N, H, 128), dtype=torch.float32, device=dev())

    def step(s, S_ref, draw_seed):
        st = make_decode_step(N, H, 128, seed=draw_seed, step=s)
        kda.kda_decode_step(up(st.q), up(st.k), up(st.v), up(st.g), up(st.beta), S_dev, o=o)
        o_ref = native.decode_step(S_ref, st.q, st.k, st.v, st.g, st.beta, bf16=True)
        return o_ref

    for s in range(60):
        step(s, S_ref, seed)
    ck = torch.empty_like(S_dev)
    kda.kda_state_checkpoint(S_dev, ck)
    S_at_60 = S_ref.copy()
    spec_ref = S_ref.copy()
    for s in range(60, 64):
        step(s, spec_ref, seed)
    torch.cuda.synchronize()
    assert not torch.equal(S_dev, ck)
    kda.kda_state_rollback(S_dev, ck)
    torch.cuda.synchronize()
    assert torch.equal(S_dev, ck)
    assert err_S(down(S_dev), S_at_60) <= 1e-5
    S_ref = S_at_60
    for s in range(60, 64):
        o_ref = step(s, S_ref, seed + 1000)
        torch.cuda.synchronize()
        assert err_o(down(o), o_ref) <= TOL_DECODE
    assert err_S(down(S_dev), S_ref) <= 1e-5


def test_decode_errors_and_empty():
    q = torch.zeros((2, 2, 128), dtype=torch.bfloat16, device=dev())
    st = torch.zeros((2, 2, 128, 128), device=dev())
    g = torch.zeros((2, 2, 128), device=dev())
    b = torch.zeros((2, 2), device=dev())
    with pytest.raises(kda.KdaError) as ei:
        kda.kda_decode_step(q, q, q, g, b, st, o=q)
    assert ei.value.status == kda.KDA_ERR_ALIAS
    e = torch.zeros((0, 2, 128), dtype=torch.bfloat16, device=dev())
    kda.kda_decode_step(e, e, e, g[:0], b[:0], st[:0], o=torch.zeros((0, 2, 128), device=dev()))


def test_checkpoint_copy_odd_sizes():
    x = torch.randn(3 * 5 * 7 + 1, device=dev())[1:].view(3, 5, 7)   # misaligned, odd count
    y = torch.empty((3, 5, 7), device=dev())
    kda.kda_state_checkpoint(x, y)
    torch.cuda.synchronize()
    assert torch.equal(x, y)
