"""GPU parity over seeded random combinations of the prefill and decode options, through
the C ABI, against the fp64 CPU oracle on the same input bytes.

The hand-picked cases elsewhere cover each option on its own; here hypothesis draws
combinations of them (batch, heads, ragged length, chunk size, segment count, gate, column
split, initial state, checkpoints, input and output dtype; for decode also the state pool
and its slots).  derandomize=True makes the draws the same on every run, so a failure
names a reproducible case.  Tolerances as in test_prefill_gpu.py and test_decode_gpu.py:
bf16 inputs err_o <= 2e-2 and err_S <= 1e-2 (bf16 output storage widens err_o by its
rounding), fp32 inputs 1e-4, decode 1e-4.
"""
import sys

import numpy as np
import pytest
import torch
from hypothesis import HealthCheck, given, settings, strategies as st

import linear_attention_sequence_kda_amd as kda
from kda_inputs import BF16, F32, f32_to_bf16, make_decode_state, make_decode_step, make_prefill, to_f64
from oracle import native, norm_gate
from gpu_util import up, down, err_o, err_S, bf16_out_tol, dev

pytestmark = pytest.mark.gpu

SETTINGS = dict(derandomize=True, database=None, deadline=None,
                suppress_health_check=[HealthCheck.too_slow, HealthCheck.data_too_large])


def _say(*a):
    print(*a, flush=True, file=sys.stderr)


@settings(max_examples=40, **SETTINGS)
@given(B=st.integers(1, 3), H=st.integers(1, 5), T=st.integers(1, 700),
       f32_in=st.booleans(), chunk64=st.booleans(), n_seg=st.integers(0, 6),
       gate=st.booleans(), v_split=st.sampled_from([0, 1, 2]), s0=st.booleans(),
       ckpt_every=st.sampled_from([0, 64, 128]), out_bf16=st.booleans())
def test_random_prefill_configs(B, H, T, f32_in, chunk64, n_seg, gate, v_split, s0, ckpt_every,
                                out_bf16):
    in_dtype = F32 if f32_in else BF16
    chunk = 64 if (chunk64 and not f32_in) else 16      # fp32 inputs run with 16-token chunks
    n_chunks = -(-T // chunk)
    n_seg = min(n_seg, n_chunks)
    if ckpt_every > T:
        ckpt_every = 0
    label = (f"B={B} H={H} T={T} {in_dtype} chunk={chunk} n_seg={n_seg} gate={gate} "
             f"v_split={v_split} S0={s0} ckpt={ckpt_every} out={'bf16' if out_bf16 else 'f32'}")
    _say(label)
    seed = (((B * 7 + H) * 1009 + T) * 3 + chunk) % 100003
    c = make_prefill(B, T, H, 128, seed=seed, in_dtype=in_dtype, s0_std=0.05 if s0 else 0.0,
                     gate=gate)
    out_dtype = torch.bfloat16 if out_bf16 else torch.float32
    o = torch.full((B, T, H, 128), float("nan"), dtype=out_dtype, device=dev())
    Sf = torch.full((B, H, 128, 128), float("nan"), device=dev())
    ck = torch.full((B, T // ckpt_every, H, 128, 128), float("nan"), device=dev()) if ckpt_every else None
    kda.kda_prefill_chunked(up(c.q), up(c.k), up(c.v), up(c.g), up(c.beta), o=o,
                            S0=up(c.S0) if s0 else None, S_final=Sf,
                            gate=up(c.gate) if gate else None, chunk=chunk, ckpt_every=ckpt_every,
                            ckpt=ck, n_segments=n_seg, v_split=v_split)
    torch.cuda.synchronize()
    o_ref, S_ref, ck_ref = native.prefill(c.q, c.k, c.v, c.g, c.beta, c.S0 if s0 else None,
                                          bf16=(in_dtype == BF16), ckpt_every=ckpt_every)
    if gate:
        o_ref = norm_gate(o_ref, to_f64(c.gate, in_dtype), 1e-6, None)
    tol_o, tol_s = (1e-4, 1e-4) if f32_in else (2e-2, 1e-2)
    if out_bf16:
        tol_o = bf16_out_tol(o_ref, tol_o)
    og = down(o)
    assert np.isfinite(og).all(), label
    eo, es = err_o(og, o_ref), err_S(down(Sf), S_ref)
    _say(f"  err_o={eo:.3e} err_S={es:.3e}")
    assert eo <= tol_o, (label, eo)
    assert es <= tol_s, (label, es)
    if ck is not None:
        for m in range(ck_ref.shape[1]):
            assert err_S(down(ck[:, m]), ck_ref[:, m]) <= tol_s, (label, "checkpoint", m)


@settings(max_examples=25, **SETTINGS)
@given(N=st.integers(1, 40), H=st.integers(1, 6), steps=st.integers(1, 5), f32_in=st.booleans(),
       gate=st.booleans(), out_bf16=st.booleans(), pool_extra=st.integers(0, 24),
       pooled=st.booleans(), seed=st.integers(0, 999))
def test_random_decode_configs(N, H, steps, f32_in, gate, out_bf16, pool_extra, pooled, seed):
    in_dtype = F32 if f32_in else BF16
    P = N + pool_extra if pooled else N
    label = (f"N={N} H={H} steps={steps} {in_dtype} gate={gate} out={'bf16' if out_bf16 else 'f32'} "
             f"pool={P if pooled else '-'}")
    _say(label)
    rng = np.random.default_rng([seed, 5])
    slots = rng.permutation(P)[:N].astype(np.int32) if pooled else None
    pool_np = make_decode_state(P, H, 128, seed=seed)
    pool = up(pool_np)
    ref = pool_np.astype(np.float64)
    slots_dev = torch.from_numpy(slots).to(dev()) if pooled else None
    out_dtype = torch.bfloat16 if out_bf16 else torch.float32
    tol = 1e-4
    for s in range(steps):
        stp = make_decode_step(N, H, 128, seed=seed, step=s, in_dtype=in_dtype)
        gt = None
        if gate:
            g32 = rng.standard_normal((N, H, 128)).astype(np.float32)
            gt = g32 if in_dtype == F32 else f32_to_bf16(g32)
        o = torch.full((N, H, 128), float("nan"), dtype=out_dtype, device=dev())
        args = (up(stp.q), up(stp.k), up(stp.v), up(stp.g), up(stp.beta))
        if pooled:
            kda.kda_decode_step_pooled(*args, pool, slots_dev, o=o, gate=up(gt) if gate else None)
        else:
            kda.kda_decode_step(*args, pool, o=o, gate=up(gt) if gate else None)
        sel = slots if pooled else np.arange(N)
        S_step = ref[sel]
        o_ref = native.decode_step(S_step, stp.q, stp.k, stp.v, stp.g, stp.beta,
                                   bf16=(in_dtype == BF16))
        ref[sel] = S_step
        if gate:
            o_ref = norm_gate(o_ref, to_f64(gt, in_dtype), 1e-6, None)
        t = bf16_out_tol(o_ref, tol) if out_bf16 else tol
        e = err_o(down(o), o_ref)
        assert e <= t, (label, "step", s, e)
    torch.cuda.synchronize()
    # every slot of the pool: stepped ones against the oracle, the others untouched
    assert err_S(down(pool), ref) <= 1e-5, label
    if pooled:
        untouched = np.setdiff1d(np.arange(P), slots)
        assert np.array_equal(down(pool)[untouched], pool_np[untouched]), label
