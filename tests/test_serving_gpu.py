"""GPU tests of the serving entry points, through the C ABI: decode over a pool of
state slots with a changing batch, indexed state copies (prefix-cache reuse from
512-token checkpoints, write-back to pinned host memory), against the fp64 CPU oracle
on the same seeded input bytes and, where the same kernel arithmetic runs, bit for bit
against the plain entry points.

Tolerance (fp32 decode): err_o <= 1e-4, err_S <= 1e-5; prefill as in the prefill
tests (err_o <= 2e-2, err_S <= 1e-2 for bf16 inputs).
"""
import sys

import numpy as np
import pytest
import torch

import linear_attention_sequence_kda_amd as kda
from kda_inputs import BF16, make_decode_state, make_decode_step, make_prefill
from oracle import native
from gpu_util import up, down, err_o, err_S, dev

pytestmark = pytest.mark.gpu

TOL_DECODE = 1e-4


def _say(*a):
    print(*a, flush=True, file=sys.stderr)


def _slots(x):
    return torch.tensor(np.asarray(x, dtype=np.int32), device=dev())


def test_pooled_decode_changing_batch_matches_oracle():
    """Three steps over a 40-slot pool, each with a different batch: every active slot
    follows the oracle; slots outside the batch keep their bytes."""
    P, H = 40, 4
    pool_np = make_decode_state(P, H, 128, seed=11)
    pool = up(pool_np)
    ref = pool_np.astype(np.float64)
    rng = np.random.default_rng(11)
    for step, N in enumerate((24, 7, 31)):
        slots = rng.permutation(P)[:N]
        st = make_decode_step(N, H, 128, seed=11, step=step)
        before = pool.clone()
        o = torch.full((N, H, 128), float("nan"), device=dev())
        kda.kda_decode_step_pooled(up(st.q), up(st.k), up(st.v), up(st.g), up(st.beta), pool,
                                   _slots(slots), o=o)
        S_act = np.ascontiguousarray(ref[slots])
        o_ref = native.decode_step(S_act, st.q, st.k, st.v, st.g, st.beta, bf16=True)
        ref[slots] = S_act
        torch.cuda.synchronize()
        e = err_o(down(o), o_ref)
        _say(f"pooled decode step {step} N={N}: err_o={e:.3e}")
        assert e <= TOL_DECODE
        idle = np.setdiff1d(np.arange(P), slots)
        assert torch.equal(pool[idle], before[idle]), "a slot outside the batch changed"
    assert err_S(down(pool), ref) <= 1e-5


def test_pooled_decode_equals_plain_decode_bitwise():
    """The pooled step runs the plain step's arithmetic on the gathered states."""
    P, H, N = 16, 3, 6
    pool = up(make_decode_state(P, H, 128, seed=12))
    slots = np.array([9, 2, 15, 0, 7, 4])
    st = make_decode_step(N, H, 128, seed=12, step=0)
    gathered = pool[slots].clone()
    o_pool = torch.empty((N, H, 128), device=dev())
    o_plain = torch.empty_like(o_pool)
    args = (up(st.q), up(st.k), up(st.v), up(st.g), up(st.beta))
    kda.kda_decode_step(*args, gathered, o=o_plain)
    kda.kda_decode_step_pooled(*args, pool, _slots(slots), o=o_pool)
    torch.cuda.synchronize()
    assert torch.equal(o_pool, o_plain)
    assert torch.equal(pool[slots], gathered)


def test_pooled_decode_slot_outside_pool():
    """A slot outside the pool gives NaN outputs for that sequence and touches nothing."""
    P, H, N = 8, 2, 3
    pool = up(make_decode_state(P, H, 128, seed=13))
    before = pool.clone()
    st = make_decode_step(N, H, 128, seed=13, step=0)
    o = torch.zeros((N, H, 128), device=dev())
    kda.kda_decode_step_pooled(up(st.q), up(st.k), up(st.v), up(st.g), up(st.beta), pool,
                               _slots([3, 8, -1]), o=o)
    torch.cuda.synchronize()
    assert torch.isnan(o[1:]).all()
    assert torch.isfinite(o[0]).all()
    assert torch.equal(pool[torch.arange(P, device=dev()) != 3], before[torch.arange(P, device=dev()) != 3])
    assert not torch.equal(pool[3], before[3])


def test_indexed_copy_gather_scatter_and_host_write_back():
    H = 4
    src = torch.randn((10, H, 128, 128), device=dev())
    dst = torch.full((6, H, 128, 128), -1.0, device=dev())
    # gather src[7], src[0], src[3] into dst[5], dst[1], dst[2]; a pair outside src is skipped
    kda.kda_state_copy_indexed(dst, src, dst_slots=_slots([5, 1, 2, 4]),
                               src_slots=_slots([7, 0, 3, 10]))
    torch.cuda.synchronize()
    assert torch.equal(dst[5], src[7]) and torch.equal(dst[1], src[0]) and torch.equal(dst[2], src[3])
    assert (dst[[0, 3, 4]] == -1.0).all()
    # write-back of three pool slots to pinned host memory, then restore into new slots
    host = torch.empty((3, H, 128, 128), pin_memory=True)
    kda.kda_state_copy_indexed(host, src, src_slots=_slots([9, 4, 1]))
    torch.cuda.synchronize()
    assert torch.equal(host, src[[9, 4, 1]].cpu())
    back = torch.zeros((5, H, 128, 128), device=dev())
    kda.kda_state_copy_indexed(back, host, dst_slots=_slots([0, 2, 4]))
    torch.cuda.synchronize()
    assert torch.equal(back[[0, 2, 4]], src[[9, 4, 1]])
    assert (back[[1, 3]] == 0).all()


def test_prefix_cache_reuse_from_checkpoint():
    """Serving reuse of a cached prefix: a prefill with 512-token checkpoints, then a new
    request that shares the first 512 tokens of sequence 1 starts from that checkpoint
    (gathered by slot) and prefills only its own suffix.  Its outputs and final state
    follow the oracle of the whole sequence (shared prefix + new suffix)."""
    B, T, H = 2, 1024, 4
    c = make_prefill(B, T, H, 128, seed=14, in_dtype=BF16, s0_std=0.05)
    ck = torch.full((B, T // 512, H, 128, 128), float("nan"), device=dev())
    o = torch.empty((B, T, H, 128), device=dev())
    kda.kda_prefill_chunked(up(c.q), up(c.k), up(c.v), up(c.g), up(c.beta), o=o, S0=up(c.S0),
                            ckpt_every=512, ckpt=ck)
    # the new request: prefix = sequence 1's first 512 tokens, suffix = 320 new tokens
    n = make_prefill(1, 320, H, 128, seed=15, in_dtype=BF16)
    S0 = torch.empty((1, H, 128, 128), device=dev())
    # checkpoint (b=1, m=0) is state 1 * (T / 512) + 0 of the checkpoint array
    kda.kda_state_copy_indexed(S0, ck.view(B * (T // 512), H, 128, 128), src_slots=_slots([2]))
    o2 = torch.empty((1, 320, H, 128), device=dev())
    S2 = torch.empty((1, H, 128, 128), device=dev())
    kda.kda_prefill_chunked(up(n.q), up(n.k), up(n.v), up(n.g), up(n.beta), o=o2, S0=S0, S_final=S2)
    torch.cuda.synchronize()
    cat = lambda a, b: np.concatenate([a[1:2, :512], b], axis=1)  # noqa: E731
    o_ref, S_ref, _ = native.prefill(cat(c.q, n.q), cat(c.k, n.k), cat(c.v, n.v), cat(c.g, n.g),
                                     cat(c.beta, n.beta), c.S0[1:2], bf16=True)
    eo = err_o(down(o2), o_ref[:, 512:])
    es = err_S(down(S2), S_ref)
    _say(f"prefix reuse: err_o={eo:.3e} err_S={es:.3e}")
    assert eo <= 2e-2 and es <= 1e-2


@pytest.mark.parametrize("pooled", [False, True], ids=["plain", "pooled"])
def test_prepared_decode_step_equals_one_shot_calls(pooled):
    """A DecodeStep bound to fixed buffers, refilled with new inputs every step, gives
    bit for bit what the one-shot call gives on the same inputs (plain and pooled)."""
    P, N, H, K = 12, 5, 3, 6
    S_init = up(make_decode_state(P if pooled else N, H, 128, seed=31))
    slots = torch.tensor([7, 0, 11, 3, 5], dtype=torch.int32, device=dev()) if pooled else None
    bufs = {n: None for n in ("q", "k", "v", "g", "beta")}
    first = make_decode_step(N, H, 128, seed=31, step=0)
    for n in bufs:
        bufs[n] = up(getattr(first, n)).clone()
    S_a, S_b = S_init.clone(), S_init.clone()
    o_a = torch.empty((N, H, 128), device=dev())
    o_b = torch.empty((N, H, 128), device=dev())
    step = kda.DecodeStep(*(bufs[n] for n in ("q", "k", "v", "g", "beta")), S_a, o=o_a, slots=slots)
    for s in range(K):
        st = make_decode_step(N, H, 128, seed=31, step=s)
        for n in bufs:                                     # refill the bound buffers
            bufs[n].copy_(up(getattr(st, n)))
        step()
        args = [up(getattr(st, n)) for n in ("q", "k", "v", "g", "beta")]
        if pooled:
            kda.kda_decode_step_pooled(*args, S_b, slots, o=o_b)
        else:
            kda.kda_decode_step(*args, S_b, o=o_b)
        torch.cuda.synchronize()
        assert torch.equal(o_a, o_b), ("step", s)
    assert torch.equal(S_a, S_b)
