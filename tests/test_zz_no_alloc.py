"""The allocation-free prefill entry point (kda_prefill_chunked_noalloc), through the C
ABI: its workspace is the library's fixed per-device array.  Two calls in a row, the
second with a smaller input (the array keeps the first call's contents), each against
kda_prefill_chunked with a caller-allocated workspace on the same inputs, and against the
oracle; a descriptor that needs more than the array holds is refused."""
import sys

import numpy as np
import pytest
import torch

import linear_attention_sequence_kda_amd as kda
from kda_inputs import BF16, make_prefill, to_f64
from oracle import native, norm_gate
from gpu_util import up, down, err_o, err_S, dev

pytestmark = pytest.mark.gpu

TOL_O, TOL_S = 2e-2, 1e-2


def _say(*a):
    print(*a, flush=True, file=sys.stderr)


def _run(c, fn, **kw):
    o = torch.full((c.B, c.T, c.H, 128), float("nan"), device=dev())
    S = torch.full((c.B, c.H, 128, 128), float("nan"), device=dev())
    fn(up(c.q), up(c.k), up(c.v), up(c.g), up(c.beta), o=o, S0=up(c.S0), S_final=S,
       gate=up(c.gate) if c.gate is not None else None, chunk=64, **kw)
    torch.cuda.synchronize()
    return o, S


@pytest.mark.parametrize("case", [
    # (B, T, H, n_segments, gate): the first fills most of the array, the second is smaller
    [(2, 2048, 4, 4, True), (1, 333, 2, 2, False)],
    [(1, 4096, 8, 0, False), (2, 700, 3, 0, True)],
])
def test_noalloc_matches_allocating_entry_point(case):
    for i, (B, T, H, n_seg, gate) in enumerate(case):
        c = make_prefill(B, T, H, 128, seed=300 + 7 * i + T, in_dtype=BF16, s0_std=0.05, gate=gate)
        kw = dict(n_segments=n_seg)
        need = kda.kda_prefill_workspace_size(up(c.q), up(c.k), up(c.v), up(c.g), up(c.beta),
                                              o=None, gate=up(c.gate) if gate else None,
                                              chunk=64, **kw)
        assert 0 < need <= kda.NOALLOC_WORKSPACE_BYTES
        _say(f"noalloc call {i}: B={B} T={T} H={H} n_seg={n_seg} gate={gate} ws={need}")
        o1, S1 = _run(c, kda.kda_prefill_chunked_noalloc, **kw)
        o2, S2 = _run(c, kda.kda_prefill_chunked, **kw)
        # the same kernels and plan on the same inputs: identical results
        assert torch.equal(o1, o2) and torch.equal(S1, S2)
        o_ref, S_ref, _ = native.prefill(c.q, c.k, c.v, c.g, c.beta, c.S0, bf16=True)
        if gate:
            o_ref = norm_gate(o_ref, to_f64(c.gate, BF16), 1e-6)
        eo, es = err_o(down(o1), o_ref), err_S(down(S1), S_ref)
        _say(f"noalloc call {i}: err_o={eo:.3e} err_S={es:.3e}")
        assert np.isfinite(down(o1)).all() and eo <= TOL_O and es <= TOL_S


def test_noalloc_refuses_more_than_the_array():
    T = 16384
    q = torch.zeros((1, T, 8, 128), dtype=torch.bfloat16, device=dev())
    g = torch.zeros((1, T, 8, 128), device=dev())
    b = torch.zeros((1, T, 8), device=dev())
    o = torch.empty((1, T, 8, 128), device=dev())
    assert kda.kda_prefill_workspace_size(q, q, q, g, b, o=None) > kda.NOALLOC_WORKSPACE_BYTES
    with pytest.raises(kda.KdaError) as ei:
        kda.kda_prefill_chunked_noalloc(q, q, q, g, b, o=o)
    assert ei.value.status == kda.KDA_ERR_WORKSPACE
