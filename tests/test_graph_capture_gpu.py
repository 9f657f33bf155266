"""The entry points can be captured into a HIP graph: a call allocates nothing, does not
synchronise with the host and records no memset node.  Captured here with torch.cuda.graph:
one prefill call (segment maps, scan, fused norm/gate, ragged tail), a run of decode steps
with a state checkpoint and a rollback, and one backward call.  Each graph is replayed
three times, with eager work and synchronisation between the replays (the outputs are
overwritten with NaN, the state is reset), and every replay must equal the eager result
bit for bit: the same kernels run on the same inputs.
"""
import sys

import pytest
import torch

import linear_attention_sequence_kda_amd as kda
from kda_inputs import make_decode_state, make_decode_steps, make_output_grads, make_prefill
from gpu_util import dev, up

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True, file=sys.stderr)


def _replay_and_compare(graph, reset, outs, expected, label):
    for r in range(3):
        for t in outs:                     # eager work between replays
            t.fill_(float("nan"))
        reset()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (got, want) in enumerate(zip(outs, expected)):
            assert torch.equal(got, want), (label, "replay", r, "output", i)
    _say(f"{label}: 3 replays equal the eager result")


def test_prefill_call_in_a_graph():
    c = make_prefill(1, 1000, 4, seed=41, s0_std=0.1, gate=True)
    q, k, v, g, beta, gate, S0 = (up(x) for x in (c.q, c.k, c.v, c.g, c.beta, c.gate, c.S0))
    kw = dict(S0=S0, gate=gate, chunk=64, n_segments=4)
    o = torch.empty((1, 1000, 4, 128), device=dev())
    Sf = torch.empty((1, 4, 128, 128), device=dev())
    ws = torch.empty(kda.kda_prefill_workspace_size(q, k, v, g, beta, o=o, S_final=Sf, **kw),
                     dtype=torch.uint8, device=dev())
    kda.kda_prefill_chunked(q, k, v, g, beta, o=o, S_final=Sf, workspace=ws, **kw)
    torch.cuda.synchronize()
    o_e, Sf_e = o.clone(), Sf.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        kda.kda_prefill_chunked(q, k, v, g, beta, o=o, S_final=Sf, workspace=ws, **kw)
    _replay_and_compare(graph, lambda: None, [o, Sf], [o_e, Sf_e], "prefill")


def test_decode_steps_with_checkpoint_and_rollback_in_a_graph():
    N, H, K = 8, 4, 4
    S_init = up(make_decode_state(N, H, 128, seed=42))
    st = make_decode_steps(N, H, 128, seed=42, steps=K)
    q, k, v, g, beta = (up(st[n]) for n in ("q", "k", "v", "g", "beta"))
    S = S_init.clone()
    ck = torch.empty_like(S)
    o = torch.empty((K + 2, N, H, 128), device=dev())

    def run():
        kda.kda_state_checkpoint(S, ck)
        for s in range(K):                 # K steps, then back to the checkpoint
            kda.kda_decode_step(q[s], k[s], v[s], g[s], beta[s], S, o=o[s])
        kda.kda_state_rollback(S, ck)
        for s in range(2):                 # two steps again from the restored state
            kda.kda_decode_step(q[s], k[s], v[s], g[s], beta[s], S, o=o[K + s])

    run()
    torch.cuda.synchronize()
    o_e, S_e = o.clone(), S.clone()
    assert torch.equal(o_e[K:], o_e[:2])   # the rollback restored the state exactly
    S.copy_(S_init)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    _replay_and_compare(graph, lambda: S.copy_(S_init), [o, S], [o_e, S_e], "decode")


def test_backward_call_in_a_graph():
    B, T, H = 1, 200, 2
    c = make_prefill(B, T, H, seed=43, s0_std=0.1)
    dO_np, dS_np = make_output_grads(B, T, H, seed=43)
    q, k, v, g, beta, S0 = (up(x) for x in (c.q, c.k, c.v, c.g, c.beta, c.S0))
    dO, dSf = up(dO_np), up(dS_np)
    grads = dict(dq=torch.empty((B, T, H, 128), device=dev()),
                 dk=torch.empty((B, T, H, 128), device=dev()),
                 dv=torch.empty((B, T, H, 128), device=dev()),
                 dg=torch.empty((B, T, H, 128), device=dev()),
                 dbeta=torch.empty((B, T, H), device=dev()),
                 dS0=torch.empty((B, H, 128, 128), device=dev()))
    ws = torch.empty(kda.kda_backward_workspace_size(q, k, v, g, beta, dO), dtype=torch.uint8,
                     device=dev())

    def run():
        kda.kda_prefill_backward(q, k, v, g, beta, dO, S0=S0, dS_final=dSf, workspace=ws, **grads)

    run()
    torch.cuda.synchronize()
    outs = list(grads.values())
    expected = [t.clone() for t in outs]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    _replay_and_compare(graph, lambda: None, outs, expected, "backward")
