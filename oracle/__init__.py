"""CPU oracle for the KDA hot path -- TEST INFRASTRUCTURE, not product code.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import,
call, link or run anything in this package.  The GPU library never uses it and
shares no source with it.

Contents (all floating point in fp64):
  sequential.py the plain definition, one token at a time
  chunkwise.py  an independent chunkwise reformulation (full-chunk factorisation)
  segments.py   per-segment state maps, their composition, fold and exclusive scan
  exact.py      exact rational brute force for tiny cases (fractions.Fraction)
  native.py     ctypes wrapper of kda_oracle.c, the same sequential recurrence in
                plain C, threaded over independent (batch, head, column block)
                units, for workload-sized cases

Sources.  The pages this follows print no formula.  What they fix:
  * "xhh.club" tag page 结构, entry on KDA's recurrent form: the state is one
    128x128 matrix per head, independent of context length; it is updated by a
    per-channel decay followed by an erase-and-write (the DeltaNet / Gated DeltaNet
    lineage); the output gets a per-head RMSNorm and a full-rank sigmoid gate.
  * same page, entry on the chunkwise-parallel algorithm: every step's log-decay
    is floored at -5; chunks are linked by a state recurrence and computed inside
    with matmuls; training and prefill use the chunkwise form, decode the
    recurrent form.
  * same page, entry on the structure's system implications: the three execution
    forms (fast kernel, intra-device context parallelism, state rollback); context
    parallelism decomposes by an associative prefix scan, never by summing states;
    the prefix cache reuses state at 512-token boundaries.
  * "nlpx.cn" Kimi K3 reading guide, section 6 (term table, self-test questions):
    KDA is recurrent attention with channel-wise decay; KCP runs the recurrent state
    in parallel through segment transitions; why the floor sits at -5, why per-rank
    states cannot simply be added, why the prefix cache needs KDA checkpoints.

Readings taken where the pages are silent (each is listed in the design notes):
  one step is  S' = Diag(exp(gt)) S,  u = beta (v - S'^T k),  S = S' + k u^T,
  o = S^T q  with  gt = min(0, max(-5, g)); the decay acts on the key axis (rows of
  S); the output reads the state after the step's write; q is not rescaled; the
  RMSNorm is over the value axis per token per head with eps 1e-6 and weight 1,
  applied before the gate  out = y * sigmoid(gate).
"""
from .sequential import recurrent, norm_gate, decode_step, clamp_decay  # noqa: F401
from .chunkwise import chunkwise  # noqa: F401
from .segments import (segment_map, compose, fold, exclusive_scan,  # noqa: F401
                       apply_map)
