"""Seeded synthetic inputs for the KDA hot path.

This module is shared by the tests, the benchmark and the CPU oracle's callers.
It holds only the input recipe (random draws, the value distributions of the
workloads, rounding to the storage dtypes) and none of the recurrence's
arithmetic.  Every array it returns holds exactly the bytes a device kernel
receives, so the oracle and the GPU path consume identical values.

Value distributions follow the workload descriptions of the KDA hot path:
  q, k  ~ N(0, 1), L2-normalised per token per head over the feature axis
  v     ~ N(0, 1)
  beta  = sigmoid(N(0, 1))
  g     = max(-5, logsigmoid(N(2, 1)))          (per-channel log-decay)
  gate  ~ N(0, 1)                               (output-gate logits)
Readings where the workloads are silent (stated once here and in the design
notes): N(mu, s) takes s as the standard deviation; the generator is NumPy's
PCG64 seeded per (seed, tensor, batch row, token block) so that large inputs
can be produced block by block and in parallel; float values are cast
fp64 -> fp32 (round to nearest even) -> bf16 (round to nearest even).

bf16 arrays are carried as ``numpy.uint16`` bit patterns.
"""
from __future__ import annotations

import concurrent.futures as _fut
import os
from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "F32", "BF16", "f32_to_bf16", "bf16_to_f32", "to_f64",
    "PrefillCase", "DecodeStep", "WORKLOADS", "make_prefill", "make_workload", "make_decode_state",
    "make_decode_step", "make_decode_steps", "workload", "make_output_grads",
]

F32 = "f32"
BF16 = "bf16"

# Tensor ids for the per-tensor random streams.
_Q, _K, _V, _G, _BETA, _GATE, _S0, _CHSEL, _DO, _DS = range(10)
_BLOCK = 1024  # tokens per random stream block


# ----------------------------------------------------------------------------
# storage-dtype rounding
# ----------------------------------------------------------------------------
def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even).

    Returns the bf16 bit patterns as uint16.  NaN stays NaN (quiet)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32)
    lsb = (bits >> 16) & np.uint32(1)
    rounded = (bits + np.uint32(0x7FFF) + lsb) >> 16
    nan = np.isnan(x)
    if nan.any():
        rounded = np.where(nan, (bits >> 16) | np.uint32(0x40), rounded)
    return rounded.astype(np.uint16)


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to float32 exactly."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def to_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact fp64 value of a stored array (bf16 bit patterns or float32)."""
    if dtype == BF16:
        return bf16_to_f32(x).astype(np.float64)
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def _store(x64: np.ndarray, dtype: str) -> np.ndarray:
    x32 = x64.astype(np.float32)
    return f32_to_bf16(x32) if dtype == BF16 else x32


def _logsigmoid(x: np.ndarray) -> np.ndarray:
    # log(1 / (1 + e^-x)) evaluated without overflow for either sign of x
    return -np.logaddexp(0.0, -x)


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return np.exp(_logsigmoid(x))


# ----------------------------------------------------------------------------
# workloads
# ----------------------------------------------------------------------------
@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    T: int
    H: int
    d: int
    chunk: int
    in_dtype: str
    out_dtype: str
    s0_std: float = 0.0
    gate: bool = False
    ckpt_every: int = 0
    n_segments: int = 0
    pinned_floor_frac: float = 0.0   # fraction of channels per head with g = -5
    slow_frac: float = 0.0           # fraction of channels per head with g ~ 0
    decode_steps: int = 0
    notes: str = ""


WORKLOADS = {
    # Tiny fp32 reference case (q/k/v fp32, o fp32), chunk 16.
    "tiny": Workload("tiny", B=1, T=256, H=2, d=128, chunk=16, in_dtype=F32, out_dtype=F32),
    # Chunkwise prefill with the per-head RMSNorm + sigmoid output gate.
    "prefill_8k": Workload("prefill_8k", B=4, T=8192, H=16, d=128, chunk=64, in_dtype=BF16,
                           out_dtype=BF16, s0_std=0.01, gate=True),
    # Recurrent decode: 256 sequences x 16 heads, 1000 single-token steps.
    "decode_256x16": Workload("decode_256x16", B=256, T=1, H=16, d=128, chunk=1, in_dtype=BF16,
                              out_dtype=F32, s0_std=0.05, decode_steps=1000),
    # Long single-sequence prefill with floor-pinned and slow-decay channels, 512-token checkpoints.
    "prefill_131k": Workload("prefill_131k", B=1, T=131072, H=16, d=128, chunk=64, in_dtype=BF16,
                             out_dtype=BF16, ckpt_every=512, pinned_floor_frac=0.1, slow_frac=0.1),
    # 1M-token prefill over 256 on-device segments, then 64 decode steps with a 4-step rollback.
    "prefill_1m": Workload("prefill_1m", B=1, T=1 << 20, H=8, d=128, chunk=64, in_dtype=BF16,
                           out_dtype=BF16, n_segments=256, ckpt_every=0, decode_steps=64),
}


def workload(name: str) -> Workload:
    return WORKLOADS[name]


@dataclass
class PrefillCase:
    B: int
    T: int
    H: int
    d_k: int
    d_v: int
    in_dtype: str
    q: np.ndarray           # [B,T,H,d_k] in_dtype storage
    k: np.ndarray           # [B,T,H,d_k]
    v: np.ndarray           # [B,T,H,d_v]
    g: np.ndarray           # [B,T,H,d_k] float32
    beta: np.ndarray        # [B,T,H] float32
    S0: np.ndarray | None   # [B,H,d_k,d_v] float32 or None (= zeros)
    gate: np.ndarray | None = None  # [B,T,H,d_v] in_dtype storage or None
    meta: dict = field(default_factory=dict)


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _normal(seed: int, tid: int, b: int, blk: int, shape, loc=0.0, scale=1.0) -> np.ndarray:
    rng = np.random.default_rng([seed, tid, b, blk])
    x = rng.standard_normal(shape)
    if scale != 1.0:
        x *= scale
    if loc != 0.0:
        x += loc
    return x


def _l2n(x: np.ndarray) -> np.ndarray:
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True))


def make_prefill(B: int, T: int, H: int, d_k: int = 128, d_v: int | None = None, *,
                 seed: int = 0, in_dtype: str = BF16, s0_std: float = 0.0, gate: bool = False,
                 pinned_floor_frac: float = 0.0, slow_frac: float = 0.0,
                 g_mode: str = "default", beta_mode: str = "default",
                 threads: int | None = None) -> PrefillCase:
    """Seeded prefill inputs.

    g_mode: "default" (max(-5, logsigmoid(N(2,1)))), "raw" (logsigmoid(N(2,1))*3, which
    crosses the floor often, for clamp tests), "floor" (all -5), "zero" (all 0),
    "below_floor" (all -7; must behave as -5).
    beta_mode: "default" (sigmoid(N(0,1))), "zero" (all 0), "one" (all 1).
    """
    d_v = d_k if d_v is None else d_v
    if in_dtype not in (F32, BF16):
        raise ValueError(in_dtype)
    q = np.empty((B, T, H, d_k), dtype=np.uint16 if in_dtype == BF16 else np.float32)
    k = np.empty_like(q)
    v = np.empty((B, T, H, d_v), dtype=q.dtype)
    g = np.empty((B, T, H, d_k), dtype=np.float32)
    beta = np.empty((B, T, H), dtype=np.float32)
    gt = np.empty((B, T, H, d_v), dtype=q.dtype) if gate else None

    # channel selection for pinned-floor / slow-decay channels: per head, fixed for all tokens
    n_pin = int(round(pinned_floor_frac * d_k))
    n_slow = int(round(slow_frac * d_k))
    pin_mask = np.zeros((H, d_k), dtype=bool)
    slow_mask = np.zeros((H, d_k), dtype=bool)
    if n_pin or n_slow:
        rng = np.random.default_rng([seed, _CHSEL])
        for h in range(H):
            perm = rng.permutation(d_k)
            pin_mask[h, perm[:n_pin]] = True
            slow_mask[h, perm[n_pin:n_pin + n_slow]] = True

    def work(b: int, blk: int) -> None:
        t0 = blk * _BLOCK
        t1 = min(T, t0 + _BLOCK)
        n = t1 - t0
        q[b, t0:t1] = _store(_l2n(_normal(seed, _Q, b, blk, (n, H, d_k))), in_dtype)
        k[b, t0:t1] = _store(_l2n(_normal(seed, _K, b, blk, (n, H, d_k))), in_dtype)
        v[b, t0:t1] = _store(_normal(seed, _V, b, blk, (n, H, d_v)), in_dtype)
        x = _normal(seed, _G, b, blk, (n, H, d_k), loc=2.0)
        if g_mode == "default":
            gg = np.maximum(-5.0, _logsigmoid(x))
        elif g_mode == "raw":
            gg = 3.0 * _logsigmoid(x)
        elif g_mode == "floor":
            gg = np.full_like(x, -5.0)
        elif g_mode == "zero":
            gg = np.zeros_like(x)
        elif g_mode == "below_floor":
            gg = np.full_like(x, -7.0)
        else:
            raise ValueError(g_mode)
        if n_pin:
            gg = np.where(pin_mask[None], -5.0, gg)
        if n_slow:
            xs = _normal(seed, _G + 100, b, blk, (n, H, d_k), loc=9.0)
            gg = np.where(slow_mask[None], _logsigmoid(xs), gg)
        g[b, t0:t1] = gg.astype(np.float32)
        xb = _normal(seed, _BETA, b, blk, (n, H))
        if beta_mode == "default":
            bb = _sigmoid(xb)
        elif beta_mode == "zero":
            bb = np.zeros_like(xb)
        elif beta_mode == "one":
            bb = np.ones_like(xb)
        else:
            raise ValueError(beta_mode)
        beta[b, t0:t1] = bb.astype(np.float32)
        if gate:
            gt[b, t0:t1] = _store(_normal(seed, _GATE, b, blk, (n, H, d_v)), in_dtype)

    jobs = [(b, blk) for b in range(B) for blk in range((T + _BLOCK - 1) // _BLOCK)]
    nt = threads or _threads()
    if nt > 1 and len(jobs) > 1:
        with _fut.ThreadPoolExecutor(nt) as ex:
            list(ex.map(lambda a: work(*a), jobs))
    else:
        for a in jobs:
            work(*a)

    S0 = None
    if s0_std > 0.0:
        S0 = _normal(seed, _S0, 0, 0, (B, H, d_k, d_v), scale=s0_std).astype(np.float32)
    return PrefillCase(B, T, H, d_k, d_v, in_dtype, q, k, v, g, beta, S0, gt,
                       meta=dict(seed=seed, pin_mask=pin_mask, slow_mask=slow_mask))


def make_workload(name: str, seed: int = 0, T: int | None = None, B: int | None = None,
                  H: int | None = None, in_dtype: str | None = None, **kw) -> PrefillCase:
    """Prefill inputs for a named workload (optionally with a shortened T / B / H)."""
    w = WORKLOADS[name]
    return make_prefill(B or w.B, T if T is not None else w.T, H or w.H, w.d, seed=seed,
                        in_dtype=in_dtype or w.in_dtype, s0_std=w.s0_std, gate=w.gate,
                        pinned_floor_frac=w.pinned_floor_frac, slow_frac=w.slow_frac, **kw)


@dataclass
class DecodeStep:
    N: int
    H: int
    d: int
    in_dtype: str
    q: np.ndarray      # [N,H,d]
    k: np.ndarray      # [N,H,d]
    v: np.ndarray      # [N,H,d]
    g: np.ndarray      # [N,H,d] float32
    beta: np.ndarray   # [N,H] float32


def make_decode_state(N: int, H: int, d: int = 128, *, seed: int = 0, std: float = 0.05) -> np.ndarray:
    """Initial decode state S ~ N(0, std) as float32 [N,H,d,d]."""
    out = np.empty((N, H, d, d), dtype=np.float32)
    for n0 in range(0, N, 64):
        n1 = min(N, n0 + 64)
        out[n0:n1] = _normal(seed, _S0, n0, 1, (n1 - n0, H, d, d), scale=std).astype(np.float32)
    return out


def make_decode_step(N: int, H: int, d: int = 128, *, seed: int = 0, step: int = 0,
                     in_dtype: str = BF16) -> DecodeStep:
    """One decode step's token inputs, drawn per step with the prefill distributions."""
    def nrm(tid, shape, loc=0.0):
        return np.random.default_rng([seed, step, tid]).standard_normal(shape) + loc

    q = _store(_l2n(nrm(_Q, (N, H, d))), in_dtype)
    k = _store(_l2n(nrm(_K, (N, H, d))), in_dtype)
    v = _store(nrm(_V, (N, H, d)), in_dtype)
    g = np.maximum(-5.0, _logsigmoid(nrm(_G, (N, H, d), loc=2.0))).astype(np.float32)
    beta = _sigmoid(nrm(_BETA, (N, H))).astype(np.float32)
    return DecodeStep(N, H, d, in_dtype, q, k, v, g, beta)


def make_decode_steps(N: int, H: int, d: int = 128, *, seed: int = 0, steps: int = 1,
                      first_step: int = 0, in_dtype: str = BF16, threads: int | None = None):
    """Token inputs of `steps` consecutive decode steps, stacked on a leading axis:
    returns dict q, k, v [S,N,H,d], g [S,N,H,d], beta [S,N,H].  Step s uses the same
    draws as make_decode_step(step=first_step + s)."""
    dt = np.uint16 if in_dtype == BF16 else np.float32
    out = dict(q=np.empty((steps, N, H, d), dt), k=np.empty((steps, N, H, d), dt),
               v=np.empty((steps, N, H, d), dt), g=np.empty((steps, N, H, d), np.float32),
               beta=np.empty((steps, N, H), np.float32))

    def work(s):
        st = make_decode_step(N, H, d, seed=seed, step=first_step + s, in_dtype=in_dtype)
        out["q"][s], out["k"][s], out["v"][s], out["g"][s], out["beta"][s] = \
            st.q, st.k, st.v, st.g, st.beta

    nt = threads or _threads()
    if nt > 1 and steps > 1:
        with _fut.ThreadPoolExecutor(nt) as ex:
            list(ex.map(work, range(steps)))
    else:
        for s in range(steps):
            work(s)
    return out


def make_output_grads(B: int, T: int, H: int, d: int = 128, *, seed: int = 0,
                      ds_std: float = 0.1) -> tuple[np.ndarray, np.ndarray]:
    """Upstream gradients for the backward pass: dO ~ N(0, 1) as float32 [B,T,H,d]
    (gradient of the raw outputs) and dS_T ~ N(0, ds_std) as float32 [B,H,d,d]
    (gradient of the final state)."""
    dO = np.empty((B, T, H, d), dtype=np.float32)
    for b in range(B):
        for blk in range((T + _BLOCK - 1) // _BLOCK):
            t0, t1 = blk * _BLOCK, min(T, (blk + 1) * _BLOCK)
            dO[b, t0:t1] = _normal(seed, _DO, b, blk, (t1 - t0, H, d)).astype(np.float32)
    dS = _normal(seed, _DS, 0, 0, (B, H, d, d), scale=ds_std).astype(np.float32)
    return dO, dS
