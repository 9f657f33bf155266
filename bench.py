"""Benchmark of the KDA hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-backward]
                    [--no-long] [--no-decode]

Headline (`value`): chunkwise prefill tokens/s on the prefill workload B=4, H=16,
T=8192, d=128, chunk 64, bf16 q/k/v/gate, fp32 g/beta/state, S0 ~ N(0, 0.01), with the
fused per-head RMSNorm and sigmoid gate, fp32 output.  One step = one prefill call over
the whole batch with inputs resident in HBM.  The same run also times:
  - decode, 256 sequences x 16 heads (fp32 states, one kernel per step), stepped over
    four such state sets in turn so that every step's 256 MiB of state comes from DRAM,
    not from the 256 MB last-level cache; and the same step on one state set (in cache);
  - decode over a pool of state slots, with write-back of states to pinned host memory;
  - the 131k-token prefill (B=1, H=16, 512-token checkpoints);
  - the 1M-token prefill over 256 segments (B=1, H=8), its 64-step decode tail and the
    rollback of 8 states;
  - the backward pass of the 8k prefill (gradients of the raw outputs, fp32 MFMA).

Prints one JSON line.  Every leg carries a `roofline` object: algorithmic bytes (each
input read once, each output written once, in the byte convention of the workload
table: bf16 activations and outputs, fp32 g, beta and states) over the event-timed
duration on the launch stream, against 8 TB/s; the backward against the fp32 matrix
peak.  `cpu_baseline` is the fp64 C oracle on the host cores over the 8k prefill,
`decode_cpu_baseline` the same oracle stepping the 256 x 16 decode workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense BF16/FP16 MFMA, TFLOP/s
FP32_PEAK_TFLOPS = 157.3       # MI355X dense FP32 MFMA, TFLOP/s
D = 128


def prefill_alg_bytes(B, T, H, out_bytes=4, gate=True, ckpt_every=0, s0=True, s_final=True):
    """Bytes the prefill must move: every input read once, every output written once.
    Per token-head: q, k, v bf16 (768 B), g fp32 (512), beta (4), the gate bf16 (256) and
    o (out_bytes per element); checkpoints add one fp32 state per ckpt_every tokens per
    head (128 B per token-head at 512); S0 and S_final one state per (sequence, head)."""
    per_tok_head = 3 * D * 2 + D * 4 + 4 + (D * 2 if gate else 0) + D * out_bytes
    total = B * T * H * per_tok_head
    if ckpt_every:
        total += B * (T // ckpt_every) * H * D * D * 4
    total += (int(s0) + int(s_final)) * B * H * D * D * 4
    return total


def table_prefill_bytes(B, T, H, **kw):
    """The workload table's convention: outputs counted as bf16 (2 B per element)."""
    return prefill_alg_bytes(B, T, H, out_bytes=2, **kw)


def prefill_alg_flops(B, T, H, chunk=64):
    """Chunkwise flops per token-head: 6 d^2 (state products) + C (3 d_k + 2 d_v)
    (intra-chunk products, triangles counted once)."""
    return B * T * H * (6 * D * D + chunk * (3 * D + 2 * D))


def backward_alg_flops(B, T, H, chunk=64):
    """Multiply-adds the chunkwise backward needs per 64-token chunk and head, x2, counting a
    triangular factor at half: chunk quantities KK, P, W, U~ (4 C^2/2 d); state sweep W S and
    K_dec^T U (2 C d^2); gradient sweep P^T dO (C^2/2 d), K_dec dS, Q~^T dO, W^T dU (3 C d^2);
    per-chunk dP (C^2/2 d), dO S^T, dU S^T, U dS^T (3 C d^2), dT (2 C^2/2 d), T^T dU, T^T dW
    (2 C^2/2 d), dM M^T and M^T Y (2 C^3/2), and the four pairwise products (4 C^2/2 d)."""
    C, d = chunk, D
    n = B * H * ((T + C - 1) // C)
    macs = (4 * C * C // 2 * d + 2 * C * d * d + C * C // 2 * d + 3 * C * d * d + C * C // 2 * d
            + 3 * C * d * d + 2 * C * C // 2 * d + 2 * C * C // 2 * d + 2 * C ** 3 // 2
            + 4 * C * C // 2 * d)
    return 2 * macs * n


def decode_alg_bytes(N, H):
    """Per step: state read + write, q/k/v bf16, g fp32, beta, o fp32."""
    return N * H * (2 * D * D * 4 + 3 * D * 2 + D * 4 + 4 + D * 4)


def _src_hash(*names):
    """Hash of the kernel sources with comments and blank space removed, so that the
    committed counter summary stays valid across comment edits but not code edits."""
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "linear_attention_sequence_kda_amd", "csrc", n), encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def _traffic_from_profiles(kernel_hash):
    """HBM bytes per prefill launch from the committed counter summary, if it was taken
    on the current kernel source; else None."""
    p = os.path.join(ROOT, "profiles", "prefill_8k_traffic.json")
    try:
        with open(p) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_src_hash") != kernel_hash:
        return None
    v = t.get("hbm_bytes_per_launch")
    return None if v is None else int(v)


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _cores():
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def _err_o(x, ref):
    return float(np.max(np.abs(x - ref)) / np.sqrt(np.mean(ref * ref)))


def _err_S(x, ref):
    return float(np.linalg.norm(x - ref) / np.linalg.norm(ref))


def cpu_baseline(c, gate, o_gpu=None, S_gpu=None):
    """Time the fp64 C oracle (plus the numpy norm/gate) on the host cores; the first
    pass's outputs also check the GPU outputs of the same run (returned as parity)."""
    from oracle import native, norm_gate
    from kda_inputs import to_f64
    threads = max(1, min(_cores(), 64))
    # whole passes over the workload until about 10 s of wall time (at most 20 passes)
    passes, dt, parity = 0, 0.0, None
    while passes < 20 and (passes == 0 or dt < 10.0):
        t0 = time.perf_counter()
        o, S, _ = native.prefill(c.q, c.k, c.v, c.g, c.beta, c.S0, bf16=True, nthreads=threads)
        o = norm_gate(o, to_f64(c.gate, "bf16"), 1e-6) if gate else o
        dt += time.perf_counter() - t0
        if passes == 0 and o_gpu is not None:
            parity = dict(err_o=_err_o(o_gpu, o), err_S=_err_S(S_gpu, S),
                          bound="err_o <= 2e-2, err_S <= 1e-2", compared="every output and final state")
        passes += 1
    return dict(value=passes * c.B * c.T / dt, unit="tokens/s", cores=threads, cpu_model=_cpu_model(), kind="oracle",
                sample=f"{passes} passes over the whole prefill workload (B={c.B}, T={c.T}, "
                       f"H={c.H}), fp64 C recurrence + numpy norm/gate, {dt:.1f} s"), parity


def prefix_cpu_baseline(pre, T_full, H, ckpt_every, what, o_gpu=None, ck_gpu=None):
    """Time the fp64 C oracle on a contiguous prefix of a long workload (all heads), for
    about 5 s, and report its tokens/s: the sequential recurrence costs the same per token,
    so the rate of the prefix is the rate of the whole (extrapolated, not run whole).  The
    GPU's outputs (and checkpoints) of those tokens do not depend on later tokens, so the
    first pass also checks them (returned as parity)."""
    from oracle import native
    threads = max(1, min(_cores(), 64))
    T = pre["q"].shape[1]
    passes, dt, parity = 0, 0.0, None
    while passes < 100 and (passes == 0 or dt < 5.0):
        t0 = time.perf_counter()
        o, _, ck = native.prefill(pre["q"], pre["k"], pre["v"], pre["g"], pre["beta"], None, bf16=True,
                                  ckpt_every=ckpt_every, nthreads=threads)
        dt += time.perf_counter() - t0
        if passes == 0 and o_gpu is not None:
            parity = dict(err_o=_err_o(o_gpu, o), bound="err_o <= 2e-2, err_S <= 1e-2",
                          compared=f"every output of the first {T} tokens, all heads")
            if ck_gpu is not None:
                parity["err_S_checkpoints"] = max(_err_S(ck_gpu[:, m], ck[:, m]) for m in range(ck.shape[1]))
                parity["compared"] += f", and their {ck.shape[1]} checkpoints"
        passes += 1
    rate = passes * T / dt
    return dict(value=round(rate, 1), unit="tokens/s", cores=threads, cpu_model=_cpu_model(),
                kind="oracle", extrapolated=True,
                sample=f"{passes} passes over the first {T} of {T_full} tokens ({what}, all {H} "
                       f"heads), fp64 C recurrence, {dt:.1f} s; whole-workload time at this rate "
                       f"{T_full / rate:.1f} s"), parity


def decode_cpu_baseline(S_np, X):
    """Time the fp64 C oracle stepping the decode workload (all states, the same step
    inputs the GPU leg uses) on the host cores, for about 10 s."""
    from oracle import native
    threads = max(1, min(_cores(), 64))
    N, H = S_np.shape[:2]
    S = S_np.astype(np.float64)
    nx = X["q"].shape[0]
    steps, dt = 0, 0.0
    while steps < 3000 and (steps < 2 or dt < 10.0):
        j = steps % nx
        t0 = time.perf_counter()
        native.decode_step(S, X["q"][j], X["k"][j], X["v"][j], X["g"][j], X["beta"][j], bf16=True,
                           nthreads=threads)
        dt += time.perf_counter() - t0
        steps += 1
    return dict(value=N * steps / dt, unit="seq-steps/s", cores=threads, cpu_model=_cpu_model(), kind="oracle",
                sample=f"{steps} steps of all {N} sequences x {H} heads (fp64 C recurrence), "
                       f"{dt:.1f} s")


def _roofline(bytes_, ms, **extra):
    gbs = bytes_ / (ms * 1e-3) / 1e9
    return dict(bound="hbm", achieved=round(gbs, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                frac=round(gbs / HBM_PEAK_GBS, 4), alg_bytes_per_launch=int(bytes_),
                kernel_ms_mean=round(ms, 4), **extra)


def _say(*x):
    print(*x, file=sys.stderr, flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-long", action="store_true", help="skip the 131k and 1M prefill legs")
    ap.add_argument("--v-split", type=int, default=0)
    ap.add_argument("--n-segments", type=int, default=0)
    a = ap.parse_args()
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the KDA hot path here has no multi-GPU mode "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import linear_attention_sequence_kda_amd as kda
    from kda_inputs import make_workload, make_decode_state, make_decode_steps

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()

    def up(x):
        x = np.ascontiguousarray(x)
        t = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16) if x.dtype == np.uint16 \
            else torch.from_numpy(x)
        return t.to(dev)

    def timed(fn, n, warmup):
        """Mean duration in ms of n calls of fn() back to back, between two events on the
        launch stream, after `warmup` calls."""
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    # ---------------- prefill workload ----------------
    B, T, H = 4, 8192, 16
    _say("bench: 8k prefill")
    c = make_workload("prefill_8k", seed=0)
    q, k, v, g, beta, gate, S0 = (up(x) for x in (c.q, c.k, c.v, c.g, c.beta, c.gate, c.S0))
    o = torch.empty((B, T, H, D), dtype=torch.float32, device=dev)
    Sf = torch.empty((B, H, D, D), dtype=torch.float32, device=dev)
    kw = dict(o=o, S0=S0, S_final=Sf, gate=gate, norm_eps=1e-6, chunk=64,
              v_split=a.v_split, n_segments=a.n_segments)
    ws_bytes = kda.kda_prefill_workspace_size(q, k, v, g, beta, **kw)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)

    def step():
        kda.kda_prefill_chunked(q, k, v, g, beta, workspace=ws, stream=stream, **kw)

    # warm-up calls (the first tens of calls on a fresh GPU run slower while its clocks
    # ramp up), then K calls back to back between two events on the launch stream,
    # bracketed by synchronisations for the wall clock
    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    e_start, e_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_start = time.perf_counter()
    e_start.record(stream)
    for _ in range(a.steps):
        step()
    e_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    ms_mean = e_start.elapsed_time(e_end) / a.steps           # average call duration
    ms_step = wall * 1e3 / a.steps
    # the outputs of the timed calls, for the parity check against the oracle's pass
    o_host = o.double().cpu().numpy() if not a.no_cpu_baseline else None
    S_host = Sf.double().cpu().numpy() if not a.no_cpu_baseline else None
    tokens = B * T
    value = tokens / (ms_step * 1e-3)
    alg_b = table_prefill_bytes(B, T, H, gate=True)
    alg_f = prefill_alg_flops(B, T, H)
    kernel_ms = ms_mean
    khash = _src_hash("tiles.h", "prefill_prep.hip", "prefill_state.hip")
    traffic = _traffic_from_profiles(khash)

    out = {
        "metric": "KDA prefill tokens/s (%MFMA peak) + decode seq-steps/s (%HBM peak), d=128",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16-in/fp16-mfma/fp32-acc",
        "arithmetic": "bf16 q/k/v/gate; BF16 MFMA on the 16-token diagonal tiles (hi/lo split "
                      "for P), FP16 MFMA for every other product, fp32 accumulation, fp32 state "
                      "and outputs",
        "data": "synthetic",
        "config": {
            "workload": "prefill B=4 H=16 T=8192 d=128 chunk=64; bf16 q/k/v/gate, fp32 g/beta/"
                        "state; S0~N(0,0.01); fused per-head RMSNorm + sigmoid gate; fp32 out",
            "global_batch": B, "seq_len": T, "heads": H, "head_dim": D, "chunk": 64,
            "parallelism": "single GPU",
        },
        "roofline": _roofline(
            alg_b, kernel_ms, traffic=traffic,
            kernel="one prefill call per step: chunk_prep_kernel, chunk_state_kernel (state "
                   "maps), segment_scan, chunk_state_kernel (outputs); their durations sum to "
                   "the call",
            bytes_convention="1796 B per token-head (q/k/v/gate bf16, g fp32, beta, o counted "
                             "as bf16) + S0 and S_final",
            frac_fp32_out=round(prefill_alg_bytes(B, T, H) / (kernel_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)),
        "prefill_mfma": {
            "alg_flops_per_launch": alg_f,
            "achieved_tflops": round(alg_f / (kernel_ms * 1e-3) / 1e12, 2),
            "peak_tflops": BF16_PEAK_TFLOPS,
            "frac": round(alg_f / (kernel_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
            # attainable = min(MFMA peak, arithmetic intensity x HBM peak): HBM-bound here,
            # so the fraction of it equals the HBM roofline fraction
            "attainable_tflops": round(min(BF16_PEAK_TFLOPS, alg_f / alg_b * HBM_PEAK_GBS * 1e9 / 1e12), 1),
            "frac_of_attainable": round(alg_f / (kernel_ms * 1e-3) / 1e12
                                        / min(BF16_PEAK_TFLOPS, alg_f / alg_b * HBM_PEAK_GBS * 1e9 / 1e12), 4),
        },
        "workspace_bytes": int(ws_bytes),
    }

    # ---------------- measured HBM ceiling ----------------
    # A copy of 1 GiB into another 1 GiB buffer (four times the last-level cache, so from
    # DRAM) with the library's own copy kernel: what a plain streaming kernel reaches on
    # this box, next to the 8 TB/s of the specification.
    _say("bench: HBM copy probe")
    n_pr = 16384                                             # 64 KiB states: 1 GiB
    pa = torch.ones((n_pr, D, D), dtype=torch.float32, device=dev)
    pb = torch.empty_like(pa)
    flip = [0]

    def probe_copy():
        flip[0] ^= 1
        src, dst = (pa, pb) if flip[0] else (pb, pa)
        kda.kda_state_checkpoint(src, dst, stream=stream)

    ms_pr = timed(probe_copy, 10, 3)
    probe_gbs = 2 * n_pr * D * D * 4 / (ms_pr * 1e-3) / 1e9
    out["hbm_probe"] = {"what": "1 GiB -> 1 GiB copy with the library's copy kernel (DRAM), "
                                "read + write bytes over time",
                        "ms": round(ms_pr, 3), "GB_per_s": round(probe_gbs, 1)}
    del pa, pb
    out["roofline"]["frac_of_measured_copy"] = round(out["roofline"]["achieved"] / probe_gbs, 4)

    # ---------------- decode workload ----------------
    if not a.no_decode:
        N, Hd, steps = 256, 16, a.decode_steps
        _say("bench: decode")
        Xd = make_decode_steps(N, Hd, D, seed=0, steps=64)
        X = {kk: up(vv) for kk, vv in Xd.items()}
        od = torch.empty((N, Hd, D), dtype=torch.float32, device=dev)
        nx = X["q"].shape[0]
        db = decode_alg_bytes(N, Hd)
        # four independent state sets of the workload (4 x 256 MiB), stepped in turn: each
        # step's states were last touched 768 MiB of traffic ago, so they come from DRAM
        sets = [up(make_decode_state(N, Hd, D, seed=i)) for i in range(4)]
        S_np0 = make_decode_state(N, Hd, D, seed=0)
        ctr = [0]

        def dstep_sets():
            s = ctr[0]
            ctr[0] += 1
            j = s % nx
            kda.kda_decode_step(X["q"][j], X["k"][j], X["v"][j], X["g"][j], X["beta"][j],
                                sets[s % 4], o=od, stream=stream)

        us_dram = timed(dstep_sets, steps, 12) * 1e3
        # per-step distribution: 200 more steps, each between its own pair of events
        per = []
        for _ in range(200):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            dstep_sets()
            e1.record(stream)
            per.append((e0, e1))
        torch.cuda.synchronize()
        per = np.sort(np.array([x.elapsed_time(y) * 1e3 for x, y in per]))
        per_step = {"min": round(float(per[0]), 2), "p50": round(float(np.median(per)), 2),
                    "p90": round(float(per[int(0.9 * len(per))]), 2), "max": round(float(per[-1]), 2),
                    "note": "200 steps, each between its own pair of events (an event pair adds "
                            "about a microsecond)"}
        St = sets[0]
        ctr[0] = 0

        def dstep_one():
            s = ctr[0]
            ctr[0] += 1
            j = s % nx
            kda.kda_decode_step(X["q"][j], X["k"][j], X["v"][j], X["g"][j], X["beta"][j], St,
                                o=od, stream=stream)

        us_cache = timed(dstep_one, steps, 10) * 1e3
        out["decode"] = {
            "workload": "decode 256 sequences x H=16, fp32 128x128 states, bf16 q/k/v, "
                        f"{steps} single-token steps (inputs cycle over {nx} seeded draws), over "
                        "four state sets (1 GiB) in turn: every step reads its 256 MiB of state "
                        "from DRAM",
            "seq_steps_per_s": round(N / (us_dram * 1e-6), 1),
            "us_per_step": round(us_dram, 2),
            "per_step_us": per_step,
            "roofline": _roofline(db, us_dram * 1e-3, kernel="decode_kernel",
                                  frac_of_measured_copy=round(db / (us_dram * 1e-6) / 1e9 / probe_gbs, 4)),
        }
        out["decode_in_cache"] = {
            "workload": "the same step on one state set (256 MiB, near the 256 MB last-level "
                        "cache size): partly served from that cache",
            "seq_steps_per_s": round(N / (us_cache * 1e-6), 1),
            "us_per_step": round(us_cache, 2),
            "roofline": _roofline(db, us_cache * 1e-3, kernel="decode_kernel"),
        }
        del sets, St
        if not a.no_cpu_baseline:
            _say("bench: decode oracle baseline")
            out["decode_cpu_baseline"] = decode_cpu_baseline(S_np0, Xd)
        del S_np0, Xd

    # ---------------- serving: decode over a state pool, write-back to host ----------------
    if not a.no_decode:
        P, N, Hs, steps = 1024, 256, 16, 200
        _say("bench: pooled decode")
        pool = torch.empty((P, Hs, D, D), dtype=torch.float32, device=dev)
        for i in range(0, P, N):                                   # seeded states, 256 at a time
            pool[i:i + N] = up(make_decode_state(N, Hs, D, seed=1 + i // N))
        # four disjoint active batches of N seeded slots, stepped in turn, so that every
        # step's states come from DRAM as in a serving loop over a large pool
        perm = np.random.default_rng(1).permutation(P).astype(np.int32)
        slot_sets = [torch.from_numpy(perm[i * N:(i + 1) * N].copy()).to(dev) for i in range(P // N)]
        slots = slot_sets[0]
        Xp = make_decode_steps(N, Hs, D, seed=1, steps=16)
        XP = {kk: up(vv) for kk, vv in Xp.items()}
        op = torch.empty((N, Hs, D), dtype=torch.float32, device=dev)
        ctr = [0]

        def pstep():
            j = ctr[0] % 16
            sl = slot_sets[ctr[0] % len(slot_sets)]
            ctr[0] += 1
            kda.kda_decode_step_pooled(XP["q"][j], XP["k"][j], XP["v"][j], XP["g"][j], XP["beta"][j],
                                       pool, sl, o=op, stream=stream)

        us = timed(pstep, steps, 5) * 1e3
        db = decode_alg_bytes(N, Hs) + N * 4
        # write-back of the active sequences' states to pinned host memory
        host = torch.empty((N, Hs, D, D), dtype=torch.float32, pin_memory=True)
        wb_ms = timed(lambda: kda.kda_state_copy_indexed(host, pool, src_slots=slots, stream=stream), 3, 1)
        out["decode_pooled"] = {
            "workload": f"decode over a pool of {P} sequences x H={Hs} (fp32 states, 1 GiB), "
                        f"{N} active sequences at seeded slots, {steps} steps over four disjoint "
                        "active batches in turn (states from DRAM)",
            "seq_steps_per_s": round(N / (us * 1e-6), 1),
            "us_per_step": round(us, 2),
            "roofline": _roofline(db, us * 1e-3, kernel="decode_kernel (pooled)"),
            "write_back_to_pinned_host": {"bytes": N * Hs * D * D * 4, "ms": round(wb_ms, 3),
                                          "GB_per_s": round(N * Hs * D * D * 4 / (wb_ms * 1e-3) / 1e9, 1)},
        }
        del pool, host

    # ---------------- backward of the prefill (training) ----------------
    if not a.no_backward:
        from kda_inputs import make_output_grads
        _say("bench: backward")
        dO_np, dS_np = make_output_grads(B, T, H, D, seed=0)
        dO, dSf = up(dO_np), up(dS_np)
        del dO_np
        grads = dict(dq=torch.empty((B, T, H, D), device=dev), dk=torch.empty((B, T, H, D), device=dev),
                     dv=torch.empty((B, T, H, D), device=dev), dg=torch.empty((B, T, H, D), device=dev),
                     dbeta=torch.empty((B, T, H), device=dev), dS0=torch.empty((B, H, D, D), device=dev))
        bws = torch.empty(kda.kda_backward_workspace_size(q, k, v, g, beta, dO), dtype=torch.uint8,
                          device=dev)

        def bstep():
            kda.kda_prefill_backward(q, k, v, g, beta, dO, S0=S0, dS_final=dSf, workspace=bws,
                                     stream=stream, **grads)

        bms = timed(bstep, 10, 5)
        bf = backward_alg_flops(B, T, H)
        out["backward"] = {
            "workload": "gradients of the raw-output prefill above (same q/k/v/g/beta/S0; "
                        "dO ~ N(0,1), dS_T ~ N(0,0.01) fp32): dq, dk, dv, dg, dbeta, dS0 fp32",
            "ms_per_call": round(bms, 3),
            "tokens_per_s": round(B * T / (bms * 1e-3), 1),
            "mfma": {"bound": "mfma", "alg_flops_per_launch": bf,
                     "achieved": round(bf / (bms * 1e-3) / 1e12, 2), "peak": FP32_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(bf / (bms * 1e-3) / 1e12 / FP32_PEAK_TFLOPS, 4),
                     "kernels": "bwd_prep, bwd_fwd, bwd_rev, bwd_grad; fp32 MFMA"},
            "workspace_bytes": int(bws.numel()),
        }
        del grads, bws, dO, dSf

    # one copy kernel of known size (state checkpoint, 64 MiB each way) after the 8k legs:
    # counter runs use it to calibrate FETCH_SIZE / WRITE_SIZE against known bytes
    cal_src = torch.zeros((1024, D, D), dtype=torch.float32, device=dev)
    cal_dst = torch.empty_like(cal_src)
    kda.kda_state_checkpoint(cal_src, cal_dst, stream=stream)
    torch.cuda.synchronize()
    del cal_src, cal_dst

    if not a.no_cpu_baseline:
        _say("bench: prefill oracle baseline")
        out["cpu_baseline"], out["parity"] = cpu_baseline(c, gate=True, o_gpu=o_host, S_gpu=S_host)
    del q, k, v, g, beta, gate, S0, o, Sf, ws, c, o_host, S_host

    # ---------------- long sequences: 131k with checkpoints, 1M over 256 segments ----------------
    if not a.no_long:
        _say("bench: 131k prefill")
        c3 = make_workload("prefill_131k", seed=0)
        T3, H3, every = c3.T, c3.H, 512
        t3 = [up(x) for x in (c3.q, c3.k, c3.v, c3.g, c3.beta)]
        pre3 = {n: np.ascontiguousarray(getattr(c3, n)[:, :8192]) for n in ("q", "k", "v", "g", "beta")}
        del c3
        o3 = torch.empty((1, T3, H3, D), dtype=torch.float32, device=dev)
        S3 = torch.empty((1, H3, D, D), dtype=torch.float32, device=dev)
        ck3 = torch.empty((1, T3 // every, H3, D, D), dtype=torch.float32, device=dev)
        kw3 = dict(o=o3, S_final=S3, chunk=64, ckpt_every=every, ckpt=ck3)
        ws3 = torch.empty(max(1, kda.kda_prefill_workspace_size(*t3, **kw3)), dtype=torch.uint8, device=dev)
        ms3 = timed(lambda: kda.kda_prefill_chunked(*t3, workspace=ws3, stream=stream, **kw3), 10, 3)
        b3 = table_prefill_bytes(1, T3, H3, gate=False, ckpt_every=every, s0=False)
        out["prefill_131k"] = {
            "workload": "prefill B=1 H=16 T=131072 chunk 64, 10% of channels at the -5 floor and "
                        "10% slow-decaying, checkpoints every 512 tokens (256 MiB), fp32 out",
            "ms_per_call": round(ms3, 3),
            "tokens_per_s": round(T3 / (ms3 * 1e-3), 1),
            "roofline": _roofline(b3, ms3, bytes_convention="1540 B per token-head (o counted as "
                                  "bf16) + 128 B of checkpoints + S_final"),
            "mfma_frac": round(prefill_alg_flops(1, T3, H3) / (ms3 * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
            "workspace_bytes": int(ws3.numel()),
        }
        o3_pre = o3[:, :8192].double().cpu().numpy()
        ck3_pre = ck3[:, :8192 // every].double().cpu().numpy()
        del t3, o3, S3, ck3, ws3
        if not a.no_cpu_baseline:
            _say("bench: 131k oracle baseline (prefix)")
            (out["prefill_131k"]["cpu_baseline"],
             out["prefill_131k"]["parity"]) = prefix_cpu_baseline(pre3, T3, H3, every, "checkpoints every 512",
                                                                  o_gpu=o3_pre, ck_gpu=ck3_pre)
        del pre3, o3_pre, ck3_pre

        _say("bench: 1M prefill")
        c4 = make_workload("prefill_1m", seed=0)
        T4, H4 = c4.T, c4.H
        t4 = [up(x) for x in (c4.q, c4.k, c4.v, c4.g, c4.beta)]
        pre4 = {n: np.ascontiguousarray(getattr(c4, n)[:, :16384]) for n in ("q", "k", "v", "g", "beta")}
        del c4
        o4 = torch.empty((1, T4, H4, D), dtype=torch.float32, device=dev)
        S4 = torch.empty((1, H4, D, D), dtype=torch.float32, device=dev)
        kw4 = dict(o=o4, S_final=S4, chunk=64, n_segments=256)
        ws4 = torch.empty(max(1, kda.kda_prefill_workspace_size(*t4, **kw4)), dtype=torch.uint8, device=dev)
        ms4 = timed(lambda: kda.kda_prefill_chunked(*t4, workspace=ws4, stream=stream, **kw4), 3, 1)
        b4 = table_prefill_bytes(1, T4, H4, gate=False, s0=False)
        leg = {
            "workload": "prefill B=1 H=8 T=1048576 chunk 64 over 256 segments combined by the "
                        "associative scan of their state maps, fp32 out",
            "ms_per_call": round(ms4, 3),
            "tokens_per_s": round(T4 / (ms4 * 1e-3), 1),
            "roofline": _roofline(b4, ms4, bytes_convention="1540 B per token-head (o counted as "
                                  "bf16) + S_final"),
            "mfma_frac": round(prefill_alg_flops(1, T4, H4) / (ms4 * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
            "workspace_bytes": int(ws4.numel()),
        }
        o4_pre = o4[:, :16384].double().cpu().numpy()
        del t4, o4, ws4
        # decode tail: 64 single-token steps of the one sequence from the prefill's final
        # state, then the rollback of its 8 states from a checkpoint
        Xt = {kk: up(vv) for kk, vv in make_decode_steps(1, H4, D, seed=7, steps=64).items()}
        st = S4.clone()
        ot = torch.empty((1, H4, D), dtype=torch.float32, device=dev)
        ctr = [0]

        def tstep():
            j = ctr[0] % 64
            ctr[0] += 1
            kda.kda_decode_step(Xt["q"][j], Xt["k"][j], Xt["v"][j], Xt["g"][j], Xt["beta"][j], st,
                                o=ot, stream=stream)

        us_tail = timed(tstep, 64, 4) * 1e3
        # the same steps through prepared DecodeStep objects (buffers checked and bound
        # once, as a serving loop would): the host cost of a launch without the checks
        prepared = [kda.DecodeStep(Xt["q"][j], Xt["k"][j], Xt["v"][j], Xt["g"][j], Xt["beta"][j], st, o=ot)
                    for j in range(64)]
        ctr[0] = 0

        def pstep_tail():
            prepared[ctr[0] % 64](stream)
            ctr[0] += 1

        us_tail_p = timed(pstep_tail, 64, 4) * 1e3
        del prepared
        ckt = torch.empty_like(st)
        kda.kda_state_checkpoint(st, ckt, stream=stream)
        us_rb = timed(lambda: kda.kda_state_rollback(st, ckt, stream=stream), 50, 5) * 1e3
        # the same 64 steps, and 16 rollbacks, captured in HIP graphs and replayed: the
        # device-side cost without one host launch per call (calls made inside the capture
        # go to the capturing stream)
        torch.cuda.synchronize()
        g_tail, g_rb = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_tail):
            for j in range(64):
                kda.kda_decode_step(Xt["q"][j], Xt["k"][j], Xt["v"][j], Xt["g"][j], Xt["beta"][j], st,
                                    o=ot)
        with torch.cuda.graph(g_rb):
            for _ in range(16):
                kda.kda_state_rollback(st, ckt)
        us_tail_g = timed(g_tail.replay, 20, 3) * 1e3 / 64
        us_rb_g = timed(g_rb.replay, 20, 3) * 1e3 / 16
        leg["decode_tail"] = {"us_per_step": round(us_tail, 2), "us_per_step_prepared": round(us_tail_p, 2),
                              "us_per_step_graph": round(us_tail_g, 2), "steps": 64,
                              "note": "one sequence x 8 heads, each state split into four 32-column "
                                      "slices (32 workgroups); us_per_step launches every step from the "
                                      "host through the checking call, us_per_step_prepared through "
                                      "prepared DecodeStep objects, us_per_step_graph replays the 64 "
                                      "steps as one HIP graph"}
        leg["rollback"] = {"us": round(us_rb, 2), "us_graph": round(us_rb_g, 2), "states": H4,
                           "bytes": H4 * D * D * 4}
        del g_tail, g_rb
        if not a.no_cpu_baseline:
            _say("bench: 1M oracle baseline (prefix)")
            leg["cpu_baseline"], leg["parity"] = prefix_cpu_baseline(
                pre4, T4, H4, 0, "no checkpoints; 4 of the 256 segments", o_gpu=o4_pre)
        out["prefill_1m"] = leg
        del S4, st, ckt, Xt, pre4, o4_pre

    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
