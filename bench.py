"""Benchmark of the KDA hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-backward]

Headline (`value`): chunkwise prefill tokens/s on the prefill workload B=4, H=16,
T=8192, d=128, chunk 64, bf16 q/k/v/gate, fp32 g/beta/state, S0 ~ N(0, 0.01), with the
fused per-head RMSNorm and sigmoid gate, fp32 output.  One step = one prefill call over
the whole batch with inputs resident in HBM.  The same run also times the decode
workload (256 sequences x 16 heads, fp32 states, one kernel per step) and reports its
sequence-steps/s, decode over a pool of state slots, and the backward pass of the same
prefill (gradients of the raw outputs, fp32 MFMA) against the fp32 matrix peak.

Prints one JSON line with a `roofline` object for the prefill kernel (algorithmic bytes
over measured duration against 8 TB/s) and a `cpu_baseline` object (the fp64 C oracle
on the host cores over the same prefill workload).
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


def prefill_alg_bytes(B, T, H, out_bytes=4):
    """Bytes the prefill must move: every input read once, every output written once."""
    per_tok_head = 3 * D * 2 + D * 4 + 4 + D * 2 + D * out_bytes   # q,k,v bf16; g; beta; gate; o
    states = 2 * B * H * D * D * 4                                   # S0 in, S_final out
    return B * T * H * per_tok_head + states


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


def cpu_baseline(c, gate):
    """Time the fp64 C oracle (plus the numpy norm/gate) on the host cores."""
    from oracle import native, norm_gate
    from kda_inputs import to_f64
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    threads = max(1, min(cores, 64))
    # whole passes over the workload until about 10 s of wall time (at most 20 passes)
    passes, dt = 0, 0.0
    while passes < 20 and (passes == 0 or dt < 10.0):
        t0 = time.perf_counter()
        o, S, _ = native.prefill(c.q, c.k, c.v, c.g, c.beta, c.S0, bf16=True, nthreads=threads)
        norm_gate(o, to_f64(c.gate, "bf16"), 1e-6) if gate else o
        dt += time.perf_counter() - t0
        passes += 1
    return dict(value=passes * c.B * c.T / dt, unit="tokens/s", cores=threads, kind="oracle",
                sample=f"{passes} passes over the whole prefill workload (B={c.B}, T={c.T}, "
                       f"H={c.H}), fp64 C recurrence + numpy norm/gate, {dt:.1f} s")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
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

    def up(x):
        x = np.ascontiguousarray(x)
        t = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16) if x.dtype == np.uint16 \
            else torch.from_numpy(x)
        return t.to(dev)

    # ---------------- prefill workload ----------------
    B, T, H = 4, 8192, 16
    c = make_workload("prefill_8k", seed=0)
    q, k, v, g, beta, gate, S0 = (up(x) for x in (c.q, c.k, c.v, c.g, c.beta, c.gate, c.S0))
    o = torch.empty((B, T, H, D), dtype=torch.float32, device=dev)
    Sf = torch.empty((B, H, D, D), dtype=torch.float32, device=dev)
    kw = dict(o=o, S0=S0, S_final=Sf, gate=gate, norm_eps=1e-6, chunk=64,
              v_split=a.v_split, n_segments=a.n_segments)
    ws_bytes = kda.kda_prefill_workspace_size(q, k, v, g, beta, **kw)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        kda.kda_prefill_chunked(q, k, v, g, beta, workspace=ws, stream=stream, **kw)

    # warm-up calls (the first tens of calls on a fresh GPU run slower while its clocks
    # ramp up), then K calls back to back between two events on the launch stream
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
    tokens = B * T
    value = tokens / (ms_step * 1e-3)
    alg_b = prefill_alg_bytes(B, T, H)
    alg_f = prefill_alg_flops(B, T, H)
    kernel_ms = ms_mean
    achieved = alg_b / (kernel_ms * 1e-3) / 1e9
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
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "prefill B=4 H=16 T=8192 d=128 chunk=64; bf16 q/k/v/gate, fp32 g/beta/"
                        "state; S0~N(0,0.01); fused per-head RMSNorm + sigmoid gate; fp32 out",
            "global_batch": B, "seq_len": T, "heads": H, "head_dim": D, "chunk": 64,
            "parallelism": "single GPU",
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "kernel": "one prefill call per step: chunk_prep_kernel, chunk_state_kernel (state "
                      "maps), segment_scan, chunk_state_kernel (outputs); their durations sum to "
                      "the call",
            "alg_bytes_per_launch": alg_b,
            "kernel_ms_mean": round(kernel_ms, 4),
        },
        "prefill_mfma": {
            "alg_flops_per_launch": alg_f,
            "achieved_tflops": round(alg_f / (kernel_ms * 1e-3) / 1e12, 2),
            "peak_tflops": BF16_PEAK_TFLOPS,
            "frac": round(alg_f / (kernel_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
        },
    }

    # ---------------- decode workload ----------------
    if not a.no_decode:
        N, Hd, steps = 256, 16, a.decode_steps
        S_np = make_decode_state(N, Hd, D, seed=0)
        Xd = make_decode_steps(N, Hd, D, seed=0, steps=min(steps, 64))
        X = {kk: up(vv) for kk, vv in Xd.items()}
        St = up(S_np)
        od = torch.empty((N, Hd, D), dtype=torch.float32, device=dev)
        nx = X["q"].shape[0]

        def dstep(s):
            j = s % nx
            kda.kda_decode_step(X["q"][j], X["k"][j], X["v"][j], X["g"][j], X["beta"][j], St,
                                o=od, stream=stream)

        for s in range(10):
            dstep(s)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for s in range(steps):
            dstep(s)
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / steps
        db = decode_alg_bytes(N, Hd)
        out["decode"] = {
            "workload": "decode 256 sequences x H=16, fp32 128x128 states, bf16 q/k/v, "
                        f"{steps} single-token steps (inputs cycle over {nx} seeded draws)",
            "seq_steps_per_s": round(N / (us * 1e-6), 1),
            "us_per_step": round(us, 2),
            "roofline": {"bound": "hbm", "achieved": round(db / (us * 1e-6) / 1e9, 1),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(db / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                         "alg_bytes_per_launch": db},
        }

    # ---------------- serving: decode over a state pool, write-back to host ----------------
    if not a.no_decode:
        P, N, Hs, steps = 1024, 256, 16, 200
        pool = torch.empty((P, Hs, D, D), dtype=torch.float32, device=dev)
        for i in range(0, P, N):                                   # seeded states, 256 at a time
            pool[i:i + N] = up(make_decode_state(N, Hs, D, seed=1 + i // N))
        slots = torch.from_numpy(np.random.default_rng(1).permutation(P)[:N].astype(np.int32)).to(dev)
        Xp = make_decode_steps(N, Hs, D, seed=1, steps=16)
        XP = {kk: up(vv) for kk, vv in Xp.items()}
        op = torch.empty((N, Hs, D), dtype=torch.float32, device=dev)

        def pstep(s):
            j = s % 16
            kda.kda_decode_step_pooled(XP["q"][j], XP["k"][j], XP["v"][j], XP["g"][j], XP["beta"][j],
                                       pool, slots, o=op, stream=stream)

        for s in range(5):
            pstep(s)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for s in range(steps):
            pstep(s)
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / steps
        db = decode_alg_bytes(N, Hs) + N * 4
        # write-back of the active sequences' states to pinned host memory
        host = torch.empty((N, Hs, D, D), dtype=torch.float32, pin_memory=True)
        kda.kda_state_copy_indexed(host, pool, src_slots=slots, stream=stream)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(3):
            kda.kda_state_copy_indexed(host, pool, src_slots=slots, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        wb_ms = e0.elapsed_time(e1) / 3
        out["decode_pooled"] = {
            "workload": f"decode over a pool of {P} sequences x H={Hs} (fp32 states, 1 GiB), "
                        f"{N} active sequences at seeded slots, {steps} steps",
            "seq_steps_per_s": round(N / (us * 1e-6), 1),
            "us_per_step": round(us, 2),
            "roofline": {"bound": "hbm", "achieved": round(db / (us * 1e-6) / 1e9, 1),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(db / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                         "alg_bytes_per_launch": db},
            "write_back_to_pinned_host": {"bytes": N * Hs * D * D * 4, "ms": round(wb_ms, 3),
                                          "GB_per_s": round(N * Hs * D * D * 4 / (wb_ms * 1e-3) / 1e9, 1)},
        }
        del pool, host

    # ---------------- backward of the prefill (training) ----------------
    if not a.no_backward:
        from kda_inputs import make_output_grads
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

        for _ in range(5):
            bstep()
        torch.cuda.synchronize()
        nb = 10
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(nb):
            bstep()
        e1.record(stream)
        torch.cuda.synchronize()
        bms = e0.elapsed_time(e1) / nb
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

    # one copy kernel of known size (state checkpoint, 64 MiB each way) after the timed regions:
    # counter runs use it to calibrate FETCH_SIZE / WRITE_SIZE against known bytes
    cal_src = torch.zeros((1024, D, D), dtype=torch.float32, device=dev)
    cal_dst = torch.empty_like(cal_src)
    kda.kda_state_checkpoint(cal_src, cal_dst, stream=stream)
    torch.cuda.synchronize()

    if not a.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(c, gate=True)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
