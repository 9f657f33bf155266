"""GPU parity of the chunkwise prefill, through the C ABI, against the fp64 CPU oracle
on the same seeded input bytes.

Tolerances (floating point, no single correct rounding):
  bf16 inputs (BF16/fp16 MFMA):  err_o <= 2e-2, err_S <= 1e-2
  fp32 inputs (fp32 MFMA):       err_o <= 1e-4, err_S <= 1e-4
err_o = max|o - o_ref| / rms(o_ref), err_S = ||S - S_ref||_F / ||S_ref||_F.  Outputs
are stored in fp32 unless a test says otherwise (bf16 storage adds up to 2^-8 of the
largest |o|).
"""
import sys

import numpy as np
import pytest
import torch

import linear_attention_sequence_kda_amd as kda
from kda_inputs import BF16, F32, f32_to_bf16, make_prefill, to_f64
from oracle import native, norm_gate
from gpu_util import up, down, err_o, err_S, bf16_out_tol, dev

pytestmark = pytest.mark.gpu

TOL_O_BF16, TOL_S_BF16 = 2e-2, 1e-2
TOL_O_F32, TOL_S_F32 = 1e-4, 1e-4


def _say(*a):
    print(*a, flush=True, file=sys.stderr)


def run_gpu(c, *, chunk=64, out_dtype=torch.float32, v_split=0, n_segments=0, ckpt_every=0,
            gate=False, norm_weight=None, eps=1e-6, S0=True):
    B, T, H = c.B, c.T, c.H
    o = torch.full((B, T, H, 128), float("nan"), dtype=out_dtype, device=dev())
    Sf = torch.full((B, H, 128, 128), float("nan"), dtype=torch.float32, device=dev())
    ck = None
    if ckpt_every:
        ck = torch.full((B, T // ckpt_every, H, 128, 128), float("nan"), device=dev())
    kda.kda_prefill_chunked(up(c.q), up(c.k), up(c.v), up(c.g), up(c.beta), o=o,
                            S0=up(c.S0) if S0 else None, S_final=Sf,
                            gate=up(c.gate) if gate else None,
                            norm_weight=None if norm_weight is None else up(norm_weight),
                            norm_eps=eps, chunk=chunk, ckpt_every=ckpt_every, ckpt=ck,
                            n_segments=n_segments, v_split=v_split)
    torch.cuda.synchronize()
    return o, Sf, ck


def run_ref(c, *, ckpt_every=0, gate=False, norm_weight=None, eps=1e-6, S0=True):
    o, S, ck = native.prefill(c.q, c.k, c.v, c.g, c.beta, c.S0 if S0 else None,
                              bf16=(c.in_dtype == BF16), ckpt_every=ckpt_every)
    if gate:
        o = norm_gate(o, to_f64(c.gate, c.in_dtype), eps, norm_weight)
    return o, S, ck


def check(c, label, tol_o=TOL_O_BF16, tol_s=TOL_S_BF16, **kw):
    gate = kw.get("gate", False)
    o, S, ck = run_gpu(c, **kw)
    o_ref, S_ref, ck_ref = run_ref(c, ckpt_every=kw.get("ckpt_every", 0), gate=gate,
                                   norm_weight=kw.get("norm_weight"), S0=kw.get("S0", True))
    og = down(o)
    eo, es = err_o(og, o_ref), err_S(down(S), S_ref)
    tol = tol_o if kw.get("out_dtype", torch.float32) == torch.float32 else bf16_out_tol(o_ref, tol_o)
    _say(f"{label}: err_o={eo:.3e} err_S={es:.3e}")
    assert np.isfinite(og).all(), "non-finite output"
    assert eo <= tol, (label, eo)
    assert es <= tol_s, (label, es)
    if ck is not None:
        for m in range(ck_ref.shape[1]):
            e = err_S(down(ck[:, m]), ck_ref[:, m])
            assert e <= tol_s, (label, "ckpt", m, e)
    return o, S


# ---------------------------------------------------------------------------
# small cases spanning several tiles and ragged tails
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("T", [1, 15, 16, 17, 64, 100, 200])
@pytest.mark.parametrize("chunk", [16, 64])
def test_bf16_small_ragged(T, chunk):
    c = make_prefill(2, T, 2, 128, seed=T + chunk, in_dtype=BF16, s0_std=0.05)
    check(c, f"bf16 T={T} chunk={chunk}", chunk=chunk, v_split=1)


@pytest.mark.parametrize("v_split", [1, 2])
def test_bf16_v_split(v_split):
    c = make_prefill(1, 300, 3, 128, seed=11, in_dtype=BF16, s0_std=0.05)
    check(c, f"bf16 v_split={v_split}", chunk=64, v_split=v_split)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_f32_tiny_workload(seed):
    """Tiny fp32 workload: B=1, H=2, T=256, chunk 16, S0 = 0."""
    c = make_prefill(1, 256, 2, 128, seed=seed, in_dtype=F32)
    check(c, f"f32 tiny seed={seed}", TOL_O_F32, TOL_S_F32, chunk=16, S0=False)


@pytest.mark.parametrize("v_split", [1, 2])
def test_f32_ragged_with_state(v_split):
    c = make_prefill(2, 37, 3, 128, seed=5, in_dtype=F32, s0_std=0.1)
    check(c, f"f32 ragged v_split={v_split}", TOL_O_F32, TOL_S_F32, chunk=16, v_split=v_split)


def test_bf16_on_tiny_shapes():
    c = make_prefill(1, 256, 2, 128, seed=0, in_dtype=BF16)
    check(c, "bf16 tiny chunk16", chunk=16, S0=False)
    check(c, "bf16 tiny chunk64", chunk=64, S0=False)


# ---------------------------------------------------------------------------
# decay floor and special cases
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("mode", ["floor", "zero", "below_floor", "raw"])
def test_decay_modes(mode):
    c = make_prefill(1, 192, 2, 128, seed=21, in_dtype=BF16, s0_std=0.1, g_mode=mode)
    check(c, f"g={mode}", chunk=64)


def test_below_floor_equals_floor():
    a = make_prefill(1, 128, 2, 128, seed=22, in_dtype=BF16, s0_std=0.1, g_mode="floor")
    b = make_prefill(1, 128, 2, 128, seed=22, in_dtype=BF16, s0_std=0.1, g_mode="below_floor")
    oa, Sa, _ = run_gpu(a)
    ob, Sb, _ = run_gpu(b)
    assert torch.equal(oa, ob) and torch.equal(Sa, Sb)


def test_beta_zero_only_decays():
    c = make_prefill(2, 150, 2, 128, seed=23, in_dtype=BF16, s0_std=0.1, beta_mode="zero")
    check(c, "beta=0", chunk=64)


def test_beta_one():
    c = make_prefill(1, 150, 2, 128, seed=24, in_dtype=BF16, s0_std=0.1, beta_mode="one")
    check(c, "beta=1", chunk=64)


# ---------------------------------------------------------------------------
# norm + gate, checkpoints, segments
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("v_split", [1, 2])
def test_norm_gate(v_split):
    c = make_prefill(2, 320, 2, 128, seed=31, in_dtype=BF16, s0_std=0.01, gate=True)
    w = np.random.default_rng(31).uniform(0.5, 1.5, 128).astype(np.float32)
    check(c, f"gate v_split={v_split}", chunk=64, v_split=v_split, gate=True, norm_weight=w)
    check(c, f"gate v_split={v_split} bf16 out", chunk=64, v_split=v_split, gate=True,
          out_dtype=torch.bfloat16)


def test_checkpoints():
    c = make_prefill(2, 640, 2, 128, seed=41, in_dtype=BF16, s0_std=0.05)
    check(c, "ckpt every 128", chunk=64, ckpt_every=128)


@pytest.mark.parametrize("n_seg", [2, 3, 8])
def test_segments(n_seg):
    c = make_prefill(1, 1024, 2, 128, seed=51, in_dtype=BF16, s0_std=0.05)
    check(c, f"segments={n_seg}", chunk=64, n_segments=n_seg, ckpt_every=256)


@pytest.mark.parametrize("v_split,out_dtype", [(1, torch.float32), (2, torch.float32),
                                               (2, torch.bfloat16)])
def test_segments_with_gate(v_split, out_dtype):
    """Segments, the fused or separate norm/gate pass, fp32 or bf16 outputs, ragged tail."""
    c = make_prefill(2, 900, 3, 128, seed=54, in_dtype=BF16, s0_std=0.05, gate=True)
    w = np.random.default_rng(54).uniform(0.5, 1.5, 128).astype(np.float32)
    check(c, f"segments gate v_split={v_split} {out_dtype}", chunk=64, n_segments=3,
          v_split=v_split, gate=True, norm_weight=w, out_dtype=out_dtype)


@pytest.mark.parametrize("seg_chunks", [3, 7, 9, 12])
def test_segment_lengths(seg_chunks):
    """Map segments of every length modulo 6 (the state map pass runs its chunks six to
    an unrolled loop iteration and leaves the loop after any of them), ragged tail."""
    n_seg = 3
    T = 64 * seg_chunks * (n_seg - 1) + 64 * (seg_chunks - 1) + 23
    c = make_prefill(1, T, 2, 128, seed=56 + seg_chunks, in_dtype=BF16, s0_std=0.05)
    check(c, f"segments of {seg_chunks} chunks", chunk=64, n_segments=n_seg)


def test_segments_chunk16_gate():
    c = make_prefill(1, 700, 2, 128, seed=55, in_dtype=BF16, s0_std=0.05, gate=True)
    check(c, "segments chunk16 gate", chunk=16, n_segments=4, gate=True, ckpt_every=128)


def test_segments_slow_decay():
    c = make_prefill(1, 2048, 2, 128, seed=52, in_dtype=BF16, pinned_floor_frac=0.1,
                     slow_frac=0.1)
    check(c, "segments slow decay", chunk=64, n_segments=8, S0=False)


def test_segment_count_agreement():
    c = make_prefill(1, 1024, 2, 128, seed=53, in_dtype=BF16, s0_std=0.05)
    outs = [run_gpu(c, n_segments=n) for n in (1, 2, 4, 16)]
    for o, S, _ in outs[1:]:
        assert err_o(down(o), down(outs[0][0])) <= 1e-2
        assert err_S(down(S), down(outs[0][1])) <= 1e-2


def test_deterministic():
    c = make_prefill(2, 200, 2, 128, seed=61, in_dtype=BF16, s0_std=0.05, gate=True)
    o1, S1, _ = run_gpu(c, gate=True, v_split=1)
    o2, S2, _ = run_gpu(c, gate=True, v_split=1)
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


def test_resume_from_checkpoint():
    """Resume = prefill the remaining tokens from a stored checkpoint."""
    c = make_prefill(1, 1024, 2, 128, seed=71, in_dtype=BF16, s0_std=0.05)
    o, S, ck = run_gpu(c, ckpt_every=512)
    tail = make_prefill(1, 1024, 2, 128, seed=71, in_dtype=BF16, s0_std=0.05)
    for name in ("q", "k", "v", "g", "beta"):
        setattr(tail, name, np.ascontiguousarray(getattr(tail, name)[:, 512:]))
    tail.T = 512
    o2 = torch.empty((1, 512, 2, 128), device=dev())
    S2 = torch.empty((1, 2, 128, 128), device=dev())
    kda.kda_prefill_chunked(up(tail.q), up(tail.k), up(tail.v), up(tail.g), up(tail.beta), o=o2,
                            S0=ck[:, 0].contiguous(), S_final=S2, chunk=64)
    torch.cuda.synchronize()
    assert err_o(down(o2), down(o[:, 512:])) <= 1e-5
    assert err_S(down(S2), down(S)) <= 1e-5


def test_empty_and_errors():
    c = make_prefill(1, 0, 2, 128, seed=0, in_dtype=BF16, s0_std=0.1)
    o = torch.empty((1, 0, 2, 128), device=dev())
    Sf = torch.empty((1, 2, 128, 128), device=dev())
    S0 = up(c.S0)
    kda.kda_prefill_chunked(up(c.q), up(c.k), up(c.v), up(c.g), up(c.beta), o=o, S0=S0, S_final=Sf)
    torch.cuda.synchronize()
    assert torch.equal(Sf, S0)
    c = make_prefill(1, 64, 2, 128, seed=0, in_dtype=BF16)
    q = up(c.q)
    with pytest.raises(kda.KdaError) as ei:
        kda.kda_prefill_chunked(q, up(c.k), up(c.v), up(c.g), up(c.beta), o=q)
    assert ei.value.status == kda.KDA_ERR_ALIAS


def test_s_final_may_alias_s0():
    c = make_prefill(1, 200, 2, 128, seed=81, in_dtype=BF16, s0_std=0.05)
    S = up(c.S0).clone()
    o = torch.empty((1, 200, 2, 128), device=dev())
    kda.kda_prefill_chunked(up(c.q), up(c.k), up(c.v), up(c.g), up(c.beta), o=o, S0=S, S_final=S,
                            n_segments=2)
    torch.cuda.synchronize()
    _, S_ref, _ = run_ref(c)
    assert err_S(down(S), S_ref) <= TOL_S_BF16


# ---------------------------------------------------------------------------
# large value magnitudes: v and the state far from the unit scale the workloads draw
# ---------------------------------------------------------------------------
def _scaled_values(c, lo_exp, hi_exp, s0_std, seed):
    """Scale every (token, head) row of v so that its largest magnitude is 10^u,
    u ~ U(lo_exp, hi_exp), and draw S0 with standard deviation s0_std: large but
    bf16-representable inputs."""
    rng = np.random.default_rng([seed, 991])
    v = to_f64(c.v, BF16)
    f = 10.0 ** rng.uniform(lo_exp, hi_exp, size=v.shape[:-1] + (1,)) / np.max(np.abs(v), -1, keepdims=True)
    c.v = f32_to_bf16((v * f).astype(np.float32))
    c.S0 = (rng.standard_normal(c.S0.shape) * s0_std).astype(np.float32)
    return c


@pytest.mark.parametrize("plan", [dict(chunk=64), dict(chunk=64, n_segments=3, ckpt_every=128),
                                  dict(chunk=16, gate=True), dict(chunk=64, v_split=2, gate=True)],
                         ids=["c64", "c64-seg3-ckpt", "c16-gate", "c64-vsplit2-gate"])
def test_large_magnitudes(plan):
    """Rows of v with largest magnitudes from 1e3 to 3e4 and S0 entries ~1e3: the fp16
    operands of the state products (v, the state copy, U) stay inside their range and
    the parity bound holds."""
    c = make_prefill(2, 650, 2, 128, seed=97, in_dtype=BF16, s0_std=1.0, gate=plan.get("gate", False))
    c = _scaled_values(c, 3.0, np.log10(3e4), 1e3, seed=97)
    assert 2e4 < np.max(np.abs(to_f64(c.v, BF16))) <= 3.01e4
    check(c, f"large magnitudes {plan}", **plan)


@pytest.mark.parametrize("plan", [dict(chunk=64), dict(chunk=64, n_segments=3, ckpt_every=128),
                                  dict(chunk=16, gate=True), dict(chunk=64, v_split=2, gate=True),
                                  dict(chunk=64, gate=True), dict(chunk=64, n_segments=40, ckpt_every=64)],
                         ids=["c64", "c64-seg3-ckpt", "c16-gate", "c64-vsplit2-gate", "c64-gate",
                              "c64-seg40-ckpt"])
def test_beyond_fp16_range(plan):
    """Rows of v with largest magnitudes from 1e5 to 3e6 and S0 entries ~1e5: bf16 holds
    them, fp16 (max 65504) does not.  Each 16-column block of the state pass carries a
    power-of-two scale, so the results are finite and meet the same parity bound."""
    T = 64 * 41 if plan.get("n_segments", 0) > 32 else 650
    c = make_prefill(2, T, 2, 128, seed=131, in_dtype=BF16, s0_std=1.0, gate=plan.get("gate", False))
    c = _scaled_values(c, 5.0, np.log10(3e6), 1e5, seed=131)
    assert np.max(np.abs(to_f64(c.v, BF16))) > 65504 and np.max(np.abs(c.S0)) > 65504
    o, S = check(c, f"beyond fp16 range {plan}", **plan)
    assert np.isfinite(down(S)).all()


def test_mixed_magnitudes_per_head():
    """One head at unit scale beside one at 1e6: the scale is per block of columns and
    per head, so the small head loses nothing (errors measured head by head)."""
    c = make_prefill(1, 300, 2, 128, seed=141, in_dtype=BF16, s0_std=0.05)
    v = to_f64(c.v, BF16)
    v[:, :, 1] *= 1e6
    c.v = f32_to_bf16(v.astype(np.float32))
    S0 = c.S0.astype(np.float64)
    S0[:, 1] *= 1e6
    c.S0 = S0.astype(np.float32)
    o, S, _ = run_gpu(c, chunk=64, n_segments=2)
    o_ref, S_ref, _ = run_ref(c)
    og, Sg = down(o), down(S)
    for h in range(2):
        eo, es = err_o(og[:, :, h], o_ref[:, :, h]), err_S(Sg[:, h], S_ref[:, h])
        _say(f"mixed magnitudes, head {h}: err_o={eo:.3e} err_S={es:.3e}")
        assert eo <= TOL_O_BF16 and es <= TOL_S_BF16, (h, eo, es)


def test_scale_returns_to_one():
    """Huge S0 that decays away (g at the floor) while v is at unit scale: the scale
    drops back to 2^0 once the state is small, and the later outputs keep the
    accuracy of an unscaled run."""
    c = make_prefill(1, 640, 1, 128, seed=151, in_dtype=BF16, s0_std=1e6, g_mode="floor")
    o, S, _ = run_gpu(c, chunk=64)
    o_ref, S_ref, _ = run_ref(c)
    og = down(o)
    eo = err_o(og[:, 128:], o_ref[:, 128:])
    _say(f"decayed scale: err_o(after 128 tokens)={eo:.3e} err_S={err_S(down(S), S_ref):.3e}")
    assert eo <= TOL_O_BF16 and err_S(down(S), S_ref) <= TOL_S_BF16


# ---------------------------------------------------------------------------
# the scan in groups (32 segments or more): compose within groups, chain the group
# maps, apply within groups; group counts that do not divide the segment count
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("T,n_seg", [(64 * 33, 33), (64 * 45 - 10, 45), (64 * 64, 64), (64 * 130, 130)])
def test_segments_grouped_scan(T, n_seg):
    c = make_prefill(1, T, 2, 128, seed=57 + n_seg, in_dtype=BF16, s0_std=0.05)
    check(c, f"grouped scan, {n_seg} segments", chunk=64, n_segments=n_seg, ckpt_every=256)


# ---------------------------------------------------------------------------
# 1024 or more chunks per head: the prep kernel takes its workgroups chunk-major (every
# head of a chunk, then the next chunk); records keep their head-major layout
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("B,H,T,chunk", [(2, 3, 16384, 16), (1, 2, 64 * 1024 + 37, 64)])
def test_prep_chunk_major_order(B, H, T, chunk):
    c = make_prefill(B, T, H, 128, seed=83 + chunk, in_dtype=BF16, s0_std=0.05)
    check(c, f"chunk-major prep, B={B} H={H} T={T} chunk={chunk}", chunk=chunk)


@pytest.mark.parametrize("H,T,n_seg,s0", [(60, 640, 3, True), (64, 512, 2, False), (12, 2560, 40, True)])
def test_scan_two_column_blocks(H, T, n_seg, s0):
    """Enough chains for the scan to give each workgroup two 16-column blocks: 60 heads in
    one chain each (padded to 64 chains, the padding exits at once); 64 heads from a zero
    initial state; and 12 heads over 40 segments, whose compose and within-group launches
    take two blocks and whose launch over the 12 group chains takes one."""
    c = make_prefill(1, T, H, 128, seed=71 + n_seg, in_dtype=BF16, s0_std=0.05)
    check(c, f"scan with two column blocks per workgroup, {H} heads, {n_seg} segments, S0={s0}",
          chunk=64, n_segments=n_seg, S0=s0)
