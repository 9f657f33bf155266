"""The Python binding rejects every mis-shaped, mis-typed or misplaced tensor of the
prefill, decode, pooled decode, indexed copy and checkpoint calls with ValueError
before any pointer reaches the library, so no caller mistake becomes an out-of-bounds
device access.  Tensors live on torch's `meta` device: they carry shapes and dtypes
but no storage, and a well-formed set gets as far as the device check (no HIP device
here), which proves that the shape and dtype checks passed."""
import pytest
import torch

import linear_attention_sequence_kda_amd as kda

META = torch.device("meta")
B, T, H, D = 2, 96, 3, 128
BF, F32 = torch.bfloat16, torch.float32


def t(*shape, dtype=F32):
    return torch.empty(shape, dtype=dtype, device=META)


def prefill_args(**over):
    a = dict(q=t(B, T, H, D, dtype=BF), k=t(B, T, H, D, dtype=BF), v=t(B, T, H, D, dtype=BF),
             g=t(B, T, H, D), beta=t(B, T, H), o=t(B, T, H, D), S0=t(B, H, D, D),
             S_final=t(B, H, D, D), gate=t(B, T, H, D, dtype=BF), norm_weight=t(D),
             ckpt_every=32, ckpt=t(B, T // 32, H, D, D))
    a.update(over)
    return a


def call_prefill(a):
    a = dict(a)
    q, k, v, g, beta = (a.pop(n) for n in ("q", "k", "v", "g", "beta"))
    kda.kda_prefill_chunked(q, k, v, g, beta, chunk=64, **a)


def test_prefill_well_formed_reaches_device_check():
    with pytest.raises(ValueError, match="HIP device"):
        call_prefill(prefill_args(ckpt_every=64, ckpt=t(B, T // 64, H, D, D)))


PREFILL_BAD = [
    ("k", t(B, T, H, 64, dtype=BF), "k has shape"),
    ("k", t(B, T, H, D, dtype=F32), "k has dtype"),
    ("v", t(B, T + 1, H, D, dtype=BF), "v has shape"),
    ("v", t(B, T, H, D, dtype=F32), "v has dtype"),
    ("g", t(B, T, H, D, dtype=BF), "g has dtype"),
    ("g", t(B, T, H, 64), "g has shape"),
    ("beta", t(B, T, H, 1), "beta has shape"),
    ("beta", t(B, T, H, dtype=BF), "beta has dtype"),
    ("o", t(B, T, H + 1, D), "o has shape"),
    ("o", t(B, T, H, D, dtype=torch.float16), "o has dtype"),
    ("S0", t(B, H, D, D, dtype=BF), "S0 has dtype"),
    ("S0", t(B, H, D), "S0 has shape"),
    ("S_final", t(1, H, D, D), "S_final has shape"),
    ("gate", t(B, T, H, D), "gate has dtype"),
    ("gate", t(B, T, H, 64, dtype=BF), "gate has shape"),
    ("norm_weight", t(D + 1), "norm_weight has shape"),
    ("norm_weight", t(D, dtype=BF), "norm_weight has dtype"),
    ("ckpt", t(B, T // 64, H, D, D), "ckpt has shape"),       # sized for another period
    ("ckpt", t(B, T // 32, H, D, D, dtype=BF), "ckpt has dtype"),
    ("ckpt", None, "ckpt is required"),
    ("q", t(B, T, H, dtype=BF), "q must be a 4-d"),
    ("q", t(B, T, H, D, dtype=torch.float16), "q has dtype"),
]


@pytest.mark.parametrize("name,bad,msg", PREFILL_BAD, ids=[f"{n}-{m}" for n, _, m in PREFILL_BAD])
def test_prefill_rejects(name, bad, msg):
    with pytest.raises(ValueError, match=msg):
        call_prefill(prefill_args(**{name: bad}))


def test_prefill_ckpt_without_period_and_other_device():
    with pytest.raises(ValueError, match="ckpt given without ckpt_every"):
        call_prefill(prefill_args(ckpt_every=0))
    with pytest.raises(ValueError, match="expected meta"):
        call_prefill(prefill_args(g=torch.empty((B, T, H, D))))     # a CPU tensor among meta ones


def test_prefill_workspace_size_checks_too():
    a = prefill_args(beta=t(B, T, 1))
    q, k, v, g, beta = (a.pop(n) for n in ("q", "k", "v", "g", "beta"))
    a.pop("o")
    with pytest.raises(ValueError, match="beta has shape"):
        kda.kda_prefill_workspace_size(q, k, v, g, beta, **a)


N = 5


def decode_args(**over):
    a = dict(q=t(N, H, D, dtype=BF), k=t(N, H, D, dtype=BF), v=t(N, H, D, dtype=BF), g=t(N, H, D),
             beta=t(N, H), state=t(N, H, D, D), o=t(N, H, D), gate=t(N, H, D, dtype=BF),
             norm_weight=t(D))
    a.update(over)
    return a


def call_decode(a, pooled=False, slots=None):
    a = dict(a)
    args = [a.pop(n) for n in ("q", "k", "v", "g", "beta", "state")]
    if pooled:
        kda.kda_decode_step_pooled(*args, slots, **a)
    else:
        kda.kda_decode_step(*args, **a)


DECODE_BAD = [
    ("k", t(N, H, 64, dtype=BF), "k has shape"),
    ("v", t(N, H, D), "v has dtype"),
    ("g", t(N, H, D, dtype=BF), "g has dtype"),
    ("g", t(N + 1, H, D), "g has shape"),
    ("beta", t(N, H, 1), "beta has shape"),
    ("state", t(N, H, D, D, dtype=BF), "state has dtype"),
    ("state", t(N - 1, H, D, D), "state has shape"),
    ("state", t(N, H, D), "state must be a 4-d"),
    ("o", t(N, H, 64), "o has shape"),
    ("gate", t(N, H, D), "gate has dtype"),
    ("norm_weight", t(64), "norm_weight has shape"),
]


def test_decode_well_formed_reaches_device_check():
    with pytest.raises(ValueError, match="HIP device"):
        call_decode(decode_args())


@pytest.mark.parametrize("name,bad,msg", DECODE_BAD, ids=[f"{n}-{m}" for n, _, m in DECODE_BAD])
def test_decode_rejects(name, bad, msg):
    with pytest.raises(ValueError, match=msg):
        call_decode(decode_args(**{name: bad}))


def test_pooled_decode_checks():
    slots = t(N, dtype=torch.int32)
    pool = t(4 * N, H, D, D)
    with pytest.raises(ValueError, match="HIP device"):          # any pool size is fine
        call_decode(decode_args(state=pool), pooled=True, slots=slots)
    with pytest.raises(ValueError, match="slots has shape"):
        call_decode(decode_args(state=pool), pooled=True, slots=t(N - 1, dtype=torch.int32))
    with pytest.raises(ValueError, match="slots has dtype"):
        call_decode(decode_args(state=pool), pooled=True, slots=t(N, dtype=torch.int64))
    with pytest.raises(ValueError, match="slots is required"):
        call_decode(decode_args(state=pool), pooled=True, slots=None)
    with pytest.raises(ValueError, match="state has shape"):     # pool with another head count
        call_decode(decode_args(state=t(4 * N, H + 1, D, D)), pooled=True, slots=slots)
    with pytest.raises(ValueError, match="g has dtype"):
        call_decode(decode_args(state=pool, g=t(N, H, D, dtype=BF)), pooled=True, slots=slots)


def test_indexed_copy_and_checkpoint_checks():
    dst, src = t(8, H, D, D), t(8, H, D, D)
    with pytest.raises(ValueError, match="fewer than n"):
        kda.kda_state_copy_indexed(dst, src, src_slots=t(3, dtype=torch.int32), n=4)
    with pytest.raises(ValueError, match="1-d int32"):
        kda.kda_state_copy_indexed(dst, src, dst_slots=t(4, dtype=torch.int64))
    with pytest.raises(ValueError, match="differ in shape"):
        kda.kda_state_copy_indexed(dst, t(8, H, D, 64))
    with pytest.raises(ValueError, match="float32"):
        kda.kda_state_checkpoint(t(2, D, D, dtype=BF), t(2, D, D, dtype=BF))
    with pytest.raises(ValueError, match="shapes differ"):
        kda.kda_state_rollback(t(2, D, D), t(3, D, D))


@pytest.mark.parametrize("name,bad,msg", DECODE_BAD[:4], ids=[f"{n}-{m}" for n, _, m in DECODE_BAD[:4]])
def test_prepared_decode_step_checks_at_construction(name, bad, msg):
    """DecodeStep checks its buffers once, when it is built (the same checks as the
    one-shot call), so that each later call only launches."""
    a = decode_args(**{name: bad})
    args = [a.pop(n) for n in ("q", "k", "v", "g", "beta", "state")]
    with pytest.raises(ValueError, match=msg):
        kda.DecodeStep(*args, **a)
    a = decode_args()
    args = [a.pop(n) for n in ("q", "k", "v", "g", "beta", "state")]
    with pytest.raises(ValueError, match="HIP device"):          # well formed: the device check
        kda.DecodeStep(*args, **a)
    with pytest.raises(ValueError, match="slots has dtype"):
        kda.DecodeStep(*args, slots=t(N, dtype=torch.int64), **a)
