"""C ABI checks that need no GPU: the library loads, exports every symbol that
include/kda.h declares, and rejects bad arguments synchronously before touching a
device.  Fake pointers used here are never dereferenced: every call either fails
validation or (with no GPU) fails the device check."""
import ctypes as C
import os
import re

import pytest

import linear_attention_sequence_kda_amd as kda
from linear_attention_sequence_kda_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "kda.h")).read()
    return sorted(set(re.findall(r"KDA_API\s+[\w\s\*]+?\b(kda_\w+)\s*\(", src)))


def test_header_declares_entry_points():
    names = _declared()
    for n in ("kda_prefill_chunked", "kda_decode_step", "kda_decode_step_pooled",
              "kda_state_checkpoint", "kda_state_rollback", "kda_state_copy_indexed",
              "kda_prefill_workspace_size", "kda_status_string", "kda_abi_version",
              "kda_prefill_backward", "kda_backward_workspace_size",
              "kda_prefill_chunked_noalloc"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = C.CDLL(_lib.LIB_PATH)
    for n in _declared():
        assert hasattr(lib, n), n


def test_status_strings_and_version():
    assert kda.kda_abi_version() == 3
    seen = set()
    for st in range(8):
        s = kda.status_string(st)
        assert s and s not in seen
        seen.add(s)
    assert kda.status_string(99) == "unknown status"


FAKE = 1 << 40   # never dereferenced


def _desc(**over):
    d = _lib.PrefillDesc()
    d.B, d.T, d.H, d.d_k, d.d_v, d.chunk = 2, 128, 4, 128, 128, 64
    d.in_dtype, d.out_dtype = _lib.KDA_BF16, _lib.KDA_F32
    n = 2 * 128 * 4 * 128
    base = FAKE
    d.q, d.k, d.v = base, base + 2 * n, base + 4 * n
    d.g, d.beta = base + 6 * n, base + 10 * n
    d.o = base + 20 * n
    d.v_split, d.n_segments = 1, 1
    for k, v in over.items():
        setattr(d, k, v)
    # every prefill with tokens needs a workspace for its per-chunk records
    n = C.c_size_t(0)
    if _lib.load().kda_prefill_workspace_size(C.byref(d), C.byref(n)) == kda.KDA_OK:
        d.workspace, d.workspace_bytes = FAKE + (1 << 36), n.value
    return d


def _call(d):
    return _lib.load().kda_prefill_chunked(C.byref(d), None)


def _gpu_present():
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:
        return False


def test_prefill_validation_errors():
    lib = _lib.load()
    assert lib.kda_prefill_chunked(None, None) == kda.KDA_ERR_NULL
    assert _call(_desc(d_k=64)) == kda.KDA_ERR_UNSUPPORTED
    assert _call(_desc(chunk=32)) == kda.KDA_ERR_UNSUPPORTED
    assert _call(_desc(in_dtype=7)) == kda.KDA_ERR_UNSUPPORTED
    assert _call(_desc(v_split=3)) == kda.KDA_ERR_UNSUPPORTED
    assert _call(_desc(v_split=4)) == kda.KDA_ERR_UNSUPPORTED
    assert _call(_desc(B=-1)) == kda.KDA_ERR_SHAPE
    assert _call(_desc(ckpt_every=100)) == kda.KDA_ERR_SHAPE
    assert _call(_desc(n_segments=3)) == kda.KDA_ERR_SHAPE           # 2 chunks only
    assert _call(_desc(B=1 << 16, H=1 << 15, T=64)) == kda.KDA_ERR_SHAPE   # 2^31 chunk-heads
    assert _call(_desc(q=None)) == kda.KDA_ERR_NULL
    assert _call(_desc(ckpt_every=64)) == kda.KDA_ERR_NULL            # ckpt missing
    d = _desc()
    d.o = d.k + 100                                                  # o overlaps k
    assert _call(d) == kda.KDA_ERR_ALIAS
    d = _desc(n_segments=2)
    d.workspace, d.workspace_bytes = None, 0                         # needs a workspace
    assert _call(d) == kda.KDA_ERR_WORKSPACE
    n = C.c_size_t(0)
    assert lib.kda_prefill_workspace_size(C.byref(d), C.byref(n)) == kda.KDA_OK
    # per-chunk records (2 chunks x 8 heads; a 64-token record holds W, Kdec and Qt,
    # 64 x 128 fp16 each, the 6 stored 16x32 blocks of T and of P, and 128 fp32
    # decays) + maps and entering states of 2 segments
    rec = 3 * 64 * 128 * 2 + 2 * 6 * 16 * 32 * 2 + 128 * 4
    assert n.value >= 2 * 4 * 2 * rec + 2 * 4 * 2 * 3 * 128 * 128 * 4
    d.workspace, d.workspace_bytes = FAKE + (1 << 36), n.value - 1
    assert _call(d) == kda.KDA_ERR_WORKSPACE
    assert lib.kda_prefill_workspace_size(C.byref(_desc()), None) == kda.KDA_ERR_NULL


def test_empty_prefill_is_a_noop():
    # B*H == 0 returns before the device check
    assert _call(_desc(B=0)) == kda.KDA_OK


@pytest.mark.skipif(_gpu_present(), reason="checks the no-device error path")
def test_prefill_without_device_reports_device_error():
    assert _call(_desc()) == kda.KDA_ERR_DEVICE
    assert _call(_desc(v_split=2)) == kda.KDA_ERR_DEVICE     # both column splits validate


def _ddesc(**over):
    d = _lib.DecodeDesc()
    d.N, d.H, d.d_k, d.d_v = 4, 2, 128, 128
    d.in_dtype, d.out_dtype = _lib.KDA_BF16, _lib.KDA_F32
    n = 4 * 2 * 128
    d.q, d.k, d.v, d.g, d.beta = FAKE, FAKE + 2 * n, FAKE + 4 * n, FAKE + 6 * n, FAKE + 10 * n
    d.state, d.o = FAKE + (1 << 30), FAKE + (1 << 31)
    for k, v in over.items():
        setattr(d, k, v)
    return d


def test_decode_validation_errors():
    lib = _lib.load()
    f = lambda d: lib.kda_decode_step(C.byref(d), None)  # noqa: E731
    assert lib.kda_decode_step(None, None) == kda.KDA_ERR_NULL
    assert f(_ddesc(d_v=64)) == kda.KDA_ERR_UNSUPPORTED
    assert f(_ddesc(N=-2)) == kda.KDA_ERR_SHAPE
    assert f(_ddesc(N=1 << 16, H=1 << 15)) == kda.KDA_ERR_SHAPE       # 2^31 states
    assert f(_ddesc(state=None)) == kda.KDA_ERR_NULL
    d = _ddesc()
    d.o = d.q
    assert f(d) == kda.KDA_ERR_ALIAS
    d = _ddesc()
    d.state = d.v
    assert f(d) == kda.KDA_ERR_ALIAS
    assert f(_ddesc(N=0)) == kda.KDA_OK


def test_copy_validation_errors():
    lib = _lib.load()
    assert lib.kda_state_checkpoint(FAKE, FAKE + 8, 1, 128, 128, None) == kda.KDA_ERR_ALIAS
    assert lib.kda_state_rollback(None, FAKE, 1, 128, 128, None) == kda.KDA_ERR_NULL
    assert lib.kda_state_rollback(FAKE, FAKE + (1 << 20), -1, 128, 128, None) == kda.KDA_ERR_SHAPE
    assert lib.kda_state_checkpoint(FAKE, FAKE + (1 << 20), 0, 128, 128, None) == kda.KDA_OK


def test_pooled_decode_validation_errors():
    lib = _lib.load()
    f = lambda d, slots, pool: lib.kda_decode_step_pooled(C.byref(d), slots, pool, None)  # noqa: E731
    assert lib.kda_decode_step_pooled(None, FAKE, 4, None) == kda.KDA_ERR_NULL
    assert f(_ddesc(), None, 8) == kda.KDA_ERR_NULL                   # slots missing
    assert f(_ddesc(), FAKE + (1 << 33), -1) == kda.KDA_ERR_SHAPE      # negative pool
    assert f(_ddesc(d_k=64), FAKE + (1 << 33), 8) == kda.KDA_ERR_UNSUPPORTED
    d = _ddesc()
    d.state = d.g - 4096                                             # an 8-slot pool over g
    assert f(d, FAKE + (1 << 33), 8) == kda.KDA_ERR_ALIAS
    assert f(_ddesc(N=0), None, 8) == kda.KDA_OK                       # empty batch: no-op


def test_indexed_copy_validation_errors():
    lib = _lib.load()
    f = lib.kda_state_copy_indexed
    S = 16 * 128 * 128
    assert f(None, None, 4, FAKE, None, 4, 4, S, None) == kda.KDA_ERR_NULL
    assert f(FAKE, None, 4, None, None, 4, 4, S, None) == kda.KDA_ERR_NULL
    assert f(FAKE, None, 4, FAKE + (1 << 34), None, 4, -1, S, None) == kda.KDA_ERR_SHAPE
    assert f(FAKE, None, 4, FAKE + (1 << 34), None, 4, 4, -5, None) == kda.KDA_ERR_SHAPE
    assert f(FAKE, None, 2, FAKE + (1 << 34), None, 4, 3, S, None) == kda.KDA_ERR_SHAPE  # n > dst_count
    assert f(FAKE, None, 4, FAKE + (1 << 34), None, 2, 3, S, None) == kda.KDA_ERR_SHAPE  # n > src_count
    # with slot arrays, counts only bound the slots (checked on the device)
    assert f(None, FAKE, 2, None, FAKE, 2, 0, S, None) == kda.KDA_OK   # nothing to copy
    assert f(FAKE, FAKE + 64, 1, FAKE + (1 << 34), None, 1 << 40, 1 << 30, 1 << 20, None) == kda.KDA_ERR_SHAPE


def _bdesc(**over):
    d = _lib.BackwardDesc()
    d.B, d.T, d.H, d.d_k, d.d_v, d.chunk, d.in_dtype = 2, 100, 3, 128, 128, 64, _lib.KDA_BF16
    n = 2 * 100 * 3 * 128 * 4          # bytes of one fp32 [B,T,H,128] array
    base = FAKE
    d.q, d.k, d.v, d.g, d.beta, d.dO = (base + i * n for i in range(6))
    d.dq, d.dk, d.dv, d.dg, d.dbeta = (base + (10 + i) * n for i in range(5))
    d.workspace, d.workspace_bytes = base + 20 * n, 1 << 30
    for k, v in over.items():
        setattr(d, k, v)
    return d


def test_backward_workspace_size():
    lib = _lib.load()
    n = C.c_size_t(0)
    assert lib.kda_backward_workspace_size(C.byref(_bdesc()), C.byref(n)) == kda.KDA_OK
    # 2 chunks per sequence (T = 100), 2 x 3 heads: record + state + state gradient + dU
    rec = 5 * 64 * 128 + 3 * 64 * 64 + 128
    assert n.value == 2 * 3 * 2 * (rec + 2 * 128 * 128 + 64 * 128) * 4
    assert lib.kda_backward_workspace_size(C.byref(_bdesc(T=0)), C.byref(n)) == kda.KDA_OK
    assert n.value == 0
    assert lib.kda_backward_workspace_size(C.byref(_bdesc(chunk=16)), C.byref(n)) == kda.KDA_ERR_UNSUPPORTED
    assert lib.kda_backward_workspace_size(None, C.byref(n)) == kda.KDA_ERR_NULL


def test_backward_validation_errors():
    lib = _lib.load()
    f = lambda d: lib.kda_prefill_backward(C.byref(d), None)  # noqa: E731
    assert lib.kda_prefill_backward(None, None) == kda.KDA_ERR_NULL
    assert f(_bdesc(d_k=64)) == kda.KDA_ERR_UNSUPPORTED
    assert f(_bdesc(chunk=16)) == kda.KDA_ERR_UNSUPPORTED
    assert f(_bdesc(in_dtype=7)) == kda.KDA_ERR_UNSUPPORTED
    assert f(_bdesc(T=-1)) == kda.KDA_ERR_SHAPE
    assert f(_bdesc(dO=None)) == kda.KDA_ERR_NULL
    assert f(_bdesc(dbeta=None)) == kda.KDA_ERR_NULL
    assert f(_bdesc(workspace=None)) == kda.KDA_ERR_WORKSPACE
    assert f(_bdesc(workspace_bytes=1000)) == kda.KDA_ERR_WORKSPACE
    d = _bdesc()
    d.dq = d.k                                   # output over an input
    assert f(d) == kda.KDA_ERR_ALIAS
    d = _bdesc()
    d.dg = d.dk + 64                             # two outputs overlap
    assert f(d) == kda.KDA_ERR_ALIAS
    d = _bdesc()
    d.workspace = d.dv                           # workspace over an output
    assert f(d) == kda.KDA_ERR_ALIAS
    assert f(_bdesc(B=0)) == kda.KDA_OK          # nothing to do


def test_backward_binding_checks_dtypes_and_shapes():
    """The binding rejects a wrong dtype or shape before any pointer reaches the library
    (tensors on the CPU never get that far either: the device check comes later)."""
    import torch
    B, T, H = 1, 5, 1
    q = torch.zeros(B, T, H, 128)
    g = torch.zeros(B, T, H, 128)
    beta = torch.zeros(B, T, H)
    good = dict(dq=torch.zeros(B, T, H, 128), dk=torch.zeros(B, T, H, 128),
                dv=torch.zeros(B, T, H, 128), dg=torch.zeros(B, T, H, 128), dbeta=torch.zeros(B, T, H))
    with pytest.raises(ValueError, match="dO must be float32"):
        kda.kda_prefill_backward(q, q, q, g, beta, torch.zeros(B, T, H, 128, dtype=torch.bfloat16), **good)
    bad = dict(good, dbeta=torch.zeros(B, T, H, 1))
    with pytest.raises(ValueError, match="dbeta has shape"):
        kda.kda_prefill_backward(q, q, q, g, beta, torch.zeros(B, T, H, 128), **bad)


def test_noalloc_refuses_descriptors_beyond_its_array():
    """kda_prefill_chunked_noalloc checks the workspace its descriptor needs against the
    fixed device array before touching a device: too large -> KDA_ERR_WORKSPACE; a
    descriptor that fits gets as far as the device check (no GPU here)."""
    lib = _lib.load()
    big = _desc(T=16384, H=8, B=1)                    # 8 x 256 chunk records of 61 KiB > 64 MiB
    assert lib.kda_prefill_chunked_noalloc(C.byref(big), None) == kda.KDA_ERR_WORKSPACE
    assert lib.kda_prefill_chunked_noalloc(C.byref(_desc(d_k=64)), None) == kda.KDA_ERR_UNSUPPORTED
    assert lib.kda_prefill_chunked_noalloc(C.byref(_desc(B=0)), None) == kda.KDA_OK
    if not _gpu_present():
        small = _desc()
        small.workspace, small.workspace_bytes = None, 0   # ignored by this entry point
        assert lib.kda_prefill_chunked_noalloc(C.byref(small), None) == kda.KDA_ERR_DEVICE
