"""ctypes binding of libkda.so (include/kda.h): argument marshalling only.

Each function has the name of the C entry point it calls, takes torch tensors that
live on the current HIP device, fills the C descriptor and raises KdaError on a
non-zero status.  Every step of the computation runs in the HIP kernels; torch only
provides device memory and the stream.  There is no fallback: if the library is
missing or the device is not gfx950, calls raise.
"""
from __future__ import annotations

import ctypes as C
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libkda.so")

KDA_OK, KDA_ERR_NULL, KDA_ERR_SHAPE, KDA_ERR_UNSUPPORTED, KDA_ERR_WORKSPACE, \
    KDA_ERR_ALIAS, KDA_ERR_DEVICE, KDA_ERR_HIP = range(8)
KDA_F32, KDA_BF16 = 0, 1

_DT = {torch.float32: KDA_F32, torch.bfloat16: KDA_BF16}


class KdaError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn}: status {status}: {msg}")
        self.status = status


class PrefillDesc(C.Structure):
    _fields_ = [
        ("B", C.c_int32), ("T", C.c_int32), ("H", C.c_int32),
        ("d_k", C.c_int32), ("d_v", C.c_int32), ("chunk", C.c_int32),
        ("in_dtype", C.c_int32), ("out_dtype", C.c_int32),
        ("q", C.c_void_p), ("k", C.c_void_p), ("v", C.c_void_p),
        ("g", C.c_void_p), ("beta", C.c_void_p), ("S0", C.c_void_p),
        ("S_final", C.c_void_p), ("o", C.c_void_p), ("gate", C.c_void_p),
        ("norm_weight", C.c_void_p), ("norm_eps", C.c_float),
        ("ckpt_every", C.c_int32), ("ckpt", C.c_void_p),
        ("n_segments", C.c_int32), ("v_split", C.c_int32),
        ("workspace", C.c_void_p), ("workspace_bytes", C.c_size_t),
    ]


class DecodeDesc(C.Structure):
    _fields_ = [
        ("N", C.c_int32), ("H", C.c_int32), ("d_k", C.c_int32), ("d_v", C.c_int32),
        ("in_dtype", C.c_int32), ("out_dtype", C.c_int32),
        ("q", C.c_void_p), ("k", C.c_void_p), ("v", C.c_void_p),
        ("g", C.c_void_p), ("beta", C.c_void_p), ("state", C.c_void_p), ("o", C.c_void_p),
        ("gate", C.c_void_p), ("norm_weight", C.c_void_p), ("norm_eps", C.c_float),
    ]


class BackwardDesc(C.Structure):
    _fields_ = [
        ("B", C.c_int32), ("T", C.c_int32), ("H", C.c_int32),
        ("d_k", C.c_int32), ("d_v", C.c_int32), ("chunk", C.c_int32), ("in_dtype", C.c_int32),
        ("q", C.c_void_p), ("k", C.c_void_p), ("v", C.c_void_p),
        ("g", C.c_void_p), ("beta", C.c_void_p), ("S0", C.c_void_p),
        ("dO", C.c_void_p), ("dS_final", C.c_void_p),
        ("dq", C.c_void_p), ("dk", C.c_void_p), ("dv", C.c_void_p), ("dg", C.c_void_p),
        ("dbeta", C.c_void_p), ("dS0", C.c_void_p),
        ("workspace", C.c_void_p), ("workspace_bytes", C.c_size_t),
    ]


_lib = None


def load(path: str = LIB_PATH):
    """Load libkda.so (raises OSError if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise OSError(f"{path} not found: build it with "
                          "`python -m linear_attention_sequence_kda_amd.build`")
        lib = C.CDLL(path)
        vp = C.c_void_p
        lib.kda_prefill_workspace_size.argtypes = [C.POINTER(PrefillDesc), C.POINTER(C.c_size_t)]
        lib.kda_prefill_workspace_size.restype = C.c_int
        lib.kda_prefill_chunked.argtypes = [C.POINTER(PrefillDesc), vp]
        lib.kda_prefill_chunked.restype = C.c_int
        lib.kda_prefill_chunked_noalloc.argtypes = [C.POINTER(PrefillDesc), vp]
        lib.kda_prefill_chunked_noalloc.restype = C.c_int
        lib.kda_decode_step.argtypes = [C.POINTER(DecodeDesc), vp]
        lib.kda_decode_step.restype = C.c_int
        lib.kda_decode_step_pooled.argtypes = [C.POINTER(DecodeDesc), vp, C.c_int32, vp]
        lib.kda_decode_step_pooled.restype = C.c_int
        lib.kda_state_copy_indexed.argtypes = [vp, vp, C.c_int64, vp, vp, C.c_int64, C.c_int64,
                                               C.c_int64, vp]
        lib.kda_state_copy_indexed.restype = C.c_int
        lib.kda_state_checkpoint.argtypes = [vp, vp, C.c_int64, C.c_int32, C.c_int32, vp]
        lib.kda_state_checkpoint.restype = C.c_int
        lib.kda_state_rollback.argtypes = [vp, vp, C.c_int64, C.c_int32, C.c_int32, vp]
        lib.kda_state_rollback.restype = C.c_int
        lib.kda_backward_workspace_size.argtypes = [C.POINTER(BackwardDesc), C.POINTER(C.c_size_t)]
        lib.kda_backward_workspace_size.restype = C.c_int
        lib.kda_prefill_backward.argtypes = [C.POINTER(BackwardDesc), vp]
        lib.kda_prefill_backward.restype = C.c_int
        lib.kda_status_string.argtypes = [C.c_int]
        lib.kda_status_string.restype = C.c_char_p
        lib.kda_abi_version.argtypes = []
        lib.kda_abi_version.restype = C.c_int32
        _lib = lib
    return _lib


def status_string(st: int) -> str:
    return load().kda_status_string(st).decode()


def _check(fn: str, st: int) -> None:
    if st != KDA_OK:
        raise KdaError(fn, st, status_string(st))


def _ptr(t):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch.Tensor")
    if not t.is_cuda:
        raise ValueError("tensor must be on the HIP device")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr() if t.numel() > 0 else None


def _ptr_any(t):
    """Device tensor, or pinned host tensor (device-accessible at the same address)."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch.Tensor")
    if not (t.is_cuda or t.is_pinned()):
        raise ValueError("tensor must be on the HIP device or in pinned host memory")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr() if t.numel() > 0 else None


def _slots(t):
    if t is None:
        return None
    if t.dtype != torch.int32:
        raise ValueError("slot arrays must be int32")
    return _ptr(t)


def _dtype(t) -> int:
    try:
        return _DT[t.dtype]
    except KeyError:
        raise ValueError(f"unsupported dtype {t.dtype}; use float32 or bfloat16") from None


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if isinstance(stream, torch.cuda.Stream) else stream


def _expect(name, t, shape, dtypes, device=None, optional=False):
    """Raise ValueError unless `t` has exactly `shape` and one of `dtypes` (and lives on
    `device` when given).  Checked before any pointer is taken, so a mis-shaped or
    mis-typed tensor never reaches a kernel."""
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype not in dtypes:
        want = " or ".join(str(d).replace("torch.", "") for d in dtypes)
        raise ValueError(f"{name} has dtype {str(t.dtype).replace('torch.', '')}, expected {want}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device} (the device of q)")


_IN_DTYPES = (torch.float32, torch.bfloat16)
_F32 = (torch.float32,)


def _check_prefill(q, k, v, g, beta, o, S0, S_final, gate, norm_weight, ckpt_every, ckpt,
                   workspace, need_o=True):
    """Shapes and dtypes of every prefill tensor against q: [B,T,H,d_k]."""
    if not isinstance(q, torch.Tensor) or q.dim() != 4:
        raise ValueError("q must be a 4-d tensor [B, T, H, d_k]")
    _expect("q", q, q.shape, _IN_DTYPES)
    B, T, H, dk = (int(x) for x in q.shape)
    dev = q.device
    if not isinstance(v, torch.Tensor) or v.dim() != 4:
        raise ValueError("v must be a 4-d tensor [B, T, H, d_v]")
    dv = int(v.shape[-1])
    _expect("k", k, (B, T, H, dk), (q.dtype,), dev)
    _expect("v", v, (B, T, H, dv), (q.dtype,), dev)
    _expect("g", g, (B, T, H, dk), _F32, dev)
    _expect("beta", beta, (B, T, H), _F32, dev)
    _expect("o", o, (B, T, H, dv), _IN_DTYPES, dev, optional=not need_o)
    _expect("S0", S0, (B, H, dk, dv), _F32, dev, optional=True)
    _expect("S_final", S_final, (B, H, dk, dv), _F32, dev, optional=True)
    _expect("gate", gate, (B, T, H, dv), (q.dtype,), dev, optional=True)
    _expect("norm_weight", norm_weight, (dv,), _F32, dev, optional=True)
    every = int(ckpt_every)
    if every < 0:
        raise ValueError("ckpt_every must be >= 0")
    if every > 0:
        _expect("ckpt", ckpt, (B, T // every, H, dk, dv), _F32, dev,
                optional=(B * H * (T // every) == 0))
    elif ckpt is not None:
        raise ValueError("ckpt given without ckpt_every")
    if workspace is not None:
        if not isinstance(workspace, torch.Tensor) or workspace.device != dev:
            raise ValueError(f"workspace must be a tensor on {dev}")


def _check_decode(q, k, v, g, beta, state, o, gate, norm_weight, pooled=False):
    """Shapes and dtypes of every decode tensor against q: [N,H,d_k]; the state holds N
    states per head, or any number (the pool) for the pooled step."""
    if not isinstance(q, torch.Tensor) or q.dim() != 3:
        raise ValueError("q must be a 3-d tensor [N, H, d_k]")
    _expect("q", q, q.shape, _IN_DTYPES)
    N, H, dk = (int(x) for x in q.shape)
    dev = q.device
    if not isinstance(v, torch.Tensor) or v.dim() != 3:
        raise ValueError("v must be a 3-d tensor [N, H, d_v]")
    dv = int(v.shape[-1])
    _expect("k", k, (N, H, dk), (q.dtype,), dev)
    _expect("v", v, (N, H, dv), (q.dtype,), dev)
    _expect("g", g, (N, H, dk), _F32, dev)
    _expect("beta", beta, (N, H), _F32, dev)
    if not isinstance(state, torch.Tensor) or state.dim() != 4:
        raise ValueError("state must be a 4-d tensor [N, H, d_k, d_v]")
    _expect("state", state, (int(state.shape[0]) if pooled else N, H, dk, dv), _F32, dev)
    _expect("o", o, (N, H, dv), _IN_DTYPES, dev)
    _expect("gate", gate, (N, H, dv), (q.dtype,), dev, optional=True)
    _expect("norm_weight", norm_weight, (dv,), _F32, dev, optional=True)


def kda_abi_version() -> int:
    return int(load().kda_abi_version())


def _prefill_desc(q, k, v, g, beta, *, o, S0=None, S_final=None, gate=None, norm_weight=None,
                  norm_eps=1e-6, chunk=64, ckpt_every=0, ckpt=None, n_segments=0, v_split=0,
                  workspace=None) -> PrefillDesc:
    _check_prefill(q, k, v, g, beta, o, S0, S_final, gate, norm_weight, ckpt_every, ckpt,
                   workspace, need_o=o is not None)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    d = PrefillDesc()
    d.B, d.T, d.H, d.d_k, d.d_v, d.chunk = B, T, H, dk, dv, chunk
    d.in_dtype = _dtype(q)
    d.out_dtype = _dtype(o) if o is not None else KDA_F32
    d.q, d.k, d.v, d.g, d.beta = _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta)
    d.S0, d.S_final, d.o, d.gate = _ptr(S0), _ptr(S_final), _ptr(o), _ptr(gate)
    d.norm_weight, d.norm_eps = _ptr(norm_weight), float(norm_eps)
    d.ckpt_every, d.ckpt = int(ckpt_every), _ptr(ckpt)
    d.n_segments, d.v_split = int(n_segments), int(v_split)
    if workspace is not None:
        d.workspace, d.workspace_bytes = _ptr(workspace), workspace.numel() * workspace.element_size()
    return d


def kda_prefill_workspace_size(q, k, v, g, beta, **kw) -> int:
    """Workspace bytes kda_prefill_chunked needs for these arguments."""
    kw.setdefault("o", None)
    d = _prefill_desc(q, k, v, g, beta, **kw)
    n = C.c_size_t(0)
    _check("kda_prefill_workspace_size", load().kda_prefill_workspace_size(C.byref(d), C.byref(n)))
    return int(n.value)


def kda_prefill_chunked(q, k, v, g, beta, *, o, S0=None, S_final=None, gate=None,
                        norm_weight=None, norm_eps=1e-6, chunk=64, ckpt_every=0, ckpt=None,
                        n_segments=0, v_split=0, workspace=None, stream=None) -> None:
    """Chunkwise prefill into the caller's `o` (and S_final / ckpt when given).

    q, k: [B,T,H,128]; v, gate: [B,T,H,128] (all float32 or all bfloat16); g: [B,T,H,128]
    float32; beta: [B,T,H] float32; S0, S_final: [B,H,128,128] float32; o: [B,T,H,128]
    float32 or bfloat16; ckpt: [B, T // ckpt_every, H, 128, 128] float32.  If the plan needs
    a workspace and none is given, one is allocated from torch's caching allocator."""
    kw = dict(o=o, S0=S0, S_final=S_final, gate=gate, norm_weight=norm_weight, norm_eps=norm_eps,
              chunk=chunk, ckpt_every=ckpt_every, ckpt=ckpt, n_segments=n_segments,
              v_split=v_split)
    if workspace is None:
        n = kda_prefill_workspace_size(q, k, v, g, beta, **kw)
        if n > 0:
            workspace = torch.empty(n, dtype=torch.uint8, device=q.device)
    d = _prefill_desc(q, k, v, g, beta, workspace=workspace, **kw)
    _check("kda_prefill_chunked", load().kda_prefill_chunked(C.byref(d), _stream(stream)))


# bytes of the fixed device workspace behind kda_prefill_chunked_noalloc (KDA_NOALLOC_WORKSPACE_BYTES)
NOALLOC_WORKSPACE_BYTES = 64 << 20


def kda_prefill_chunked_noalloc(q, k, v, g, beta, *, o, S0=None, S_final=None, gate=None,
                                norm_weight=None, norm_eps=1e-6, chunk=64, ckpt_every=0,
                                ckpt=None, n_segments=0, v_split=0, stream=None) -> None:
    """kda_prefill_chunked without any allocation: the workspace is the library's fixed
    per-device array of NOALLOC_WORKSPACE_BYTES (calls on one device must not overlap in
    time).  Raises KdaError with KDA_ERR_WORKSPACE when the call needs more than that."""
    d = _prefill_desc(q, k, v, g, beta, o=o, S0=S0, S_final=S_final, gate=gate,
                      norm_weight=norm_weight, norm_eps=norm_eps, chunk=chunk,
                      ckpt_every=ckpt_every, ckpt=ckpt, n_segments=n_segments, v_split=v_split)
    _check("kda_prefill_chunked_noalloc", load().kda_prefill_chunked_noalloc(C.byref(d), _stream(stream)))


def _decode_desc(q, k, v, g, beta, state, o, gate, norm_weight, norm_eps, pooled=False) -> DecodeDesc:
    _check_decode(q, k, v, g, beta, state, o, gate, norm_weight, pooled)
    N, H, dk = q.shape
    d = DecodeDesc()
    d.N, d.H, d.d_k, d.d_v = N, H, dk, v.shape[-1]
    d.in_dtype, d.out_dtype = _dtype(q), _dtype(o)
    d.q, d.k, d.v, d.g, d.beta = _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta)
    d.state, d.o, d.gate = _ptr(state), _ptr(o), _ptr(gate)
    d.norm_weight, d.norm_eps = _ptr(norm_weight), float(norm_eps)
    return d


def kda_decode_step(q, k, v, g, beta, state, *, o, gate=None, norm_weight=None, norm_eps=1e-6,
                    stream=None) -> None:
    """One decode step for [N,H,*] inputs; `state` [N,H,128,128] float32 is updated in place."""
    d = _decode_desc(q, k, v, g, beta, state, o, gate, norm_weight, norm_eps)
    _check("kda_decode_step", load().kda_decode_step(C.byref(d), _stream(stream)))


def kda_decode_step_pooled(q, k, v, g, beta, pool, slots, *, o, gate=None, norm_weight=None,
                           norm_eps=1e-6, stream=None) -> None:
    """One decode step for [N,H,*] inputs whose states are pool[slots[n]]: `pool`
    [P,H,128,128] float32 is updated in place; `slots` is an int32 device tensor [N]."""
    _expect("slots", slots, (int(q.shape[0]),), (torch.int32,), q.device)
    d = _decode_desc(q, k, v, g, beta, pool, o, gate, norm_weight, norm_eps, pooled=True)
    _check("kda_decode_step_pooled",
           load().kda_decode_step_pooled(C.byref(d), _slots(slots), int(pool.shape[0]),
                                         _stream(stream)))


class DecodeStep:
    """kda_decode_step (or, with `slots`, kda_decode_step_pooled) bound to fixed buffers,
    for loops that refill the same input buffers every step, as a serving loop does: the
    tensors are checked and the C descriptor is built once, and each call only launches.
    The object keeps the tensors alive; their contents may change between calls, their
    storage may not (no resize, no reassignment of the tensors' data).  Calling it runs
    the same kernel on the same arguments as the one-shot functions, with bit-identical
    results."""

    def __init__(self, q, k, v, g, beta, state, *, o, gate=None, norm_weight=None,
                 norm_eps=1e-6, slots=None):
        self._pooled = slots is not None
        if self._pooled:
            _expect("slots", slots, (int(q.shape[0]),), (torch.int32,), q.device)
        self._d = _decode_desc(q, k, v, g, beta, state, o, gate, norm_weight, norm_eps,
                               pooled=self._pooled)
        self._keep = (q, k, v, g, beta, state, o, gate, norm_weight, slots)
        self._ref = C.byref(self._d)
        self._lib = load()
        if self._pooled:
            self._slots, self._pool = _slots(slots), int(state.shape[0])

    def __call__(self, stream=None) -> None:
        s = _stream(stream)
        if self._pooled:
            st = self._lib.kda_decode_step_pooled(self._ref, self._slots, self._pool, s)
        else:
            st = self._lib.kda_decode_step(self._ref, s)
        _check("kda_decode_step_pooled" if self._pooled else "kda_decode_step", st)


def kda_state_copy_indexed(dst, src, *, dst_slots=None, src_slots=None, n=None,
                           stream=None) -> None:
    """dst[dst_slots[i]] = src[src_slots[i]] for i < n (slot i where a slot tensor is None).

    dst, src: float32 [count, ...] with equal trailing shapes (one state per leading
    index), on the device or in pinned host memory; slot tensors: int32 on the device."""
    if dst.dtype != torch.float32 or src.dtype != torch.float32:
        raise ValueError("states are float32")
    if dst.shape[1:] != src.shape[1:]:
        raise ValueError("dst and src states differ in shape")
    if n is None:
        n = (dst_slots if dst_slots is not None else src_slots if src_slots is not None else dst).shape[0]
    n = int(n)
    for name, sl in (("dst_slots", dst_slots), ("src_slots", src_slots)):
        if sl is None:
            continue
        if not isinstance(sl, torch.Tensor) or sl.dim() != 1 or sl.dtype != torch.int32:
            raise ValueError(f"{name} must be a 1-d int32 tensor")
        if sl.shape[0] < n:
            raise ValueError(f"{name} holds {sl.shape[0]} slots, fewer than n = {n}")
    elems = 1
    for x in dst.shape[1:]:
        elems *= int(x)
    _check("kda_state_copy_indexed",
           load().kda_state_copy_indexed(_ptr_any(dst), _slots(dst_slots), int(dst.shape[0]),
                                         _ptr_any(src), _slots(src_slots), int(src.shape[0]),
                                         int(n), elems, _stream(stream)))


def _n_states(t) -> int:
    return t.numel() // (t.shape[-1] * t.shape[-2]) if t.dim() >= 2 else 0


def kda_state_checkpoint(state, ckpt, *, stream=None) -> None:
    """ckpt[...] = state[...] (fp32 states of shape [..., d_k, d_v])."""
    if ckpt.shape != state.shape:
        raise ValueError("state and checkpoint shapes differ")
    if state.dtype != torch.float32 or ckpt.dtype != torch.float32:
        raise ValueError("states and checkpoints are float32")
    if state.dim() < 2:
        raise ValueError("states have shape [..., d_k, d_v]")
    _check("kda_state_checkpoint",
           load().kda_state_checkpoint(_ptr(state), _ptr(ckpt), _n_states(state), state.shape[-2],
                                       state.shape[-1], _stream(stream)))


def kda_state_rollback(state, ckpt, *, stream=None) -> None:
    """state[...] = ckpt[...] (fp32 states of shape [..., d_k, d_v])."""
    if ckpt.shape != state.shape:
        raise ValueError("state and checkpoint shapes differ")
    if state.dtype != torch.float32 or ckpt.dtype != torch.float32:
        raise ValueError("states and checkpoints are float32")
    if state.dim() < 2:
        raise ValueError("states have shape [..., d_k, d_v]")
    _check("kda_state_rollback",
           load().kda_state_rollback(_ptr(state), _ptr(ckpt), _n_states(state), state.shape[-2],
                                     state.shape[-1], _stream(stream)))


def _backward_desc(q, k, v, g, beta, dO, *, dq=None, dk=None, dv=None, dg=None, dbeta=None,
                   S0=None, dS_final=None, dS0=None, chunk=64, workspace=None) -> BackwardDesc:
    B, T, H, dk_ = q.shape
    d = BackwardDesc()
    d.B, d.T, d.H, d.d_k, d.d_v, d.chunk = B, T, H, dk_, v.shape[-1], chunk
    d.in_dtype = _dtype(q)
    d.q, d.k, d.v, d.g, d.beta = _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta)
    d.S0, d.dO, d.dS_final = _ptr(S0), _ptr(dO), _ptr(dS_final)
    d.dq, d.dk, d.dv, d.dg, d.dbeta, d.dS0 = (_ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg), _ptr(dbeta),
                                              _ptr(dS0))
    if workspace is not None:
        d.workspace, d.workspace_bytes = _ptr(workspace), workspace.numel() * workspace.element_size()
    return d


def kda_backward_workspace_size(q, k, v, g, beta, dO, chunk=64) -> int:
    """Workspace bytes kda_prefill_backward needs for these arguments."""
    d = _backward_desc(q, k, v, g, beta, dO, chunk=chunk)
    n = C.c_size_t(0)
    _check("kda_backward_workspace_size", load().kda_backward_workspace_size(C.byref(d), C.byref(n)))
    return int(n.value)


def kda_prefill_backward(q, k, v, g, beta, dO, *, dq, dk, dv, dg, dbeta, S0=None, dS_final=None,
                         dS0=None, chunk=64, workspace=None, stream=None) -> None:
    """Gradients of the chunkwise prefill into the caller's float32 tensors.

    q, k, v: [B,T,H,128] (float32 or bfloat16, as given to the prefill); g: [B,T,H,128] and
    beta: [B,T,H] float32; dO: [B,T,H,128] float32 gradient of the raw outputs; S0,
    dS_final, dS0: [B,H,128,128] float32 or None.  dq, dk, dv, dg: [B,T,H,128] float32;
    dbeta: [B,T,H] float32.  Without a workspace, one is allocated from torch's caching
    allocator."""
    if not isinstance(q, torch.Tensor) or q.dim() != 4 or not isinstance(v, torch.Tensor) or v.dim() != 4:
        raise ValueError("q and v must be 4-d tensors [B, T, H, d]")
    _expect("q", q, q.shape, _IN_DTYPES)
    B, T, H, dk_ = q.shape
    _expect("k", k, q.shape, (q.dtype,), q.device)
    _expect("v", v, (B, T, H, v.shape[-1]), (q.dtype,), q.device)
    _expect("g", g, q.shape, _F32, q.device)
    _expect("beta", beta, (B, T, H), _F32, q.device)
    for name, t, shape in (("dO", dO, (B, T, H, v.shape[-1])), ("dq", dq, q.shape), ("dk", dk, q.shape),
                           ("dv", dv, v.shape), ("dg", dg, g.shape), ("dbeta", dbeta, beta.shape),
                           ("S0", S0, (B, H, dk_, v.shape[-1])), ("dS_final", dS_final, (B, H, dk_, v.shape[-1])),
                           ("dS0", dS0, (B, H, dk_, v.shape[-1]))):
        if t is None:
            continue
        if t.dtype != torch.float32:
            raise ValueError(f"{name} must be float32")
        if tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if workspace is None:
        n = kda_backward_workspace_size(q, k, v, g, beta, dO, chunk=chunk)
        if n > 0:
            workspace = torch.empty(n, dtype=torch.uint8, device=q.device)
    d = _backward_desc(q, k, v, g, beta, dO, dq=dq, dk=dk, dv=dv, dg=dg, dbeta=dbeta, S0=S0,
                       dS_final=dS_final, dS0=dS0, chunk=chunk, workspace=workspace)
    _check("kda_prefill_backward", load().kda_prefill_backward(C.byref(d), _stream(stream)))
