"""Helpers for GPU tests: upload of stored input bytes and the error metrics.

err_o = max |o_gpu - o_ref| / rms(o_ref)   (whole tensor)
err_S = ||S_gpu - S_ref||_F / ||S_ref||_F
"""
import numpy as np
import torch

from kda_inputs import BF16, F32


def dev():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a HIP device")
    return torch.device("cuda:0")


def up(a, dtype=None):
    """numpy -> device tensor holding the same bytes (uint16 arrays become bfloat16)."""
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(a)
    return t.to(dev())


def down(t):
    """device tensor -> float64 numpy (exact widening)."""
    return t.detach().to(torch.float64).cpu().numpy()


def err_o(o, ref):
    ref = np.asarray(ref, np.float64)
    rms = float(np.sqrt(np.mean(ref * ref)))
    return float(np.max(np.abs(np.asarray(o, np.float64) - ref))) / rms


def err_S(S, ref):
    ref = np.asarray(ref, np.float64)
    return float(np.linalg.norm(np.asarray(S, np.float64) - ref) / np.linalg.norm(ref))


def bf16_out_tol(ref, base):
    """Tolerance for bf16-stored outputs: the storage rounding alone is up to 2^-8 of the
    largest magnitude, on top of the arithmetic tolerance `base`."""
    ref = np.asarray(ref, np.float64)
    rms = float(np.sqrt(np.mean(ref * ref)))
    return base + 2.0 ** -8 * float(np.max(np.abs(ref))) / rms
