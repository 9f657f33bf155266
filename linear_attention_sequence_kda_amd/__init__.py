"""MI355X (gfx950) Kimi Delta Attention hot path.

The computation lives in libkda.so (HIP kernels behind the C ABI of include/kda.h);
this package is its thin Python binding.  Functions carry the names of the C entry
points.  There is no CPU or PyTorch fallback.
"""
from ._lib import (  # noqa: F401
    KdaError, KDA_OK, KDA_ERR_NULL, KDA_ERR_SHAPE, KDA_ERR_UNSUPPORTED, KDA_ERR_WORKSPACE,
    KDA_ERR_ALIAS, KDA_ERR_DEVICE, KDA_ERR_HIP, KDA_F32, KDA_BF16, LIB_PATH, load,
    status_string, kda_abi_version, kda_prefill_workspace_size, kda_prefill_chunked,
    kda_prefill_chunked_noalloc, NOALLOC_WORKSPACE_BYTES,
    kda_decode_step, kda_decode_step_pooled, DecodeStep, kda_state_copy_indexed, kda_state_checkpoint,
    kda_state_rollback, kda_backward_workspace_size, kda_prefill_backward, PrefillDesc,
    DecodeDesc, BackwardDesc,
)
