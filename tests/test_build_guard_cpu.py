"""The build's guard against register spills (no GPU needed: hipcc cross-compiles for
gfx950 here).  Kernels that wait for their own asynchronous global->LDS copies with an
exact vector-memory count, and barriers that order LDS without waiting for vector
memory, are correct only if the compiler adds no memory operation of its own: a spill
to scratch would.  Every kernel source is compiled into a temporary directory and every
kernel must report zero scratch bytes."""
import concurrent.futures as cf
import os
import shutil

import pytest

from linear_attention_sequence_kda_amd import build as B

HIP_SOURCES = [s for s in B.SOURCES if s.endswith(".hip")]

pytestmark = pytest.mark.skipif(not (os.path.exists(B.HIPCC) or shutil.which("hipcc")),
                                reason="hipcc not installed")


def test_every_kernel_compiles_without_scratch(tmp_path):
    with cf.ThreadPoolExecutor(min(8, len(HIP_SOURCES))) as ex:
        list(ex.map(lambda s: B._compile(s, False, str(tmp_path)), HIP_SOURCES))


def test_resource_table_lists_the_exact_wait_kernels(tmp_path):
    import subprocess
    cmd = [B.HIPCC, *B.COMMON, B.RESOURCE_FLAG, "-c", os.path.join(B.CSRC, "prefill_state.hip"),
           "-o", str(tmp_path / "ps.o")]
    r = subprocess.run(cmd, capture_output=True, text=True, check=True)
    res = B.check_no_scratch("prefill_state.hip", r.stderr)
    names = " ".join(res)
    assert "chunk_state_kernel" in names and "map_chain" in names
    assert all(v["scratch"] == 0 and v["vgpr"] > 0 for v in res.values())


def test_guard_rejects_a_spilling_kernel():
    remarks = ("x.hip:1:1: remark: Function Name: k_spill [-Rpass-analysis=kernel-resource-usage]\n"
               "x.hip:1:1: remark:     VGPRs: 256 [-Rpass-analysis=kernel-resource-usage]\n"
               "x.hip:1:1: remark:     ScratchSize [bytes/lane]: 12 [-Rpass-analysis=kernel-resource-usage]\n")
    with pytest.raises(RuntimeError, match="k_spill"):
        B.check_no_scratch("x.hip", remarks)
    with pytest.raises(RuntimeError, match="no kernel resource usage"):
        B.check_no_scratch("x.hip", "")
