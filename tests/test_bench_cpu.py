"""Host-side pieces of bench.py (no GPU): the algorithmic byte and flop counts the
roofline objects divide by, the refusal of several GPUs, and the source hash that keys
the committed traffic summary to the kernels it was measured on.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_prefill_alg_bytes_per_token_head():
    # q, k, v, gate bf16 (4 x 256 B), g fp32 (512 B), beta (4 B), o fp32 (512 B)
    assert bench.prefill_alg_bytes(1, 1, 1) - 2 * 128 * 128 * 4 == 2052
    # the 8k workload: 2052 B per token-head plus S0 and S_final (64 KiB each per head)
    assert bench.prefill_alg_bytes(4, 8192, 16) == 4 * 8192 * 16 * 2052 + 2 * 4 * 16 * 65536
    # bf16 output storage: 256 B less per token-head
    assert bench.prefill_alg_bytes(1, 1, 1, out_bytes=2) - 2 * 128 * 128 * 4 == 2052 - 256


def test_table_bytes_match_the_workload_table():
    """The roofline's byte convention: bf16 activations and outputs, fp32 g, beta and states.
    8k prefill 1796 B per token-head + S0/S_T = 0.950 GB; 131k 1540 B + 128 B of 512-token
    checkpoints = 3.50 GB; 1M 1540 B = 12.9 GB."""
    c1 = bench.table_prefill_bytes(4, 8192, 16, gate=True)
    assert c1 == 4 * 8192 * 16 * 1796 + 2 * 4 * 16 * 65536 and round(c1 / 1e9, 3) == 0.950
    c3 = bench.table_prefill_bytes(1, 131072, 16, gate=False, ckpt_every=512, s0=False)
    assert c3 == 131072 * 16 * (1540 + 128) + 16 * 65536 and round(c3 / 1e9, 2) == 3.50
    c4 = bench.table_prefill_bytes(1, 1 << 20, 8, gate=False, s0=False)
    assert c4 == (1 << 20) * 8 * 1540 + 8 * 65536 and round(c4 / 1e10, 2) == 1.29


def test_decode_alg_bytes_per_state():
    # state read and written (2 x 64 KiB), q/k/v bf16, g fp32, beta, o fp32
    assert bench.decode_alg_bytes(1, 1) == 2 * 65536 + 3 * 256 + 512 + 4 + 512


def test_prefill_alg_flops_per_token_head():
    # 6 d^2 for the state products plus C (3 d_k + 2 d_v) inside the chunk, C = 64
    assert bench.prefill_alg_flops(1, 1, 1) == 6 * 128 * 128 + 64 * 5 * 128 == 139264


def test_backward_alg_flops_scale_with_chunks():
    one = bench.backward_alg_flops(1, 64, 1)
    assert one > 0
    assert bench.backward_alg_flops(1, 65, 1) == 2 * one        # a ragged chunk counts whole
    assert bench.backward_alg_flops(4, 8192, 16) == 4 * 128 * 16 * one


def test_source_hash_ignores_comments_but_not_code(tmp_path, monkeypatch):
    csrc = tmp_path / "linear_attention_sequence_kda_amd" / "csrc"
    csrc.mkdir(parents=True)
    f = csrc / "k.hip"
    f.write_text("int a = 1;  // one\n/* block\n comment */ int b = 2;\n", encoding="utf-8")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h0 = bench._src_hash("k.hip")
    f.write_text("int a = 1;  // first\n\n/* another\n comment */  int b = 2;\n", encoding="utf-8")
    assert bench._src_hash("k.hip") == h0
    f.write_text("int a = 1;  // one\n/* block\n comment */ int b = 3;\n", encoding="utf-8")
    assert bench._src_hash("k.hip") != h0


@pytest.mark.parametrize("n", ["2", "8"])
def test_several_gpus_are_refused(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", n],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)
