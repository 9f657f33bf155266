"""Build libkda.so (the HIP library behind include/kda.h) for gfx950 with hipcc.

    python -m linear_attention_sequence_kda_amd.build [-v] [-j N]

Compiles every source under csrc/ into _build/ and links the shared library next to
this file.  Always rebuilds (the sources are small); objects are compiled in parallel.

Every compile also asks the compiler for each kernel's resource usage, and the build
fails if any kernel needs scratch memory (register spills).  Several kernels wait for
their own global->LDS copies and loads with exact vector-memory counts, and order LDS
with barriers that do not wait for vector memory: both assume that the compiler adds no
memory operation of its own, which a spill to scratch would.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import re
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libkda.so")

SOURCES = ["api.cpp", "decode.hip", "state_copy.hip", "prefill_prep.hip", "prefill_state.hip",
           "backward.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # Packed fp32 instructions are kept out of generated code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC, "-fvisibility=hidden", "-Wall", "-Wno-unused-function",
]


RESOURCE_FLAG = "-Rpass-analysis=kernel-resource-usage"


def kernel_resources(remarks: str) -> dict:
    """{kernel symbol: {"vgpr": n, "agpr": n, "scratch": bytes per lane, "lds": bytes}} parsed
    from the compiler's kernel-resource-usage remarks."""
    out, cur = {}, None
    keys = {"VGPRs": "vgpr", "AGPRs": "agpr", "ScratchSize [bytes/lane]": "scratch",
            "LDS Size [bytes/block]": "lds"}
    for line in remarks.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            cur = out.setdefault(m.group(1), {})
            continue
        m = re.search(r"remark:\s+(VGPRs|AGPRs|ScratchSize \[bytes/lane\]|LDS Size \[bytes/block\]): (\d+)", line)
        if m and cur is not None:
            cur[keys[m.group(1)]] = int(m.group(2))
    return out


def check_no_scratch(src: str, remarks: str) -> dict:
    """Raise if a kernel of `src` spills to scratch; return its resource table."""
    res = kernel_resources(remarks)
    if src.endswith(".hip") and not res:
        raise RuntimeError(f"{src}: the compiler reported no kernel resource usage")
    spill = {k: v["scratch"] for k, v in res.items() if v.get("scratch", 0) > 0}
    if spill:
        raise RuntimeError(f"{src}: kernels use scratch memory (register spills), which breaks "
                           f"their exact memory wait counts: {spill}")
    return res


def _compile(src: str, verbose: bool, out_dir: str = BUILD) -> str:
    obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *COMMON, RESOURCE_FLAG, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    check_no_scratch(src, r.stderr)
    if verbose:
        warn = [l for l in r.stderr.splitlines() if RESOURCE_FLAG not in l]
        if warn:
            print("\n".join(warn), file=sys.stderr)
    return obj


def build(verbose: bool = False, jobs: int = 0) -> str:
    if not os.path.exists(HIPCC) and shutil.which("hipcc") is None:
        raise RuntimeError("hipcc not found; install ROCm or set HIPCC")
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 1, 8)
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("-v", "--verbose", action="store_true")
    ap.add_argument("-j", "--jobs", type=int, default=0)
    a = ap.parse_args()
    print(build(a.verbose, a.jobs))


if __name__ == "__main__":
    main()
