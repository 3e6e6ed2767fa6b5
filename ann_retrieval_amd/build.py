"""Compiles the HIP sources of the library into ``ann_retrieval_amd/libice.so``.

Run as ``python -m ann_retrieval_amd.build`` (or through
``__graft_entry__.build()``). Every source is compiled for gfx950 only; object
files go to ``ann_retrieval_amd/_build/``.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT_DIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libice.so")
SOURCES = ["ice_api.hip", "k_build.hip", "k_gemm.hip", "k_pdci.hip", "k_insert.hip", "k_select.hip", "k_attend.hip"]
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    # no packed fp32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
]


# per-source additions: the parent GEMM keeps its MFMA accumulators in
# ordinary VGPRs, so its argmax reads them without accumulator-register copies
EXTRA = {"k_gemm.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src: str) -> str:
    obj = os.path.join(OUT_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    noise = "'-packed-fp32-ops' is not a recognized feature"
    err = "\n".join(line for line in r.stderr.splitlines() if noise not in line)
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build(jobs: int = 6) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    # -z defs: a symbol no object defines fails the link instead of the load
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Wl,-z,defs", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
