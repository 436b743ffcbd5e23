"""Builds libcsa_index.so (gfx950) in-tree with hipcc.

    python -m streaming_top_selection_csa_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libcsa_index.so")
OBJDIR = os.path.join(HERE, "_build")

# the scoring-kernel instantiations first: they take longest
SOURCES = ["csa_stream_bf16_d128.hip", "csa_stream_list.hip", "csa_stream_fp8_d128.hip",
           "csa_stream_bf16_d64.hip", "csa_stream_fp8_d64.hip", "csa_stream_bf16_d32.hip",
           "csa_kernels.hip", "csa_attn.hip", "csa_sort.hip", "csa_plan.cpp", "csa_abi.cpp",
           "csa_static.hip", "csa_group.hip", "csa_grouped.cpp"]

ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    # packed fp32 vector ops stay off (the host pass ignores this feature)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results in VGPRs: the epilogue reads every accumulator with the
    # VALU (at two waves per SIMD a wave's 256 registers are all VGPRs)
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-I", INCLUDE, "-I", CSRC,
]


def _compile(src: str) -> str:
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
    cmd = ["hipcc", *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed on {src}")
    return obj


def build() -> str:
    """Compile every source for gfx950 and link libcsa_index.so."""
    os.makedirs(OBJDIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = ["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc link failed")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
