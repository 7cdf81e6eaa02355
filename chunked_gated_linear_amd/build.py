"""Build liblinattn.so (HIP kernels for gfx950 + the C ABI) in-tree with hipcc.

    python -m chunked_gated_linear_amd.build

Objects go to _build/ at the repository root; the library lands next to this
file so the binding finds it without any install step.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "liblinattn.so")
SOURCES = ["chunk_fwd.hip", "chunk_pair.hip", "chunk_bwd.hip", "chunk_bwd_bf16.hip",
           "chunk_bwd_bf16_states.hip", "chunk_channel.hip",
           "chunk_channel_pair.hip",
           "decode.hip",
           "noalloc.hip", "lin_attn_abi.cpp"]
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def flags() -> list[str]:
    return [f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
            # packed fp32 VALU ops stay off (see the project notes on gfx950)
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            # keep MFMA accumulators in VGPRs: the state is rescaled by VALU
            # every tile, and AGPR accumulators would cost a move each way
            "-mllvm", "-amdgpu-mfma-vgpr-form",
            "-I", INCLUDE, "-I", CSRC]


# Per-file additions.  The reverse-pass gradient kernel is latency-bound at
# one workgroup per compute unit (its LDS); the scheduler that favours
# instruction-level parallelism over occupancy measured 2-3 % faster there
# and no better on the forward files.  It stops the compiler (a crash in
# register allocation) on the serial-chain kernel, which therefore sits in a
# file of its own, chunk_bwd_bf16_states.hip, with the default scheduler.
SRC_FLAGS = {
    "chunk_bwd_bf16.hip": ["-mllvm", "-amdgpu-sched-strategy=iterative-ilp"],
}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *flags(), *SRC_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
