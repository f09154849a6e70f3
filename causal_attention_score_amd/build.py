"""Build ``libcas.so`` (the C-ABI library of HIP kernels) for gfx950 with hipcc.

Each ``csrc/*.hip`` file is compiled to an object in ``_build/`` (in parallel)
and the objects are linked into ``causal_attention_score_amd/libcas.so``.
hipcc cross-compiles, so this runs on a machine without a GPU.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libcas.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -packed-fp32-ops off: hipcc would otherwise form v_pk_{add,mul,fma}_f32 from
# ordinary float code; the host pass warns that it does not know the feature.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-command-line-argument",
         "-I", os.path.join(ROOT, "include"), "-I", CSRC]


# Per-file extra flags. The softmax kernels keep their MFMA accumulators in
# ordinary VGPRs: the row-statistics kernel reads every accumulator with
# vector-ALU instructions, which would otherwise first copy each one out of
# the accumulation registers (64 extra VALU instructions per step).
EXTRA = {"softmax_f32.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
         "softmax_bf16.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
         "softmax_f16.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *EXTRA.get(os.path.basename(src), []), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    jobs = min(len(srcs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 4)), 16)
    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
