"""Build libnq.so (the gfx950 HIP kernels behind include/nq.h) in-tree.

    python -m fp4_quantization_amd.build

Every source is compiled for gfx950 only, with floating-point contraction off
(every expression is the rounded operation sequence it spells out),
correctly rounded binary32 division and square root, denormals preserved,
and packed-fp32 instruction selection disabled.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD_DIR = os.path.join(HERE, "_build")
LIB_PATH = os.path.join(HERE, "libnq.so")

SOURCES = [
    "nq_rmsnorm_fp8.hip",
    "nq_rmsnorm_fp8_group.hip",
    "nq_layernorm_fp8.hip",
    "nq_rmsnorm_nvfp4.hip",
    "nq_group_fp8.hip",
    "nq_unfused.hip",
    "nq_misc.hip",
]

ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; the library needs ROCm's HIP compiler")
    return path


def _compile(src: str, extra: list[str]) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so
    noise = "'-packed-fp32-ops' is not a recognized feature"
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msg}")
    if msg.strip():
        print(msg, file=sys.stderr)
    return obj


def build(extra_flags: list[str] | None = None, jobs: int | None = None) -> str:
    """Compile every source and link libnq.so; returns the library path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    extra = list(extra_flags or [])
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 4, 16)
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra), SOURCES))
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    subprocess.run(cmd, check=True, capture_output=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build())
