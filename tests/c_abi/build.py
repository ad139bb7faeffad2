"""Build the plain C++ client of libnq.so (tests/c_abi/nq_c_client.cpp).

It links the in-tree library with an rpath relative to the executable, so
the test runs it as built here, with no environment setup."""
from __future__ import annotations

import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "nq_c_client.cpp")
EXE = os.path.join(HERE, "nq_c_client")


def build() -> str:
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    cmd = [hipcc, "--offload-arch=gfx950", "-O2", "-std=c++17", "-Wall",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"), SRC,
           "-L", os.path.join(ROOT, "fp4_quantization_amd"), "-lnq",
           "-Wl,-rpath,$ORIGIN/../../fp4_quantization_amd", "-o", EXE + ".tmp"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"building the C client failed:\n{r.stdout}{r.stderr}")
    os.replace(EXE + ".tmp", EXE)
    return EXE


if __name__ == "__main__":
    print(build())
