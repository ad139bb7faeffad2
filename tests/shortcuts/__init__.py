"""Host checks of the kernels' arithmetic shortcuts (test infrastructure)."""
import ctypes
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "shortcut_proofs.c")
LIB = os.path.join(HERE, "libshortcut_proofs.so")


def build() -> str:
    cmd = ["gcc", "-std=gnu11", "-O2", "-march=native", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
           "-fPIC", "-shared", "-Wall", "-Werror", SRC, "-o", LIB + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


def lib() -> ctypes.CDLL:
    L = ctypes.CDLL(build())
    L.sp_div_len_check.restype = ctypes.c_int64
    L.sp_div_len_check.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_uint64,
                                   ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int32)]
    L.sp_div6_check.restype = ctypes.c_int64
    L.sp_div6_check.argtypes = [ctypes.c_uint32, ctypes.c_uint32, ctypes.POINTER(ctypes.c_uint32),
                                ctypes.POINTER(ctypes.c_uint32)]
    return L
