"""CPU oracle for fused normalization + FP8 / NVFP4 quantization.

TEST INFRASTRUCTURE ONLY.  This package wraps ``liboracle.so`` (plain C,
``nq_oracle.c``) with numpy marshalling.  Only the test suite, the smoke check
and the CPU-baseline leg of the benchmark may import it; the GPU library
(``fp4_quantization_amd``) never does, and this package imports nothing from
it.  The arithmetic, the readings of the pages it follows and the citations
are in ``nq_oracle.c``.

All arrays are numpy arrays on the host.  bf16 tensors travel as ``uint16``
bit patterns; e4m3 and packed E2M1 codes as ``uint8``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
SRC_PATH = os.path.join(_HERE, "nq_oracle.c")

_c_u16p = ctypes.POINTER(ctypes.c_uint16)
_c_u8p = ctypes.POINTER(ctypes.c_uint8)
_c_f32p = ctypes.POINTER(ctypes.c_float)
_i64 = ctypes.c_int64


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc: IEEE binary32, no contraction, no fast-math."""
    if force or not os.path.exists(LIB_PATH):
        cmd = ["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math",
               "-fPIC", "-shared", "-Wall", "-Wextra", "-Werror",
               SRC_PATH, "-o", LIB_PATH + ".tmp", "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(LIB_PATH + ".tmp", LIB_PATH)
    return LIB_PATH


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        L = ctypes.CDLL(LIB_PATH)
        L.or_bf16_encode.restype = ctypes.c_uint16
        L.or_bf16_encode.argtypes = [ctypes.c_float]
        L.or_bf16_decode.restype = ctypes.c_float
        L.or_bf16_decode.argtypes = [ctypes.c_uint16]
        L.or_e4m3_encode.restype = ctypes.c_uint8
        L.or_e4m3_encode.argtypes = [ctypes.c_float]
        L.or_e4m3_decode.restype = ctypes.c_float
        L.or_e4m3_decode.argtypes = [ctypes.c_uint8]
        L.or_e2m1_encode.restype = ctypes.c_uint8
        L.or_e2m1_encode.argtypes = [ctypes.c_float]
        L.or_e2m1_decode.restype = ctypes.c_float
        L.or_e2m1_decode.argtypes = [ctypes.c_uint8]
        L.or_e5m2_encode.restype = ctypes.c_uint8
        L.or_e5m2_encode.argtypes = [ctypes.c_float]
        L.or_e5m2_decode.restype = ctypes.c_float
        L.or_e5m2_decode.argtypes = [ctypes.c_uint8]
        for name in ("or_bf16_encode_n", "or_e4m3_encode_n", "or_e4m3_decode_n", "or_e2m1_encode_n",
                     "or_e5m2_encode_n", "or_e5m2_decode_n"):
            getattr(L, name).restype = None
        L.or_name.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _p(a: np.ndarray | None, ctype):
    if a is None:
        return ctypes.cast(None, ctype)
    assert a.flags["C_CONTIGUOUS"] or a.ndim == 1
    return a.ctypes.data_as(ctype)


def _u16(a):
    a = np.ascontiguousarray(a)
    assert a.dtype == np.uint16, a.dtype
    return a


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


# ---------------------------------------------------------------- codecs ---

def bf16_encode(v) -> np.ndarray:
    v = _f32(v).ravel()
    out = np.empty(v.shape, np.uint16)
    lib().or_bf16_encode_n(_p(v, _c_f32p), _p(out, _c_u16p), _i64(v.size))
    return out


def bf16_decode(h) -> np.ndarray:
    h = np.ascontiguousarray(h, dtype=np.uint16)
    return (h.astype(np.uint32) << 16).view(np.float32)


def e4m3_encode(v) -> np.ndarray:
    v = _f32(v)
    flat = v.ravel()
    out = np.empty(flat.shape, np.uint8)
    lib().or_e4m3_encode_n(_p(flat, _c_f32p), _p(out, _c_u8p), _i64(flat.size))
    return out.reshape(v.shape)


def e4m3_decode(c) -> np.ndarray:
    c = np.ascontiguousarray(c, dtype=np.uint8)
    flat = c.ravel()
    out = np.empty(flat.shape, np.float32)
    lib().or_e4m3_decode_n(_p(flat, _c_u8p), _p(out, _c_f32p), _i64(flat.size))
    return out.reshape(c.shape)


def e5m2_encode(v) -> np.ndarray:
    v = _f32(v)
    flat = v.ravel()
    out = np.empty(flat.shape, np.uint8)
    lib().or_e5m2_encode_n(_p(flat, _c_f32p), _p(out, _c_u8p), _i64(flat.size))
    return out.reshape(v.shape)


def e5m2_decode(c) -> np.ndarray:
    c = np.ascontiguousarray(c, dtype=np.uint8)
    flat = c.ravel()
    out = np.empty(flat.shape, np.float32)
    lib().or_e5m2_decode_n(_p(flat, _c_u8p), _p(out, _c_f32p), _i64(flat.size))
    return out.reshape(c.shape)


FP8_FORMATS = {"e4m3": 0, "e5m2": 1}


def _fmt(fmt: str) -> ctypes.c_int32:
    return ctypes.c_int32(FP8_FORMATS[fmt])


def e2m1_encode(v) -> np.ndarray:
    v = _f32(v)
    flat = v.ravel()
    out = np.empty(flat.shape, np.uint8)
    lib().or_e2m1_encode_n(_p(flat, _c_f32p), _p(out, _c_u8p), _i64(flat.size))
    return out.reshape(v.shape)


def e2m1_decode(c) -> np.ndarray:
    c = np.asarray(c, dtype=np.uint8)
    return np.array([lib().or_e2m1_decode(int(v)) for v in c.ravel()], np.float32).reshape(c.shape)


def _rows(x: np.ndarray, d: int | None):
    """Return (M, d, ld) for a 2-D uint16 row-major buffer read as [M, d]."""
    assert x.ndim == 2
    M, ld = x.shape
    return M, (ld if d is None else d), ld


def _check(rc):
    if rc != 0:
        raise ValueError(f"oracle rejected the arguments (status {rc})")


# ------------------------------------------------------------------- ops ---

def fused_add_rmsnorm_quant_fp8(x, residual, gamma, eps, static_scale=None, d=None,
                                want_norm_out=False, want_y=False, fmt="e4m3"):
    """O2.  x, residual: uint16 [M, ld] (residual may be None); reads the
    first d columns; fmt "e4m3" or "e5m2".  Returns dict(q, scale,
    residual_out, norm_out, y)."""
    x = _u16(x)
    M, d, ld_x = _rows(x, d)
    r = None if residual is None else _u16(residual)
    ld_r = 0 if r is None else r.shape[1]
    r_out = None if r is None else np.empty((M, d), np.uint16)
    g = _f32(gamma)
    assert g.size >= d
    q = np.empty((M, d), np.uint8)
    scale = None if static_scale is not None else np.empty(M, np.float32)
    ss = None if static_scale is None else np.array([static_scale], np.float32)
    n_out = np.empty((M, d), np.uint16) if want_norm_out else None
    y = np.empty((M, d), np.float32) if want_y else None
    zb = np.empty(d, np.float32)
    yb = np.empty(d, np.float32)
    _check(lib().or_fused_add_rmsnorm_quant_fp8(
        _p(x, _c_u16p), _i64(ld_x), _p(r, _c_u16p), _i64(ld_r),
        _p(r_out, _c_u16p), _i64(d), _p(g, _c_f32p), ctypes.c_float(eps),
        _p(ss, _c_f32p), _p(q, _c_u8p), _i64(d), _p(scale, _c_f32p),
        _p(n_out, _c_u16p), _i64(d), _p(y, _c_f32p), _i64(d),
        _p(zb, _c_f32p), _p(yb, _c_f32p), _fmt(fmt), _i64(M), _i64(d)))
    return dict(q=q, scale=scale, residual_out=r_out, norm_out=n_out, y=y)


def quant_fp8_rows(y, static_scale=None, fmt="e4m3"):
    """The quantization step of O2 alone, on fp32 rows y [M, d]."""
    y = _f32(y)
    M, d = y.shape
    q = np.empty((M, d), np.uint8)
    scale = None if static_scale is not None else np.empty(M, np.float32)
    ss = None if static_scale is None else np.array([static_scale], np.float32)
    _check(lib().or_quant_fp8_rows(_p(y, _c_f32p), _i64(M), _i64(d), _p(ss, _c_f32p),
                                   _p(q, _c_u8p), _p(scale, _c_f32p), _fmt(fmt)))
    return dict(q=q, scale=scale)


def unfused_rmsnorm_quant_fp8(x, residual, gamma, eps, static_scale=None, d=None):
    """O6: the two-kernel pipeline (norm output rounded to bf16, then quantized)."""
    x = _u16(x)
    M, d, ld_x = _rows(x, d)
    r = None if residual is None else _u16(residual)
    ld_r = 0 if r is None else r.shape[1]
    g = _f32(gamma)
    q = np.empty((M, d), np.uint8)
    scale = None if static_scale is not None else np.empty(M, np.float32)
    ss = None if static_scale is None else np.array([static_scale], np.float32)
    zb = np.empty(d, np.float32)
    yb = np.empty(d, np.float32)
    _check(lib().or_unfused_rmsnorm_quant_fp8(
        _p(x, _c_u16p), _i64(ld_x), _p(r, _c_u16p), _i64(ld_r), _p(g, _c_f32p),
        ctypes.c_float(eps), _p(ss, _c_f32p), _p(q, _c_u8p), _i64(d),
        _p(scale, _c_f32p), _p(zb, _c_f32p), _p(yb, _c_f32p), _i64(M), _i64(d)))
    return dict(q=q, scale=scale)


def layernorm_quant_fp8(x, gamma, beta, eps, scale=None, d=None, want_y=False, fmt="e4m3"):
    """O3 (static: `scale` given) or O8 (dynamic per-token: scale None).
    Returns dict(q, scale (dynamic only), y)."""
    x = _u16(x)
    M, d, ld_x = _rows(x, d)
    g, b = _f32(gamma), _f32(beta)
    q = np.empty((M, d), np.uint8)
    y = np.empty((M, d), np.float32) if want_y else None
    ss = None if scale is None else np.array([scale], np.float32)
    so = np.empty(M, np.float32) if scale is None else None
    cb = np.empty(d, np.float32)
    yb = np.empty(d, np.float32)
    _check(lib().or_layernorm_quant_fp8(
        _p(x, _c_u16p), _i64(ld_x), _p(g, _c_f32p), _p(b, _c_f32p), ctypes.c_float(eps),
        _p(ss, _c_f32p), _p(q, _c_u8p), _i64(d), _p(so, _c_f32p), _p(y, _c_f32p), _i64(d),
        _p(cb, _c_f32p), _p(yb, _c_f32p), _fmt(fmt), _i64(M), _i64(d)))
    return dict(q=q, scale=so, y=y)


def per_token_group_quant_fp8(x, group=128, ue8m0=False, K=None, fmt="e4m3"):
    """O4.  Returns dict(q [M, K], scale [M, K/group])."""
    x = _u16(x)
    M, K, ld_x = _rows(x, K)
    q = np.empty((M, K), np.uint8)
    s = np.empty((M, K // group), np.float32)
    _check(lib().or_per_token_group_quant_fp8(
        _p(x, _c_u16p), _i64(ld_x), _i64(M), _i64(K), ctypes.c_int32(group),
        ctypes.c_int32(1 if ue8m0 else 0), _p(q, _c_u8p), _i64(K), _p(s, _c_f32p), _fmt(fmt)))
    return dict(q=q, scale=s)


def fused_add_rmsnorm_quant_fp8_group(x, residual, gamma, eps, group=128, ue8m0=False,
                                      bf16_source=False, d=None, want_norm_out=False, want_y=False,
                                      fmt="e4m3"):
    """O7.  Returns dict(q [M, d], scale [M, d/group], residual_out, norm_out, y)."""
    x = _u16(x)
    M, d, ld_x = _rows(x, d)
    r = None if residual is None else _u16(residual)
    ld_r = 0 if r is None else r.shape[1]
    r_out = None if r is None else np.empty((M, d), np.uint16)
    g = _f32(gamma)
    assert g.size >= d
    q = np.empty((M, d), np.uint8)
    s = np.empty((M, d // group), np.float32)
    n_out = np.empty((M, d), np.uint16) if want_norm_out else None
    y = np.empty((M, d), np.float32) if want_y else None
    zb = np.empty(d, np.float32)
    yb = np.empty(d, np.float32)
    _check(lib().or_fused_add_rmsnorm_quant_fp8_group(
        _p(x, _c_u16p), _i64(ld_x), _p(r, _c_u16p), _i64(ld_r), _p(r_out, _c_u16p), _i64(d),
        _p(g, _c_f32p), ctypes.c_float(eps), ctypes.c_int32(group), ctypes.c_int32(1 if ue8m0 else 0),
        ctypes.c_int32(1 if bf16_source else 0), _p(q, _c_u8p), _i64(d), _p(s, _c_f32p), _i64(d // group),
        _p(n_out, _c_u16p), _i64(d), _p(y, _c_f32p), _i64(d), _p(zb, _c_f32p), _p(yb, _c_f32p),
        _fmt(fmt), _i64(M), _i64(d)))
    return dict(q=q, scale=s, residual_out=r_out, norm_out=n_out, y=y)


def rmsnorm_quant_nvfp4(x, residual, gamma, eps, global_scale, d=None,
                        want_norm_out=False, want_y=False, mode_b=False):
    """O5.  Returns dict(q [M, d/2], sf [M, d/16], residual_out, norm_out, y)."""
    x = _u16(x)
    M, d, ld_x = _rows(x, d)
    r = None if residual is None else _u16(residual)
    ld_r = 0 if r is None else r.shape[1]
    r_out = None if r is None else np.empty((M, d), np.uint16)
    g = _f32(gamma)
    q = np.empty((M, d // 2), np.uint8)
    sf = np.empty((M, d // 16), np.uint8)
    n_out = np.empty((M, d), np.uint16) if want_norm_out else None
    y = np.empty((M, d), np.float32) if want_y else None
    gs = np.array([global_scale], np.float32)
    zb = np.empty(d, np.float32)
    yb = np.empty(d, np.float32)
    _check(lib().or_rmsnorm_quant_nvfp4(
        _p(x, _c_u16p), _i64(ld_x), _p(r, _c_u16p), _i64(ld_r), _p(r_out, _c_u16p), _i64(d),
        _p(g, _c_f32p), ctypes.c_float(eps), _p(gs, _c_f32p), _p(q, _c_u8p), _i64(d // 2),
        _p(sf, _c_u8p), _i64(d // 16), _p(n_out, _c_u16p), _i64(d), _p(y, _c_f32p), _i64(d),
        _p(zb, _c_f32p), _p(yb, _c_f32p), ctypes.c_int32(1 if mode_b else 0), _i64(M), _i64(d)))
    return dict(q=q, sf=sf, residual_out=r_out, norm_out=n_out, y=y)
