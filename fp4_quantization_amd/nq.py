"""Thin Python binding of libnq.so (include/nq.h), same names as the C ABI.

Argument marshalling only: each function checks the PyTorch tensors' dtype,
device and layout, turns them into device pointers and leading dimensions,
and calls the C entry point on the given stream (default: PyTorch's current
stream).  Every step of the computation runs in the HIP kernels; there is no
CPU or PyTorch fallback, and importing this module fails if the library is
not built.

Tensor conventions: bf16 tensors are ``torch.bfloat16``; e4m3 codes are
``torch.float8_e4m3fn`` or ``torch.uint8``; packed E2M1 and block-scale codes
are ``torch.uint8``; scales are ``torch.float32``.  Matrices are 2-D with unit
column stride; their row stride becomes the leading dimension, so a column
slice such as ``buf[:, :1536]`` of a wider buffer is read in place.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libnq.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "nq.h")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run `python -m fp4_quantization_amd.build` "
                      "(there is no fallback implementation)")

_lib = ctypes.CDLL(LIB_PATH)

_vp, _i64, _i32, _u32, _f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_uint32, ctypes.c_float

_SIGS = {
    "nq_fused_add_rmsnorm_quant_fp8": [_vp, _i64, _vp, _i64, _vp, _i64, _vp, _f32, _vp, _vp, _i64,
                                       _vp, _vp, _i64, _i64, _i64, _vp],
    "nq_fused_add_rmsnorm_quant_fp8_group": [_vp, _i64, _vp, _i64, _vp, _i64, _vp, _f32, _i32, _i32, _u32,
                                             _vp, _i64, _vp, _i64, _vp, _i64, _i64, _i64, _vp],
    "nq_fused_add_rmsnorm_quant_fp8_ex": [_vp, _i64, _vp, _i64, _vp, _i64, _vp, _f32, _vp, _u32, _vp, _i64,
                                          _vp, _vp, _i64, _i64, _i64, _vp],
    "nq_layernorm_quant_fp8": [_vp, _i64, _vp, _vp, _f32, _vp, _vp, _i64, _i64, _i64, _vp],
    "nq_layernorm_quant_fp8_ex": [_vp, _i64, _vp, _vp, _f32, _vp, _u32, _vp, _i64, _vp, _i64, _i64, _vp],
    "nq_per_token_group_quant_fp8_ex": [_vp, _i64, _i64, _i64, _i32, _i32, _u32, _vp, _i64, _vp, _vp],
    "nq_per_token_group_quant_fp8": [_vp, _i64, _i64, _i64, _i32, _i32, _vp, _i64, _vp, _vp],
    "nq_rmsnorm_quant_nvfp4": [_vp, _i64, _vp, _i64, _vp, _i64, _vp, _f32, _vp, _vp, _i64, _vp, _i64,
                               _vp, _i64, _i64, _i64, _vp],
    "nq_rmsnorm_quant_nvfp4_ex": [_vp, _i64, _vp, _i64, _vp, _i64, _vp, _f32, _vp, _u32, _vp, _i64, _vp, _i64,
                                  _vp, _i64, _i64, _i64, _vp],
    "nq_fused_add_rmsnorm_bf16": [_vp, _i64, _vp, _i64, _vp, _i64, _vp, _f32, _vp, _i64, _i64, _i64, _vp],
    "nq_per_token_quant_fp8": [_vp, _i64, _vp, _u32, _vp, _i64, _vp, _i64, _i64, _vp],
    "nq_diag_codec": [_i32, _vp, _vp, _i64, _vp],
    "nq_diag_arith": [_i32, _vp, _vp, _vp, _i64, _vp],
    "nq_diag_copy": [_vp, _vp, _i64, _vp],
}
for _name, _args in _SIGS.items():
    _fn = getattr(_lib, _name)
    _fn.argtypes = _args
    _fn.restype = ctypes.c_int
_lib.nq_status_string.argtypes = [ctypes.c_int]
_lib.nq_status_string.restype = ctypes.c_char_p
_lib.nq_version.argtypes = []
_lib.nq_version.restype = ctypes.c_char_p


NQ_OK = 0
NQ_SCALE_FP32 = 0
NQ_SCALE_UE8M0 = 1
NQ_FLAG_BF16_SOURCE = 1
NQ_FLAG_E5M2 = 2
NQ_FLAG_GAMMA_BF16 = 4
NQ_CODEC_E4M3 = 0
NQ_CODEC_E2M1 = 1
NQ_CODEC_BF16 = 2
NQ_CODEC_E5M2 = 3
NQ_CODEC_E4M3_BOUNDED = 4
NQ_CODEC_E5M2_BOUNDED = 5
NQ_ARITH_RCP = 0
NQ_ARITH_RSQRT = 1
NQ_ARITH_DIV = 2
NQ_ARITH_DIV_LEN = 3
NQ_ARITH_DIV6 = 4
NQ_ARITH_SUM_BF16X2 = 5
NQ_ARITH_TOKEN_SCALE_E4M3 = 6
NQ_ARITH_TOKEN_SCALE_E5M2 = 7
NQ_MAX_D = 32768  # widest row of the row kernels (include/nq.h)


class NQError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: status {status} ({nq_status_string(status)})")
        self.status = status


def nq_status_string(status: int) -> str:
    return _lib.nq_status_string(int(status)).decode()


def nq_version() -> str:
    return _lib.nq_version().decode()


def library() -> ctypes.CDLL:
    """The loaded libnq.so (for callers that marshal raw pointers)."""
    return _lib


# ------------------------------------------------------------ marshalling --

_BF16 = (torch.bfloat16,)
_CODES8 = (torch.uint8, torch.float8_e4m3fn, torch.float8_e5m2)


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _mat(t: torch.Tensor | None, dtypes, name: str, cols: int | None = None):
    """(pointer, leading dimension) of a 2-D device matrix with unit column stride."""
    if t is None:
        return None, 0
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not in {dtypes}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dim() != 2 or (t.size(1) > 1 and t.stride(1) != 1):
        raise ValueError(f"{name} must be 2-D with unit column stride")
    if cols is not None and t.size(1) != cols:
        raise ValueError(f"{name}: expected {cols} columns, got {t.size(1)}")
    return t.data_ptr(), (t.stride(0) if t.size(0) > 1 else max(t.size(1), t.stride(0)))


def _vec(t: torch.Tensor | None, dtype, name: str, n: int | None = None):
    if t is None:
        return None
    if t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous device tensor")
    if n is not None and t.numel() < n:
        raise ValueError(f"{name}: needs {n} elements, has {t.numel()}")
    return t.data_ptr()


def _gvec(*ts, n: int, names=("gamma", "beta")):
    """Pointers of the per-row vectors (gamma, beta) and the flag bit for
    their dtype: all fp32, or all bf16 (NQ_FLAG_GAMMA_BF16)."""
    dt = ts[0].dtype
    if dt not in (torch.float32, torch.bfloat16):
        raise TypeError(f"{names[0]}: dtype {dt}, expected float32 or bfloat16")
    ptrs = tuple(_vec(t, dt, nm, n) for t, nm in zip(ts, names))
    return ptrs, (NQ_FLAG_GAMMA_BF16 if dt == torch.bfloat16 else 0)


def _same_rows(M: int, **tensors):
    """Every given matrix has the input's M rows."""
    for name, t in tensors.items():
        if t is not None and t.size(0) != M:
            raise ValueError(f"{name}: expected {M} rows")


def _check(status: int, where: str):
    if status != NQ_OK:
        raise NQError(status, where)


# ------------------------------------------------------------ entry points --

def nq_fused_add_rmsnorm_quant_fp8(x, residual_in, residual_out, gamma, eps, static_scale,
                                   q_out, scale_out, norm_out=None, stream=None):
    """Fused (residual-add +) RMSNorm + per-token FP8 e4m3 (include/nq.h)."""
    M, d = x.shape
    px, ldx = _mat(x, _BF16, "x")
    pr, ldr = _mat(residual_in, _BF16, "residual_in", d)
    pro, ldro = _mat(residual_out, _BF16, "residual_out", d)
    pq, ldq = _mat(q_out, _CODES8, "q_out", d)
    pn, ldn = _mat(norm_out, _BF16, "norm_out", d)
    for t, n in ((residual_in, "residual_in"), (residual_out, "residual_out"), (q_out, "q_out"),
                 (norm_out, "norm_out")):
        if t is not None and t.size(0) != M:
            raise ValueError(f"{n}: expected {M} rows")
    st = _lib.nq_fused_add_rmsnorm_quant_fp8(
        px, ldx, pr, ldr, pro, ldro, _vec(gamma, torch.float32, "gamma", d), float(eps),
        _vec(static_scale, torch.float32, "static_scale", 1), pq, ldq,
        _vec(scale_out, torch.float32, "scale_out", M if static_scale is None else None),
        pn, ldn, M, d, _stream(stream))
    _check(st, "nq_fused_add_rmsnorm_quant_fp8")


def nq_fused_add_rmsnorm_quant_fp8_group(x, residual_in, residual_out, gamma, eps, q_out, scale_out,
                                         group_size=128, scale_mode=NQ_SCALE_FP32, flags=0,
                                         norm_out=None, stream=None):
    """Fused (residual-add +) RMSNorm + per-token-group FP8 e4m3 (include/nq.h).
    scale_out is a 2-D fp32 matrix [M, d / group_size] (its row stride is
    passed through)."""
    M, d = x.shape
    px, ldx = _mat(x, _BF16, "x")
    pr, ldr = _mat(residual_in, _BF16, "residual_in", d)
    pro, ldro = _mat(residual_out, _BF16, "residual_out", d)
    pq, ldq = _mat(q_out, _CODES8, "q_out", d)
    ngroups = d // group_size if group_size > 0 else 0
    ps, lds = _mat(scale_out, (torch.float32,), "scale_out", ngroups)
    pn, ldn = _mat(norm_out, _BF16, "norm_out", d)
    for t, n in ((residual_in, "residual_in"), (residual_out, "residual_out"), (q_out, "q_out"),
                 (scale_out, "scale_out"), (norm_out, "norm_out")):
        if t is not None and t.size(0) != M:
            raise ValueError(f"{n}: expected {M} rows")
    (pg,), gf = _gvec(gamma, n=d)
    st = _lib.nq_fused_add_rmsnorm_quant_fp8_group(
        px, ldx, pr, ldr, pro, ldro, pg, float(eps),
        int(group_size), int(scale_mode), int(flags) | gf, pq, ldq, ps, lds, pn, ldn, M, d, _stream(stream))
    _check(st, "nq_fused_add_rmsnorm_quant_fp8_group")


def nq_fused_add_rmsnorm_quant_fp8_ex(x, residual_in, residual_out, gamma, eps, static_scale, flags,
                                      q_out, scale_out, norm_out=None, stream=None):
    """nq_fused_add_rmsnorm_quant_fp8 with an output-format flag (include/nq.h)."""
    M, d = x.shape
    px, ldx = _mat(x, _BF16, "x")
    pr, ldr = _mat(residual_in, _BF16, "residual_in", d)
    pro, ldro = _mat(residual_out, _BF16, "residual_out", d)
    pq, ldq = _mat(q_out, _CODES8, "q_out", d)
    pn, ldn = _mat(norm_out, _BF16, "norm_out", d)
    for t, n in ((residual_in, "residual_in"), (residual_out, "residual_out"), (q_out, "q_out"),
                 (norm_out, "norm_out")):
        if t is not None and t.size(0) != M:
            raise ValueError(f"{n}: expected {M} rows")
    (pg,), gf = _gvec(gamma, n=d)
    st = _lib.nq_fused_add_rmsnorm_quant_fp8_ex(
        px, ldx, pr, ldr, pro, ldro, pg, float(eps),
        _vec(static_scale, torch.float32, "static_scale", 1), int(flags) | gf, pq, ldq,
        _vec(scale_out, torch.float32, "scale_out", M if static_scale is None else None),
        pn, ldn, M, d, _stream(stream))
    _check(st, "nq_fused_add_rmsnorm_quant_fp8_ex")


def nq_layernorm_quant_fp8_ex(x, gamma, beta, eps, scale, flags, q_out, scale_out=None, stream=None):
    """LayerNorm + FP8, static (scale given) or dynamic per-token (scale None,
    scale_out [M] fp32), e4m3 or e5m2 (include/nq.h)."""
    M, d = x.shape
    px, ldx = _mat(x, _BF16, "x")
    pq, ldq = _mat(q_out, _CODES8, "q_out", d)
    if q_out.size(0) != M:
        raise ValueError(f"q_out: expected {M} rows")
    (pg, pb), gf = _gvec(gamma, beta, n=d)
    st = _lib.nq_layernorm_quant_fp8_ex(
        px, ldx, pg, pb, float(eps), _vec(scale, torch.float32, "scale", 1), int(flags) | gf, pq, ldq,
        _vec(scale_out, torch.float32, "scale_out", M if scale is None else None), M, d, _stream(stream))
    _check(st, "nq_layernorm_quant_fp8_ex")


def nq_layernorm_quant_fp8(x, gamma, beta, eps, scale, q_out, stream=None):
    """LayerNorm + static per-tensor FP8 e4m3 (include/nq.h)."""
    M, d = x.shape
    px, ldx = _mat(x, _BF16, "x")
    pq, ldq = _mat(q_out, _CODES8, "q_out", d)
    if q_out.size(0) != M:
        raise ValueError(f"q_out: expected {M} rows")
    st = _lib.nq_layernorm_quant_fp8(
        px, ldx, _vec(gamma, torch.float32, "gamma", d), _vec(beta, torch.float32, "beta", d),
        float(eps), _vec(scale, torch.float32, "scale", 1), pq, ldq, M, d, _stream(stream))
    _check(st, "nq_layernorm_quant_fp8")


def nq_per_token_group_quant_fp8(x, q_out, scale_out, group_size=128, scale_mode=NQ_SCALE_FP32,
                                 stream=None):
    """Per-token-group FP8 e4m3 with one reciprocal per group (include/nq.h)."""
    M, K = x.shape
    px, ldx = _mat(x, _BF16, "x")
    pq, ldq = _mat(q_out, _CODES8, "q_out", K)
    if q_out.size(0) != M:
        raise ValueError(f"q_out: expected {M} rows")
    ngroups = M * (K // group_size) if group_size > 0 else 0
    st = _lib.nq_per_token_group_quant_fp8(
        px, ldx, M, K, int(group_size), int(scale_mode), pq, ldq,
        _vec(scale_out, torch.float32, "scale_out", ngroups), _stream(stream))
    _check(st, "nq_per_token_group_quant_fp8")


def nq_per_token_group_quant_fp8_ex(x, q_out, scale_out, group_size=128, scale_mode=NQ_SCALE_FP32, flags=0,
                                    stream=None):
    """Per-token-group FP8 with an output-format flag (include/nq.h)."""
    M, K = x.shape
    px, ldx = _mat(x, _BF16, "x")
    pq, ldq = _mat(q_out, _CODES8, "q_out", K)
    if q_out.size(0) != M:
        raise ValueError(f"q_out: expected {M} rows")
    ngroups = M * (K // group_size) if group_size > 0 else 0
    st = _lib.nq_per_token_group_quant_fp8_ex(
        px, ldx, M, K, int(group_size), int(scale_mode), int(flags), pq, ldq,
        _vec(scale_out, torch.float32, "scale_out", ngroups), _stream(stream))
    _check(st, "nq_per_token_group_quant_fp8_ex")


def nq_rmsnorm_quant_nvfp4(x, residual_in, residual_out, gamma, eps, global_scale,
                           q_packed, block_scale, norm_out=None, stream=None):
    """(Residual-add +) RMSNorm + NVFP4 (include/nq.h)."""
    M, d = x.shape
    px, ldx = _mat(x, _BF16, "x")
    pr, ldr = _mat(residual_in, _BF16, "residual_in", d)
    pro, ldro = _mat(residual_out, _BF16, "residual_out", d)
    pq, ldq = _mat(q_packed, (torch.uint8,), "q_packed", d // 2)
    psf, ldsf = _mat(block_scale, _CODES8, "block_scale", d // 16)
    pn, ldn = _mat(norm_out, _BF16, "norm_out", d)
    _same_rows(M, residual_in=residual_in, residual_out=residual_out, q_packed=q_packed,
               block_scale=block_scale, norm_out=norm_out)
    st = _lib.nq_rmsnorm_quant_nvfp4(
        px, ldx, pr, ldr, pro, ldro, _vec(gamma, torch.float32, "gamma", d), float(eps),
        _vec(global_scale, torch.float32, "global_scale", 1), pq, ldq, psf, ldsf, pn, ldn,
        M, d, _stream(stream))
    _check(st, "nq_rmsnorm_quant_nvfp4")


def nq_rmsnorm_quant_nvfp4_ex(x, residual_in, residual_out, gamma, eps, global_scale, flags,
                              q_packed, block_scale, norm_out=None, stream=None):
    """(Residual-add +) RMSNorm + NVFP4 with an option flag (include/nq.h)."""
    M, d = x.shape
    px, ldx = _mat(x, _BF16, "x")
    pr, ldr = _mat(residual_in, _BF16, "residual_in", d)
    pro, ldro = _mat(residual_out, _BF16, "residual_out", d)
    pq, ldq = _mat(q_packed, (torch.uint8,), "q_packed", d // 2)
    psf, ldsf = _mat(block_scale, _CODES8, "block_scale", d // 16)
    pn, ldn = _mat(norm_out, _BF16, "norm_out", d)
    _same_rows(M, residual_in=residual_in, residual_out=residual_out, q_packed=q_packed,
               block_scale=block_scale, norm_out=norm_out)
    (pg,), gf = _gvec(gamma, n=d)
    st = _lib.nq_rmsnorm_quant_nvfp4_ex(
        px, ldx, pr, ldr, pro, ldro, pg, float(eps),
        _vec(global_scale, torch.float32, "global_scale", 1), int(flags) | gf, pq, ldq, psf, ldsf, pn, ldn,
        M, d, _stream(stream))
    _check(st, "nq_rmsnorm_quant_nvfp4_ex")


def nq_fused_add_rmsnorm_bf16(x, residual_in, residual_out, gamma, eps, out, stream=None):
    """(Residual-add +) RMSNorm with a bf16 output: the first kernel of the
    unfused pipeline (include/nq.h)."""
    M, d = x.shape
    px, ldx = _mat(x, _BF16, "x")
    pr, ldr = _mat(residual_in, _BF16, "residual_in", d)
    pro, ldro = _mat(residual_out, _BF16, "residual_out", d)
    po, ldo = _mat(out, _BF16, "out", d)
    for t, n in ((residual_in, "residual_in"), (residual_out, "residual_out"), (out, "out")):
        if t is not None and t.size(0) != M:
            raise ValueError(f"{n}: expected {M} rows")
    st = _lib.nq_fused_add_rmsnorm_bf16(px, ldx, pr, ldr, pro, ldro, _vec(gamma, torch.float32, "gamma", d),
                                        float(eps), po, ldo, M, d, _stream(stream))
    _check(st, "nq_fused_add_rmsnorm_bf16")


def nq_per_token_quant_fp8(x, static_scale, flags, q_out, scale_out, stream=None):
    """FP8 of bf16 rows with per-token (or static) scales: the second kernel
    of the unfused pipeline (include/nq.h)."""
    M, d = x.shape
    px, ldx = _mat(x, _BF16, "x")
    pq, ldq = _mat(q_out, _CODES8, "q_out", d)
    if q_out.size(0) != M:
        raise ValueError(f"q_out: expected {M} rows")
    st = _lib.nq_per_token_quant_fp8(
        px, ldx, _vec(static_scale, torch.float32, "static_scale", 1), int(flags), pq, ldq,
        _vec(scale_out, torch.float32, "scale_out", M if static_scale is None else None), M, d, _stream(stream))
    _check(st, "nq_per_token_quant_fp8")


def nq_diag_codec(kind: int, x: torch.Tensor, out: torch.Tensor, stream=None):
    """Apply the kernels' device conversion routine element-wise (include/nq.h)."""
    n = x.numel()
    px = _vec(x, torch.float32, "x", n)
    if kind == NQ_CODEC_BF16:
        if out.dtype not in (torch.int16, torch.bfloat16):
            raise TypeError(f"out: dtype {out.dtype}, expected int16 or bfloat16 bits")
        pout = _vec(out, out.dtype, "out", n)
    else:
        pout = _vec(out, torch.uint8, "out", n)
    st = _lib.nq_diag_codec(int(kind), px, pout, n, _stream(stream))
    _check(st, "nq_diag_codec")


_ARITH_TYPES = {  # kind -> (a dtype, b dtype or None, out dtype)
    NQ_ARITH_RCP: (torch.float32, None, torch.float32),
    NQ_ARITH_RSQRT: (torch.float32, None, torch.float32),
    NQ_ARITH_DIV: (torch.float32, torch.float32, torch.float32),
    NQ_ARITH_DIV_LEN: (torch.float64, torch.int32, torch.float64),
    NQ_ARITH_DIV6: (torch.float32, None, torch.float32),
    NQ_ARITH_SUM_BF16X2: (torch.int32, torch.float32, torch.float32),
    NQ_ARITH_TOKEN_SCALE_E4M3: (torch.float32, None, torch.float32),  # out: (scale, reciprocal) pairs
    NQ_ARITH_TOKEN_SCALE_E5M2: (torch.float32, None, torch.float32),
}
_ARITH_PAIR_OUT = (NQ_ARITH_TOKEN_SCALE_E4M3, NQ_ARITH_TOKEN_SCALE_E5M2)


def nq_diag_arith(kind: int, a: torch.Tensor, b, out: torch.Tensor, stream=None):
    """Apply one of the kernels' arithmetic shortcuts element-wise (include/nq.h)."""
    if kind not in _ARITH_TYPES:
        raise ValueError(f"nq_diag_arith: unknown kind {kind}")
    ta, tb, tout = _ARITH_TYPES[kind]
    n = a.numel()
    pa = _vec(a, ta, "a", n)
    pb = _vec(b, tb, "b", n) if tb is not None else None
    if tb is None and b is not None:
        raise ValueError("nq_diag_arith: this kind takes one operand")
    pout = _vec(out, tout, "out", 2 * n if kind in _ARITH_PAIR_OUT else n)
    st = _lib.nq_diag_arith(int(kind), pa, pb, pout, n, _stream(stream))
    _check(st, "nq_diag_arith")


def nq_diag_copy(src: torch.Tensor, dst: torch.Tensor, stream=None):
    """128-bit device copy of src's bytes into dst (include/nq.h)."""
    for t, name in ((src, "src"), (dst, "dst")):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous device tensor")
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < nbytes:
        raise ValueError("nq_diag_copy: destination too small")
    st = _lib.nq_diag_copy(src.data_ptr(), dst.data_ptr(), nbytes, _stream(stream))
    _check(st, "nq_diag_copy")
