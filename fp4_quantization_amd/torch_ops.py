"""torch.library custom ops over libnq.so, for torch.compile and CUDA graphs.

Each op allocates its outputs and calls the C entry point through the
binding (``fp4_quantization_amd.nq``) on PyTorch's current stream; every step
of the computation runs in the HIP kernels.  Outputs are fresh tensors, never
views of or writes into the inputs, so the compiler sees no aliasing: the
residual sum comes back as a new tensor rather than updating the residual in
place ("RMSNorm nvfp4 quant fusion for DS V3.2 / Kimi-K2.5", commit notes: the
fused add op hands back x + residual in a newly allocated tensor, and its
fake implementation allocates with new_empty so the trace holds no
layout-copying node).  Each op has a fake implementation (shapes and dtypes only) so it
traces under FakeTensor / torch.compile without running.

FP8 codes are returned as ``torch.float8_e4m3fn`` or, with ``e5m2=True``,
``torch.float8_e5m2``; packed E2M1 pairs and e4m3 block-scale codes of NVFP4
as ``torch.uint8``; scales as ``torch.float32``.  Importing this module
registers the ops under the ``nq`` namespace (``torch.ops.nq.*``).
"""
from __future__ import annotations

import torch

from fp4_quantization_amd import nq

GROUP = 128
NVFP4_BLOCK = 16

_E4M3, _E5M2 = torch.float8_e4m3fn, torch.float8_e5m2


def _fp8(e5m2: bool) -> torch.dtype:
    return _E5M2 if e5m2 else _E4M3


def _flags(e5m2: bool) -> int:
    return nq.NQ_FLAG_E5M2 if e5m2 else 0


def _codes(x: torch.Tensor, cols: int, e5m2: bool) -> torch.Tensor:
    return x.new_empty((x.shape[0], cols), dtype=_fp8(e5m2))


def _f32(x: torch.Tensor, *shape) -> torch.Tensor:
    return x.new_empty(shape, dtype=torch.float32)


def _bf16_like(x: torch.Tensor) -> torch.Tensor:
    return x.new_empty((x.shape[0], x.shape[1]), dtype=torch.bfloat16)


# ---------------------------------------------- RMSNorm + per-token FP8 ----

@torch.library.custom_op("nq::add_rmsnorm_fp8", mutates_args=())
def add_rmsnorm_fp8(x: torch.Tensor, residual: torch.Tensor, gamma: torch.Tensor, eps: float,
                    e5m2: bool = False) -> tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """z = bf16(x + residual) (returned fresh), y = RMSNorm(z) * gamma,
    per-token dynamic FP8 of y: (codes [M, d], scales [M], z [M, d])."""
    q, s, ro = _codes(x, x.shape[1], e5m2), _f32(x, x.shape[0]), _bf16_like(x)
    nq.nq_fused_add_rmsnorm_quant_fp8_ex(x, residual, ro, gamma, eps, None, _flags(e5m2), q, s)
    return q, s, ro


@add_rmsnorm_fp8.register_fake
def _(x, residual, gamma, eps, e5m2=False):
    return _codes(x, x.shape[1], e5m2), _f32(x, x.shape[0]), _bf16_like(x)


@torch.library.custom_op("nq::rmsnorm_fp8", mutates_args=())
def rmsnorm_fp8(x: torch.Tensor, gamma: torch.Tensor, eps: float,
                e5m2: bool = False) -> tuple[torch.Tensor, torch.Tensor]:
    """Residual-less RMSNorm + per-token dynamic FP8: (codes, scales)."""
    q, s = _codes(x, x.shape[1], e5m2), _f32(x, x.shape[0])
    nq.nq_fused_add_rmsnorm_quant_fp8_ex(x, None, None, gamma, eps, None, _flags(e5m2), q, s)
    return q, s


@rmsnorm_fp8.register_fake
def _(x, gamma, eps, e5m2=False):
    return _codes(x, x.shape[1], e5m2), _f32(x, x.shape[0])


@torch.library.custom_op("nq::add_rmsnorm_fp8_static", mutates_args=())
def add_rmsnorm_fp8_static(x: torch.Tensor, residual: torch.Tensor, gamma: torch.Tensor, eps: float,
                           scale: torch.Tensor, e5m2: bool = False) -> tuple[torch.Tensor, torch.Tensor]:
    """Static-scale form: codes = fp8(y * (1 / scale[0])), the one-element
    scale read on the device; (codes, z)."""
    q, ro = _codes(x, x.shape[1], e5m2), _bf16_like(x)
    nq.nq_fused_add_rmsnorm_quant_fp8_ex(x, residual, ro, gamma, eps, scale, _flags(e5m2), q, None)
    return q, ro


@add_rmsnorm_fp8_static.register_fake
def _(x, residual, gamma, eps, scale, e5m2=False):
    return _codes(x, x.shape[1], e5m2), _bf16_like(x)


@torch.library.custom_op("nq::rmsnorm_fp8_static", mutates_args=())
def rmsnorm_fp8_static(x: torch.Tensor, gamma: torch.Tensor, eps: float, scale: torch.Tensor,
                       e5m2: bool = False) -> torch.Tensor:
    q = _codes(x, x.shape[1], e5m2)
    nq.nq_fused_add_rmsnorm_quant_fp8_ex(x, None, None, gamma, eps, scale, _flags(e5m2), q, None)
    return q


@rmsnorm_fp8_static.register_fake
def _(x, gamma, eps, scale, e5m2=False):
    return _codes(x, x.shape[1], e5m2)


# --------------------------------------- RMSNorm + per-token-group FP8 ------

def _group_flags(bf16_source: bool, e5m2: bool) -> int:
    return (nq.NQ_FLAG_BF16_SOURCE if bf16_source else 0) | _flags(e5m2)


@torch.library.custom_op("nq::add_rmsnorm_fp8_group", mutates_args=())
def add_rmsnorm_fp8_group(x: torch.Tensor, residual: torch.Tensor, gamma: torch.Tensor, eps: float,
                          ue8m0: bool = False, bf16_source: bool = False,
                          e5m2: bool = False) -> tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """RMSNorm fused with per-token-group (128) FP8: (codes, scales [M, d/128], z)."""
    M, d = x.shape
    q, s, ro = _codes(x, d, e5m2), _f32(x, M, d // GROUP), _bf16_like(x)
    nq.nq_fused_add_rmsnorm_quant_fp8_group(x, residual, ro, gamma, eps, q, s, GROUP,
                                            nq.NQ_SCALE_UE8M0 if ue8m0 else nq.NQ_SCALE_FP32,
                                            _group_flags(bf16_source, e5m2))
    return q, s, ro


@add_rmsnorm_fp8_group.register_fake
def _(x, residual, gamma, eps, ue8m0=False, bf16_source=False, e5m2=False):
    M, d = x.shape
    return _codes(x, d, e5m2), _f32(x, M, d // GROUP), _bf16_like(x)


@torch.library.custom_op("nq::rmsnorm_fp8_group", mutates_args=())
def rmsnorm_fp8_group(x: torch.Tensor, gamma: torch.Tensor, eps: float, ue8m0: bool = False,
                      bf16_source: bool = False, e5m2: bool = False) -> tuple[torch.Tensor, torch.Tensor]:
    M, d = x.shape
    q, s = _codes(x, d, e5m2), _f32(x, M, d // GROUP)
    nq.nq_fused_add_rmsnorm_quant_fp8_group(x, None, None, gamma, eps, q, s, GROUP,
                                            nq.NQ_SCALE_UE8M0 if ue8m0 else nq.NQ_SCALE_FP32,
                                            _group_flags(bf16_source, e5m2))
    return q, s


@rmsnorm_fp8_group.register_fake
def _(x, gamma, eps, ue8m0=False, bf16_source=False, e5m2=False):
    M, d = x.shape
    return _codes(x, d, e5m2), _f32(x, M, d // GROUP)


# ------------------------------------------------- standalone group FP8 -----

@torch.library.custom_op("nq::group_quant_fp8", mutates_args=())
def group_quant_fp8(x: torch.Tensor, ue8m0: bool = False, e5m2: bool = False) -> tuple[torch.Tensor, torch.Tensor]:
    """Per-token-group (128) FP8 of bf16 rows: (codes [M, K], scales [M, K/128])."""
    M, K = x.shape
    q, s = _codes(x, K, e5m2), _f32(x, M, K // GROUP)
    nq.nq_per_token_group_quant_fp8_ex(x, q, s.view(-1), GROUP, nq.NQ_SCALE_UE8M0 if ue8m0 else nq.NQ_SCALE_FP32,
                                       _flags(e5m2))
    return q, s


@group_quant_fp8.register_fake
def _(x, ue8m0=False, e5m2=False):
    M, K = x.shape
    return _codes(x, K, e5m2), _f32(x, M, K // GROUP)


# --------------------------------------------------------- LayerNorm FP8 ----

@torch.library.custom_op("nq::layernorm_fp8_static", mutates_args=())
def layernorm_fp8_static(x: torch.Tensor, gamma: torch.Tensor, beta: torch.Tensor, eps: float,
                         scale: torch.Tensor, e5m2: bool = False) -> torch.Tensor:
    """LayerNorm + static FP8 (out = y / scale[0], scale read on the device)."""
    q = _codes(x, x.shape[1], e5m2)
    nq.nq_layernorm_quant_fp8_ex(x, gamma, beta, eps, scale, _flags(e5m2), q, None)
    return q


@layernorm_fp8_static.register_fake
def _(x, gamma, beta, eps, scale, e5m2=False):
    return _codes(x, x.shape[1], e5m2)


@torch.library.custom_op("nq::layernorm_fp8", mutates_args=())
def layernorm_fp8(x: torch.Tensor, gamma: torch.Tensor, beta: torch.Tensor, eps: float,
                  e5m2: bool = False) -> tuple[torch.Tensor, torch.Tensor]:
    """LayerNorm + dynamic per-token FP8: (codes, scales [M])."""
    q, s = _codes(x, x.shape[1], e5m2), _f32(x, x.shape[0])
    nq.nq_layernorm_quant_fp8_ex(x, gamma, beta, eps, None, _flags(e5m2), q, s)
    return q, s


@layernorm_fp8.register_fake
def _(x, gamma, beta, eps, e5m2=False):
    return _codes(x, x.shape[1], e5m2), _f32(x, x.shape[0])


# ------------------------------------------------------- RMSNorm + NVFP4 ----

def _fp4_outputs(x: torch.Tensor):
    M, d = x.shape
    return (x.new_empty((M, d // 2), dtype=torch.uint8), x.new_empty((M, d // NVFP4_BLOCK), dtype=torch.uint8))


@torch.library.custom_op("nq::add_rmsnorm_nvfp4", mutates_args=())
def add_rmsnorm_nvfp4(x: torch.Tensor, residual: torch.Tensor, gamma: torch.Tensor, eps: float,
                      global_scale: torch.Tensor,
                      bf16_source: bool = False) -> tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """(packed E2M1 [M, d/2], e4m3 block scales [M, d/16], z)."""
    q, sf = _fp4_outputs(x)
    ro = _bf16_like(x)
    nq.nq_rmsnorm_quant_nvfp4_ex(x, residual, ro, gamma, eps, global_scale,
                                 nq.NQ_FLAG_BF16_SOURCE if bf16_source else 0, q, sf)
    return q, sf, ro


@add_rmsnorm_nvfp4.register_fake
def _(x, residual, gamma, eps, global_scale, bf16_source=False):
    q, sf = _fp4_outputs(x)
    return q, sf, _bf16_like(x)


@torch.library.custom_op("nq::rmsnorm_nvfp4", mutates_args=())
def rmsnorm_nvfp4(x: torch.Tensor, gamma: torch.Tensor, eps: float, global_scale: torch.Tensor,
                  bf16_source: bool = False) -> tuple[torch.Tensor, torch.Tensor]:
    """Residual-less form; x may be a row-strided column slice (read in place)."""
    q, sf = _fp4_outputs(x)
    nq.nq_rmsnorm_quant_nvfp4_ex(x, None, None, gamma, eps, global_scale,
                                 nq.NQ_FLAG_BF16_SOURCE if bf16_source else 0, q, sf)
    return q, sf


@rmsnorm_nvfp4.register_fake
def _(x, gamma, eps, global_scale, bf16_source=False):
    return _fp4_outputs(x)


# ------------------------------------------------- the unfused pipeline -----

@torch.library.custom_op("nq::add_rmsnorm_bf16", mutates_args=())
def add_rmsnorm_bf16(x: torch.Tensor, residual: torch.Tensor, gamma: torch.Tensor,
                     eps: float) -> tuple[torch.Tensor, torch.Tensor]:
    """(bf16(y), z): the norm half of the unfused pipeline."""
    out, ro = _bf16_like(x), _bf16_like(x)
    nq.nq_fused_add_rmsnorm_bf16(x, residual, ro, gamma, eps, out)
    return out, ro


@add_rmsnorm_bf16.register_fake
def _(x, residual, gamma, eps):
    return _bf16_like(x), _bf16_like(x)


@torch.library.custom_op("nq::per_token_quant_fp8", mutates_args=())
def per_token_quant_fp8(x: torch.Tensor, e5m2: bool = False) -> tuple[torch.Tensor, torch.Tensor]:
    """Per-token dynamic FP8 of bf16 rows: (codes, scales [M])."""
    q, s = _codes(x, x.shape[1], e5m2), _f32(x, x.shape[0])
    nq.nq_per_token_quant_fp8(x, None, _flags(e5m2), q, s)
    return q, s


@per_token_quant_fp8.register_fake
def _(x, e5m2=False):
    return _codes(x, x.shape[1], e5m2), _f32(x, x.shape[0])


OPS = ("add_rmsnorm_fp8", "rmsnorm_fp8", "add_rmsnorm_fp8_static", "rmsnorm_fp8_static",
       "add_rmsnorm_fp8_group", "rmsnorm_fp8_group", "group_quant_fp8", "layernorm_fp8_static",
       "layernorm_fp8", "add_rmsnorm_nvfp4", "rmsnorm_nvfp4", "add_rmsnorm_bf16", "per_token_quant_fp8")
