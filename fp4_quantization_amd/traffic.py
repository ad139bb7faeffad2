"""Algorithmic HBM byte model of each entry point.

The bytes a call must move at minimum: every input element read once, every
output element written once, per-row/per-group scales, and the small
row-invariant vectors (gamma, beta, scale scalars) counted once per call.  The
optional bf16 ``norm_out`` is never counted.  This is the model the pages use
when they quote bandwidth:
  * "per_token_group_quant_8bit: multiply by reciprocal ..." (Microbenchmarks):
    input + fp8 output + fp32 scales;
  * "feat: fused FP8 quantization output for LayerNorm" (Description):
    3 bytes per element fused (bf16 in, fp8 out) against 7 unfused;
  * "Fusing RMSNorm and FP8 Quantization Under torch.compile" (TL;DR): the
    fusion deletes the bf16 re-read, 2*d bytes per token.
"""
from __future__ import annotations


def fused_add_rmsnorm_fp8(M: int, d: int, residual: bool = True, static: bool = False):
    """(bytes read, bytes written) for nq_fused_add_rmsnorm_quant_fp8."""
    rd = M * (2 * d + (2 * d if residual else 0)) + 4 * d + (4 if static else 0)
    wr = M * ((2 * d if residual else 0) + d + (0 if static else 4))
    return rd, wr


def fused_add_rmsnorm_fp8_group(M: int, d: int, residual: bool = True, group: int = 128):
    """(bytes read, bytes written) for nq_fused_add_rmsnorm_quant_fp8_group:
    the per-token op's traffic with one fp32 scale per group instead of per row."""
    rd = M * (2 * d + (2 * d if residual else 0)) + 4 * d
    wr = M * ((2 * d if residual else 0) + d + 4 * (d // group))
    return rd, wr


def layernorm_fp8(M: int, d: int, dynamic: bool = False):
    """Static: the one-element scale is read once; dynamic: a scale per row
    is written instead."""
    rd = M * 2 * d + 8 * d + (0 if dynamic else 4)
    wr = M * (d + (4 if dynamic else 0))
    return rd, wr


def group_fp8(M: int, K: int, group: int = 128):
    rd = M * 2 * K
    wr = M * (K + 4 * (K // group))
    return rd, wr


def rmsnorm_nvfp4(M: int, d: int, residual: bool = True):
    rd = M * (2 * d + (2 * d if residual else 0)) + 4 * d + 4
    wr = M * ((2 * d if residual else 0) + d // 2 + d // 16)
    return rd, wr


def total(rw) -> int:
    return int(rw[0] + rw[1])


# The two-kernel pipelines the fused kernels replace, per row, for comparison
# with the pages' traffic statements (the norm kernel writes a bf16 output
# that the quantizer reads back).
def unfused_add_rmsnorm_fp8_per_row(d: int) -> int:
    norm_kernel = 2 * d + 2 * d + 2 * d + 2 * d   # read x, r; write residual, bf16 normed
    quant_kernel = 2 * d + d + 4                  # read bf16 normed; write fp8, scale
    return norm_kernel + quant_kernel


def fused_add_rmsnorm_fp8_with_norm_out_per_row(d: int) -> int:
    """The fused kernel as first shipped, which still writes the bf16 normed
    output as the hand-off anchor."""
    return 2 * d + 2 * d + 2 * d + 2 * d + d + 4


def unfused_layernorm_fp8_per_element() -> int:
    return 2 + 2 + 2 + 1  # read bf16, write bf16 normed, read it back, write fp8
