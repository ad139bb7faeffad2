"""Seeded synthetic inputs for the five workloads, shared by tests and bench.

This module holds input generation only -- none of the method's arithmetic --
so that both the GPU path and the CPU oracle can be fed identical bits
without either importing the other.  Everything is drawn on the host with
``numpy.random.default_rng(seed)`` in fp32 and rounded to bf16 with PyTorch's
round-to-nearest-even cast.  Every array is a numpy array; bf16 tensors are
``uint16`` bit patterns.

Workloads (shapes and distributions follow the pages' serving settings):
  rms_small   M=64, d=256: x, residual ~ N(0,1) with 2 outlier channels x20
              (per-token dynamic FP8 after residual-add + RMSNorm)
  rms_2816    d=2816 (a 5.6 KB bf16 row), M in {1, 16, 256, 8192}: x, residual
              ~ N(0,1) with 1% (28) outlier channels x50
  group       K=4096, M in {1, 32768}: heavy-tailed activations, standard
              Student-t with 3 degrees of freedom; group size 128
  layernorm   M=16384, d=4096: x ~ N(0.5, 1); beta ~ 0.1 N(0,1); eps 1e-5;
              static scale 0.05
  nvfp4_7168  residual-add + RMSNorm at d=7168, M in {1, 64, 8192}
  nvfp4_slice residual-less RMSNorm on columns 0..1535 of rows of stride 2112,
              M in {1, 64, 8192}
gamma is 1 + 0.1 N(0,1) in fp32 everywhere.  Outlier channels are drawn with
``rng.choice(d, n, replace=False)`` and scale both x and the residual (they
are a property of the residual-stream channel).
"""
from __future__ import annotations

import numpy as np
import torch


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 (round-to-nearest-even, PyTorch cast) as uint16 bits."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(h, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _gamma(rng, d):
    return (1.0 + 0.1 * rng.standard_normal(d)).astype(np.float32)


def rms_rows(M: int, d: int, n_outlier: int, outlier_mult: float, seed: int = 0,
             residual: bool = True, ld: int | None = None):
    """x, residual ~ N(0,1) bf16 [M, ld] (the first d columns are the row),
    `n_outlier` channels multiplied by `outlier_mult`; gamma fp32 [d]."""
    rng = np.random.default_rng(seed)
    ld = d if ld is None else ld
    x = rng.standard_normal((M, ld), dtype=np.float32)
    r = rng.standard_normal((M, ld), dtype=np.float32) if residual else None
    gamma = _gamma(rng, d)
    if n_outlier:
        ch = rng.choice(d, n_outlier, replace=False)
        x[:, ch] *= outlier_mult
        if r is not None:
            r[:, ch] *= outlier_mult
    return dict(x=to_bf16_bits(x), residual=None if r is None else to_bf16_bits(r),
                gamma=gamma, eps=1e-6, M=M, d=d, ld=ld)


def rms_small(seed: int = 0, M: int = 64):
    """M=64 tokens, d=256, 2 outlier channels x20, eps 1e-6."""
    return rms_rows(M, 256, 2, 20.0, seed)


def rms_2816(M: int, seed: int = 0):
    """d=2816, 1% = 28 outlier channels x50, eps 1e-6."""
    return rms_rows(M, 2816, 28, 50.0, seed)


def rms_group_7168(M: int, seed: int = 0):
    """Block-FP8 consumer rows for the fused RMSNorm + group-128 quantizer:
    d=7168, 1% = 72 outlier channels x50 (the d=2816 recipe), eps 1e-6."""
    return rms_rows(M, 7168, 72, 50.0, seed)


def group_t3(M: int, K: int = 4096, seed: int = 0):
    """Student-t (nu = 3) activations, bf16 [M, K]."""
    rng = np.random.default_rng(seed)
    x = rng.standard_t(3.0, size=(M, K)).astype(np.float32)
    return dict(x=to_bf16_bits(x), M=M, K=K, group=128)


def layernorm_rows(M: int = 16384, d: int = 4096, seed: int = 0):
    """x ~ N(0.5, 1) bf16; gamma 1 + 0.1 N, beta 0.1 N fp32; eps 1e-5; scale 0.05."""
    rng = np.random.default_rng(seed)
    x = (0.5 + rng.standard_normal((M, d), dtype=np.float32)).astype(np.float32)
    gamma = _gamma(rng, d)
    beta = (0.1 * rng.standard_normal(d)).astype(np.float32)
    return dict(x=to_bf16_bits(x), gamma=gamma, beta=beta, eps=1e-5, scale=0.05, M=M, d=d)


def nvfp4_7168(M: int, seed: int = 0):
    """Residual-add + RMSNorm at d=7168, x and residual ~ N(0,1), eps 1e-6."""
    return rms_rows(M, 7168, 0, 1.0, seed)


def nvfp4_slice(M: int, seed: int = 0):
    """Residual-less RMSNorm reading columns 0..1535 of [M, 2112] rows in place."""
    return rms_rows(M, 1536, 0, 1.0, seed, residual=False, ld=2112)


# A nominal NVFP4 global decode scale for unit-variance normalized rows:
# y has max |y| of about 6 over millions of N(0,1)-like samples, and the
# largest block scale times the largest element is 448 * 6 = 2688.
NVFP4_NOMINAL_GLOBAL_SCALE = 6.0 / 2688.0
