"""Comparison helpers for GPU-vs-oracle parity (test infrastructure).

Acceptance, stated once here and used by every parity test:
  * bf16 residual outputs: bit-exact;
  * scales (fp32 per token / per group): within 1e-6 relative;
  * e4m3 and E2M1 codes: identical, except that at most 0.1% of the elements
    may differ by one code step (a reduction-order tie at a rounding
    midpoint); +0 and -0 count as the same code.
The kernels accumulate row sums in binary64 like the oracle, so the expected
outcome is bit-exact; the tolerance is the acceptance bound, not the
expectation, and every test also reports the exact mismatch count.
"""
from __future__ import annotations

import numpy as np
import torch

SCALE_RTOL = 1e-6
CODE_FLIP_FRAC = 1e-3


def to_dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits)).view(torch.bfloat16).cuda()


def to_dev_f32(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(np.asarray(a, np.float32))).cuda()


def host_u16(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def host_u8(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.uint8).cpu().numpy()


def assert_bits_equal(got: np.ndarray, want: np.ndarray, what: str):
    assert got.shape == want.shape, (what, got.shape, want.shape)
    bad = np.count_nonzero(got != want)
    assert bad == 0, f"{what}: {bad} of {want.size} differ"


def assert_scales(got: np.ndarray, want: np.ndarray, what: str):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    zero = want == 0
    assert np.all(got[zero] == 0), f"{what}: nonzero scale where the oracle has 0"
    rel = np.abs(got[~zero] - want[~zero]) / np.abs(want[~zero])
    worst = float(rel.max()) if rel.size else 0.0
    assert worst <= SCALE_RTOL, f"{what}: worst relative scale error {worst:.3g}"
    return worst


def _code_steps(a: np.ndarray, b: np.ndarray, mag_mask: int, sign_bit: int):
    a = a.astype(np.int32)
    b = b.astype(np.int32)
    am, bm = a & mag_mask, b & mag_mask
    same = (a == b) | ((am == 0) & (bm == 0))
    # one step: same sign and adjacent magnitudes, or zero against the
    # smallest magnitude of either sign
    adjacent = (np.abs(am - bm) == 1) & (((a & sign_bit) == (b & sign_bit)) | (np.minimum(am, bm) == 0))
    return same, adjacent


def assert_codes(got: np.ndarray, want: np.ndarray, what: str, fmt: str = "e4m3"):
    """e4m3 / e5m2 codes (uint8 per element) or E2M1 codes (uint8, one per element)."""
    assert got.shape == want.shape, (what, got.shape, want.shape)
    # e4m3 and e5m2 codes both order magnitudes by their low 7 bits
    mag, sign = (0x7F, 0x80) if fmt in ("e4m3", "e5m2") else (0x7, 0x8)
    same, adjacent = _code_steps(got, want, mag, sign)
    diff = ~same
    n = diff.sum()
    far = diff & ~adjacent
    assert not far.any(), f"{what}: {far.sum()} codes differ by more than one step"
    assert n <= CODE_FLIP_FRAC * got.size, f"{what}: {n} of {got.size} codes differ by one step"
    return int(n)


def unpack_nibbles(packed: np.ndarray) -> np.ndarray:
    """[rows, d/2] bytes -> [rows, d] E2M1 codes (element 2k in the low nibble)."""
    lo = packed & 0xF
    hi = packed >> 4
    return np.stack([lo, hi], axis=-1).reshape(packed.shape[0], -1)
