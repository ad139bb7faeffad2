"""Host checks of the arithmetic shortcuts the kernels take in place of a
correctly rounded division (CPU only; the device routines themselves are
compared on the GPU in tests/test_gpu_arith.py).

* The binary64 quotient of a row sum by the row length d (mean, mean
  square, variance): Markstein's correction of a * RN(1/d) equals RN(a/d)
  for every d <= 2^15.  Checked for every d with random numerators over the
  whole range the kernels divide, with numerators built to put a/d within a
  few ulps of 2^-53 (relative) of a rounding boundary, and with exact
  quotients.
* The NVFP4 block maximum over 6 in binary32: the same correction from
  RN(1/6) equals RN(amax/6) for every finite amax >= 2^-120 (exhaustive),
  and fails only far below that bound, where the kernels divide instead.

Page: "per_token_group_quant_8bit: multiply by reciprocal instead of
dividing per element", "Details" (one correctly rounded division per group;
the exact reciprocal).
"""
import ctypes
import struct

import pytest

from tests import shortcuts


@pytest.fixture(scope="module")
def sp():
    return shortcuts.lib()


def _bits(v: float) -> int:
    return struct.unpack("<I", struct.pack("<f", v))[0]


def test_div_by_len_every_row_length(sp):
    bad_a, bad_d = ctypes.c_double(0.0), ctypes.c_int32(0)
    n = sp.sp_div_len_check(32768, 64, 20241203, ctypes.byref(bad_a), ctypes.byref(bad_d))
    # 32768 lengths x 64 x 5 numerators = 10.5 M quotients
    assert n == 0, f"{n} mismatches, first a={bad_a.value!r} d={bad_d.value}"


def test_div6_exact_for_every_binary32_from_2_pow_minus_120(sp):
    lo, hi = _bits(2.0 ** -120), 0x7F7FFFFF  # 2^-120 .. largest finite
    fb, lb = ctypes.c_uint32(0), ctypes.c_uint32(0)
    n = sp.sp_div6_check(lo, hi, ctypes.byref(fb), ctypes.byref(lb))
    assert n == 0, f"{n} mismatches from {fb.value:#x} to {lb.value:#x}"


def test_div6_fails_only_below_2_pow_minus_125(sp):
    # Below 2^-120 the correction is not exact everywhere: the kernels take
    # the division there.  The failures lie between 1.125 * 2^-146 and just
    # under 2^-125 (subnormal quotients), so the bound 2^-120 the kernels
    # use has a margin of 2^5.
    fb, lb = ctypes.c_uint32(0), ctypes.c_uint32(0)
    n = sp.sp_div6_check(1, _bits(2.0 ** -120) - 1, ctypes.byref(fb), ctypes.byref(lb))
    assert n > 0
    first = struct.unpack("<f", struct.pack("<I", fb.value))[0]
    last = struct.unpack("<f", struct.pack("<I", lb.value))[0]
    assert first == 1.125 * 2.0 ** -146 and last < 2.0 ** -125, (first, last)
