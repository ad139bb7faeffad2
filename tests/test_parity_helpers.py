"""The acceptance helpers of the GPU parity tests (tests/parity.py), on the
CPU: the tolerance they apply and the stricter bit-exact form."""
import numpy as np
import pytest

from tests.parity import assert_codes, assert_scales


def test_codes_tolerance_and_exact_form():
    want = np.arange(0, 4000, dtype=np.int64).astype(np.uint8)
    got = want.copy()
    assert assert_codes(got, want, "same", exact=True) == 0
    got[10] = want[10] + 1  # code 10 -> 11: the next magnitude, same sign
    assert assert_codes(got, want, "one step") == 1          # within the 0.1 % tolerance
    with pytest.raises(AssertionError, match="bit-exact"):
        assert_codes(got, want, "one step", exact=True)
    got[20] = want[20] + 2  # code 20 -> 22
    with pytest.raises(AssertionError, match="more than one step"):
        assert_codes(got, want, "two steps")


def test_signed_zero_counts_as_a_step():
    want = np.zeros(2000, np.uint8)
    got = want.copy()
    got[0] = 0x80
    assert assert_codes(got, want, "signed zero") == 1
    with pytest.raises(AssertionError):
        assert_codes(got, want, "signed zero", exact=True)


def test_scales_tolerance_and_exact_form():
    want = np.linspace(0.5, 2.0, 100).astype(np.float32)
    got = want.copy()
    got[3] = np.nextafter(want[3], np.float32(np.inf))        # one unit in the last place: 1.2e-7 relative
    assert assert_scales(got, want, "ulp") > 0
    with pytest.raises(AssertionError, match="bit-exact"):
        assert_scales(got, want, "ulp", exact=True)
    got[4] = want[4] * np.float32(1.00001)
    with pytest.raises(AssertionError, match="worst relative"):
        assert_scales(got, want, "1e-5")
    z = np.zeros(4, np.float32)
    with pytest.raises(AssertionError, match="nonzero scale"):
        assert_scales(np.float32([0, 1e-30, 0, 0]), z, "zero")
