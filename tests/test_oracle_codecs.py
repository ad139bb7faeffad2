"""Pins of the oracle's number formats against things other than itself.

e4m3, e5m2 and bf16 are checked against PyTorch's own casts (library routines, a
different implementation) and against a brute-force nearest-value search in
binary64 written here; E2M1 against the brute-force search and the format's
eight magnitudes.  Format sources: the FP8 formats paper that "Fusing RMSNorm
and FP8 Quantization Under torch.compile" cites under "References" (e4m3
without infinities, largest finite 448), and the NVFP4 element format of
"RMSNorm nvfp4 quant fusion for DS V3.2 / Kimi-K2.5" ("Description").
"""
import json
import os

import numpy as np
import pytest
import torch

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")))


def _fp32_patterns(exp_field: int, sign: int = 0) -> np.ndarray:
    """All 2^23 binary32 values with the given biased exponent field."""
    m = np.arange(1 << 23, dtype=np.uint32)
    bits = (np.uint32(sign) << np.uint32(31)) | (np.uint32(exp_field) << np.uint32(23)) | m
    return bits.view(np.float32)


def _torch_e4m3(v: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.clip(v, -448.0, 448.0).astype(np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _nearest_by_search(v: np.ndarray, mags: np.ndarray) -> np.ndarray:
    """Index of the nearest magnitude to |v| (clamped), ties to the even index,
    by exhaustive comparison in binary64."""
    a = np.minimum(np.abs(v.astype(np.float64)), mags[-1])
    dist = np.abs(a[:, None] - mags[None, :])
    best = dist.min(axis=1, keepdims=True)
    cand = dist == best
    idx = np.arange(mags.size)
    # among equally near candidates prefer an even index, then the smaller
    score = np.where(cand, (idx % 2) * 1000 + idx, 10**9)
    return score.argmin(axis=1)


# ----------------------------------------------------------------- e4m3 ----

def test_e4m3_decode_matches_torch_all_codes(orc):
    codes = np.arange(256, dtype=np.uint8)
    ours = orc.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert sorted(np.nonzero(nan)[0].tolist()) == [0x7F, 0xFF]


def test_e4m3_landmarks(orc):
    codes = np.arange(256, dtype=np.uint8)
    v = orc.e4m3_decode(codes)
    finite = v[~np.isnan(v)]
    assert finite.size == 254  # +-0 counted separately: 127 magnitudes x 2 signs
    assert float(np.max(finite)) == GOLDEN["e4m3_max"]["value"] == float(v[0x7E])
    assert float(v[0x01]) == 2.0 ** -9  # smallest subnormal
    assert float(v[0x08]) == 2.0 ** -6  # smallest normal
    pos = v[:0x7F]
    assert np.all(np.diff(pos) > 0)  # codes 0..126 strictly increasing
    assert np.array_equal(v[0x80:0xFF], -v[0x00:0x7F])


@pytest.mark.parametrize("exp_field", list(range(127 - 11, 127 + 10)))
def test_e4m3_encode_matches_torch_exhaustive_binade(orc, exp_field):
    """Every binary32 in the binades that reach e4m3 (2^-11 .. 2^9), both signs."""
    for sign in (0, 1):
        v = _fp32_patterns(exp_field, sign)
        assert np.array_equal(orc.e4m3_encode(v), _torch_e4m3(v))


def test_e4m3_encode_tiny_huge_zero(orc):
    v = np.array([0.0, -0.0, 1e-30, -1e-30, 2.0 ** -10, -(2.0 ** -10), 2.0 ** -10 * (1 + 2 ** -23),
                  448.0, 449.0, 464.0, 480.0, 1e30, -1e30, 3.0e38], np.float32)
    ours = orc.e4m3_encode(v)
    assert ours.tolist() == [0x00, 0x80, 0x00, 0x80, 0x00, 0x80, 0x01,
                             0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0x7E]
    assert np.array_equal(ours, _torch_e4m3(v))


def test_e4m3_encode_nearest_by_search(orc):
    rng = np.random.default_rng(1)
    # log-uniform magnitudes across the whole e4m3 range plus exact midpoints
    mags = orc.e4m3_decode(np.arange(127, dtype=np.uint8)).astype(np.float64)
    mids = ((mags[1:] + mags[:-1]) / 2).astype(np.float32)
    v = np.concatenate([
        (np.exp2(rng.uniform(-12, 9.5, 200_000)) * rng.choice([-1, 1], 200_000)).astype(np.float32),
        mids, -mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9))])
    idx = _nearest_by_search(v, mags)
    expect = (idx | np.where(np.signbit(v), 0x80, 0)).astype(np.uint8)
    assert np.array_equal(orc.e4m3_encode(v), expect)


# ----------------------------------------------------------------- E2M1 ----

E2M1_MAGS = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


# ----------------------------------------------------------------- e5m2 ----
# OCP FP8 e5m2 (the second FP8 output format of "feat: fused FP8 quantization
# output for LayerNorm", "Description" and "Tests"): bias 15, 2 mantissa bits,
# exponent 31 for infinities and NaNs, largest finite 57344.

def _torch_e5m2(v: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.clip(v, -57344.0, 57344.0).astype(np.float32))
    return t.to(torch.float8_e5m2).view(torch.uint8).numpy()


def test_e5m2_decode_matches_torch_all_codes(orc):
    codes = np.arange(256, dtype=np.uint8)
    ours = orc.e5m2_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e5m2).to(torch.float32).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert sorted(np.nonzero(nan)[0].tolist()) == [0x7D, 0x7E, 0x7F, 0xFD, 0xFE, 0xFF]
    assert ours[0x7C] == np.inf and ours[0xFC] == -np.inf


def test_e5m2_landmarks(orc):
    v = orc.e5m2_decode(np.arange(256, dtype=np.uint8))
    assert float(v[0x7B]) == 57344.0                    # largest finite
    assert float(v[0x01]) == 2.0 ** -16                 # smallest subnormal
    assert float(v[0x04]) == 2.0 ** -14                 # smallest normal
    pos = v[:0x7C]
    assert np.all(np.diff(pos) > 0)
    assert np.array_equal(v[0x80:0xFC], -v[0x00:0x7C])


@pytest.mark.parametrize("exp_field", list(range(127 - 18, 127 + 17)))
def test_e5m2_encode_matches_torch_exhaustive_binade(orc, exp_field):
    """Every binary32 in the binades that reach e5m2 (2^-18 .. 2^16), both signs."""
    for sign in (0, 1):
        v = _fp32_patterns(exp_field, sign)
        assert np.array_equal(orc.e5m2_encode(v), _torch_e5m2(v))


def test_e5m2_encode_random_and_saturation(orc):
    rng = np.random.default_rng(5)
    bits = rng.integers(0, 2**32, 2_000_000, dtype=np.uint64).astype(np.uint32)
    v = bits.view(np.float32)
    v = v[np.isfinite(v)]
    assert np.array_equal(orc.e5m2_encode(v), _torch_e5m2(v))
    big = np.array([57344.0, 61439.0, 61440.0, 1e30, -1e30, np.float32(3.4e38)], np.float32)
    assert orc.e5m2_encode(big).tolist() == [0x7B, 0x7B, 0x7B, 0x7B, 0xFB, 0x7B]  # saturates, never inf
    assert orc.e5m2_encode(np.array([0.0, -0.0, 2.0 ** -17, -(2.0 ** -17)], np.float32)).tolist() == \
        [0x00, 0x80, 0x00, 0x80]  # the tie at half the smallest subnormal goes to even (zero)


def test_e5m2_encode_nearest_by_search(orc):
    """Against a brute-force nearest search on values straddling every
    e5m2 midpoint."""
    mags = orc.e5m2_decode(np.arange(0x7C, dtype=np.uint8)).astype(np.float64)
    mids = (mags[:-1] + mags[1:]) / 2
    v = np.concatenate([mids, np.nextafter(mids.astype(np.float32), np.float32(np.inf)),
                        np.nextafter(mids.astype(np.float32), np.float32(0)), mags]).astype(np.float32)
    want = _nearest_by_search(v, mags)
    assert np.array_equal(orc.e5m2_encode(v).astype(np.int64) & 0x7F, want)


def test_e2m1_decode_table(orc):
    vals = orc.e2m1_decode(np.arange(16, dtype=np.uint8))
    assert vals[:8].tolist() == E2M1_MAGS.tolist()
    assert vals[8:].tolist() == (-E2M1_MAGS).tolist()


@pytest.mark.parametrize("exp_field", list(range(127 - 4, 127 + 4)))
def test_e2m1_encode_exhaustive_binade_vs_search(orc, exp_field):
    """Every binary32 in 2^-4 .. 2^4 (one sign; sign symmetry checked below)."""
    v = _fp32_patterns(exp_field)
    got = orc.e2m1_encode(v)
    # the search is O(8) per element; do it on the whole binade in chunks
    for s in range(0, v.size, 1 << 20):
        idx = _nearest_by_search(v[s:s + (1 << 20)], E2M1_MAGS)
        assert np.array_equal(got[s:s + (1 << 20)], idx.astype(np.uint8))


def test_e2m1_encode_ties_sign_and_clamp(orc):
    v = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 7.0, 100.0, 1e-20, 0.0,
                  -0.25, -0.75, -5.0, -100.0, -0.0, -1e-20], np.float32)
    got = orc.e2m1_encode(v).tolist()
    # ties go to the even code: 0.25->0, 0.75->1.0(2), 1.25->1.0(2), 1.75->2.0(4),
    # 2.5->2.0(4), 3.5->4.0(6), 5.0->4.0(6); beyond 6 saturates to 6 (7)
    assert got == [0, 2, 2, 4, 4, 6, 6, 7, 7, 7, 0, 0, 8, 8 | 2, 8 | 6, 8 | 7, 8, 8]
    rng = np.random.default_rng(2)
    w = rng.uniform(-8, 8, 100_000).astype(np.float32)
    assert np.array_equal(orc.e2m1_encode(-w), orc.e2m1_encode(w) ^ 8)


# ----------------------------------------------------------------- bf16 ----

def _torch_bf16(v):
    return torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("exp_field", [1, 100, 126, 127, 128, 140, 254])
def test_bf16_encode_matches_torch_exhaustive_binade(orc, exp_field):
    for sign in (0, 1):
        v = _fp32_patterns(exp_field, sign)
        assert np.array_equal(orc.bf16_encode(v), _torch_bf16(v))


def test_bf16_encode_random_and_subnormal(orc):
    rng = np.random.default_rng(3)
    bits = rng.integers(0, 1 << 32, 4_000_000, dtype=np.uint64).astype(np.uint32)
    v = bits.view(np.float32)
    v = v[np.isfinite(v)]
    assert np.array_equal(orc.bf16_encode(v), _torch_bf16(v))
    sub = _fp32_patterns(0, 0)[::17]
    assert np.array_equal(orc.bf16_encode(sub), _torch_bf16(sub))
