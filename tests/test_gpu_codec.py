"""GPU parity of the device conversion routines the kernels use (e4m3 and
e5m2 with clamp, E2M1 with clamp, bf16) against the oracle's codecs, over every binary32
in the binades that reach each format, both signs, plus midpoints and
saturation edges.  Through nq_diag_codec, i.e. the C ABI."""
import numpy as np
import pytest
import torch

from tests.parity import host_u8, host_u16

pytestmark = pytest.mark.gpu


def _binade(exp_field: int, sign: int) -> np.ndarray:
    m = np.arange(1 << 23, dtype=np.uint32)
    return ((np.uint32(sign) << np.uint32(31)) | (np.uint32(exp_field) << np.uint32(23)) | m).view(np.float32)


def _run(nq, kind, v: np.ndarray) -> np.ndarray:
    x = torch.from_numpy(np.ascontiguousarray(v, np.float32)).cuda()
    if kind == nq.NQ_CODEC_BF16:
        out = torch.empty(v.size, dtype=torch.int16, device="cuda")
        nq.nq_diag_codec(kind, x, out)
        torch.cuda.synchronize()
        return host_u16(out)
    out = torch.full((v.size,), 0xA5, dtype=torch.uint8, device="cuda")
    nq.nq_diag_codec(kind, x, out)
    torch.cuda.synchronize()
    return host_u8(out)


@pytest.fixture(scope="module")
def nq():
    import fp4_quantization_amd.nq as m
    return m


@pytest.mark.parametrize("exp_lo", [116, 123, 130])
def test_e4m3_device_codec_exhaustive(nq, orc, exp_lo):
    """Binades 2^-11 .. 2^9 split over three tests, both signs."""
    for e in range(exp_lo, min(exp_lo + 7, 137)):
        for sign in (0, 1):
            v = _binade(e, sign)
            got = _run(nq, nq.NQ_CODEC_E4M3, v)
            want = orc.e4m3_encode(v)
            bad = np.nonzero(got != want)[0]
            assert bad.size == 0, (e, sign, bad.size, v[bad[:4]], got[bad[:4]], want[bad[:4]])


def test_e4m3_device_codec_edges(nq, orc):
    mags = orc.e4m3_decode(np.arange(127, dtype=np.uint8)).astype(np.float64)
    mids = ((mags[1:] + mags[:-1]) / 2).astype(np.float32)
    v = np.concatenate([mids, -mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9)),
                        np.array([0.0, -0.0, 448.0, 449.0, 464.0, 480.0, 1e6, 3e38, -3e38, 1e-40, -1e-40,
                                  2.0 ** -10, -(2.0 ** -10)], np.float32)]).astype(np.float32)
    for n in (v.size, 1, 7, 9):  # ragged tails of the 8-per-thread packing
        got = _run(nq, nq.NQ_CODEC_E4M3, v[:n])
        assert np.array_equal(got, orc.e4m3_encode(v[:n]))


@pytest.mark.parametrize("exp_lo", [109, 116, 123, 130, 137])
def test_e5m2_device_codec_exhaustive(nq, orc, exp_lo):
    """Binades 2^-18 .. 2^16 (every value that reaches e5m2, the clamp above)
    split over five tests, both signs."""
    for e in range(exp_lo, min(exp_lo + 7, 144)):
        for sign in (0, 1):
            v = _binade(e, sign)
            got = _run(nq, nq.NQ_CODEC_E5M2, v)
            want = orc.e5m2_encode(v)
            bad = np.nonzero(got != want)[0]
            assert bad.size == 0, (e, sign, bad.size, v[bad[:4]], got[bad[:4]], want[bad[:4]])


def test_e5m2_device_codec_edges(nq, orc):
    mags = orc.e5m2_decode(np.arange(124, dtype=np.uint8)).astype(np.float64)
    mids = ((mags[1:] + mags[:-1]) / 2).astype(np.float32)
    v = np.concatenate([mids, -mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9)),
                        np.array([0.0, -0.0, 57344.0, 61439.0, 61440.0, 1e6, 3e38, -3e38, 1e-40, -1e-40,
                                  2.0 ** -17, -(2.0 ** -17)], np.float32)]).astype(np.float32)
    for n in (v.size, 1, 7, 9):
        got = _run(nq, nq.NQ_CODEC_E5M2, v[:n])
        assert np.array_equal(got, orc.e5m2_encode(v[:n]))


@pytest.mark.parametrize("exp_field", list(range(121, 130)) + [0, 1, 100, 130, 131, 160, 200, 254])
def test_e2m1_device_codec_exhaustive(nq, orc, exp_field):
    """Every binary32 of the binade, both signs: the rounding binades around
    the E2M1 magnitudes, the subnormals, and binades far above 6 where the
    conversion must saturate to code 7 / 15."""
    for sign in (0, 1):
        v = _binade(exp_field, sign)
        got = _run(nq, nq.NQ_CODEC_E2M1, v)
        want = orc.e2m1_encode(v)
        bad = np.nonzero(got != want)[0]
        assert bad.size == 0, (exp_field, sign, bad.size, v[bad[:4]], got[bad[:4]], want[bad[:4]])


def test_e2m1_device_codec_edges(nq, orc):
    v = np.array([0.0, -0.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 6.5, 7.0, 100.0, 1e30, np.inf, -np.inf,
                  -0.25, -0.75, -5.0, -6.0, -7.0, -1e30, 1e-30, -1e-30, 1e-40, -1e-40,
                  np.nextafter(np.float32(0.25), np.float32(1)), np.nextafter(np.float32(5.0), np.float32(0))],
                 np.float32)
    got = _run(nq, nq.NQ_CODEC_E2M1, v)
    assert np.array_equal(got, orc.e2m1_encode(v)), (got, orc.e2m1_encode(v))


@pytest.mark.parametrize("exp_field", [0, 1, 100, 126, 127, 140, 254])
def test_bf16_device_codec_exhaustive(nq, orc, exp_field):
    for sign in (0, 1):
        v = _binade(exp_field, sign)
        assert np.array_equal(_run(nq, nq.NQ_CODEC_BF16, v), orc.bf16_encode(v))


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_bounded_fp8_device_codec_exhaustive(nq, orc, fmt):
    """The clamp-free conversion the dynamic-scale kernels use when every
    scale of the wavefront is normal: every binary32 of magnitude up to
    fmax * (1 + 2^-21) that reaches the format (from half its smallest
    subnormal), both signs, equals the clamped oracle code; this includes
    the few values just above fmax that a quotient by a normal dynamic
    scale can reach."""
    kind = nq.NQ_CODEC_E4M3_BOUNDED if fmt == "e4m3" else nq.NQ_CODEC_E5M2_BOUNDED
    enc = orc.e4m3_encode if fmt == "e4m3" else orc.e5m2_encode
    fmax = 448.0 if fmt == "e4m3" else 57344.0
    lo_field = 116 if fmt == "e4m3" else 109           # 2^-11 / 2^-18
    top_field = 127 + int(np.log2(fmax))               # binade holding fmax
    bound = np.float32(fmax * (1.0 + 2.0 ** -21))
    for e in range(lo_field, top_field + 1):
        for sign in (0, 1):
            v = _binade(e, sign)
            if e == top_field:
                v = v[np.abs(v) <= bound]
            got = _run(nq, kind, v)
            want = enc(v)
            bad = np.nonzero(got != want)[0]
            assert bad.size == 0, (fmt, e, sign, bad.size, v[bad[:4]], got[bad[:4]], want[bad[:4]])
    tiny = np.array([0.0, -0.0, 1e-40, -1e-40, 2.0 ** -30, -(2.0 ** -30)], np.float32)
    assert np.array_equal(_run(nq, kind, tiny), enc(tiny))


@pytest.mark.parametrize("nbytes", [16, 4096 + 16, 3 * 4096 * 16 + 48, 33 << 20])
def test_diag_copy_moves_every_byte(nq, nbytes):
    """The bandwidth-reference copy: every byte copied, nothing written past
    the end (ragged last block included)."""
    g = torch.Generator(device="cuda").manual_seed(nbytes)
    src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device="cuda", generator=g)
    dst = torch.full((nbytes + 64,), 0xA5, dtype=torch.uint8, device="cuda")
    nq.nq_diag_copy(src, dst)
    torch.cuda.synchronize()
    assert torch.equal(dst[:nbytes], src)
    assert bool((dst[nbytes:] == 0xA5).all())
