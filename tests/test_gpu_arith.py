"""Device checks of the arithmetic shortcuts the kernels take in place of a
correctly rounded operation, through nq_diag_arith (the C ABI), against
correctly rounded results computed on the host with numpy:

* rcp_rn (hardware reciprocal + one Newton step): every binary32 s in
  [2^-75, 2^64), the range sqrt(mean + eps) can take;
* rsqrt_rn (correctly rounded sqrt, then rcp_rn): every non-negative
  binary32, 0 and infinity;
* div_by (Markstein's correction of y * RN(1/s), the per-token quotient):
  random and edge operands over the scales and quotients the kernels see;
* div_by_len (binary64 quotient by the row length): every d <= 32768 with
  random, near-midpoint and exact numerators;
* div6_rn (RN(amax/6), with its ballot-guarded division for tiny maxima):
  every finite non-negative binary32;
* token_scale (the per-token scale RN(amax / fmax) by Markstein's quotient
  and its reciprocal by rcp_rn, with a voted fallback): every finite
  non-negative binary32 amax, both FP8 formats;
* sum2_bf16 (the packed bf16 dot product of LayerNorm's binary32 chunk
  sums, which is not rounded to nearest): its error bound and where it is
  exact, for every bf16 of 2^-96 .. 2^96 in each half.

Whole binades are checked through one table of the significands: for a
normal result, RN(f(m * 2^k)) is RN(f(m)) with its exponent moved by the
power of two, so each binade's expected bit patterns are the table's plus
a constant.  Division and square root on the host are IEEE binary64 (or
binary32 sqrt), and rounding a binary64 quotient or root of binary32
operands to binary32 is correctly rounded (double rounding is innocuous
there), so every expected value is the correctly rounded one.

Page: "per_token_group_quant_8bit: multiply by reciprocal instead of
dividing per element", "Details" (one correctly rounded division per group;
the exact reciprocal).
"""
import numpy as np
import pytest
import torch

from tests.parity import assert_codes

pytestmark = pytest.mark.gpu

N_SIG = 1 << 23


@pytest.fixture(scope="module")
def nq():
    import fp4_quantization_amd.nq as m
    return m


def note(msg):
    print(f"[case] {msg}", flush=True)


def _significands() -> np.ndarray:
    """Every binary32 in [1, 2)."""
    return ((np.arange(N_SIG, dtype=np.uint32)) | np.uint32(127 << 23)).view(np.float32)


def _binade_dev(field: int, mant: torch.Tensor) -> torch.Tensor:
    return (mant | (field << 23)).view(torch.float32)


def _run(nq, kind, a, b=None):
    out = torch.empty_like(a)
    nq.nq_diag_arith(kind, a, b, out)
    return out


def _host_rcp(s32: np.ndarray) -> np.ndarray:
    return (1.0 / s32.astype(np.float64)).astype(np.float32)


def test_rcp_rn_every_significand(nq):
    note("rcp_rn, binades 2^-75 .. 2^63")
    table = torch.from_numpy(_host_rcp(_significands()).view(np.int32)).cuda()
    mant = torch.arange(N_SIG, dtype=torch.int32, device="cuda")
    bad = {}
    for field in range(127 - 75, 127 + 64):
        got = _run(nq, nq.NQ_ARITH_RCP, _binade_dev(field, mant)).view(torch.int32)
        want = table - ((field - 127) << 23)  # RN(1/(m 2^k)) = RN(1/m) 2^-k
        n = int((got != want).sum())
        if n:
            bad[field - 127] = n
    torch.cuda.synchronize()
    assert not bad, f"binades (exponent: mismatches) {bad}"


def test_rsqrt_rn_every_binary32(nq):
    note("rsqrt_rn, every non-negative binary32")
    m = _significands()
    # x = m 2^k: k even -> RN(1/RN(sqrt m)) 2^(-k/2); k odd -> with 2m, 2^(-(k-1)/2)
    even = _host_rcp(np.sqrt(m)).view(np.int32)
    odd = _host_rcp(np.sqrt(2.0 * m.astype(np.float32))).view(np.int32)
    tables = [torch.from_numpy(even).cuda(), torch.from_numpy(odd).cuda()]
    mant = torch.arange(N_SIG, dtype=torch.int32, device="cuda")
    bad = {}
    for field in range(1, 255):
        k = field - 127
        got = _run(nq, nq.NQ_ARITH_RSQRT, _binade_dev(field, mant)).view(torch.int32)
        want = tables[k & 1] - ((k >> 1) << 23)
        n = int((got != want).sum())
        if n:
            bad[k] = n
    assert not bad, f"binades (exponent: mismatches) {bad}"
    # subnormal x (and 0 -> infinity), +infinity -> 0
    sub = np.arange(N_SIG, dtype=np.uint32).view(np.float32)
    got = _run(nq, nq.NQ_ARITH_RSQRT, torch.from_numpy(sub).cuda()).cpu().numpy()
    with np.errstate(divide="ignore"):
        want = _host_rcp(np.sqrt(sub))
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    assert got[0] == np.inf
    inf = _run(nq, nq.NQ_ARITH_RSQRT, torch.tensor([np.inf], dtype=torch.float32, device="cuda"))
    assert inf.item() == 0.0


def test_div_by_matches_division(nq, orc):
    """y / s for s = RN(amax / fmax) over normal scales and |y| up to about
    fmax * s (both FP8 formats), signs mixed, plus edges.  Markstein's
    correction needs its remainder y - s * q0 to be exact: it is a multiple of
    2^(e_y - 46) below 2^(e_y - 22), so exact for |y| >= 2^-103.  There, with a
    quotient of at least 2^-126, the result must be the correctly rounded
    quotient.  Elsewhere its e4m3 and e5m2 codes must meet the parity bound
    against those of the correctly rounded quotient (the kernels quantize it
    next)."""
    rng = np.random.default_rng(5)
    n = 1 << 24
    checked = exact_checked = 0
    for part in range(4):
        note(f"div_by part {part}")
        e = rng.integers(-126, 113, n)
        s = np.ldexp(1.0 + rng.random(n), e).astype(np.float32)
        if part == 0:  # quotients spread over the whole FP8 range, log-uniform
            u = np.exp2(rng.uniform(-30.0, 16.0, n))
        elif part == 1:  # uniform up to the e5m2 maximum
            u = rng.uniform(0.0, 57344.0 * 1.001, n)
        elif part == 2:  # uniform up to the e4m3 maximum
            u = rng.uniform(0.0, 448.0 * 1.001, n)
        else:  # y = the row maximum itself, s = RN(amax / 448) or RN(amax / 57344)
            amax = np.ldexp(1.0 + rng.random(n), rng.integers(-110, 120, n)).astype(np.float32)
            fmax = np.where(rng.random(n) < 0.5, 448.0, 57344.0)
            s = (amax.astype(np.float64) / fmax).astype(np.float32)
            u = amax.astype(np.float64) / s.astype(np.float64)
        sign = np.where(rng.random(n) < 0.5, -1.0, 1.0)
        y = (sign * u * s.astype(np.float64)).astype(np.float32) if part < 3 else (sign * amax).astype(np.float32)
        keep = np.isfinite(y) & (s > 0)
        y, s = y[keep], s[keep]
        got = _run(nq, nq.NQ_ARITH_DIV, torch.from_numpy(y).cuda(), torch.from_numpy(s).cuda()).cpu().numpy()
        exact = y.astype(np.float64) / s.astype(np.float64)
        want = exact.astype(np.float32)
        ok_range = (np.abs(exact) >= 2.0 ** -126) & (np.abs(y) >= 2.0 ** -103)
        differ = got.view(np.uint32) != want.view(np.uint32)
        mism = np.nonzero(ok_range & differ)[0]
        assert mism.size == 0, (part, mism.size, y[mism[:3]], s[mism[:3]], got[mism[:3]], want[mism[:3]])
        # outside that range the quotient is not always the correctly
        # rounded one; its FP8 codes (what the kernels make of it) must meet
        # the parity bound against those of the correctly rounded quotient
        out = ~ok_range
        for fmt, enc in (("e4m3", orc.e4m3_encode), ("e5m2", orc.e5m2_encode)):
            assert_codes(enc(got[out]), enc(want[out]), f"div_by codes outside the exact range ({fmt})", fmt=fmt)
        checked += y.size
        exact_checked += int(ok_range.sum())
    # edges: power-of-two scales, quotients exactly 448 / 57344, y = +0 and
    # -0 (the sign of a zero quotient is kept: -0 / s = -0), and tiny y of
    # both signs whose quotient underflows to a signed zero; compared bit
    # for bit
    s = np.ldexp(np.ones(200), np.arange(-120, 80)).astype(np.float32)
    tiny = np.float32(2.0 ** -149)
    y = np.concatenate([s * 448, -s * 57344, 0 * s, np.full(200, -0.0), np.full(200, tiny),
                        np.full(200, -tiny)]).astype(np.float32)
    s3 = np.concatenate([s] * 6)
    got = _run(nq, nq.NQ_ARITH_DIV, torch.from_numpy(y).cuda(), torch.from_numpy(s3).cuda()).cpu().numpy()
    want = (y.astype(np.float64) / s3.astype(np.float64)).astype(np.float32)
    assert np.signbit(want[600:800]).all() and np.signbit(want[1000:]).all()
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    assert checked > 60_000_000 and exact_checked > 55_000_000


def _near_midpoint_numerators(d: np.ndarray, rng) -> np.ndarray:
    """For each d: the double nearest to d times a midpoint between two
    consecutive doubles (exact integer arithmetic)."""
    out = np.empty(d.size, np.float64)
    Q = (rng.integers(0, 1 << 52, d.size, dtype=np.int64) | (1 << 52)).tolist()
    E = rng.integers(-200, 200, d.size).tolist()
    for i, (di, q, e) in enumerate(zip(d.tolist(), Q, E)):
        n = di * (2 * q + 1)
        shift = max(n.bit_length() - 53, 0)
        a, rem = n >> shift, n & ((1 << shift) - 1)
        half = (1 << (shift - 1)) if shift else 0
        if shift and (rem > half or (rem == half and a & 1)):
            a += 1
        out[i] = np.ldexp(float(a), e - 53 + shift)
    return out


def test_div_by_len_every_row_length(nq):
    note("div_by_len, d = 1 .. 32768")
    rng = np.random.default_rng(6)
    d_all = np.arange(1, 32769, dtype=np.int32)
    parts = []
    # random numerators over the range the kernels divide: 2^-266 .. 2^272
    d_r = np.repeat(d_all, 24)
    a_r = np.ldexp(1.0 + rng.random(d_r.size), rng.integers(-266, 272, d_r.size))
    parts.append((a_r, d_r))
    # near-midpoint quotients, and their neighbours
    d_m = np.repeat(d_all, 4)
    a_m = _near_midpoint_numerators(d_m, rng)
    parts += [(a_m, d_m), (np.nextafter(a_m, 0.0), d_m), (np.nextafter(a_m, np.inf), d_m)]
    # exact quotients
    d_e = np.repeat(d_all, 4)
    a_e = d_e.astype(np.float64) * rng.integers(1, 1 << 38, d_e.size).astype(np.float64)
    parts.append((a_e, d_e))
    a = np.concatenate([p[0] for p in parts])
    d = np.concatenate([p[1] for p in parts])
    a = np.where(rng.random(a.size) < 0.5, -a, a)
    got = _run(nq, nq.NQ_ARITH_DIV_LEN, torch.from_numpy(a).cuda(), torch.from_numpy(d).cuda()).cpu().numpy()
    want = a / d.astype(np.float64)
    mism = np.nonzero(got.view(np.uint64) != want.view(np.uint64))[0]
    assert mism.size == 0, (mism.size, a[mism[:3]], d[mism[:3]])
    assert a.size == 32768 * 40


def test_div6_every_binary32(nq):
    note("div6_rn, every finite non-negative binary32")
    m = _significands()
    table = torch.from_numpy((m.astype(np.float64) / 6.0).astype(np.float32).view(np.int32)).cuda()
    mant = torch.arange(N_SIG, dtype=torch.int32, device="cuda")
    bad = {}
    for field in range(0, 255):
        a = _binade_dev(field, mant)
        got = _run(nq, nq.NQ_ARITH_DIV6, a)
        if field >= 8:  # quotient normal: the table, exponent moved
            want = table + ((field - 127) << 23)
            n = int((got.view(torch.int32) != want).sum())
        else:  # tiny maxima (the ballot-guarded division) and subnormals: directly
            ah = a.cpu().numpy()
            w = (ah.astype(np.float64) / 6.0).astype(np.float32)
            n = int(np.count_nonzero(got.cpu().numpy().view(np.uint32) != w.view(np.uint32)))
        if n:
            bad[field] = n
    assert not bad, f"exponent fields (field: mismatches) {bad}"



def _run2(nq, kind, a, b):
    out = torch.empty(a.shape, dtype=torch.float32, device=a.device)
    nq.nq_diag_arith(kind, a, b, out)
    return out


def _bf16_round(v: np.ndarray) -> np.ndarray:
    """binary32 -> bf16 bits, round to nearest even (finite inputs)."""
    b = v.astype(np.float32).view(np.uint32)
    return ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint32)


def _lowest_bit(v: np.ndarray) -> np.ndarray:
    """Exponent of the lowest set bit of each binary64 |v| (a large value
    for zeros, which constrain nothing)."""
    m, e = np.frexp(np.abs(v))
    sig = np.ldexp(m, 53).astype(np.int64)
    tz = np.log2((sig & -sig).astype(np.float64), where=sig > 0, out=np.zeros(v.shape)).astype(np.int64)
    return np.where(sig > 0, e - 53 + tz, 1 << 20)


def _f32_neighbours(v: np.ndarray):
    """The binary32 numbers just below and just above each binary64 v
    (both v itself when v is a binary32 number)."""
    with np.errstate(over="ignore"):
        f = v.astype(np.float32)
    up = f.astype(np.float64) > v
    down = f.astype(np.float64) < v
    lo = np.where(up, np.nextafter(f, np.float32(-np.inf)), f)
    hi = np.where(down, np.nextafter(f, np.float32(np.inf)), f)
    return lo, hi


def test_sum_bf16x2_error_bound(nq):
    """The packed bf16 dot product behind LayerNorm's binary32 chunk sums
    (lo + hi + acc, weights (1, 1)).  Every finite bf16 of magnitude
    2^-96 .. 2^96 takes each half of the word in turn, beside a random
    partner and a random accumulator within 20 binades of it (so the exact
    sum is a binary64 number), with zero partners, zero accumulators and
    near-cancelling accumulators among them.  Wherever the exact sum lies in
    the range the chunk sums trust ([2^-100, 2^100] in magnitude, or zero):

    * the result is within two units in the last place of the largest
      magnitude among the terms and the sum (the instruction aligns its
      terms with a truncated sum, so it is not always the nearest binary32,
      nor even one of the two neighbours of a much smaller, cancelled sum);
    * it is the exact sum whenever that is a binary32 number and every
      term's bits lie within the 24 bits below the largest term's leading
      bit (all terms written exactly on one binary32 grid).  Wider spreads
      can round even a representable sum: the count is printed, with the
      count of results that are not the nearest binary32."""
    note("sum2_bf16, every bf16 of 2^-96 .. 2^96 in each half")
    rng = np.random.default_rng(9)
    bits = np.arange(1 << 16, dtype=np.uint32)
    field = (bits >> 7) & 0xFF
    xb = bits[(field >= 127 - 96) & (field <= 127 + 95)]
    x = (xb << 16).view(np.float32).astype(np.float64)
    n = xb.size
    total = over_bound = inexact_narrow = wide_inexact = not_nearest = narrow_exact = 0
    worst = 0.0
    for trial in range(10):
        reach = 20 if trial < 6 else 8  # the last trials keep the terms within 2^8 of each other
        scale_o = 2.0 ** rng.integers(-reach, reach + 1, n) * rng.choice([-1.0, 1.0], n)
        scale_a = 2.0 ** rng.integers(-reach, reach + 1, n) * rng.choice([-1.0, 1.0], n)
        ob = _bf16_round(np.abs(x) * scale_o * (1.0 + rng.random(n)))
        acc = (np.abs(x) * scale_a * (1.0 + rng.random(n))).astype(np.float32)
        if trial == 0:
            ob[:] = 0  # a zero partner
        if trial == 1:
            acc[:] = 0.0  # the first step of a chunk
        if trial in (2, 6):  # cancellation: the accumulator near -(x + partner)
            acc = (-(x + (ob << 16).view(np.float32)) * (1.0 + rng.normal(0.0, 2.0 ** -12, n))).astype(np.float32)
        if trial == 7:  # accumulators that are sums of a few bf16 values (exact chunk partials)
            acc = (x * rng.integers(-3, 4, n) + (ob << 16).view(np.float32) * rng.integers(-3, 4, n)).astype(np.float32)
        o = (ob << 16).view(np.float32).astype(np.float64)
        a64 = acc.astype(np.float64)
        exact = x + o + a64
        terms = np.stack([np.abs(x), np.abs(o), np.abs(a64)])
        big = terms.max(0)
        # bits from the largest term's leading bit down to the lowest set bit of any term
        width = np.frexp(big)[1] - np.stack([_lowest_bit(t) for t in terms]).min(0)
        narrow = width <= 24
        lo, hi = _f32_neighbours(exact)
        representable = lo == hi
        checked = ((np.abs(exact) >= 2.0 ** -100) & (np.abs(exact) <= 2.0 ** 100)) | (exact == 0)
        with np.errstate(over="ignore"):
            ulp_big = np.spacing(np.maximum(big, np.abs(exact)).astype(np.float32)).astype(np.float64)
        for half in (0, 1):
            words = (xb << 16) | ob if half == 1 else xb | (ob << 16)
            got = _run2(nq, nq.NQ_ARITH_SUM_BF16X2, torch.from_numpy(words.view(np.int32)).cuda(),
                        torch.from_numpy(acc).cuda()).cpu().numpy().astype(np.float64)
            err = np.abs(got - exact) / ulp_big
            worst = max(worst, float(np.max(np.where(checked, err, 0.0))))
            over_bound += int(np.count_nonzero(checked & (err > 2.0)))
            sel = checked & representable & narrow
            narrow_exact += int(np.count_nonzero(sel))
            inexact_narrow += int(np.count_nonzero(sel & (got != exact)))
            wide_inexact += int(np.count_nonzero(checked & representable & ~narrow & (got != exact)))
            with np.errstate(over="ignore"):
                not_nearest += int(np.count_nonzero(checked & (got != exact.astype(np.float32))))
            total += int(np.count_nonzero(checked))
    print(f"sum2_bf16: {total} sums checked, worst error {worst:.3f} units in the last place of the largest "
          f"term or the sum, {over_bound} above 2; {narrow_exact} representable sums of terms on one 24-bit grid, "
          f"{inexact_narrow} of them not exact; {wide_inexact} representable sums of wider terms not exact; "
          f"{not_nearest} results not the nearest binary32", flush=True)
    assert over_bound == 0
    assert inexact_narrow == 0


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_token_scale_every_amax(nq, fmt):
    """The per-token dynamic scale s = RN(amax / fmax) and its reciprocal
    RN(1 / s) (0 for s = 0) as the kernels form them (token_scale: Markstein's
    quotient and the corrected hardware reciprocal, with a voted fallback to
    division), for every finite non-negative binary32 amax.  fmax = 7 * 2^e
    (448 = 7 * 2^6, 57344 = 7 * 2^13), so for amax = m * 2^k with m in [1, 2)
    s is RN(m / 7) * 2^(k - e) and 1 / s is RN(1 / RN(m / 7)) * 2^(e - k)
    wherever both are normal: those binades are checked through one table of
    the significands; the others (tiny maxima: subnormal scales, infinite
    reciprocals, zero) directly against the host's divisions."""
    note(f"token_scale {fmt}, every finite non-negative binary32 amax")
    kind = nq.NQ_ARITH_TOKEN_SCALE_E4M3 if fmt == "e4m3" else nq.NQ_ARITH_TOKEN_SCALE_E5M2
    e = 6 if fmt == "e4m3" else 13
    fmax = 7.0 * 2.0 ** e
    m = _significands().astype(np.float64)
    ts = (m / 7.0).astype(np.float32)
    ti = (1.0 / ts.astype(np.float64)).astype(np.float32)
    ts_dev = torch.from_numpy(ts.view(np.int32)).cuda()
    ti_dev = torch.from_numpy(ti.view(np.int32)).cuda()
    mant = torch.arange(N_SIG, dtype=torch.int32, device="cuda")
    out = torch.empty(2 * N_SIG, dtype=torch.float32, device="cuda")
    bad = {}
    for field in range(0, 255):
        a = _binade_dev(field, mant)
        nq.nq_diag_arith(kind, a, None, out)
        got = out.view(-1, 2).view(torch.int32)
        k = field - 127 - e
        if field >= 1 and k >= -123:  # s in [2^-126, 2^128), 1/s normal: the table, exponents moved
            n = int((got[:, 0] != ts_dev + (k << 23)).sum()) + int((got[:, 1] != ti_dev - (k << 23)).sum())
        else:
            ah = a.cpu().numpy().astype(np.float64)
            s = (ah / fmax).astype(np.float32)
            with np.errstate(over="ignore", divide="ignore"):
                inv = np.where(s > 0, (1.0 / s.astype(np.float64)).astype(np.float32), np.float32(0.0))
            gh = got.cpu().numpy().view(np.uint32)
            n = int(np.count_nonzero(gh[:, 0] != s.view(np.uint32))) + \
                int(np.count_nonzero(gh[:, 1] != inv.astype(np.float32).view(np.uint32)))
        if n:
            bad[field] = n
    assert not bad, f"exponent fields (field: mismatches) {bad}"
