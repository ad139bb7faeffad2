"""Comparison helpers for GPU-vs-oracle parity (test infrastructure).

Acceptance, stated once here and used by every parity test:
  * bf16 residual outputs: bit-exact;
  * scales (fp32 per token / per group): within 1e-6 relative;
  * e4m3 and E2M1 codes: identical, except that at most 0.1% of the elements
    may differ by one code step (a reduction-order tie at a rounding
    midpoint); +0 against -0 is such a step, so it is counted as a
    difference, not hidden.
The tolerance is the acceptance bound.  Comparisons of kernels whose results
are stated to be bit-exact (every one but LayerNorm, which sums its rows in
binary32 chunks) pass exact=True and are held to that: no differing code and
scales equal bit for bit.  Every comparison is also recorded
(test, output, elements compared, codes one step apart, worst relative scale
error), and the test session prints the records of the full-size outputs and
the totals at its end (tests/conftest.py), so the exact agreement is visible
in every run.

`ParallelOracle` runs the oracle's row operations over blocks of rows on host
threads (the oracle's C calls release the interpreter lock), so whole
full-size outputs are compared, not samples.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

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


# (test id, output, kind, elements, differing, worst relative scale error)
REPORT: list[tuple] = []


def _record(what, kind, size, differing, worst=0.0):
    test = os.environ.get("PYTEST_CURRENT_TEST", "?").split(" ")[0]
    REPORT.append((test, what, kind, int(size), int(differing), float(worst)))


def assert_bits_equal(got: np.ndarray, want: np.ndarray, what: str):
    assert got.shape == want.shape, (what, got.shape, want.shape)
    bad = np.count_nonzero(got != want)
    _record(what, "bits", want.size, bad)
    assert bad == 0, f"{what}: {bad} of {want.size} differ"


def assert_scales(got: np.ndarray, want: np.ndarray, what: str, exact: bool = False):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    zero = want == 0
    assert np.all(got[zero] == 0), f"{what}: nonzero scale where the oracle has 0"
    rel = np.abs(got[~zero] - want[~zero]) / np.abs(want[~zero])
    worst = float(rel.max()) if rel.size else 0.0
    differing = int(np.count_nonzero(got != want))
    _record(what, "scale", want.size, differing, worst)
    assert worst <= SCALE_RTOL, f"{what}: worst relative scale error {worst:.3g}"
    if exact:
        assert differing == 0, f"{what}: {differing} of {want.size} scales differ from a bit-exact kernel's"
    return worst


def _code_steps(a: np.ndarray, b: np.ndarray, mag_mask: int, sign_bit: int):
    a = a.astype(np.int32)
    b = b.astype(np.int32)
    am, bm = a & mag_mask, b & mag_mask
    same = a == b
    # one step: same sign and adjacent magnitudes, zero against the smallest
    # magnitude of either sign, or +0 against -0 (a sign-only difference of
    # zero counts as a differing code, so the exact-agreement counts see it)
    adjacent = (((np.abs(am - bm) == 1) & (((a & sign_bit) == (b & sign_bit)) | (np.minimum(am, bm) == 0)))
                | ((am == 0) & (bm == 0)))
    return same, adjacent


def assert_codes(got: np.ndarray, want: np.ndarray, what: str, fmt: str = "e4m3", exact: bool = False):
    """e4m3 / e5m2 codes (uint8 per element) or E2M1 codes (uint8, one per element)."""
    assert got.shape == want.shape, (what, got.shape, want.shape)
    # e4m3 and e5m2 codes both order magnitudes by their low 7 bits
    mag, sign = (0x7F, 0x80) if fmt in ("e4m3", "e5m2") else (0x7, 0x8)
    idx = np.flatnonzero(got != want)  # classify only the differing bytes
    same, adjacent = _code_steps(got.ravel()[idx], want.ravel()[idx], mag, sign)
    diff = ~same
    n = int(diff.sum())
    far = diff & ~adjacent
    _record(what, fmt, got.size, n)
    assert not far.any(), f"{what}: {far.sum()} codes differ by more than one step"
    assert n <= CODE_FLIP_FRAC * got.size, f"{what}: {n} of {got.size} codes differ by one step"
    if exact:
        assert n == 0, f"{what}: {n} of {got.size} codes differ from a bit-exact kernel's"
    return n


def unpack_nibbles(packed: np.ndarray) -> np.ndarray:
    """[rows, d/2] bytes -> [rows, d] E2M1 codes (element 2k in the low nibble)."""
    lo = packed & 0xF
    hi = packed >> 4
    return np.stack([lo, hi], axis=-1).reshape(packed.shape[0], -1)


def host_threads() -> int:
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    return max(1, min(16, cores))


class ParallelOracle:
    """The oracle module, with its row operations run over blocks of rows on
    host threads.  Every row of every operation is computed independently by
    the oracle (scales are per row or per group of a row; static and global
    scales are scalars), so splitting the rows changes no result.  A 2-D
    array argument with as many rows as the first argument is split; vectors
    (gamma, beta) and scalars are passed whole; the outputs' rows are joined
    in order."""

    ROW_OPS = ("fused_add_rmsnorm_quant_fp8", "quant_fp8_rows", "unfused_rmsnorm_quant_fp8",
               "layernorm_quant_fp8", "per_token_group_quant_fp8", "fused_add_rmsnorm_quant_fp8_group",
               "rmsnorm_quant_nvfp4")
    MIN_ROWS = 64

    def __init__(self, module):
        self._m = module

    def __getattr__(self, name):
        fn = getattr(self._m, name)
        if name not in self.ROW_OPS:
            return fn

        def run(x, *args, **kw):
            M = x.shape[0]
            if M < 2 * self.MIN_ROWS:
                return fn(x, *args, **kw)
            parts = min(4 * host_threads(), M // self.MIN_ROWS)
            bounds = np.linspace(0, M, parts + 1).astype(int)

            def cut(v, lo, hi):
                return v[lo:hi] if isinstance(v, np.ndarray) and v.ndim == 2 and v.shape[0] == M else v

            def one(k):
                lo, hi = bounds[k], bounds[k + 1]
                return fn(cut(x, lo, hi), *(cut(a, lo, hi) for a in args),
                          **{key: cut(v, lo, hi) for key, v in kw.items()})

            with ThreadPoolExecutor(host_threads()) as ex:
                outs = list(ex.map(one, range(parts)))
            return {key: (None if outs[0][key] is None else np.concatenate([o[key] for o in outs], axis=0))
                    for key in outs[0]}

        return run
