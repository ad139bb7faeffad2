"""Shared pytest configuration.

Markers:
  gpu -- needs an AMD MI355X (gfx950) and the built libnq.so; everything else
         runs on a CPU-only host.
"""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X GPU and the built HIP library")


@pytest.fixture(scope="session")
def orc():
    """The CPU oracle (built on first use); its row operations run over
    blocks of rows on host threads (tests/parity.py: ParallelOracle)."""
    import oracle
    from tests.parity import ParallelOracle
    oracle.lib()
    return ParallelOracle(oracle)


FULL_SIZE = 1_000_000  # outputs with at least this many elements are listed one by one


def pytest_terminal_summary(terminalreporter):
    """Exact GPU-vs-oracle agreement of this session's comparisons: every
    full-size output listed, then totals per kind of output."""
    try:
        from tests.parity import REPORT
    except Exception:
        return
    if not REPORT:
        return
    tr = terminalreporter
    tr.section("GPU-vs-oracle agreement (exact counts)")
    for test, what, kind, size, diff, worst in REPORT:
        if size < FULL_SIZE:
            continue
        extra = f", worst relative scale error {worst:.3g}" if kind == "scale" else ""
        label = "differ" if kind in ("bits", "scale") else "codes one step apart"
        tr.write_line(f"{test} {what}: {diff} of {size} {label}{extra}")
    tot = {}
    for _, _, kind, size, diff, worst in REPORT:
        k = tot.setdefault(kind, [0, 0, 0, 0.0])
        k[0] += 1
        k[1] += size
        k[2] += diff
        k[3] = max(k[3], worst)
    for kind, (n, size, diff, worst) in sorted(tot.items()):
        extra = f", worst relative error {worst:.3g}" if kind == "scale" else ""
        tr.write_line(f"total {kind}: {n} comparisons, {size} elements, {diff} differing{extra}")
