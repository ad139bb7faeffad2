"""Row alignment: every row entry point on rows that do not start on 16-byte
boundaries, and with gamma / beta that do not.

Rows of whole 8-element chunks take the 128-bit path wherever they start
(each row tensor here, inputs and outputs alike, begins one element past a
16-byte boundary and has an odd row stride, so consecutive rows sit at
different offsets).  Gamma / beta one element off a 16-byte boundary select
the element-wise path.  Both must give the aligned call's outputs bit for bit
and write nothing outside their rows.
"""
import numpy as np
import pytest
import torch

from fp4_quantization_amd import workloads as W
from tests.parity import assert_bits_equal, to_dev_bf16, to_dev_f32
from tests.test_gpu_parity import calibrated_sg, note

pytestmark = pytest.mark.gpu

FILL = {torch.uint8: 0xA5, torch.bfloat16: -23131, torch.float32: -1}  # raw bit patterns
RAW = {torch.uint8: torch.uint8, torch.bfloat16: torch.int16, torch.float32: torch.int32}


@pytest.fixture(scope="module")
def nq():
    import fp4_quantization_amd.nq as m
    return m


class Rows:
    """A [M, cols] device view whose first row starts `off` elements into its
    buffer (a 16-byte aligned allocation) with row stride cols + pad; every
    other element of the buffer holds a fill pattern."""

    def __init__(self, M, cols, dtype, off=1, pad=3, data=None):
        self.M, self.cols, self.ld, self.off, self.dtype = M, cols, cols + pad, off, dtype
        n = off + M * self.ld + 16
        self.buf = torch.full((n,), FILL[dtype], dtype=RAW[dtype], device="cuda")
        assert self.buf.data_ptr() % 16 == 0
        self.view = self.buf[off:off + M * self.ld].view(M, self.ld)[:, :cols].view(dtype)
        if data is not None:
            self.view.copy_(data)

    def untouched(self):
        """Every element outside the rows still holds the fill."""
        raw = self.buf.cpu().numpy()
        mask = np.ones(raw.shape, bool)
        idx = self.off + np.arange(self.M)[:, None] * self.ld + np.arange(self.cols)[None, :]
        mask[idx.ravel()] = False
        return bool(np.all(raw[mask] == raw.dtype.type(FILL[self.dtype])))


def off_vec(v: torch.Tensor) -> torch.Tensor:
    """A contiguous copy of v that starts one element past a 16-byte boundary."""
    buf = torch.empty(v.numel() + 1, dtype=v.dtype, device="cuda")
    assert buf.data_ptr() % 16 == 0
    out = buf[1:]
    out.copy_(v)
    return out


def same(got, want, what):
    a = got.contiguous().view(RAW[got.dtype]).cpu().numpy()
    b = want.contiguous().view(RAW[want.dtype]).cpu().numpy()
    assert_bits_equal(a, b, what)


def outputs(spec, layout):
    """Fresh output tensors: contiguous (layout 'aligned') or Rows views."""
    out = {}
    for name, (M, cols, dtype) in spec.items():
        if layout == "rows":
            out[name] = Rows(M, cols, dtype, off=1 if dtype != torch.uint8 else 3)
        else:
            out[name] = torch.empty(M, cols, dtype=dtype, device="cuda")
    return out


def tensor(o):
    return o.view if isinstance(o, Rows) else o


def check(results, spec):
    ref = results["aligned"]
    for layout in ("rows", "gamma"):
        for name in spec:
            same(tensor(results[layout][name]), ref[name], f"{name} ({layout} vs aligned)")
            if isinstance(results[layout][name], Rows):
                assert results[layout][name].untouched(), f"{name}: write outside the rows"


def inputs(arrays, layout):
    """Device copies of host bf16 bit matrices: contiguous, or Rows views."""
    out = {}
    for name, a in arrays.items():
        dev = to_dev_bf16(a)
        out[name] = Rows(*a.shape, torch.bfloat16, data=dev) if layout == "rows" else dev
    return out


LAYOUTS = ("aligned", "rows", "gamma")


@pytest.mark.parametrize("M", [3, 600])
@pytest.mark.parametrize("d", [2816, 256, 64])
def test_rmsnorm_fp8_alignment(nq, M, d):
    """d = 256 and 64 take teams narrower than a wavefront (several rows per
    buffer resource)."""
    note(f"alignment rms fp8 M={M} d={d}")
    w = W.rms_2816(M, seed=31 + M) if d == 2816 else W.rms_rows(M, d, 2, 20.0, seed=31 + M)
    g = to_dev_f32(w["gamma"])
    spec = {"ro": (M, d, torch.bfloat16), "q": (M, d, torch.uint8), "n": (M, d, torch.bfloat16)}
    res = {}
    for lay in LAYOUTS:
        i = inputs({"x": w["x"], "r": w["residual"]}, "rows" if lay == "rows" else "aligned")
        o = outputs(spec, "rows" if lay == "rows" else "aligned")
        s = torch.empty(M, device="cuda")
        nq.nq_fused_add_rmsnorm_quant_fp8(tensor(i["x"]), tensor(i["r"]), tensor(o["ro"]),
                                          off_vec(g) if lay == "gamma" else g, w["eps"], None,
                                          tensor(o["q"]), s, norm_out=tensor(o["n"]))
        torch.cuda.synchronize()
        o["s"] = s.view(1, M)
        res[lay] = o
    check(res, dict(spec, s=None))


@pytest.mark.parametrize("M", [3, 600])
def test_rmsnorm_group_alignment(nq, M):
    note(f"alignment rms group M={M}")
    d = 2816
    w = W.rms_2816(M, seed=41 + M)
    g = to_dev_f32(w["gamma"])
    spec = {"ro": (M, d, torch.bfloat16), "q": (M, d, torch.uint8), "s": (M, d // 128, torch.float32),
            "n": (M, d, torch.bfloat16)}
    res = {}
    for lay in LAYOUTS:
        i = inputs({"x": w["x"], "r": w["residual"]}, "rows" if lay == "rows" else "aligned")
        o = outputs(spec, "rows" if lay == "rows" else "aligned")
        nq.nq_fused_add_rmsnorm_quant_fp8_group(tensor(i["x"]), tensor(i["r"]), tensor(o["ro"]),
                                                off_vec(g) if lay == "gamma" else g, w["eps"],
                                                tensor(o["q"]), tensor(o["s"]), norm_out=tensor(o["n"]))
        torch.cuda.synchronize()
        res[lay] = o
    check(res, spec)


@pytest.mark.parametrize("M", [3, 600])
def test_rmsnorm_nvfp4_alignment(nq, orc, M):
    note(f"alignment rms nvfp4 M={M}")
    d = 2816
    w = W.rms_2816(M, seed=51 + M)
    g = to_dev_f32(w["gamma"])
    sg = to_dev_f32([calibrated_sg(orc, w)])
    spec = {"ro": (M, d, torch.bfloat16), "q": (M, d // 2, torch.uint8), "sf": (M, d // 16, torch.uint8),
            "n": (M, d, torch.bfloat16)}
    res = {}
    for lay in LAYOUTS:
        i = inputs({"x": w["x"], "r": w["residual"]}, "rows" if lay == "rows" else "aligned")
        o = outputs(spec, "rows" if lay == "rows" else "aligned")
        nq.nq_rmsnorm_quant_nvfp4(tensor(i["x"]), tensor(i["r"]), tensor(o["ro"]),
                                  off_vec(g) if lay == "gamma" else g, w["eps"], sg,
                                  tensor(o["q"]), tensor(o["sf"]), norm_out=tensor(o["n"]))
        torch.cuda.synchronize()
        res[lay] = o
    check(res, spec)


@pytest.mark.parametrize("M", [3, 600])
@pytest.mark.parametrize("dynamic", [False, True])
@pytest.mark.parametrize("d", [4096, 256])
def test_layernorm_alignment(nq, M, dynamic, d):
    note(f"alignment layernorm M={M} dynamic={dynamic} d={d}")
    w = W.layernorm_rows(M=M, d=d, seed=61 + M)
    g, b = to_dev_f32(w["gamma"]), to_dev_f32(w["beta"])
    sc = None if dynamic else to_dev_f32([0.05])
    spec = {"q": (M, d, torch.uint8)}
    res = {}
    for lay in LAYOUTS:
        i = inputs({"x": w["x"]}, "rows" if lay == "rows" else "aligned")
        o = outputs(spec, "rows" if lay == "rows" else "aligned")
        s = torch.empty(M, device="cuda")
        nq.nq_layernorm_quant_fp8_ex(tensor(i["x"]), off_vec(g) if lay == "gamma" else g,
                                     off_vec(b) if lay == "gamma" else b, w["eps"], sc, 0,
                                     tensor(o["q"]), s if dynamic else None)
        torch.cuda.synchronize()
        if dynamic:
            o["s"] = s.view(1, M)
        res[lay] = o
    check(res, dict(spec, **({"s": None} if dynamic else {})))


@pytest.mark.parametrize("M", [3, 600])
def test_unfused_alignment(nq, M):
    note(f"alignment unfused M={M}")
    d = 2816
    w = W.rms_2816(M, seed=71 + M)
    g = to_dev_f32(w["gamma"])
    spec = {"ro": (M, d, torch.bfloat16), "n": (M, d, torch.bfloat16), "q": (M, d, torch.uint8)}
    res = {}
    for lay in LAYOUTS:
        i = inputs({"x": w["x"], "r": w["residual"]}, "rows" if lay == "rows" else "aligned")
        o = outputs(spec, "rows" if lay == "rows" else "aligned")
        s = torch.empty(M, device="cuda")
        nq.nq_fused_add_rmsnorm_bf16(tensor(i["x"]), tensor(i["r"]), tensor(o["ro"]),
                                     off_vec(g) if lay == "gamma" else g, w["eps"], tensor(o["n"]))
        nq.nq_per_token_quant_fp8(tensor(o["n"]), None, 0, tensor(o["q"]), s)
        torch.cuda.synchronize()
        o["s"] = s.view(1, M)
        res[lay] = o
    check(res, dict(spec, s=None))


@pytest.mark.parametrize("M", [3, 600])
def test_group_quant_alignment(nq, M):
    """The standalone group quantizer has no shared vectors: its only layouts
    are aligned and unaligned rows (both 128-bit)."""
    note(f"alignment group quant M={M}")
    K = 4096
    w = W.group_t3(M, K)
    ref_q = torch.empty(M, K, dtype=torch.uint8, device="cuda")
    ref_s = torch.empty(M * K // 128, device="cuda")
    nq.nq_per_token_group_quant_fp8(to_dev_bf16(w["x"]), ref_q, ref_s)
    x = Rows(M, K, torch.bfloat16, data=to_dev_bf16(w["x"]))
    q = Rows(M, K, torch.uint8, off=5)
    sbuf = torch.full((M * K // 128 + 2,), -1, dtype=torch.int32, device="cuda")
    s = sbuf[1:1 + M * K // 128].view(torch.float32)
    nq.nq_per_token_group_quant_fp8(x.view, q.view, s)
    torch.cuda.synchronize()
    same(q.view, ref_q, "group codes (unaligned rows vs aligned)")
    same(s, ref_s, "group scales (unaligned vs aligned)")
    assert q.untouched(), "write outside the rows"
    edges = sbuf.cpu().numpy()[[0, -1]]
    assert np.all(edges == -1), "write outside the scales"
