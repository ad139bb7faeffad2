"""Seeded random configurations of every row entry point against the oracle.

Each case draws, from its own seed, a combination that hand-picked cases may
miss: the row length (ragged, under one chunk, aligned, up to NQ_MAX_D), the
row count, padded leading dimensions, a pointer one element off 16-byte
alignment (rows off 16-byte boundaries), a gamma one element off a 16-byte
boundary (the element-wise path), fresh / in-place / absent residual,
static or dynamic scale, e4m3 or e5m2, fp32 or bf16 gamma (and beta),
norm_out, UE8M0, the bf16-sourced epilogues and strided scale rows.  Every
output row is compared with the oracle under the tolerances of
tests/parity.py; guard bands catch writes past any output.
"""
import os

import numpy as np
import pytest
import torch

from fp4_quantization_amd import workloads as W
from tests.parity import (assert_bits_equal, assert_codes, assert_scales, host_u16, host_u8,
                          to_dev_bf16, to_dev_f32, unpack_nibbles)
from tests.test_gpu_parity import (calibrated_sg, check_guard_bf16, check_guard_u8, guarded_bf16, guarded_f32, guarded_u8,
                                   note, EVERY_ROW)

pytestmark = pytest.mark.gpu
N_CASES = int(os.environ.get("NQ_RANDOM_CASES", "100"))  # cases per entry point; raise for a wider sweep
MAX_ELEMS = 6_000_000  # rows x row length per case


@pytest.fixture(scope="module")
def nq():
    import fp4_quantization_amd.nq as m
    return m


def _rng(kind, seed):
    return np.random.default_rng(7919 * kind + seed)


def _rows_for(rng, d):
    M = int(rng.choice([1, 2, 3, int(rng.integers(4, 64)), int(rng.integers(64, 3000))]))
    return max(1, min(M, MAX_ELEMS // d))


def _width(rng, align):
    """A row length: multiples of `align`, biased toward the interesting ends."""
    hi = 32768 // align
    pick = int(rng.integers(0, 4))
    n = [int(rng.integers(1, 9)), int(rng.integers(1, 64)), int(rng.integers(64, max(65, 8192 // align))),
         int(rng.integers(max(1, hi // 2), hi + 1))][pick]
    return max(1, min(n, hi)) * align


def _vec(rng, v, allow_bf16=True, off=False):
    """(fp32 values the oracle uses, device tensor, is_bf16); with `off` the
    device copy starts one element past a 16-byte boundary (the element-wise
    path)."""
    if allow_bf16 and rng.random() < 0.3:
        bits = W.to_bf16_bits(np.asarray(v, np.float32))
        vals, dev, b16 = W.bf16_bits_to_f32(bits), to_dev_bf16(bits), True
    else:
        vals, dev, b16 = np.asarray(v, np.float32), to_dev_f32(v), False
    return vals, (_off_copy(dev) if off else dev), b16


def _off_copy(dev):
    """A contiguous copy of a device vector starting one element past a
    16-byte boundary."""
    buf = torch.empty(dev.numel() + 1, dtype=dev.dtype, device="cuda")
    buf[1:].copy_(dev)
    return buf[1:]


def _gamma_off(kind, seed):
    """Whether this case's gamma starts off a 16-byte boundary (drawn from a
    generator of its own, so the other draws of the case do not change)."""
    return bool(_rng(100 + kind, seed).random() < 0.3)


def _input(rng, x_bits, d):
    """Device view of the first d columns of x_bits with a random leading
    dimension and, sometimes, a pointer one element off alignment; also the
    host copy the oracle reads."""
    M = x_bits.shape[0]
    pad = int(rng.choice([0, 0, 8, 13]))
    off = int(rng.random() < 0.25)
    full = np.zeros((M, d + pad + off), np.uint16)
    full[:, off:off + d] = x_bits[:, :d]
    dev = to_dev_bf16(full)[:, off:off + d]
    return dev, np.ascontiguousarray(x_bits[:, :d]), dict(pad=pad, misaligned=bool(off))


def _residual(rng, w, d):
    mode = str(rng.choice(["fresh", "inplace", "none"]))
    if mode == "none":
        return mode, None, None, None
    r_np = np.ascontiguousarray(w["residual"][:, :d])
    r = to_dev_bf16(r_np)
    return mode, r_np, r, (r if mode == "inplace" else None)


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_rmsnorm_fp8(nq, orc, seed):
    rng = _rng(1, seed)
    d = _width(rng, 1 if rng.random() < 0.5 else 8)
    M = _rows_for(rng, d)
    w = W.rms_rows(M, d, min(2, d // 8), 20.0, seed=seed)
    x, x_np, lay = _input(rng, w["x"], d)
    mode, r_np, r, ro = _residual(rng, w, d)
    ro_buf = None
    if mode == "fresh":
        ro_buf, ro = guarded_bf16(M, d)
    g32, g, gb = _vec(rng, w["gamma"], off=_gamma_off(1, seed))
    static = float(rng.choice([0.01, 0.05, 1.0])) if rng.random() < 0.3 else None
    fmt = "e5m2" if rng.random() < 0.3 else "e4m3"
    want_n = rng.random() < 0.3
    note(f"random rms fp8 seed={seed} M={M} d={d} {lay} residual={mode} static={static} {fmt} "
         f"gamma_bf16={gb} gamma_off={g.data_ptr() % 16 != 0} norm_out={want_n}")
    q_buf, q = guarded_u8(M, d)
    s_buf, s = guarded_f32(M)
    n_buf, n = guarded_bf16(M, d) if want_n else (None, None)
    nq.nq_fused_add_rmsnorm_quant_fp8_ex(x, r, ro, g, w["eps"], to_dev_f32([static]) if static else None,
                                         nq.NQ_FLAG_E5M2 if fmt == "e5m2" else 0, q,
                                         None if static else s, n)
    torch.cuda.synchronize()
    check_guard_u8(q_buf, M * d)
    check_guard_bf16(ro_buf, M * d)
    check_guard_bf16(n_buf, M * d)
    rows = EVERY_ROW
    o = orc.fused_add_rmsnorm_quant_fp8(x_np[rows], None if r_np is None else r_np[rows], g32, w["eps"],
                                        static_scale=static, want_norm_out=want_n, fmt=fmt)
    if r_np is not None:
        assert_bits_equal(host_u16(ro)[rows], o["residual_out"], "residual_out")
    if static is None:
        assert_scales(s.cpu().numpy()[rows], o["scale"], "scale", exact=True)
        assert np.all(np.isnan(s_buf[M:].cpu().numpy()))
    assert_codes(host_u8(q)[rows], o["q"], "q", fmt=fmt, exact=True)
    if want_n:
        assert_bits_equal(host_u16(n)[rows], o["norm_out"], "norm_out")


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_layernorm_fp8(nq, orc, seed):
    rng = _rng(2, seed)
    d = _width(rng, 1 if rng.random() < 0.5 else 8)
    M = _rows_for(rng, d)
    w = W.layernorm_rows(M=M, d=d, seed=seed)
    x, x_np, lay = _input(rng, w["x"], d)
    bf = rng.random() < 0.3
    if bf:
        gbits, bbits = W.to_bf16_bits(w["gamma"]), W.to_bf16_bits(w["beta"])
        g32, b32 = W.bf16_bits_to_f32(gbits), W.bf16_bits_to_f32(bbits)
        g, b = to_dev_bf16(gbits), to_dev_bf16(bbits)
    else:
        g32, b32 = w["gamma"], w["beta"]
        g, b = to_dev_f32(g32), to_dev_f32(b32)
    goff = _gamma_off(2, seed)
    if goff:  # both vectors one element past a 16-byte boundary
        g, b = (_off_copy(t) for t in (g, b))
    static = float(rng.choice([0.01, 0.05, 1.0])) if rng.random() < 0.5 else None
    fmt = "e5m2" if rng.random() < 0.3 else "e4m3"
    note(f"random layernorm seed={seed} M={M} d={d} {lay} static={static} {fmt} bf16_vectors={bf} "
         f"vectors_off={goff}")
    q_buf, q = guarded_u8(M, d)
    s_buf, s = guarded_f32(M)
    nq.nq_layernorm_quant_fp8_ex(x, g, b, w["eps"], to_dev_f32([static]) if static else None,
                                 nq.NQ_FLAG_E5M2 if fmt == "e5m2" else 0, q, None if static else s)
    torch.cuda.synchronize()
    check_guard_u8(q_buf, M * d)
    rows = EVERY_ROW
    o = orc.layernorm_quant_fp8(x_np[rows], g32, b32, w["eps"], static, fmt=fmt)
    if static is None:
        assert_scales(s.cpu().numpy()[rows], o["scale"], "scale")
        assert np.all(np.isnan(s_buf[M:].cpu().numpy()))
    assert_codes(host_u8(q)[rows], o["q"], "q", fmt=fmt)


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_rmsnorm_nvfp4(nq, orc, seed):
    rng = _rng(3, seed)
    d = _width(rng, 16)
    M = _rows_for(rng, d)
    w = W.rms_rows(M, d, min(2, d // 16), 20.0, seed=seed)
    x, x_np, lay = _input(rng, w["x"], d)
    mode, r_np, r, ro = _residual(rng, w, d)
    if mode == "fresh":
        ro = torch.empty(M, d, dtype=torch.bfloat16, device="cuda")
    g32, g, gb = _vec(rng, w["gamma"], off=_gamma_off(3, seed))
    mode_b = rng.random() < 0.3
    want_n = rng.random() < 0.3
    sg = calibrated_sg(orc, dict(w, x=x_np, residual=r_np, gamma=g32)) * float(rng.choice([1.0, 1.0, 0.25]))
    note(f"random nvfp4 seed={seed} M={M} d={d} {lay} residual={mode} bf16_source={mode_b} "
         f"gamma_bf16={gb} gamma_off={g.data_ptr() % 16 != 0} norm_out={want_n}")
    q_buf, q = guarded_u8(M, d // 2)
    sf_buf, sf = guarded_u8(M, d // 16)
    n = torch.empty(M, d, dtype=torch.bfloat16, device="cuda") if want_n else None
    nq.nq_rmsnorm_quant_nvfp4_ex(x, r, ro, g, w["eps"], to_dev_f32([sg]),
                                 nq.NQ_FLAG_BF16_SOURCE if mode_b else 0, q, sf, n)
    torch.cuda.synchronize()
    check_guard_u8(q_buf, M * d // 2)
    check_guard_u8(sf_buf, M * d // 16)
    rows = EVERY_ROW
    o = orc.rmsnorm_quant_nvfp4(x_np[rows], None if r_np is None else r_np[rows], g32, w["eps"], sg,
                                want_norm_out=want_n, mode_b=mode_b)
    if r_np is not None:
        assert_bits_equal(host_u16(ro)[rows], o["residual_out"], "residual_out")
    assert_codes(host_u8(sf)[rows], o["sf"], "block scales", exact=True)
    assert_codes(unpack_nibbles(host_u8(q)[rows]), unpack_nibbles(o["q"]), "e2m1 codes", fmt="e2m1", exact=True)
    if want_n:
        assert_bits_equal(host_u16(n)[rows], o["norm_out"], "norm_out")


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_rmsnorm_fp8_group(nq, orc, seed):
    rng = _rng(4, seed)
    d = _width(rng, 128)
    M = _rows_for(rng, d)
    G = d // 128
    w = W.rms_rows(M, d, min(2, d // 64), 50.0, seed=seed)
    x, x_np, lay = _input(rng, w["x"], d)
    mode, r_np, r, ro = _residual(rng, w, d)
    if mode == "fresh":
        ro = torch.empty(M, d, dtype=torch.bfloat16, device="cuda")
    g32, g, gb = _vec(rng, w["gamma"], off=_gamma_off(4, seed))
    ue8m0 = rng.random() < 0.5
    src = rng.random() < 0.3
    fmt = "e5m2" if rng.random() < 0.3 else "e4m3"
    want_n = rng.random() < 0.3
    ld_s = G + int(rng.choice([0, 0, 3]))
    note(f"random rms group seed={seed} M={M} d={d} {lay} residual={mode} ue8m0={ue8m0} bf16_source={src} "
         f"{fmt} gamma_bf16={gb} gamma_off={g.data_ptr() % 16 != 0} norm_out={want_n} ld_s={ld_s}")
    q_buf, q = guarded_u8(M, d)
    s_buf = torch.full((M * ld_s + 16,), float("nan"), dtype=torch.float32, device="cuda")
    s = s_buf[: M * ld_s].view(M, ld_s)[:, :G]
    n = torch.empty(M, d, dtype=torch.bfloat16, device="cuda") if want_n else None
    flags = (nq.NQ_FLAG_BF16_SOURCE if src else 0) | (nq.NQ_FLAG_E5M2 if fmt == "e5m2" else 0)
    nq.nq_fused_add_rmsnorm_quant_fp8_group(x, r, ro, g, w["eps"], q, s,
                                            scale_mode=nq.NQ_SCALE_UE8M0 if ue8m0 else nq.NQ_SCALE_FP32,
                                            flags=flags, norm_out=n)
    torch.cuda.synchronize()
    check_guard_u8(q_buf, M * d)
    sh = s_buf.cpu().numpy()
    assert np.all(np.isnan(sh[M * ld_s:]))
    if ld_s > G:
        assert np.all(np.isnan(sh[: M * ld_s].reshape(M, ld_s)[:, G:]))
    rows = EVERY_ROW
    o = orc.fused_add_rmsnorm_quant_fp8_group(x_np[rows], None if r_np is None else r_np[rows], g32, w["eps"],
                                              ue8m0=ue8m0, bf16_source=src, want_norm_out=want_n, fmt=fmt)
    if r_np is not None:
        assert_bits_equal(host_u16(ro)[rows], o["residual_out"], "residual_out")
    got_s = s.cpu().numpy()[rows]
    if ue8m0:
        assert_bits_equal(got_s.view(np.uint32), o["scale"].view(np.uint32), "ue8m0 scales")
    else:
        assert_scales(got_s, o["scale"], "group scales", exact=True)
    assert_codes(host_u8(q)[rows], o["q"], "q", fmt=fmt, exact=True)
    if want_n:
        assert_bits_equal(host_u16(n)[rows], o["norm_out"], "norm_out")


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_group_quant(nq, orc, seed):
    rng = _rng(5, seed)
    K = _width(rng, 128)
    M = _rows_for(rng, K)
    w = W.group_t3(M, K=K, seed=seed)
    x, x_np, lay = _input(rng, w["x"], K)
    ue8m0 = rng.random() < 0.5
    fmt = "e5m2" if rng.random() < 0.3 else "e4m3"
    note(f"random group seed={seed} M={M} K={K} {lay} ue8m0={ue8m0} {fmt}")
    G = K // 128
    q_buf, q = guarded_u8(M, K)
    s_buf, s = guarded_f32(M * G)
    nq.nq_per_token_group_quant_fp8_ex(x, q, s, scale_mode=nq.NQ_SCALE_UE8M0 if ue8m0 else nq.NQ_SCALE_FP32,
                                       flags=nq.NQ_FLAG_E5M2 if fmt == "e5m2" else 0)
    torch.cuda.synchronize()
    check_guard_u8(q_buf, M * K)
    assert np.all(np.isnan(s_buf[M * G:].cpu().numpy()))
    rows = EVERY_ROW
    o = orc.per_token_group_quant_fp8(x_np[rows], 128, ue8m0=ue8m0, fmt=fmt)
    # exact max, one correctly rounded division and reciprocal per group
    assert_bits_equal(s.cpu().numpy().reshape(M, G)[rows].view(np.uint32), o["scale"].view(np.uint32), "scales")
    assert_bits_equal(host_u8(q)[rows], o["q"], "codes")
