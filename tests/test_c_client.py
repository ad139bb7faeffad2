"""The C ABI from a plain C++ program (tests/c_abi/nq_c_client.cpp, no
PyTorch): hipMalloc'd buffers, the client's own stream, an eager call, the
same call captured in a hipGraph and replayed, per-token-group FP8, the fused
RMSNorm + group FP8, LayerNorm (static e4m3 and dynamic e5m2), RMSNorm +
NVFP4, and a rejected call.  Its outputs are compared with the oracle."""
import os
import subprocess

import numpy as np
import pytest

from fp4_quantization_amd import workloads as W
from tests.parity import assert_bits_equal, assert_codes, assert_scales

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "nq_c_client")


@pytest.mark.gpu
def test_c_client_matches_the_oracle(orc, tmp_path):
    if not os.path.exists(EXE):
        pytest.fail("tests/c_abi/nq_c_client is not built (run __graft_entry__.build())")
    M, D = 64, 2816
    w = W.rms_2816(M, seed=21)
    w["x"].tofile(tmp_path / "x.bin")
    w["residual"].tofile(tmp_path / "r.bin")
    w["gamma"].astype(np.float32).tofile(tmp_path / "gamma.bin")
    beta = (0.1 * np.random.default_rng(22).standard_normal(D)).astype(np.float32)
    beta.tofile(tmp_path / "beta.bin")
    np.array([0.05], np.float32).tofile(tmp_path / "lnscale.bin")
    sg = np.float32(W.NVFP4_NOMINAL_GLOBAL_SCALE)
    np.array([sg], np.float32).tofile(tmp_path / "nvsg.bin")
    print(f"[case] C client M={M} D={D}", flush=True)
    r = subprocess.run([EXE, str(tmp_path), str(M), str(D)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "ok" in r.stdout and "stride" in r.stdout

    o = orc.fused_add_rmsnorm_quant_fp8(w["x"], w["residual"], w["gamma"], w["eps"])
    q = np.fromfile(tmp_path / "q.bin", np.uint8).reshape(M, D)
    s = np.fromfile(tmp_path / "s.bin", np.float32)
    ro = np.fromfile(tmp_path / "ro.bin", np.uint16).reshape(M, D)
    assert_bits_equal(ro, o["residual_out"], "residual_out")
    assert_scales(s, o["scale"], "scale")
    assert_codes(q, o["q"], "q")
    # the graph replays give the eager call's bits
    assert_bits_equal(np.fromfile(tmp_path / "qg.bin", np.uint8).reshape(M, D), q, "graph codes")
    assert_bits_equal(np.fromfile(tmp_path / "sg.bin", np.float32).view(np.uint32), s.view(np.uint32), "graph scales")

    og = orc.per_token_group_quant_fp8(w["x"], 128)
    gq = np.fromfile(tmp_path / "gq.bin", np.uint8).reshape(M, D)
    gs = np.fromfile(tmp_path / "gs.bin", np.float32).reshape(M, D // 128)
    assert_bits_equal(gs.view(np.uint32), og["scale"].view(np.uint32), "group scales")
    assert_bits_equal(gq, og["q"], "group codes")

    of = orc.fused_add_rmsnorm_quant_fp8_group(w["x"], w["residual"], w["gamma"], w["eps"])
    assert_bits_equal(np.fromfile(tmp_path / "fro.bin", np.uint16).reshape(M, D), of["residual_out"],
                      "fused group residual_out")
    assert_bits_equal(np.fromfile(tmp_path / "fs.bin", np.float32).reshape(M, D // 128).view(np.uint32),
                      of["scale"].view(np.uint32), "fused group scales")
    assert_bits_equal(np.fromfile(tmp_path / "fq.bin", np.uint8).reshape(M, D), of["q"], "fused group codes")

    ol = orc.layernorm_quant_fp8(w["x"], w["gamma"], beta, 1e-5, 0.05)
    assert_codes(np.fromfile(tmp_path / "lq.bin", np.uint8).reshape(M, D), ol["q"], "layernorm static codes")
    old = orc.layernorm_quant_fp8(w["x"], w["gamma"], beta, 1e-5, None, fmt="e5m2")
    assert_scales(np.fromfile(tmp_path / "lds.bin", np.float32), old["scale"], "layernorm dynamic scales")
    assert_codes(np.fromfile(tmp_path / "ldq.bin", np.uint8).reshape(M, D), old["q"], "layernorm dynamic codes",
                 fmt="e5m2")

    on = orc.rmsnorm_quant_nvfp4(w["x"], w["residual"], w["gamma"], w["eps"], float(sg))
    assert_bits_equal(np.fromfile(tmp_path / "nro.bin", np.uint16).reshape(M, D), on["residual_out"],
                      "nvfp4 residual_out")
    assert_bits_equal(np.fromfile(tmp_path / "nsf.bin", np.uint8).reshape(M, D // 16), on["sf"], "nvfp4 block scales")
    assert_bits_equal(np.fromfile(tmp_path / "nq.bin", np.uint8).reshape(M, D // 2), on["q"], "nvfp4 codes")
