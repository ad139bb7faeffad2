"""CPU checks of the Python binding (fp4_quantization_amd/nq.py): every entry
point refuses host tensors and wrong dtypes with a Python exception before it
calls into the library, so a device kernel can never receive a host pointer.
No GPU is needed (nothing reaches a HIP call)."""
import pytest
import torch


@pytest.fixture(scope="module")
def nq():
    import fp4_quantization_amd.nq as m
    return m


M, D = 4, 256


def _host():
    bf = lambda *s: torch.zeros(*s, dtype=torch.bfloat16)
    f32 = lambda *s: torch.zeros(*s, dtype=torch.float32)
    u8 = lambda *s: torch.zeros(*s, dtype=torch.uint8)
    return dict(x=bf(M, D), r=bf(M, D), ro=bf(M, D), g=f32(D), b=f32(D), sc=f32(1), q=u8(M, D), s=f32(M),
                sg=f32(M, D // 128), qf=u8(M, D // 2), sf=u8(M, D // 16), n=bf(M, D))


def _calls(nq, t):
    return {
        "nq_fused_add_rmsnorm_quant_fp8":
            lambda: nq.nq_fused_add_rmsnorm_quant_fp8(t["x"], t["r"], t["ro"], t["g"], 1e-6, None, t["q"], t["s"]),
        "nq_fused_add_rmsnorm_quant_fp8_ex":
            lambda: nq.nq_fused_add_rmsnorm_quant_fp8_ex(t["x"], t["r"], t["ro"], t["g"], 1e-6, None, 0, t["q"],
                                                         t["s"]),
        "nq_fused_add_rmsnorm_quant_fp8_group":
            lambda: nq.nq_fused_add_rmsnorm_quant_fp8_group(t["x"], t["r"], t["ro"], t["g"], 1e-6, t["q"], t["sg"]),
        "nq_layernorm_quant_fp8":
            lambda: nq.nq_layernorm_quant_fp8(t["x"], t["g"], t["b"], 1e-5, t["sc"], t["q"]),
        "nq_layernorm_quant_fp8_ex":
            lambda: nq.nq_layernorm_quant_fp8_ex(t["x"], t["g"], t["b"], 1e-5, None, 0, t["q"], t["s"]),
        "nq_per_token_group_quant_fp8":
            lambda: nq.nq_per_token_group_quant_fp8(t["x"], t["q"], t["sg"].view(-1)),
        "nq_per_token_group_quant_fp8_ex":
            lambda: nq.nq_per_token_group_quant_fp8_ex(t["x"], t["q"], t["sg"].view(-1), flags=nq.NQ_FLAG_E5M2),
        "nq_rmsnorm_quant_nvfp4":
            lambda: nq.nq_rmsnorm_quant_nvfp4(t["x"], t["r"], t["ro"], t["g"], 1e-6, t["sc"], t["qf"], t["sf"]),
        "nq_rmsnorm_quant_nvfp4_ex":
            lambda: nq.nq_rmsnorm_quant_nvfp4_ex(t["x"], t["r"], t["ro"], t["g"], 1e-6, t["sc"], 0, t["qf"],
                                                 t["sf"]),
        "nq_fused_add_rmsnorm_bf16":
            lambda: nq.nq_fused_add_rmsnorm_bf16(t["x"], t["r"], t["ro"], t["g"], 1e-6, t["n"]),
        "nq_per_token_quant_fp8":
            lambda: nq.nq_per_token_quant_fp8(t["x"], None, 0, t["q"], t["s"]),
        "nq_diag_copy":
            lambda: nq.nq_diag_copy(t["q"].view(-1), t["n"].view(torch.uint8).view(-1)),
        "nq_diag_codec":
            lambda: nq.nq_diag_codec(nq.NQ_CODEC_E4M3, t["g"], t["q"].view(-1)[:D]),
        "nq_diag_arith":
            lambda: nq.nq_diag_arith(nq.NQ_ARITH_RCP, t["g"], None, t["b"]),
    }


def test_every_compute_entry_point_is_covered(nq):
    names = {n for n in dir(nq) if n.startswith("nq_") and callable(getattr(nq, n))}
    names -= {"nq_status_string", "nq_version"}
    assert names == set(_calls(nq, _host())), names ^ set(_calls(nq, _host()))


def test_host_tensors_are_refused(nq):
    for name, call in _calls(nq, _host()).items():
        with pytest.raises(ValueError, match="device"):
            call()


def test_wrong_dtypes_are_refused(nq):
    t = _host()
    t["x"] = t["x"].float()          # bf16 rows expected
    t["q"] = t["q"].to(torch.int16)  # byte codes expected
    t["g"] = t["g"].to(torch.float64)
    for name, call in _calls(nq, t).items():
        if name == "nq_diag_copy":  # copies bytes of any dtype
            continue
        with pytest.raises(TypeError):
            call()


@pytest.mark.gpu
def test_row_count_mismatches_are_refused(nq):
    """An output (or residual) with fewer rows than the input is refused
    before the call: the kernel would otherwise write past it."""
    dev = {k: v.cuda() for k, v in _host().items()}
    short = {k: v[: M - 1] if v.dim() == 2 else v for k, v in dev.items()}
    for key in ("r", "ro", "q", "qf", "sf", "n", "sg"):
        t = dict(dev)
        t[key] = short[key]
        for name, call in _calls(nq, t).items():
            if name.startswith("nq_diag") or key not in _uses(name):
                continue
            with pytest.raises(ValueError, match="rows|elements"):
                call()


def _uses(name):
    """The matrix arguments each entry point takes, by the keys of _host()."""
    return {
        "nq_fused_add_rmsnorm_quant_fp8": ("r", "ro", "q"),
        "nq_fused_add_rmsnorm_quant_fp8_ex": ("r", "ro", "q"),
        "nq_fused_add_rmsnorm_quant_fp8_group": ("r", "ro", "q", "sg"),
        "nq_layernorm_quant_fp8": ("q",),
        "nq_layernorm_quant_fp8_ex": ("q",),
        "nq_per_token_group_quant_fp8": ("q",),
        "nq_per_token_group_quant_fp8_ex": ("q",),
        "nq_rmsnorm_quant_nvfp4": ("r", "ro", "qf", "sf"),
        "nq_rmsnorm_quant_nvfp4_ex": ("r", "ro", "qf", "sf"),
        "nq_fused_add_rmsnorm_bf16": ("r", "ro", "n"),
        "nq_per_token_quant_fp8": ("q",),
    }[name]
