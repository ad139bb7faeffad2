"""CPU checks of the C ABI: the library loads, exports every function
include/nq.h declares, and rejects bad arguments on the host before any HIP
call (so these run without a GPU).  No compute call is made here."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nq.h")
LIB = os.path.join(ROOT, "fp4_quantization_amd", "libnq.so")

NQ_OK, NQ_ERR_NULL, NQ_ERR_SHAPE, NQ_ERR_STRIDE, NQ_ERR_ALIAS, NQ_ERR_ARG = 0, -1, -2, -3, -4, -6


def _gpu_visible() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


# The validation calls below pass fake device addresses and expect every one
# to be rejected on the host; where a GPU is visible a validation regression
# would launch a kernel on them, so these run only where none is.
pytestmark = pytest.mark.skipif(_gpu_visible(), reason="host-validation tests pass fake device addresses")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(nq_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libnq.so is not built (run __graft_entry__.build())")
    L = ctypes.CDLL(LIB)
    v, i64, i32, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float
    L.nq_fused_add_rmsnorm_quant_fp8.argtypes = [v, i64, v, i64, v, i64, v, f32, v, v, i64, v, v, i64, i64, i64, v]
    L.nq_fused_add_rmsnorm_quant_fp8_group.argtypes = [v, i64, v, i64, v, i64, v, f32, i32, i32,
                                                       ctypes.c_uint32, v, i64, v, i64, v, i64, i64, i64, v]
    L.nq_layernorm_quant_fp8.argtypes = [v, i64, v, v, f32, v, v, i64, i64, i64, v]
    u32 = ctypes.c_uint32
    L.nq_fused_add_rmsnorm_quant_fp8_ex.argtypes = [v, i64, v, i64, v, i64, v, f32, v, u32, v, i64, v, v, i64,
                                                    i64, i64, v]
    L.nq_layernorm_quant_fp8_ex.argtypes = [v, i64, v, v, f32, v, u32, v, i64, v, i64, i64, v]
    L.nq_per_token_group_quant_fp8_ex.argtypes = [v, i64, i64, i64, i32, i32, u32, v, i64, v, v]
    L.nq_rmsnorm_quant_nvfp4_ex.argtypes = [v, i64, v, i64, v, i64, v, f32, v, u32, v, i64, v, i64, v, i64, i64,
                                            i64, v]
    L.nq_fused_add_rmsnorm_bf16.argtypes = [v, i64, v, i64, v, i64, v, f32, v, i64, i64, i64, v]
    L.nq_per_token_quant_fp8.argtypes = [v, i64, v, u32, v, i64, v, i64, i64, v]
    L.nq_per_token_group_quant_fp8.argtypes = [v, i64, i64, i64, i32, i32, v, i64, v, v]
    L.nq_rmsnorm_quant_nvfp4.argtypes = [v, i64, v, i64, v, i64, v, f32, v, v, i64, v, i64, v, i64, i64, i64, v]
    L.nq_diag_codec.argtypes = [i32, v, v, i64, v]
    L.nq_diag_copy.argtypes = [v, v, i64, v]
    L.nq_diag_arith.argtypes = [i32, v, v, v, i64, v]
    L.nq_status_string.restype = ctypes.c_char_p
    L.nq_version.restype = ctypes.c_char_p
    return L


def test_header_declares_the_four_entry_points():
    fns = declared_functions()
    for name in ("nq_fused_add_rmsnorm_quant_fp8", "nq_fused_add_rmsnorm_quant_fp8_ex",
                 "nq_fused_add_rmsnorm_quant_fp8_group", "nq_layernorm_quant_fp8_ex",
                 "nq_per_token_group_quant_fp8_ex",
                 "nq_layernorm_quant_fp8",
                 "nq_per_token_group_quant_fp8", "nq_rmsnorm_quant_nvfp4", "nq_status_string"):
        assert name in fns


def test_library_exports_every_declared_symbol(lib):
    missing = [f for f in declared_functions() if not hasattr(lib, f)]
    assert not missing, missing


def test_status_strings_and_version(lib):
    assert lib.nq_status_string(0) == b"ok"
    for s in (-1, -2, -3, -4, -5, -6):
        assert lib.nq_status_string(s) not in (b"ok", b"unknown status")
    assert lib.nq_status_string(123) == b"unknown status"
    assert b"gfx950" in lib.nq_version()


# Fake device addresses: every call below is rejected (or is a no-op with
# M = 0) before anything dereferences them or touches HIP.
X, R, RO, G, B, S, Q, SC, N = (0x10_0000 * (i + 1) for i in range(9))


def rms(lib, **kw):
    a = dict(x=X, ld_x=256, r=R, ld_r=256, ro=RO, ld_ro=256, g=G, eps=1e-6, ss=None, q=Q, ld_q=256,
             sc=SC, n=None, ld_n=0, M=4, d=256)
    a.update(kw)
    return lib.nq_fused_add_rmsnorm_quant_fp8(a["x"], a["ld_x"], a["r"], a["ld_r"], a["ro"], a["ld_ro"],
                                              a["g"], a["eps"], a["ss"], a["q"], a["ld_q"], a["sc"],
                                              a["n"], a["ld_n"], a["M"], a["d"], None)


def test_rmsnorm_fp8_validation(lib):
    assert rms(lib, M=0) == NQ_OK
    assert rms(lib, M=0, ro=R) == NQ_OK           # exact in-place residual allowed
    assert rms(lib, x=None) == NQ_ERR_NULL
    assert rms(lib, g=None) == NQ_ERR_NULL
    assert rms(lib, q=None) == NQ_ERR_NULL
    assert rms(lib, sc=None) == NQ_ERR_NULL        # dynamic needs scale_out
    assert rms(lib, ro=None) == NQ_ERR_NULL        # residual_in without residual_out
    assert rms(lib, r=None, M=0, ro=None) == NQ_OK  # residual-less
    assert rms(lib, d=0) == NQ_ERR_SHAPE
    assert rms(lib, M=-1) == NQ_ERR_SHAPE
    assert rms(lib, d=32769, ld_x=40000, ld_r=40000, ld_ro=40000, ld_q=40000) == NQ_ERR_SHAPE
    assert rms(lib, ld_x=255) == NQ_ERR_STRIDE
    assert rms(lib, ld_q=100) == NQ_ERR_STRIDE
    assert rms(lib, n=N, ld_n=10) == NQ_ERR_STRIDE
    assert rms(lib, eps=-1.0) == NQ_ERR_ARG
    assert rms(lib, eps=float("nan")) == NQ_ERR_ARG
    # aliasing: outputs over inputs or over each other
    assert rms(lib, q=X + 100) == NQ_ERR_ALIAS
    assert rms(lib, ro=R + 2) == NQ_ERR_ALIAS     # partial overlap of the in-place pair
    assert rms(lib, ro=X) == NQ_ERR_ALIAS         # residual_out over x
    assert rms(lib, sc=Q + 8) == NQ_ERR_ALIAS
    assert rms(lib, n=Q, ld_n=256) == NQ_ERR_ALIAS
    assert rms(lib, q=G) == NQ_ERR_ALIAS


def test_extreme_rows_and_strides_are_checked_without_overflow(lib):
    """At the row limit (2^36 rows) and the stride limit (2^24 elements) the
    host still forms every address range exactly: an overlapping output is
    found (NQ_ERR_ALIAS), one more row is a shape error."""
    big_m, big_ld = 1 << 36, 1 << 24
    assert rms(lib, M=big_m + 1) == NQ_ERR_SHAPE
    assert rms(lib, M=big_m, ld_x=big_ld, ld_r=big_ld, ld_ro=big_ld, ld_q=big_ld, q=X + 100) == NQ_ERR_ALIAS
    assert rms(lib, ld_x=big_ld + 1) == NQ_ERR_STRIDE
    ln = lambda **k: lib.nq_layernorm_quant_fp8(
        X, k.get("ld", 512), G, B, 1e-5, S, k.get("q", Q), k.get("ld", 512), k.get("M", 2), 512, None)
    assert ln(M=big_m + 1) == NQ_ERR_SHAPE
    assert ln(M=big_m, ld=big_ld, q=X + 4096) == NQ_ERR_ALIAS
    fp4 = lambda **k: lib.nq_rmsnorm_quant_nvfp4(
        X, k.get("ld", 2112), None, 0, None, 0, G, 1e-6, S, k.get("q", Q), k.get("ld_q", 768), SC,
        k.get("ld_sf", 96), None, 0, k.get("M", 2), 1536, None)
    assert fp4(M=big_m + 1) == NQ_ERR_SHAPE
    assert fp4(M=big_m, ld=big_ld, ld_q=big_ld, ld_sf=big_ld, q=X + 64) == NQ_ERR_ALIAS
    grp = lambda **k: lib.nq_per_token_group_quant_fp8(
        X, k.get("ld", 4096), k.get("M", 2), 4096, 128, 0, k.get("q", Q), k.get("ld", 4096), SC, None)
    assert grp(M=big_m) == NQ_ERR_SHAPE        # M * K / 128 must stay below 2^31
    assert grp(M=(1 << 31) // 32 - 1, ld=big_ld, q=X + 64) == NQ_ERR_ALIAS


def test_rmsnorm_fp8_group_validation(lib):
    def call(**kw):
        a = dict(x=X, ld_x=2816, r=R, ld_r=2816, ro=RO, ld_ro=2816, g=G, eps=1e-6, gs=128, mode=0,
                 flags=0, q=Q, ld_q=2816, s=SC, ld_s=22, n=None, ld_n=0, M=4, d=2816)
        a.update(kw)
        return lib.nq_fused_add_rmsnorm_quant_fp8_group(
            a["x"], a["ld_x"], a["r"], a["ld_r"], a["ro"], a["ld_ro"], a["g"], a["eps"], a["gs"], a["mode"],
            a["flags"], a["q"], a["ld_q"], a["s"], a["ld_s"], a["n"], a["ld_n"], a["M"], a["d"], None)
    assert call(M=0) == NQ_OK
    assert call(M=0, ro=R, mode=1, flags=1) == NQ_OK
    assert call(gs=64) == NQ_ERR_ARG
    assert call(mode=2) == NQ_ERR_ARG
    assert call(flags=0x100) == NQ_ERR_ARG     # unknown bit
    assert call(eps=-1.0) == NQ_ERR_ARG
    assert call(d=2800, ld_x=2800, ld_r=2800, ld_ro=2800, ld_q=2800) == NQ_ERR_SHAPE  # d % 128
    assert call(ld_s=21) == NQ_ERR_STRIDE
    assert call(ld_q=2815) == NQ_ERR_STRIDE
    assert call(s=None) == NQ_ERR_NULL
    assert call(ro=None) == NQ_ERR_NULL
    assert call(s=Q + 64) == NQ_ERR_ALIAS
    assert call(s=G + 64) == NQ_ERR_ALIAS
    assert call(ro=R + 2) == NQ_ERR_ALIAS
    assert call(d=32896, ld_x=32896, ld_r=32896, ld_ro=32896, ld_q=32896, ld_s=257) == NQ_ERR_SHAPE  # > NQ_MAX_D


def test_layernorm_fp8_validation(lib):
    call = lambda **k: lib.nq_layernorm_quant_fp8(
        k.get("x", X), k.get("ld_x", 512), k.get("g", G), k.get("b", B), k.get("eps", 1e-5),
        k.get("s", S), k.get("q", Q), k.get("ld_q", 512), k.get("M", 2), k.get("d", 512), None)
    assert call(M=0) == NQ_OK
    assert call(s=None) == NQ_ERR_NULL
    assert call(b=None) == NQ_ERR_NULL
    assert call(ld_x=511) == NQ_ERR_STRIDE
    assert call(q=X) == NQ_ERR_ALIAS
    assert call(q=S) == NQ_ERR_ALIAS
    assert call(d=-3) == NQ_ERR_SHAPE
    assert call(d=32776, ld_x=32776, ld_q=32776) == NQ_ERR_SHAPE  # > NQ_MAX_D


def test_group_fp8_validation(lib):
    call = lambda **k: lib.nq_per_token_group_quant_fp8(
        k.get("x", X), k.get("ld_x", 4096), k.get("M", 2), k.get("K", 4096), k.get("g", 128),
        k.get("mode", 0), k.get("q", Q), k.get("ld_q", 4096), k.get("s", SC), None)
    assert call(M=0) == NQ_OK
    assert call(M=0, mode=1) == NQ_OK
    assert call(g=64) == NQ_ERR_ARG
    assert call(mode=2) == NQ_ERR_ARG
    assert call(K=4000, ld_x=4000, ld_q=4000) == NQ_ERR_SHAPE
    assert call(ld_q=4095) == NQ_ERR_STRIDE
    assert call(s=None) == NQ_ERR_NULL
    assert call(s=X + 64) == NQ_ERR_ALIAS


def test_ex_entry_points_validation(lib):
    """The format-flag forms: unknown bits are rejected, the dynamic LayerNorm
    needs scale_out, and aliasing / NULL checks apply as in the base forms."""
    rms = lambda **k: lib.nq_fused_add_rmsnorm_quant_fp8_ex(
        X, 256, R, 256, RO, 256, G, 1e-6, k.get("ss", None), k.get("flags", 0), k.get("q", Q), 256,
        k.get("sc", SC), None, 0, k.get("M", 4), 256, None)
    assert rms(M=0, flags=2) == NQ_OK
    assert rms(flags=1) == NQ_ERR_ARG          # the bf16-source bit is not an option here
    assert rms(flags=0x102) == NQ_ERR_ARG       # unknown bit
    assert rms(flags=2, sc=None) == NQ_ERR_NULL
    assert rms(flags=2, q=X) == NQ_ERR_ALIAS
    ln = lambda **k: lib.nq_layernorm_quant_fp8_ex(
        X, 512, G, B, 1e-5, k.get("s", None), k.get("flags", 0), k.get("q", Q), 512, k.get("so", SC),
        k.get("M", 2), 512, None)
    assert ln(M=0) == NQ_OK
    assert ln(M=0, flags=2, s=S) == NQ_OK
    assert ln(flags=0x100) == NQ_ERR_ARG
    assert ln(so=None) == NQ_ERR_NULL          # dynamic without scale_out
    assert ln(so=Q + 16) == NQ_ERR_ALIAS       # scale_out over the codes
    assert ln(so=G + 4) == NQ_ERR_ALIAS        # scale_out over gamma
    assert ln(s=S, so=None, q=X) == NQ_ERR_ALIAS
    # the static base form still requires its scale
    assert lib.nq_layernorm_quant_fp8(X, 512, G, B, 1e-5, None, Q, 512, 2, 512, None) == NQ_ERR_NULL
    grp = lambda **k: lib.nq_per_token_group_quant_fp8_ex(
        X, 4096, k.get("M", 2), 4096, 128, k.get("mode", 0), k.get("flags", 0), Q, 4096, k.get("s", SC), None)
    assert grp(M=0, flags=2, mode=1) == NQ_OK
    assert grp(flags=1) == NQ_ERR_ARG
    assert grp(flags=2, s=None) == NQ_ERR_NULL
    assert grp(flags=2, s=X + 64) == NQ_ERR_ALIAS


def test_unfused_pair_and_nvfp4_ex_validation(lib):
    norm = lambda **k: lib.nq_fused_add_rmsnorm_bf16(
        X, 256, k.get("r", R), 256, k.get("ro", RO), 256, G, k.get("eps", 1e-6), k.get("o", N),
        k.get("ld_o", 256), k.get("M", 4), 256, None)
    assert norm(M=0) == NQ_OK
    assert norm(o=None) == NQ_ERR_NULL
    assert norm(ro=None) == NQ_ERR_NULL
    assert norm(ld_o=255) == NQ_ERR_STRIDE
    assert norm(eps=-1.0) == NQ_ERR_ARG
    assert norm(o=X + 2) == NQ_ERR_ALIAS
    assert norm(o=RO + 64) == NQ_ERR_ALIAS
    assert lib.nq_fused_add_rmsnorm_bf16(X, 32776, R, 32776, RO, 32776, G, 1e-6, N, 32776, 4, 32776,
                                         None) == NQ_ERR_SHAPE  # > NQ_MAX_D
    quant = lambda **k: lib.nq_per_token_quant_fp8(
        k.get("x", X), 256, k.get("ss", None), k.get("flags", 0), k.get("q", Q), k.get("ld_q", 256),
        k.get("sc", SC), k.get("M", 4), 256, None)
    assert quant(M=0, flags=2) == NQ_OK
    assert quant(flags=1) == NQ_ERR_ARG
    assert quant(sc=None) == NQ_ERR_NULL
    assert quant(ss=S, sc=None, M=0) == NQ_OK
    assert quant(ld_q=100) == NQ_ERR_STRIDE
    assert quant(q=X + 16) == NQ_ERR_ALIAS
    assert quant(sc=Q + 8) == NQ_ERR_ALIAS
    assert lib.nq_per_token_quant_fp8(X, 32776, None, 0, Q, 32776, SC, 4, 32776, None) == NQ_ERR_SHAPE
    fp4 = lambda **k: lib.nq_rmsnorm_quant_nvfp4_ex(
        X, 2112, None, 0, None, 0, G, 1e-6, S, k.get("flags", 0), Q, 768, SC, 96, None, 0, k.get("M", 2),
        1536, None)
    assert fp4(M=0, flags=1) == NQ_OK
    assert fp4(flags=2) == NQ_ERR_ARG          # no e5m2 form of NVFP4


def test_nvfp4_validation(lib):
    call = lambda **k: lib.nq_rmsnorm_quant_nvfp4(
        k.get("x", X), k.get("ld_x", 2112), k.get("r", None), k.get("ld_r", 0), k.get("ro", None),
        k.get("ld_ro", 0), k.get("g", G), 1e-6, k.get("gs", S), k.get("q", Q), k.get("ld_q", 768),
        k.get("sf", SC), k.get("ld_sf", 96), k.get("n", None), k.get("ld_n", 0), k.get("M", 2),
        k.get("d", 1536), None)
    assert call(M=0) == NQ_OK                      # residual-less column slice
    assert call(d=1544, ld_q=772, ld_sf=97) == NQ_ERR_SHAPE   # d % 16
    assert call(d=32784, ld_x=32784, ld_q=16392, ld_sf=2049) == NQ_ERR_SHAPE  # > NQ_MAX_D
    assert call(gs=None) == NQ_ERR_NULL
    assert call(sf=None) == NQ_ERR_NULL
    assert call(r=R, ld_r=1536, ld_ro=1536) == NQ_ERR_NULL   # residual_in without residual_out
    assert call(r=R) == NQ_ERR_STRIDE
    assert call(ld_q=700) == NQ_ERR_STRIDE
    assert call(ld_sf=95) == NQ_ERR_STRIDE
    assert call(sf=Q + 10) == NQ_ERR_ALIAS
    # the output may not be placed in the unread columns of x's own rows:
    # overlap is decided on address ranges
    assert call(q=X + 2 * 1536) == NQ_ERR_ALIAS


def test_diag_validation(lib):
    assert lib.nq_diag_codec(7, X, Q, 16, None) == NQ_ERR_ARG
    assert lib.nq_diag_codec(0, X, Q, 0, None) == NQ_OK
    assert lib.nq_diag_codec(0, X, X + 4, 16, None) == NQ_ERR_ALIAS
    assert lib.nq_diag_copy(X, Q, 15, None) == NQ_ERR_SHAPE
    assert lib.nq_diag_copy(X + 4, Q, 16, None) == NQ_ERR_ARG
    assert lib.nq_diag_copy(X, Q, 0, None) == NQ_OK
    assert lib.nq_diag_arith(8, X, None, Q, 16, None) == NQ_ERR_ARG
    assert lib.nq_diag_arith(6, X + 100, None, X, 16, None) == NQ_ERR_ALIAS  # out holds 2n floats: [X, X+128)
    assert lib.nq_diag_arith(7, X + 100, None, X, 16, None) == NQ_ERR_ALIAS
    assert lib.nq_diag_arith(5, X, None, Q, 16, None) == NQ_ERR_NULL   # the packed sum needs b
    assert lib.nq_diag_arith(-1, X, None, Q, 16, None) == NQ_ERR_ARG
    assert lib.nq_diag_arith(0, X, None, Q, -1, None) == NQ_ERR_SHAPE
    assert lib.nq_diag_arith(0, X, None, Q, 0, None) == NQ_OK
    assert lib.nq_diag_arith(2, X, None, Q, 16, None) == NQ_ERR_NULL   # division needs b
    assert lib.nq_diag_arith(0, None, None, Q, 16, None) == NQ_ERR_NULL
    assert lib.nq_diag_arith(0, X, None, X + 60, 16, None) == NQ_ERR_ALIAS
    assert lib.nq_diag_arith(3, X, Q, Q + 32, 16, None) == NQ_ERR_ALIAS  # int32 b [Q, Q+64), double out
    assert lib.nq_diag_arith(3, X + 64, Q, X, 16, None) == NQ_ERR_ALIAS  # double a [X+64, X+192)


def test_binding_imports_without_gpu():
    import fp4_quantization_amd.nq as nq
    assert "gfx950" in nq.nq_version()
    assert nq.nq_status_string(-4).startswith("an output overlaps")


def test_binding_constants_match_the_header():
    """The Python binding's NQ_* constants are the header's values, and every
    scale mode, flag, codec and the row-width limit is exported."""
    import fp4_quantization_amd.nq as nq
    text = open(HEADER).read()
    defs = {k: int(v) for k, v in re.findall(r"^#define (NQ_[A-Z0-9_]+) \(?(-?\d+)u?\)?", text, re.M)}
    needed = [k for k in defs if k.startswith(("NQ_SCALE_", "NQ_FLAG_", "NQ_CODEC_", "NQ_ARITH_"))
              or k == "NQ_MAX_D"]
    assert len(needed) >= 9
    for k in needed:
        assert getattr(nq, k) == defs[k], k
    for k, v in defs.items():
        if hasattr(nq, k):
            assert getattr(nq, k) == v, k


# ---------------------------------------------------- alias detection ------
# The host rejects an output that overlaps an input or another output
# (NQ_ERR_ALIAS), except residual_out == residual_in exactly.  Random
# placements of every tensor of the per-token entry point in a small fake
# address space are checked against an independent interval model: with
# every other argument valid, the call must be refused as aliased exactly
# when the model finds a forbidden overlap, and otherwise pass validation
# (then the launch fails on a machine without a GPU: NQ_ERR_LAUNCH).

NQ_ERR_LAUNCH = -5


def _span(p, rows, ld, cols, esize):
    return None if p is None else (p, p + ((rows - 1) * ld + cols) * esize)


def _overlap(a, b):
    return a is not None and b is not None and a[0] < b[1] and b[0] < a[1]


def test_alias_detection_matches_an_interval_model(lib):
    hyp = pytest.importorskip("hypothesis")
    st = pytest.importorskip("hypothesis.strategies")
    base = 0x200000

    @hyp.settings(max_examples=1500, deadline=None, derandomize=True)
    @hyp.given(M=st.integers(1, 3), d=st.integers(1, 40), pads=st.lists(st.integers(0, 6), min_size=5, max_size=5),
               offs=st.lists(st.integers(0, 300), min_size=8, max_size=8), residual=st.sampled_from(["none", "fresh", "inplace"]),
               static=st.booleans(), with_norm=st.booleans())
    def check(M, d, pads, offs, residual, static, with_norm):
        ldx, ldr, ldro, ldq, ldn = (d + p for p in pads)
        x, r, ro, g, q, s, n, ss = (base + 2 * o for o in offs)
        if residual == "none":
            r = ro = None
        elif residual == "inplace":
            ro, ldro = r, ldr
        if not static:
            ss = None
        if not with_norm:
            n = None
        ins = [_span(x, M, ldx, d, 2), _span(r, M, ldr, d, 2), _span(g, 1, d, d, 4), _span(ss, 1, 1, 1, 4)]
        outs = [_span(ro, M, ldro, d, 2), _span(q, M, ldq, d, 1), None if static else _span(s, 1, M, M, 4),
                _span(n, M, ldn, d, 2)]
        bad = any(_overlap(o, i) and not (ii == 1 and oi == 0 and o == i)
                  for oi, o in enumerate(outs) for ii, i in enumerate(ins))
        bad = bad or any(_overlap(outs[a], outs[b]) for a in range(4) for b in range(a + 1, 4))
        got = lib.nq_fused_add_rmsnorm_quant_fp8(x, ldx, r, ldr, ro, ldro, g, 1e-6, ss, q, ldq, s, n, ldn, M, d, None)
        assert got == (NQ_ERR_ALIAS if bad else NQ_ERR_LAUNCH), (M, d, pads, offs, residual, static, with_norm, got)

    check()


def _expect(ins, outs, exact=None):
    """NQ_ERR_ALIAS when an output overlaps an input (other than the exact
    pair `exact` = (input index, output index) coinciding) or another output."""
    bad = any(_overlap(o, i) and not (exact == (ii, oi) and o == i)
              for oi, o in enumerate(outs) for ii, i in enumerate(ins))
    bad = bad or any(_overlap(outs[a], outs[b]) for a in range(len(outs)) for b in range(a + 1, len(outs)))
    return NQ_ERR_ALIAS if bad else NQ_ERR_LAUNCH


def test_alias_detection_other_entry_points(lib):
    """The same interval model for the fused group, NVFP4 and LayerNorm entry
    points (a column-slice input's unread columns count as part of its range)."""
    hyp = pytest.importorskip("hypothesis")
    st = pytest.importorskip("hypothesis.strategies")
    base = 0x300000
    offs_s = st.lists(st.integers(0, 400), min_size=8, max_size=8)
    pads_s = st.lists(st.integers(0, 6), min_size=6, max_size=6)
    res_s = st.sampled_from(["none", "fresh", "inplace"])

    def residual_ptrs(mode, r, ro, ldr, ldro):
        if mode == "none":
            return None, None, ldr, ldro
        if mode == "inplace":
            return r, r, ldr, ldr
        return r, ro, ldr, ldro

    @hyp.settings(max_examples=600, deadline=None, derandomize=True)
    @hyp.given(M=st.integers(1, 3), gsel=st.integers(1, 2), pads=pads_s, offs=offs_s, mode=res_s,
               with_norm=st.booleans())
    def group(M, gsel, pads, offs, mode, with_norm):
        d, G = 128 * gsel, gsel
        ldx, ldr, ldro, ldq, lds, ldn = d + pads[0], d + pads[1], d + pads[2], d + pads[3], G + pads[4], d + pads[5]
        x, r, ro, g, q, s, n, _ = (base + 4 * o for o in offs)
        r, ro, ldr, ldro = residual_ptrs(mode, r, ro, ldr, ldro)
        n = n if with_norm else None
        ins = [_span(x, M, ldx, d, 2), _span(r, M, ldr, d, 2), _span(g, 1, d, d, 4)]
        outs = [_span(ro, M, ldro, d, 2), _span(q, M, ldq, d, 1), _span(s, M, lds, G, 4), _span(n, M, ldn, d, 2)]
        got = lib.nq_fused_add_rmsnorm_quant_fp8_group(x, ldx, r, ldr, ro, ldro, g, 1e-6, 128, 0, 0, q, ldq, s,
                                                       lds, n, ldn, M, d, None)
        assert got == _expect(ins, outs, (1, 0)), ("group", M, d, pads, offs, mode, with_norm, got)

    @hyp.settings(max_examples=600, deadline=None, derandomize=True)
    @hyp.given(M=st.integers(1, 3), dsel=st.integers(1, 4), pads=pads_s, offs=offs_s, mode=res_s,
               with_norm=st.booleans())
    def nvfp4(M, dsel, pads, offs, mode, with_norm):
        d = 16 * dsel
        ldx, ldr, ldro, ldq, ldsf, ldn = d + pads[0], d + pads[1], d + pads[2], d // 2 + pads[3], d // 16 + pads[4], d + pads[5]
        x, r, ro, g, gs, q, sf, n = (base + 2 * o for o in offs)
        r, ro, ldr, ldro = residual_ptrs(mode, r, ro, ldr, ldro)
        n = n if with_norm else None
        ins = [_span(x, M, ldx, d, 2), _span(r, M, ldr, d, 2), _span(g, 1, d, d, 4), _span(gs, 1, 1, 1, 4)]
        outs = [_span(ro, M, ldro, d, 2), _span(q, M, ldq, d // 2, 1), _span(sf, M, ldsf, d // 16, 1),
                _span(n, M, ldn, d, 2)]
        got = lib.nq_rmsnorm_quant_nvfp4(x, ldx, r, ldr, ro, ldro, g, 1e-6, gs, q, ldq, sf, ldsf, n, ldn, M, d, None)
        assert got == _expect(ins, outs, (1, 0)), ("nvfp4", M, d, pads, offs, mode, with_norm, got)

    @hyp.settings(max_examples=600, deadline=None, derandomize=True)
    @hyp.given(M=st.integers(1, 3), d=st.integers(1, 40), pads=pads_s, offs=offs_s, static=st.booleans())
    def layernorm(M, d, pads, offs, static):
        ldx, ldq = d + pads[0], d + pads[1]
        x, g, b, sc, q, so, _, _ = (base + 2 * o for o in offs)
        sc = sc if static else None
        ins = [_span(x, M, ldx, d, 2), _span(g, 1, d, d, 4), _span(b, 1, d, d, 4), _span(sc, 1, 1, 1, 4)]
        outs = [_span(q, M, ldq, d, 1), None if static else _span(so, 1, M, M, 4)]
        got = lib.nq_layernorm_quant_fp8_ex(x, ldx, g, b, 1e-5, sc, 0, q, ldq, so, M, d, None)
        assert got == _expect(ins, outs), ("layernorm", M, d, pads, offs, static, got)

    group()
    nvfp4()
    layernorm()
