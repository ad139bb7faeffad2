// nq_unfused.hip -- the two-kernel pipeline the fusion replaces, for gfx950:
// (1) residual-add + RMSNorm writing the normalized rows as bf16, then
// (2) FP8 quantization of bf16 rows with per-token (or static) scales.
//
// Pages: [FUSE] "Fusing RMSNorm and FP8 Quantization Under torch.compile"
// ("TL;DR", "Where norm+quant sits": the norm stores a bf16 activation that
// a separate quantization kernel loads again for its maximum and its codes --
// one more HBM round trip and one more rounding); [LNQ] "feat: fused FP8
// quantization output for LayerNorm" ("Description": roughly 7 bytes move
// per element in two kernels, 3 in one).  Run back to back they give the codes of
// the unfused reference and the time the fusion saves on this GPU.
//
// Both are row kernels on the same team layout as the fused ones: (1) is the
// fused kernel's front half with a bf16 store in place of the quantizer;
// (2) holds the bf16 row in registers across its one row reduction (the
// absolute maximum) and divides once per element.
#include "nq_device.hpp"
#include "nq_host.hpp"
#include "nq_rms_front.hpp"
#include "nq_rows.hpp"

namespace nq {

struct RmsBf16Args {
    const uint16_t* x;
    const uint16_t* r;      // NULL: residual-less
    uint16_t* ro;           // NULL iff r is NULL
    const float* gamma;
    uint16_t* out;          // bf16(y)
    int64_t ld_x, ld_r, ld_ro, ld_o;
    int64_t M;
    int d;
    float eps;
    double inv_d;           // RN(1 / d), formed on the host
};

template <int TEAM, int CPL, bool VEC, bool STAGE, bool RES = true, int BLOCK = row_block<TEAM, CPL, 1, VEC, STAGE>()>
__global__ __launch_bounds__(BLOCK) void k_add_rmsnorm_bf16(RmsBf16Args a)
{
    using S = TeamShape<TEAM, BLOCK>;
    __shared__ double lds_sum[S::kWaves];

    const int t = threadIdx.x % TEAM;
    const RowMap m = row_map<TEAM, BLOCK>(a.M);
    const int d = a.d;
    using SV = SharedVectors<TEAM, CPL, VEC, 1, BLOCK, STAGE>;
    __shared__ typename SV::Lds lds_gamma;
    SV gamma({a.gamma}, d);

    uint4 zw[CPL];
    const float rstd = rms_front<TEAM, CPL, VEC, RES>(a.x, a.ld_x, a.r, a.ld_r, a.ro, a.ld_ro, m, t, d, a.inv_d,
                                                      a.eps, gamma, lds_gamma, lds_sum, zw);

    const RowIO<VEC, kStoreRows, uint16_t> oio(a.out, a.ld_o, m, d);
    const int t1 = opaque(t);
#pragma unroll
    for (int j = 0; j < CPL; ++j) opaque(zw[j]);
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
        const int e = (j * TEAM + t1) * 8;
        float g[8], z[8], y[8];
        gamma.chunk(lds_gamma, 0, j, e, g);
        unpack_bf16x8(zw[j], z);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const float n = z[k] * rstd;
            y[k] = n * g[k];
        }
        oio.store16(e, col_live<TEAM, VEC>(e, d), make_uint4(pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]),
                                         pack_bf16x2(y[4], y[5]), pack_bf16x2(y[6], y[7])));
    }
}

template <int TEAM, int CPL, bool VEC>
struct RmsBf16Kernel {
    template <bool STAGE>
    static constexpr int block() { return row_block<TEAM, CPL, 1, VEC, STAGE>(); }
    template <bool STAGE>
    static void launch(const RmsBf16Args& a, dim3 grid, dim3 block, hipStream_t s)
    {
        if (a.r != nullptr) hipLaunchKernelGGL((k_add_rmsnorm_bf16<TEAM, CPL, VEC, STAGE, true>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((k_add_rmsnorm_bf16<TEAM, CPL, VEC, STAGE, false>), grid, block, 0, s, a);
    }
};

struct QuantRowsArgs {
    const uint16_t* x;
    const float* static_scale;  // NULL: dynamic per-token
    uint8_t* q;
    float* scale_out;
    int64_t ld_x, ld_q;
    int64_t M;
    int d;
    bool e5m2;
};

template <int TEAM, int CPL, bool VEC, Fp8 F>
__global__ __launch_bounds__(default_block<TEAM>()) void k_quant_fp8_rows(QuantRowsArgs a)
{
    using S = TeamShape<TEAM>;
    __shared__ float lds_max[S::kWaves];

    const int t = threadIdx.x % TEAM;
    const RowMap m = row_map<TEAM>(a.M);
    const int d = a.d;
    const RowIO<VEC, kLoadStream, uint16_t> xio(a.x, a.ld_x, m, d);
    const RowIO<VEC, kStoreCodes, uint8_t> qio(a.q, a.ld_q, m, d);
    const bool is_static = a.static_scale != nullptr;
    const float scale = is_static ? a.static_scale[0] : 1.0f;

    uint4 xw[CPL];
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
        const int e = (j * TEAM + t) * 8;
        xw[j] = xio.load16(e, col_live<TEAM, VEC>(e, d));  // zeros past the row end
    }

    if (is_static) {
        const float inv = 1.0f / scale;
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            const int e = (j * TEAM + t) * 8;
            float v[8];
            unpack_bf16x8(xw[j], v);
#pragma unroll
            for (int k = 0; k < 8; ++k) v[k] = v[k] * inv;
            qio.store8(e, col_live<TEAM, VEC>(e, d), fp8x8<F>(v));
        }
    } else {
        float amax = 0.0f;
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            float v[8];
            unpack_bf16x8(xw[j], v);
#pragma unroll
            for (int k = 0; k < 8; ++k) amax = fmaxf(amax, fabsf(v[k]));
        }
        amax = team_max<TEAM>(amax, lds_max);
        float s, inv;
        token_scale<F>(amax, s, inv);
        if (t == 0 && m.ok) a.scale_out[m.row] = s;
        // A zero scale (an all-zero row) stores +0 codes, -0 inputs included;
        // the select runs only in a wavefront that holds such a row.
        const bool zero_scales = __builtin_amdgcn_ballot_w64(!(s > 0.0f)) != 0;
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            const int e = (j * TEAM + t) * 8;
            float v[8];
            unpack_bf16x8(xw[j], v);
#pragma unroll
            for (int k = 0; k < 8; ++k) v[k] = div_by(v[k], s, inv);
            if (zero_scales) {
                __asm__ volatile("");  // keep it a branch
#pragma unroll
                for (int k = 0; k < 8; ++k) v[k] = s > 0.0f ? v[k] : 0.0f;
            }
            qio.store8(e, col_live<TEAM, VEC>(e, d), fp8x8<F>(v));
        }
    }
}

template <int TEAM, int CPL, bool VEC>
struct QuantRowsKernel {
    template <bool STAGE>
    static constexpr int block() { return default_block<TEAM>(); }
    template <bool STAGE>
    static void launch(const QuantRowsArgs& a, dim3 grid, dim3 block, hipStream_t s)
    {
        if (a.e5m2) hipLaunchKernelGGL((k_quant_fp8_rows<TEAM, CPL, VEC, Fp8::E5M2>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((k_quant_fp8_rows<TEAM, CPL, VEC, Fp8::E4M3>), grid, block, 0, s, a);
    }
};

} // namespace nq

using namespace nq;

extern "C" nq_status nq_fused_add_rmsnorm_bf16(
    const uint16_t* x, int64_t ld_x,
    const uint16_t* residual_in, int64_t ld_r,
    uint16_t* residual_out, int64_t ld_ro,
    const float* gamma, float eps,
    uint16_t* out, int64_t ld_o,
    int64_t M, int64_t d, void* stream)
{
    if (M < 0 || d <= 0 || d > NQ_MAX_D || M > kMaxRows) return NQ_ERR_SHAPE;
    if (!(eps >= 0.0f) || eps > 1e30f) return NQ_ERR_ARG;
    if (bad_ld(ld_x, d) || bad_ld(ld_o, d)) return NQ_ERR_STRIDE;
    if (residual_in && (bad_ld(ld_r, d) || bad_ld(ld_ro, d))) return NQ_ERR_STRIDE;
    if (M == 0) return NQ_OK;  // empty tensors may carry NULL data pointers
    if (!x || !gamma || !out) return NQ_ERR_NULL;
    if ((residual_in == nullptr) != (residual_out == nullptr)) return NQ_ERR_NULL;

    const Region in[] = {region(x, M, ld_x, d, 2), region(residual_in, M, ld_r, d, 2),
                         region(gamma, 1, d, d, 4)};
    const Region out_[] = {region(residual_out, M, ld_ro, d, 2), region(out, M, ld_o, d, 2)};
    if (any_alias(in, out_, /*exact_in=*/1, /*exact_out=*/0)) return NQ_ERR_ALIAS;

    const RowShape shape = pick_row_shape(M, d, vector_rows(d, gamma));
    if (shape.team == 0) return NQ_ERR_SHAPE;

    RmsBf16Args a;
    a.x = x; a.r = residual_in; a.ro = residual_out; a.gamma = gamma; a.out = out;
    a.ld_x = ld_x; a.ld_r = ld_r; a.ld_ro = ld_ro; a.ld_o = ld_o;
    a.M = M; a.d = (int)d; a.eps = eps; a.inv_d = 1.0 / (double)d;
    if (!launch_row_shape<RmsBf16Kernel>(shape, a, M, (hipStream_t)stream)) return NQ_ERR_SHAPE;
    return hipGetLastError() == hipSuccess ? NQ_OK : NQ_ERR_LAUNCH;
}

extern "C" nq_status nq_per_token_quant_fp8(
    const uint16_t* x, int64_t ld_x,
    const float* static_scale, uint32_t flags,
    uint8_t* q_out, int64_t ld_q,
    float* scale_out,
    int64_t M, int64_t d, void* stream)
{
    if ((flags & ~(uint32_t)NQ_FLAG_E5M2) != 0) return NQ_ERR_ARG;
    if (M < 0 || d <= 0 || d > NQ_MAX_D || M > kMaxRows) return NQ_ERR_SHAPE;
    if (bad_ld(ld_x, d) || bad_ld(ld_q, d)) return NQ_ERR_STRIDE;
    if (M == 0) return NQ_OK;  // empty tensors may carry NULL data pointers
    if (!x || !q_out) return NQ_ERR_NULL;
    if (!static_scale && !scale_out) return NQ_ERR_NULL;

    const Region in[] = {region(x, M, ld_x, d, 2), region(static_scale, 1, 1, 1, 4)};
    const Region out[] = {region(q_out, M, ld_q, d, 1), region(static_scale ? nullptr : scale_out, 1, M, M, 4)};
    if (any_alias(in, out)) return NQ_ERR_ALIAS;

    RowShape shape = pick_row_shape(M, d, vector_rows(d, nullptr));
    if (shape.team == 0) return NQ_ERR_SHAPE;
    shape.stage = false;  // no shared vectors

    QuantRowsArgs a;
    a.x = x; a.static_scale = static_scale; a.q = q_out; a.scale_out = static_scale ? nullptr : scale_out;
    a.ld_x = ld_x; a.ld_q = ld_q; a.M = M; a.d = (int)d;
    a.e5m2 = (flags & NQ_FLAG_E5M2) != 0;
    if (!launch_row_shape<QuantRowsKernel>(shape, a, M, (hipStream_t)stream)) return NQ_ERR_SHAPE;
    return hipGetLastError() == hipSuccess ? NQ_OK : NQ_ERR_LAUNCH;
}
