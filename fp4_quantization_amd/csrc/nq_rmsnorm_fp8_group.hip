// nq_rmsnorm_fp8_group.hip -- fused (residual-add +) RMSNorm + per-token-
// group FP8 e4m3 (groups of 128, one reciprocal per group) for gfx950.
//
// Pages: [GRP] "per_token_group_quant_8bit: multiply by reciprocal instead of
// dividing per element" ("Details": the fused RMSNorm + group-quant kernel,
// the fusion target for block-FP8 models, uses the standalone group
// quantizer's reciprocal-multiply numerics; one correctly rounded division
// per group); [FUSE] "Fusing RMSNorm and FP8 Quantization Under
// torch.compile" (the norm output stays in fp32 registers and is quantized
// in the same pass).
//
// The front half (loads, z = bf16(x + r), residual write-back, rstd) is the
// per-token kernel's.  The epilogue needs no second row reduction: a group
// of 128 contiguous elements is chunk j of the 16 lanes of one DPP row
// (chunk j of lane t covers elements (j*TEAM + t)*8 .. +7, TEAM and the
// DPP row both 16-aligned), so the group maximum is four DPP steps and each
// chunk is normalized, scaled, quantized and stored as it is produced.
#include "nq_device.hpp"
#include "nq_host.hpp"
#include "nq_rms_front.hpp"
#include "nq_rows.hpp"

namespace nq {

constexpr int kRowGroup = 128;  // elements per scale: 16 lanes x 8

struct RmsGroupArgs {
    const uint16_t* x;
    const uint16_t* r;      // NULL: residual-less
    uint16_t* ro;           // NULL iff r is NULL
    const void* gamma;      // fp32, or bf16 when gamma_bf16
    uint8_t* q;
    float* scale_out;       // [M, d / 128], row stride ld_s
    uint16_t* norm_out;     // optional
    int64_t ld_x, ld_r, ld_ro, ld_q, ld_s, ld_n;
    int64_t M;
    uint16_t d;             // row length, at most NQ_MAX_D
    uint8_t ue8m0;          // scales rounded up to powers of two
    uint8_t bf16_source;    // quantize bf16(y) (the unfused pipeline's values)
    float eps;
    double inv_d;           // RN(1 / d), formed on the host
};
// Two 64-byte lines of the kernel-argument segment (a third costs a
// single-row call about 70 ns on MI355X), hence the 16-bit row length.
static_assert(sizeof(RmsGroupArgs) <= 128, "kernel arguments fit two 64-byte lines");
static_assert(NQ_MAX_D <= 0xFFFF, "the row length fits its 16-bit field");

// Host-side launch request: the kernel arguments and the instance choices.
struct RmsGroupLaunch {
    RmsGroupArgs k;
    bool e5m2;              // output format (e4m3 otherwise)
    bool gamma_bf16;
};

template <int TEAM, int CPL, bool VEC, bool STAGE, Fp8 F = Fp8::E4M3, bool GB = false, bool RES = true,
          int BLOCK = row_block<TEAM, CPL, 1, VEC, STAGE>()>
__global__ __launch_bounds__(BLOCK) void k_add_rmsnorm_fp8_group(RmsGroupArgs a)
{
    static_assert(TEAM % 16 == 0, "a group is one 16-lane DPP row");
    using S = TeamShape<TEAM, BLOCK>;
    __shared__ double lds_sum[S::kWaves];

    const int t = threadIdx.x % TEAM;
    const RowMap m = row_map<TEAM, BLOCK>(a.M);
    const int d = a.d;
    using SV = SharedVectors<TEAM, CPL, VEC, 1, BLOCK, STAGE, GB>;
    __shared__ typename SV::Lds lds_gamma;
    SV gamma({a.gamma}, d);

    uint4 zw[CPL];
    const float rstd = rms_front<TEAM, CPL, VEC, RES>(a.x, a.ld_x, a.r, a.ld_r, a.ro, a.ld_ro, m, t, d, a.inv_d,
                                                      a.eps, gamma, lds_gamma, lds_sum, zw);

    const RowIO<VEC, kStoreRows, uint16_t> nio(a.norm_out, a.ld_n, m, d);
    const RowIO<VEC, kStoreCodes, uint8_t> qio(a.q, a.ld_q, m, d);
    const RowIO<VEC, kStoreScales, float> sio(a.scale_out, a.ld_s, m, d / kRowGroup);
    const int t1 = opaque(t);
    const bool ue8m0 = a.ue8m0 != 0;
    float sc[CPL];  // this lane's group scale of each chunk
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
        if (a.bf16_source || a.norm_out) {
            const uint4 nw = make_uint4(pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]),
                                        pack_bf16x2(y[4], y[5]), pack_bf16x2(y[6], y[7]));
            nio.store16(e, col_live<TEAM, VEC>(e, d), nw);  // dropped when norm_out is NULL
            if (a.bf16_source) unpack_bf16x8(nw, y);
        }
        float amax = 0.0f;
#pragma unroll
        for (int k = 0; k < 8; ++k) amax = fmaxf(amax, fabsf(y[k]));
        // The group's 16 lanes: every lane of the DPP row gets its maximum.
        amax = max16_dpp(amax);
        const float s0 = amax / fp8_max<F>();
        const float s = ue8m0 ? pow2_ceil(s0) : s0;
        const float inv = s > 0.0f ? 1.0f / s : 0.0f;
        float v[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = y[k] * inv;
        qio.store8(e, col_live<TEAM, VEC>(e, d), fp8x8<F>(v));
        sc[j] = s;
    }
    // Every lane of a DPP row holds its group's scale for each chunk, so lane
    // t = 16q + j stores chunk j's scale: one store instruction per
    // wavefront carries all of its groups' scales.
    const int sel = t1 & 15;
    float mine = sc[0];
#pragma unroll
    for (int j = 1; j < CPL; ++j) mine = sel == j ? sc[j] : mine;
    const int es = (sel * TEAM + t1 - sel) * 8;  // first element of chunk sel's group
    sio.store4(es / kRowGroup, sel < CPL && es < d, __float_as_uint(mine));
}

template <int TEAM, int CPL, bool VEC>
struct RmsGroupKernel {
    template <bool STAGE>
    static constexpr int block() { return row_block<TEAM, CPL, 1, VEC, STAGE>(); }
    template <bool STAGE>
    static void launch(const RmsGroupLaunch& a, dim3 grid, dim3 block, hipStream_t s)
    {
        if (a.k.r != nullptr) go<STAGE, true>(a, grid, block, s);
        else go<STAGE, false>(a, grid, block, s);
    }
    template <bool STAGE, bool RES>
    static void go(const RmsGroupLaunch& a, dim3 grid, dim3 block, hipStream_t s)
    {
        if (a.gamma_bf16) {
            if (a.e5m2) hipLaunchKernelGGL((k_add_rmsnorm_fp8_group<TEAM, CPL, VEC, STAGE, Fp8::E5M2, true, RES>), grid, block, 0, s, a.k);
            else hipLaunchKernelGGL((k_add_rmsnorm_fp8_group<TEAM, CPL, VEC, STAGE, Fp8::E4M3, true, RES>), grid, block, 0, s, a.k);
        } else {
            if (a.e5m2) hipLaunchKernelGGL((k_add_rmsnorm_fp8_group<TEAM, CPL, VEC, STAGE, Fp8::E5M2, false, RES>), grid, block, 0, s, a.k);
            else hipLaunchKernelGGL((k_add_rmsnorm_fp8_group<TEAM, CPL, VEC, STAGE, Fp8::E4M3, false, RES>), grid, block, 0, s, a.k);
        }
    }
};

} // namespace nq

using namespace nq;

extern "C" nq_status nq_fused_add_rmsnorm_quant_fp8_group(
    const uint16_t* x, int64_t ld_x,
    const uint16_t* residual_in, int64_t ld_r,
    uint16_t* residual_out, int64_t ld_ro,
    const void* gamma, float eps,
    int32_t group_size, int32_t scale_mode, uint32_t flags,
    uint8_t* q_out, int64_t ld_q,
    float* scale_out, int64_t ld_s,
    uint16_t* norm_out, int64_t ld_n,
    int64_t M, int64_t d, void* stream)
{
    if (group_size != kRowGroup) return NQ_ERR_ARG;
    if (scale_mode != NQ_SCALE_FP32 && scale_mode != NQ_SCALE_UE8M0) return NQ_ERR_ARG;
    if ((flags & ~(uint32_t)(NQ_FLAG_BF16_SOURCE | NQ_FLAG_E5M2 | NQ_FLAG_GAMMA_BF16)) != 0) return NQ_ERR_ARG;
    const int64_t gsz = (flags & NQ_FLAG_GAMMA_BF16) ? 2 : 4;
    if (M < 0 || d <= 0 || d > NQ_MAX_D || d % group_size != 0 || M > kMaxRows) return NQ_ERR_SHAPE;
    if (!(eps >= 0.0f) || eps > 1e30f) return NQ_ERR_ARG;
    const int64_t G = d / group_size;
    if (bad_ld(ld_x, d) || bad_ld(ld_q, d) || bad_ld(ld_s, G)) return NQ_ERR_STRIDE;
    if (residual_in && (bad_ld(ld_r, d) || bad_ld(ld_ro, d))) return NQ_ERR_STRIDE;
    if (norm_out && bad_ld(ld_n, d)) return NQ_ERR_STRIDE;
    if (M == 0) return NQ_OK;  // empty tensors may carry NULL data pointers
    if (!x || !gamma || !q_out || !scale_out) return NQ_ERR_NULL;
    if ((residual_in == nullptr) != (residual_out == nullptr)) return NQ_ERR_NULL;

    const Region in[] = {region(x, M, ld_x, d, 2), region(residual_in, M, ld_r, d, 2),
                         region(gamma, 1, d, d, gsz)};
    const Region out[] = {region(residual_out, M, ld_ro, d, 2), region(q_out, M, ld_q, d, 1),
                          region(scale_out, M, ld_s, G, 4), region(norm_out, M, ld_n, d, 2)};
    if (any_alias(in, out, /*exact_in=*/1, /*exact_out=*/0)) return NQ_ERR_ALIAS;

    const RowShape shape = pick_row_shape(M, d, vector_rows(d, gamma));
    if (shape.team == 0) return NQ_ERR_SHAPE;

    RmsGroupLaunch L;
    RmsGroupArgs& a = L.k;
    a.x = x; a.r = residual_in; a.ro = residual_out; a.gamma = gamma;
    a.q = q_out; a.scale_out = scale_out; a.norm_out = norm_out;
    a.ld_x = ld_x; a.ld_r = ld_r; a.ld_ro = ld_ro; a.ld_q = ld_q; a.ld_s = ld_s; a.ld_n = ld_n;
    a.M = M; a.d = (uint16_t)d; a.eps = eps; a.inv_d = 1.0 / (double)d;
    a.ue8m0 = scale_mode == NQ_SCALE_UE8M0 ? 1 : 0;
    a.bf16_source = (flags & NQ_FLAG_BF16_SOURCE) != 0 ? 1 : 0;
    L.e5m2 = (flags & NQ_FLAG_E5M2) != 0;
    L.gamma_bf16 = (flags & NQ_FLAG_GAMMA_BF16) != 0;
    if (!launch_row_shape<RmsGroupKernel>(shape, L, M, (hipStream_t)stream)) return NQ_ERR_SHAPE;
    return hipGetLastError() == hipSuccess ? NQ_OK : NQ_ERR_LAUNCH;
}
