// nq_rmsnorm_fp8.hip -- fused (residual-add +) RMSNorm + per-token FP8 e4m3
// for gfx950.
//
// Pages: [FUSE] "Fusing RMSNorm and FP8 Quantization Under torch.compile"
// ("TL;DR", "Where norm+quant sits", "FAQ"); [GRAPH] "RMSNorm/FusedRMSNorm +
// Quant kernels cuda graph fixes" ("Description", "Changes": the static
// scale is a one-element device tensor read by the kernel); [GRP]
// "per_token_group_quant_8bit: multiply by reciprocal instead of dividing per
// element" ("Details": per-token FP8 keeps per-element division).
//
// One pass over HBM per row: the bf16 row and residual are loaded once with
// 128-bit loads, z = bf16(x + r) is written back as the new residual, the
// sum of squares is reduced (binary64 partials, so the mean rounds to
// binary32 once regardless of the reduction tree), y = (z * rstd) * gamma
// stays in fp32 registers, its absolute maximum is reduced a second time,
// and the codes are produced straight from those registers: one rounding
// (fp32 -> e4m3) instead of the unfused pipeline's two.  Teams hold at most
// 32 elements per lane, so x, the residual, z (as packed bf16: it is exactly
// a bf16 value) and y all fit at full occupancy; every masked access goes
// through buffer-resource range checks instead of branches.
#include "nq_device.hpp"
#include "nq_host.hpp"
#include "nq_rms_front.hpp"
#include "nq_rows.hpp"

namespace nq {

struct RmsFp8Args {
    const uint16_t* x;
    const uint16_t* r;      // NULL: residual-less
    uint16_t* ro;           // residual_out (NULL iff r is NULL)
    const void* gamma;      // fp32, or bf16 when gamma_bf16
    const float* static_scale;  // NULL: dynamic per-token scale
    uint8_t* q;
    float* scale_out;
    uint16_t* norm_out;     // optional
    int64_t ld_x, ld_r, ld_ro, ld_q, ld_n;
    int64_t M;
    int d;
    float eps;
    double inv_d;           // RN(1 / d), formed on the host
};
// Two 64-byte lines of the kernel-argument segment: a third line measured
// about 70 ns (2 %) slower for a single-row call on MI355X.
static_assert(sizeof(RmsFp8Args) <= 128, "kernel arguments fit two 64-byte lines");

// Host-side launch request: the kernel arguments and the instance choices.
struct RmsFp8Launch {
    RmsFp8Args k;
    bool e5m2;              // output format (e4m3 otherwise)
    bool gamma_bf16;
};

template <int TEAM, int CPL, bool VEC, bool STAGE, Fp8 F = Fp8::E4M3, bool GB = false, bool RES = true,
          int BLOCK = row_block<TEAM, CPL, 1, VEC, STAGE>()>
__global__ __launch_bounds__(BLOCK) void k_add_rmsnorm_fp8(RmsFp8Args a)
{
    using S = TeamShape<TEAM, BLOCK>;
    __shared__ double lds_sum[S::kWaves];
    __shared__ float lds_max[S::kWaves];

    const int t = threadIdx.x % TEAM;
    const RowMap m = row_map<TEAM, BLOCK>(a.M);
    const int d = a.d;
    using SV = SharedVectors<TEAM, CPL, VEC, 1, BLOCK, STAGE, GB>;
    __shared__ typename SV::Lds lds_gamma;
    SV gamma({a.gamma}, d);

    uint4 zw[CPL];
    const float rstd = rms_front<TEAM, CPL, VEC, RES>(a.x, a.ld_x, a.r, a.ld_r, a.ro, a.ld_ro, m, t, d, a.inv_d,
                                                      a.eps, gamma, lds_gamma, lds_sum, zw);

    // y = (z * rstd) * gamma, held in fp32 registers (at most 32 per lane),
    // its absolute maximum, and the optional bf16 copy of y.
    float y[CPL][8];
    float amax = 0.0f;
    const RowIO<VEC, kStoreRows, uint16_t> nio(a.norm_out, a.ld_n, m, d);
    const int t1 = opaque(t);
#pragma unroll
    for (int j = 0; j < CPL; ++j) opaque(zw[j]);
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
        const int e = (j * TEAM + t1) * 8;
        float g[8], z[8];
        gamma.chunk(lds_gamma, 0, j, e, g);
        unpack_bf16x8(zw[j], z);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const float n = z[k] * rstd;
            y[j][k] = n * g[k];
            amax = fmaxf(amax, fabsf(y[j][k]));
        }
        amax = opaque(amax);  // fold each chunk as it is produced
        if (a.norm_out) {
            const uint4 nw = make_uint4(pack_bf16x2(y[j][0], y[j][1]), pack_bf16x2(y[j][2], y[j][3]),
                                        pack_bf16x2(y[j][4], y[j][5]), pack_bf16x2(y[j][6], y[j][7]));
            nio.store16(e, col_live<TEAM, VEC>(e, d), nw);
        }
    }

    // Static: out = y / scale, applied as y * (1 / scale[0]); the scale is
    // read on the device so a graph replay sees its current value.
    // Dynamic (reduction 2): s = amax / 448 (57344 for e5m2) and
    // q = fp8(y / s), one correctly rounded quotient per element (div_by).
    const RowIO<VEC, kStoreCodes, uint8_t> qio(a.q, a.ld_q, m, d);
    if (a.static_scale == nullptr) {
        amax = team_max<TEAM>(amax, lds_max);
        float s, inv;
        token_scale<F>(amax, s, inv);
        if (t == 0 && m.ok) a.scale_out[m.row] = s;
        if (wave_scales_normal(s)) {
#pragma unroll
            for (int j = 0; j < CPL; ++j) {
                const int e = (j * TEAM + t1) * 8;
                float v[8];
#pragma unroll
                for (int k = 0; k < 8; ++k) v[k] = div_by(y[j][k], s, inv);
                qio.store8(e, col_live<TEAM, VEC>(e, d), fp8x8_bounded<F>(v));
            }
        } else {
            // A zero scale (an all-zero row, or amax / fmax below the
            // smallest subnormal) stores +0 codes whatever the signs of y.
#pragma unroll
            for (int j = 0; j < CPL; ++j) {
                const int e = (j * TEAM + t1) * 8;
                float v[8];
#pragma unroll
                for (int k = 0; k < 8; ++k) v[k] = s > 0.0f ? div_by(y[j][k], s, inv) : 0.0f;
                qio.store8(e, col_live<TEAM, VEC>(e, d), fp8x8<F>(v));
            }
        }
    } else {
        const float inv = 1.0f / a.static_scale[0];
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            const int e = (j * TEAM + t1) * 8;
            float v[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) v[k] = y[j][k] * inv;
            qio.store8(e, col_live<TEAM, VEC>(e, d), fp8x8<F>(v));
        }
    }
}

template <int TEAM, int CPL, bool VEC>
struct RmsFp8Kernel {
    template <bool STAGE>
    static constexpr int block() { return row_block<TEAM, CPL, 1, VEC, STAGE>(); }
    template <bool STAGE>
    static void launch(const RmsFp8Launch& a, dim3 grid, dim3 block, hipStream_t s)
    {
        if (a.k.r != nullptr) go<STAGE, true>(a, grid, block, s);
        else go<STAGE, false>(a, grid, block, s);
    }
    template <bool STAGE, bool RES>
    static void go(const RmsFp8Launch& a, dim3 grid, dim3 block, hipStream_t s)
    {
        if (a.gamma_bf16) {
            if (a.e5m2) hipLaunchKernelGGL((k_add_rmsnorm_fp8<TEAM, CPL, VEC, STAGE, Fp8::E5M2, true, RES>), grid, block, 0, s, a.k);
            else hipLaunchKernelGGL((k_add_rmsnorm_fp8<TEAM, CPL, VEC, STAGE, Fp8::E4M3, true, RES>), grid, block, 0, s, a.k);
        } else {
            if (a.e5m2) hipLaunchKernelGGL((k_add_rmsnorm_fp8<TEAM, CPL, VEC, STAGE, Fp8::E5M2, false, RES>), grid, block, 0, s, a.k);
            else hipLaunchKernelGGL((k_add_rmsnorm_fp8<TEAM, CPL, VEC, STAGE, Fp8::E4M3, false, RES>), grid, block, 0, s, a.k);
        }
    }
};

} // namespace nq

using namespace nq;

extern "C" nq_status nq_fused_add_rmsnorm_quant_fp8_ex(
    const uint16_t* x, int64_t ld_x,
    const uint16_t* residual_in, int64_t ld_r,
    uint16_t* residual_out, int64_t ld_ro,
    const void* gamma, float eps,
    const float* static_scale, uint32_t flags,
    uint8_t* q_out, int64_t ld_q,
    float* scale_out,
    uint16_t* norm_out, int64_t ld_n,
    int64_t M, int64_t d, void* stream)
{
    if ((flags & ~(uint32_t)(NQ_FLAG_E5M2 | NQ_FLAG_GAMMA_BF16)) != 0) return NQ_ERR_ARG;
    const int64_t gsz = (flags & NQ_FLAG_GAMMA_BF16) ? 2 : 4;
    if (M < 0 || d <= 0 || d > NQ_MAX_D || M > kMaxRows) return NQ_ERR_SHAPE;
    if (!(eps >= 0.0f) || eps > 1e30f) return NQ_ERR_ARG;
    if (bad_ld(ld_x, d) || bad_ld(ld_q, d)) return NQ_ERR_STRIDE;
    if (residual_in && (bad_ld(ld_r, d) || bad_ld(ld_ro, d))) return NQ_ERR_STRIDE;
    if (norm_out && bad_ld(ld_n, d)) return NQ_ERR_STRIDE;
    if (M == 0) return NQ_OK;  // empty tensors may carry NULL data pointers
    if (!x || !gamma || !q_out) return NQ_ERR_NULL;
    if (!static_scale && !scale_out) return NQ_ERR_NULL;
    if ((residual_in == nullptr) != (residual_out == nullptr)) return NQ_ERR_NULL;

    const Region in[] = {region(x, M, ld_x, d, 2), region(residual_in, M, ld_r, d, 2),
                         region(gamma, 1, d, d, gsz), region(static_scale, 1, 1, 1, 4)};
    const Region out[] = {region(residual_out, M, ld_ro, d, 2), region(q_out, M, ld_q, d, 1),
                          region(static_scale ? nullptr : scale_out, 1, M, M, 4),
                          region(norm_out, M, ld_n, d, 2)};
    if (any_alias(in, out, /*exact_in=*/1, /*exact_out=*/0)) return NQ_ERR_ALIAS;

    const RowShape shape = pick_row_shape(M, d, vector_rows(d, gamma));
    if (shape.team == 0) return NQ_ERR_SHAPE;

    RmsFp8Launch L;
    RmsFp8Args& a = L.k;
    a.x = x; a.r = residual_in; a.ro = residual_out; a.gamma = gamma;
    a.static_scale = static_scale; a.q = q_out; a.scale_out = scale_out; a.norm_out = norm_out;
    a.ld_x = ld_x; a.ld_r = ld_r; a.ld_ro = ld_ro; a.ld_q = ld_q; a.ld_n = ld_n;
    a.M = M; a.d = (int)d; a.eps = eps; a.inv_d = 1.0 / (double)d;
    L.e5m2 = (flags & NQ_FLAG_E5M2) != 0;
    L.gamma_bf16 = (flags & NQ_FLAG_GAMMA_BF16) != 0;
    if (!launch_row_shape<RmsFp8Kernel>(shape, L, M, (hipStream_t)stream)) return NQ_ERR_SHAPE;
    return hipGetLastError() == hipSuccess ? NQ_OK : NQ_ERR_LAUNCH;
}

extern "C" nq_status nq_fused_add_rmsnorm_quant_fp8(
    const uint16_t* x, int64_t ld_x,
    const uint16_t* residual_in, int64_t ld_r,
    uint16_t* residual_out, int64_t ld_ro,
    const float* gamma, float eps,
    const float* static_scale,
    uint8_t* q_out, int64_t ld_q,
    float* scale_out,
    uint16_t* norm_out, int64_t ld_n,
    int64_t M, int64_t d, void* stream)
{
    return nq_fused_add_rmsnorm_quant_fp8_ex(x, ld_x, residual_in, ld_r, residual_out, ld_ro, gamma, eps,
                                             static_scale, 0u, q_out, ld_q, scale_out, norm_out, ld_n, M, d,
                                             stream);
}
