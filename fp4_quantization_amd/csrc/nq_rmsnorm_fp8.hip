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
// (fp32 -> e4m3) instead of the unfused pipeline's two.
#include "nq_device.hpp"
#include "nq_host.hpp"
#include "nq_rows.hpp"

namespace nq {

struct RmsFp8Args {
    const uint16_t* x;
    const uint16_t* r;      // NULL: residual-less
    uint16_t* ro;           // residual_out (NULL iff r is NULL)
    const float* gamma;
    const float* static_scale;  // NULL: dynamic per-token scale
    uint8_t* q;
    float* scale_out;
    uint16_t* norm_out;     // optional
    int64_t ld_x, ld_r, ld_ro, ld_q, ld_n;
    int64_t M;
    int d;
    float eps;
};

template <int TEAM, int CPL, bool VEC>
__global__ __launch_bounds__(TeamShape<TEAM>::kBlock) void k_add_rmsnorm_fp8(RmsFp8Args a)
{
    using S = TeamShape<TEAM>;
    __shared__ double lds_sum[S::kWaves];
    __shared__ float lds_max[S::kWaves];

    const int t = threadIdx.x % TEAM;
    const int64_t row = (int64_t)blockIdx.x * S::kRows + threadIdx.x / TEAM;
    const bool row_ok = row < a.M;
    const int64_t rr = row_ok ? row : 0;  // keeps addresses formed below in range
    const int d = a.d;
    const bool has_r = a.r != nullptr;

    const uint16_t* xr = a.x + rr * a.ld_x;
    const uint16_t* rrow = has_r ? a.r + rr * a.ld_r : nullptr;

    // Issue every load of the row before the first use.
    uint4 xw[CPL], rw[CPL];
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
        const int e = (j * TEAM + t) * 8;
        const bool ok = row_ok && e < d;
        xw[j] = load_bf16x8<VEC>(xr, e, d, ok);
        rw[j] = has_r ? load_bf16x8<VEC>(rrow, e, d, ok) : make_uint4(0u, 0u, 0u, 0u);
    }

    // z = bf16(x + r); residual write-back; sum of z^2.
    float z[CPL][8];
    double acc = 0.0;
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
        const int e = (j * TEAM + t) * 8;
        const bool ok = row_ok && e < d;
        float xv[8];
        unpack_bf16x8(xw[j], xv);
        if (has_r) {
            float rv[8];
            unpack_bf16x8(rw[j], rv);
            uint32_t p[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) p[k] = pack_bf16x2(xv[2 * k] + rv[2 * k], xv[2 * k + 1] + rv[2 * k + 1]);
            const uint4 zw = make_uint4(p[0], p[1], p[2], p[3]);
            store_bf16x8<VEC>(a.ro + rr * a.ld_ro, e, d, ok, zw);
            unpack_bf16x8(zw, z[j]);
        } else {
#pragma unroll
            for (int k = 0; k < 8; ++k) z[j][k] = xv[k];
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const double zd = (double)z[j][k];
            acc = fma(zd, zd, acc);  // z^2 is exact in binary64
        }
    }

    // Reduction 1: rstd = 1 / sqrt(mean(z^2) + eps).
    acc = team_sum<TEAM>(acc, lds_sum);
    const float ms = (float)(acc / (double)d);
    const float rstd = 1.0f / sqrtf(ms + a.eps);

    // y = (z * rstd) * gamma, kept in registers.
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
        const int e = (j * TEAM + t) * 8;
        const bool ok = row_ok && e < d;
        float g[8];
        load_f32x8<VEC>(a.gamma, e, d, ok, g);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const float n = z[j][k] * rstd;
            z[j][k] = n * g[k];
            amax = fmaxf(amax, fabsf(z[j][k]));
        }
        if (a.norm_out) {
            const uint4 nw = make_uint4(pack_bf16x2(z[j][0], z[j][1]), pack_bf16x2(z[j][2], z[j][3]),
                                        pack_bf16x2(z[j][4], z[j][5]), pack_bf16x2(z[j][6], z[j][7]));
            store_bf16x8<VEC>(a.norm_out + rr * a.ld_n, e, d, ok, nw);
        }
    }

    uint8_t* qr = a.q + rr * a.ld_q;
    if (a.static_scale) {
        // out = y / scale, applied as y * (1 / scale[0]); the scale is read
        // on the device so a graph replay sees its current value.
        const float inv = 1.0f / a.static_scale[0];
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            const int e = (j * TEAM + t) * 8;
            const float* y = z[j];
            const uint2 w = make_uint2(e4m3x4(y[0] * inv, y[1] * inv, y[2] * inv, y[3] * inv),
                                       e4m3x4(y[4] * inv, y[5] * inv, y[6] * inv, y[7] * inv));
            store_u8x8<VEC>(qr, e, d, row_ok && e < d, w);
        }
    } else {
        // Reduction 2: per-token scale s = amax / 448; q = e4m3(y / s).
        amax = team_max<TEAM>(amax, lds_max);
        const float s = amax / kE4M3Max;
        if (t == 0 && row_ok) a.scale_out[row] = s;
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            const int e = (j * TEAM + t) * 8;
            const float* y = z[j];
            uint2 w = make_uint2(0u, 0u);
            if (s > 0.0f)
                w = make_uint2(e4m3x4(y[0] / s, y[1] / s, y[2] / s, y[3] / s),
                               e4m3x4(y[4] / s, y[5] / s, y[6] / s, y[7] / s));
            store_u8x8<VEC>(qr, e, d, row_ok && e < d, w);
        }
    }
}

template <int TEAM, int CPL, bool VEC>
struct RmsFp8Kernel {
    static void launch(const RmsFp8Args& a, dim3 grid, dim3 block, hipStream_t s)
    {
        hipLaunchKernelGGL((k_add_rmsnorm_fp8<TEAM, CPL, VEC>), grid, block, 0, s, a);
    }
};

} // namespace nq

using namespace nq;

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
                         region(gamma, 1, d, d, 4), region(static_scale, 1, 1, 1, 4)};
    const Region out[] = {region(residual_out, M, ld_ro, d, 2), region(q_out, M, ld_q, d, 1),
                          region(static_scale ? nullptr : scale_out, 1, M, M, 4),
                          region(norm_out, M, ld_n, d, 2)};
    if (any_alias(in, out, /*exact_in=*/1, /*exact_out=*/0)) return NQ_ERR_ALIAS;

    // 128-bit path: whole chunks and 16-byte aligned bases and strides.
    bool vec = d % 8 == 0 && aligned(x, 16) && ld_x % 8 == 0 && aligned(gamma, 16) &&
               aligned(q_out, 8) && ld_q % 8 == 0;
    if (residual_in)
        vec = vec && aligned(residual_in, 16) && ld_r % 8 == 0 && aligned(residual_out, 16) &&
              ld_ro % 8 == 0;
    if (norm_out) vec = vec && aligned(norm_out, 16) && ld_n % 8 == 0;

    const RowShape shape = pick_row_shape(M, d, vec);
    if (shape.team == 0) return NQ_ERR_SHAPE;

    RmsFp8Args a;
    a.x = x; a.r = residual_in; a.ro = residual_out; a.gamma = gamma;
    a.static_scale = static_scale; a.q = q_out; a.scale_out = scale_out; a.norm_out = norm_out;
    a.ld_x = ld_x; a.ld_r = ld_r; a.ld_ro = ld_ro; a.ld_q = ld_q; a.ld_n = ld_n;
    a.M = M; a.d = (int)d; a.eps = eps;
    if (!launch_row_shape<RmsFp8Kernel>(shape, a, M, (hipStream_t)stream)) return NQ_ERR_SHAPE;
    return hipGetLastError() == hipSuccess ? NQ_OK : NQ_ERR_LAUNCH;
}
