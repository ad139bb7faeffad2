// nq_layernorm_fp8.hip -- LayerNorm + static per-tensor FP8 e4m3 for gfx950.
//
// Pages: [LNQ] "feat: fused FP8 quantization output for LayerNorm"
// ("Description": the quantization scale divides, out = normed / scale; the
// review thread; "Tests": the scale is read on the device so graph replays
// see updates); [GRAPH] "RMSNorm/FusedRMSNorm + Quant kernels cuda graph
// fixes" ("Changes": scale_inv = 1 / scale[0] formed in the kernel).
//
// One HBM read of the bf16 row and one write of its codes (3 bytes per
// element, [LNQ] "Description").  Both statistics come from the registers:
// the mean (binary64 partial sums, rounded to binary32 once), then the
// population variance of c = x - mean (c^2 is exact in binary64), so a
// large mean costs no precision.
#include "nq_device.hpp"
#include "nq_host.hpp"
#include "nq_rows.hpp"

namespace nq {

struct LnFp8Args {
    const uint16_t* x;
    const float* gamma;
    const float* beta;
    const float* scale;
    uint8_t* q;
    int64_t ld_x, ld_q;
    int64_t M;
    int d;
    float eps;
};

template <int TEAM, int CPL, bool VEC>
__global__ __launch_bounds__(TeamShape<TEAM>::kBlock) void k_layernorm_fp8(LnFp8Args a)
{
    using S = TeamShape<TEAM>;
    __shared__ double lds_mean[S::kWaves];
    __shared__ double lds_var[S::kWaves];

    const int t = threadIdx.x % TEAM;
    const int64_t row = (int64_t)blockIdx.x * S::kRows + threadIdx.x / TEAM;
    const bool row_ok = row < a.M;
    const int64_t rr = row_ok ? row : 0;
    const int d = a.d;
    const uint16_t* xr = a.x + rr * a.ld_x;

    uint4 xw[CPL];
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
        const int e = (j * TEAM + t) * 8;
        xw[j] = load_bf16x8<VEC>(xr, e, d, row_ok && e < d);
    }

    // mean = sum(x) / d; every bf16 x is exact in binary64.
    float c[CPL][8];
    double acc = 0.0;
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
        unpack_bf16x8(xw[j], c[j]);
#pragma unroll
        for (int k = 0; k < 8; ++k) acc += (double)c[j][k];
    }
    acc = team_sum<TEAM>(acc, lds_mean);
    const float mu = (float)(acc / (double)d);

    // c = x - mean (binary32); var = sum(c^2) / d over the d real elements.
    double acc2 = 0.0;
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
        const int e = (j * TEAM + t) * 8;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const bool live = row_ok && e + k < d;
            c[j][k] = live ? c[j][k] - mu : 0.0f;
            const double cd = (double)c[j][k];
            acc2 = fma(cd, cd, acc2);
        }
    }
    acc2 = team_sum<TEAM>(acc2, lds_var);
    const float var = (float)(acc2 / (double)d);
    const float rstd = 1.0f / sqrtf(var + a.eps);
    const float inv = 1.0f / a.scale[0];

    uint8_t* qr = a.q + rr * a.ld_q;
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
        const int e = (j * TEAM + t) * 8;
        const bool ok = row_ok && e < d;
        float g[8], b[8], v[8];
        load_f32x8<VEC>(a.gamma, e, d, ok, g);
        load_f32x8<VEC>(a.beta, e, d, ok, b);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const float n = c[j][k] * rstd;
            const float gn = n * g[k];
            const float y = gn + b[k];
            v[k] = y * inv;
        }
        const uint2 w = make_uint2(e4m3x4(v[0], v[1], v[2], v[3]), e4m3x4(v[4], v[5], v[6], v[7]));
        store_u8x8<VEC>(qr, e, d, ok, w);
    }
}

template <int TEAM, int CPL, bool VEC>
struct LnFp8Kernel {
    static void launch(const LnFp8Args& a, dim3 grid, dim3 block, hipStream_t s)
    {
        hipLaunchKernelGGL((k_layernorm_fp8<TEAM, CPL, VEC>), grid, block, 0, s, a);
    }
};

} // namespace nq

using namespace nq;

extern "C" nq_status nq_layernorm_quant_fp8(
    const uint16_t* x, int64_t ld_x,
    const float* gamma, const float* beta, float eps,
    const float* scale,
    uint8_t* q_out, int64_t ld_q,
    int64_t M, int64_t d, void* stream)
{
    if (M < 0 || d <= 0 || d > NQ_MAX_D || M > kMaxRows) return NQ_ERR_SHAPE;
    if (!(eps >= 0.0f) || eps > 1e30f) return NQ_ERR_ARG;
    if (bad_ld(ld_x, d) || bad_ld(ld_q, d)) return NQ_ERR_STRIDE;
    if (M == 0) return NQ_OK;  // empty tensors may carry NULL data pointers
    if (!x || !gamma || !beta || !scale || !q_out) return NQ_ERR_NULL;

    const Region in[] = {region(x, M, ld_x, d, 2), region(gamma, 1, d, d, 4),
                         region(beta, 1, d, d, 4), region(scale, 1, 1, 1, 4)};
    const Region out[] = {region(q_out, M, ld_q, d, 1)};
    if (any_alias(in, out)) return NQ_ERR_ALIAS;

    const bool vec = d % 8 == 0 && aligned(x, 16) && ld_x % 8 == 0 && aligned(gamma, 16) &&
                     aligned(beta, 16) && aligned(q_out, 8) && ld_q % 8 == 0;
    const RowShape shape = pick_row_shape(M, d, vec);
    if (shape.team == 0) return NQ_ERR_SHAPE;

    LnFp8Args a;
    a.x = x; a.gamma = gamma; a.beta = beta; a.scale = scale; a.q = q_out;
    a.ld_x = ld_x; a.ld_q = ld_q; a.M = M; a.d = (int)d; a.eps = eps;
    if (!launch_row_shape<LnFp8Kernel>(shape, a, M, (hipStream_t)stream)) return NQ_ERR_SHAPE;
    return hipGetLastError() == hipSuccess ? NQ_OK : NQ_ERR_LAUNCH;
}
