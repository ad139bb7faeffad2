// nq_layernorm_fp8.hip -- LayerNorm + FP8 (e4m3 or e5m2) with a static
// per-tensor or a dynamic per-token scale, for gfx950.
//
// Pages: [LNQ] "feat: fused FP8 quantization output for LayerNorm"
// ("Description": the quantization scale divides, out = normed / scale; the
// review thread; "Tests": the scale is read on the device so graph replays
// see updates); [GRAPH] "RMSNorm/FusedRMSNorm + Quant kernels cuda graph
// fixes" ("Changes": scale_inv = 1 / scale[0] formed in the kernel).
//
// One HBM read of the bf16 row and one write of its codes (3 bytes per
// element, [LNQ] "Description").  Both statistics come from the registers:
// the mean, then the population variance of c = x - mean (two passes, so a
// large mean costs no precision).  Each 8-element chunk is summed in
// binary32 (sum_chunk / sumsq_chunk in nq_device.hpp: a packed bf16 dot
// product for the mean, fused multiply-adds for c^2), the chunk sums are
// added in binary64, and a chunk whose binary32 sum leaves a safe range is
// summed exactly in binary64 instead.  The result is the binary64 row sum
// to within a few binary32 roundings of the chunk sums -- a relative 2^-22 of
// the variance at most; the dot products of the mean's chunks round each
// step to within 2 units in the last place of its largest term -- so a
// row's mean and rstd can differ from the exactly summed ones by a unit in
// the last place: within the reduction-order tolerance, and the kernel's
// instruction count drops by a fifth (it is bound by vector issue as much as
// by HBM).
#include "nq_device.hpp"
#include "nq_host.hpp"
#include "nq_rows.hpp"

namespace nq {

struct LnFp8Args {
    const uint16_t* x;
    const void* gamma;      // fp32, or bf16 when vec_bf16
    const void* beta;
    const float* scale;     // static per-tensor scale, or NULL: dynamic per-token
    uint8_t* q;
    float* scale_out;       // [M] per-token scales (dynamic only)
    int64_t ld_x, ld_q;
    int64_t M;
    int d;
    float eps;
    double inv_d;           // RN(1 / d), formed on the host
    bool e5m2;              // output format (e4m3 otherwise)
    bool vec_bf16;          // gamma and beta are bf16
};

template <int TEAM, int CPL, bool VEC, bool STAGE, Fp8 F = Fp8::E4M3, bool DYN = false, bool GB = false,
          int BLOCK = row_block<TEAM, CPL, 2, VEC, STAGE>()>
__global__ __launch_bounds__(BLOCK) void k_layernorm_fp8(LnFp8Args a)
{
    using S = TeamShape<TEAM, BLOCK>;
    __shared__ double lds_mean[S::kWaves];
    __shared__ double lds_var[S::kWaves];
    __shared__ float lds_max[S::kWaves];

    const int t = threadIdx.x % TEAM;
    const RowMap m = row_map<TEAM, BLOCK>(a.M);
    const int d = a.d;
    const RowIO<VEC, kLoadStream, uint16_t> xio(a.x, a.ld_x, m, d);
    using SV = SharedVectors<TEAM, CPL, VEC, 2, BLOCK, STAGE, GB, /*DMA=*/DYN>;
    __shared__ typename SV::Lds lds_gb;
    SV gb({a.gamma, a.beta}, d);
    const RowIO<VEC, kStoreCodesOnly, uint8_t> qio(a.q, a.ld_q, m, d);
    float scale = 1.0f;
    if constexpr (!DYN) scale = a.scale[0];  // issued early: read on the device at run time

    uint4 xw[CPL];
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
        const int e = (j * TEAM + t) * 8;
        xw[j] = xio.load16(e, col_live<TEAM, VEC>(e, d));
    }
    gb.issue(t, lds_gb);

    // mean = sum(x) / d (masked elements load as 0).  The unpacked row is
    // what c replaces below, so it stays unpacked.
    float c[CPL][8];
    double acc = 0.0;
    bool ok = true;
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
        const float p = sum_chunk_f32(xw[j]);
        ok = ok && sum_ok(p);
        acc += (double)p;
        unpack_bf16x8(xw[j], c[j]);
    }
    if (__builtin_amdgcn_ballot_w64(!ok) != 0) {
        __asm__ volatile("");  // keep it a branch
        if (!ok) {
            acc = 0.0;
#pragma unroll
            for (int j = 0; j < CPL; ++j)
#pragma unroll
                for (int k = 0; k < 8; ++k) acc += (double)c[j][k];
        }
    }
    gb.publish(lds_gb);
    acc = team_sum<TEAM>(acc, lds_mean);
    const float mu = (float)div_by_len(acc, (double)d, a.inv_d);
    __builtin_amdgcn_sched_barrier(0);

    // c = x - mean (binary32), held in registers (at most 32 per lane);
    // var = sum(c^2) / d over the d real elements.  A chunk past the row end
    // contributes nothing; on the element-wise path the elements of the last
    // chunk past the end are left out of its sum.
    double acc2 = 0.0;
    bool ok2 = true;
    const int t1 = opaque(t);
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
        const int e = (j * TEAM + t1) * 8;
        float sq[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            c[j][k] = c[j][k] - mu;
            const bool live = VEC || e + k < d;  // whole chunks on the 128-bit path
            sq[k] = live ? c[j][k] : 0.0f;
        }
        const float p = sumsq_chunk_f32(sq);
        const bool in_row = e < d;
        ok2 = ok2 && (sumsq_ok(p) || !in_row);
        acc2 += in_row ? (double)p : 0.0;
    }
    if (__builtin_amdgcn_ballot_w64(!ok2) != 0) {
        __asm__ volatile("");  // keep it a branch
        if (!ok2) {
            acc2 = 0.0;
#pragma unroll
            for (int j = 0; j < CPL; ++j) {
                const int e = (j * TEAM + t1) * 8;
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const double cd = (VEC ? e < d : e + k < d) ? (double)c[j][k] : 0.0;
                    acc2 = fma(cd, cd, acc2);
                }
            }
        }
    }
    acc2 = team_sum<TEAM>(acc2, lds_var);
    const float var = (float)div_by_len(acc2, (double)d, a.inv_d);
    const float rstd = rsqrt_rn(var + a.eps);
    __builtin_amdgcn_sched_barrier(0);

    if constexpr (!DYN) {
        // Static: y = ((c * rstd) * gamma) + beta; v = y * (1 / scale) in
        // place of c.  A wavefront whose values all lie within the format's
        // finite range converts them with no clamp (the same codes, one
        // instruction per element fewer); one holding a saturating value
        // clamps them first.
        const float inv = 1.0f / scale;
        float vmax = 0.0f;
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            const int e = (j * TEAM + t1) * 8;
            float g[8], b[8];
            gb.chunk(lds_gb, 0, j, e, g);
            gb.chunk(lds_gb, 1, j, e, b);
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const float n = c[j][k] * rstd;
                const float gn = n * g[k];
                const float y = gn + b[k];
                c[j][k] = y * inv;
                vmax = fmaxf(vmax, fabsf(c[j][k]));
            }
        }
        if (__builtin_amdgcn_ballot_w64(!(vmax <= fp8_max<F>())) != 0) {
            __asm__ volatile("");  // keep it a branch
#pragma unroll
            for (int j = 0; j < CPL; ++j)
#pragma unroll
                for (int k = 0; k < 8; ++k) c[j][k] = fp8_clamp<F>(c[j][k]);
        }
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            const int e = (j * TEAM + t1) * 8;
            qio.store8(e, col_live<TEAM, VEC>(e, d), fp8x8_bounded<F>(c[j]));
        }
    } else {
        // Dynamic per-token: y replaces c in the registers, its absolute
        // maximum is reduced over the team (past the row end gamma and beta
        // are zero, so y is too), s = amax / fmax, q = fp8(y / s) with one
        // correctly rounded quotient per element (div_by).
        float amax = 0.0f;
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            const int e = (j * TEAM + t1) * 8;
            if constexpr (SV::kStaged) {
                // half a chunk of gamma and beta at a time: 8 registers fewer
                // at the kernel's peak, which sets its occupancy
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    float g[4], b[4];
                    gb.half(lds_gb, 0, e, h, g);
                    gb.half(lds_gb, 1, e, h, b);
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        const float n = c[j][4 * h + k] * rstd;
                        const float gn = n * g[k];
                        c[j][4 * h + k] = gn + b[k];
                        amax = fmaxf(amax, fabsf(c[j][4 * h + k]));
                    }
                }
            } else {
                float g[8], b[8];
                gb.chunk(lds_gb, 0, j, e, g);
                gb.chunk(lds_gb, 1, j, e, b);
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const float n = c[j][k] * rstd;
                    const float gn = n * g[k];
                    c[j][k] = gn + b[k];
                    amax = fmaxf(amax, fabsf(c[j][k]));
                }
            }
        }
        amax = team_max<TEAM>(amax, lds_max);
        float s, inv;
        token_scale<F>(amax, s, inv);
        if (t == 0 && m.ok) a.scale_out[m.row] = s;
        // The quotients replace y in place.  With a normal scale in every
        // lane they are bounded as the clamp-free conversion needs; otherwise
        // the wavefront clamps them first (the same codes either way), and a
        // zero scale stores +0 codes whatever the signs of y.
#pragma unroll
        for (int j = 0; j < CPL; ++j)
#pragma unroll
            for (int k = 0; k < 8; ++k) c[j][k] = div_by(c[j][k], s, inv);
        if (!wave_scales_normal(s)) {
            __asm__ volatile("");  // keep it a branch
#pragma unroll
            for (int j = 0; j < CPL; ++j)
#pragma unroll
                for (int k = 0; k < 8; ++k) c[j][k] = s > 0.0f ? fp8_clamp<F>(c[j][k]) : 0.0f;
        }
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            const int e = (j * TEAM + t1) * 8;
            qio.store8(e, col_live<TEAM, VEC>(e, d), fp8x8_bounded<F>(c[j]));
        }
    }
}

template <int TEAM, int CPL, bool VEC>
struct LnFp8Kernel {
    template <bool STAGE>
    static constexpr int block() { return row_block<TEAM, CPL, 2, VEC, STAGE>(); }
    template <bool STAGE>
    static void launch(const LnFp8Args& a, dim3 grid, dim3 block, hipStream_t s)
    {
        if (a.vec_bf16) go<STAGE, true>(a, grid, block, s);
        else go<STAGE, false>(a, grid, block, s);
    }
    template <bool STAGE, bool GB>
    static void go(const LnFp8Args& a, dim3 grid, dim3 block, hipStream_t s)
    {
        const bool dyn = a.scale == nullptr;
        if (a.e5m2) {
            if (dyn) hipLaunchKernelGGL((k_layernorm_fp8<TEAM, CPL, VEC, STAGE, Fp8::E5M2, true, GB>), grid, block, 0, s, a);
            else hipLaunchKernelGGL((k_layernorm_fp8<TEAM, CPL, VEC, STAGE, Fp8::E5M2, false, GB>), grid, block, 0, s, a);
        } else {
            if (dyn) hipLaunchKernelGGL((k_layernorm_fp8<TEAM, CPL, VEC, STAGE, Fp8::E4M3, true, GB>), grid, block, 0, s, a);
            else hipLaunchKernelGGL((k_layernorm_fp8<TEAM, CPL, VEC, STAGE, Fp8::E4M3, false, GB>), grid, block, 0, s, a);
        }
    }
};

} // namespace nq

using namespace nq;

extern "C" nq_status nq_layernorm_quant_fp8_ex(
    const uint16_t* x, int64_t ld_x,
    const void* gamma, const void* beta, float eps,
    const float* scale, uint32_t flags,
    uint8_t* q_out, int64_t ld_q,
    float* scale_out,
    int64_t M, int64_t d, void* stream)
{
    if ((flags & ~(uint32_t)(NQ_FLAG_E5M2 | NQ_FLAG_GAMMA_BF16)) != 0) return NQ_ERR_ARG;
    const int64_t gsz = (flags & NQ_FLAG_GAMMA_BF16) ? 2 : 4;
    if (M < 0 || d <= 0 || d > NQ_MAX_D || M > kMaxRows) return NQ_ERR_SHAPE;
    if (!(eps >= 0.0f) || eps > 1e30f) return NQ_ERR_ARG;
    if (bad_ld(ld_x, d) || bad_ld(ld_q, d)) return NQ_ERR_STRIDE;
    if (M == 0) return NQ_OK;  // empty tensors may carry NULL data pointers
    if (!x || !gamma || !beta || !q_out) return NQ_ERR_NULL;
    if (!scale && !scale_out) return NQ_ERR_NULL;  // dynamic scales need somewhere to go

    const Region in[] = {region(x, M, ld_x, d, 2), region(gamma, 1, d, d, gsz),
                         region(beta, 1, d, d, gsz), region(scale, 1, 1, 1, 4)};
    const Region out[] = {region(q_out, M, ld_q, d, 1), region(scale ? nullptr : scale_out, 1, M, M, 4)};
    if (any_alias(in, out)) return NQ_ERR_ALIAS;

    const RowShape shape = pick_row_shape(M, d, vector_rows(d, gamma, beta));
    if (shape.team == 0) return NQ_ERR_SHAPE;

    LnFp8Args a;
    a.x = x; a.gamma = gamma; a.beta = beta; a.scale = scale; a.q = q_out;
    a.scale_out = scale ? nullptr : scale_out;
    a.ld_x = ld_x; a.ld_q = ld_q; a.M = M; a.d = (int)d; a.eps = eps; a.inv_d = 1.0 / (double)d;
    a.e5m2 = (flags & NQ_FLAG_E5M2) != 0;
    a.vec_bf16 = (flags & NQ_FLAG_GAMMA_BF16) != 0;
    if (!launch_row_shape<LnFp8Kernel>(shape, a, M, (hipStream_t)stream)) return NQ_ERR_SHAPE;
    return hipGetLastError() == hipSuccess ? NQ_OK : NQ_ERR_LAUNCH;
}

extern "C" nq_status nq_layernorm_quant_fp8(
    const uint16_t* x, int64_t ld_x,
    const float* gamma, const float* beta, float eps,
    const float* scale,
    uint8_t* q_out, int64_t ld_q,
    int64_t M, int64_t d, void* stream)
{
    if (M > 0 && !scale) return NQ_ERR_NULL;  // this form is static-scale only
    return nq_layernorm_quant_fp8_ex(x, ld_x, gamma, beta, eps, scale, 0u, q_out, ld_q, nullptr, M, d, stream);
}
