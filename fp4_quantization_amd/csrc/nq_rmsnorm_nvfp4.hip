// nq_rmsnorm_nvfp4.hip -- (residual-add +) RMSNorm + NVFP4 for gfx950:
// packed E2M1 elements, one e4m3 scale per 16 elements, a global fp32 scale.
//
// Pages: [NVFP4] "RMSNorm nvfp4 quant fusion for DS V3.2 / Kimi-K2.5"
// ("Description": one pass normalizes in registers and writes the 4-bit
// codes with their 16-element e4m3 scales; the residual-less form takes a
// column slice of wider rows through a row stride, without a copy; commit
// notes: optional bf16 norm output, a fresh residual buffer, hidden % 16 ==
// 0, loop bounds uniform across the lanes that shuffle together).
//
// With NQ_FLAG_BF16_SOURCE the values quantized are bf16(y), the rounding a
// bf16 norm_out stores, so the codes and block scales equal the standalone
// quantizer applied to norm_out ([NVFP4] commit notes: the fused op's codes
// and scale factors match, bit for bit, what the standalone quantizer makes
// of the norm_out it returns).
//
// The row is held in registers exactly as in the per-token FP8 kernel.  A
// 16-element block is two adjacent chunks, owned by lanes t and t^1 of the
// same load instruction, so the block maximum is one DPP exchange.
// Lanes past the end of the row still execute every exchange with zeros
// (d % 16 == 0 keeps both halves of a block on the same side of the end).
#include "nq_device.hpp"
#include "nq_host.hpp"
#include "nq_rms_front.hpp"
#include "nq_rows.hpp"

namespace nq {

struct RmsFp4Args {
    const uint16_t* x;
    const uint16_t* r;
    uint16_t* ro;
    const void* gamma;      // fp32, or bf16 when gamma_bf16
    const float* global_scale;
    uint8_t* q;        // [M, d/2]
    uint8_t* sf;       // [M, d/16]
    uint16_t* norm_out;
    int64_t ld_x, ld_r, ld_ro, ld_q, ld_sf, ld_n;
    int64_t M;
    int d;
    float eps;
    double inv_d;           // RN(1 / d), formed on the host
    bool bf16_source;  // quantize bf16(y): the standalone quantizer applied to norm_out
    bool gamma_bf16;
};

template <int TEAM, int CPL, bool VEC, bool STAGE, bool GB = false, bool RES = true,
          int BLOCK = row_block<TEAM, CPL, 1, VEC, STAGE>()>
__global__ __launch_bounds__(BLOCK) void k_add_rmsnorm_nvfp4(RmsFp4Args a)
{
    using S = TeamShape<TEAM, BLOCK>;
    static_assert(BLOCK >= 128, "128 lanes fill the block-scale table");
    __shared__ double lds_sum[S::kWaves];
    __shared__ float lds_mult[128];  // RN(G / value(code)) for every block-scale code

    const int t = threadIdx.x % TEAM;
    const RowMap m = row_map<TEAM, BLOCK>(a.M);
    const int d = a.d;
    using SV = SharedVectors<TEAM, CPL, VEC, 1, BLOCK, STAGE, GB>;
    __shared__ typename SV::Lds lds_gamma;
    SV gamma({a.gamma}, d);

    const float sg = a.global_scale[0];  // issued early: read on the device at run time
    const float G = 1.0f / sg;            // encode scale

    // The element multiplier depends only on the block-scale code: one
    // correctly rounded quotient per code and block instead of one per chunk.
    // The table is filled while the row loads are in flight, before the
    // front half's first barrier, which then also publishes it.
    const auto fill_table = [&]() {
        if (threadIdx.x < 128) {
            const float sfd = e4m3_value(threadIdx.x);
            lds_mult[threadIdx.x] = sfd > 0.0f ? G / sfd : 0.0f;
        }
    };
    // Residual-less rows keep z unpacked from the sum of squares (these
    // instances have registers to spare); the others unpack it again below.
    constexpr bool KEEP = !RES;
    uint4 zw[CPL];
    float zf[KEEP ? CPL : 1][8];
    const float rstd = rms_front<TEAM, CPL, VEC, RES, SV, KEEP, true>(a.x, a.ld_x, a.r, a.ld_r, a.ro, a.ld_ro, m, t, d,
                                                               a.inv_d, a.eps, gamma, lds_gamma, lds_sum, zw,
                                                               KEEP ? zf : nullptr, fill_table);
    if constexpr (!rms_front_syncs<TEAM, SV>()) __syncthreads();

    const RowIO<VEC, kStoreRows, uint16_t> nio(a.norm_out, a.ld_n, m, d);
    const RowIO<VEC, kStoreCodes, uint8_t> qio(a.q, a.ld_q, m, d / 2);
    const RowIO<VEC, kStoreScales, uint8_t> sfio(a.sf, a.ld_sf, m, d / 16);
    const int t1 = opaque(t);
    if constexpr (!KEEP) {
#pragma unroll
        for (int j = 0; j < CPL; ++j) opaque(zw[j]);
    }
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
        const int e = (j * TEAM + t1) * 8;
        float g[8], z[8], y[8];
        gamma.chunk(lds_gamma, 0, j, e, g);
        if constexpr (KEEP) {
#pragma unroll
            for (int k = 0; k < 8; ++k) z[k] = zf[j][k];
        } else {
            unpack_bf16x8(zw[j], z);
        }
        float amax = 0.0f;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const float n = z[k] * rstd;
            y[k] = n * g[k];
        }
        if (a.norm_out || a.bf16_source) {
            const uint4 nw = make_uint4(pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]),
                                        pack_bf16x2(y[4], y[5]), pack_bf16x2(y[6], y[7]));
            nio.store16(e, col_live<TEAM, VEC>(e, d), nw);  // dropped when norm_out is NULL
            if (a.bf16_source) unpack_bf16x8(nw, y);
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) amax = fmaxf(amax, fabsf(y[k]));
        // Block of 16 = this chunk and the partner lane's (same load
        // instruction, lanes t and t^1: one DPP exchange inside a quad).
        amax = pair_max(amax);
        const float per = div6_rn(amax);  // RN(amax / 6)
        const uint32_t sf = e4m3x4(per * G, 0.0f, 0.0f, 0.0f) & 0x7Fu;  // amax >= 0: codes 0 .. 0x7E
        const float mult = lds_mult[sf];
        float v[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = y[k] * mult;
        // Offsets of codes (e / 2) and block scale (e / 16) as a lane part
        // plus a per-chunk constant the store instruction carries itself.
        qio.store4(t1 * 4 + j * TEAM * 4, col_live<TEAM, VEC>(e, d), e2m1x8(v));
        sfio.store1((t1 >> 1) + j * (TEAM / 2), col_live<TEAM, VEC>(e, d) && (t1 & 1) == 0, sf);
    }
}

template <int TEAM, int CPL, bool VEC>
struct RmsFp4Kernel {
    template <bool STAGE>
    static constexpr int block() { return row_block<TEAM, CPL, 1, VEC, STAGE>(); }
    template <bool STAGE>
    static void launch(const RmsFp4Args& a, dim3 grid, dim3 block, hipStream_t s)
    {
        if (a.r != nullptr) go<STAGE, true>(a, grid, block, s);
        else go<STAGE, false>(a, grid, block, s);
    }
    template <bool STAGE, bool RES>
    static void go(const RmsFp4Args& a, dim3 grid, dim3 block, hipStream_t s)
    {
        if (a.gamma_bf16) hipLaunchKernelGGL((k_add_rmsnorm_nvfp4<TEAM, CPL, VEC, STAGE, true, RES>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((k_add_rmsnorm_nvfp4<TEAM, CPL, VEC, STAGE, false, RES>), grid, block, 0, s, a);
    }
};

} // namespace nq

using namespace nq;

extern "C" nq_status nq_rmsnorm_quant_nvfp4_ex(
    const uint16_t* x, int64_t ld_x,
    const uint16_t* residual_in, int64_t ld_r,
    uint16_t* residual_out, int64_t ld_ro,
    const void* gamma, float eps,
    const float* global_scale, uint32_t flags,
    uint8_t* q_packed, int64_t ld_q,
    uint8_t* block_scale, int64_t ld_sf,
    uint16_t* norm_out, int64_t ld_n,
    int64_t M, int64_t d, void* stream)
{
    if ((flags & ~(uint32_t)(NQ_FLAG_BF16_SOURCE | NQ_FLAG_GAMMA_BF16)) != 0) return NQ_ERR_ARG;
    const int64_t gsz = (flags & NQ_FLAG_GAMMA_BF16) ? 2 : 4;
    if (M < 0 || d <= 0 || d > NQ_MAX_D || d % 16 != 0 || M > kMaxRows) return NQ_ERR_SHAPE;
    if (!(eps >= 0.0f) || eps > 1e30f) return NQ_ERR_ARG;
    if (bad_ld(ld_x, d) || bad_ld(ld_q, d / 2) || bad_ld(ld_sf, d / 16)) return NQ_ERR_STRIDE;
    if (residual_in && (bad_ld(ld_r, d) || bad_ld(ld_ro, d))) return NQ_ERR_STRIDE;
    if (norm_out && bad_ld(ld_n, d)) return NQ_ERR_STRIDE;
    if (M == 0) return NQ_OK;  // empty tensors may carry NULL data pointers
    if (!x || !gamma || !global_scale || !q_packed || !block_scale) return NQ_ERR_NULL;
    if ((residual_in == nullptr) != (residual_out == nullptr)) return NQ_ERR_NULL;

    const Region in[] = {region(x, M, ld_x, d, 2), region(residual_in, M, ld_r, d, 2),
                         region(gamma, 1, d, d, gsz), region(global_scale, 1, 1, 1, 4)};
    const Region out[] = {region(residual_out, M, ld_ro, d, 2), region(q_packed, M, ld_q, d / 2, 1),
                          region(block_scale, M, ld_sf, d / 16, 1), region(norm_out, M, ld_n, d, 2)};
    if (any_alias(in, out, /*exact_in=*/1, /*exact_out=*/0)) return NQ_ERR_ALIAS;

    const RowShape shape = pick_row_shape(M, d, vector_rows(d, gamma));
    if (shape.team == 0) return NQ_ERR_SHAPE;

    RmsFp4Args a;
    a.x = x; a.r = residual_in; a.ro = residual_out; a.gamma = gamma;
    a.global_scale = global_scale; a.q = q_packed; a.sf = block_scale; a.norm_out = norm_out;
    a.ld_x = ld_x; a.ld_r = ld_r; a.ld_ro = ld_ro; a.ld_q = ld_q; a.ld_sf = ld_sf; a.ld_n = ld_n;
    a.M = M; a.d = (int)d; a.eps = eps; a.inv_d = 1.0 / (double)d;
    a.bf16_source = (flags & NQ_FLAG_BF16_SOURCE) != 0;
    a.gamma_bf16 = (flags & NQ_FLAG_GAMMA_BF16) != 0;
    if (!launch_row_shape<RmsFp4Kernel>(shape, a, M, (hipStream_t)stream)) return NQ_ERR_SHAPE;
    return hipGetLastError() == hipSuccess ? NQ_OK : NQ_ERR_LAUNCH;
}

extern "C" nq_status nq_rmsnorm_quant_nvfp4(
    const uint16_t* x, int64_t ld_x,
    const uint16_t* residual_in, int64_t ld_r,
    uint16_t* residual_out, int64_t ld_ro,
    const float* gamma, float eps,
    const float* global_scale,
    uint8_t* q_packed, int64_t ld_q,
    uint8_t* block_scale, int64_t ld_sf,
    uint16_t* norm_out, int64_t ld_n,
    int64_t M, int64_t d, void* stream)
{
    return nq_rmsnorm_quant_nvfp4_ex(x, ld_x, residual_in, ld_r, residual_out, ld_ro, gamma, eps, global_scale,
                                     0u, q_packed, ld_q, block_scale, ld_sf, norm_out, ld_n, M, d, stream);
}
