// nq_group_fp8.hip -- per-token-group FP8 e4m3 with one reciprocal per group,
// for gfx950.
//
// Pages: [GRP] "per_token_group_quant_8bit: multiply by reciprocal instead of
// dividing per element" (commit message and "Details": one correctly
// rounded division per 128-element group, then a multiply per element; the
// UE8M0 power-of-two scales make the reciprocal exact; "Microbenchmarks":
// the kernel is memory-bound at about 2 FLOPs per element, and a flat
// index over all groups of the grid is the fastest schedule at large M).
//
// Flat schedule: group i of the whole [M, K] matrix (row i / (K/128),
// column group i % (K/128)) is owned by 16 lanes, 8 elements (one 128-bit
// load) each, so a wavefront covers 4 groups and each of its load
// instructions reads 1 KB of contiguous row.  The group maximum is four DPP
// steps inside a 16-lane DPP row.  Each lane handles kGroupUnroll groups,
// all loads issued before the first use.
#include "nq_device.hpp"
#include "nq_host.hpp"

namespace nq {

struct GroupArgs {
    const uint16_t* x;
    uint8_t* q;
    float* scale_out;
    int64_t ld_x, ld_q;
    uint32_t groups_per_row;  // K / 128
    uint32_t total;           // M * K / 128
};

constexpr int kGroup = 128;
constexpr int kGroupBlock = 256;   // 16 groups per block per step
constexpr int kGroupUnroll = 2;  // measured: 2 beats 1, 3, 4 and 8 at 32768 x 4096

template <bool UE8M0, Fp8 F>
__global__ __launch_bounds__(kGroupBlock) void k_group_fp8(GroupArgs a)
{
    const int lane16 = threadIdx.x & 15;
    const uint32_t base = (uint32_t)blockIdx.x * (kGroupBlock / 16) * kGroupUnroll + threadIdx.x / 16;

    // Idle lanes of the last block read group 0 (always in bounds) and
    // store nothing, so every load is unconditional.
    uint4 w[kGroupUnroll];
    int64_t qoff[kGroupUnroll];
    bool ok[kGroupUnroll];
#pragma unroll
    for (int u = 0; u < kGroupUnroll; ++u) {
        const uint32_t gi = base + (uint32_t)u * (kGroupBlock / 16);
        ok[u] = gi < a.total;
        const uint32_t g = ok[u] ? gi : 0u;
        const uint32_t m = g / a.groups_per_row, c = g - m * a.groups_per_row;
        const int col = (int)c * kGroup + lane16 * 8;
        const uint16_t* px = a.x + (int64_t)m * a.ld_x + col;
        qoff[u] = (int64_t)m * a.ld_q + col;
        w[u] = ld_global_stream16(px);
    }

#pragma unroll
    for (int u = 0; u < kGroupUnroll; ++u) {
        float v[8];
        unpack_bf16x8(w[u], v);
        float amax = 0.0f;
#pragma unroll
        for (int k = 0; k < 8; ++k) amax = fmaxf(amax, fabsf(v[k]));
        amax = max16_dpp(amax);
        float s = amax / fp8_max<F>();
        if constexpr (UE8M0) s = pow2_ceil(s);
        const float inv = s > 0.0f ? 1.0f / s : 0.0f;
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = v[k] * inv;
        const uint2 q = fp8x8<F>(v);
        if (ok[u]) {
            st_global_stream8(a.q + qoff[u], q);
            if (lane16 == 0) a.scale_out[base + (uint32_t)u * (kGroupBlock / 16)] = s;
        }
    }
}

template <bool UE8M0>
static void launch_group(const GroupArgs& a, bool e5m2, hipStream_t s)
{
    const uint32_t per_block = (kGroupBlock / 16) * kGroupUnroll;
    const uint32_t blocks = (a.total + per_block - 1) / per_block;
    if (e5m2) hipLaunchKernelGGL((k_group_fp8<UE8M0, Fp8::E5M2>), dim3(blocks), dim3(kGroupBlock), 0, s, a);
    else hipLaunchKernelGGL((k_group_fp8<UE8M0, Fp8::E4M3>), dim3(blocks), dim3(kGroupBlock), 0, s, a);
}

} // namespace nq

using namespace nq;

extern "C" nq_status nq_per_token_group_quant_fp8_ex(
    const uint16_t* x, int64_t ld_x, int64_t M, int64_t K,
    int32_t group_size, int32_t scale_mode, uint32_t flags,
    uint8_t* q_out, int64_t ld_q, float* scale_out, void* stream)
{
    if (group_size != kGroup) return NQ_ERR_ARG;
    if ((flags & ~(uint32_t)NQ_FLAG_E5M2) != 0) return NQ_ERR_ARG;
    if (scale_mode != NQ_SCALE_FP32 && scale_mode != NQ_SCALE_UE8M0) return NQ_ERR_ARG;
    if (M < 0 || K <= 0 || K % group_size != 0 || M > kMaxRows) return NQ_ERR_SHAPE;
    if (bad_ld(ld_x, K) || bad_ld(ld_q, K)) return NQ_ERR_STRIDE;
    const int64_t G = K / group_size;
    if (M * G >= (int64_t(1) << 31)) return NQ_ERR_SHAPE;
    if (M == 0) return NQ_OK;  // empty tensors may carry NULL data pointers
    if (!x || !q_out || !scale_out) return NQ_ERR_NULL;

    const Region in[] = {region(x, M, ld_x, K, 2)};
    const Region out[] = {region(q_out, M, ld_q, K, 1), region(scale_out, 1, M * G, M * G, 4)};
    if (any_alias(in, out)) return NQ_ERR_ALIAS;

    // Rows are whole 8-element chunks (K % 128 == 0); pointers and strides
    // need no alignment (see vector_rows).
    GroupArgs a;
    a.x = x; a.q = q_out; a.scale_out = scale_out; a.ld_x = ld_x; a.ld_q = ld_q;
    a.groups_per_row = (uint32_t)G;
    a.total = (uint32_t)(M * G);
    hipStream_t s = (hipStream_t)stream;
    const bool ue = scale_mode == NQ_SCALE_UE8M0;
    const bool e5 = (flags & NQ_FLAG_E5M2) != 0;
    ue ? launch_group<true>(a, e5, s) : launch_group<false>(a, e5, s);
    return hipGetLastError() == hipSuccess ? NQ_OK : NQ_ERR_LAUNCH;
}

extern "C" nq_status nq_per_token_group_quant_fp8(
    const uint16_t* x, int64_t ld_x, int64_t M, int64_t K,
    int32_t group_size, int32_t scale_mode,
    uint8_t* q_out, int64_t ld_q, float* scale_out, void* stream)
{
    return nq_per_token_group_quant_fp8_ex(x, ld_x, M, K, group_size, scale_mode, 0u, q_out, ld_q, scale_out,
                                           stream);
}
