// nq_misc.hip -- status strings, version, and the diagnostic kernels: the
// device conversion routines and the arithmetic shortcuts applied
// element-wise (so their rounding can be compared with an independent host
// computation) and a 128-bit copy used as the bandwidth reference for the
// same HBM.
#include "nq_device.hpp"
#include "nq_host.hpp"

namespace nq {

// One thread converts 8 consecutive inputs through the same packing
// routines the quantization kernels use (so byte and nibble order are
// exercised too); the tail beyond n is padded with zeros and not stored.
__global__ __launch_bounds__(256) void k_diag_codec(int kind, const float* in, void* out, int64_t n)
{
    const int64_t i0 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 8;
    if (i0 >= n) return;
    float v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = i0 + k < n ? in[i0 + k] : 0.0f;
    if (kind == NQ_CODEC_E4M3 || kind == NQ_CODEC_E5M2 || kind == NQ_CODEC_E4M3_BOUNDED ||
        kind == NQ_CODEC_E5M2_BOUNDED) {
        const uint2 w2 = kind == NQ_CODEC_E4M3 ? fp8x8<Fp8::E4M3>(v)
                       : kind == NQ_CODEC_E5M2 ? fp8x8<Fp8::E5M2>(v)
                       : kind == NQ_CODEC_E4M3_BOUNDED ? fp8x8_bounded<Fp8::E4M3>(v)
                                                       : fp8x8_bounded<Fp8::E5M2>(v);
        const uint32_t w[2] = {w2.x, w2.y};
        uint8_t* o = (uint8_t*)out;
#pragma unroll
        for (int k = 0; k < 8; ++k)
            if (i0 + k < n) o[i0 + k] = (uint8_t)(w[k / 4] >> (8 * (k & 3)));
    } else if (kind == NQ_CODEC_E2M1) {
        const uint32_t w = e2m1x8(v);
        uint8_t* o = (uint8_t*)out;
#pragma unroll
        for (int k = 0; k < 8; ++k)
            if (i0 + k < n) o[i0 + k] = (uint8_t)((w >> (4 * k)) & 0xFu);
    } else {
        uint16_t* o = (uint16_t*)out;
#pragma unroll
        for (int k = 0; k < 8; k += 2) {
            const uint32_t p = pack_bf16x2(v[k], v[k + 1]);
            if (i0 + k < n) o[i0 + k] = (uint16_t)p;
            if (i0 + k + 1 < n) o[i0 + k + 1] = (uint16_t)(p >> 16);
        }
    }
}

// One element per thread through the kernels' own arithmetic routines.
// Operand and result types per kind are given in include/nq.h.
__global__ __launch_bounds__(256) void k_diag_arith(int kind, const void* a, const void* b, void* out, int64_t n)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    // Lanes past n compute on a harmless operand and store nothing, so the
    // wavefront-wide ballot inside div6_rn sees every lane.
    const bool live = i < n;
    const int64_t k = live ? i : 0;
    switch (kind) {
    case NQ_ARITH_RCP: {
        const float r = rcp_rn(static_cast<const float*>(a)[k]);
        if (live) static_cast<float*>(out)[i] = r;
        break;
    }
    case NQ_ARITH_RSQRT: {
        const float r = rsqrt_rn(static_cast<const float*>(a)[k]);
        if (live) static_cast<float*>(out)[i] = r;
        break;
    }
    case NQ_ARITH_DIV: {
        const float y = static_cast<const float*>(a)[k], s = static_cast<const float*>(b)[k];
        const float r = div_by(y, s, 1.0f / s);
        if (live) static_cast<float*>(out)[i] = r;
        break;
    }
    case NQ_ARITH_DIV_LEN: {
        const double d = (double)static_cast<const int32_t*>(b)[k];
        const double r = div_by_len(static_cast<const double*>(a)[k], d, 1.0 / d);
        if (live) static_cast<double*>(out)[i] = r;
        break;
    }
    case NQ_ARITH_SUM_BF16X2: {
        const float r = sum2_bf16(static_cast<const uint32_t*>(a)[k], static_cast<const float*>(b)[k]);
        if (live) static_cast<float*>(out)[i] = r;
        break;
    }
    case NQ_ARITH_TOKEN_SCALE_E4M3:
    case NQ_ARITH_TOKEN_SCALE_E5M2: {
        const float amax = static_cast<const float*>(a)[k];
        float sc, inv;
        if (kind == NQ_ARITH_TOKEN_SCALE_E4M3) token_scale<Fp8::E4M3>(amax, sc, inv);
        else token_scale<Fp8::E5M2>(amax, sc, inv);
        if (live) {
            static_cast<float*>(out)[2 * i] = sc;
            static_cast<float*>(out)[2 * i + 1] = inv;
        }
        break;
    }
    default: {  // NQ_ARITH_DIV6
        const float r = div6_rn(static_cast<const float*>(a)[k]);
        if (live) static_cast<float*>(out)[i] = r;
        break;
    }
    }
}

// One pass over the data: each lane moves kCopyUnroll 16-byte pieces, a
// wavefront's pieces contiguous per step (1 KB per load instruction), every
// load issued before the first store, both non-temporal (the data is used
// once).  Measured on MI355X over 161.5 MB (half read, half written), same
// box: one piece per lane 27.2 us, two 27.7, four 28.8, eight 30.0; blocks of
// 128 or 1024 lanes no faster; a grid-stride loop of one piece 29.3.
constexpr int kCopyBlock = 256;
constexpr int kCopyUnroll = 1;

__global__ __launch_bounds__(kCopyBlock) void k_diag_copy(const uint4* src, uint4* dst, int64_t n16)
{
    const int64_t base = (int64_t)blockIdx.x * kCopyBlock * kCopyUnroll + threadIdx.x;
    u32x4_t v[kCopyUnroll];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
        const int64_t i = base + (int64_t)u * kCopyBlock;
        v[u] = i < n16 ? __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(src) + i) : u32x4_t{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
        const int64_t i = base + (int64_t)u * kCopyBlock;
        if (i < n16) __builtin_nontemporal_store(v[u], reinterpret_cast<u32x4_t*>(dst) + i);
    }
}

} // namespace nq

using namespace nq;

extern "C" const char* nq_status_string(nq_status status)
{
    switch (status) {
    case NQ_OK: return "ok";
    case NQ_ERR_NULL: return "a mandatory pointer is NULL";
    case NQ_ERR_SHAPE: return "unsupported shape (M, d, K or group layout)";
    case NQ_ERR_STRIDE: return "a leading dimension is smaller than the row length";
    case NQ_ERR_ALIAS: return "an output overlaps an input or another output";
    case NQ_ERR_LAUNCH: return "kernel launch failed";
    case NQ_ERR_ARG: return "an argument is outside its domain";
    default: return "unknown status";
    }
}

extern "C" const char* nq_version(void) { return "nq 0.1.0 gfx950"; }

extern "C" nq_status nq_diag_codec(int32_t kind, const float* in, void* out, int64_t n, void* stream)
{
    if (kind < NQ_CODEC_E4M3 || kind > NQ_CODEC_E5M2_BOUNDED) return NQ_ERR_ARG;
    if (n < 0 || n > (int64_t(1) << 40)) return NQ_ERR_SHAPE;
    if (n == 0) return NQ_OK;
    if (!in || !out) return NQ_ERR_NULL;
    const int64_t esize = kind == NQ_CODEC_BF16 ? 2 : 1;
    const Region rin[] = {region(in, 1, n, n, 4)};
    const Region rout[] = {region(out, 1, n, n, esize)};
    if (any_alias(rin, rout)) return NQ_ERR_ALIAS;
    const int64_t threads = (n + 7) / 8;
    const int64_t blocks = (threads + 255) / 256;
    if (blocks > 0x7FFFFFFF) return NQ_ERR_SHAPE;
    hipLaunchKernelGGL(k_diag_codec, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                       (int)kind, in, out, n);
    return hipGetLastError() == hipSuccess ? NQ_OK : NQ_ERR_LAUNCH;
}

extern "C" nq_status nq_diag_arith(int32_t kind, const void* a, const void* b, void* out, int64_t n,
                                   void* stream)
{
    if (kind < NQ_ARITH_RCP || kind > NQ_ARITH_TOKEN_SCALE_E5M2) return NQ_ERR_ARG;
    if (n < 0 || n > (int64_t(1) << 36)) return NQ_ERR_SHAPE;
    if (n == 0) return NQ_OK;
    const bool two = kind == NQ_ARITH_DIV || kind == NQ_ARITH_DIV_LEN || kind == NQ_ARITH_SUM_BF16X2;
    if (!a || !out || (two && !b)) return NQ_ERR_NULL;
    const int64_t asz = kind == NQ_ARITH_DIV_LEN ? 8 : 4;
    const Region rin[] = {region(a, 1, n, n, asz), region(two ? b : nullptr, 1, n, n, 4)};
    const bool pair = kind == NQ_ARITH_TOKEN_SCALE_E4M3 || kind == NQ_ARITH_TOKEN_SCALE_E5M2;
    const Region rout[] = {region(out, 1, n, n, pair ? 8 : asz)};
    if (any_alias(rin, rout)) return NQ_ERR_ALIAS;
    const int64_t blocks = (n + 255) / 256;
    if (blocks > 0x7FFFFFFF) return NQ_ERR_SHAPE;
    hipLaunchKernelGGL(k_diag_arith, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, (int)kind, a,
                       b, out, n);
    return hipGetLastError() == hipSuccess ? NQ_OK : NQ_ERR_LAUNCH;
}

extern "C" nq_status nq_diag_copy(const void* src, void* dst, int64_t bytes, void* stream)
{
    if (bytes < 0 || bytes % 16 != 0) return NQ_ERR_SHAPE;
    if (bytes == 0) return NQ_OK;
    if (!src || !dst) return NQ_ERR_NULL;
    if (!aligned(src, 16) || !aligned(dst, 16)) return NQ_ERR_ARG;
    const Region rin[] = {region(src, 1, bytes, bytes, 1)};
    const Region rout[] = {region(dst, 1, bytes, bytes, 1)};
    if (any_alias(rin, rout)) return NQ_ERR_ALIAS;
    const int64_t n16 = bytes / 16;
    const int64_t per_block = (int64_t)kCopyBlock * kCopyUnroll;
    const int64_t blocks = (n16 + per_block - 1) / per_block;
    if (blocks > 0x7FFFFFFF) return NQ_ERR_SHAPE;
    hipLaunchKernelGGL(k_diag_copy, dim3((unsigned)blocks), dim3(kCopyBlock), 0, (hipStream_t)stream,
                       (const uint4*)src, (uint4*)dst, n16);
    return hipGetLastError() == hipSuccess ? NQ_OK : NQ_ERR_LAUNCH;
}
