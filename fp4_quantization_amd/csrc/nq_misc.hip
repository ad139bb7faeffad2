// nq_misc.hip -- status strings, version, and the two diagnostic kernels:
// the device conversion routines applied element-wise (so their rounding can
// be compared with an independent host codec) and a 128-bit copy used as
// the bandwidth reference for the same HBM.
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
    if (kind == NQ_CODEC_E4M3 || kind == NQ_CODEC_E5M2) {
        const uint2 w2 = kind == NQ_CODEC_E4M3 ? fp8x8<Fp8::E4M3>(v) : fp8x8<Fp8::E5M2>(v);
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

__global__ __launch_bounds__(256) void k_diag_copy(const uint4* src, uint4* dst, int64_t n16)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
        dst[i] = src[i];
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
    if (kind != NQ_CODEC_E4M3 && kind != NQ_CODEC_E2M1 && kind != NQ_CODEC_BF16 && kind != NQ_CODEC_E5M2)
        return NQ_ERR_ARG;
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
    // enough blocks to fill every CU several times over; grid-stride beyond
    int64_t blocks = (n16 + 255) / 256;
    if (blocks > 256 * 64) blocks = 256 * 64;
    hipLaunchKernelGGL(k_diag_copy, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                       (const uint4*)src, (uint4*)dst, n16);
    return hipGetLastError() == hipSuccess ? NQ_OK : NQ_ERR_LAUNCH;
}
