// nq_device.hpp -- device building blocks shared by the gfx950 kernels:
// bf16 unpack/pack, e4m3 and E2M1 packing with the native gfx950
// conversions, team reductions (DPP / cross-lane within a wavefront, LDS
// across wavefronts), and 128-bit row-chunk loads and stores.
//
// Pages cited: [FUSE] "Fusing RMSNorm and FP8 Quantization Under
// torch.compile"; [NVFP4] "RMSNorm nvfp4 quant fusion for DS V3.2 /
// Kimi-K2.5"; [GRP] "per_token_group_quant_8bit: multiply by reciprocal
// instead of dividing per element".
//
// Built with -ffp-contract=off: every float expression below is the
// sequence of correctly rounded binary32 operations it spells out (HIP's
// default float division and sqrtf are correctly rounded on gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nq {

constexpr int kWave = 64;          // CDNA wavefront width
constexpr float kE4M3Max = 448.0f; // largest finite OCP e4m3fn value
constexpr float kE2M1Max = 6.0f;   // largest E2M1 magnitude

// ------------------------------------------------------------ bf16 -------
// A bf16 is the upper half of a binary32, so widening is exact.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two binary32 -> two bf16 (round to nearest even, v_cvt_pk_bf16_f32);
// `a` lands in bits 0-15.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b)
{
    f32x2_t v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// Round a binary32 to bf16 and widen it back (the value a bf16 store keeps).
__device__ __forceinline__ float round_bf16(float a) { return bf16_lo(pack_bf16x2(a, 0.0f)); }

// ------------------------------------------------------------ e4m3 -------
// e4m3(v): clamp to [-448, 448] (the format has no infinities, so
// saturation is the only overflow), then the native round-to-nearest-even
// conversion.  Four values -> one dword, value 0 in byte 0.
__device__ __forceinline__ float clamp_e4m3(float v)
{
    return __builtin_amdgcn_fmed3f(v, -kE4M3Max, kE4M3Max);
}

__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d)
{
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(clamp_e4m3(a), clamp_e4m3(b), 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(clamp_e4m3(c), clamp_e4m3(d), w, true);
    return (uint32_t)w;
}

// Decode of an e4m3 code (used for the NVFP4 block scale): sign, 4-bit
// exponent with bias 7, 3-bit mantissa, subnormals at exponent 0.  Codes
// reaching here come from e4m3x4 of a non-negative clamped value, so never
// NaN.
__device__ __forceinline__ float e4m3_value(uint32_t c)
{
    const uint32_t e = (c >> 3) & 0xFu, m = c & 0x7u;
    // normal: 2^(e-7) * (1 + m/8) -> binary32 exponent e - 7 + 127
    const float normal = __uint_as_float(((e + 120u) << 23) | (m << 20));
    const float sub = (float)m * 0.001953125f; // m * 2^-9
    const float mag = e ? normal : sub;
    return (c & 0x80u) ? -mag : mag;
}

// ------------------------------------------------------------ E2M1 -------
// E2M1 magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6 (codes 0-7), bit 3 the sign.
// Two values -> one byte, the first in bits 0-3 ([NVFP4]: packed E2M1).
#ifndef NQ_E2M1_SOFTWARE
// Native gfx950 conversion.  The scale operand is 1.0 (the block
// multiplier is applied beforehand with an ordinary binary32 multiply, so
// the rounding input is exactly that product); the input is clamped to
// [-6, 6] first.
__device__ __forceinline__ uint32_t e2m1x8(const float v[8])
{
    uint32_t w = 0;
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(
        w, __builtin_amdgcn_fmed3f(v[0], -kE2M1Max, kE2M1Max),
        __builtin_amdgcn_fmed3f(v[1], -kE2M1Max, kE2M1Max), 1.0f, 0);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(
        w, __builtin_amdgcn_fmed3f(v[2], -kE2M1Max, kE2M1Max),
        __builtin_amdgcn_fmed3f(v[3], -kE2M1Max, kE2M1Max), 1.0f, 1);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(
        w, __builtin_amdgcn_fmed3f(v[4], -kE2M1Max, kE2M1Max),
        __builtin_amdgcn_fmed3f(v[5], -kE2M1Max, kE2M1Max), 1.0f, 2);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(
        w, __builtin_amdgcn_fmed3f(v[6], -kE2M1Max, kE2M1Max),
        __builtin_amdgcn_fmed3f(v[7], -kE2M1Max, kE2M1Max), 1.0f, 3);
    return w;
}
#else
// Comparison form: each threshold is a midpoint between neighbouring
// magnitudes; ">" at a midpoint whose lower neighbour has the even code
// and ">=" where the upper one does implements ties-to-even.
__device__ __forceinline__ uint32_t e2m1_code(float v)
{
    const float a = fabsf(v);
    uint32_t c = (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) +
                 (a > 2.5f) + (a >= 3.5f) + (a > 5.0f);
    return c | (__float_as_uint(v) >> 31 << 3);
}
__device__ __forceinline__ uint32_t e2m1x8(const float v[8])
{
    uint32_t w = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) w |= e2m1_code(v[k]) << (4 * k);
    return w;
}
#endif

// ------------------------------------------------------- reductions -------
// Butterfly over aligned groups of W lanes (W a power of two <= 64): every
// lane ends with the same value, because each step adds the same two
// operands (a + b == b + a exactly).
template <int W>
__device__ __forceinline__ double group_sum(double v)
{
#pragma unroll
    for (int off = W / 2; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
    return v;
}

template <int W>
__device__ __forceinline__ float group_max(float v)
{
#pragma unroll
    for (int off = W / 2; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
    return v;
}

// Max over each aligned group of 16 lanes (one DPP row) with four DPP
// moves: xor 1, xor 2 inside each quad, then the half-row and row mirrors.
__device__ __forceinline__ float max16_dpp(float v)
{
    v = fmaxf(v, __builtin_amdgcn_update_dpp(0.0f, v, 0xB1, 0xF, 0xF, false));  // quad_perm 1,0,3,2
    v = fmaxf(v, __builtin_amdgcn_update_dpp(0.0f, v, 0x4E, 0xF, 0xF, false));  // quad_perm 2,3,0,1
    v = fmaxf(v, __builtin_amdgcn_update_dpp(0.0f, v, 0x141, 0xF, 0xF, false)); // row_half_mirror
    v = fmaxf(v, __builtin_amdgcn_update_dpp(0.0f, v, 0x140, 0xF, 0xF, false)); // row_mirror
    return v;
}

// Team reductions.  A team of TEAM lanes owns one row; TEAM <= 64 stays
// inside a wavefront, TEAM > 64 spans TEAM/64 wavefronts of the block and
// finishes through `lds` (one slot per wavefront of the block) in a fixed
// order, so every lane of the team gets the bitwise same result.
template <int TEAM>
__device__ __forceinline__ double team_sum(double v, double* lds)
{
    constexpr int W = TEAM < kWave ? TEAM : kWave;
    v = group_sum<W>(v);
    if constexpr (TEAM > kWave) {
        constexpr int NW = TEAM / kWave;
        const int wave = threadIdx.x / kWave;
        if ((threadIdx.x & (kWave - 1)) == 0) lds[wave] = v;
        __syncthreads();
        const int first = wave / NW * NW;
        double s = lds[first];
#pragma unroll
        for (int i = 1; i < NW; ++i) s += lds[first + i];
        v = s;
    }
    return v;
}

template <int TEAM>
__device__ __forceinline__ float team_max(float v, float* lds)
{
    constexpr int W = TEAM < kWave ? TEAM : kWave;
    v = group_max<W>(v);
    if constexpr (TEAM > kWave) {
        constexpr int NW = TEAM / kWave;
        const int wave = threadIdx.x / kWave;
        if ((threadIdx.x & (kWave - 1)) == 0) lds[wave] = v;
        __syncthreads();
        const int first = wave / NW * NW;
        float s = lds[first];
#pragma unroll
        for (int i = 1; i < NW; ++i) s = fmaxf(s, lds[first + i]);
        v = s;
    }
    return v;
}

// ------------------------------------------------------- row chunks -------
// A chunk is 8 consecutive elements of a row.  VEC: the chunk is complete
// (d % 8 == 0) and every base and stride is aligned for a 128-bit access.
// Otherwise elements are accessed one by one and those at or beyond d are
// skipped (loads give 0).

template <bool VEC>
__device__ __forceinline__ uint4 load_bf16x8(const uint16_t* row, int e, int d, bool ok)
{
    if constexpr (VEC) {
        if (ok) return *reinterpret_cast<const uint4*>(row + e);
        return make_uint4(0u, 0u, 0u, 0u);
    } else {
        uint32_t h[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) h[k] = (ok && e + k < d) ? (uint32_t)row[e + k] : 0u;
        return make_uint4(h[0] | h[1] << 16, h[2] | h[3] << 16, h[4] | h[5] << 16, h[6] | h[7] << 16);
    }
}

__device__ __forceinline__ void unpack_bf16x8(uint4 w, float v[8])
{
    v[0] = bf16_lo(w.x); v[1] = bf16_hi(w.x);
    v[2] = bf16_lo(w.y); v[3] = bf16_hi(w.y);
    v[4] = bf16_lo(w.z); v[5] = bf16_hi(w.z);
    v[6] = bf16_lo(w.w); v[7] = bf16_hi(w.w);
}

template <bool VEC>
__device__ __forceinline__ void store_bf16x8(uint16_t* row, int e, int d, bool ok, uint4 w)
{
    if constexpr (VEC) {
        if (ok) *reinterpret_cast<uint4*>(row + e) = w;
    } else {
        const uint32_t p[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int k = 0; k < 8; ++k)
            if (ok && e + k < d) row[e + k] = (uint16_t)(p[k / 2] >> (16 * (k & 1)));
    }
}

template <bool VEC>
__device__ __forceinline__ void load_f32x8(const float* p, int e, int d, bool ok, float v[8])
{
    if constexpr (VEC) {
        if (ok) {
            const float4 a = reinterpret_cast<const float4*>(p + e)[0];
            const float4 b = reinterpret_cast<const float4*>(p + e)[1];
            v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
            v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
        } else {
#pragma unroll
            for (int k = 0; k < 8; ++k) v[k] = 0.0f;
        }
    } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = (ok && e + k < d) ? p[e + k] : 0.0f;
    }
}

// 8 e4m3 codes of a chunk: 64-bit store.
template <bool VEC>
__device__ __forceinline__ void store_u8x8(uint8_t* row, int e, int d, bool ok, uint2 w)
{
    if constexpr (VEC) {
        if (ok) *reinterpret_cast<uint2*>(row + e) = w;
    } else {
        const uint32_t p[2] = {w.x, w.y};
#pragma unroll
        for (int k = 0; k < 8; ++k)
            if (ok && e + k < d) row[e + k] = (uint8_t)(p[k / 4] >> (8 * (k & 3)));
    }
}

} // namespace nq
