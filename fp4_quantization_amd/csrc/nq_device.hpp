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
constexpr float kInvE2M1Max = 0x1.555556p-3f;   // RN(1/6)
// amax at or above 6 * 2^-126 gives a normal amax / 6 (with margin: 2^-120).
constexpr float kMinNormalE2M1Quotient = 0x1p-120f;

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

// The packed conversions write one half (FP8) or one byte (E2M1) of their
// destination and keep the rest; every part is written before the word is
// used, so the first conversion of a word starts from whatever its first
// operand's register holds (no register to zero first).
__device__ __forceinline__ int any_bits(float v) { return __builtin_bit_cast(int, v); }

__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d)
{
    const float ca = clamp_e4m3(a);
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(ca, clamp_e4m3(b), any_bits(ca), false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(clamp_e4m3(c), clamp_e4m3(d), w, true);
    return (uint32_t)w;
}

// ------------------------------------------------------------ e5m2 -------
// e5m2(v): clamp to [-57344, 57344] (saturating like e4m3, so a scaled value
// never becomes infinite), then the native round-to-nearest-even conversion
// (v_cvt_pk_bf8_f32).  Four values -> one dword, value 0 in byte 0.
constexpr float kE5M2Max = 57344.0f;  // largest finite OCP e5m2 value

__device__ __forceinline__ float clamp_e5m2(float v)
{
    return __builtin_amdgcn_fmed3f(v, -kE5M2Max, kE5M2Max);
}

__device__ __forceinline__ uint32_t e5m2x4(float a, float b, float c, float d)
{
    const float ca = clamp_e5m2(a);
    int w = __builtin_amdgcn_cvt_pk_bf8_f32(ca, clamp_e5m2(b), any_bits(ca), false);
    w = __builtin_amdgcn_cvt_pk_bf8_f32(clamp_e5m2(c), clamp_e5m2(d), w, true);
    return (uint32_t)w;
}

// The FP8 output format of a kernel instance, and its largest finite value
// (the divisor of dynamic scales).
enum class Fp8 { E4M3, E5M2 };

template <Fp8 F>
constexpr float fp8_max() { return F == Fp8::E5M2 ? kE5M2Max : kE4M3Max; }

template <Fp8 F>
__device__ __forceinline__ float fp8_clamp(float v)
{
    if constexpr (F == Fp8::E5M2) return clamp_e5m2(v);
    else return clamp_e4m3(v);
}

template <Fp8 F>
__device__ __forceinline__ uint32_t fp8x4(float a, float b, float c, float d)
{
    if constexpr (F == Fp8::E5M2) return e5m2x4(a, b, c, d);
    else return e4m3x4(a, b, c, d);
}

// 8 values -> two dwords
template <Fp8 F>
__device__ __forceinline__ uint2 fp8x8(const float v[8])
{
    return make_uint2(fp8x4<F>(v[0], v[1], v[2], v[3]), fp8x4<F>(v[4], v[5], v[6], v[7]));
}

// FP8 of values known to be at most fmax * (1 + 2^-21) in magnitude: the
// native conversion alone, with no clamp.  It rounds to nearest even and
// first leaves the finite range at 464 (e4m3) and 61440 (e5m2), so every
// such value gets the code of its clamped value.  Quotients by a dynamic
// scale s = RN(amax / fmax) that is a normal number are bounded so:
// |y| / s <= amax / s <= fmax / (1 - 2^-24), and the quotient's rounding
// adds one more unit in the last place.  Checked exhaustively against the
// oracle's codec up to that bound (NQ_CODEC_*_BOUNDED).
template <Fp8 F>
__device__ __forceinline__ uint32_t fp8x4_bounded(float a, float b, float c, float d)
{
    if constexpr (F == Fp8::E5M2) {
        int w = __builtin_amdgcn_cvt_pk_bf8_f32(a, b, any_bits(a), false);
        return (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(c, d, w, true);
    } else {
        int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, any_bits(a), false);
        return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
    }
}

template <Fp8 F>
__device__ __forceinline__ uint2 fp8x8_bounded(const float v[8])
{
    return make_uint2(fp8x4_bounded<F>(v[0], v[1], v[2], v[3]), fp8x4_bounded<F>(v[4], v[5], v[6], v[7]));
}

// True when every lane of the wavefront holds a normal dynamic scale, so
// its quotients are bounded as fp8x8_bounded needs (a zero, subnormal or
// non-finite scale anywhere sends the whole wavefront through the clamped
// conversion).
__device__ __forceinline__ bool wave_scales_normal(float s)
{
    return __builtin_amdgcn_ballot_w64(!(s >= 0x1p-126f && s <= 0x1p127f)) == 0;
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
// Native gfx950 conversion.  The scale operand is 1.0 (the block
// multiplier is applied beforehand with an ordinary binary32 multiply, so
// the rounding input is exactly that product).  No clamp: measured on
// MI355X, the conversion saturates by itself (every value >= 6, infinity
// included, gives code 7; <= -6 gives 15), so it equals the nearest-even
// code of the value clamped to [-6, 6] for every non-NaN input.
__device__ __forceinline__ uint32_t e2m1x8(const float v[8])
{
    uint32_t w = (uint32_t)any_bits(v[0]);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[0], v[1], 1.0f, 0);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[2], v[3], 1.0f, 1);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[4], v[5], 1.0f, 2);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[6], v[7], 1.0f, 3);
    return w;
}

// ------------------------------------------------------- reductions -------
// Within a 16-lane DPP row: xor 1 and xor 2 inside each quad, then the
// half-row mirror (lane i <-> 7-i) and the row mirror (i <-> 15-i).  Each
// step combines the same two operands on both partner lanes (a + b == b + a
// exactly), so every lane of the row ends with bitwise the same value.
// Across the four rows of a wavefront the row results are read into scalar
// registers and combined in a fixed order; across 32 lanes one cross-lane
// exchange finishes the pair of rows.
//
// Every lane of the wavefront executes these exchanges (no reduction sits in
// a divergent branch), and every pattern reads a lane of the same row, so
// the moves are issued with bound_ctrl: no lane ever keeps its old value,
// and the compiler needs no register initialised for it (and can fold a
// move into the instruction that consumes it).
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, true);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v)
{
    return __builtin_bit_cast(float, dpp_u32<CTRL>(__builtin_bit_cast(uint32_t, v)));
}
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v)
{
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = dpp_u32<CTRL>((uint32_t)u);
    const uint32_t hi = dpp_u32<CTRL>((uint32_t)(u >> 32));
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ double readlane_f64(double v, int lane)
{
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, lane);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), lane);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ uint32_t readlane_u32(uint32_t v, int lane)
{
    return (uint32_t)__builtin_amdgcn_readlane((int)v, lane);
}

constexpr int kDppXor1 = 0xB1;        // quad_perm 1,0,3,2
constexpr int kDppXor2 = 0x4E;        // quad_perm 2,3,0,1
constexpr int kDppHalfMirror = 0x141; // row_half_mirror
constexpr int kDppMirror = 0x140;     // row_mirror

template <int W>
__device__ __forceinline__ double group_sum(double v)
{
    static_assert(W == 16 || W == 32 || W == 64, "group of 16, 32 or 64 lanes");
    v += dpp_f64<kDppXor1>(v);
    v += dpp_f64<kDppXor2>(v);
    v += dpp_f64<kDppHalfMirror>(v);
    v += dpp_f64<kDppMirror>(v);
    if constexpr (W == 32) v += __shfl_xor(v, 16, kWave);
    if constexpr (W == 64)
        v = (readlane_f64(v, 0) + readlane_f64(v, 16)) + (readlane_f64(v, 32) + readlane_f64(v, 48));
    return v;
}

// Maxima here are maxima of absolute values: non-negative binary32 (or NaN
// from a non-finite input) order exactly as their bit patterns do as
// unsigned integers, so one integer max per step replaces the float max and
// the quieting of its DPP operand (NaN, 0x7FC00000 and up, still wins).
__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }

template <int W>
__device__ __forceinline__ float group_max(float x)
{
    static_assert(W == 16 || W == 32 || W == 64, "group of 16, 32 or 64 lanes");
    uint32_t v = __builtin_bit_cast(uint32_t, x);
    v = umax(v, dpp_u32<kDppXor1>(v));
    v = umax(v, dpp_u32<kDppXor2>(v));
    v = umax(v, dpp_u32<kDppHalfMirror>(v));
    v = umax(v, dpp_u32<kDppMirror>(v));
    if constexpr (W == 32) v = umax(v, (uint32_t)__shfl_xor((int)v, 16, kWave));
    if constexpr (W == 64)
        v = umax(umax(readlane_u32(v, 0), readlane_u32(v, 16)), umax(readlane_u32(v, 32), readlane_u32(v, 48)));
    return __builtin_bit_cast(float, v);
}

// Maximum of a non-negative value (an absolute maximum) over lanes t and
// t ^ 1: one DPP exchange inside each quad.
__device__ __forceinline__ float pair_max(float x)
{
    const uint32_t v = __builtin_bit_cast(uint32_t, x);
    return __builtin_bit_cast(float, umax(v, dpp_u32<kDppXor1>(v)));
}

// Max over each aligned group of 16 lanes (one DPP row).
__device__ __forceinline__ float max16_dpp(float v) { return group_max<16>(v); }

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
        uint32_t s = __builtin_bit_cast(uint32_t, lds[first]);
#pragma unroll
        for (int i = 1; i < NW; ++i) s = umax(s, __builtin_bit_cast(uint32_t, lds[first + i]));
        v = __builtin_bit_cast(float, s);
    }
    return v;
}

// Smallest power of two >= t (t itself when it already is one; 0 stays 0):
// with t = m * 2^e, 0.5 <= m < 1, that is t when m == 0.5, else 2^e.
__device__ __forceinline__ float pow2_ceil(float t)
{
    if (t == 0.0f) return 0.0f;
    const float m = __builtin_amdgcn_frexp_mantf(t);
    const int e = __builtin_amdgcn_frexp_expf(t);
    return m == 0.5f ? t : __builtin_amdgcn_ldexpf(1.0f, e);
}

// ------------------------------------------------------- division -------
// Correctly rounded q = y / s from inv = 1 / s (itself correctly rounded):
// q0 = y * inv is within one ulp of y / s, the remainder y - s * q0 is
// exact in one fused multiply-add, and q0 + r * inv rounded once is the
// correctly rounded quotient (Markstein's theorem for round-to-nearest
// binary floating point).  The remainder is a multiple of 2^(e_y - 46)
// below 2^(e_y - 22), so it is exact for |y| >= 2^-103; the theorem also
// needs a normal s, no overflow and a quotient of at least 2^-126.  For
// smaller y the quotient can be off, but a kernel meets such y with a
// quotient whose FP8 code can be non-zero only in rows whose maximum is
// below 2^-84.  Three operations per element instead of a full division
// sequence.  The remainder is formed as -(q0 * s - y): the same value, but
// for y = -0 it is -0 rather than y + (+0) = +0, so the sum keeps the sign
// of a zero quotient (-0 / s = -0, as correctly rounded division gives);
// both negations are source modifiers, so this costs nothing.  Checked on
// the device against correctly rounded division over random and edge
// operands, signed zeros included, codes included where the quotient is
// not exact (test_div_by_matches_division).
__device__ __forceinline__ float div_by(float y, float s, float inv)
{
    const float q0 = y * inv;
    const float t = __builtin_fmaf(q0, s, -y);  // -(remainder)
    return __builtin_fmaf(-t, inv, q0);
}

// Correctly rounded binary64 a / d for a row length 1 <= d <= 2^15, from
// inv_d = RN(1 / d) formed on the host.  The same three steps as div_by:
// the remainder is exact, and the corrected sum lies within about 2^-52 ulp
// of a / d, while a / d (d has at most 15 significant bits) is either
// representable or at least 2^-16 ulp away from every rounding midpoint, so
// the final rounding agrees with the quotient's.  The sums divided here are
// 0 or at least 2^-266 in magnitude (squares and values of bf16 numbers),
// far from underflow.  Three binary64 operations instead of a division.
// Checked for every d <= 2^15 on the host (tests/test_shortcut_proofs.py)
// and on the device (test_div_by_len_every_row_length).
__device__ __forceinline__ double div_by_len(double a, double d, double inv_d)
{
    const double q0 = a * inv_d;
    const double r = __builtin_fma(-q0, d, a);
    return __builtin_fma(r, inv_d, q0);
}

// RN(1 / s) for a normal s in [2^-75, 2^64]: the hardware reciprocal
// (v_rcp_f32, about one ulp) corrected by one Newton step with fused
// multiply-adds.  One step from a one-ulp seed is not correctly rounded for
// every significand in theory; on this hardware it is exact over that whole
// range -- the device test test_rcp_rn_every_significand (tests/
// test_gpu_arith.py, through nq_diag_arith) compares it with the correctly
// rounded reciprocal for every binary32 s of those binades.
__device__ __forceinline__ float rcp_rn(float s)
{
    const float y0 = __builtin_amdgcn_rcpf(s);
    const float e = __builtin_fmaf(-s, y0, 1.0f);
    return __builtin_fmaf(e, y0, y0);
}

// 1 / sqrt(x) as two correctly rounded steps, x >= 0: s = sqrt(x)
// (correctly rounded), then RN(1 / s) by rcp_rn; the s of a positive
// binary32 x lie in [2^-75, 2^64].  s = 0 and s = infinity take the
// division's results (infinity and 0) explicitly.  Checked on the device for
// every non-negative binary32 x (test_rsqrt_rn_every_binary32).
__device__ __forceinline__ float rsqrt_rn(float x)
{
    const float s = sqrtf(x);
    float r = rcp_rn(s);
    r = s == 0.0f ? __builtin_inff() : r;
    r = s == __builtin_inff() ? 0.0f : r;
    return r;
}

// RN(amax / 6) for a block maximum amax >= 0 (the NVFP4 block scale's
// first step).  Markstein's correction from RN(1/6) (div_by) is exact
// whenever the quotient is normal (amax >= 2^-120 with margin) and gives 0
// for 0; a wavefront holding a smaller non-zero maximum takes the
// correctly rounded division instead, behind a ballot so that ordinary data
// never runs it.  Checked on the device for every finite non-negative
// binary32 (test_div6_every_binary32).
__device__ __forceinline__ float div6_rn(float amax)
{
    float per = div_by(amax, kE2M1Max, kInvE2M1Max);
    const bool tiny = amax > 0.0f && amax < kMinNormalE2M1Quotient;
    if (__builtin_amdgcn_ballot_w64(tiny) != 0) {
        // The empty volatile statement keeps this a branch: without it the
        // compiler evaluates the full division for every block and selects
        // (about 12 vector instructions per chunk).
        __asm__ volatile("");
        if (tiny) per = amax / kE2M1Max;
    }
    return per;
}

// A per-token dynamic scale s = RN(amax / fmax) and its reciprocal
// inv = RN(1 / s) (0 for a zero scale), from three-instruction sequences in
// place of two correctly rounded divisions: the quotient by Markstein's
// correction from RN(1 / fmax) (div_by: exact for a normal quotient of an
// amax far above 2^-103), the reciprocal by rcp_rn (exact for s in
// [2^-75, 2^64)).  A wavefront holding a scale outside that range -- zero,
// tiny or huge row maxima -- computes both by division instead, behind a
// vote.  Checked on the device against the divisions for every e4m3 and
// e5m2 scale an amax can give (test_token_scale_every_amax).
template <Fp8 F>
__device__ __forceinline__ void token_scale(float amax, float& s, float& inv)
{
    constexpr float kMax = fp8_max<F>();
    constexpr float kInvMax = 1.0f / kMax;  // RN(1 / fmax), formed by the compiler
    s = div_by(amax, kMax, kInvMax);
    inv = rcp_rn(s);
    const bool fast = s >= 0x1p-75f && s < 0x1p64f;
    if (__builtin_amdgcn_ballot_w64(!fast) != 0) {
        __asm__ volatile("");  // keep it a branch
        if (!fast) {
            s = amax / kMax;
            inv = s > 0.0f ? 1.0f / s : 0.0f;
        }
    }
}

// ------------------------------------------------------- row access -------
// Rows are read and written through one of two RowIO flavours:
//
//  * RowIO<true>: a buffer resource per wavefront whose base is the first
//    row the wavefront owns and whose size ends at the last element it may
//    touch.  Lanes pass 32-bit byte offsets; a masked lane passes kOOB.  The
//    hardware range check returns zeros for out-of-range loads and drops
//    out-of-range stores, so masking (the row tail, rows past M) costs no
//    branch.  Needs d % 8 == 0 for 128-bit chunks; rows may start anywhere
//    (unaligned access is enabled on this target).
//  * RowIO<false>: the same resource, for d % 8 != 0 or gamma / beta off
//    16-byte boundaries: 128-bit accesses inside the row, element by element
//    across its end (shapes with one row per wavefront only).
//
// Cache policies (the aux bits of gfx950 buffer instructions: bit 0 sc0,
// bit 1 nt, bit 4 sc1), chosen by measurement on MI355X for these streams:
// inputs read once are non-temporal, bf16 row outputs (residual, norm_out)
// are written with sc1, quantized codes non-temporal, per-group and NVFP4
// block scale rows (small pieces per row) with sc0 -- 0.3 to 1 % faster than
// non-temporal; gamma / beta use the default policy.  LayerNorm, whose codes
// are its only output, writes them with sc1: 3 % faster than non-temporal
// there, while sc1 codes slowed the RMSNorm kernels by 1-11 %.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kLoadStream = 2;              // nt
constexpr int kStoreRows = 16;              // sc1
constexpr int kStoreCodes = 2;              // nt
constexpr int kStoreCodesOnly = 16;         // sc1: codes that are a kernel's only output (LayerNorm)
constexpr int kStoreScales = 1;             // sc0: small scale rows, written in pieces
constexpr int kKeep = 0;                    // default
constexpr uint32_t kOOB = 0x80000000u;      // beyond any resource size used here
constexpr int kRsrcWord3 = 0x00020000;      // gfx9-family raw buffer descriptor word 3

// The rows a wavefront owns: `row0` and `nrows` are wavefront-uniform.
struct RowMap {
    int64_t row;   // this lane's row
    bool ok;       // row < M
    int64_t row0;  // first row of the wavefront
    int nrows;     // valid rows of the wavefront from row0 (0 when past M)
    int rel;       // row - row0
};

template <bool VEC, int POLICY, typename T>
struct RowIO;

template <int POLICY, typename T>
struct RowIO<true, POLICY, T> {
    __amdgpu_buffer_rsrc_t rsrc;
    uint32_t lane_base;  // byte offset of this lane's row from the resource base
    int cols;

    RowIO() = default;
    __device__ __forceinline__ RowIO(const T* base, int64_t ld, const RowMap& m, int ncols)
    {
        // A NULL tensor (absent residual or norm_out) gets an empty range:
        // its loads read zeros and its stores are dropped.
        const T* p = base ? base + m.row0 * ld : base;
        const uint32_t bytes = (base && m.nrows > 0)
            ? (uint32_t)(((int64_t)(m.nrows - 1) * ld + ncols) * (int64_t)sizeof(T)) : 0u;
        rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(p), (short)0, (int)bytes, kRsrcWord3);
        lane_base = (uint32_t)((int64_t)m.rel * ld * (int64_t)sizeof(T));
        cols = ncols;
    }
    __device__ __forceinline__ uint32_t off(int i, bool live) const
    {
        return live ? lane_base + (uint32_t)i * (uint32_t)sizeof(T) : kOOB;
    }
    // 16 bytes starting at element i (zeros when masked or out of range)
    __device__ __forceinline__ uint4 load16(int i, bool live) const
    {
        const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(rsrc, (int)off(i, live), 0, POLICY);
        return make_uint4(v.x, v.y, v.z, v.w);
    }
    // 16 bytes starting at element i, written by the load itself to LDS at
    // `lds` + 16 * (lane within the wavefront) (zeros when masked or out of
    // range); `lds` must be the same for every lane of the wavefront.
    __device__ __forceinline__ void load16_lds(int i, bool live, void* lds) const
    {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)lds, 16,
                                                 (int)off(i, live), 0, 0, POLICY);
    }
    // 8 bytes starting at element i
    __device__ __forceinline__ uint2 load8(int i, bool live) const
    {
        const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(rsrc, (int)off(i, live), 0, POLICY);
        return make_uint2(v.x, v.y);
    }
    __device__ __forceinline__ void store16(int i, bool live, uint4 w) const
    {
        const u32x4_t v = {w.x, w.y, w.z, w.w};
        __builtin_amdgcn_raw_buffer_store_b128(v, rsrc, (int)off(i, live), 0, POLICY);
    }
    __device__ __forceinline__ void store8(int i, bool live, uint2 w) const
    {
        const u32x2_t v = {w.x, w.y};
        __builtin_amdgcn_raw_buffer_store_b64(v, rsrc, (int)off(i, live), 0, POLICY);
    }
    __device__ __forceinline__ void store4(int i, bool live, uint32_t w) const
    {
        __builtin_amdgcn_raw_buffer_store_b32(w, rsrc, (int)off(i, live), 0, POLICY);
    }
    __device__ __forceinline__ void store1(int i, bool live, uint32_t w) const
    {
        __builtin_amdgcn_raw_buffer_store_b8((uint8_t)w, rsrc, (int)off(i, live), 0, POLICY);
    }
};

template <int POLICY, typename T>
struct RowIO<false, POLICY, T> : RowIO<true, POLICY, T> {
    // For rows whose length is not a multiple of 8 elements, and shared
    // vectors off 16-byte boundaries: an access that lies wholly inside the
    // row is the 128-bit path's; one that crosses the row's end goes element
    // by element.  Every shape on this path gives each wavefront one row, so
    // the resource ends at the row's last element and its range check drops
    // the elements past it (loads read zeros there).
    using Base = RowIO<true, POLICY, T>;
    RowIO() = default;
    __device__ __forceinline__ RowIO(const T* base, int64_t ld, const RowMap& m, int ncols)
        : Base(base, ld, m, ncols) {}

    template <int N>
    __device__ __forceinline__ bool inside(int i) const { return i + N / (int)sizeof(T) <= this->cols; }
    __device__ __forceinline__ uint32_t elem(int i, bool live) const
    {
        const int o = (int)this->off(i, live);
        if constexpr (sizeof(T) == 1) return __builtin_amdgcn_raw_buffer_load_b8(this->rsrc, o, 0, POLICY);
        else if constexpr (sizeof(T) == 2) return __builtin_amdgcn_raw_buffer_load_b16(this->rsrc, o, 0, POLICY);
        else return __builtin_amdgcn_raw_buffer_load_b32(this->rsrc, o, 0, POLICY);
    }
    __device__ __forceinline__ void put(int i, bool live, uint32_t v) const
    {
        const int o = (int)this->off(i, live);
        if constexpr (sizeof(T) == 1) __builtin_amdgcn_raw_buffer_store_b8((uint8_t)v, this->rsrc, o, 0, POLICY);
        else if constexpr (sizeof(T) == 2) __builtin_amdgcn_raw_buffer_store_b16((uint16_t)v, this->rsrc, o, 0, POLICY);
        else __builtin_amdgcn_raw_buffer_store_b32(v, this->rsrc, o, 0, POLICY);
    }
    // N bytes from element i, one element per access
    template <int N>
    __device__ __forceinline__ void load_words(int i, bool live, uint32_t (&w)[N / 4]) const
    {
        constexpr int E = N / (int)sizeof(T), PER = 4 / (int)sizeof(T);
#pragma unroll
        for (int q = 0; q < N / 4; ++q) w[q] = 0u;
#pragma unroll
        for (int k = 0; k < E; ++k) w[k / PER] |= elem(i + k, live) << (8 * sizeof(T) * (k % PER));
    }
    template <int N>
    __device__ __forceinline__ void store_words(int i, bool live, const uint32_t (&w)[N / 4]) const
    {
        constexpr int E = N / (int)sizeof(T), PER = 4 / (int)sizeof(T);
#pragma unroll
        for (int k = 0; k < E; ++k) put(i + k, live, w[k / PER] >> (8 * sizeof(T) * (k % PER)));
    }
    __device__ __forceinline__ uint2 load8(int i, bool live) const
    {
        if (inside<8>(i)) return Base::load8(i, live);
        uint32_t w[2];
        load_words<8>(i, live, w);
        return make_uint2(w[0], w[1]);
    }
    __device__ __forceinline__ uint4 load16(int i, bool live) const
    {
        if (inside<16>(i)) return Base::load16(i, live);
        uint32_t w[4];
        load_words<16>(i, live, w);
        return make_uint4(w[0], w[1], w[2], w[3]);
    }
    __device__ __forceinline__ void store16(int i, bool live, uint4 v) const
    {
        if (inside<16>(i)) return Base::store16(i, live, v);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
        store_words<16>(i, live, w);
    }
    __device__ __forceinline__ void store8(int i, bool live, uint2 v) const
    {
        if (inside<8>(i)) return Base::store8(i, live, v);
        const uint32_t w[2] = {v.x, v.y};
        store_words<8>(i, live, w);
    }
    __device__ __forceinline__ void store4(int i, bool live, uint32_t v) const
    {
        if (inside<4>(i)) return Base::store4(i, live, v);
        const uint32_t w[1] = {v};
        store_words<4>(i, live, w);
    }
    __device__ __forceinline__ void store1(int i, bool live, uint32_t v) const { put(i, live, v); }
};

// Plain global streaming accesses (non-temporal) for kernels that index a
// whole tensor rather than per-wavefront rows.  The pointers may be
// misaligned: the types say so (byte alignment), and the accesses stay one
// 128-bit or 64-bit instruction (unaligned access is enabled on this target).
typedef u32x4_t u32x4_any_t __attribute__((aligned(1)));
typedef u32x2_t u32x2_any_t __attribute__((aligned(1)));
__device__ __forceinline__ uint4 ld_global_stream16(const void* p)
{
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_any_t*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void st_global_stream8(void* p, uint2 w)
{
    const u32x2_any_t v = {w.x, w.y};
    __builtin_nontemporal_store(v, reinterpret_cast<u32x2_any_t*>(p));
}

// Hides a value's provenance from the optimizer (an empty register-only asm
// statement, no memory access), so values recomputed in a later phase are
// not merged with the earlier phase's copies and kept live in between.
__device__ __forceinline__ void opaque(uint4& w)
{
    asm volatile("" : "+v"(w.x), "+v"(w.y), "+v"(w.z), "+v"(w.w));
}
__device__ __forceinline__ int opaque(int v)
{
    asm volatile("" : "+v"(v));
    return v;
}
__device__ __forceinline__ float opaque(float v)
{
    asm volatile("" : "+v"(v));
    return v;
}

__device__ __forceinline__ void unpack_bf16x8(uint4 w, float v[8])
{
    v[0] = bf16_lo(w.x); v[1] = bf16_hi(w.x);
    v[2] = bf16_lo(w.y); v[3] = bf16_hi(w.y);
    v[4] = bf16_lo(w.z); v[5] = bf16_hi(w.z);
    v[6] = bf16_lo(w.w); v[7] = bf16_hi(w.w);
}

// Sum of the squares of one chunk of 8 bf16 values (packed), in binary64.
// Every square is exact in binary64, so the chunk sum rounds at most in its
// last bit.
__device__ __forceinline__ double sumsq_chunk_unpacked(const float z[8])
{
    double acc = 0.0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const double zd = (double)z[k];
        acc = fma(zd, zd, acc);
    }
    return acc;
}
__device__ __forceinline__ double sumsq_chunk(uint4 w)
{
    float z[8];
    unpack_bf16x8(w, z);
    return sumsq_chunk_unpacked(z);
}


// Row sums in binary32 chunks with a binary64 safety net.  Each 8-element
// chunk is summed in binary32 and the chunk sums are added in binary64.  A
// chunk sum is trusted while it lies in a range where neither an overflow
// nor flushed or subnormal products can have touched it; a lane holding a
// chunk outside that range sums all its chunks exactly in binary64 instead
// (a branch no wavefront takes on ordinary data).  Within the range the
// binary32 sum is the exact one to within its few roundings: 2^-24
// relative each for the fused multiply-adds of a sum of squares (which has
// no cancellation); for the packed dot products of a plain sum, each step
// lands within 2 units in the last place (1.47 measured at worst) of the
// largest magnitude among its terms and its result -- it truncates the terms it
// aligns, so it is not always the nearest binary32 -- and is exact while
// every term's bits lie within the 24 bits below the largest one's leading
// bit (test_sum_bf16x2_error_bound).

// lo + hi + acc for the two bf16 halves of a packed word: one packed bf16
// dot product with (1, 1).
__device__ __forceinline__ float sum2_bf16(uint32_t w, float acc)
{
    const bf16x2_t one = __builtin_bit_cast(bf16x2_t, 0x3F803F80u);
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w), one, acc, false);
}

// Sum of the 8 bf16 values of a packed chunk: four packed bf16 dot products
// with (1, 1).
__device__ __forceinline__ float sum_chunk_f32(uint4 w)
{
    return sum2_bf16(w.w, sum2_bf16(w.z, sum2_bf16(w.y, sum2_bf16(w.x, 0.0f))));
}
// Whether a chunk's binary32 plain sum can be trusted: tiny (or cancelled),
// huge and non-finite sums are recomputed.
__device__ __forceinline__ bool sum_ok(float p)
{
    const float a = __builtin_fabsf(p);
    return a >= 0x1p-100f && a <= 0x1p100f;
}

// Sum of the squares of 8 binary32 values.
__device__ __forceinline__ float sumsq_chunk_f32(const float c[8])
{
    float p = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k) p = __builtin_fmaf(c[k], c[k], p);
    return p;
}
// Whether a chunk's binary32 sum of squares can be trusted (its squares
// cannot have underflowed or overflowed).
__device__ __forceinline__ bool sumsq_ok(float p) { return p >= 0x1p-60f && p <= 0x1p60f; }

// 8 fp32 (two 16-byte loads) of a vector such as gamma.
template <bool VEC, int POLICY>
__device__ __forceinline__ void load_f32x8(const RowIO<VEC, POLICY, float>& io, int e, bool live, float v[8])
{
    const uint4 a = io.load16(e, live);
    const uint4 b = io.load16(e + 4, live);
    v[0] = __uint_as_float(a.x); v[1] = __uint_as_float(a.y);
    v[2] = __uint_as_float(a.z); v[3] = __uint_as_float(a.w);
    v[4] = __uint_as_float(b.x); v[5] = __uint_as_float(b.y);
    v[6] = __uint_as_float(b.z); v[7] = __uint_as_float(b.w);
}

} // namespace nq
