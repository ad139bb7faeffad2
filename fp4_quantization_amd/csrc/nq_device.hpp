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

__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d)
{
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(clamp_e4m3(a), clamp_e4m3(b), 0, false);
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
    int w = __builtin_amdgcn_cvt_pk_bf8_f32(clamp_e5m2(a), clamp_e5m2(b), 0, false);
    w = __builtin_amdgcn_cvt_pk_bf8_f32(clamp_e5m2(c), clamp_e5m2(d), w, true);
    return (uint32_t)w;
}

// The FP8 output format of a kernel instance, and its largest finite value
// (the divisor of dynamic scales).
enum class Fp8 { E4M3, E5M2 };

template <Fp8 F>
constexpr float fp8_max() { return F == Fp8::E5M2 ? kE5M2Max : kE4M3Max; }

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
    uint32_t w = 0;
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
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v)
{
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, CTRL, 0xF, 0xF, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), CTRL, 0xF, 0xF, false);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ double readlane_f64(double v, int lane)
{
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, lane);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), lane);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ float readlane_f32(float v, int lane)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
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

template <int W>
__device__ __forceinline__ float group_max(float v)
{
    static_assert(W == 16 || W == 32 || W == 64, "group of 16, 32 or 64 lanes");
    v = fmaxf(v, dpp_f32<kDppXor1>(v));
    v = fmaxf(v, dpp_f32<kDppXor2>(v));
    v = fmaxf(v, dpp_f32<kDppHalfMirror>(v));
    v = fmaxf(v, dpp_f32<kDppMirror>(v));
    if constexpr (W == 32) v = fmaxf(v, __shfl_xor(v, 16, kWave));
    if constexpr (W == 64)
        v = fmaxf(fmaxf(readlane_f32(v, 0), readlane_f32(v, 16)), fmaxf(readlane_f32(v, 32), readlane_f32(v, 48)));
    return v;
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
        float s = lds[first];
#pragma unroll
        for (int i = 1; i < NW; ++i) s = fmaxf(s, lds[first + i]);
        v = s;
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
// binary floating point; it needs no overflow and a normal s, and a
// quotient below 2^-126 only arises where every e4m3/E2M1 code is zero).
// Three operations per element instead of a full division sequence.
__device__ __forceinline__ float div_by(float y, float s, float inv)
{
    const float q0 = y * inv;
    const float r = __builtin_fmaf(-q0, s, y);
    return __builtin_fmaf(r, inv, q0);
}

// Correctly rounded binary64 a / d for a row length 1 <= d <= 2^15, from
// inv_d = RN(1 / d) formed on the host.  The same three steps as div_by:
// the remainder is exact, and the corrected sum lies within about 2^-52 ulp
// of a / d, while a / d (d has at most 15 significant bits) is either
// representable or at least 2^-16 ulp away from every rounding midpoint, so
// the final rounding agrees with the quotient's.  The sums divided here are
// 0 or at least 2^-266 in magnitude (squares and values of bf16 numbers),
// far from underflow.  Three binary64 operations instead of a division.
__device__ __forceinline__ double div_by_len(double a, double d, double inv_d)
{
    const double q0 = a * inv_d;
    const double r = __builtin_fma(-q0, d, a);
    return __builtin_fma(r, inv_d, q0);
}

// 1 / sqrt(x) as two correctly rounded steps, x >= 0: s = sqrt(x), then
// RN(1 / s) by one Newton step from the hardware reciprocal.  An exhaustive
// run on MI355X found that step exact for every normal s up to 2^125; the
// s of a positive binary32 x lie in [2^-75, 2^64].  s = 0 and s = infinity
// take the division's results (infinity and 0) explicitly.
__device__ __forceinline__ float rsqrt_rn(float x)
{
    const float s = sqrtf(x);
    const float y0 = __builtin_amdgcn_rcpf(s);
    const float e = __builtin_fmaf(-s, y0, 1.0f);
    float r = __builtin_fmaf(e, y0, y0);
    r = s == 0.0f ? __builtin_inff() : r;
    r = s == __builtin_inff() ? 0.0f : r;
    return r;
}

// ------------------------------------------------------- row access -------
// Rows are read and written through one of two RowIO flavours:
//
//  * RowIO<true>: a buffer resource per wavefront whose base is the first
//    row the wavefront owns and whose size ends at the last element it may
//    touch.  Lanes pass 32-bit byte offsets; a masked lane passes kOOB.  The
//    hardware range check returns zeros for out-of-range loads and drops
//    out-of-range stores, so masking (the row tail, rows past M) costs no
//    branch.  Needs 16-byte aligned rows and d % 8 == 0 for 128-bit chunks.
//  * RowIO<false>: plain per-element global accesses with explicit bounds
//    checks, for odd d or misaligned pointers.
//
// Cache policies (the aux bits of gfx950 buffer instructions: bit 0 sc0,
// bit 1 nt, bit 4 sc1), chosen by measurement on MI355X for these streams:
// inputs read once are non-temporal, bf16 row outputs (residual, norm_out)
// are written with sc1, quantized codes non-temporal, per-group and NVFP4
// block scale rows (small pieces per row) with sc0 -- 0.3 to 1 % faster than
// non-temporal; gamma / beta use the default policy.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kLoadStream = 2;              // nt
constexpr int kStoreRows = 16;              // sc1
constexpr int kStoreCodes = 2;              // nt
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
struct RowIO<false, POLICY, T> {
    T* row;
    bool ok;
    int cols;

    RowIO() = default;
    __device__ __forceinline__ RowIO(const T* base, int64_t ld, const RowMap& m, int ncols)
        : row(const_cast<T*>(base) + (m.ok ? m.row : 0) * ld), ok(m.ok && base != nullptr), cols(ncols) {}

    // element-wise: n bytes from element i, each element bounds-checked
    template <int N>
    __device__ __forceinline__ void load_bytes(int i, bool live, uint8_t (&b)[N]) const
    {
        constexpr int E = N / (int)sizeof(T);
#pragma unroll
        for (int k = 0; k < E; ++k) {
            T v = (ok && live && i + k < cols) ? row[i + k] : T(0);
            __builtin_memcpy(&b[k * sizeof(T)], &v, sizeof(T));
        }
    }
    template <int N>
    __device__ __forceinline__ void store_bytes(int i, bool live, const uint8_t (&b)[N]) const
    {
        constexpr int E = N / (int)sizeof(T);
#pragma unroll
        for (int k = 0; k < E; ++k) {
            if (ok && live && i + k < cols) {
                T v;
                __builtin_memcpy(&v, &b[k * sizeof(T)], sizeof(T));
                row[i + k] = v;
            }
        }
    }
    __device__ __forceinline__ uint2 load8(int i, bool live) const
    {
        uint8_t b[8];
        load_bytes<8>(i, live, b);
        uint2 w;
        __builtin_memcpy(&w, b, 8);
        return w;
    }
    __device__ __forceinline__ uint4 load16(int i, bool live) const
    {
        uint8_t b[16];
        load_bytes<16>(i, live, b);
        uint4 w;
        __builtin_memcpy(&w, b, 16);
        return w;
    }
    __device__ __forceinline__ void store16(int i, bool live, uint4 w) const
    {
        uint8_t b[16];
        __builtin_memcpy(b, &w, 16);
        store_bytes<16>(i, live, b);
    }
    __device__ __forceinline__ void store8(int i, bool live, uint2 w) const
    {
        uint8_t b[8];
        __builtin_memcpy(b, &w, 8);
        store_bytes<8>(i, live, b);
    }
    __device__ __forceinline__ void store4(int i, bool live, uint32_t w) const
    {
        uint8_t b[4];
        __builtin_memcpy(b, &w, 4);
        store_bytes<4>(i, live, b);
    }
    __device__ __forceinline__ void store1(int i, bool live, uint32_t w) const
    {
        if (ok && live && i < cols) row[i] = (T)w;
    }
};

// Plain global streaming accesses (non-temporal) for kernels that index a
// whole tensor rather than per-wavefront rows.
__device__ __forceinline__ uint4 ld_global_stream16(const void* p)
{
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void st_global_stream8(void* p, uint2 w)
{
    const u32x2_t v = {w.x, w.y};
    __builtin_nontemporal_store(v, reinterpret_cast<u32x2_t*>(p));
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
