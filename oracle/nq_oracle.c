/*
 * nq_oracle.c -- plain, slow, single-threaded CPU oracle for fused
 * normalization + FP8 / NVFP4 activation quantization.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the yardstick the GPU library is
 * checked against.  Only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark may load it.  It shares no code, header, table or
 * constant generator with the GPU library (fp4_quantization_amd/csrc), and
 * the GPU library never loads it.
 *
 * Pages cited (title, then the section named in brackets):
 *   [FUSE]  "Fusing RMSNorm and FP8 Quantization Under torch.compile"
 *           (netraruntime.com blog)
 *   [LNQ]   "feat: fused FP8 quantization output for LayerNorm"
 *           (FlashInfer pull request 3962)
 *   [NVFP4] "RMSNorm nvfp4 quant fusion for DS V3.2 / Kimi-K2.5"
 *           (TensorRT-LLM pull request 14848)
 *   [GRP]   "per_token_group_quant_8bit: multiply by reciprocal instead of
 *           dividing per element" (vLLM pull request 61343)
 *   [GRAPH] "RMSNorm/FusedRMSNorm + Quant kernels cuda graph fixes"
 *           (FlashInfer pull request 2459)
 *
 * Arithmetic rules.  Every float operation is one IEEE binary32 operation
 * rounded to nearest-even (x86-64 SSE, built with -ffp-contract=off, no
 * -ffast-math, so no fused multiply-add and no excess precision).  Row sums
 * are accumulated in binary64 and rounded to binary32 once; every summand is
 * exact in binary64.  The pages fix neither the accumulator precision nor the
 * operation order; the readings taken here are listed in the repository's
 * design notes and repeated at each function.
 *
 * FP8 outputs are e4m3 (largest finite 448) or e5m2 (largest finite 57344),
 * chosen per call; dynamic scales divide by the chosen format's largest
 * finite value.
 *
 * Pinning.  Every function here is checked by the CPU tests against things
 * other than itself: closed forms of the formats, library conversions
 * (PyTorch's bf16, float8_e4m3fn and float8_e5m2 casts), brute force on small inputs, an
 * independent binary64 recomputation, and invariants and statistics the pages
 * state.  One part is "parity unpinned": the NVFP4 block-scale operation order
 * and the meaning of the global scale (or_rmsnorm_quant_nvfp4) are fixed by no
 * page; they are checked only for self-consistency and the invariants below.
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>
#include <string.h>

#define OR_OK 0
#define OR_ERR_ARG (-1)

/* ------------------------------------------------------------------------ */
/* bf16: the upper half of a binary32.                                       */
/* ------------------------------------------------------------------------ */

static uint32_t f2u(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float u2f(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

float or_bf16_decode(uint16_t h) { return u2f((uint32_t)h << 16); }

/* Round a binary32 to the nearest bf16, ties to even mantissa.  The 16 bits
 * that are dropped are compared with the halfway pattern 0x8000 directly. */
uint16_t or_bf16_encode(float v)
{
    uint32_t u = f2u(v);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) /* NaN */
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t keep = u >> 16, drop = u & 0xFFFFu;
    if (drop > 0x8000u || (drop == 0x8000u && (keep & 1u)))
        keep += 1u; /* carries into the exponent correctly, up to inf */
    return (uint16_t)keep;
}

/* ------------------------------------------------------------------------ */
/* OCP FP8 E4M3 ("e4m3fn"): 1 sign, 4 exponent bits (bias 7), 3 mantissa     */
/* bits, no infinities, 0x7F / 0xFF are NaN, largest finite 448.  The format */
/* is the one [FUSE] names under "References" (FP8 formats for deep          */
/* learning); the largest finite value 448 is the divisor of the dynamic     */
/* scale.                                                                    */
/* ------------------------------------------------------------------------ */

float or_e4m3_decode(uint8_t c)
{
    int sign = c >> 7, e = (c >> 3) & 0xF, m = c & 0x7;
    float mag;
    if (e == 0xF && m == 0x7) return NAN;
    if (e == 0) mag = ldexpf((float)m / 8.0f, -6);          /* subnormal */
    else        mag = ldexpf(1.0f + (float)m / 8.0f, e - 7); /* normal */
    return sign ? -mag : mag;
}

/* Nearest-value encoder shared by both small formats: `mags` lists the
 * non-negative finite values in code order (code i has magnitude mags[i],
 * strictly increasing).  The input magnitude is first clamped to the largest
 * value; then the two neighbours lo <= a <= hi are found by comparison and a
 * is compared with their midpoint, which is exact in binary64.  A tie goes to
 * the even code. */
static unsigned nearest_code(float a, const double *mags, unsigned n)
{
    if (!(a > 0.0f)) return 0; /* zero (NaN is outside the contract) */
    if ((double)a >= mags[n - 1]) return n - 1;
    unsigned lo = 0;
    while (lo + 1 < n && mags[lo + 1] <= (double)a) ++lo;
    if (mags[lo] == (double)a) return lo;
    unsigned hi = lo + 1;
    double mid = (mags[lo] + mags[hi]) / 2.0;
    if ((double)a < mid) return lo;
    if ((double)a > mid) return hi;
    return (lo % 2u == 0u) ? lo : hi;
}

static double e4m3_mags[127];
static double e2m1_mags[8];
static int tables_ready = 0;

static void init_tables(void)
{
    if (tables_ready) return;
    for (unsigned c = 0; c < 127; ++c) e4m3_mags[c] = (double)or_e4m3_decode((uint8_t)c);
    static const double e2[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
    for (unsigned c = 0; c < 8; ++c) e2m1_mags[c] = e2[c];
    tables_ready = 1;
}

/* E4(v): clamp to [-448, 448], round to nearest e4m3 value, ties to even.
 * The sign bit is kept, so a negative value that rounds to zero gives 0x80. */
uint8_t or_e4m3_encode(float v)
{
    init_tables();
    float a = fabsf(v);
    unsigned code = nearest_code(a, e4m3_mags, 127);
    return (uint8_t)(code | (signbit(v) ? 0x80u : 0u));
}

/* ------------------------------------------------------------------------ */
/* OCP FP8 E5M2: 1 sign, 5 exponent bits (bias 15), 2 mantissa bits;         */
/* exponent 31 holds infinities (mantissa 0) and NaNs; largest finite 57344. */
/* [LNQ] "Description" and "Tests": the FP8 output may be e4m3 or e5m2.      */
/* The encoder saturates like the e4m3 one (clamp to +-57344, then nearest,  */
/* ties to even): a scaled value never becomes infinite.                     */
/* ------------------------------------------------------------------------ */

float or_e5m2_decode(uint8_t c)
{
    int sign = c >> 7, e = (c >> 2) & 0x1F, m = c & 0x3;
    float mag;
    if (e == 0x1F) mag = m ? NAN : INFINITY;
    else if (e == 0) mag = ldexpf((float)m / 4.0f, -14);          /* subnormal */
    else             mag = ldexpf(1.0f + (float)m / 4.0f, e - 15); /* normal */
    return sign ? -mag : mag;
}

static double e5m2_mags[124];
static int e5m2_ready = 0;

uint8_t or_e5m2_encode(float v)
{
    if (!e5m2_ready) {
        for (unsigned c = 0; c < 124; ++c) e5m2_mags[c] = (double)or_e5m2_decode((uint8_t)c);
        e5m2_ready = 1;
    }
    unsigned code = nearest_code(fabsf(v), e5m2_mags, 124);
    return (uint8_t)(code | (signbit(v) ? 0x80u : 0u));
}

/* The FP8 format an op writes: 0 = e4m3 (largest finite 448), 1 = e5m2
 * (largest finite 57344).  Dynamic scales divide the absolute maximum by
 * the format's largest finite value. */
#define OR_FP8_E4M3 0
#define OR_FP8_E5M2 1

static float fp8_max(int32_t fmt) { return fmt == OR_FP8_E5M2 ? 57344.0f : 448.0f; }
static uint8_t fp8_encode(float v, int32_t fmt)
{ return fmt == OR_FP8_E5M2 ? or_e5m2_encode(v) : or_e4m3_encode(v); }

/* E2M1 (the 4-bit element of NVFP4 [NVFP4] "Description"): magnitudes
 * 0, 0.5, 1, 1.5, 2, 3, 4, 6 for codes 0..7 and bit 3 the sign. */
float or_e2m1_decode(uint8_t c)
{
    static const float mag[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};
    float v = mag[c & 7u];
    return (c & 8u) ? -v : v;
}

/* E2(v): clamp to [-6, 6], nearest E2M1 value, ties to the even code. */
uint8_t or_e2m1_encode(float v)
{
    init_tables();
    unsigned code = nearest_code(fabsf(v), e2m1_mags, 8);
    return (uint8_t)(code | (signbit(v) ? 8u : 0u));
}

/* Bulk forms for the tests. */
void or_bf16_encode_n(const float *v, uint16_t *out, int64_t n)
{ for (int64_t i = 0; i < n; ++i) out[i] = or_bf16_encode(v[i]); }
void or_e4m3_encode_n(const float *v, uint8_t *out, int64_t n)
{ for (int64_t i = 0; i < n; ++i) out[i] = or_e4m3_encode(v[i]); }
void or_e4m3_decode_n(const uint8_t *c, float *out, int64_t n)
{ for (int64_t i = 0; i < n; ++i) out[i] = or_e4m3_decode(c[i]); }
void or_e2m1_encode_n(const float *v, uint8_t *out, int64_t n)
{ for (int64_t i = 0; i < n; ++i) out[i] = or_e2m1_encode(v[i]); }
void or_e5m2_encode_n(const float *v, uint8_t *out, int64_t n)
{ for (int64_t i = 0; i < n; ++i) out[i] = or_e5m2_encode(v[i]); }
void or_e5m2_decode_n(const uint8_t *c, float *out, int64_t n)
{ for (int64_t i = 0; i < n; ++i) out[i] = or_e5m2_decode(c[i]); }

/* ------------------------------------------------------------------------ */
/* Shared row steps, written out once in the order the pages describe.       */
/* ------------------------------------------------------------------------ */

/* RMSNorm reciprocal: rstd = 1 / sqrt(mean(z^2) + eps), the mean over d
 * (not d-1) and eps inside the square root; z^2 is exact in binary64 because
 * z is a bf16 value, the sum is rounded to binary32 once, and the square
 * root and the reciprocal are each correctly rounded binary32 operations.
 * [FUSE] "FAQ": the first of the two reductions gives rstd. */
static float rms_rstd(const float *z, int64_t d, float eps)
{
    double s = 0.0;
    for (int64_t i = 0; i < d; ++i) s += (double)z[i] * (double)z[i];
    float ms = (float)(s / (double)d);
    float t = ms + eps;
    float root = sqrtf(t);
    return 1.0f / root;
}

/* Residual add and RMSNorm of one row into fp32 y (kept, as the fused kernel
 * keeps it in registers: [FUSE] "Where norm+quant sits").
 *   z_i = bf16(x_i + r_i)  (the add is a binary32 add, then one bf16
 *                           rounding; residual_out receives z)
 *   y_i = (z_i * rstd) * gamma_i
 * With no residual, z_i = x_i. */
static void add_rmsnorm_row(const uint16_t *x, const uint16_t *r, uint16_t *r_out,
                            const float *gamma, float eps, int64_t d,
                            float *z, float *y)
{
    for (int64_t i = 0; i < d; ++i) {
        float xi = or_bf16_decode(x[i]);
        if (r) {
            float sum = xi + or_bf16_decode(r[i]);
            uint16_t zb = or_bf16_encode(sum);
            z[i] = or_bf16_decode(zb);
        } else {
            z[i] = xi;
        }
    }
    /* Written after all reads so that residual_out may alias residual_in. */
    if (r_out)
        for (int64_t i = 0; i < d; ++i) r_out[i] = or_bf16_encode(z[i]);
    float rstd = rms_rstd(z, d, eps);
    for (int64_t i = 0; i < d; ++i) {
        float n = z[i] * rstd;
        y[i] = n * gamma[i];
    }
}

/* Per-token dynamic FP8 of one fp32 row ([FUSE] "Where norm+quant sits";
 * the formula itself is not printed there, so this follows the plain
 * reading: scale = amax / 448, code = E4(y / scale), one division per
 * element ([GRP] "Details": the per-token path was left dividing each
 * element exactly); for e5m2 the divisor is 57344.  An all-zero row stores scale
 * 0 and codes 0. */
static float quant_fp8_dynamic_row(const float *y, int64_t d, uint8_t *q, int32_t fmt)
{
    float amax = 0.0f;
    for (int64_t i = 0; i < d; ++i) {
        float a = fabsf(y[i]);
        if (a > amax) amax = a;
    }
    float s = amax / fp8_max(fmt);
    for (int64_t i = 0; i < d; ++i)
        q[i] = (s > 0.0f) ? fp8_encode(y[i] / s, fmt) : 0u;
    return s;
}

/* Static FP8 of one fp32 row: out = y / scale, applied as y * (1 / scale)
 * ([LNQ] "Description": the scale divides; [GRAPH] "Changes": the kernel
 * forms scale_inv = 1 / scale[0] from the one-element tensor). */
static void quant_fp8_static_row(const float *y, int64_t d, float inv, uint8_t *q, int32_t fmt)
{
    for (int64_t i = 0; i < d; ++i) q[i] = fp8_encode(y[i] * inv, fmt);
}

/* The quantization step of O2 on its own, for rows of fp32 values the test
 * chooses (dynamic when static_scale is NULL).  Same code as above. */
int or_quant_fp8_rows(const float *y, int64_t M, int64_t d, const float *static_scale,
                      uint8_t *q, float *scale_out, int32_t fmt)
{
    if (M < 0 || d <= 0 || !y || !q || (!static_scale && !scale_out)) return OR_ERR_ARG;
    float inv = static_scale ? 1.0f / static_scale[0] : 0.0f;
    for (int64_t m = 0; m < M; ++m) {
        if (static_scale) quant_fp8_static_row(y + m * d, d, inv, q + m * d, fmt);
        else scale_out[m] = quant_fp8_dynamic_row(y + m * d, d, q + m * d, fmt);
    }
    return OR_OK;
}

static int check_rows(int64_t M, int64_t d, int64_t ld_x)
{ return (M < 0 || d <= 0 || ld_x < d) ? OR_ERR_ARG : OR_OK; }

/* ------------------------------------------------------------------------ */
/* O2: fused (residual-add +) RMSNorm + per-token FP8, dynamic or static.    */
/* [FUSE] "TL;DR", "Where norm+quant sits", "FAQ"; static scale as a         */
/* one-element device tensor: [GRAPH] "Description", "Changes".              */
/* ------------------------------------------------------------------------ */
int or_fused_add_rmsnorm_quant_fp8(
    const uint16_t *x, int64_t ld_x,
    const uint16_t *residual_in, int64_t ld_r,
    uint16_t *residual_out, int64_t ld_ro,
    const float *gamma, float eps,
    const float *static_scale,       /* host pointer, NULL = dynamic */
    uint8_t *q_out, int64_t ld_q,
    float *scale_out,                /* [M], dynamic only */
    uint16_t *norm_out, int64_t ld_n,/* optional bf16(y) */
    float *y_out, int64_t ld_y,      /* optional fp32 y, for the tests */
    float *zbuf, float *ybuf,        /* caller scratch, d floats each */
    int32_t fmt,                     /* OR_FP8_E4M3 or OR_FP8_E5M2 */
    int64_t M, int64_t d)
{
    if (check_rows(M, d, ld_x) || !gamma || !q_out || !zbuf || !ybuf) return OR_ERR_ARG;
    if (!static_scale && !scale_out) return OR_ERR_ARG;
    float inv = static_scale ? 1.0f / static_scale[0] : 0.0f;
    for (int64_t m = 0; m < M; ++m) {
        add_rmsnorm_row(x + m * ld_x, residual_in ? residual_in + m * ld_r : NULL,
                        residual_out ? residual_out + m * ld_ro : NULL,
                        gamma, eps, d, zbuf, ybuf);
        if (static_scale) quant_fp8_static_row(ybuf, d, inv, q_out + m * ld_q, fmt);
        else scale_out[m] = quant_fp8_dynamic_row(ybuf, d, q_out + m * ld_q, fmt);
        if (norm_out)
            for (int64_t i = 0; i < d; ++i) norm_out[m * ld_n + i] = or_bf16_encode(ybuf[i]);
        if (y_out) memcpy(y_out + m * ld_y, ybuf, (size_t)d * sizeof(float));
    }
    return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* O6: the unfused two-kernel pipeline the fusion replaces: the norm output  */
/* is rounded to bf16 first, and the quantizer reads that ([FUSE] "TL;DR",   */
/* "Where norm+quant sits": two roundings instead of one).  Used only to     */
/* reproduce the pages' fused-vs-unfused statistics; never a parity target.  */
/* ------------------------------------------------------------------------ */
int or_unfused_rmsnorm_quant_fp8(
    const uint16_t *x, int64_t ld_x,
    const uint16_t *residual_in, int64_t ld_r,
    const float *gamma, float eps,
    const float *static_scale,
    uint8_t *q_out, int64_t ld_q, float *scale_out,
    float *zbuf, float *ybuf, int64_t M, int64_t d)
{
    if (check_rows(M, d, ld_x) || !gamma || !q_out || !zbuf || !ybuf) return OR_ERR_ARG;
    if (!static_scale && !scale_out) return OR_ERR_ARG;
    float inv = static_scale ? 1.0f / static_scale[0] : 0.0f;
    for (int64_t m = 0; m < M; ++m) {
        add_rmsnorm_row(x + m * ld_x, residual_in ? residual_in + m * ld_r : NULL,
                        NULL, gamma, eps, d, zbuf, ybuf);
        for (int64_t i = 0; i < d; ++i) ybuf[i] = or_bf16_decode(or_bf16_encode(ybuf[i]));
        if (static_scale) quant_fp8_static_row(ybuf, d, inv, q_out + m * ld_q, OR_FP8_E4M3);
        else scale_out[m] = quant_fp8_dynamic_row(ybuf, d, q_out + m * ld_q, OR_FP8_E4M3);
    }
    return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* O3: LayerNorm + static-scale FP8 ([LNQ] "Description", review thread).    */
/*   mu  = mean(x)                     (binary64 sum, rounded once)          */
/*   c_i = x_i - mu                                                          */
/*   var = mean(c^2)                   (population variance, two passes)     */
/*   rstd = 1 / sqrt(var + eps)                                              */
/*   y_i = ((c_i * rstd) * gamma_i) + beta_i                                 */
/*   q_i = E(y_i * (1 / scale[0]))                                           */
/* O8: the same y with a dynamic per-token scale instead ([LNQ]             */
/* "Description": the library's LayerNorm also has a per-token path, left   */
/* unconnected there): s = amax(y) / fmax -> scale_out[m], q_i = E(y_i / s), */
/* one division per element like the RMSNorm per-token op ([GRP] "Details"). */
/* E is e4m3 or e5m2 (fmt; [LNQ] "Tests" cover both).                       */
/* ------------------------------------------------------------------------ */
int or_layernorm_quant_fp8(
    const uint16_t *x, int64_t ld_x,
    const float *gamma, const float *beta, float eps,
    const float *scale,               /* host pointer to the one element; NULL = dynamic */
    uint8_t *q_out, int64_t ld_q,
    float *scale_out,                 /* [M], dynamic only */
    float *y_out, int64_t ld_y,       /* optional */
    float *cbuf, float *ybuf, int32_t fmt, int64_t M, int64_t d)
{
    if (check_rows(M, d, ld_x) || !gamma || !beta || !q_out || !cbuf || !ybuf) return OR_ERR_ARG;
    if (!scale && !scale_out) return OR_ERR_ARG;
    float inv = scale ? 1.0f / scale[0] : 0.0f;
    for (int64_t m = 0; m < M; ++m) {
        const uint16_t *xr = x + m * ld_x;
        double s = 0.0;
        for (int64_t i = 0; i < d; ++i) s += (double)or_bf16_decode(xr[i]);
        float mu = (float)(s / (double)d);
        for (int64_t i = 0; i < d; ++i) cbuf[i] = or_bf16_decode(xr[i]) - mu;
        double v = 0.0;
        for (int64_t i = 0; i < d; ++i) v += (double)cbuf[i] * (double)cbuf[i];
        float var = (float)(v / (double)d);
        float t = var + eps;
        float rstd = 1.0f / sqrtf(t);
        for (int64_t i = 0; i < d; ++i) {
            float n = cbuf[i] * rstd;
            float g = n * gamma[i];
            ybuf[i] = g + beta[i];
        }
        if (scale) quant_fp8_static_row(ybuf, d, inv, q_out + m * ld_q, fmt);
        else scale_out[m] = quant_fp8_dynamic_row(ybuf, d, q_out + m * ld_q, fmt);
        if (y_out) memcpy(y_out + m * ld_y, ybuf, (size_t)d * sizeof(float));
    }
    return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* O4: per-token-group FP8 with reciprocal multiply ([GRP] "Overview",       */
/* "Details").  Per group of `group` contiguous elements along K:            */
/*   amax = max |x_i|                                                        */
/*   fp32 mode : s = amax / 448                                              */
/*   UE8M0 mode: t = amax / 448; s = t when t is 0 or a power of two, else   */
/*               the next power of two above t (so |x| / s <= 448)           */
/*   inv = 1 / s (one correctly rounded division per group; 0 when s = 0)    */
/*   q_i = E4(x_i * inv);  scales stored row-major [M, K / group]            */
/* For e5m2 output (fmt) 448 becomes 57344 and E4 becomes E5.                */
/* ------------------------------------------------------------------------ */
static float pow2_ceil(float t)
{
    if (t == 0.0f) return 0.0f;
    int e;
    float m = frexpf(t, &e); /* t = m * 2^e, 0.5 <= m < 1 */
    if (m == 0.5f) return t;
    return ldexpf(1.0f, e);
}

int or_per_token_group_quant_fp8(
    const uint16_t *x, int64_t ld_x, int64_t M, int64_t K, int32_t group,
    int32_t ue8m0, uint8_t *q_out, int64_t ld_q, float *scale_out, int32_t fmt)
{
    if (M < 0 || K <= 0 || group <= 0 || K % group || ld_x < K || !q_out || !scale_out)
        return OR_ERR_ARG;
    int64_t G = K / group;
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t g = 0; g < G; ++g) {
            const uint16_t *xg = x + m * ld_x + g * group;
            float amax = 0.0f;
            for (int32_t i = 0; i < group; ++i) {
                float a = fabsf(or_bf16_decode(xg[i]));
                if (a > amax) amax = a;
            }
            float s = amax / fp8_max(fmt);
            if (ue8m0) s = pow2_ceil(s);
            float inv = (s > 0.0f) ? 1.0f / s : 0.0f;
            for (int32_t i = 0; i < group; ++i)
                q_out[m * ld_q + g * group + i] = fp8_encode(or_bf16_decode(xg[i]) * inv, fmt);
            scale_out[m * G + g] = s;
        }
    }
    return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* O7: fused (residual-add +) RMSNorm + per-token-group FP8 with reciprocal  */
/* multiply ([GRP] "Details": the fused RMSNorm + group-quant kernel, the    */
/* fusion pass's target for block-FP8 models, uses the same reciprocal-     */
/* multiply numerics as the standalone group quantizer).  z, residual_out,  */
/* rstd and y as in O2; then per group of `group` contiguous elements of    */
/* the row, exactly O4's steps on the group's values v_i:                   */
/*   amax = max |v_i|; s = amax / 448 (UE8M0: next power of two, as O4);     */
/*   inv = 1 / s (0 when s = 0); q_i = E4(v_i * inv); scale_out[m, g] = s.    */
/* (e5m2 output: 57344 and E5 in place of 448 and E4.)                      */
/* Source of v: y itself (fp32, the default), or with bf16_source the bf16  */
/* rounding of y -- the unfused pipeline (norm output stored as bf16, then  */
/* quantized), which the page's fused/unfused agreement implies.            */
/* ------------------------------------------------------------------------ */
int or_fused_add_rmsnorm_quant_fp8_group(
    const uint16_t *x, int64_t ld_x,
    const uint16_t *residual_in, int64_t ld_r,
    uint16_t *residual_out, int64_t ld_ro,
    const float *gamma, float eps,
    int32_t group, int32_t ue8m0, int32_t bf16_source,
    uint8_t *q_out, int64_t ld_q,
    float *scale_out, int64_t ld_s,   /* [M, d / group], row stride ld_s */
    uint16_t *norm_out, int64_t ld_n,
    float *y_out, int64_t ld_y,
    float *zbuf, float *ybuf, int32_t fmt, int64_t M, int64_t d)
{
    if (check_rows(M, d, ld_x) || group <= 0 || d % group || !gamma || !q_out || !scale_out ||
        ld_s < d / group || !zbuf || !ybuf)
        return OR_ERR_ARG;
    int64_t G = d / group;
    for (int64_t m = 0; m < M; ++m) {
        add_rmsnorm_row(x + m * ld_x, residual_in ? residual_in + m * ld_r : NULL,
                        residual_out ? residual_out + m * ld_ro : NULL,
                        gamma, eps, d, zbuf, ybuf);
        if (norm_out)
            for (int64_t i = 0; i < d; ++i) norm_out[m * ld_n + i] = or_bf16_encode(ybuf[i]);
        if (y_out) memcpy(y_out + m * ld_y, ybuf, (size_t)d * sizeof(float));
        if (bf16_source)
            for (int64_t i = 0; i < d; ++i) ybuf[i] = or_bf16_decode(or_bf16_encode(ybuf[i]));
        for (int64_t g = 0; g < G; ++g) {
            const float *v = ybuf + g * group;
            float amax = 0.0f;
            for (int32_t i = 0; i < group; ++i) {
                float a = fabsf(v[i]);
                if (a > amax) amax = a;
            }
            float s = amax / fp8_max(fmt);
            if (ue8m0) s = pow2_ceil(s);
            float inv = (s > 0.0f) ? 1.0f / s : 0.0f;
            for (int32_t i = 0; i < group; ++i)
                q_out[m * ld_q + g * group + i] = fp8_encode(v[i] * inv, fmt);
            scale_out[m * ld_s + g] = s;
        }
    }
    return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* O5: (residual-add +) RMSNorm + NVFP4 ([NVFP4] "Description", commit       */
/* notes).  z, residual_out, rstd and y as in O2, x read with row stride     */
/* ld_x (an in-place column slice).  With the global decode scale s_g > 0:   */
/*   G = 1 / s_g                                                             */
/*   per block of 16 elements: amax_b = max |y_i|                            */
/*     sf  = E4((amax_b / 6) * G)        (stored code, e4m3)                 */
/*     sfd = value of sf                                                     */
/*     m_b = G / sfd  (0 when sfd = 0)                                       */
/*     q_i = E2(y_i * m_b)                                                   */
/*   byte k of a block holds element 2k in the low nibble, 2k+1 in the high. */
/* so that y_i ~= dec2(q_i) * sfd * s_g.  mode_b = 1 quantizes bf16(y_i)     */
/* instead of y_i (the bf16-sourced epilogue the pull request checks        */
/* against its standalone quantizer).                                        */
/* PARITY UNPINNED: the block-scale operation order and the global-scale    */
/* semantics above are printed on no page; they are the plain reading.      */
/* Tests pin the saturation invariants, sign symmetry, equivariance under   */
/* halving s_g, permutation within blocks and the bf16-sourced mode, but a  */
/* different rounding order of the block scale would pass them too.         */
/* ------------------------------------------------------------------------ */
int or_rmsnorm_quant_nvfp4(
    const uint16_t *x, int64_t ld_x,
    const uint16_t *residual_in, int64_t ld_r,
    uint16_t *residual_out, int64_t ld_ro,
    const float *gamma, float eps,
    const float *global_scale,        /* host pointer, s_g */
    uint8_t *q_packed, int64_t ld_q,  /* [M, d/2] */
    uint8_t *block_scale, int64_t ld_sf, /* [M, d/16] */
    uint16_t *norm_out, int64_t ld_n,
    float *y_out, int64_t ld_y,
    float *zbuf, float *ybuf, int32_t mode_b, int64_t M, int64_t d)
{
    if (check_rows(M, d, ld_x) || d % 16 || !gamma || !global_scale || !q_packed ||
        !block_scale || !zbuf || !ybuf)
        return OR_ERR_ARG;
    float Genc = 1.0f / global_scale[0];
    for (int64_t m = 0; m < M; ++m) {
        add_rmsnorm_row(x + m * ld_x, residual_in ? residual_in + m * ld_r : NULL,
                        residual_out ? residual_out + m * ld_ro : NULL,
                        gamma, eps, d, zbuf, ybuf);
        if (norm_out)
            for (int64_t i = 0; i < d; ++i) norm_out[m * ld_n + i] = or_bf16_encode(ybuf[i]);
        if (y_out) memcpy(y_out + m * ld_y, ybuf, (size_t)d * sizeof(float));
        if (mode_b)
            for (int64_t i = 0; i < d; ++i) ybuf[i] = or_bf16_decode(or_bf16_encode(ybuf[i]));
        for (int64_t b = 0; b < d / 16; ++b) {
            const float *yb = ybuf + b * 16;
            float amax = 0.0f;
            for (int i = 0; i < 16; ++i) {
                float a = fabsf(yb[i]);
                if (a > amax) amax = a;
            }
            float per = amax / 6.0f;
            uint8_t sf = or_e4m3_encode(per * Genc);
            float sfd = or_e4m3_decode(sf);
            float mult = (sfd > 0.0f) ? Genc / sfd : 0.0f;
            block_scale[m * ld_sf + b] = sf;
            for (int k = 0; k < 8; ++k) {
                uint8_t lo = or_e2m1_encode(yb[2 * k] * mult);
                uint8_t hi = or_e2m1_encode(yb[2 * k + 1] * mult);
                q_packed[m * ld_q + b * 8 + k] = (uint8_t)(lo | (hi << 4));
            }
        }
    }
    return OR_OK;
}

/* Library identity, so the tests can tell this build from the GPU one. */
const char *or_name(void) { return "nq_oracle (plain C, single-threaded)"; }
