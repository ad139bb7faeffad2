/*
 * nq.h -- C ABI of libnq.so: fused normalization + FP8 / NVFP4 activation
 * quantization for AMD Instinct MI355X (gfx950).
 *
 * Pages cited (title, then the section in brackets):
 *   [FUSE]  "Fusing RMSNorm and FP8 Quantization Under torch.compile"
 *   [LNQ]   "feat: fused FP8 quantization output for LayerNorm"
 *           (FlashInfer pull request 3962)
 *   [NVFP4] "RMSNorm nvfp4 quant fusion for DS V3.2 / Kimi-K2.5"
 *           (TensorRT-LLM pull request 14848)
 *   [GRP]   "per_token_group_quant_8bit: multiply by reciprocal instead of
 *           dividing per element" (vLLM pull request 61343)
 *   [GRAPH] "RMSNorm/FusedRMSNorm + Quant kernels cuda graph fixes"
 *           (FlashInfer pull request 2459)
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Types.  bf16 tensors are passed as uint16_t bit patterns; OCP FP8 e4m3fn
 *   codes (largest finite 448, no infinities), packed E2M1 pairs and e4m3
 *   block-scale codes as uint8_t; scales as IEEE float.
 * Layout.  Every matrix is row-major.  A leading dimension `ld_*` is the
 *   distance between consecutive rows, in elements of that tensor, and must
 *   be >= the row length that is read or written.  A row stride larger than
 *   the row length reads a column slice in place.
 * Memory.  Every pointer is a device pointer (hipMalloc / PyTorch CUDA
 *   memory) owned by the caller.  The library never allocates, frees or
 *   synchronizes; all work is enqueued on `stream` (a hipStream_t passed as
 *   void*; NULL selects the null stream).  Scale pointers are read on the
 *   device when the kernel runs, never on the host, so every call can be
 *   captured into a hipGraph and a scale updated between replays is honoured
 *   ([LNQ] "Tests"; [GRAPH] "Description").
 * Errors.  Arguments are checked on the host before anything is enqueued.  A
 *   non-zero status means nothing was launched, except NQ_ERR_LAUNCH, which
 *   reports a failed launch.  M == 0 is a no-op that returns NQ_OK.
 *   Pointers and strides need no alignment.  Rows are read and written 16
 *   bytes at a time wherever d is a multiple of 8 and gamma / beta start on
 *   16-byte boundaries, also when the rows themselves do not (up to about a
 *   fifth slower there); otherwise an element-wise path runs (about 1.5 to
 *   1.8 times slower), with identical results.
 * Device-side preconditions (documented, not checked: checking would need a
 *   host synchronization): inputs and scales are finite; static scales are
 *   > 0 and the NVFP4 global scale is at least 2^-118; no row or group has a
 *   non-zero absolute maximum below fmax * 2^-128 (fmax = 448, or 57344 for
 *   e5m2), where the reciprocal of its scale would overflow (subnormal
 *   scales above that are handled exactly); with eps = 0 no row is all
 *   zero.
 * Aliasing.  No output may overlap an input or another output, except that
 *   residual_out may be exactly residual_in (same pointer, same ld: in-place
 *   residual update, [FUSE] "FAQ").  Overlap is decided on address ranges.
 * Threads.  The library keeps no mutable global state; calls are thread-safe.
 */
#ifndef NQ_H
#define NQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int nq_status;

#define NQ_OK 0
#define NQ_ERR_NULL (-1)        /* a mandatory pointer is NULL */
#define NQ_ERR_SHAPE (-2)       /* M < 0, M above 2^36, d <= 0, d above NQ_MAX_D, d % 16 for
                                   NVFP4, K % group, M * K / 128 of 2^31 or more for group quant */
#define NQ_ERR_STRIDE (-3)      /* a leading dimension is smaller than the row length or above
                                   2^24 elements */
#define NQ_ERR_ALIAS (-4)       /* an output overlaps an input or another output */
#define NQ_ERR_LAUNCH (-5)      /* the HIP launch failed (hipGetLastError) */
#define NQ_ERR_ARG (-6)         /* an argument value is outside its domain (eps, mode, group) */

/* Largest row length any entry point accepts. */
#define NQ_MAX_D 32768

/* Group-quant scale encodings ([GRP] "Overview", "Details"). */
#define NQ_SCALE_FP32 0         /* s = amax / 448 */
#define NQ_SCALE_UE8M0 1        /* s = amax / 448 rounded up to a power of two */

/* Option bits of the entry points that take `flags`. */
#define NQ_FLAG_BF16_SOURCE 1u  /* quantize bf16(y) instead of the fp32 y */
#define NQ_FLAG_E5M2 2u         /* FP8 codes in OCP e5m2 (largest finite 57344) instead of e4m3:
                                   dynamic scales divide by 57344, e5m2() clamps to +-57344 */
#define NQ_FLAG_GAMMA_BF16 4u   /* gamma (and beta) are bf16 [d] instead of fp32: each value is
                                   widened exactly, so the results equal those of the fp32 vector
                                   holding the same values */

/*
 * Fused (residual-add +) RMSNorm + per-token FP8 e4m3.
 * Defined by [FUSE] "TL;DR", "Where norm+quant sits" and "FAQ"; the static
 * variant's one-element device scale by [GRAPH] "Description", "Changes".
 *
 * Per row m (0 <= m < M) and column i (0 <= i < d):
 *   z_i  = bf16(x_i + r_i)        binary32 add, one bf16 rounding (RNE);
 *                                 z_i = x_i when residual_in is NULL
 *   residual_out_i = z_i          (bit-exact; may update residual_in in place)
 *   rstd = 1 / sqrt(sum_i z_i^2 / d + eps)
 *   y_i  = (z_i * rstd) * gamma_i kept in fp32 registers, never rounded to bf16
 *   dynamic (static_scale == NULL):
 *     s = max_i |y_i| / 448  -> scale_out[m];  q_i = e4m3(y_i / s)  (code 0x00
 *     for every element if s == 0, whatever the sign of y_i)
 *   static (static_scale != NULL):
 *     q_i = e4m3(y_i * (1 / static_scale[0]))  i.e. out = y / scale
 *   norm_out_i = bf16(y_i)        only when norm_out != NULL
 * e4m3() clamps to [-448, 448] and rounds to nearest-even.
 *
 *   x            [M, d] bf16, row stride ld_x               (read)
 *   residual_in  [M, d] bf16, row stride ld_r, or NULL       (read)
 *   residual_out [M, d] bf16, row stride ld_ro; NULL iff residual_in is NULL
 *   gamma        [d] fp32                                   (read)
 *   eps          >= 0, added inside the square root
 *   static_scale one fp32 on the device, or NULL for dynamic per-token scales
 *   q_out        [M, d] e4m3 codes, row stride ld_q          (written)
 *   scale_out    [M] fp32 per-token scales; required when dynamic, unused
 *                (may be NULL) when static
 *   norm_out     [M, d] bf16, row stride ld_n, or NULL
 */
nq_status nq_fused_add_rmsnorm_quant_fp8(
    const uint16_t* x, int64_t ld_x,
    const uint16_t* residual_in, int64_t ld_r,
    uint16_t* residual_out, int64_t ld_ro,
    const float* gamma, float eps,
    const float* static_scale,
    uint8_t* q_out, int64_t ld_q,
    float* scale_out,
    uint16_t* norm_out, int64_t ld_n,
    int64_t M, int64_t d, void* stream);

/*
 * The same op with an output-format choice ([LNQ] "Description" and "Tests":
 * the FP8 output may be e4m3 or e5m2).  flags: any of NQ_FLAG_E5M2,
 * NQ_FLAG_GAMMA_BF16 (NQ_ERR_ARG for other bits); every other argument as
 * above (gamma fp32, or bf16 with NQ_FLAG_GAMMA_BF16).  With NQ_FLAG_E5M2 the
 * dynamic scale is max_i |y_i| / 57344 and codes are e5m2.
 */
nq_status nq_fused_add_rmsnorm_quant_fp8_ex(
    const uint16_t* x, int64_t ld_x,
    const uint16_t* residual_in, int64_t ld_r,
    uint16_t* residual_out, int64_t ld_ro,
    const void* gamma, float eps,
    const float* static_scale, uint32_t flags,
    uint8_t* q_out, int64_t ld_q,
    float* scale_out,
    uint16_t* norm_out, int64_t ld_n,
    int64_t M, int64_t d, void* stream);

/*
 * LayerNorm + static per-tensor FP8 e4m3.
 * Defined by [LNQ] "Description" (the scale divides: out = normed / scale)
 * and the review thread; the scale is a one-element device tensor read when
 * the kernel runs ([LNQ] "Tests"; [GRAPH] "Changes").
 *
 * Per row:
 *   mu   = sum_i x_i / d
 *   c_i  = x_i - mu
 *   rstd = 1 / sqrt(sum_i c_i^2 / d + eps)      (population variance)
 *   y_i  = ((c_i * rstd) * gamma_i) + beta_i    (no fused multiply-add)
 *   q_i  = e4m3(y_i * (1 / scale[0]))
 * The two row sums are taken over 8-element chunks in binary32 and added in
 * binary64 (a chunk whose binary32 sum leaves a safe range is summed exactly
 * instead), so mu and the variance are within a few binary32 roundings of
 * the exactly summed values; rstd can differ from theirs by one unit in the
 * last place.
 *
 *   x      [M, d] bf16, row stride ld_x
 *   gamma, beta [d] fp32
 *   scale  one fp32 on the device (> 0)
 *   q_out  [M, d] e4m3 codes, row stride ld_q
 */
nq_status nq_layernorm_quant_fp8(
    const uint16_t* x, int64_t ld_x,
    const float* gamma, const float* beta, float eps,
    const float* scale,
    uint8_t* q_out, int64_t ld_q,
    int64_t M, int64_t d, void* stream);

/*
 * LayerNorm + FP8 with a static per-tensor or a dynamic per-token scale, and
 * an output-format choice.  [LNQ] "Description": the library LayerNorm has a
 * per-token quantization path besides the per-tensor one, and the FP8
 * output may be e4m3 or e5m2 ("Tests" cover both).
 *
 *   y_i as nq_layernorm_quant_fp8
 *   scale != NULL (static):  q_i = fp8(y_i * (1 / scale[0])); scale_out unused
 *   scale == NULL (dynamic): s = max_i |y_i| / fmax -> scale_out[m];
 *                            q_i = fp8(y_i / s)  (one correctly rounded
 *                            quotient per element; code 0x00 for
 *                            every element when s == 0)
 *   fmax = 448 (e4m3) or 57344 (NQ_FLAG_E5M2)
 *   flags      any of NQ_FLAG_E5M2, NQ_FLAG_GAMMA_BF16 (gamma and beta bf16);
 *              NQ_ERR_ARG for other bits
 *   scale_out  [M] fp32, required when scale is NULL
 */
nq_status nq_layernorm_quant_fp8_ex(
    const uint16_t* x, int64_t ld_x,
    const void* gamma, const void* beta, float eps,
    const float* scale, uint32_t flags,
    uint8_t* q_out, int64_t ld_q,
    float* scale_out,
    int64_t M, int64_t d, void* stream);

/*
 * Per-token-group FP8 e4m3 with one reciprocal per group.
 * Defined by [GRP] "Overview", "Details" and the commit message: scales are
 * amax / 448 per group of `group_size` contiguous elements, and elements are
 * multiplied by the correctly rounded reciprocal of the scale.
 *
 * Per row m and group g (K / group_size groups per row):
 *   amax = max |x_i| over the group
 *   NQ_SCALE_FP32:  s = amax / 448
 *   NQ_SCALE_UE8M0: s = amax / 448 rounded up to a power of two
 *                   (unchanged when already a power of two or zero)
 *   inv  = 1 / s (0 when s == 0);  q_i = e4m3(x_i * inv)
 *   scale_out[m * (K / group_size) + g] = s
 *
 *   x          [M, K] bf16, row stride ld_x
 *   group_size 128 (the only size the pages use); K % group_size == 0
 *   q_out      [M, K] e4m3 codes, row stride ld_q
 *   scale_out  [M, K / group_size] fp32, dense row-major
 */
nq_status nq_per_token_group_quant_fp8(
    const uint16_t* x, int64_t ld_x, int64_t M, int64_t K,
    int32_t group_size, int32_t scale_mode,
    uint8_t* q_out, int64_t ld_q, float* scale_out, void* stream);

/*
 * The same op with an output-format choice: flags 0 or NQ_FLAG_E5M2 (then
 * s = amax / 57344, rounded up to a power of two with NQ_SCALE_UE8M0, and
 * e5m2 codes).  Other arguments as above.
 */
nq_status nq_per_token_group_quant_fp8_ex(
    const uint16_t* x, int64_t ld_x, int64_t M, int64_t K,
    int32_t group_size, int32_t scale_mode, uint32_t flags,
    uint8_t* q_out, int64_t ld_q, float* scale_out, void* stream);

/*
 * Fused (residual-add +) RMSNorm + per-token-group FP8 e4m3, one reciprocal
 * per group (block-FP8 consumers).
 * Defined by [GRP] "Details": the fused RMSNorm + group-quant kernel (the
 * fusion target for block-FP8 models) quantizes with the standalone group
 * quantizer's reciprocal-multiply numerics; the steps per group are those of
 * nq_per_token_group_quant_fp8.
 *
 * Per row m:
 *   z_i, residual_out_i, rstd, y_i   exactly as nq_fused_add_rmsnorm_quant_fp8
 *   v_i  = y_i, or bf16(y_i) with NQ_FLAG_BF16_SOURCE (then the codes equal
 *          the unfused pipeline: a bf16 RMSNorm output fed to
 *          nq_per_token_group_quant_fp8)
 *   per group g of group_size contiguous elements (d / group_size groups):
 *     amax = max |v_i|;  s = amax / 448 (NQ_SCALE_FP32) or that value
 *     rounded up to a power of two (NQ_SCALE_UE8M0)
 *     inv = 1 / s (0 when s == 0);  q_i = e4m3(v_i * inv)
 *     scale_out[m * ld_s + g] = s
 *   norm_out_i = bf16(y_i)        only when norm_out != NULL
 *
 *   x            [M, d] bf16, row stride ld_x
 *   residual_in  [M, d] bf16, row stride ld_r, or NULL (residual-less)
 *   residual_out [M, d] bf16, row stride ld_ro; NULL iff residual_in is NULL;
 *                may equal residual_in (in place)
 *   gamma        [d] fp32
 *   group_size   128 (NQ_ERR_ARG otherwise); d % group_size == 0
 *   scale_mode   NQ_SCALE_FP32 or NQ_SCALE_UE8M0 (NQ_ERR_ARG otherwise)
 *   flags        any of NQ_FLAG_BF16_SOURCE, NQ_FLAG_E5M2 (then 448 above is
 *                57344 and the codes are e5m2), NQ_FLAG_GAMMA_BF16 (gamma is
 *                bf16); NQ_ERR_ARG for other bits
 *   q_out        [M, d] e4m3 codes, row stride ld_q
 *   scale_out    [M, d / group_size] fp32, row stride ld_s (>= d / group_size)
 *   norm_out     [M, d] bf16, row stride ld_n, or NULL
 */
nq_status nq_fused_add_rmsnorm_quant_fp8_group(
    const uint16_t* x, int64_t ld_x,
    const uint16_t* residual_in, int64_t ld_r,
    uint16_t* residual_out, int64_t ld_ro,
    const void* gamma, float eps,
    int32_t group_size, int32_t scale_mode, uint32_t flags,
    uint8_t* q_out, int64_t ld_q,
    float* scale_out, int64_t ld_s,
    uint16_t* norm_out, int64_t ld_n,
    int64_t M, int64_t d, void* stream);

/*
 * (Residual-add +) RMSNorm + NVFP4: packed E2M1 elements with one e4m3 scale
 * per 16 elements and a global fp32 decode scale.
 * Defined by [NVFP4] "Description" and the commit notes (optional residual,
 * row-strided column-slice input, d % 16 == 0, optional bf16 norm_out, a
 * fresh or in-place residual).  The block-scale formula is printed on no
 * page; this library uses:
 *   z, residual_out, rstd, y_i   exactly as nq_fused_add_rmsnorm_quant_fp8
 *   G    = 1 / global_scale[0]                    (encode scale)
 *   per block b of 16 elements:
 *     sf_b = e4m3((max |y_i| / 6) * G)            -> block_scale
 *     m_b  = G / value(sf_b)  (0 when sf_b decodes to 0)
 *     q_i  = e2m1(y_i * m_b)  (clamped to [-6, 6], nearest-even)
 *   so that y_i ~= value(q_i) * value(sf_b) * global_scale[0].
 * Packing: byte k of a block holds element 2k in bits 0-3 and element 2k+1
 * in bits 4-7; E2M1 bit 3 is the sign, magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6.
 *
 *   x            [M, d] bf16, row stride ld_x (may be a column slice)
 *   residual_in  [M, d] bf16, row stride ld_r, or NULL (residual-less)
 *   residual_out [M, d] bf16, row stride ld_ro; NULL iff residual_in is NULL
 *   gamma        [d] fp32
 *   global_scale one fp32 on the device, at least 2^-118 (then G / value(sf)
 *                is finite for every block-scale code; below that a zero
 *                element can meet an infinite multiplier, outside the contract)
 *   q_packed     [M, d/2] bytes, row stride ld_q (in bytes)
 *   block_scale  [M, d/16] e4m3 codes, row stride ld_sf, linear layout
 *   norm_out     [M, d] bf16, row stride ld_n, or NULL
 */
nq_status nq_rmsnorm_quant_nvfp4(
    const uint16_t* x, int64_t ld_x,
    const uint16_t* residual_in, int64_t ld_r,
    uint16_t* residual_out, int64_t ld_ro,
    const float* gamma, float eps,
    const float* global_scale,
    uint8_t* q_packed, int64_t ld_q,
    uint8_t* block_scale, int64_t ld_sf,
    uint16_t* norm_out, int64_t ld_n,
    int64_t M, int64_t d, void* stream);

/*
 * The same NVFP4 op with options: flags any of NQ_FLAG_BF16_SOURCE (the
 * values quantized are bf16(y_i), so the codes and block scales equal the
 * standalone quantizer applied to the bf16 norm_out -- [NVFP4] commit notes:
 * the fused op's outputs match, bit for bit, the standalone quantizer run on
 * the norm_out it returns), NQ_FLAG_GAMMA_BF16 (gamma is bf16).  NQ_ERR_ARG for other bits.
 */
nq_status nq_rmsnorm_quant_nvfp4_ex(
    const uint16_t* x, int64_t ld_x,
    const uint16_t* residual_in, int64_t ld_r,
    uint16_t* residual_out, int64_t ld_ro,
    const void* gamma, float eps,
    const float* global_scale, uint32_t flags,
    uint8_t* q_packed, int64_t ld_q,
    uint8_t* block_scale, int64_t ld_sf,
    uint16_t* norm_out, int64_t ld_n,
    int64_t M, int64_t d, void* stream);

/*
 * The unfused pipeline the fused ops replace ([FUSE] "TL;DR", "Where
 * norm+quant sits": the norm writes a bf16 activation that a second kernel
 * reads back and quantizes).  Run back to back they reproduce the unfused
 * codes and the traffic the fusion removes.
 *
 * nq_fused_add_rmsnorm_bf16: z_i, residual_out_i, rstd and y_i exactly as
 *   nq_fused_add_rmsnorm_quant_fp8; out_i = bf16(y_i).
 *     out  [M, d] bf16, row stride ld_o (written)
 *
 * nq_per_token_quant_fp8: FP8 of bf16 rows x, the quantization step of
 *   nq_fused_add_rmsnorm_quant_fp8 on y_i = x_i:
 *     dynamic (static_scale == NULL): s = max_i |x_i| / fmax -> scale_out[m],
 *       q_i = fp8(x_i / s) (code 0x00 for every element if s == 0)
 *     static: q_i = fp8(x_i * (1 / static_scale[0]))
 *   fmax = 448 (e4m3) or 57344 (flags = NQ_FLAG_E5M2; NQ_ERR_ARG for other bits)
 *     x          [M, d] bf16, row stride ld_x
 *     q_out      [M, d] FP8 codes, row stride ld_q
 *     scale_out  [M] fp32 (dynamic only)
 */
nq_status nq_fused_add_rmsnorm_bf16(
    const uint16_t* x, int64_t ld_x,
    const uint16_t* residual_in, int64_t ld_r,
    uint16_t* residual_out, int64_t ld_ro,
    const float* gamma, float eps,
    uint16_t* out, int64_t ld_o,
    int64_t M, int64_t d, void* stream);

nq_status nq_per_token_quant_fp8(
    const uint16_t* x, int64_t ld_x,
    const float* static_scale, uint32_t flags,
    uint8_t* q_out, int64_t ld_q,
    float* scale_out,
    int64_t M, int64_t d, void* stream);

/* Human-readable name of a status code (static storage, never NULL). */
const char* nq_status_string(nq_status status);

/* Library version string, e.g. "nq 0.1.0 gfx950" (static storage). */
const char* nq_version(void);

/*
 * Diagnostics (not part of the quantization path).
 *
 * nq_diag_codec: applies, element by element on the device, the exact device
 * conversion routine the kernels use, so its rounding can be compared with an
 * independent host implementation.  kind:
 *   NQ_CODEC_E4M3: out[i] = e4m3 code of in[i]   (clamp to +-448, nearest-even)
 *   NQ_CODEC_E2M1: out[i] = E2M1 code of in[i]   (clamp to +-6, nearest-even)
 *   NQ_CODEC_BF16: out16[i] = bf16 bits of in[i] (nearest-even)
 *   NQ_CODEC_E5M2: out[i] = e5m2 code of in[i]   (clamp to +-57344, nearest-even)
 *   NQ_CODEC_E4M3_BOUNDED, NQ_CODEC_E5M2_BOUNDED: the conversion without the
 *     clamp, which the dynamic-scale kernels use for quotients by a normal
 *     scale (|in[i]| at most 448 resp. 57344 times 1 + 2^-21); defined, and
 *     equal to the clamped code, only for inputs within that bound
 * `out` is uint8_t for the 8-bit formats and uint16_t for bf16.
 *
 * nq_diag_arith: applies, element by element on the device, the arithmetic
 * shortcuts the kernels take in place of a correctly rounded operation, so
 * that each can be compared with the correctly rounded result on the host
 * ([GRP] "Details": one correctly rounded division per group, the exact
 * reciprocal).  n elements; kind:
 *   NQ_ARITH_RCP:     out[i] = RN(1 / a[i]) by the hardware reciprocal and one
 *                     Newton step (the reciprocal inside 1/sqrt); fp32
 *   NQ_ARITH_RSQRT:   out[i] = RN(1 / RN(sqrt(a[i]))), the kernels' rstd step
 *                     on its argument mean + eps; fp32
 *   NQ_ARITH_DIV:     out[i] = RN(a[i] / b[i]) by Markstein's correction of
 *                     a[i] * RN(1 / b[i]) (the per-token FP8 quotient); fp32
 *   NQ_ARITH_DIV_LEN: out[i] = RN(a[i] / b[i]) in binary64 for an integer row
 *                     length b[i] in [1, 32768] (int32), from RN(1 / b[i]);
 *                     a and out are double
 *   NQ_ARITH_DIV6:    out[i] = RN(a[i] / 6) for a block maximum a[i] >= 0 (the
 *                     NVFP4 block scale's first step); fp32
 *   NQ_ARITH_SUM_BF16X2: out[i] = lo + hi + b[i] for the two bf16 halves of
 *                     the word a[i], one packed bf16 dot product with (1, 1)
 *                     (a step of LayerNorm's binary32 chunk sums; it is not
 *                     always rounded to nearest); a is uint32, b and out fp32
 *   NQ_ARITH_TOKEN_SCALE_E4M3, NQ_ARITH_TOKEN_SCALE_E5M2: out[2i] = RN(a[i] /
 *                     fmax) and out[2i + 1] = RN(1 / out[2i]) (0 for a zero
 *                     scale), fmax 448 or 57344: the per-token dynamic scale
 *                     and its reciprocal as the kernels form them from a row
 *                     maximum a[i] >= 0; a fp32, out 2n fp32
 * b is NULL for the one-operand kinds.  Errors: NQ_ERR_ARG (unknown kind),
 * NQ_ERR_NULL, NQ_ERR_SHAPE (n < 0 or n > 2^36), NQ_ERR_ALIAS (out overlaps
 * an operand).
 *
 * nq_diag_copy: copies `bytes` (a multiple of 16, both pointers 16-byte
 * aligned) with 128-bit loads and stores, a bandwidth reference for the same
 * HBM the quantization kernels stream through.
 */
#define NQ_CODEC_E4M3 0
#define NQ_CODEC_E2M1 1
#define NQ_CODEC_BF16 2
#define NQ_CODEC_E5M2 3
#define NQ_CODEC_E4M3_BOUNDED 4
#define NQ_CODEC_E5M2_BOUNDED 5
nq_status nq_diag_codec(int32_t kind, const float* in, void* out, int64_t n, void* stream);
#define NQ_ARITH_RCP 0
#define NQ_ARITH_RSQRT 1
#define NQ_ARITH_DIV 2
#define NQ_ARITH_DIV_LEN 3
#define NQ_ARITH_DIV6 4
#define NQ_ARITH_SUM_BF16X2 5
#define NQ_ARITH_TOKEN_SCALE_E4M3 6
#define NQ_ARITH_TOKEN_SCALE_E5M2 7
nq_status nq_diag_arith(int32_t kind, const void* a, const void* b, void* out, int64_t n, void* stream);
nq_status nq_diag_copy(const void* src, void* dst, int64_t bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* NQ_H */
