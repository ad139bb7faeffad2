/* shortcut_proofs.c -- host checks of two arithmetic shortcuts the GPU
 * kernels take in place of a correctly rounded division (test code; it
 * restates the kernels' operation sequences in plain C with fma()/fmaf(),
 * and compares them with IEEE division, which the host computes correctly
 * rounded).
 *
 *   quotient by a row length, binary64:
 *       q0 = a * RN(1/d);  r = fma(-q0, d, a);  q = fma(r, RN(1/d), q0)
 *     claimed equal to RN(a / d) for every integer 1 <= d <= 2^15 and every
 *     a that is 0 or of magnitude in [2^-266, 2^272] (the sums of squares and
 *     of values of bf16 numbers that the kernels divide).
 *   block maximum over 6, binary32:
 *       q0 = a * RN(1/6);  r = fmaf(-q0, 6, a);  q = fmaf(r, RN(1/6), q0)
 *     claimed equal to RN(a / 6) for every finite a >= 2^-120.
 *
 * Page: "per_token_group_quant_8bit: multiply by reciprocal instead of
 * dividing per element" (vLLM pull request 61343), "Details": one correctly
 * rounded division per group, an exact reciprocal.
 *
 * Built with -ffp-contract=off (nothing fused beyond the explicit fma calls).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

static uint64_t splitmix(uint64_t *s)
{
    uint64_t z = (*s += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

static double div_len(double a, double d, double inv)
{
    const double q0 = a * inv;
    const double r = fma(-q0, d, a);
    return fma(r, inv, q0);
}

static int bad64(double a, int32_t d)
{
    const double dd = (double)d;
    const double got = div_len(a, dd, 1.0 / dd);
    const double want = a / dd;
    return memcmp(&got, &want, 8) != 0;
}

/* Round the non-negative integer n (< 2^127) to 53 significant bits, nearest
 * even, and return it times 2^e as a double. */
static double round_to_double(unsigned __int128 n, int e)
{
    int len = 0;
    for (unsigned __int128 t = n; t; t >>= 1) ++len;
    int shift = len > 53 ? len - 53 : 0;
    if (shift > 0) {
        const unsigned __int128 half = (unsigned __int128)1 << (shift - 1);
        const unsigned __int128 mask = ((unsigned __int128)1 << shift) - 1;
        const unsigned __int128 rem = n & mask;
        n >>= shift;
        if (rem > half || (rem == half && (n & 1))) ++n;
    }
    return ldexp((double)(uint64_t)n, e + shift);
}

/* Every d in [1, dmax], `per_d` numerators of each of three kinds:
 *   random: a random 53-bit significand at a random exponent in range;
 *   near-midpoint: the double nearest to d times a midpoint between two
 *     consecutive doubles, and its two neighbours (quotients within a few
 *     ulps of 2^-53 relative of a rounding boundary, the hardest cases);
 *   exact: d times a random integer of at most 38 bits (exact quotients).
 * Returns the number of mismatches; the first one is written to bad_a/bad_d. */
int64_t sp_div_len_check(int32_t dmax, int32_t per_d, uint64_t seed, double *bad_a, int32_t *bad_d)
{
    int64_t bad = 0;
    for (int32_t d = 1; d <= dmax; ++d) {
        uint64_t s = seed ^ ((uint64_t)d * 0x632BE59BD9B4E019ull);
        for (int32_t i = 0; i < per_d; ++i) {
            double cand[5];
            int nc = 0;
            /* random */
            const uint64_t sig = (splitmix(&s) >> 11) | (1ull << 52);
            const int e = (int)(splitmix(&s) % 538) - 266 - 52;  /* magnitude in [2^-266, 2^272) */
            cand[nc++] = ldexp((double)sig, e);
            /* near-midpoint: d * (2Q + 1) * 2^(e2 - 53), Q a 53-bit significand */
            const uint64_t Q = (splitmix(&s) >> 11) | (1ull << 52);
            const int e2 = (int)(splitmix(&s) % 400) - 200;
            const unsigned __int128 N = (unsigned __int128)(uint64_t)d * (unsigned __int128)(2 * Q + 1);
            const double a = round_to_double(N, e2 - 53);
            cand[nc++] = a;
            cand[nc++] = nextafter(a, 0.0);
            cand[nc++] = nextafter(a, INFINITY);
            /* exact */
            const uint64_t k = splitmix(&s) >> 26;  /* 38 bits */
            cand[nc++] = ldexp((double)((uint64_t)d * k), (int)(splitmix(&s) % 200) - 100);
            for (int c = 0; c < nc; ++c) {
                const double v = (splitmix(&s) & 1) ? -cand[c] : cand[c];
                if (bad64(v, d)) {
                    if (bad == 0) { *bad_a = v; *bad_d = d; }
                    ++bad;
                }
            }
        }
    }
    return bad;
}

static float div6(float a)
{
    const float inv = 0x1.555556p-3f;  /* RN(1/6) */
    const float q0 = a * inv;
    const float r = fmaf(-q0, 6.0f, a);
    return fmaf(r, inv, q0);
}

/* Every binary32 bit pattern in [lo, hi] (non-negative finite values);
 * returns the number of mismatches against RN(a / 6) and the smallest and
 * largest mismatching patterns. */
int64_t sp_div6_check(uint32_t lo, uint32_t hi, uint32_t *first_bad, uint32_t *last_bad)
{
    int64_t bad = 0;
    uint32_t fb = 0xFFFFFFFFu, lb = 0;
#pragma omp parallel for reduction(+ : bad) reduction(min : fb) reduction(max : lb) schedule(static)
    for (int64_t u = lo; u <= (int64_t)hi; ++u) {
        float a;
        const uint32_t bits = (uint32_t)u;
        memcpy(&a, &bits, 4);
        const float got = div6(a);
        const float want = (float)((double)a / 6.0);  /* double rounding is innocuous for division */
        if (memcmp(&got, &want, 4) != 0) {
            ++bad;
            if (bits < fb) fb = bits;
            if (bits > lb) lb = bits;
        }
    }
    *first_bad = fb;
    *last_bad = lb;
    return bad;
}
