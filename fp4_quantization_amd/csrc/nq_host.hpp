// nq_host.hpp -- host-side argument checks shared by the C-ABI entry points.
// Everything here runs before any HIP call, so a rejected call enqueues
// nothing and the checks work on a machine without a GPU.
#pragma once

#include <stdint.h>

#include "../../include/nq.h"

namespace nq {

// Address range [lo, hi) touched by a row-major [rows, cols] view with row
// stride `ld` (elements of `esize` bytes).  Empty when rows or cols is 0.
struct Region {
    uintptr_t lo = 0, hi = 0;
};

inline Region region(const void* p, int64_t rows, int64_t ld, int64_t cols, int64_t esize)
{
    Region r;
    if (!p || rows <= 0 || cols <= 0) return r;
    r.lo = (uintptr_t)p;
    r.hi = r.lo + (uintptr_t)(((rows - 1) * ld + cols) * esize);
    return r;
}

inline bool overlaps(const Region& a, const Region& b)
{
    return a.hi > a.lo && b.hi > b.lo && a.lo < b.hi && b.lo < a.hi;
}

inline bool aligned(const void* p, uintptr_t bytes) { return ((uintptr_t)p % bytes) == 0; }

// Rows take the 128-bit path when they hold whole 8-element chunks and the
// shared vectors (gamma, beta; NULL for none) start on 16-byte boundaries:
// they are staged through LDS in 16-byte pieces.  Row pointers and strides
// need no alignment.  gfx950 code under the HSA runtime runs with unaligned
// memory access enabled (the compiler itself lowers a byte-aligned 16-byte
// copy to one 128-bit access for this target), so a row that starts off a
// 16-byte boundary is still read and written 16 bytes at a time.
inline bool vector_rows(int64_t d, const void* gamma, const void* beta = nullptr)
{
    return d % 8 == 0 && aligned(gamma, 16) && aligned(beta, 16);
}

// Bounds that keep every offset formed on the host or in a kernel in range:
// a tensor's extent (M - 1) * ld + cols stays below 2^60 elements, so its
// byte size (at most 4 bytes each) and every int64 row offset fit without
// overflow; the per-wavefront buffer offsets (at most 4 rows of at most 2^24
// elements of at most 4 bytes) stay below 2^31.
constexpr int64_t kMaxRows = int64_t(1) << 36;
constexpr int64_t kMaxLd = int64_t(1) << 24;

inline bool bad_ld(int64_t ld, int64_t cols) { return ld < cols || ld > kMaxLd; }

// Rejects any output region overlapping an input region or another output
// region.  `allow_exact` names one (input, output) pair that may coincide
// exactly (in-place residual update).
template <int NI, int NO>
inline bool any_alias(const Region (&in)[NI], const Region (&out)[NO], int exact_in = -1,
                      int exact_out = -1)
{
    for (int o = 0; o < NO; ++o) {
        for (int i = 0; i < NI; ++i) {
            if (!overlaps(out[o], in[i])) continue;
            if (i == exact_in && o == exact_out && out[o].lo == in[i].lo && out[o].hi == in[i].hi)
                continue;
            return true;
        }
        for (int p = o + 1; p < NO; ++p)
            if (overlaps(out[o], out[p])) return true;
    }
    return false;
}

} // namespace nq
