// nq_rows.hpp -- how a row is spread over lanes, and which kernel shape a
// call uses.
//
// A "team" of TEAM lanes owns one row.  Lane t of the team holds CPL
// chunks of 8 consecutive elements: chunk j covers elements
// [(j*TEAM + t)*8, +8), so each load instruction of a wavefront touches
// one contiguous 512-byte (64 lanes x 16 B of bf16) stretch of the row.
// The row stays in registers between the two reductions ([FUSE] "FAQ": the
// vector is held in registers through both phases, with the residual
// written in place).  Blocks are 256 lanes (several rows per block) or
// TEAM lanes when a team is larger; consecutive blocks are dealt round-robin
// over the 8 XCDs, which measured faster than keeping neighbouring rows on
// one XCD.
//
// Shape choice (pages: [NVFP4] commit notes gate schedules on problem size;
// here the gate keys on M and d): see pick_row_shape.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nq_device.hpp"

namespace nq {

template <int TEAM>
constexpr int default_block() { return TEAM > 256 ? TEAM : 256; }

template <int TEAM, int BLOCK = default_block<TEAM>()>
struct TeamShape {
    static_assert(BLOCK % TEAM == 0 && BLOCK % 64 == 0, "a block holds whole teams and wavefronts");
    static constexpr int kBlock = BLOCK;
    static constexpr int kRows = kBlock / TEAM;   // rows per block
    static constexpr int kWaves = kBlock / 64;    // wavefronts per block
};

// Logical block index.  With XCD set, consecutive logical blocks (and so
// consecutive rows) stay on one XCD: the dispatcher deals physical blocks
// round-robin over the 8 XCDs, so physical block b runs on XCD b % 8.
template <bool XCD>
__device__ __forceinline__ int64_t logical_block()
{
    if constexpr (!XCD) {
        return blockIdx.x;
    } else {
        const uint32_t n = gridDim.x, b = blockIdx.x;
        const uint32_t per = n / 8, rem = n % 8, x = b % 8, i = b / 8;
        // XCD x owns logical blocks [x*per + min(x, rem), ...) of length per + (x < rem)
        return (int64_t)x * per + (x < rem ? x : rem) + i;
    }
}

// Rows owned by this lane and its wavefront.  The wavefront-uniform parts
// come from blockIdx and a readfirstlane'd wave index, so they sit in scalar
// registers and the per-wavefront buffer resources need no waterfall.
template <int TEAM, int BLOCK = default_block<TEAM>(), bool XCD = false>
__device__ __forceinline__ RowMap row_map(int64_t M)
{
    using S = TeamShape<TEAM, BLOCK>;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
    const int64_t blk = logical_block<XCD>();
    RowMap m;
    m.row = blk * S::kRows + threadIdx.x / TEAM;
    m.ok = m.row < M;
    if constexpr (TEAM >= kWave) {
        m.row0 = blk * S::kRows + wave / (TEAM / kWave);
        m.nrows = m.row0 < M ? 1 : 0;
        m.rel = 0;
    } else {
        constexpr int kPerWave = kWave / TEAM;
        m.row0 = blk * S::kRows + (int64_t)wave * kPerWave;
        const int64_t left = M - m.row0;
        m.nrows = left <= 0 ? 0 : (left < kPerWave ? (int)left : kPerWave);
        m.rel = (int)(m.row - m.row0);
    }
    return m;
}

// A one-row view for vectors shared by every row (gamma, beta).
__device__ __forceinline__ RowMap vector_map()
{
    RowMap m;
    m.row = 0; m.ok = true; m.row0 = 0; m.nrows = 1; m.rel = 0;
    return m;
}

// Every (TEAM, CPL, VEC) shape that is compiled: teams of 16..1024 lanes
// with at most 4 chunks (32 elements) per lane, so the fp32 row fits in
// registers at full occupancy, plus the element-wise path (VEC = false) for
// odd d or misaligned pointers.
#define NQ_ROW_SHAPES(X)                                                                    \
    X(16, 1, true) X(16, 2, true) X(16, 3, true) X(16, 4, true)                             \
    X(32, 1, true) X(32, 2, true) X(32, 3, true) X(32, 4, true)                             \
    X(64, 1, true) X(64, 2, true) X(64, 3, true) X(64, 4, true)                             \
    X(128, 1, true) X(128, 2, true) X(128, 3, true) X(128, 4, true)                         \
    X(256, 1, true) X(256, 2, true) X(256, 3, true) X(256, 4, true)                         \
    X(512, 1, true) X(512, 2, true) X(512, 3, true) X(512, 4, true)                         \
    X(1024, 1, true) X(1024, 2, true) X(1024, 3, true) X(1024, 4, true)                     \
    X(64, 4, false) X(256, 4, false) X(1024, 4, false)

struct RowShape {
    int team = 0, cpl = 0;
    bool vec = false;
};

// Rows below which the wide-team shape is used: the many-rows grid would
// give fewer than 4 wavefronts per compute unit of a 256-CU MI355X.
constexpr int64_t kFewRowsWaves = 1024;

// Narrowest team (>= 16 lanes) whose lanes need at most `max_cpl` chunks.
inline RowShape narrowest_team(int64_t d, int max_cpl)
{
    RowShape s;
    s.vec = true;
    for (int team = 16; team <= 1024; team *= 2) {
        const int64_t need = (d + team * 8 - 1) / (team * 8);
        if (need <= max_cpl) {
            s.team = team;
            s.cpl = (int)need;
            return s;
        }
    }
    return s;  // d > 32768: team stays 0 (not supported)
}

// Many rows: the narrowest team holding the row in at most 4 chunks per
// lane (measured on MI355X at d = 2816: 128 lanes x 3 chunks beats 64 x 6
// and 32 x 11 -- more, shorter wavefronts keep more rows in flight).  Few
// rows: at most 2 chunks per lane, so one row is spread over many SIMDs and
// its latency is close to one memory round trip.
inline RowShape pick_row_shape(int64_t M, int64_t d, bool vec)
{
    if (!vec) {
        RowShape s;
        s.cpl = 4;
        s.team = d <= 2048 ? 64 : d <= 8192 ? 256 : 1024;
        return s;
    }
    RowShape s = narrowest_team(d, 4);
    if (s.team == 0) return s;
    const int64_t waves = M * ((s.team + 63) / 64);
    if (waves >= kFewRowsWaves) return s;
    const RowShape wide = narrowest_team(d, 2);
    return wide.team ? wide : s;
}

// Largest grid the launcher accepts.
constexpr int64_t kMaxBlocks = 0x7FFFFFFF;

// Launches K<TEAM, CPL, VEC>::launch(args, grid, block, stream) for the
// chosen shape; false if the shape is not compiled or the grid would exceed
// kMaxBlocks.
template <template <int, int, bool> class K, typename Args>
inline bool launch_row_shape(const RowShape& s, const Args& a, int64_t M, hipStream_t stream)
{
#define NQ_X(T, C, V)                                                                       \
    if (s.team == T && s.cpl == C && s.vec == V) {                                          \
        const int64_t blocks = (M + TeamShape<T>::kRows - 1) / TeamShape<T>::kRows;         \
        if (blocks > kMaxBlocks) return false;                                               \
        K<T, C, V>::launch(a, dim3((unsigned)blocks), dim3(TeamShape<T>::kBlock), stream);   \
        return true;                                                                         \
    }
    NQ_ROW_SHAPES(NQ_X)
#undef NQ_X
    return false;
}

} // namespace nq
