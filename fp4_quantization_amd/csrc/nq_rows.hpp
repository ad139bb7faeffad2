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
// TEAM lanes when a team is larger.
//
// Shape choice (pages: [NVFP4] commit notes gate schedules on problem size;
// here the gate keys on M and d):
//  * many rows: the smallest team whose registers hold the row, so a
//    wavefront (or less) owns a row and no barrier is needed;
//  * few rows: a wider team with at most two chunks per lane, so a single
//    row is spread over many SIMDs and its latency is one memory round trip.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nq {

template <int TEAM>
struct TeamShape {
    static constexpr int kBlock = TEAM > 256 ? TEAM : 256;
    static constexpr int kRows = kBlock / TEAM;   // rows per block
    static constexpr int kWaves = kBlock / 64;    // wavefronts per block
};

// Every (TEAM, CPL, VEC) shape that is compiled.  VEC = false is the
// element-wise path for odd d or misaligned pointers.
#define NQ_ROW_SHAPES(X)                                                                   \
    X(16, 1, true) X(16, 2, true) X(32, 2, true) X(64, 2, true) X(64, 3, true)             \
    X(64, 4, true) X(64, 6, true) X(64, 8, true) X(128, 2, true) X(128, 4, true)           \
    X(128, 6, true) X(128, 8, true) X(256, 2, true) X(256, 4, true) X(256, 6, true)        \
    X(256, 8, true) X(512, 2, true) X(512, 4, true) X(512, 8, true) X(1024, 2, true)       \
    X(1024, 4, true) X(64, 4, false) X(256, 4, false) X(1024, 4, false)

struct RowShape {
    int team = 0, cpl = 0;
    bool vec = false;
};

inline bool shape_compiled(int team, int cpl, bool vec)
{
#define NQ_X(T, C, V) if (team == T && cpl == C && vec == V) return true;
    NQ_ROW_SHAPES(NQ_X)
#undef NQ_X
    return false;
}

// Smallest compiled CPL >= need for this team (0 if none).
inline int smallest_cpl(int team, int64_t need, bool vec)
{
    for (int c = 1; c <= 8; ++c)
        if (c >= need && shape_compiled(team, c, vec)) return c;
    return 0;
}

// Rows below which the wide-team shape is used: a wave-per-row grid would
// give fewer than 4 wavefronts per compute unit of a 256-CU MI355X.
constexpr int64_t kFewRowsWaves = 1024;

inline RowShape pick_row_shape(int64_t M, int64_t d, bool vec)
{
    RowShape s;
    s.vec = vec;
    if (!vec) {
        s.cpl = 4;
        s.team = d <= 2048 ? 64 : d <= 8192 ? 256 : 1024;
        return s;
    }
    static const int teams[] = {16, 32, 64, 128, 256, 512, 1024};
    // Many rows: smallest team that holds the row in registers.
    for (int team : teams) {
        int c = smallest_cpl(team, (d + team * 8 - 1) / (team * 8), true);
        if (c) { s.team = team; s.cpl = c; break; }
    }
    const int64_t waves = M * ((s.team + 63) / 64);
    if (waves >= kFewRowsWaves) return s;
    // Few rows: a wide team with at most two chunks per lane.
    for (int team : teams) {
        if ((int64_t)team * 16 < d) continue;
        int c = smallest_cpl(team, (d + team * 8 - 1) / (team * 8), true);
        if (c) { s.team = team; s.cpl = c; break; }
    }
    return s;
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
