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
// TEAM lanes when a team is larger, and grow to 512 or 1024 lanes where that
// lets the vectors every row shares (gamma, beta) be staged in LDS (see
// SharedVectors); consecutive blocks are dealt round-robin over the 8 XCDs,
// which measured faster than keeping neighbouring rows on one XCD.
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
template <int TEAM, int BLOCK = default_block<TEAM>()>
__device__ __forceinline__ RowMap row_map_at(int64_t M, int64_t blk)
{
    using S = TeamShape<TEAM, BLOCK>;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
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

template <int TEAM, int BLOCK = default_block<TEAM>(), bool XCD = false>
__device__ __forceinline__ RowMap row_map(int64_t M)
{
    return row_map_at<TEAM, BLOCK>(M, logical_block<XCD>());
}

// Whether an access at element e of a d-element row needs its explicit
// mask.  A buffer resource that holds exactly one row -- a team of one or
// more whole wavefronts owns one row per wavefront -- drops every access
// past the row's end by itself (chunks are whole 16-byte pieces and d % 8 ==
// 0 on this path, so a chunk is entirely inside or entirely past the end).
// A resource shared by the rows of several narrower teams, and the
// element-wise path, need the mask.
template <int TEAM, bool VEC>
__device__ __forceinline__ bool col_live(int e, int d)
{
    return (VEC && TEAM >= kWave) || e < d;
}

// A one-row view for vectors shared by every row (gamma, beta).
__device__ __forceinline__ RowMap vector_map()
{
    RowMap m;
    m.row = 0; m.ok = true; m.row0 = 0; m.nrows = 1; m.rel = 0;
    return m;
}

// Vectors shared by every row (gamma, beta).  Loading them per row doubles
// the load traffic that reaches the caches (measured on MI355X at d = 2816:
// ~1.3 us of a 28 us call).  Where a block holds several rows, the block
// loads each vector once, cooperatively, right after the first row loads
// (or, where a kernel asks, right before them, writing LDS as soon as they
// arrive), writes it to LDS before the first reduction (whose barrier, or
// one of its own for teams within a wavefront, orders the writes before
// every read), and the lanes read their chunks from LDS (the dynamic
// LayerNorm's fp32 vectors are loaded straight into LDS, buffer_load ...
// lds, see kDma).
// Staged only while the LDS of the blocks that fill a compute unit (32
// wavefronts) stays within its 160 KB; otherwise each lane loads its chunks
// from memory.
constexpr int kLanesPerCU = 2048;        // 8 wavefronts per SIMD x 4 SIMDs x 64
constexpr int kLdsPerCU = 160 * 1024;

constexpr bool stages_vectors(int team, int cpl, int nv, int block)
{
    return block / team >= 2 && team * cpl * 2 * 16 * nv * (kLanesPerCU / block) <= kLdsPerCU;
}

// Block size of a row kernel with NV shared vectors: with STAGE, the
// default or the smallest larger block (up to 1024 lanes) that lets the
// vectors be staged.  Measured at d = 2816: 2 rows per block beat 4 and 8.
template <int TEAM, int CPL, int NV, bool VEC, bool STAGE>
constexpr int row_block()
{
    if (STAGE && NV > 0)
        for (int b = default_block<TEAM>(); b <= 1024; b *= 2)
            if (stages_vectors(TEAM, CPL, NV, b)) return b;
    return default_block<TEAM>();
}

template <int TEAM, int CPL, bool VEC, int NV, int BLOCK, bool STAGE, bool BF16 = false, bool DMA = false>
class SharedVectors {
  public:
    using S = TeamShape<TEAM, BLOCK>;
    static constexpr int kSlots = TEAM * CPL * 2;  // 16-byte fp32 slots covering one row's chunks
    static constexpr bool kStaged = STAGE && stages_vectors(TEAM, CPL, NV, BLOCK);
    static constexpr int kPer = kStaged ? (kSlots + S::kBlock - 1) / S::kBlock : 1;
    // Unstaged instances with at most 2 chunks per lane (the few-rows
    // shapes, where latency rules) load each lane's chunks with the row
    // loads instead of after the first reduction, taking one memory round
    // trip off the critical path for at most 16 more registers per vector.
    static constexpr bool kPrefetch = !kStaged && CPL <= 2;
    // DMA: staged fp32 vectors are loaded straight into LDS (bf16 ones are
    // widened on the way, through registers).  Measured on MI355X against
    // the register path: the dynamic LayerNorm 1.5 % faster, the static one
    // within noise (and 12 more vector instructions per wavefront), the
    // RMSNorm kernels 0.3-1.8 % slower, so only the dynamic LayerNorm asks
    // for it.
    static constexpr bool kDma = DMA && kStaged && !BF16 && VEC;  // whole 16-byte slots only
    typedef uint4 Lds[kStaged ? NV : 1][kStaged ? kSlots : 1];
    static_assert(!kStaged || kSlots * 16 * NV <= 64 * 1024, "staged vectors fit one block's LDS");

    // The vectors are fp32 or (BF16) bf16; both are read through a
    // 2-byte-element view, so element e of an fp32 vector starts at 2e.
    // On the 128-bit path each vector's resource holds exactly the vector,
    // so reads past its end return zeros with no mask.
    __device__ __forceinline__ SharedVectors(const void* const (&p)[NV], int d) : d_(d)
    {
#pragma unroll
        for (int v = 0; v < NV; ++v)
            io_[v] = RowIO<VEC, kKeep, uint16_t>(static_cast<const uint16_t*>(p[v]), 0, vector_map(),
                                                 BF16 ? d : 2 * d);
    }
    // Issue the loads: staged, the block's cooperative loads (fp32 slot i
    // holds elements 4i .. 4i+3, loaded as 16 bytes, or as 8 bytes of bf16
    // widened at publish); prefetching, lane t's own chunks.
    __device__ __forceinline__ void issue(int t, Lds& lds)
    {
        if constexpr (kPrefetch) {
#pragma unroll
            for (int v = 0; v < NV; ++v)
#pragma unroll
                for (int j = 0; j < CPL; ++j) {
                    const int e = (j * TEAM + t) * 8;
                    if constexpr (BF16) {
                        pre_[v][j][0] = io_[v].load16(e, VEC || e < d_);
                    } else {
                        pre_[v][j][0] = io_[v].load16(2 * e, VEC || e < d_);
                        pre_[v][j][1] = io_[v].load16(2 * e + 8, VEC || e < d_);
                    }
                }
        }
        if constexpr (kDma) {
            // fp32 vectors go straight to LDS: each wavefront's 64 lanes
            // fill 64 consecutive slots, with no registers held and no LDS
            // writes of their own (the barrier that publishes them waits for
            // the loads)
            const int wave_first = (int)(threadIdx.x & ~(kWave - 1));
#pragma unroll
            for (int v = 0; v < NV; ++v)
#pragma unroll
                for (int u = 0; u < kPer; ++u) {
                    const int i = u * S::kBlock + (int)threadIdx.x;
                    if (u * S::kBlock + wave_first < kSlots && i < kSlots)
                        io_[v].load16_lds(i * 8, VEC || i * 4 < d_, &lds[v][u * S::kBlock + wave_first]);
                }
        } else if constexpr (kStaged) {
#pragma unroll
            for (int v = 0; v < NV; ++v)
#pragma unroll
                for (int u = 0; u < kPer; ++u) {
                    const int i = u * S::kBlock + (int)threadIdx.x;
                    if constexpr (BF16) {
                        const uint2 h = io_[v].load8(i * 4, VEC || i * 4 < d_);
                        held_[v][u] = make_uint4(h.x, h.y, 0u, 0u);
                    } else {
                        held_[v][u] = io_[v].load16(i * 8, VEC || i * 4 < d_);
                    }
                }
        }
    }
    // Write the staged vectors to LDS as fp32 (staged only; before the first
    // reduction, which every lane of the block reaches).
    __device__ __forceinline__ void publish(Lds& lds)
    {
        if constexpr (kDma) {
            // This wavefront's loads into LDS have landed before it reaches
            // the barrier that publishes them (s_waitcnt vmcnt(0); the row
            // loads, issued first, are already in use here).
            __builtin_amdgcn_s_waitcnt(0x0F70);
            if constexpr (TEAM <= kWave) __syncthreads();
        } else if constexpr (kStaged) {
#pragma unroll
            for (int v = 0; v < NV; ++v)
#pragma unroll
                for (int u = 0; u < kPer; ++u) {
                    const int i = u * S::kBlock + (int)threadIdx.x;
                    uint4 w = held_[v][u];
                    if constexpr (BF16) w = make_uint4(w.x << 16, w.x & 0xFFFF0000u, w.y << 16, w.y & 0xFFFF0000u);
                    if (i < kSlots) lds[v][i] = w;
                }
            if constexpr (TEAM <= kWave) __syncthreads();
        }
    }
    // 8 fp32 of vector v from element e = (j * TEAM + t) * 8 (zeros past the end).
    __device__ __forceinline__ void chunk(const Lds& lds, int v, int j, int e, float g[8]) const
    {
        if constexpr (kPrefetch) {
            if constexpr (BF16) {
                unpack_bf16x8(pre_[v][j][0], g);
            } else {
                const uint4 a = pre_[v][j][0], b = pre_[v][j][1];
                g[0] = __uint_as_float(a.x); g[1] = __uint_as_float(a.y);
                g[2] = __uint_as_float(a.z); g[3] = __uint_as_float(a.w);
                g[4] = __uint_as_float(b.x); g[5] = __uint_as_float(b.y);
                g[6] = __uint_as_float(b.z); g[7] = __uint_as_float(b.w);
            }
        } else if constexpr (kStaged) {
            const uint4 a = lds[v][e >> 2], b = lds[v][(e >> 2) + 1];  // e >= 0
            g[0] = __uint_as_float(a.x); g[1] = __uint_as_float(a.y);
            g[2] = __uint_as_float(a.z); g[3] = __uint_as_float(a.w);
            g[4] = __uint_as_float(b.x); g[5] = __uint_as_float(b.y);
            g[6] = __uint_as_float(b.z); g[7] = __uint_as_float(b.w);
        } else if constexpr (BF16) {
            unpack_bf16x8(io_[v].load16(e, VEC || e < d_), g);
        } else {
            const uint4 a = io_[v].load16(2 * e, VEC || e < d_), b = io_[v].load16(2 * e + 8, VEC || e < d_);
            g[0] = __uint_as_float(a.x); g[1] = __uint_as_float(a.y);
            g[2] = __uint_as_float(a.z); g[3] = __uint_as_float(a.w);
            g[4] = __uint_as_float(b.x); g[5] = __uint_as_float(b.y);
            g[6] = __uint_as_float(b.z); g[7] = __uint_as_float(b.w);
        }
    }

    // Elements 4h .. 4h+3 of the chunk at e (staged only: one LDS read, so a
    // loop over the chunk's halves holds 4 registers per vector, not 8).
    __device__ __forceinline__ void half(const Lds& lds, int v, int e, int h, float g[4]) const
    {
        static_assert(kStaged, "half chunks come from the staged copy");
        const uint4 a = lds[v][(e >> 2) + h];  // e >= 0
        g[0] = __uint_as_float(a.x); g[1] = __uint_as_float(a.y);
        g[2] = __uint_as_float(a.z); g[3] = __uint_as_float(a.w);
    }

  private:
    RowIO<VEC, kKeep, uint16_t> io_[NV];
    uint4 held_[kStaged && !kDma ? NV : 1][kStaged && !kDma ? kPer : 1];
    uint4 pre_[kPrefetch ? NV : 1][kPrefetch ? CPL : 1][BF16 ? 1 : 2];
    int d_;
};

// Every (TEAM, CPL, VEC) shape that is compiled: teams of 16..1024 lanes
// with at most 4 chunks (32 elements) per lane, so the fp32 row fits in
// registers at full occupancy, plus the element-wise path (VEC = false) for
// d % 8 != 0 or gamma / beta off 16-byte boundaries.
#define NQ_ROW_SHAPES(X)                                                                    \
    X(16, 1, true) X(16, 2, true) X(16, 3, true) X(16, 4, true)                             \
    X(32, 1, true) X(32, 2, true) X(32, 3, true) X(32, 4, true)                             \
    X(64, 1, true) X(64, 2, true) X(64, 3, true) X(64, 4, true)                             \
    X(128, 1, true) X(128, 2, true) X(128, 3, true) X(128, 4, true)                         \
    X(256, 1, true) X(256, 2, true) X(256, 3, true) X(256, 4, true)                         \
    X(512, 1, true) X(512, 2, true) X(512, 3, true) X(512, 4, true)                         \
    X(1024, 1, true) X(1024, 2, true) X(1024, 3, true) X(1024, 4, true)                     \
    X(64, 4, false) X(128, 4, false) X(256, 4, false) X(512, 4, false) X(1024, 4, false)

struct RowShape {
    int team = 0, cpl = 0;
    bool vec = false;
    bool stage = true;  // stage shared vectors in LDS (many rows only)
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
// its latency is close to one memory round trip, and no staging of the
// shared vectors (its barrier and LDS round trip cost ~0.45 us at M <= 128,
// with nothing to share across a block's rows).
inline RowShape pick_row_shape(int64_t M, int64_t d, bool vec)
{
    if (!vec) {
        // element-wise: whole wavefronts per row (the narrowest that holds
        // the row in 4 chunks per lane), staged vectors for many rows
        RowShape s;
        s.cpl = 4;
        for (s.team = 64; s.team < 1024 && (int64_t)s.team * 32 < d; s.team *= 2) {}
        s.stage = M * (s.team / 64) >= kFewRowsWaves;
        return s;
    }
    RowShape s = narrowest_team(d, 4);
    if (s.team == 0) return s;
    const int64_t waves = M * ((s.team + 63) / 64);
    if (waves >= kFewRowsWaves) return s;
    RowShape wide = narrowest_team(d, 2);
    if (wide.team == 0) wide = s;
    wide.stage = false;
    return wide;
}

// Largest grid the launcher accepts.
constexpr int64_t kMaxBlocks = 0x7FFFFFFF;

// One launch of kernel shape KS with or without staging: KS::block<STAGE>()
// lanes per block, KS::launch<STAGE>(args, grid, block, stream).
template <class KS, int TEAM, bool STAGE, typename Args>
inline bool launch_rows(const Args& a, int64_t M, hipStream_t stream)
{
    constexpr int block = KS::template block<STAGE>();
    constexpr int rows = block / TEAM;
    const int64_t blocks = (M + rows - 1) / rows;
    if (blocks > kMaxBlocks) return false;
    KS::template launch<STAGE>(a, dim3((unsigned)blocks), dim3(block), stream);
    return true;
}

template <template <int, int, bool> class K, int T, int C, bool V, typename Args>
inline bool launch_shape(bool stage, const Args& a, int64_t M, hipStream_t stream)
{
    // The element-wise row access relies on the range check of a resource
    // that ends at the row's end: one row per wavefront.
    static_assert(V || T >= kWave, "element-wise shapes give each wavefront one row");
    if (stage) return launch_rows<K<T, C, V>, T, true>(a, M, stream);
    return launch_rows<K<T, C, V>, T, false>(a, M, stream);
}

// Launches kernel K for the chosen shape; false if the shape is not
// compiled or the grid would exceed kMaxBlocks.
template <template <int, int, bool> class K, typename Args>
inline bool launch_row_shape(const RowShape& s, const Args& a, int64_t M, hipStream_t stream)
{
#define NQ_X(T, C, V)                                                                       \
    if (s.team == T && s.cpl == C && s.vec == V) return launch_shape<K, T, C, V>(s.stage, a, M, stream);
    NQ_ROW_SHAPES(NQ_X)
#undef NQ_X
    return false;
}

} // namespace nq
