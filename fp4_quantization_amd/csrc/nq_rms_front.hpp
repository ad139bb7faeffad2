// nq_rms_front.hpp -- the front half every (residual-add +) RMSNorm kernel
// shares: one pass of 128-bit loads over the row (and residual), the bf16
// sum z written back as the new residual, the sum of squares reduced over
// the team, and rstd.
//
// Pages: [FUSE] "Fusing RMSNorm and FP8 Quantization Under torch.compile"
// ("TL;DR": z = x + residual is the residual written back; "FAQ": the row
// stays in registers and the residual update matches the reference
// exactly); [NVFP4] "RMSNorm nvfp4 quant fusion for DS V3.2 / Kimi-K2.5"
// (commit notes: optional residual, fresh or in-place residual buffer).
//
//   z_i  = bf16(x_i + r_i), or x_i itself when residual-less (RES false: a
//          separate instance with no add, repacking or write-back)
//   rstd = 1 / sqrt(sum z_i^2 / d + eps), the sum in binary64 (every z_i^2 is
//          exact there; the sum rounds, if at all, only in its last bit), its
//          quotient by d correctly rounded in binary64 and then to binary32,
//          so the reduction order changes the result only if that sum lies
//          within about 2^-52 of a binary32 rounding boundary; the square
//          root and the reciprocal are each correctly rounded.
#pragma once

#include "nq_device.hpp"
#include "nq_rows.hpp"

namespace nq {

// Returns rstd; zw[j] holds chunk j of z as packed bf16 (it is exactly a
// bf16 value, so nothing is lost).  Callers launder zw (opaque) before
// unpacking it again, so the unpacked copy from the sum is not kept alive
// across the reduction -- except with KEEP, where the residual-less path
// also leaves z unpacked in zf (for kernels with registers to spare, which
// then skip the second unpacking).  `vecs` are the block's shared vectors:
// their cooperative loads are issued with the row loads and they are
// published before the reduction's barrier.
struct NoBlockWork {
    __device__ __forceinline__ void operator()() const {}
};

// Whether rms_front passes a block barrier after it has run `before_barrier`
// (the staged vectors' barrier, or the cross-wavefront reduction's).
template <int TEAM, class SV>
constexpr bool rms_front_syncs() { return SV::kStaged || TEAM > kWave; }

// `before_barrier` runs once the row loads are issued and before the block's
// first barrier, so block-wide LDS a kernel fills there (a table) is
// visible to every lane after rms_front without a barrier of its own when
// rms_front_syncs() holds.
//
// EARLY (with a residual and staged vectors): the block's vector loads are
// issued before the row loads and written to LDS as soon as they arrive,
// so their registers are free before the row is unpacked.  Measured on
// MI355X: the NVFP4 kernel at d = 7168 drops from 65 to 62 VGPRs (8
// wavefronts per SIMD instead of 7) and runs 1.2 % faster; the FP8 kernels,
// already at 8, ran 0.4-0.5 % slower with it, so only the NVFP4 kernel asks.
template <int TEAM, int CPL, bool VEC, bool RES, class SV, bool KEEP = false, bool EARLY = false,
          class Pre = NoBlockWork>
__device__ __forceinline__ float rms_front(const uint16_t* x, int64_t ld_x, const uint16_t* r, int64_t ld_r,
                                           uint16_t* ro, int64_t ld_ro, const RowMap& m, int t, int d,
                                           double inv_d, float eps, SV& vecs, typename SV::Lds& lds_vec,
                                           double* lds_sum, uint4 (&zw)[CPL], float (*zf)[8] = nullptr,
                                           const Pre& before_barrier = Pre())
{
    constexpr bool kEarly = EARLY && RES && SV::kStaged;
    const RowIO<VEC, kLoadStream, uint16_t> xio(x, ld_x, m, d);
    double acc = 0.0;
    if constexpr (RES) {
        const RowIO<VEC, kLoadStream, uint16_t> rio(r, ld_r, m, d);
        const RowIO<VEC, kStoreRows, uint16_t> roio(ro, ld_ro, m, d);
        // Issue every load of the row before the first use.
        if constexpr (kEarly) vecs.issue(t, lds_vec);
        uint4 xw[CPL], rw[CPL];
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            const int e = (j * TEAM + t) * 8;
            xw[j] = xio.load16(e, col_live<TEAM, VEC>(e, d));
            rw[j] = rio.load16(e, col_live<TEAM, VEC>(e, d));
        }
        if constexpr (kEarly) {
            before_barrier();
            vecs.publish(lds_vec);
        } else {
            vecs.issue(t, lds_vec);
        }
        // z = bf16(x + r), kept packed; residual write-back; sum of z^2.
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            const int e = (j * TEAM + t) * 8;
            float xv[8], rv[8];
            unpack_bf16x8(xw[j], xv);
            unpack_bf16x8(rw[j], rv);
            uint32_t p[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) p[k] = pack_bf16x2(xv[2 * k] + rv[2 * k], xv[2 * k + 1] + rv[2 * k + 1]);
            zw[j] = make_uint4(p[0], p[1], p[2], p[3]);
            roio.store16(e, col_live<TEAM, VEC>(e, d), zw[j]);
            acc += sumsq_chunk(zw[j]);
        }
    } else {
        // Residual-less: z is x itself (a bf16 value).
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            const int e = (j * TEAM + t) * 8;
            zw[j] = xio.load16(e, col_live<TEAM, VEC>(e, d));
        }
        vecs.issue(t, lds_vec);
        if constexpr (KEEP) {
#pragma unroll
            for (int j = 0; j < CPL; ++j) {
                unpack_bf16x8(zw[j], zf[j]);
                acc += sumsq_chunk_unpacked(zf[j]);
            }
        } else {
#pragma unroll
            for (int j = 0; j < CPL; ++j) acc += sumsq_chunk(zw[j]);
        }
    }
    __builtin_amdgcn_sched_barrier(0);

    if constexpr (!kEarly) {
        before_barrier();
        vecs.publish(lds_vec);
    }
    acc = team_sum<TEAM>(acc, lds_sum);
    const float ms = (float)div_by_len(acc, (double)d, inv_d);
    const float rstd = rsqrt_rn(ms + eps);
    __builtin_amdgcn_sched_barrier(0);
    return rstd;
}

} // namespace nq
