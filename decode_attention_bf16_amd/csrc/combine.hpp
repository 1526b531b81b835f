// Log-sum-exp combine of split-KV partial results.
//
// A sequence whose cache rows were split over several workers has one partial
// (out_r normalized by its own softmax sum and stored as bf16, lse_r in log2
// units, fp32) per segment.
// The merged result is lse = log(sum_r 2^lse_r) and out = sum_r 2^(lse_r - lse)
// out_r, which equals softmax attention over the union of the segments' rows.
// Empty segments carry lse_r = -inf and weigh nothing. Sequences with no cache
// row at all (no segment) get out = 0, lse = -inf here; sequences with a
// single segment were written by their worker and are skipped.
#pragma once

#include "common.hpp"
#include "plan.hpp"

namespace da {

// One wave per query row (grid-stride over rows); DV output columns spread
// over the 64 lanes. A launch of a few blocks per CU keeps the cost low when
// most rows belong to single-segment sequences and are skipped.
template <int DV>
__global__ void __launch_bounds__(256) combine_kernel(int B, int M, const PlanHeader *__restrict__ hdr,
                                                      const int *__restrict__ slot_start,
                                                      const uint16_t *__restrict__ part_out,
                                                      const float *__restrict__ part_lse,
                                                      uint16_t *__restrict__ out, float *__restrict__ lse)
{
    static_assert(DV % 64 == 0, "whole columns per lane");
    if (hdr->merge_seqs == 0) return;  // every sequence was written by its one worker
    constexpr int CPL = DV / 64;
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const long rows = (long)B * M;
    for (long row_g = (long)blockIdx.x * 4 + wave; row_g < rows; row_g += (long)gridDim.x * 4) {
        const int bq = (int)(row_g / M);
        const int row = (int)(row_g - (long)bq * M);
        const int s0 = slot_start[bq];
        const int nseg = slot_start[bq + 1] - s0;
        if (nseg == 1) continue;

        float m = -INFINITY;
        for (int r = 0; r < nseg; ++r) m = fmaxf(m, part_lse[(size_t)(s0 + r) * M + row]);

        float acc[CPL];
#pragma unroll
        for (int c = 0; c < CPL; ++c) acc[c] = 0.f;
        float wsum = 0.f;
        if (m != -INFINITY) {
            for (int r = 0; r < nseg; ++r) {
                const float wgt = fast_exp2(part_lse[(size_t)(s0 + r) * M + row] - m);
                wsum += wgt;
                const uint16_t *src = part_out + ((size_t)(s0 + r) * M + row) * DV + lane * CPL;
                if constexpr (CPL % 2 == 0) {
#pragma unroll
                    for (int c = 0; c < CPL / 2; ++c) {
                        const uint32_t u = ((const uint32_t *)src)[c];
                        acc[2 * c] += wgt * bf16lo_to_f32(u);
                        acc[2 * c + 1] += wgt * bf16hi_to_f32(u);
                    }
                } else {
#pragma unroll
                    for (int c = 0; c < CPL; ++c) acc[c] += wgt * bf16lo_to_f32(src[c]);
                }
            }
        }
        const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
        if constexpr (CPL % 2 == 0) {
            uint32_t *dst = (uint32_t *)(out + (size_t)row_g * DV + lane * CPL);
#pragma unroll
            for (int c = 0; c < CPL / 2; ++c) dst[c] = pack_bf16x2(acc[2 * c] * inv, acc[2 * c + 1] * inv);
        } else {
            uint16_t *dst = out + (size_t)row_g * DV + lane * CPL;
#pragma unroll
            for (int c = 0; c < CPL; ++c) dst[c] = to_bf16_bits(acc[c] * inv);
        }
        if (lane == 0) lse[row_g] = wsum > 0.f ? (m + fast_log2(wsum)) * kLn2 : -INFINITY;
    }
}

// Blocks of the combine launch: enough to cover the rows with a few waves per
// CU, never more than one block per four rows.
inline unsigned combine_grid(long rows, int cus)
{
    const long want = (long)cus * 4;
    const long need = (rows + 3) / 4;
    return (unsigned)(need < want ? (need > 0 ? need : 1) : want);
}

}  // namespace da
