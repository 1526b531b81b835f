// Log-sum-exp combine of split-KV partial results.
//
// A sequence whose cache rows were split over several workers has one partial
// (out_r normalized by its own softmax sum and stored as bf16, lse_r in log2
// units, fp32) per segment. The merged result is lse = log(sum_r 2^lse_r) and
// out = sum_r 2^(lse_r - lse) out_r, which equals softmax attention over the
// union of the segments' rows. Empty segments carry lse_r = -inf and weigh
// nothing. Sequences with no cache row at all (no segment) get out = 0,
// lse = -inf here; sequences with a single segment were written by their worker
// and are skipped.
//
// Two launch shapes: combine_kernel gives each query row one wave (the usual
// case, a few segments per row); combine_wide_kernel gives each row a block of
// sixteen waves that split its segments (long sequences split over many
// workers, where one wave walking a hundred segments would be latency-bound).
#pragma once

#include "common.hpp"
#include "plan.hpp"

namespace da {

__device__ __forceinline__ float wave_max64(float v)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
    return v;
}

// This lane's CPL columns of segment partial `src` (bf16) as floats.
template <int CPL>
__device__ __forceinline__ void load_partial(const uint16_t *__restrict__ src, float (&o)[CPL])
{
    if constexpr (CPL % 2 == 0) {
#pragma unroll
        for (int c = 0; c < CPL / 2; ++c) {
            const uint32_t u = ((const uint32_t *)src)[c];
            o[2 * c] = bf16lo_to_f32(u);
            o[2 * c + 1] = bf16hi_to_f32(u);
        }
    } else {
#pragma unroll
        for (int c = 0; c < CPL; ++c) o[c] = bf16lo_to_f32(src[c]);
    }
}

// acc += sum over segments r = r0, r0 + step, ... < nseg of 2^(lse_r - m) out_r
// (this lane's columns), wsum += the weights. Four segments per round, so
// their loads are in flight together.
template <int DV>
__device__ __forceinline__ void combine_accumulate(const uint16_t *__restrict__ part_out,
                                                   const float *__restrict__ part_lse, int M, int row, int s0,
                                                   int r0, int step, int nseg, float m, int lane,
                                                   float (&acc)[DV / 64], float &wsum)
{
    constexpr int CPL = DV / 64;
    auto src = [&](int r) { return part_out + ((size_t)(s0 + r) * M + row) * DV + lane * CPL; };
    auto lse_of = [&](int r) { return part_lse[(size_t)(s0 + r) * M + row]; };
    int r = r0;
    for (; r + 3 * step < nseg; r += 4 * step) {
        float wr[4], o[4][CPL];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            wr[u] = lse_of(r + u * step);
            load_partial<CPL>(src(r + u * step), o[u]);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const float wgt = fast_exp2(wr[u] - m);
            wsum += wgt;
#pragma unroll
            for (int c = 0; c < CPL; ++c) acc[c] += wgt * o[u][c];
        }
    }
    for (; r < nseg; r += step) {
        float o[CPL];
        const float wgt = fast_exp2(lse_of(r) - m);
        load_partial<CPL>(src(r), o);
        wsum += wgt;
#pragma unroll
        for (int c = 0; c < CPL; ++c) acc[c] += wgt * o[c];
    }
}

// The merged row: out (bf16) and lse (natural log).
template <int DV>
__device__ __forceinline__ void combine_write(uint16_t *__restrict__ out, float *__restrict__ lse, long row_g, int lane,
                                              const float (&acc)[DV / 64], float wsum, float m)
{
    constexpr int CPL = DV / 64;
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

// One wave per query row (grid-stride over rows); DV output columns spread
// over the 64 lanes. A launch of a few blocks per CU keeps the cost low when
// most rows belong to single-segment sequences and are skipped. The kernel is
// bound by the latency of its dependent loads, so the chain is kept short: the
// first row's segment range loads together with the plan header, and a row of
// at most four segments loads its segment lse values (every lane reads the
// same ones, so no cross-lane maximum is needed) together with its partials.
template <int DV>
__global__ void __launch_bounds__(256) combine_kernel(int B, int M, const PlanHeader *__restrict__ hdr,
                                                      const int *__restrict__ slot_start,
                                                      const uint16_t *__restrict__ part_out,
                                                      const float *__restrict__ part_lse,
                                                      uint16_t *__restrict__ out, float *__restrict__ lse)
{
    static_assert(DV % 64 == 0, "whole columns per lane");
    constexpr int CPL = DV / 64;
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const long rows = (long)B * M;
    const long first = (long)blockIdx.x * 4 + wave;
    int s0 = 0, s1 = 0;
    if (first < rows) {
        const int bq = (int)(first / M);
        s0 = slot_start[bq];
        s1 = slot_start[bq + 1];
    }
    if (hdr->merge_seqs == 0) return;  // every sequence was written by its one worker
    for (long row_g = first; row_g < rows; row_g += (long)gridDim.x * 4) {
        const int bq = (int)(row_g / M);
        const int row = (int)(row_g - (long)bq * M);
        if (row_g != first) {
            s0 = slot_start[bq];
            s1 = slot_start[bq + 1];
        }
        const int nseg = s1 - s0;
        if (nseg == 1) continue;

        float acc[CPL];
#pragma unroll
        for (int c = 0; c < CPL; ++c) acc[c] = 0.f;
        float wsum = 0.f, m = -INFINITY;
        if (nseg <= 4) {
            float l[4], o[4][CPL];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                l[u] = -INFINITY;
                if (u < nseg) {
                    l[u] = part_lse[(size_t)(s0 + u) * M + row];
                    load_partial<CPL>(part_out + ((size_t)(s0 + u) * M + row) * DV + lane * CPL, o[u]);
                }
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) m = fmaxf(m, l[u]);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                if (l[u] != -INFINITY) {  // empty segments (and absent ones) weigh nothing
                    const float wgt = fast_exp2(l[u] - m);
                    wsum += wgt;
#pragma unroll
                    for (int c = 0; c < CPL; ++c) acc[c] += wgt * o[u][c];
                }
            }
        } else {
            for (int r = lane; r < nseg; r += 64) m = fmaxf(m, part_lse[(size_t)(s0 + r) * M + row]);
            m = wave_max64(m);
            if (m != -INFINITY)
                combine_accumulate<DV>(part_out, part_lse, M, row, s0, 0, 1, nseg, m, lane, acc, wsum);
        }
        combine_write<DV>(out, lse, row_g, lane, acc, wsum, m);
    }
}

// One block of sixteen waves per query row (grid-stride over rows): the waves
// take the row's segments in turn and their sums meet in LDS.
constexpr int kCombineWideWaves = 16;

template <int DV>
__global__ void __launch_bounds__(64 * kCombineWideWaves) combine_wide_kernel(
    int B, int M, const PlanHeader *__restrict__ hdr, const int *__restrict__ slot_start,
    const uint16_t *__restrict__ part_out, const float *__restrict__ part_lse, uint16_t *__restrict__ out,
    float *__restrict__ lse)
{
    constexpr int NW = kCombineWideWaves, CPL = DV / 64;
    if (hdr->merge_seqs == 0) return;
    __shared__ float red_m[NW];
    __shared__ float red_w[NW];
    __shared__ float red_acc[NW][DV];  // [wave][column-in-lane c * 64 + lane]
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const long rows = (long)B * M;
    for (long row_g = blockIdx.x; row_g < rows; row_g += gridDim.x) {
        const int bq = (int)(row_g / M);
        const int row = (int)(row_g - (long)bq * M);
        const int s0 = slot_start[bq];
        const int nseg = slot_start[bq + 1] - s0;
        if (nseg == 1) continue;  // the same for the whole block

        float m = -INFINITY;
        for (int r = threadIdx.x; r < nseg; r += 64 * NW) m = fmaxf(m, part_lse[(size_t)(s0 + r) * M + row]);
        m = wave_max64(m);
        if (lane == 0) red_m[wave] = m;
        __syncthreads();
        m = red_m[0];
#pragma unroll
        for (int w2 = 1; w2 < NW; ++w2) m = fmaxf(m, red_m[w2]);

        float acc[CPL];
#pragma unroll
        for (int c = 0; c < CPL; ++c) acc[c] = 0.f;
        float wsum = 0.f;
        if (m != -INFINITY)
            combine_accumulate<DV>(part_out, part_lse, M, row, s0, wave, NW, nseg, m, lane, acc, wsum);
#pragma unroll
        for (int c = 0; c < CPL; ++c) red_acc[wave][c * 64 + lane] = acc[c];
        if (lane == 0) red_w[wave] = wsum;
        __syncthreads();
        if (wave == 0) {
            float tot[CPL];
            float ws = 0.f;
#pragma unroll
            for (int c = 0; c < CPL; ++c) tot[c] = 0.f;
            for (int w2 = 0; w2 < NW; ++w2) {
                ws += red_w[w2];
#pragma unroll
                for (int c = 0; c < CPL; ++c) tot[c] += red_acc[w2][c * 64 + lane];
            }
            combine_write<DV>(out, lse, row_g, lane, tot, ws, m);
        }
        __syncthreads();  // red_* are reused by the next row
    }
}

// Merge of two attention results over disjoint sets of cache rows (natural-log
// lse): lse = log(e^l1 + e^l2), out = (e^l1 o1 + e^l2 o2) / (e^l1 + e^l2); a
// side with lse = -inf weighs nothing, and both -inf give out = 0, lse = -inf.
// One wave per row (grid-stride), DV columns over the 64 lanes.
template <int DV>
__global__ void __launch_bounds__(256) merge2_kernel(long rows, const uint16_t *__restrict__ o1,
                                                     const float *__restrict__ l1, const uint16_t *__restrict__ o2,
                                                     const float *__restrict__ l2, uint16_t *__restrict__ out,
                                                     float *__restrict__ lse)
{
    constexpr int CPL = DV / 64;
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    for (long row = (long)blockIdx.x * 4 + wave; row < rows; row += (long)gridDim.x * 4) {
        const float a = l1[row], b = l2[row];
        const float m = fmaxf(a, b);
        float acc[CPL];
#pragma unroll
        for (int c = 0; c < CPL; ++c) acc[c] = 0.f;
        float wsum = 0.f;
        if (m != -INFINITY) {
            const float wa = fast_exp2((a - m) * kLog2e), wb = fast_exp2((b - m) * kLog2e);
            float o[CPL];
            if (wa > 0.f) {  // a side that weighs nothing is not read
                load_partial<CPL>(o1 + (size_t)row * DV + lane * CPL, o);
#pragma unroll
                for (int c = 0; c < CPL; ++c) acc[c] += wa * o[c];
            }
            if (wb > 0.f) {
                load_partial<CPL>(o2 + (size_t)row * DV + lane * CPL, o);
#pragma unroll
                for (int c = 0; c < CPL; ++c) acc[c] += wb * o[c];
            }
            wsum = wa + wb;
        }
        // combine_write takes the maximum in log2 units
        combine_write<DV>(out, lse, row, lane, acc, wsum, m * kLog2e);
    }
}

// out[row] = [a[row] | b[row]] for rows of wa and wb bf16 values (both
// multiples of 8): 16-byte chunks, one per thread (grid-stride).
__global__ void __launch_bounds__(256) concat_rows_kernel(const uint16_t *__restrict__ a, int wa,
                                                          const uint16_t *__restrict__ b, int wb,
                                                          uint16_t *__restrict__ out, long rows)
{
    const int ca = wa / 8, cb = wb / 8, cr = ca + cb;
    const long total = rows * cr;
    for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (long)gridDim.x * blockDim.x) {
        const long row = i / cr;
        const int c = (int)(i - row * cr);
        const u32x4 v = c < ca ? *(const u32x4 *)(a + row * wa + 8 * c) : *(const u32x4 *)(b + row * wb + 8 * (c - ca));
        *(u32x4 *)(out + row * (wa + wb) + 8 * c) = v;
    }
}

// Blocks of the one-wave-per-row launch: enough to cover the rows with a few
// waves per CU, never more than one block per four rows.
inline unsigned combine_grid(long rows, int cus)
{
    const long want = (long)cus * 4;
    const long need = (rows + 3) / 4;
    return (unsigned)(need < want ? (need > 0 ? need : 1) : want);
}

// Whether a split over `workers` workers leaves the b sequences more than 16
// segments each on average: then the combine gives each row a block.
inline bool combine_use_wide(int b, int workers) { return (long)b + workers > 16L * b; }

inline unsigned combine_wide_grid(long rows, int cus)
{
    return (unsigned)(rows < cus ? (rows > 0 ? rows : 1) : cus);
}

}  // namespace da
