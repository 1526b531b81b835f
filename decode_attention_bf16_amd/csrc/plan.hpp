// Split-KV work partition, computed on the device from seqlens (no host sync).
//
// The cache rows of every sequence are cut into tiles of `tile` tokens; tile j
// of sequence b covers rows [j*tile, min((j+1)*tile, L_b)). The flat list of
// all tiles (sequence-major) is divided into equal runs of `per` tiles, one run
// per worker. A worker's run may cover parts of several sequences; each
// (worker, sequence) overlap is a "segment" with its own partial result slot.
// Slots are numbered in the flat order, so the segments of one sequence occupy
// slot_start[b] .. slot_start[b+1]-1. A sequence with exactly one segment is
// finished by its worker; one with several is merged by the combine kernel.
// The total number of segments is at most b + workers - 1.
#pragma once

#include "common.hpp"

namespace da {

struct PlanHeader {
    int total_tiles;
    int per;  // tiles per worker (>= 1)
    int workers;
    int tile;
};

// Workspace layout (all offsets 256-byte aligned), shared by MLA and GQA.
struct WsLayout {
    size_t header, tile_start, slot_start, part_lse, part_out, total;
    int max_slots;
};

static inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

static inline WsLayout ws_layout(int b, int rows_per_seq, int dv, int workers)
{
    WsLayout w;
    w.max_slots = b + workers;
    size_t off = 0;
    w.header = off;
    off = align256(off + sizeof(PlanHeader));
    w.tile_start = off;
    off = align256(off + sizeof(int) * (size_t)(b + 1));
    w.slot_start = off;
    off = align256(off + sizeof(int) * (size_t)(b + 1));
    w.part_lse = off;
    off = align256(off + sizeof(float) * (size_t)w.max_slots * rows_per_seq);
    w.part_out = off;
    off = align256(off + sizeof(float) * (size_t)w.max_slots * rows_per_seq * dv);
    w.total = off;
    return w;
}

constexpr int kPlanThreads = 64;  // one wave: no block barriers on the planner's short critical path

// Exclusive prefix sum of `v` across the wave's 64 lanes; `total` gets the sum.
__device__ __forceinline__ int wave_exclusive_scan(int v, int &total)
{
    const int lane = threadIdx.x & 63;
    int incl = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(incl, off);
        if (lane >= off) incl += y;
    }
    total = __shfl(incl, 63);
    return incl - v;
}

// One wave. Lane l owns a contiguous run of ceil(b / 64) sequences.
__global__ void __launch_bounds__(kPlanThreads) plan_kernel(const int32_t *__restrict__ seqlens, int b, int t_max,
                                                            int tile, int workers, PlanHeader *__restrict__ hdr,
                                                            int *__restrict__ tile_start,
                                                            int *__restrict__ slot_start)
{
    const int lane = threadIdx.x;
    const int chunk = (b + kPlanThreads - 1) / kPlanThreads;
    const int lo = min(b, lane * chunk);
    const int hi = min(b, lo + chunk);

    // Pass 1: tiles per sequence -> tile_start (exclusive prefix), total.
    int local = 0;
    for (int i = lo; i < hi; ++i) {
        const int L = clamp_len(seqlens[i], t_max);
        local += (L + tile - 1) / tile;
    }
    int total = 0;
    int run = wave_exclusive_scan(local, total);
    for (int i = lo; i < hi; ++i) {
        tile_start[i] = run;
        const int L = clamp_len(seqlens[i], t_max);
        run += (L + tile - 1) / tile;
    }
    const int per = max(1, (total + workers - 1) / workers);

    // Pass 2: segments per sequence -> slot_start.
    int segs = 0;
    for (int i = lo; i < hi; ++i) {
        const int L = clamp_len(seqlens[i], t_max);
        const int nt = (L + tile - 1) / tile;
        if (nt > 0) {
            const int first = tile_start[i];
            segs += (first + nt - 1) / per - first / per + 1;
        }
    }
    int segs_total = 0;
    int srun = wave_exclusive_scan(segs, segs_total);
    for (int i = lo; i < hi; ++i) {
        slot_start[i] = srun;
        const int L = clamp_len(seqlens[i], t_max);
        const int nt = (L + tile - 1) / tile;
        if (nt > 0) {
            const int first = tile_start[i];
            srun += (first + nt - 1) / per - first / per + 1;
        }
    }
    if (lane == 0) {
        tile_start[b] = total;
        slot_start[b] = segs_total;
        hdr->total_tiles = total;
        hdr->per = per;
        hdr->workers = workers;
        hdr->tile = tile;
    }
}

// Largest index i in [0, b] with tile_start[i] <= t (tile_start[b] = total).
__device__ __forceinline__ int find_sequence(const int *__restrict__ tile_start, int b, int t)
{
    int lo = 0, hi = b;  // invariant: tile_start[lo] <= t
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (tile_start[mid] <= t)
            lo = mid;
        else
            hi = mid - 1;
    }
    return lo;
}

}  // namespace da
