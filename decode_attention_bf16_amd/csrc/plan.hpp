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
//
// The plan costs no launch of its own: every wave of a tile kernel derives the
// part it needs (PlanWalk: totals by a wave scan over seqlens, then a cursor
// walking forward through its worker's sequences), and one wave of the tile
// kernel's first block writes the whole plan as arrays for the combine kernel
// that follows on the stream (write_plan).
#pragma once

#include "common.hpp"

namespace da {

struct PlanHeader {
    int total_tiles;
    int per;  // tiles per worker (>= 1)
    int workers;
    int tile;
    int merge_seqs;  // sequences the combine kernel must write (segments != 1)
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
    w.part_out = off;  // bf16 partial outputs, normalized by their own softmax sums
    off = align256(off + sizeof(uint16_t) * (size_t)w.max_slots * rows_per_seq * dv);
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

constexpr int kPlanRegChunks = 4;  // chunks of 64 sequences kept in registers between the passes

// Segments of a sequence whose nt tiles start at flat tile `first`.
__device__ __forceinline__ int plan_segments(int first, int nt, int per)
{
    return nt > 0 ? (first + nt - 1) / per - first / per + 1 : 0;
}

// The whole plan as arrays (tile_start, slot_start, header) for the combine
// kernel, written by one wave of the tile kernel. Sequence i is lane i % 64 of
// chunk i / 64; the first kPlanRegChunks chunks stay in registers from the
// first pass to the second, so a batch of up to 256 sequences costs one
// dependent round trip to memory (the seqlens loads); larger batches reload
// their later chunks.
__device__ __noinline__ void write_plan(const int32_t *__restrict__ seqlens, int b, int t_max, int tile, int workers,
                                        PlanHeader *__restrict__ hdr, int *__restrict__ tile_start,
                                        int *__restrict__ slot_start)
{
    const int lane = threadIdx.x & 63;
    // Pass 1: tiles per sequence -> tile_start (exclusive prefix), total.
    int nt_r[kPlanRegChunks], first_r[kPlanRegChunks];
#pragma unroll
    for (int c = 0; c < kPlanRegChunks; ++c) {
        const int i = c * kPlanThreads + lane;
        const int L = i < b ? clamp_len(seqlens[i], t_max) : 0;
        nt_r[c] = (L + tile - 1) / tile;
    }
    int run = 0;
#pragma unroll
    for (int c = 0; c < kPlanRegChunks; ++c) {
        int tot;
        const int ex = wave_exclusive_scan(nt_r[c], tot);
        first_r[c] = run + ex;
        const int i = c * kPlanThreads + lane;
        if (i < b) tile_start[i] = first_r[c];
        run += tot;
    }
    for (int base = kPlanRegChunks * kPlanThreads; base < b; base += kPlanThreads) {
        const int i = base + lane;
        const int L = i < b ? clamp_len(seqlens[i], t_max) : 0;
        int tot;
        const int ex = wave_exclusive_scan((L + tile - 1) / tile, tot);
        if (i < b) tile_start[i] = run + ex;
        run += tot;
    }
    const int total = run;
    const int per = max(1, (total + workers - 1) / workers);

    // Pass 2: segments per sequence -> slot_start; sequences to merge.
    int srun = 0, nmerge = 0;
    auto chunk2 = [&](int base, int nt, int first) {
        const int i = base + lane;
        const int segs = i < b ? plan_segments(first, nt, per) : 1;
        int tot;
        const int ex = wave_exclusive_scan(i < b ? segs : 0, tot);
        if (i < b) slot_start[i] = srun + ex;
        srun += tot;
        nmerge += __builtin_popcountll(__builtin_amdgcn_ballot_w64(segs != 1));
    };
#pragma unroll
    for (int c = 0; c < kPlanRegChunks; ++c)
        if (c * kPlanThreads < b) chunk2(c * kPlanThreads, nt_r[c], first_r[c]);
    for (int base = kPlanRegChunks * kPlanThreads; base < b; base += kPlanThreads) {
        const int i = base + lane;
        const int L = i < b ? clamp_len(seqlens[i], t_max) : 0;
        chunk2(base, (L + tile - 1) / tile, i < b ? tile_start[i] : 0);
    }
    if (lane == 0) {
        tile_start[b] = total;
        slot_start[b] = srun;
        hdr->total_tiles = total;
        hdr->per = per;
        hdr->workers = workers;
        hdr->tile = tile;
        hdr->merge_seqs = nmerge;
    }
}


// A wave's own view of the plan, computed from seqlens with no global scratch
// and no other wave: the total tile count, `per`, this worker's tile range and
// a cursor over the sequences of that range. For the cursor's sequence b it
// holds b's tiles [ts, te), the first partial slot of b (ss = segments of all
// sequences before b) and b's segment count ns. Every member is wave-uniform.
struct PlanWalk {
    int total = 0, per = 1, tile_lo = 0, tile_hi = 0;
    int b = 0, ts = 0, te = 0, ss = 0, ns = 0;
    int nb = 0, tmax = 0, tile = 1;

    // Returns false when the worker has no tile (then nothing else is set).
    __device__ bool init(const int32_t *__restrict__ seqlens, int B, int t_max, int tile_, int workers, int worker)
    {
        nb = B;
        tmax = t_max;
        tile = tile_;
        const int lane = threadIdx.x & 63;
        int nt_r[kPlanRegChunks];
        int run = 0;
#pragma unroll
        for (int c = 0; c < kPlanRegChunks; ++c) {
            const int i = c * kPlanThreads + lane;
            const int L = i < B ? clamp_len(seqlens[i], t_max) : 0;
            nt_r[c] = (L + tile - 1) / tile;
        }
#pragma unroll
        for (int c = 0; c < kPlanRegChunks; ++c) {
            int tot;
            wave_exclusive_scan(nt_r[c], tot);
            run += __builtin_amdgcn_readfirstlane(tot);
        }
        for (int base = kPlanRegChunks * kPlanThreads; base < B; base += kPlanThreads) {
            const int i = base + lane;
            const int L = i < B ? clamp_len(seqlens[i], t_max) : 0;
            int tot;
            wave_exclusive_scan((L + tile - 1) / tile, tot);
            run += __builtin_amdgcn_readfirstlane(tot);
        }
        total = run;
        per = max(1, (total + workers - 1) / workers);
        tile_lo = worker * per;
        if (tile_lo >= total) return false;
        tile_hi = min(total, tile_lo + per);

        // the sequence holding tile_lo, and the slots of the sequences before it
        int run_t = 0, run_s = 0;
        auto chunk = [&](int base, int nt) -> bool {
            const int i = base + lane;
            int t_tot, s_tot;
            const int first = run_t + wave_exclusive_scan(nt, t_tot);
            const int seg = i < B ? plan_segments(first, nt, per) : 0;
            const int sfirst = run_s + wave_exclusive_scan(seg, s_tot);
            const uint64_t hit = __builtin_amdgcn_ballot_w64(nt > 0 && first <= tile_lo && tile_lo < first + nt);
            if (hit) {
                const int l = (int)__builtin_ctzll(hit);
                b = base + l;
                ts = __builtin_amdgcn_readlane(first, l);
                te = ts + __builtin_amdgcn_readlane(nt, l);
                ss = __builtin_amdgcn_readlane(sfirst, l);
                ns = __builtin_amdgcn_readlane(seg, l);
                return true;
            }
            run_t += __builtin_amdgcn_readfirstlane(t_tot);
            run_s += __builtin_amdgcn_readfirstlane(s_tot);
            return false;
        };
#pragma unroll
        for (int c = 0; c < kPlanRegChunks; ++c)
            if (c * kPlanThreads < B && chunk(c * kPlanThreads, nt_r[c])) return true;
        for (int base = kPlanRegChunks * kPlanThreads; base < B; base += kPlanThreads) {
            const int i = base + lane;
            const int L = i < B ? clamp_len(seqlens[i], t_max) : 0;
            if (chunk(base, (L + tile - 1) / tile)) return true;
        }
        return true;  // not reached: some sequence holds tile_lo < total
    }

    // The plan without a workspace: worker w is sequence w, whose tiles are
    // all its own (one segment, written directly, never merged). Tile indices
    // are local to the sequence. Returns false for an empty sequence.
    __device__ bool init_per_sequence(const int32_t *__restrict__ seqlens, int t_max, int tile_, int seq)
    {
        tmax = t_max;
        tile = tile_;
        const int nt = (clamp_len(seqlens[seq], t_max) + tile - 1) / tile;
        nb = seq + 1;
        b = seq;
        total = nt;
        per = max(1, nt);
        tile_lo = 0;
        tile_hi = nt;
        ts = 0;
        te = nt;
        ss = seq;
        ns = 1;
        return nt > 0;
    }

    // Moves the cursor forward to the sequence holding tile tt (tt >= ts).
    __device__ __forceinline__ void seek(const int32_t *__restrict__ seqlens, int tt)
    {
        if (tt < te) return;
        do {
            ss += ns;
            ++b;
            const int nt = (clamp_len(seqlens[b], tmax) + tile - 1) / tile;
            ts = te;
            te = ts + nt;
            ns = plan_segments(ts, nt, per);
        } while (tt >= te);
        wait_lgkm_visible();
    }

    // Slot of this worker's segment of the cursor's sequence.
    __device__ __forceinline__ int slot(int worker) const { return ss + (worker - ts / per); }
};

}  // namespace da
