// Absorbed-latent MLA decode tile kernel for gfx950.
//
// What it computes ("Mla Analysis" skill page, "Absorption Trick (FlashMLA)"):
// for every query row (b, draft i, head) the scores are [q_lat | q_rope] . Z_j
// over the cached rows Z_j = [latent | rope], and the output is the
// softmax-weighted sum of the latent parts, so attention never leaves latent
// space. In decode all heads of a sequence read the same latent cache, so the
// s*h query rows of a sequence are the M dimension of two dense contractions
// (scores and values) against one shared [tokens, k+p] tile.
//
// Work decomposition: a block (4 score waves plus NVW = 4 value waves, two
// waves per SIMD, when k is a multiple of 128; 4 + 2 otherwise) is one worker
// of the split-KV plan times one block of 64 query rows. The waves have two
// roles and form a two-stage software pipeline over 32-token tiles:
//   score waves (0..3), wave w = 32-row block w/2 x token half w%2 of every
//     tile: S^T[16 tokens, 32 rows] = tile half . Q^T with MFMA 16x16x32 bf16
//     (A = 16 cache rows from LDS, read once and used for both 16-row halves;
//     B = the 32 rows' queries held in registers for the whole segment), then
//     the fp32 online softmax of those 32 rows over its 16 tokens. Holding 32
//     rows per wave halves the LDS tile reads against 16-row waves, which is
//     what bounds a step. The two waves of a row block share one reference
//     maximum per row (below). They publish the bf16 probabilities in the value
//     product's operand layout and, at the end of a segment, each row's
//     (reference, partial sum) of their token half.
//   value waves (4 .. 3+NVW), all 64 rows x k/NVW latent columns each:
//     O^T += V^T . P^T with MFMA 32x32x16 bf16 (two 16-token k-steps per tile,
//     one per token half), A = latent columns of the same LDS tile through the
//     transposing LDS read (ds_read_b64_tr_b16), B = the published
//     probabilities. They also copy the cache tiles HBM -> LDS (buffer_load ...
//     lds, 16 bytes per lane, no registers) two tiles ahead, and write their
//     columns of the outputs.
// In step j the score waves work on tile j while the value waves work on tile
// j-1, so on every SIMD one wave's softmax and LDS traffic overlap the other's
// matrix work, and the score waves never wait for HBM. One barrier per step;
// four tile buffers (j-1 values, j scores, j+1 landed, j+2 in flight). The
// buffer resource covers the sequence's valid rows only, so rows past the
// sequence length (and padding columns) read as zeros whatever the cache holds.
//
// Shared reference maximum. Probabilities are exp2(score - m) against a lazily
// moved per-row reference m (moved only when a score exceeds it by more than
// 2^kRescaleSlack), kept an integer so that every rescale factor is an exact
// power of two. Both token-half waves of a row start a step with the same m.
// A wave that must move it uses its own new reference for that step and flags
// it; after the barrier both waves and the value waves take the larger of the
// two halves' references as the common one, rescaling the partial row sums,
// the accumulators and the probabilities of the half that stayed behind (exact
// in bf16, being a power of two). The common case (no move) costs one flag read.
//
// The score MFMA's output layout (lane: query row l%16, tokens 4(l/16)+i of the
// half) packed to bf16 is directly the value MFMA's B operand for that half's
// k-step once each lane pair (l/16 = 2c, 2c+1) writes its two 8-byte parts.
//
// LDS tile layout: row r (token) holds ROW_CHUNKS 16-byte chunks; logical chunk
// c is stored at c ^ tile_swz(r) (see tile_swz).
#pragma once

#include "common.hpp"
#include "plan.hpp"

namespace da {

constexpr int kMlaTile = 32;  // tokens per tile (also the planner's tile)
constexpr int kMlaRows = 64;  // query rows per block

template <int K, int P>
struct MlaCfg {
    static_assert(K % 64 == 0 && P % 8 == 0, "latent width multiple of 64, rope width multiple of 8");
    static constexpr int KP = K + P;
    static constexpr int KSTEPS = (KP + 31) / 32;               // 32-wide MFMA k-steps of the scores
    static constexpr int SRC_CHUNKS = KP / 8;                   // 16-byte chunks per cache row in HBM
    static constexpr int ROW_CHUNKS = (KSTEPS * 4 + 7) / 8 * 8; // chunks per LDS row (multiple of 8)
    static constexpr int ROW_BYTES = ROW_CHUNKS * 16;
    static constexpr int T = kMlaTile;
    static constexpr int TILE_BYTES = T * ROW_BYTES;
    static constexpr int NBUF = 4;
    // value waves: four when k is a multiple of 128 (each owns k/4 latent
    // columns), else two (k/2 columns, a multiple of 32)
    static constexpr int NVW = K % 128 == 0 ? 4 : 2;
    static constexpr int THREADS = 64 * (4 + NVW);
    static constexpr int ROWS = kMlaRows;
    static constexpr int LPW = T * ROW_CHUNKS / (64 * NVW);     // copy instructions per value wave per tile
    static_assert(T * ROW_CHUNKS % (64 * NVW) == 0, "tile chunks divisible among the value waves");
    static constexpr int CB32 = K / (32 * NVW);                 // 32-column output blocks per value wave
    static constexpr int QCH = 2;                               // score k-steps per LDS read chunk
    static constexpr int QPF = 2;                               // chunks in flight ahead of the MFMAs
    // latent queries of the block's rows, staged once in the space of tile buffers 2 and 3
    static constexpr int KL = K / 32;                           // k-steps that are latent only
    static constexpr int QW = K / 8;                            // 16-byte chunks per latent query row
    static constexpr int QCOPIES = ROWS * QW / 64 / 4;          // copy instructions per score wave
    static constexpr int QLDS_OFF = 2 * TILE_BYTES;
    static_assert(ROWS * QW * 16 <= 2 * TILE_BYTES && NBUF == 4, "the query rows fit tile buffers 2 and 3");
    static_assert(64 % QW == 0, "query rows pack whole copy instructions");
    static constexpr int PBUF_OFF = NBUF * TILE_BYTES;          // [2 slots][2 row blocks][2 halves][64 lanes] x 16 B
    static constexpr int MREF_OFF = PBUF_OFF + 2 * 4 * 64 * 16;   // [2 slots][2 halves][64 rows] float
    static constexpr int FLAG_OFF = MREF_OFF + 2 * 2 * 64 * 4;    // [2 slots][4 score waves] int
    static constexpr int SEG_OFF = FLAG_OFF + 2 * 4 * 4;          // [2 slots][2 halves][64 rows] (ref, sum)
    static constexpr int LDS_BYTES = SEG_OFF + 2 * 2 * 64 * 8;
    static_assert(LDS_BYTES <= 163840, "LDS budget");
    // LDS read offsets that the compiler folds into the 16-bit instruction offset
    static_assert(128 * ((KSTEPS - 1) / 2) + 128 < 65536, "score read offsets");
    static_assert(16 * ROW_BYTES + 2 * K + 128 < 65536, "value read offsets");
};

// Chunk swizzle of tile row r: logical 16-byte chunk c of row r is stored at
// c ^ tile_swz(r) (the low three bits, i.e. within its 128-byte group). A tile
// row is an odd multiple of 128 bytes, so with 64 four-byte banks the row's
// parity picks the bank half and the swizzle the 16-byte group inside it. The
// map is linear in bits 1..3 of r and was chosen, by modelling every access
// pattern of this kernel on the CPU, so that each pass of the LDS (16 lanes of
// a ds_read_b128, 32 lanes of a ds_read_b64_tr_b16; contiguous lanes, or lanes
// l and l+32 together) touches every bank at most once: the 16-row score reads
// need it bijective on bits 1..3, and the transposing reads, whose 32-lane pass
// spans four consecutive rows, need bit 2 of the result to follow bit 1 of r.
__device__ __forceinline__ int tile_swz(int r)
{
    const int i0 = (r >> 1) & 1, i1 = (r >> 2) & 1, i2 = (r >> 3) & 1;
    return i0 | ((i1 ^ i2) << 1) | ((i0 ^ i2) << 2);
}

// Chunk swizzle of the staged latent query rows (QW 16-byte chunks each): chunk
// c of row r is stored at c ^ qlat_swz(r). Rows of 256 bytes or more all start
// on the same bank, so the low four bits take r mod 16; rows of 128 bytes (QW =
// 8) alternate between the two bank halves, so bits 1..3 of r pick the chunk.
// Either way the 16 lanes reading one chunk of 16 consecutive rows touch every
// bank once.
template <int QW>
__device__ __forceinline__ int qlat_swz(int r)
{
    return QW >= 16 ? (r & 15) : ((r >> 1) & 7);
}

// Eight bf16 values times a power of two (exact unless the result leaves the
// normal range; rounded to nearest even then).
__device__ __forceinline__ bf16x8 scale_bf16x8(const bf16x8 &v, float f)
{
    const u32x4 u = __builtin_bit_cast(u32x4, v);
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = pack_bf16x2(bf16lo_to_f32(u[i]) * f, bf16hi_to_f32(u[i]) * f);
    return __builtin_bit_cast(bf16x8, r);
}

template <int K, int P>
__global__ void __launch_bounds__((MlaCfg<K, P>::THREADS), 1)
    mla_decode_kernel(const uint16_t *__restrict__ q_lat, const uint16_t *__restrict__ q_rope,
                      const uint16_t *__restrict__ cache, const int32_t *__restrict__ seqlens, int B, int s,
                      int h, int t_max, float scale_log2, int row_blocks, int units,
                      PlanHeader *__restrict__ hdr, int *__restrict__ tile_start, int *__restrict__ slot_start,
                      uint16_t *__restrict__ out, float *__restrict__ lse, uint16_t *__restrict__ part_out,
                      float *__restrict__ part_lse)
{
    using C = MlaCfg<K, P>;
    extern __shared__ __attribute__((aligned(1024))) char smem[];
    DA_LDS char *lds = (DA_LDS char *)smem;

    // Every early exit below is taken by the whole block.
    const int unit = xcd_linear_unit(blockIdx.x, gridDim.x);
    if (unit >= units) return;
    const int worker = unit / row_blocks;
    const int rb = unit - worker * row_blocks;
    const int workers = units / row_blocks;
    const int M = s * h;  // query rows per sequence
    // Without a workspace (hdr == nullptr) worker w is sequence w and writes its
    // rows directly; otherwise one wave writes the plan as arrays for the
    // combine kernel, and every wave derives its own view of it.
    const bool per_seq = hdr == nullptr;
    // The first segment's latent queries are staged through LDS (below) when every query
    // row block is read by four or more workers (split-KV with workers >= 4 b): their
    // copies then mostly hit L2 and land well before the direct loads would. The staging
    // holds back the third tile's copy until the queries are read out of its buffer, which
    // costs more than it gains where the queries come from HBM. Measured per call: s = 1,
    // b = 32, h = 128 (four workers per sequence) 47.7-47.8 against 49.7-49.8 us; one worker
    // per sequence (s = 4) 141.6-146.1 against 140.3-141.4; ragged b = 64 (two per
    // sequence) 384.4-385.3 against 380.0-382.4.
    const bool stage_q = !per_seq && workers >= 4 * B;
    if (!per_seq && unit == 0 && threadIdx.x < 64)
        write_plan(seqlens, B, t_max, C::T, workers, hdr, tile_start, slot_start);
    PlanWalk plan;
    if (per_seq ? !plan.init_per_sequence(seqlens, t_max, C::T, worker)
                : !plan.init(seqlens, B, t_max, C::T, workers, worker)) {
        if (per_seq) {
            // a sequence with no cache row: its rows are out = 0, lse = -inf
            const int r0 = rb * C::ROWS;
            const int nr = min(C::ROWS, M - r0);
            uint16_t *o = out + ((size_t)worker * M + r0) * K;
            for (int i = threadIdx.x; i < nr * (K / 8); i += C::THREADS)
                *(u32x4 *)(o + (size_t)i * 8) = u32x4{0u, 0u, 0u, 0u};
            for (int i = threadIdx.x; i < nr; i += C::THREADS) lse[(size_t)worker * M + r0 + i] = -INFINITY;
        }
        return;
    }
    const int tile_lo = plan.tile_lo;
    const int ntiles = plan.tile_hi - tile_lo;

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int n = lane & 15;
    const int g = lane >> 4;

    DA_LDS char *pbuf = lds + C::PBUF_OFF;
    DA_LDS float *mref_buf = (DA_LDS float *)(lds + C::MREF_OFF);
    DA_LDS int *flag_buf = (DA_LDS int *)(lds + C::FLAG_OFF);
    DA_LDS float *seg_buf = (DA_LDS float *)(lds + C::SEG_OFF);

    if (w < 4) {
        // ============================================================ score waves
        const int r2 = w >> 1;          // 32-row block of the block's 64 rows
        const int tb = w & 1;           // token half: tokens 16 tb .. 16 tb + 15 of every tile
        const int rowl = 32 * r2 + n;   // block-local rows rowl (rr = 0) and rowl + 16 (rr = 1)
        int row[2];
        bool row_ok[2];
#pragma unroll
        for (int rr = 0; rr < 2; ++rr) {
            row[rr] = rb * C::ROWS + rowl + 16 * rr;
            row_ok[rr] = row[rr] < M;
        }
        const int sq = tile_swz(n);  // = tile_swz(16 tb + n): the swizzle ignores bit 4
        const int trow = (16 * tb + n) * C::ROW_BYTES;
        const int qk_off0 = trow + ((g ^ sq) << 4);        // even k-steps
        const int qk_off1 = trow + (((4 + g) ^ sq) << 4);  // odd k-steps

        bf16x8 qB[2][C::KSTEPS];
        // mref: the common reference of the rows at the start of a step (log2
        // units, integer or -inf); muse: this wave's reference in the step just
        // done; moved: whether this wave moved it there
        float mref[2] = {-INFINITY, -INFINITY}, muse[2] = {-INFINITY, -INFINITY}, lsum[2] = {0.f, 0.f};
        bool moved = false;
        int nvis[2] = {0, 0}, nvis_min = 0;
        PlanWalk cur = plan;
        // a segment starts: its rows' queries, visible lengths and fresh softmax state
        // (lat_in_lds: the latent k-steps' queries come from LDS instead, below)
        auto start_segment = [&](bool lat_in_lds) {
            const int L = clamp_len(seqlens[cur.b], t_max);
#pragma unroll
            for (int rr = 0; rr < 2; ++rr) {
                nvis[rr] = row_ok[rr] ? (L - s + row[rr] / h + 1) : 0;
#pragma unroll
                for (int kk = 0; kk < C::KSTEPS; ++kk) {
                    if (lat_in_lds && kk < C::KL) continue;
                    u32x4 v = {0u, 0u, 0u, 0u};
                    const int e0 = kk * 32 + g * 8;
                    if (row_ok[rr]) {
                        if (e0 < K)
                            v = *(const u32x4 *)(q_lat + ((size_t)cur.b * M + row[rr]) * K + e0);
                        else if (e0 - K < P)
                            v = *(const u32x4 *)(q_rope + ((size_t)cur.b * M + row[rr]) * P + (e0 - K));
                    }
                    qB[rr][kk] = as_bf16x8(v);
                }
                mref[rr] = -INFINITY;
                muse[rr] = -INFINITY;
                lsum[rr] = 0.f;
            }
            moved = false;
            int mn = min(nvis[0], nvis[1]);
            for (int off = 1; off < 64; off <<= 1) mn = min(mn, __shfl_xor(mn, off));
            nvis_min = mn;
        };
        if (stage_q) {
            // The first segment's latent queries come through LDS: the block's 64 rows are
            // copied HBM -> LDS whole (a row's 2K bytes in one run; loads straight into the
            // MFMA operand layout move 16 rows x 64 bytes each), into the space of tile
            // buffers 2 and 3, which the value waves fill only once the queries are read.
            // Rows past M read as zeros. Row r's chunk c is stored at c ^ qlat_swz(r).
            const int r0 = rb * C::ROWS;
            const u32x4 rq = raw_buffer_rsrc(q_lat + ((size_t)cur.b * M + r0) * K, (uint32_t)(M - r0) * K * 2);
#pragma unroll
            for (int it = 0; it < C::QCOPIES; ++it) {
                const int i = it * 4 + w;
                const int r = i * (64 / C::QW) + lane / C::QW;
                const int c = (lane % C::QW) ^ qlat_swz<C::QW>(r);
                lds_dma16(rq, lds + C::QLDS_OFF + i * 1024, (uint32_t)((r * K + c * 8) * 2));
            }
            start_segment(true);  // the rope k-steps' queries: registers
            wait_vmcnt<0>();
            lds_barrier();  // every wave's query rows, and tile 0, have landed
#pragma unroll
            for (int rr = 0; rr < 2; ++rr) {
                const int rq = rowl + 16 * rr;
#pragma unroll
                for (int kk = 0; kk < C::KL; ++kk)
                    qB[rr][kk] = *(const DA_LDS bf16x8 *)(lds + C::QLDS_OFF + rq * C::QW * 16 +
                                                          (((kk * 4 + g) ^ qlat_swz<C::QW>(rq)) << 4));
            }
            lds_barrier();  // the query rows are read: the value waves may refill that space
        } else {
            start_segment(false);  // the first queries load while the first tiles are copied
            lds_barrier();         // tile 0 has landed
        }
        for (int j = 0; j <= ntiles; ++j) {
            if (j < ntiles) {
                const int tt = tile_lo + j;
                const bool new_seg = j > 0 && tt >= cur.te;
                cur.seek(seqlens, tt);
                const int slot = j & 1;
                // the partner half's flag of the previous step, consumed after the MFMAs
                int pflag = 0;
                if (j > 0 && !new_seg) pflag = flag_buf[(slot ^ 1) * 4 + (w ^ 1)];
                if (new_seg) start_segment(false);
                const DA_LDS char *tile = lds + (j % C::NBUF) * C::TILE_BYTES;

                // S^T[16 tokens, 32 rows]. The tile's A fragments are read in
                // chunks of QCH k-steps, QPF chunks ahead of the MFMAs that use
                // them, so LDS latency hides behind matrix work; each fragment
                // feeds the MFMAs of both 16-row halves.
                f32x4 S[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
                {
                    constexpr int QCH = C::QCH, QPF = C::QPF;
                    constexpr int NQC = (C::KSTEPS + QCH - 1) / QCH;
                    bf16x8 af[QPF][QCH];
                    auto load_chunk = [&](int c, bf16x8(&d)[QCH]) {
#pragma unroll
                        for (int i = 0; i < QCH; ++i) {
                            const int kk = c * QCH + i;
                            if (kk < C::KSTEPS)
                                d[i] = *(const DA_LDS bf16x8 *)(tile + ((kk & 1) ? qk_off1 : qk_off0) + 128 * (kk >> 1));
                        }
                    };
#pragma unroll
                    for (int c = 0; c < QPF; ++c)
                        if (c < NQC) load_chunk(c, af[c]);
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int c = 0; c < NQC; ++c) {
#pragma unroll
                        for (int i = 0; i < QCH; ++i) {
                            const int kk = c * QCH + i;
                            if (kk < C::KSTEPS) {
                                S[0] = mfma16x16x32(af[c % QPF][i], qB[0][kk], S[0]);
                                S[1] = mfma16x16x32(af[c % QPF][i], qB[1][kk], S[1]);
                            }
                        }
                        __builtin_amdgcn_sched_barrier(0);
                        if (c + QPF < NQC) load_chunk(c + QPF, af[c % QPF]);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
                // draft / length mask, only on tiles that reach past some row's visible end
                const int tokh = (tt - cur.ts) * C::T + 16 * tb;  // first token of this half
                if (tokh + 16 > nvis_min) {
#pragma unroll
                    for (int rr = 0; rr < 2; ++rr)
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            if (tokh + 4 * g + i >= nvis[rr]) S[rr][i] = -INFINITY;
                }
                // the common reference after the previous step: the larger of the
                // two halves' references (both waves of the row block agree)
                const bool pf = __builtin_amdgcn_readfirstlane(pflag) != 0;
                if (pf || moved) {
#pragma unroll
                    for (int rr = 0; rr < 2; ++rr) {
                        const float mp = pf ? mref_buf[((slot ^ 1) * 2 + (tb ^ 1)) * 64 + rowl + 16 * rr] : mref[rr];
                        const float mc = fmaxf(muse[rr], mp);
                        lsum[rr] *= mc == -INFINITY ? 1.f : fast_exp2(muse[rr] - mc);
                        mref[rr] = mc;
                    }
                }
                // online softmax of the 32 rows over this half's 16 tokens. Lane
                // (n, g) holds 4 scores of each of rows rowl and rowl + 16; the
                // references are kept identical on a row's four lanes (g = 0..3).
                // A lane-local test decides whether any reference must move
                // (rare: mostly the first tile of a segment); only then is the
                // row maximum formed across the four lanes.
                float m[2] = {-INFINITY, -INFINITY};
#pragma unroll
                for (int rr = 0; rr < 2; ++rr)
#pragma unroll
                    for (int i = 0; i < 4; ++i) m[rr] = fmaxf(m[rr], S[rr][i]);
                const bool upd = __builtin_amdgcn_ballot_w64(m[0] * scale_log2 > mref[0] + kRescaleSlack ||
                                                             m[1] * scale_log2 > mref[1] + kRescaleSlack) != 0;
                float mu[2] = {mref[0], mref[1]};
                if (upd) {
#pragma unroll
                    for (int rr = 0; rr < 2; ++rr) {
                        const float mt = wave_max_across_groups16(m[rr]) * scale_log2;  // row max, log2 units
                        mu[rr] = fmaxf(mref[rr], __builtin_ceilf(mt));
                        lsum[rr] *= mu[rr] == -INFINITY ? 1.f : fast_exp2(mref[rr] - mu[rr]);
                        if (g == 0) mref_buf[(slot * 2 + tb) * 64 + rowl + 16 * rr] = mu[rr];
                    }
                }
                if (lane == 0) flag_buf[slot * 4 + w] = upd ? 1 : 0;
                moved = upd;
#pragma unroll
                for (int rr = 0; rr < 2; ++rr) {
                    muse[rr] = mu[rr];
                    const float ms = mu[rr] == -INFINITY ? 0.f : mu[rr];
                    float p[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        p[i] = fast_exp2(__builtin_fmaf(S[rr][i], scale_log2, -ms));
                        lsum[rr] += p[i];
                    }
                    // B operand of the 32x32x16 value MFMA: [slot][row block][half][lane]
                    // 16 bytes, lane l = row l%32 of the block and tokens 8(l/32) + 0..7
                    // of the half; this lane holds tokens 4g .. 4g + 3 of the half
                    const int l2 = 32 * (g >> 1) + 16 * rr + n;
                    *(DA_LDS u32x2 *)(pbuf + ((((slot * 2 + r2) * 2 + tb) * 64 + l2) * 16 + 8 * (g & 1))) =
                        u32x2{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])};
                }
                if (tt + 1 >= cur.te || j + 1 == ntiles) {
#pragma unroll
                    for (int rr = 0; rr < 2; ++rr) {
                        const float ls = wave_sum_across_groups16(lsum[rr]);
                        if (g == 0) {
                            seg_buf[((slot * 2 + tb) * 64 + rowl + 16 * rr) * 2 + 0] = mu[rr];
                            seg_buf[((slot * 2 + tb) * 64 + rowl + 16 * rr) * 2 + 1] = ls;
                        }
                    }
                }
            }
            lds_barrier();
        }
    } else {
        // ============================================================ value waves
        const int vw = w - 4;

        // HBM -> LDS copy of tile j of this worker into buffer j % NBUF:
        // copy_setup resolves the sequence, copy_part issues copy instruction
        // `it` of this wave (LPW per wave per tile).
        PlanWalk dma = plan;
        int dma_b = -1, dma_len = 0;
        auto copy_setup = [&](int j, u32x4 &rsrc, uint32_t &tile_bytes_in_seq) {
            const int tt = tile_lo + j;
            dma.seek(seqlens, tt);
            if (dma.b != dma_b) {
                dma_b = dma.b;
                dma_len = clamp_len(seqlens[dma.b], t_max);
                wait_lgkm_visible();
            }
            rsrc = raw_buffer_rsrc(cache + (size_t)dma.b * t_max * C::KP, (uint32_t)dma_len * C::KP * 2);
            tile_bytes_in_seq = (uint32_t)(tt - dma.ts) * C::T * C::KP * 2;
        };
        auto copy_part = [&](int j, const u32x4 &rsrc, uint32_t tile_bytes_in_seq, int it) {
            const int pch = (it * C::NVW + vw) * 64 + lane;  // physical chunk within the tile
            const int r = pch / C::ROW_CHUNKS;
            const int c = (pch - r * C::ROW_CHUNKS) ^ tile_swz(r);
            const uint32_t off =
                c < C::SRC_CHUNKS ? (uint32_t)((r * C::KP + c * 8) * 2) + tile_bytes_in_seq : 0x80000000u;
            lds_dma16(rsrc, lds + (j % C::NBUF) * C::TILE_BYTES + (it * C::NVW + vw) * 1024, off);
        };
        auto issue_tile = [&](int j) {
            u32x4 rsrc;
            uint32_t tbs;
            copy_setup(j, rsrc, tbs);
#pragma unroll
            for (int it = 0; it < C::LPW; ++it) copy_part(j, rsrc, tbs, it);
        };

        // accumulators [32-row block][32-column block]; lane l holds query row
        // 32 r2 + l%32 of the block. macc: the reference of those rows.
        typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
        f32x16 acw[2][C::CB32];
        float macc[2] = {-INFINITY, -INFINITY};
        auto zero_acc = [&]() {
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                macc[r] = -INFINITY;
#pragma unroll
                for (int cb = 0; cb < C::CB32; ++cb)
#pragma unroll
                    for (int e = 0; e < 16; ++e) acw[r][cb][e] = 0.f;
            }
        };
        zero_acc();
        // byte offset (within a tile) of transposing read hh of k-step ks for
        // 32-column block cb; lane l gets tokens 16ks + 8(l/32) + 4hh + 0..3 of
        // column 32cb + l%32 of this wave's columns
        auto tr32_addr = [&](int cb, int ks, int hh) -> int {
            const int tok = 16 * ks + 8 * (g >> 1) + 4 * hh + (n >> 2);
            const int chunk = (vw * (K / C::NVW) + 32 * cb) / 8 + 2 * (g & 1) + ((n >> 1) & 1);
            return tok * C::ROW_BYTES + (((chunk & ~7) | ((chunk ^ tile_swz(tok)) & 7)) << 4) + ((n & 1) << 3);
        };
        PlanWalk cur = plan;

        // the first three tiles before step 0 (buffers 0..2), then tile j+2 in step j >= 1
        issue_tile(0);
        if (ntiles > 1) issue_tile(1);
        if (stage_q) {
            if (ntiles > 1)
                wait_vmcnt<C::LPW>();
            else
                wait_vmcnt<0>();
            lds_barrier();  // tile 0 has landed (and the score waves' query rows)
            lds_barrier();  // the score waves have read their queries: buffer 2 is free
            if (ntiles > 2) issue_tile(2);
        } else {
            if (ntiles > 2) issue_tile(2);
            if (ntiles > 2)
                wait_vmcnt<2 * C::LPW>();
            else if (ntiles > 1)
                wait_vmcnt<C::LPW>();
            else
                wait_vmcnt<0>();
            lds_barrier();  // tile 0 has landed
        }
        for (int j = 0; j <= ntiles; ++j) {
            const bool issued = j >= 1 && j + 2 < ntiles;
            bool stored = false;
            const int tt = tile_lo + j - 1;
            const int slot = (j - 1) & 1;
            const DA_LDS char *tile = lds + ((j + C::NBUF - 1) % C::NBUF) * C::TILE_BYTES;
            // all LDS reads of the step first (flags, probabilities, then every
            // transposed latent fragment), the copy and the matrix work after them
            u32x4 fl = {0u, 0u, 0u, 0u};
            bf16x8 pB[4];
            i16x4 vlo[2 * C::CB32], vhi[2 * C::CB32];
            if (j >= 1) {
                fl = *(const DA_LDS u32x4 *)(flag_buf + slot * 4);
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4)
                    pB[r4] = *(const DA_LDS bf16x8 *)(pbuf + ((slot * 4 + r4) * 64 + lane) * 16);
#pragma unroll
                for (int cb = 0; cb < C::CB32; ++cb)
#pragma unroll
                    for (int ks = 0; ks < 2; ++ks) {
                        vlo[2 * cb + ks] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((DA_LDS i16x4 *)(tile + tr32_addr(cb, ks, 0)));
                        vhi[2 * cb + ks] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((DA_LDS i16x4 *)(tile + tr32_addr(cb, ks, 1)));
                    }
            }
            __builtin_amdgcn_sched_barrier(0);
            // the copy of tile j+2 is spread over the matrix work below, so that
            // a stall on a full memory queue overlaps MFMA execution
            u32x4 crsrc = {0u, 0u, 0u, 0u};
            uint32_t ctbs = 0;
            if (issued) copy_setup(j + 2, crsrc, ctbs);
            __builtin_amdgcn_sched_barrier(0);
            if (j >= 1) {
                const bool new_seg = j == 1 || tt >= cur.te;
                cur.seek(seqlens, tt);
                if (new_seg) zero_acc();
                // a half moved its reference: take the larger of the two as the
                // rows' reference and bring the sums and the other half's
                // probabilities to it (powers of two)
                if (__builtin_amdgcn_readfirstlane(fl[0] | fl[1] | fl[2] | fl[3])) {
#pragma unroll
                    for (int r2 = 0; r2 < 2; ++r2) {
                        if (__builtin_amdgcn_readfirstlane(fl[2 * r2] | fl[2 * r2 + 1])) {
                            const int rl = 32 * r2 + (lane & 31);
                            const float ma = fl[2 * r2] ? mref_buf[(slot * 2 + 0) * 64 + rl] : macc[r2];
                            const float mb = fl[2 * r2 + 1] ? mref_buf[(slot * 2 + 1) * 64 + rl] : macc[r2];
                            const float mc = fmaxf(ma, mb);
                            if (mc != -INFINITY) {
                                const float al = fast_exp2(macc[r2] - mc);
#pragma unroll
                                for (int cb = 0; cb < C::CB32; ++cb) acw[r2][cb] *= al;
                                pB[2 * r2] = scale_bf16x8(pB[2 * r2], fast_exp2(ma - mc));
                                pB[2 * r2 + 1] = scale_bf16x8(pB[2 * r2 + 1], fast_exp2(mb - mc));
                            }
                            macc[r2] = mc;
                        }
                    }
                }
                // pB[2 * r2 + ks] = B operand of 32-row block r2, k-step (token half) ks
#pragma unroll
                for (int cb = 0; cb < C::CB32; ++cb) {
                    const bf16x8 a0 = __builtin_bit_cast(
                        bf16x8, __builtin_shufflevector(vlo[2 * cb], vhi[2 * cb], 0, 1, 2, 3, 4, 5, 6, 7));
                    const bf16x8 a1 = __builtin_bit_cast(
                        bf16x8, __builtin_shufflevector(vlo[2 * cb + 1], vhi[2 * cb + 1], 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
                    for (int r2 = 0; r2 < 2; ++r2) {
                        acw[r2][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, pB[2 * r2], acw[r2][cb], 0, 0, 0);
                        acw[r2][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, pB[2 * r2 + 1], acw[r2][cb], 0, 0, 0);
                    }
                    if (issued) {
#pragma unroll
                        for (int it = 0; it < C::LPW; ++it)
                            if ((it * C::CB32) / C::LPW == cb) copy_part(j + 2, crsrc, ctbs, it);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
                // end of a segment: normalize and write the result or the partial
                if (tt + 1 >= cur.te || j == ntiles) {
                    const int bq = cur.b;
                    const int nseg = cur.ns;
                    const int sl = cur.slot(worker);
                    // the result, or this segment's bf16 partial for the combine
                    uint16_t *const dst = nseg == 1 ? out + (size_t)bq * M * K : part_out + (size_t)sl * M * K;
                    auto put4 = [&](int row, int col, const f32x4 &v, float inv) {
                        *(u32x2 *)(dst + (size_t)row * K + col) =
                            u32x2{pack_bf16x2(v[0] * inv, v[1] * inv), pack_bf16x2(v[2] * inv, v[3] * inv)};
                    };
#pragma unroll
                    for (int r2 = 0; r2 < 2; ++r2) {
                        // lane l: query row 32*r2 + l%32; value e of block cb is column
                        // 32cb + 8(e/4) + 4(l/32) + e%4 of this wave's columns
                        const int rloc = 32 * r2 + (lane & 31);
                        const int row = rb * C::ROWS + rloc;
                        if (row < M) {
                            // the row's sum over both halves, at the common reference
                            const float mc = macc[r2];
                            float l = 0.f;
#pragma unroll
                            for (int hh = 0; hh < 2; ++hh) {
                                const float mh = seg_buf[((slot * 2 + hh) * 64 + rloc) * 2 + 0];
                                const float lh = seg_buf[((slot * 2 + hh) * 64 + rloc) * 2 + 1];
                                if (lh > 0.f) l += lh * fast_exp2(mh - mc);
                            }
                            const float inv = l > 0.f ? 1.f / l : 0.f;
                            const float lse2 = l > 0.f ? mc + fast_log2(l) : -INFINITY;
                            const int col0 = vw * (K / C::NVW) + 4 * (g >> 1);
#pragma unroll
                            for (int cb = 0; cb < C::CB32; ++cb)
#pragma unroll
                                for (int qq = 0; qq < 4; ++qq)
                                    put4(row, col0 + 32 * cb + 8 * qq,
                                         f32x4{acw[r2][cb][4 * qq], acw[r2][cb][4 * qq + 1], acw[r2][cb][4 * qq + 2],
                                               acw[r2][cb][4 * qq + 3]},
                                         inv);
                            // one writer per row: lanes 0..31 of the first value wave
                            if (g < 2 && vw == 0) {
                                if (nseg == 1)
                                    lse[(size_t)bq * M + row] = lse2 * kLn2;
                                else
                                    part_lse[(size_t)sl * M + row] = lse2;
                            }
                        }
                    }
                    stored = true;
                }
            }
            // tile j+1 (issued a step ago) must be in LDS before the barrier publishes it
            // (tile j+2, if any, was issued after it: in this step, or before step 0
            // when j = 0; the epilogue's stores come after both)
            if (j + 1 < ntiles) {
                if (j + 2 < ntiles && !stored)
                    wait_vmcnt<C::LPW>();
                else
                    wait_vmcnt<0>();
            }
            lds_barrier();
        }
    }
}

}  // namespace da
