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
// Work decomposition: a block (4 score waves plus NVW = 8 value waves, three
// waves per SIMD, when k >= 256; 4 + 4 otherwise) is one worker of the
// split-KV plan times one block of 64 query rows. The waves have two roles and
// form a two-stage software pipeline over 32-token tiles:
//   score waves (0..3), 16 rows each: S^T[32 tokens, 16 rows] = tile . Q^T with
//     MFMA 16x16x32 bf16 (A = cache tile from LDS, B = the rows' queries held
//     in registers), then the fp32 online softmax of those rows (exp2 domain,
//     lazily moved reference maximum). They publish the bf16 probabilities in
//     the value product's operand layout, the per-row rescale factors when the
//     reference moved and, at the end of a segment, each row's (max, sum).
//   value waves (4 .. 3+NVW), all 64 rows x k/NVW latent columns each:
//     O^T += V^T . P^T with MFMA 32x32x16 bf16 when those columns fill 32-wide
//     blocks (16x16x32 otherwise), A = latent columns of the same LDS tile
//     through the transposing LDS read (ds_read_b64_tr_b16), B = the published
//     probabilities. The first four also copy the cache tiles HBM -> LDS
//     (buffer_load ... lds, 16 bytes per lane, no registers) two tiles ahead;
//     all write their columns of the outputs.
// In step j the score waves work on tile j while the value waves work on tile
// j-1, so on every SIMD one wave's softmax and LDS traffic overlap the other's
// matrix work, and the score waves never wait for HBM. One barrier per step;
// four tile buffers (j-1 values, j scores, j+1 landed, j+2 in flight). The
// buffer resource covers the sequence's valid rows only, so rows past the
// sequence length (and padding columns) read as zeros whatever the cache holds.
//
// The score MFMA's output layout (lane: query row l%16, tokens 4(l/16)+i and
// 16+4(l/16)+i) packed to bf16 is directly the value MFMA's B operand when the
// A operand's tokens are permuted the same way: the transposing reads start at
// tile rows 4(l/16)+(l%16)/4 and 16 more, which yields exactly those tokens.
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
    // value waves: eight when k >= 256 (each owns k/8 latent columns), else four
    static constexpr int NVW = K >= 256 ? 8 : 4;
    static constexpr int THREADS = 64 * (4 + NVW);
    static constexpr int ROWS = kMlaRows;
    static constexpr int LPW = T * ROW_CHUNKS / 256;            // copy instructions per value wave per tile
    static_assert(T * ROW_CHUNKS % 256 == 0, "tile chunks divisible among the four copying waves");
    static constexpr int CBV = K / (16 * NVW);                  // 16-column output blocks per value wave
    // value product with v_mfma_f32_32x32x16_bf16 (two chained 16-token k-steps
    // per accumulator and tile) when a value wave's columns fill 32-column blocks
    static constexpr bool WIDE = K % (32 * NVW) == 0;
    static constexpr int CB32 = K / (32 * NVW);                 // 32-column output blocks per value wave
    static constexpr int QCH = 2;                               // score k-steps per LDS read chunk
    static constexpr int QPF = 2;                               // chunks in flight ahead of the MFMAs
    static constexpr int PBUF_OFF = NBUF * TILE_BYTES;          // [2 slots][4 row blocks][64 lanes] x 16 B
    static constexpr int ALPHA_OFF = PBUF_OFF + 2 * 4 * 64 * 16;  // [2 slots][64 rows] float
    static constexpr int FLAG_OFF = ALPHA_OFF + 2 * 64 * 4;       // [2 slots][4 row blocks] int
    static constexpr int SEG_OFF = FLAG_OFF + 2 * 4 * 4;          // [2 slots][64 rows] (max, sum)
    static constexpr int LDS_BYTES = SEG_OFF + 2 * 64 * 8;
    static_assert(LDS_BYTES <= 163840, "LDS budget");
    // LDS read offsets that the compiler folds into the 16-bit instruction offset
    static_assert(16 * ROW_BYTES + 128 * ((KSTEPS - 1) / 2) + 128 < 65536, "score read offsets");
    static_assert(16 * ROW_BYTES + 2 * K + 128 < 65536, "value read offsets");
};

// Chunk swizzle of tile row r: logical 16-byte chunk c of row r is stored at
// c ^ tile_swz(r) (the low three bits, i.e. within its 128-byte group). A tile
// row is an odd multiple of 128 bytes, so with 64 four-byte banks the row's
// parity picks the bank half and the swizzle the 16-byte group inside it. The
// map is linear in bits 1..3 of r (columns 3, 4, 5 for bits 1, 2, 3) and was
// chosen, by checking every access pattern of this kernel on the CPU, so that
// the 16-row score reads (ds_read_b128) and the 4-row transposing reads
// (ds_read_b64_tr_b16) hit 64 distinct banks under every plausible grouping of
// the 64 lanes into 16- or 32-lane passes (contiguous, or lanes l and l+32).
__device__ __forceinline__ int tile_swz(int r)
{
    const int i0 = (r >> 1) & 1, i1 = (r >> 2) & 1, i2 = (r >> 3) & 1;
    return (i0 ^ i2) | (i0 << 1) | ((i1 ^ i2) << 2);
}

template <int K, int P>
__global__ void __launch_bounds__((MlaCfg<K, P>::THREADS), 1)
    mla_decode_kernel(const uint16_t *__restrict__ q_lat, const uint16_t *__restrict__ q_rope,
                      const uint16_t *__restrict__ cache, const int32_t *__restrict__ seqlens, int B, int s,
                      int h, int t_max, float scale_log2, int row_blocks, int units,
                      PlanHeader *__restrict__ hdr, int *__restrict__ tile_start, int *__restrict__ slot_start,
                      uint16_t *__restrict__ out, float *__restrict__ lse, float *__restrict__ part_out,
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
    // the plan as arrays for the combine kernel; every wave derives its own view
    if (unit == 0 && threadIdx.x < 64) write_plan(seqlens, B, t_max, C::T, workers, hdr, tile_start, slot_start);
    PlanWalk plan;
    if (!plan.init(seqlens, B, t_max, C::T, workers, worker)) return;
    const int tile_lo = plan.tile_lo;
    const int ntiles = plan.tile_hi - tile_lo;

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int n = lane & 15;
    const int g = lane >> 4;
    const int M = s * h;  // query rows per sequence

    DA_LDS char *pbuf = lds + C::PBUF_OFF;
    DA_LDS float *alpha_buf = (DA_LDS float *)(lds + C::ALPHA_OFF);
    DA_LDS int *flag_buf = (DA_LDS int *)(lds + C::FLAG_OFF);
    DA_LDS float *seg_buf = (DA_LDS float *)(lds + C::SEG_OFF);

    if (w < 4) {
        // ============================================================ score waves
        const int sw = w;
        const int row = rb * C::ROWS + sw * 16 + n;  // this lane's query row
        const bool row_ok = row < M;
        const int sq = tile_swz(n);  // rows n and n + 16 share it
        const int qk_off0 = n * C::ROW_BYTES + ((g ^ sq) << 4);        // even k-steps
        const int qk_off1 = n * C::ROW_BYTES + (((4 + g) ^ sq) << 4);  // odd k-steps

        bf16x8 qB[C::KSTEPS];
        float mref = -INFINITY, lsum = 0.f;
        int nvis = 0, nvis_min = 0;
        PlanWalk cur = plan;

        lds_barrier();  // tile 0 has landed
        for (int j = 0; j <= ntiles; ++j) {
            if (j < ntiles) {
                const int tt = tile_lo + j;
                const bool new_seg = j == 0 || tt >= cur.te;
                cur.seek(seqlens, tt);
                if (new_seg) {
                    const int L = clamp_len(seqlens[cur.b], t_max);
                    nvis = row_ok ? (L - s + row / h + 1) : 0;
#pragma unroll
                    for (int kk = 0; kk < C::KSTEPS; ++kk) {
                        u32x4 v = {0u, 0u, 0u, 0u};
                        const int e0 = kk * 32 + g * 8;
                        if (row_ok) {
                            if (e0 < K)
                                v = *(const u32x4 *)(q_lat + ((size_t)cur.b * M + row) * K + e0);
                            else if (e0 - K < P)
                                v = *(const u32x4 *)(q_rope + ((size_t)cur.b * M + row) * P + (e0 - K));
                        }
                        qB[kk] = as_bf16x8(v);
                    }
                    mref = -INFINITY;
                    lsum = 0.f;
                    int mn = nvis;
                    for (int off = 1; off < 64; off <<= 1) mn = min(mn, __shfl_xor(mn, off));
                    nvis_min = mn;
                }
                const DA_LDS char *tile = lds + (j % C::NBUF) * C::TILE_BYTES;

                // S^T[32 tokens, 16 rows]. The tile's A fragments are read in
                // chunks of QCH k-steps, QPF chunks ahead of the MFMAs that use
                // them, so LDS latency hides behind matrix work. Each 16-token
                // block accumulates in one chain: back-to-back MFMAs on the same
                // accumulator forward it without a register read, which measured
                // faster than spreading the k-steps over more accumulators.
                f32x4 S[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
                {
                    constexpr int QCH = C::QCH, QPF = C::QPF;
                    constexpr int NQC = (C::KSTEPS + QCH - 1) / QCH;
                    bf16x8 af[QPF][2 * QCH];
                    auto load_chunk = [&](int c, bf16x8(&d)[2 * QCH]) {
#pragma unroll
                        for (int i = 0; i < QCH; ++i) {
                            const int kk = c * QCH + i;
                            if (kk < C::KSTEPS) {
                                const DA_LDS char *p = tile + ((kk & 1) ? qk_off1 : qk_off0) + 128 * (kk >> 1);
                                d[2 * i] = *(const DA_LDS bf16x8 *)(p);
                                d[2 * i + 1] = *(const DA_LDS bf16x8 *)(p + 16 * C::ROW_BYTES);
                            }
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
                                S[0] = mfma16x16x32(af[c % QPF][2 * i], qB[kk], S[0]);
                                S[1] = mfma16x16x32(af[c % QPF][2 * i + 1], qB[kk], S[1]);
                            }
                        }
                        __builtin_amdgcn_sched_barrier(0);
                        if (c + QPF < NQC) load_chunk(c + QPF, af[c % QPF]);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
                // draft / length mask, only on tiles that reach past some row's visible end
                const int tok0 = (tt - cur.ts) * C::T;
                if (tok0 + C::T > nvis_min) {
#pragma unroll
                    for (int bt = 0; bt < 2; ++bt)
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            if (tok0 + bt * 16 + g * 4 + i >= nvis) S[bt][i] = -INFINITY;
                }
                // online softmax of the 16 rows. Lane (n, g) holds 8 scores of
                // row n; the row's reference maximum mref is kept identical on
                // the row's four lanes (g = 0..3). A lane-local test decides
                // whether any reference must move (rare: mostly the first tile
                // of a segment); only then is the row maximum formed across the
                // four lanes. Row sums stay per lane until the segment ends.
                float m = -INFINITY;
#pragma unroll
                for (int bt = 0; bt < 2; ++bt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) m = fmaxf(m, S[bt][i]);
                const int slot = j & 1;
                const bool upd = __builtin_amdgcn_ballot_w64(m * scale_log2 > mref + kRescaleSlack) != 0;
                if (upd) {
                    const float mt = wave_max_across_groups16(m) * scale_log2;  // row max, log2 units
                    const float mnew = fmaxf(mref, mt);
                    const float alpha = mnew == -INFINITY ? 1.f : fast_exp2(mref - mnew);
                    mref = mnew;
                    lsum *= alpha;
                    if (g == 0) alpha_buf[slot * 64 + sw * 16 + n] = alpha;
                }
                if (lane == 0) flag_buf[slot * 4 + sw] = upd ? 1 : 0;
                const float ms = mref == -INFINITY ? 0.f : mref;
                uint32_t pk[4];
#pragma unroll
                for (int bt = 0; bt < 2; ++bt) {
                    float p[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        p[i] = fast_exp2(__builtin_fmaf(S[bt][i], scale_log2, -ms));
                        lsum += p[i];
                    }
                    pk[2 * bt] = pack_bf16x2(p[0], p[1]);
                    pk[2 * bt + 1] = pack_bf16x2(p[2], p[3]);
                }
                if constexpr (C::WIDE) {
                    // B operand of the 32x32x16 value MFMA: [row block of 32][k-step][lane]
                    // 16 bytes, lane l = row l%32 and tokens 16*ks + 8*(l/32) + 0..7
                    const int l2 = 32 * (g >> 1) + 16 * (sw & 1) + n;
#pragma unroll
                    for (int bt = 0; bt < 2; ++bt)
                        *(DA_LDS u32x2 *)(pbuf + ((((slot * 2 + (sw >> 1)) * 2 + bt) * 64 + l2) * 16 + 8 * (g & 1))) =
                            u32x2{pk[2 * bt], pk[2 * bt + 1]};
                } else {
                    *(DA_LDS u32x4 *)(pbuf + ((slot * 4 + sw) * 64 + lane) * 16) = u32x4{pk[0], pk[1], pk[2], pk[3]};
                }
                if (tt + 1 >= cur.te || j + 1 == ntiles) {
                    const float ls = wave_sum_across_groups16(lsum);
                    if (g == 0) {
                        seg_buf[(slot * 64 + sw * 16 + n) * 2 + 0] = mref;
                        seg_buf[(slot * 64 + sw * 16 + n) * 2 + 1] = ls;
                    }
                }
            }
            lds_barrier();
        }
    } else {
        // ============================================================ value waves
        const int vw = w - 4;
        const int trr = 4 * g + (n >> 2);  // first tile row of this lane's transposing read
        const int st = tile_swz(trr);      // rows trr and trr + 16 share it
        const int hsel = (n & 3) >> 1;
        const int tr_row = trr * C::ROW_BYTES + ((n & 1) << 3);
        int tr_off[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) tr_off[jj] = tr_row + (((2 * jj + hsel) ^ st) << 4);
        // byte offset (within a tile) of this lane's read for output column block cb
        auto tr_addr = [&](int cb) -> int {
            if constexpr (C::CBV % 4 == 0) {
                return tr_off[cb & 3] + 128 * (vw * (C::CBV / 4) + (cb >> 2));
            } else {
                const int jj = vw * C::CBV + cb;  // 16-column block across the full latent width
                return tr_row + (((2 * (jj & 3) + hsel) ^ st) << 4) + 128 * (jj >> 2);
            }
        };

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
            const int pch = (it * 4 + vw) * 64 + lane;  // physical chunk within the tile
            const int r = pch / C::ROW_CHUNKS;
            const int c = (pch - r * C::ROW_CHUNKS) ^ tile_swz(r);
            const uint32_t off =
                c < C::SRC_CHUNKS ? (uint32_t)((r * C::KP + c * 8) * 2) + tile_bytes_in_seq : 0x80000000u;
            lds_dma16(rsrc, lds + (j % C::NBUF) * C::TILE_BYTES + (it * 4 + vw) * 1024, off);
        };
        auto issue_tile = [&](int j) {
            u32x4 rsrc;
            uint32_t tbs;
            copy_setup(j, rsrc, tbs);
#pragma unroll
            for (int it = 0; it < C::LPW; ++it) copy_part(j, rsrc, tbs, it);
        };

        // accumulators: narrow form [16-row block][16-column block] (16x16x32),
        // wide form [32-row block][32-column block] (32x32x16)
        typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
        constexpr int NA4 = C::WIDE ? 1 : 4, NAC = C::WIDE ? 1 : C::CBV;
        constexpr int NW2 = C::WIDE ? 2 : 1, NWC = C::WIDE ? C::CB32 : 1;
        f32x4 acc[NA4][NAC];
        f32x16 acw[NW2][NWC];
        auto zero_acc = [&]() {
            if constexpr (C::WIDE) {
#pragma unroll
                for (int r = 0; r < NW2; ++r)
#pragma unroll
                    for (int cb = 0; cb < NWC; ++cb)
#pragma unroll
                        for (int e = 0; e < 16; ++e) acw[r][cb][e] = 0.f;
            } else {
#pragma unroll
                for (int r4 = 0; r4 < NA4; ++r4)
#pragma unroll
                    for (int cb = 0; cb < NAC; ++cb) acc[r4][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
        };
        zero_acc();
        // wide form: byte offset (within a tile) of transposing read h of k-step
        // ks for 32-column block cb; lane l gets tokens 16ks + 8(l/32) + 4h + 0..3
        // of column 32cb + l%32 of this wave's columns
        auto tr32_addr = [&](int cb, int ks, int h) -> int {
            const int tok = 16 * ks + 8 * (g >> 1) + 4 * h + (n >> 2);
            const int chunk = (vw * (K / C::NVW) + 32 * cb) / 8 + 2 * (g & 1) + ((n >> 1) & 1);
            return tok * C::ROW_BYTES + (((chunk & ~7) | ((chunk ^ tile_swz(tok)) & 7)) << 4) + ((n & 1) << 3);
        };
        PlanWalk cur = plan;

        // the first four value waves copy the tiles (LPW copies each per tile)
        const bool copier = vw < 4;
        if (copier) {
            issue_tile(0);
            if (ntiles > 1) {
                issue_tile(1);
                wait_vmcnt<C::LPW>();
            } else {
                wait_vmcnt<0>();
            }
        }
        lds_barrier();  // tile 0 has landed
        for (int j = 0; j <= ntiles; ++j) {
            const bool issued = copier && j + 2 < ntiles;
            bool stored = false;
            const int tt = tile_lo + j - 1;
            const int slot = (j - 1) & 1;
            const DA_LDS char *tile = lds + ((j + C::NBUF - 1) % C::NBUF) * C::TILE_BYTES;
            // all LDS reads of the step first (flags, probabilities, then every
            // transposed latent fragment), the copy and the matrix work after them
            u32x4 fl = {0u, 0u, 0u, 0u};
            bf16x8 pB[4];
            constexpr int NTR = C::WIDE ? 4 * C::CB32 : C::CBV;
            i16x4 vlo[NTR], vhi[NTR];
            if (j >= 1) {
                fl = *(const DA_LDS u32x4 *)(flag_buf + slot * 4);
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4)
                    pB[r4] = *(const DA_LDS bf16x8 *)(pbuf + ((slot * 4 + r4) * 64 + lane) * 16);
                if constexpr (C::WIDE) {
#pragma unroll
                    for (int cb = 0; cb < C::CB32; ++cb)
#pragma unroll
                        for (int ks = 0; ks < 2; ++ks) {
                            vlo[2 * cb + ks] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((DA_LDS i16x4 *)(tile + tr32_addr(cb, ks, 0)));
                            vhi[2 * cb + ks] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((DA_LDS i16x4 *)(tile + tr32_addr(cb, ks, 1)));
                        }
                } else {
#pragma unroll
                    for (int cb = 0; cb < C::CBV; ++cb) {
                        const DA_LDS char *vb = tile + tr_addr(cb);
                        vlo[cb] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((DA_LDS i16x4 *)(vb));
                        vhi[cb] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((DA_LDS i16x4 *)(vb + 16 * C::ROW_BYTES));
                    }
                }
            }
            __builtin_amdgcn_sched_barrier(0);
            // the copy of tile j+2 is spread over the matrix work below, so that
            // a stall on a full memory queue overlaps MFMA execution
            u32x4 crsrc = {0u, 0u, 0u, 0u};
            uint32_t ctbs = 0;
            if (issued) copy_setup(j + 2, crsrc, ctbs);
            if (j == 0 && issued) {
#pragma unroll
                for (int it = 0; it < C::LPW; ++it) copy_part(j + 2, crsrc, ctbs, it);
            }
            __builtin_amdgcn_sched_barrier(0);
            if (j >= 1) {
                const bool new_seg = j == 1 || tt >= cur.te;
                cur.seek(seqlens, tt);
                if (new_seg) zero_acc();
                // rows whose reference maximum moved: bring the sums to the new reference
                if (__builtin_amdgcn_readfirstlane(fl[0] | fl[1] | fl[2] | fl[3])) {
                    if constexpr (C::WIDE) {
#pragma unroll
                        for (int r2 = 0; r2 < 2; ++r2) {
                            const int r4 = 2 * r2 + (g & 1);  // this lane's 16-row block
                            const float al = fl[r4] ? alpha_buf[slot * 64 + 16 * r4 + n] : 1.f;
#pragma unroll
                            for (int cb = 0; cb < C::CB32; ++cb) acw[r2][cb] *= al;
                        }
                    } else {
#pragma unroll
                        for (int r4 = 0; r4 < NA4; ++r4) {
                            if (__builtin_amdgcn_readfirstlane(fl[r4])) {
                                const float al = alpha_buf[slot * 64 + r4 * 16 + n];
#pragma unroll
                                for (int cb = 0; cb < NAC; ++cb) acc[r4][cb] *= al;
                            }
                        }
                    }
                }
                if constexpr (C::WIDE) {
                    // pB[2 * r2 + ks] = B operand of 32-row block r2, k-step ks
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
                } else {
#pragma unroll
                    for (int cb = 0; cb < C::CBV; ++cb) {
                        const bf16x8 a = __builtin_bit_cast(
                            bf16x8, __builtin_shufflevector(vlo[cb], vhi[cb], 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
                        for (int r4 = 0; r4 < 4; ++r4) acc[r4][cb] = mfma16x16x32(a, pB[r4], acc[r4][cb]);
                        if (issued) {
#pragma unroll
                            for (int it = 0; it < C::LPW; ++it)
                                if ((it * C::CBV) / C::LPW == cb) copy_part(j + 2, crsrc, ctbs, it);
                        }
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
                // end of a segment: normalize and write the result or the partial
                if (tt + 1 >= cur.te || j == ntiles) {
                    const int bq = cur.b;
                    const int nseg = cur.ns;
                    const int sl = cur.slot(worker);
                    // normalization of query row rloc (row of the block) and its output place
                    auto row_info = [&](int rloc, float &inv, float &lse2) {
                        const float mr = seg_buf[(slot * 64 + rloc) * 2 + 0];
                        const float ls = seg_buf[(slot * 64 + rloc) * 2 + 1];
                        inv = ls > 0.f ? 1.f / ls : 0.f;
                        lse2 = ls > 0.f ? mr + fast_log2(ls) : -INFINITY;
                    };
                    auto put4 = [&](int row, int col, const f32x4 &v, float inv) {
                        if (nseg == 1) {
                            *(u32x2 *)(out + ((size_t)bq * M + row) * K + col) =
                                u32x2{pack_bf16x2(v[0] * inv, v[1] * inv), pack_bf16x2(v[2] * inv, v[3] * inv)};
                        } else {
                            *(f32x4 *)(part_out + ((size_t)sl * M + row) * K + col) = v * inv;
                        }
                    };
                    auto put_lse = [&](int row, float lse2) {
                        // one writer per row: the wide layout spreads a row block over
                        // lane groups 0 and 1, the narrow one keeps it in group 0
                        if ((C::WIDE ? (g >> 1) : g) != 0 || vw != 0) return;
                        if (nseg == 1)
                            lse[(size_t)bq * M + row] = lse2 * kLn2;
                        else
                            part_lse[(size_t)sl * M + row] = lse2;
                    };
                    if constexpr (C::WIDE) {
#pragma unroll
                        for (int r2 = 0; r2 < 2; ++r2) {
                            // lane l: query row 32*r2 + l%32; value e of block cb is column
                            // 32cb + 8(e/4) + 4(l/32) + e%4 of this wave's columns
                            const int rloc = 32 * r2 + 16 * (g & 1) + n;
                            const int row = rb * C::ROWS + rloc;
                            if (row < M) {
                                float inv, lse2;
                                row_info(rloc, inv, lse2);
                                const int col0 = vw * (K / C::NVW) + 4 * (g >> 1);
#pragma unroll
                                for (int cb = 0; cb < C::CB32; ++cb)
#pragma unroll
                                    for (int qq = 0; qq < 4; ++qq)
                                        put4(row, col0 + 32 * cb + 8 * qq,
                                             f32x4{acw[r2][cb][4 * qq], acw[r2][cb][4 * qq + 1], acw[r2][cb][4 * qq + 2],
                                                   acw[r2][cb][4 * qq + 3]},
                                             inv);
                                put_lse(row, lse2);
                            }
                        }
                    } else {
#pragma unroll
                        for (int r4 = 0; r4 < 4; ++r4) {
                            const int rloc = 16 * r4 + n;
                            const int row = rb * C::ROWS + rloc;
                            if (row < M) {
                                float inv, lse2;
                                row_info(rloc, inv, lse2);
                                const int col0 = vw * (K / C::NVW) + g * 4;
#pragma unroll
                                for (int cb = 0; cb < C::CBV; ++cb) put4(row, col0 + 16 * cb, acc[r4][cb], inv);
                                put_lse(row, lse2);
                            }
                        }
                    }
                    stored = true;
                }
            }
            // tile j+1 (issued a step ago) must be in LDS before the barrier publishes it
            if (copier && j + 1 < ntiles) {
                if (issued && !stored)
                    wait_vmcnt<C::LPW>();
                else
                    wait_vmcnt<0>();
            }
            lds_barrier();
        }
    }
}

}  // namespace da
