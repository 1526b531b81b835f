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
// Work decomposition
//   block (256 threads, 4 waves) = one worker of the split-KV plan x one block
//   of 64 query rows. The worker walks its run of 64-token tiles; each tile is
//   copied HBM -> LDS once (16-byte loads, prefetched one tile ahead into
//   registers, double-buffered LDS) and is read from LDS by all four waves for
//   both contractions.
//   wave w: row half rh = w/2 (32 rows), column half ch = w%2.
//     scores: S^T[64 tokens, 32 rows] over the k-steps of latent half ch
//       (MFMA 16x16x32 bf16, A = cache tile from LDS, B = queries in
//       registers); the two waves of a row half swap their partial scores
//       through LDS so both hold the full scores.
//     softmax: fp32, exp2 domain, lazy rescale of the running maximum.
//     values: O^T[k/2 columns of half ch, 32 rows] += V^T . P^T, A = latent
//       columns read from the same LDS tile with the transposing LDS read
//       (ds_read_b64_tr_b16), B = probabilities straight from the score
//       registers (the score MFMA's output layout is the value MFMA's B layout).
//
// LDS tile layout: row r (token) holds ROW_CHUNKS 16-byte chunks; logical chunk
// c is stored at chunk c ^ sw(r), sw(r) = 2*(r%4) + (r/4)%2, which keeps the
// 8-row score reads and the 4-row transposing reads free of bank conflicts.
#pragma once

#include "common.hpp"
#include "plan.hpp"

namespace da {

template <int K, int P>
struct MlaCfg {
    static_assert(K % 32 == 0 && P % 8 == 0, "latent width multiple of 32, rope width multiple of 8");
    static constexpr int KP = K + P;
    static constexpr int KSTEPS = (KP + 31) / 32;               // 32-wide MFMA k-steps
    static constexpr int SRC_CHUNKS = KP / 8;                   // 16-byte chunks per cache row in HBM
    static constexpr int ROW_CHUNKS = (KSTEPS * 4 + 7) / 8 * 8; // chunks per LDS row (multiple of 8)
    static constexpr int ROW_BYTES = ROW_CHUNKS * 16;
    static constexpr int T = 64;                                // tokens per tile
    static constexpr int TILE_BYTES = T * ROW_BYTES;
    static constexpr int LPT = T * ROW_CHUNKS / 256;            // 16-byte loads per thread per tile
    static_assert(T * ROW_CHUNKS % 256 == 0, "tile chunks divisible by block size");
    static constexpr int KS0 = (KSTEPS + 1) / 2;                // k-steps of column half 0
    static constexpr int KS1 = KSTEPS - KS0;                    // k-steps of column half 1
    static constexpr int COLS_HALF = K / 2;                     // output columns per wave
    static constexpr int CB = COLS_HALF / 16;                   // 16-column MFMA blocks per wave
    // Partial-score exchange: 8 float4 per lane per wave. It lives inside the
    // idle tile buffer when every wave writes at least 8 KB of each tile
    // (LPT >= 8), else in a dedicated area.
    static constexpr bool XCHG_IN_TILE = LPT >= 8;
    static constexpr int XCHG_BYTES = XCHG_IN_TILE ? 0 : 8 * 4096;
    static constexpr int LDS_BYTES = 2 * TILE_BYTES + XCHG_BYTES;
    static constexpr int ROWS = 64;                              // query rows per block
};

__device__ __forceinline__ int tile_swz(int r) { return ((r & 3) << 1) | ((r >> 2) & 1); }

template <int K, int P>
__global__ void __launch_bounds__(256, 1)
    mla_decode_kernel(const uint16_t *__restrict__ q_lat, const uint16_t *__restrict__ q_rope,
                      const uint16_t *__restrict__ cache, const int32_t *__restrict__ seqlens, int B, int s,
                      int h, int t_max, float scale_log2, int row_blocks, int units,
                      const PlanHeader *__restrict__ hdr, const int *__restrict__ tile_start,
                      const int *__restrict__ slot_start, uint16_t *__restrict__ out, float *__restrict__ lse,
                      float *__restrict__ part_out, float *__restrict__ part_lse)
{
    using C = MlaCfg<K, P>;
    extern __shared__ __attribute__((aligned(1024))) char smem[];

    const int unit = xcd_linear_unit(blockIdx.x, gridDim.x);
    if (unit >= units) return;
    const int worker = unit / row_blocks;
    const int rb = unit - worker * row_blocks;

    const int total = hdr->total_tiles;
    const int per = hdr->per;
    const int tile_lo = worker * per;
    if (tile_lo >= total) return;
    const int tile_hi = min(total, tile_lo + per);

    const int tid = threadIdx.x;
    const int w = tid >> 6;
    const int lane = tid & 63;
    const int n = lane & 15;
    const int g = lane >> 4;
    const int rh = w >> 1;
    const int ch = w & 1;
    const int M = s * h;  // query rows per sequence

    char *buf0 = smem;
    char *buf1 = smem + C::TILE_BYTES;
    char *xchg_dedicated = smem + 2 * C::TILE_BYTES;

    // ---------------- tile copy HBM -> registers -> LDS
    u32x4 pre[C::LPT];
    auto load_tile = [&](int bq, int jt) {
        const int L = clamp_len(seqlens[bq], t_max);
        const uint16_t *base = cache + (size_t)bq * t_max * C::KP;
#pragma unroll
        for (int it = 0; it < C::LPT; ++it) {
            const int q = it * 256 + tid;
            const int row = q / C::ROW_CHUNKS;
            const int c = q - row * C::ROW_CHUNKS;
            const int tok = jt * C::T + row;
            u32x4 v = {0u, 0u, 0u, 0u};
            if (tok < L && c < C::SRC_CHUNKS)
                v = *(const u32x4 *)(base + (size_t)tok * C::KP + c * 8);
            pre[it] = v;
        }
    };
    auto store_tile = [&](char *dst) {
#pragma unroll
        for (int it = 0; it < C::LPT; ++it) {
            const int q = it * 256 + tid;
            const int row = q / C::ROW_CHUNKS;
            const int c = q - row * C::ROW_CHUNKS;
            *(u32x4 *)(dst + row * C::ROW_BYTES + ((c ^ tile_swz(row)) << 4)) = pre[it];
        }
    };

    // ---------------- per-segment state
    const int kbeg = ch == 0 ? 0 : C::KS0;
    const int kcnt = ch == 0 ? C::KS0 : C::KS1;
    bf16x8 qB[C::KS0][2];
    f32x4 acc[C::CB][2];
    float mref[2], lsum[2];
    int nvis[2];
    int nvis_min = 0;

    int bcur = find_sequence(tile_start, B, tile_lo);
    int ts_cur = tile_start[bcur];
    int te_cur = tile_start[bcur + 1];

    auto begin_segment = [&](int bq) {
        const int L = clamp_len(seqlens[bq], t_max);
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const int row = rb * C::ROWS + rh * 32 + r * 16 + n;
            const bool valid = row < M;
            nvis[r] = valid ? (L - s + row / h + 1) : 0;
#pragma unroll
            for (int kk = 0; kk < C::KS0; ++kk) {
                u32x4 v = {0u, 0u, 0u, 0u};
                const int e0 = (kbeg + kk) * 32 + g * 8;
                if (valid && kk < kcnt) {
                    if (e0 < K)
                        v = *(const u32x4 *)(q_lat + ((size_t)bq * M + row) * K + e0);
                    else if (e0 - K < P)
                        v = *(const u32x4 *)(q_rope + ((size_t)bq * M + row) * P + (e0 - K));
                }
                qB[kk][r] = as_bf16x8(v);
            }
            mref[r] = -INFINITY;
            lsum[r] = 0.f;
#pragma unroll
            for (int cb = 0; cb < C::CB; ++cb) acc[cb][r] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        // smallest visible count over this wave's 32 rows (uniform)
        int mn = min(nvis[0], nvis[1]);
        for (int off = 1; off < 64; off <<= 1) mn = min(mn, __shfl_xor(mn, off));
        nvis_min = mn;
    };

    auto end_segment = [&](int bq, int first_tile_of_seq) {
        const int nseg = slot_start[bq + 1] - slot_start[bq];
        const bool direct = nseg == 1;
        const int slot = slot_start[bq] + (worker - first_tile_of_seq / per);
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const int row = rb * C::ROWS + rh * 32 + r * 16 + n;
            if (row >= M) continue;
            const float l = lsum[r];
            const float inv = l > 0.f ? 1.f / l : 0.f;
            const float lse2 = l > 0.f ? mref[r] + fast_log2(l) : -INFINITY;
            if (direct) {
                uint16_t *o = out + ((size_t)bq * M + row) * K + ch * C::COLS_HALF + g * 4;
#pragma unroll
                for (int cb = 0; cb < C::CB; ++cb) {
                    u32x2 v;
                    v[0] = pack_bf16x2(acc[cb][r][0] * inv, acc[cb][r][1] * inv);
                    v[1] = pack_bf16x2(acc[cb][r][2] * inv, acc[cb][r][3] * inv);
                    *(u32x2 *)(o + cb * 16) = v;
                }
                if (ch == 0 && g == 0) lse[(size_t)bq * M + row] = lse2 * kLn2;
            } else {
                float *o = part_out + ((size_t)slot * M + row) * K + ch * C::COLS_HALF + g * 4;
#pragma unroll
                for (int cb = 0; cb < C::CB; ++cb) {
                    f32x4 v = acc[cb][r] * inv;
                    *(f32x4 *)(o + cb * 16) = v;
                }
                if (ch == 0 && g == 0) part_lse[(size_t)slot * M + row] = lse2;
            }
        }
    };

    // ---------------- prologue: first tile
    load_tile(bcur, tile_lo - ts_cur);
    store_tile(buf0);
    begin_segment(bcur);
    __syncthreads();

    for (int tt = tile_lo; tt < tile_hi; ++tt) {
        char *cur = ((tt - tile_lo) & 1) ? buf1 : buf0;
        char *nxt = ((tt - tile_lo) & 1) ? buf0 : buf1;
        const int jt = tt - ts_cur;  // tile index within sequence bcur

        // prefetch the next tile of this worker into registers
        const bool has_next = tt + 1 < tile_hi;
        int bnext = bcur;
        if (has_next) {
            if (tt + 1 >= te_cur) bnext = find_sequence(tile_start, B, tt + 1);
            load_tile(bnext, tt + 1 - tile_start[bnext]);
        }

        // ---- partial scores S^T[64 tokens, 32 rows] over this wave's k-steps
        f32x4 S[4][2];
#pragma unroll
        for (int bt = 0; bt < 4; ++bt)
#pragma unroll
            for (int r = 0; r < 2; ++r) S[bt][r] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < C::KS0; ++kk) {
            if (kk < kcnt) {
                const int chunk = (kbeg + kk) * 4 + g;
#pragma unroll
                for (int bt = 0; bt < 4; ++bt) {
                    const int row = bt * 16 + n;
                    const bf16x8 a = *(const bf16x8 *)(cur + row * C::ROW_BYTES + ((chunk ^ tile_swz(row)) << 4));
                    S[bt][0] = mfma16x16x32(a, qB[kk][0], S[bt][0]);
                    S[bt][1] = mfma16x16x32(a, qB[kk][1], S[bt][1]);
                }
            }
        }

        // ---- swap partial scores with the other wave of this row half
        {
            char *xw;  // where my partner will read my partial
            char *xr;  // where I read my partner's partial
            if constexpr (C::XCHG_IN_TILE) {
                xw = nxt + (w ^ 1) * 1024 + lane * 16;
                xr = nxt + w * 1024 + lane * 16;
            } else {
                xw = xchg_dedicated + (w ^ 1) * 1024 + lane * 16;
                xr = xchg_dedicated + w * 1024 + lane * 16;
            }
#pragma unroll
            for (int bt = 0; bt < 4; ++bt)
#pragma unroll
                for (int r = 0; r < 2; ++r) *(f32x4 *)(xw + (bt * 2 + r) * 4096) = S[bt][r];
            __syncthreads();
#pragma unroll
            for (int bt = 0; bt < 4; ++bt)
#pragma unroll
                for (int r = 0; r < 2; ++r) S[bt][r] += *(const f32x4 *)(xr + (bt * 2 + r) * 4096);
        }

        // ---- draft / length mask (only tiles that reach past some row's visible end)
        const int tok0 = jt * C::T;
        if (tok0 + C::T > nvis_min) {
#pragma unroll
            for (int bt = 0; bt < 4; ++bt)
#pragma unroll
                for (int r = 0; r < 2; ++r)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (tok0 + bt * 16 + g * 4 + i >= nvis[r]) S[bt][r][i] = -INFINITY;
        }

        // ---- online softmax (exp2 domain)
        float mt[2];
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            float m = -INFINITY;
#pragma unroll
            for (int bt = 0; bt < 4; ++bt)
#pragma unroll
                for (int i = 0; i < 4; ++i) m = fmaxf(m, S[bt][r][i]);
            mt[r] = wave_max_across_groups16(m) * scale_log2;
        }
        const bool upd = (mt[0] > mref[0] + kRescaleSlack) || (mt[1] > mref[1] + kRescaleSlack);
        if (__builtin_amdgcn_ballot_w64(upd)) {
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                const float mnew = fmaxf(mref[r], mt[r]);
                const float alpha = mnew == -INFINITY ? 1.f : fast_exp2(mref[r] - mnew);
                mref[r] = mnew;
                lsum[r] *= alpha;
#pragma unroll
                for (int cb = 0; cb < C::CB; ++cb) acc[cb][r] *= alpha;
            }
        }
        bf16x8 pB[2][2];
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const float msafe = mref[r] == -INFINITY ? 0.f : mref[r];
            float part = 0.f;
            uint32_t pk[4][2];
#pragma unroll
            for (int bt = 0; bt < 4; ++bt) {
                float p[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    p[i] = fast_exp2(__builtin_fmaf(S[bt][r][i], scale_log2, -msafe));
                    part += p[i];
                }
                pk[bt][0] = pack_bf16x2(p[0], p[1]);
                pk[bt][1] = pack_bf16x2(p[2], p[3]);
            }
            lsum[r] += wave_sum_across_groups16(part);
#pragma unroll
            for (int tau = 0; tau < 2; ++tau) {
                u32x4 v = {pk[2 * tau][0], pk[2 * tau][1], pk[2 * tau + 1][0], pk[2 * tau + 1][1]};
                pB[tau][r] = as_bf16x8(v);
            }
        }

        // ---- O^T += V^T . P^T over the 64 tokens, this wave's column half
#pragma unroll
        for (int cb = 0; cb < C::CB; ++cb) {
            const int col = ch * C::COLS_HALF + cb * 16 + (n & 3) * 4;
            const int cchunk = col >> 3;
            const int cbyte = (col & 7) << 1;
#pragma unroll
            for (int tau = 0; tau < 2; ++tau) {
                const int r0 = tau * 32 + g * 4 + (n >> 2);
                const int r1 = r0 + 16;
                const i16x4 lo = lds_read_tr16(cur + r0 * C::ROW_BYTES + ((cchunk ^ tile_swz(r0)) << 4) + cbyte);
                const i16x4 hi = lds_read_tr16(cur + r1 * C::ROW_BYTES + ((cchunk ^ tile_swz(r1)) << 4) + cbyte);
                typedef __attribute__((__vector_size__(8 * sizeof(short)))) short i16x8;
                const i16x8 cat = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                const bf16x8 a = __builtin_bit_cast(bf16x8, cat);
                acc[cb][0] = mfma16x16x32(a, pB[tau][0], acc[cb][0]);
                acc[cb][1] = mfma16x16x32(a, pB[tau][1], acc[cb][1]);
            }
        }

        // ---- stage the prefetched tile, then the segment bookkeeping
        if (has_next) store_tile(nxt);
        __syncthreads();

        const bool seg_ends = (tt + 1 == tile_hi) || (tt + 1 >= te_cur);
        if (seg_ends) {
            end_segment(bcur, ts_cur);
            if (has_next) {
                bcur = bnext;
                ts_cur = tile_start[bcur];
                te_cur = tile_start[bcur + 1];
                begin_segment(bcur);
            }
        }
    }
}

}  // namespace da
