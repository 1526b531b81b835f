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
//   block (512 threads, 8 waves, 2 per SIMD) = one worker of the split-KV plan
//   x one block of 64 query rows. Wave w = (r, c): rows 16r..16r+15, half c.
//     scores S^T[32 tokens of half c, 16 rows] = tile . Q^T, MFMA 16x16x32
//       bf16, A = cache tile from LDS (ds_read_b128), B = the 16 rows' queries
//       held in registers;
//     softmax in fp32 (exp2 domain) against a reference maximum shared by the
//       two waves of a row group; each wave exponentiates its own 32 tokens and
//       the pair swaps the bf16 probabilities (and partial sums) through LDS;
//     values O^T[k/2 columns of half c, 16 rows] += V^T . P^T over all 64
//       tokens, A = latent columns of the same LDS tile through the
//       transposing LDS read (ds_read_b64_tr_b16), B = probabilities (the score
//       MFMA's output layout is the value MFMA's B layout).
//   The shared reference maximum only moves when a score exceeds it by more
//   than kPairSlack powers of two (in practice: the first tile of a segment).
//   Each wave computes its probabilities optimistically against the current
//   reference; when either wave of the pair sees a score past the slack, both
//   take the repair path (swap maxima, rescale, recompute). Every wave reads all
//   eight flags, so the repair round's extra barrier is taken by the whole
//   block or by none of it.
//
// Tile pipeline: 64-token tiles, two LDS buffers. Tile i+1 is copied HBM -> LDS
// with buffer_load ... lds (16 bytes per lane, no registers) while tile i is
// computed. The buffer resource covers the sequence's valid rows only, so rows
// past the sequence length (and padding columns) read as zeros whatever the
// cache holds there.
//
// LDS tile layout: row r (token) holds ROW_CHUNKS 16-byte chunks; logical chunk
// c is stored at chunk c ^ sw(r) (see tile_swz), which keeps the 16-row score
// reads and the 4-row transposing reads free of bank conflicts on 64 banks.
#pragma once

#include "common.hpp"
#include "plan.hpp"

namespace da {

constexpr float kPairSlack = 16.0f;

template <int K, int P>
struct MlaCfg {
    static_assert(K % 64 == 0 && P % 8 == 0, "latent width multiple of 64, rope width multiple of 8");
    static constexpr int KP = K + P;
    static constexpr int KSTEPS = (KP + 31) / 32;               // 32-wide MFMA k-steps
    static constexpr int SRC_CHUNKS = KP / 8;                   // 16-byte chunks per cache row in HBM
    static constexpr int ROW_CHUNKS = (KSTEPS * 4 + 7) / 8 * 8; // chunks per LDS row (multiple of 8)
    static constexpr int ROW_BYTES = ROW_CHUNKS * 16;
    static constexpr int T = 64;                                // tokens per tile
    static constexpr int TILE_BYTES = T * ROW_BYTES;
    static constexpr int THREADS = 512;
    static constexpr int LPT = T * ROW_CHUNKS / THREADS;        // 16-byte loads per thread per tile
    static_assert(T * ROW_CHUNKS % THREADS == 0, "tile chunks divisible by block size");
    static constexpr int CB = K / 32;                           // 16-column output blocks per wave (half of K)
    static constexpr int XCHG_STRIDE = 1280;                    // per-wave exchange bytes
    static constexpr int XCHG_OFF = 2 * TILE_BYTES;
    static constexpr int FLAG_OFF = XCHG_OFF + 8 * XCHG_STRIDE;   // 8 ints: per-wave repair flags
    static constexpr int LDS_BYTES = FLAG_OFF + 32;
    static constexpr int ROWS = 64;                             // query rows per block
    static_assert(LDS_BYTES <= 163840, "LDS budget");
    // every LDS read offset below must fit the 16-bit instruction offset
    static_assert((32 + 16) * ROW_BYTES + 128 * ((KSTEPS - 1) / 2) < 65536, "score read offsets");
    static_assert(48 * ROW_BYTES + 128 * ((CB - 1) / 4) < 65536, "value read offsets");
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
__global__ void __launch_bounds__(512, 1)
    mla_decode_kernel(const uint16_t *__restrict__ q_lat, const uint16_t *__restrict__ q_rope,
                      const uint16_t *__restrict__ cache, const int32_t *__restrict__ seqlens, int B, int s,
                      int h, int t_max, float scale_log2, int row_blocks, int units,
                      const PlanHeader *__restrict__ hdr, const int *__restrict__ tile_start,
                      const int *__restrict__ slot_start, uint16_t *__restrict__ out, float *__restrict__ lse,
                      float *__restrict__ part_out, float *__restrict__ part_lse)
{
    using C = MlaCfg<K, P>;
    extern __shared__ __attribute__((aligned(1024))) char smem[];
    DA_LDS char *lds = (DA_LDS char *)smem;

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
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index (uniform)
    const int rg = w >> 1;                                     // row group
    const int hc = w & 1;                                      // token half (scores) / column half (values)
    const int lane = tid & 63;
    const int n = lane & 15;
    const int g = lane >> 4;
    const int M = s * h;                         // query rows per sequence
    const int row = rb * C::ROWS + rg * 16 + n;  // this lane's query row
    const bool row_ok = row < M;

    // ---- per-lane LDS offsets (bytes within a tile buffer)
    const int sq = tile_swz(n);
    const int qk_off0 = (hc * 32 + n) * C::ROW_BYTES + ((g ^ sq) << 4);        // even k-steps
    const int qk_off1 = (hc * 32 + n) * C::ROW_BYTES + (((4 + g) ^ sq) << 4);  // odd k-steps
    const int st = tile_swz(4 * g + (n >> 2));  // swizzle of the transposing reads' rows (same for +16, +32)
    const int hsel = (n & 3) >> 1;
    const int tr_row = (4 * g + (n >> 2)) * C::ROW_BYTES + ((n & 1) << 3);
    int tr_off[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) tr_off[j] = tr_row + (((2 * j + hsel) ^ st) << 4);
    // byte offset of value block cb (16 latent columns of my half) in a tile row
    auto tr_addr = [&](int cb) -> int {
        if constexpr (K % 128 == 0) {
            return tr_off[cb & 3] + 128 * (hc * (K / 128) + (cb >> 2));
        } else {
            const int jj = hc * (K / 32) + cb;  // column block across the full width
            return tr_row + (((2 * (jj & 3) + hsel) ^ st) << 4) + 128 * (jj >> 2);
        }
    };
    DA_LDS char *xme = lds + C::XCHG_OFF + w * C::XCHG_STRIDE;         // my exchange slot
    DA_LDS char *xpa = lds + C::XCHG_OFF + (w ^ 1) * C::XCHG_STRIDE;   // partner's

    // ---- HBM -> LDS tile copy (per wave: LPT instructions of 64 x 16 bytes)
    auto src_off = [&](int it) -> uint32_t {
        const int pch = (it * 8 + w) * 64 + lane;  // physical chunk in the tile
        const int r = pch / C::ROW_CHUNKS;
        const int c = (pch - r * C::ROW_CHUNKS) ^ tile_swz(r);
        return c < C::SRC_CHUNKS ? (uint32_t)((r * C::KP + c * 8) * 2) : 0x80000000u;
    };
    auto issue_tile = [&](int bq, int jt, int buf) {
        const int L = clamp_len(seqlens[bq], t_max);
        __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(cache + (size_t)bq * t_max * C::KP), (short)0, L * C::KP * 2, 0x00020000);
        const uint32_t tile_bytes_in_seq = (uint32_t)jt * C::T * C::KP * 2;
#pragma unroll
        for (int it = 0; it < C::LPT; ++it) {
            uint32_t off = src_off(it);
            off = off >= 0x80000000u ? off : off + tile_bytes_in_seq;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rsrc, (DA_LDS void *)(lds + buf * C::TILE_BYTES + (it * 8 + w) * 1024), 16, (int)off, 0, 0, 0);
        }
    };

    // ---- per-segment state
    bf16x8 qB[C::KSTEPS];
    f32x4 acc[C::CB];
    float mref = -INFINITY, lsum = 0.f;
    int nvis = 0, nvis_min = 0;

    auto begin_segment = [&](int bq) {
        const int L = clamp_len(seqlens[bq], t_max);
        nvis = row_ok ? (L - s + row / h + 1) : 0;
#pragma unroll
        for (int kk = 0; kk < C::KSTEPS; ++kk) {
            u32x4 v = {0u, 0u, 0u, 0u};
            const int e0 = kk * 32 + g * 8;
            if (row_ok) {
                if (e0 < K)
                    v = *(const u32x4 *)(q_lat + ((size_t)bq * M + row) * K + e0);
                else if (e0 - K < P)
                    v = *(const u32x4 *)(q_rope + ((size_t)bq * M + row) * P + (e0 - K));
            }
            qB[kk] = as_bf16x8(v);
        }
        mref = -INFINITY;
        lsum = 0.f;
#pragma unroll
        for (int cb = 0; cb < C::CB; ++cb) acc[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
        int mn = nvis;
        for (int off = 1; off < 64; off <<= 1) mn = min(mn, __shfl_xor(mn, off));
        nvis_min = mn;
    };

    auto end_segment = [&](int bq, int first_tile_of_seq) {
        if (!row_ok) return;
        const int nseg = slot_start[bq + 1] - slot_start[bq];
        const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
        const float lse2 = lsum > 0.f ? mref + fast_log2(lsum) : -INFINITY;
        const int col0 = hc * (K / 2) + g * 4;
        if (nseg == 1) {
            uint16_t *o = out + ((size_t)bq * M + row) * K + col0;
#pragma unroll
            for (int cb = 0; cb < C::CB; ++cb) {
                u32x2 v;
                v[0] = pack_bf16x2(acc[cb][0] * inv, acc[cb][1] * inv);
                v[1] = pack_bf16x2(acc[cb][2] * inv, acc[cb][3] * inv);
                *(u32x2 *)(o + cb * 16) = v;
            }
            if (g == 0 && hc == 0) lse[(size_t)bq * M + row] = lse2 * kLn2;
        } else {
            const int slot = slot_start[bq] + (worker - first_tile_of_seq / per);
            float *o = part_out + ((size_t)slot * M + row) * K + col0;
#pragma unroll
            for (int cb = 0; cb < C::CB; ++cb) *(f32x4 *)(o + cb * 16) = acc[cb] * inv;
            if (g == 0 && hc == 0) part_lse[(size_t)slot * M + row] = lse2;
        }
    };

    // exp of my 32 tokens against reference `mr`; returns the packed B operand
    // for my k-step of the value product and my partial row sum.
    auto probs = [&](const f32x4 (&S)[2], float mr, float &part) -> u32x4 {
        const float ms = mr == -INFINITY ? 0.f : mr;
        part = 0.f;
        uint32_t pk[4];
#pragma unroll
        for (int bt = 0; bt < 2; ++bt) {
            float p[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                p[i] = fast_exp2(__builtin_fmaf(S[bt][i], scale_log2, -ms));
                part += p[i];
            }
            pk[2 * bt] = pack_bf16x2(p[0], p[1]);
            pk[2 * bt + 1] = pack_bf16x2(p[2], p[3]);
        }
        return u32x4{pk[0], pk[1], pk[2], pk[3]};
    };

    int bcur = find_sequence(tile_start, B, tile_lo);
    int ts_cur = tile_start[bcur];
    int te_cur = tile_start[bcur + 1];

    // ---- prologue: first tile
    issue_tile(bcur, tile_lo - ts_cur, 0);
    begin_segment(bcur);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    lds_barrier();

    for (int tt = tile_lo; tt < tile_hi; ++tt) {
        const int cbuf = (tt - tile_lo) & 1;
        const DA_LDS char *cur = lds + cbuf * C::TILE_BYTES;
        const int jt = tt - ts_cur;

        // copy the next tile of this worker into the other buffer
        const bool has_next = tt + 1 < tile_hi;
        int bnext = bcur;
        if (has_next) {
            if (tt + 1 >= te_cur) bnext = find_sequence(tile_start, B, tt + 1);
            issue_tile(bnext, tt + 1 - tile_start[bnext], cbuf ^ 1);
        }

        // ---- scores S^T[32 tokens of my half, 16 rows]
        f32x4 S[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
        {
            bf16x8 a0 = *(const DA_LDS bf16x8 *)(cur + qk_off0);
            bf16x8 a1 = *(const DA_LDS bf16x8 *)(cur + qk_off0 + 16 * C::ROW_BYTES);
#pragma unroll
            for (int kk = 0; kk < C::KSTEPS; ++kk) {
                bf16x8 b0 = a0, b1 = a1;
                if (kk + 1 < C::KSTEPS) {
                    const DA_LDS char *nb = cur + (((kk + 1) & 1) ? qk_off1 : qk_off0) + 128 * ((kk + 1) >> 1);
                    a0 = *(const DA_LDS bf16x8 *)(nb);
                    a1 = *(const DA_LDS bf16x8 *)(nb + 16 * C::ROW_BYTES);
                }
                S[0] = mfma16x16x32(b0, qB[kk], S[0]);
                S[1] = mfma16x16x32(b1, qB[kk], S[1]);
            }
        }

        // ---- draft / length mask (only tiles reaching past some row's visible end)
        const int tok0 = jt * C::T + hc * 32;
        if (jt * C::T + C::T > nvis_min) {
#pragma unroll
            for (int bt = 0; bt < 2; ++bt)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (tok0 + bt * 16 + g * 4 + i >= nvis) S[bt][i] = -INFINITY;
        }

        // ---- softmax against the pair's shared reference
        float m = -INFINITY;
#pragma unroll
        for (int bt = 0; bt < 2; ++bt)
#pragma unroll
            for (int i = 0; i < 4; ++i) m = fmaxf(m, S[bt][i]);
        const float mloc = wave_max_across_groups16(m) * scale_log2;
        const int need = __builtin_amdgcn_ballot_w64(mloc > mref + kPairSlack) != 0;
        float part;
        u32x4 pown = probs(S, mref, part);
        part = wave_sum_across_groups16(part);
        *(DA_LDS u32x4 *)(xme + lane * 16) = pown;
        if (g == 0) {
            *(DA_LDS float *)(xme + 1024 + n * 4) = part;
            *(DA_LDS float *)(xme + 1088 + n * 4) = mloc;
        }
        if (lane == 0) *(DA_LDS int *)(lds + C::FLAG_OFF + w * 4) = need;
        lds_barrier();
        // s_barrier is block-wide: the repair round (one more barrier) is taken
        // by every wave whenever any wave asks for it; only the pairs that asked
        // change anything.
        const u32x4 fl0 = *(const DA_LDS u32x4 *)(lds + C::FLAG_OFF);
        const u32x4 fl1 = *(const DA_LDS u32x4 *)(lds + C::FLAG_OFF + 16);
        const uint32_t any_need = fl0[0] | fl0[1] | fl0[2] | fl0[3] | fl1[0] | fl1[1] | fl1[2] | fl1[3];
        if (any_need) {
            const int need_pair = need | *(const DA_LDS int *)(lds + C::FLAG_OFF + (w ^ 1) * 4);
            if (need_pair) {
                // agree on a new reference, rescale, recompute, swap again
                const float mnew = fmaxf(mref, fmaxf(mloc, *(const DA_LDS float *)(xpa + 1088 + n * 4)));
                const float alpha = mnew == -INFINITY ? 1.f : fast_exp2(mref - mnew);
                mref = mnew;
                lsum *= alpha;
#pragma unroll
                for (int cb = 0; cb < C::CB; ++cb) acc[cb] *= alpha;
                pown = probs(S, mref, part);
                part = wave_sum_across_groups16(part);
                // the partner reads only my maximum (untouched here) before the next barrier
                *(DA_LDS u32x4 *)(xme + lane * 16) = pown;
                if (g == 0) *(DA_LDS float *)(xme + 1024 + n * 4) = part;
            }
            lds_barrier();
        }
        const u32x4 ppar = *(const DA_LDS u32x4 *)(xpa + lane * 16);
        lsum += part + *(const DA_LDS float *)(xpa + 1024 + n * 4);
        // B operands for the two 32-token k-steps: mine is k-step hc (selected
        // per dword: a dynamic index into a register array would go through
        // element-wise selects)
        bf16x8 pB[2];
        {
            const bool h1 = hc != 0;
            u32x4 k0, k1;
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                k0[d] = h1 ? ppar[d] : pown[d];
                k1[d] = h1 ? pown[d] : ppar[d];
            }
            pB[0] = as_bf16x8(k0);
            pB[1] = as_bf16x8(k1);
        }

        // ---- O^T[k/2 columns of my half, 16 rows] += V^T . P^T over the 64 tokens
        typedef __attribute__((__vector_size__(8 * sizeof(short)))) short i16x8;
#pragma unroll
        for (int cb = 0; cb < C::CB; ++cb) {
            const DA_LDS char *vb = cur + tr_addr(cb);
#pragma unroll
            for (int tau = 0; tau < 2; ++tau) {
                const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((DA_LDS i16x4 *)(vb + tau * 32 * C::ROW_BYTES));
                const i16x4 hi =
                    __builtin_amdgcn_ds_read_tr16_b64_v4i16((DA_LDS i16x4 *)(vb + (tau * 32 + 16) * C::ROW_BYTES));
                const i16x8 cat = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                acc[cb] = mfma16x16x32(__builtin_bit_cast(bf16x8, cat), pB[tau], acc[cb]);
            }
        }

        // ---- next tile landed in LDS; everybody is done with this one and the exchange slots
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        lds_barrier();

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
