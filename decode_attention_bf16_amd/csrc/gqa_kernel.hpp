// Grouped-query decode kernels for gfx950 (MHA / GQA / MQA).
//
// The query heads of a sequence form contiguous groups of g = hq/hkv heads and
// every group reads one K/V head ("Why MLA and MTP Fight Each Other",
// introduction table: arithmetic intensity hq/hkv; "MHA vs GQA 70B", section 1:
// 64 query heads over 8 KV heads). With s draft tokens a KV head serves
// R = g*s query rows. Decode reads each cached K/V row once and does only
// 4*R*d FLOPs on it, so the kernel is bound by HBM bandwidth: the design goal
// is to keep 16-byte loads in flight and the per-byte ALU work small.
//
// VALU kernel (R <= 16): one wave per (KV head, segment). Lanes are split into
// NSLOT token slots of D/8 lanes; lane (dg, slot) holds dims 8*dg..8*dg+7 of
// one token per step (a 16-byte load of K and one of V). Scores: 4 bf16 dot2
// per row, then a mirror-butterfly DPP sum over the D/8 lanes of the slot.
// Each slot runs its own online softmax (no cross-slot traffic per step); the
// slots are merged once at the end of the segment. Values: bf16 dot2 over
// pairs of tokens (probabilities rounded to bf16, as an MFMA path would).
#pragma once

#include "common.hpp"
#include "plan.hpp"

namespace da {

constexpr int kGqaTile = 64;  // planner tile (tokens) for GQA

template <int D, int R>
struct GqaValuCfg {
    static_assert(D == 64 || D == 128 || D == 256, "head dim");
    static constexpr int LPT = D / 8;       // lanes per token
    static constexpr int NSLOT = 64 / LPT;  // token slots per wave
    static constexpr int U = 4;             // tokens per slot per step (even)
    static constexpr int STEP = NSLOT * U;  // tokens per wave step
    static_assert(kGqaTile % STEP == 0, "tile multiple of step");
};

template <int D, int R>
__global__ void __launch_bounds__(256)
    gqa_valu_kernel(const uint16_t *__restrict__ q, const uint16_t *__restrict__ kc,
                    const uint16_t *__restrict__ vc, const int32_t *__restrict__ seqlens, int B, int s, int hq,
                    int hkv, int t_max, float scale_log2, int head_blocks, int units,
                    PlanHeader *__restrict__ hdr, int *__restrict__ tile_start,
                    int *__restrict__ slot_start, uint16_t *__restrict__ out, float *__restrict__ lse,
                    uint16_t *__restrict__ part_out, float *__restrict__ part_lse)
{
    using C = GqaValuCfg<D, R>;
    const int unit = xcd_linear_unit(blockIdx.x, gridDim.x);
    if (unit >= units) return;
    const int worker = unit / head_blocks;
    const int hb = unit - worker * head_blocks;
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int kvh = hb * 4 + wave;
    // the plan as arrays for the combine kernel; every wave derives its own view
    if (unit == 0 && wave == 0) write_plan(seqlens, B, t_max, kGqaTile, units / head_blocks, hdr, tile_start, slot_start);
    if (kvh >= hkv) return;

    PlanWalk cur;
    if (!cur.init(seqlens, B, t_max, kGqaTile, units / head_blocks, worker)) return;
    const int tile_lo = cur.tile_lo;
    const int tile_hi = cur.tile_hi;

    const int dg = lane % C::LPT;
    const int slot = lane / C::LPT;
    const int grp = hq / hkv;
    const int Rr = grp * s;  // real rows of this KV head
    const int M = s * hq;    // query rows per sequence
    const size_t tok_stride = (size_t)hkv * D;

    uint32_t qv[R][4];
    float m[R], l[R], acc[R][8];
    int nvis[R];
    int nvis_min = 0;

    auto row_of = [&](int r) {  // row within the sequence: (draft i, head kvh*grp + j)
        const int i = r / grp;
        const int j = r - i * grp;
        return i * hq + kvh * grp + j;
    };

    auto begin_segment = [&](int bq) {
        const int L = clamp_len(seqlens[bq], t_max);
        int mn = 0x7fffffff;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            u32x4 v = {0u, 0u, 0u, 0u};
            if (r < Rr) {
                v = *(const u32x4 *)(q + ((size_t)bq * M + row_of(r)) * D + dg * 8);
                nvis[r] = L - s + r / grp + 1;
            } else {
                nvis[r] = 0;
            }
            mn = min(mn, r < Rr ? nvis[r] : mn);
            qv[r][0] = v[0];
            qv[r][1] = v[1];
            qv[r][2] = v[2];
            qv[r][3] = v[3];
            m[r] = -INFINITY;
            l[r] = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[r][e] = 0.f;
        }
        nvis_min = mn;
    };

    auto end_segment = [&](int bq, int first_tile_of_seq) {
        // merge the token slots: common reference max per row
#pragma unroll
        for (int r = 0; r < R; ++r) {
            float mm = m[r];
            for (int off = C::LPT; off < 64; off <<= 1) mm = fmaxf(mm, __shfl_xor(mm, off));
            const float f = mm == -INFINITY ? 0.f : fast_exp2(m[r] - mm);
            float lr = l[r] * f;
            for (int off = C::LPT; off < 64; off <<= 1) lr += __shfl_xor(lr, off);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float a = acc[r][e] * f;
                for (int off = C::LPT; off < 64; off <<= 1) a += __shfl_xor(a, off);
                acc[r][e] = a;
            }
            m[r] = mm;
            l[r] = lr;
        }
        if (slot != 0) return;
        const int nseg = cur.ns;
        const bool direct = nseg == 1;
        const int sl = cur.slot(worker);
#pragma unroll
        for (int r = 0; r < R; ++r) {
            if (r >= Rr) continue;
            const int row = row_of(r);
            const float inv = l[r] > 0.f ? 1.f / l[r] : 0.f;
            const float lse2 = l[r] > 0.f ? m[r] + fast_log2(l[r]) : -INFINITY;
            // the result, or this segment's bf16 partial for the combine
            u32x4 v;
            v[0] = pack_bf16x2(acc[r][0] * inv, acc[r][1] * inv);
            v[1] = pack_bf16x2(acc[r][2] * inv, acc[r][3] * inv);
            v[2] = pack_bf16x2(acc[r][4] * inv, acc[r][5] * inv);
            v[3] = pack_bf16x2(acc[r][6] * inv, acc[r][7] * inv);
            if (direct) {
                *(u32x4 *)(out + ((size_t)bq * M + row) * D + dg * 8) = v;
                if (dg == 0) lse[(size_t)bq * M + row] = lse2 * kLn2;
            } else {
                *(u32x4 *)(part_out + ((size_t)sl * M + row) * D + dg * 8) = v;
                if (dg == 0) part_lse[(size_t)sl * M + row] = lse2;
            }
        }
    };

    int bcur = cur.b;
    int ts_cur = cur.ts;
    int te_cur = cur.te;
    int L = clamp_len(seqlens[bcur], t_max);
    begin_segment(bcur);

    for (int tt = tile_lo; tt < tile_hi; ++tt) {
        if (tt >= te_cur) {
            end_segment(bcur, ts_cur);
            cur.seek(seqlens, tt);
            bcur = cur.b;
            ts_cur = cur.ts;
            te_cur = cur.te;
            L = clamp_len(seqlens[bcur], t_max);
            begin_segment(bcur);
        }
        const int t_tile = (tt - ts_cur) * kGqaTile;
        const int t_stop = min(L, t_tile + kGqaTile);
        const uint16_t *kb = kc + (size_t)bcur * t_max * tok_stride + (size_t)kvh * D + dg * 8;
        const uint16_t *vb = vc + (size_t)bcur * t_max * tok_stride + (size_t)kvh * D + dg * 8;

        for (int t0 = t_tile; t0 < t_stop; t0 += C::STEP) {
            u32x4 kk[C::U], vv[C::U];
#pragma unroll
            for (int u = 0; u < C::U; ++u) {
                const int tok = t0 + u * C::NSLOT + slot;
                kk[u] = u32x4{0u, 0u, 0u, 0u};
                vv[u] = u32x4{0u, 0u, 0u, 0u};
                if (tok < t_stop) {
                    kk[u] = *(const u32x4 *)(kb + (size_t)tok * tok_stride);
                    vv[u] = *(const u32x4 *)(vb + (size_t)tok * tok_stride);
                }
            }
            // scores
            float sc[C::U][R];
#pragma unroll
            for (int u = 0; u < C::U; ++u) {
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    float d = 0.f;
                    d = dot2_bf16(qv[r][0], kk[u][0], d);
                    d = dot2_bf16(qv[r][1], kk[u][1], d);
                    d = dot2_bf16(qv[r][2], kk[u][2], d);
                    d = dot2_bf16(qv[r][3], kk[u][3], d);
                    sc[u][r] = group_sum<C::LPT>(d);
                }
            }
            // mask: tokens past a row's visible end (and past the tile end)
            if (t0 + C::STEP > nvis_min || t0 + C::STEP > t_stop) {
#pragma unroll
                for (int u = 0; u < C::U; ++u) {
                    const int tok = t0 + u * C::NSLOT + slot;
#pragma unroll
                    for (int r = 0; r < R; ++r)
                        if (tok >= t_stop || tok >= nvis[r]) sc[u][r] = -INFINITY;
                }
            }
            // per-slot online softmax
            bool need = false;
            float mt[R];
#pragma unroll
            for (int r = 0; r < R; ++r) {
                float mx = sc[0][r];
#pragma unroll
                for (int u = 1; u < C::U; ++u) mx = fmaxf(mx, sc[u][r]);
                mt[r] = mx * scale_log2;
                need |= mt[r] > m[r] + kRescaleSlack;
            }
            if (__builtin_amdgcn_ballot_w64(need)) {
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const float mn = fmaxf(m[r], mt[r]);
                    const float al = mn == -INFINITY ? 1.f : fast_exp2(m[r] - mn);
                    m[r] = mn;
                    l[r] *= al;
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc[r][e] *= al;
                }
            }
            uint32_t pp[C::U / 2][R];
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const float ms = m[r] == -INFINITY ? 0.f : m[r];
#pragma unroll
                for (int u = 0; u < C::U; u += 2) {
                    const float p0 = fast_exp2(__builtin_fmaf(sc[u][r], scale_log2, -ms));
                    const float p1 = fast_exp2(__builtin_fmaf(sc[u + 1][r], scale_log2, -ms));
                    l[r] += p0 + p1;
                    pp[u / 2][r] = pack_bf16x2(p0, p1);
                }
            }
            // values: pairs of tokens through bf16 dot2
#pragma unroll
            for (int u = 0; u < C::U; u += 2) {
                uint32_t vp[8];
#pragma unroll
                for (int dw = 0; dw < 4; ++dw) {
                    const uint32_t a = vv[u][dw], b2 = vv[u + 1][dw];
                    vp[2 * dw] = (a & 0xffffu) | (b2 << 16);
                    vp[2 * dw + 1] = (a >> 16) | (b2 & 0xffff0000u);
                }
#pragma unroll
                for (int r = 0; r < R; ++r)
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc[r][e] = dot2_bf16(pp[u / 2][r], vp[e], acc[r][e]);
            }
        }
    }
    end_segment(bcur, ts_cur);
}

}  // namespace da

namespace da {

// ----------------------------------------------------------------------------
// MFMA kernel (any R = g*s up to 64, rows padded to blocks of 16).
//
// Block = 512/D... waves (one KV head each); the block streams 16-token stages
// of its heads' K and V rows HBM -> LDS with buffer_load ... lds (a ring of 4
// stages, 3 in flight while one is computed; rows past the sequence length read
// as zeros through the buffer bounds). Per wave and stage:
//   S^T[16 tokens, 16 rows] = K . Q^T   MFMA 16x16x32 bf16, K from LDS, Q in registers
//   softmax (fp32, exp2 domain, lazily moved per-row reference maximum)
//   O^T[d, 16 rows] += V^T . P^T        MFMA 16x16x16 bf16, V^T through the LDS
//                                       transposing read, P^T straight from the
//                                       score registers
// LDS stage layout: 16 K token rows then 16 V token rows of 1 KB (the block's
// heads, d contiguous); 16-byte chunk c of token row t is stored at
// c ^ gqa_swz(t), which keeps the score reads and the transposing reads free of
// bank conflicts on 64 banks.
// Waits until at most `later` * LW copies of this wave are outstanding (`later`
// runs from 0 to MAXL; the counter limit needs constants).
template <int LW, int MAXL>
__device__ __forceinline__ void wait_stage_copies(int later)
{
    if constexpr (MAXL > 0) {
        if (later >= MAXL) {
            wait_vmcnt<MAXL * LW>();
            return;
        }
        wait_stage_copies<LW, MAXL - 1>(later);
    } else {
        wait_vmcnt<0>();
    }
}

// D: width of the query and key rows (the score dot products); DV: width of
// the value and output rows (D unless the keys carry extra columns, as the
// un-absorbed MLA form's decoupled rope part does).
template <int D, int RBLK, int HPB_ = 512 / D, int NST_ = 4, int DV_ = D>
struct GqaMfmaCfg {
    static constexpr int DK = D, DV = DV_;
    static_assert((DK == 64 || DK == 128 || DK == 192 || DK == 256) && (DV == 64 || DV == 128 || DV == 256),
                  "head dims");
    static constexpr int HPB = HPB_;             // KV heads (waves) per block
    static_assert(HPB >= 1 && HPB * DK <= 512 && HPB * DV <= 512, "token rows of the block's heads fit 1 KB");
    static constexpr int THREADS = 64 * HPB;
    static constexpr int T = 16;                 // tokens per stage
    static constexpr int ROWK = HPB * DK * 2;    // bytes of one K token row (HPB heads x DK)
    static constexpr int ROWV = HPB * DV * 2;    // bytes of one V token row
    static_assert(ROWK % 256 == 0 && ROWV % 256 == 0, "token rows are whole 16-chunk swizzle groups");
    static constexpr int KCH = T * ROWK / 16;    // 16-byte chunks of a stage's K rows
    static_assert(KCH % 64 == 0, "the K rows fill whole copy instructions");
    static constexpr int STAGE_BYTES = T * (ROWK + ROWV);
    static constexpr int NST = NST_;             // ring depth (NST - 1 stages in flight)
    static constexpr int LDS_BYTES = NST * STAGE_BYTES;
    static constexpr int LW = STAGE_BYTES / 1024 / HPB;  // copy instructions per wave per stage
    static_assert(LW * HPB * 1024 == STAGE_BYTES, "stage splits into whole copies per wave");
    static_assert((NST - 2) * LW <= 63, "outstanding copies fit the vmcnt counter");
    static constexpr int KS = DK / 32;           // score k-steps
    static constexpr int DB = DV / 16;           // 16-wide output blocks
};

// XOR applied to the chunk index (low four bits) of token row t of a stage. A
// linear map of the token's low four bits (bit 2 ^= bit 0, bit 3 ^= bit 0 ^ bit 1),
// chosen by checking this kernel's access patterns on the CPU: the 16-token
// score reads and the 4-token transposing reads use 64 distinct banks under
// every plausible grouping of the lanes into passes.
__device__ __forceinline__ int gqa_swz(int t)
{
    t &= 15;
    return t ^ ((t & 1) << 2) ^ ((((t >> 1) ^ t) & 1) << 3);
}


template <int D, int RBLK, int HPB, int NST, int DV = D>
__global__ void __launch_bounds__(64 * HPB, 1)
    gqa_mfma_kernel(const uint16_t *__restrict__ q, const uint16_t *__restrict__ kc,
                    const uint16_t *__restrict__ vc, const int32_t *__restrict__ seqlens, int B, int s, int hq,
                    int hkv, int t_max, float scale_log2, int head_blocks, int units,
                    PlanHeader *__restrict__ hdr, int *__restrict__ tile_start,
                    int *__restrict__ slot_start, uint16_t *__restrict__ out, float *__restrict__ lse,
                    uint16_t *__restrict__ part_out, float *__restrict__ part_lse)
{
    using C = GqaMfmaCfg<D, RBLK, HPB, NST, DV>;
    constexpr int SUB = kGqaTile / C::T;  // stages per planner tile
    extern __shared__ __attribute__((aligned(1024))) char smem[];
    DA_LDS char *lds = (DA_LDS char *)smem;

    const int unit = xcd_linear_unit(blockIdx.x, gridDim.x);
    if (unit >= units) return;
    const int worker = unit / head_blocks;
    const int hb = unit - worker * head_blocks;
    // the plan as arrays for the combine kernel; every wave derives its own view
    if (unit == 0 && threadIdx.x < 64)
        write_plan(seqlens, B, t_max, kGqaTile, units / head_blocks, hdr, tile_start, slot_start);
    PlanWalk cur;
    if (!cur.init(seqlens, B, t_max, kGqaTile, units / head_blocks, worker)) return;
    const int tile_lo = cur.tile_lo;
    const int tile_hi = cur.tile_hi;
    const int nst = (tile_hi - tile_lo) * SUB;

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int n = lane & 15;
    const int g = lane >> 4;
    const int kvh = hb * C::HPB + w;
    const bool active = kvh < hkv;
    const int grp = hq / hkv;
    const int R = grp * s;       // query rows of this KV head
    const int M = s * hq;        // query rows per sequence
    const int tok_k = hkv * D;   // elements of one token's K row (all KV heads)
    const int tok_v = hkv * DV;  // ... and V row

    // ---- per-lane LDS offsets (stage: T K token rows, then T V token rows)
    const int qk_base = n * C::ROWK;  // + ((chunk ^ gsw(n)) << 4)
    const int sq = gqa_swz(n);
    const int tr_tok = 4 * g + (n >> 2);
    const int st = gqa_swz(tr_tok);
    const int hsel = (n & 3) >> 1;
    const int tr_base = C::T * C::ROWK + tr_tok * C::ROWV + ((n & 1) << 3);

    // ---- DMA of one stage: 1 KB copies w, w + HPB, ... (the K rows' chunks, then the V rows')
    PlanWalk icur = cur;  // the copies' own cursor, ahead of the compute's
    auto stage_pos = [&](int sg, int &bq, int &tok0) {
        const int tt = tile_lo + sg / SUB;
        icur.seek(seqlens, tt);
        bq = icur.b;
        tok0 = (tt - icur.ts) * kGqaTile + (sg % SUB) * C::T;
    };
    auto issue_stage = [&](int sg) {
        int bq, tok0;
        stage_pos(sg, bq, tok0);
        const int L = clamp_len(seqlens[bq], t_max);
        DA_LDS char *dst = lds + (sg % C::NST) * C::STAGE_BYTES;
#pragma unroll
        for (int i = 0; i < C::LW; ++i) {
            const int cp = w + i * C::HPB;  // wave-uniform copy index
            const int p = cp * 64 + lane;   // 16-byte chunk of the stage
            const bool is_k = cp * 64 < C::KCH;
            const int rch = is_k ? C::ROWK / 16 : C::ROWV / 16;  // chunks per token row
            const int q = is_k ? p : p - C::KCH;
            const int tk = q / rch;                             // token row of the stage
            const int c = (q - tk * rch) ^ gqa_swz(tk);         // logical chunk in that row
            const int te = is_k ? tok_k : tok_v;
            const uint16_t *base = (is_k ? kc : vc) + (size_t)bq * t_max * te;
            const u32x4 rsrc = raw_buffer_rsrc(base, (uint32_t)(L * te * 2));
            const uint32_t off = (uint32_t)(((tok0 + tk) * te + hb * C::HPB * (is_k ? D : DV)) * 2 + c * 16);
            // each K/V byte is read by this wave's block only: a streaming copy
            lds_dma16_stream(rsrc, dst + cp * 1024, off);
        }
    };

    bf16x8 qB[RBLK][C::KS];
    f32x4 acc[RBLK][C::DB];
    float mref[RBLK], lsum[RBLK];
    int nvis[RBLK];
    int nvis_min = 0;

    auto row_of = [&](int r) {
        const int i = r / grp;
        const int j = r - i * grp;
        return i * hq + kvh * grp + j;
    };
    auto begin_segment = [&](int bq) {
        const int L = clamp_len(seqlens[bq], t_max);
        int mn = 0x7fffffff;
#pragma unroll
        for (int rb = 0; rb < RBLK; ++rb) {
            const int r = rb * 16 + n;
            const bool ok = active && r < R;
            nvis[rb] = ok ? L - s + r / grp + 1 : 0;
            mn = min(mn, nvis[rb]);
#pragma unroll
            for (int kk = 0; kk < C::KS; ++kk) {
                u32x4 v = {0u, 0u, 0u, 0u};
                if (ok) v = *(const u32x4 *)(q + ((size_t)bq * M + row_of(r)) * D + kk * 32 + g * 8);
                qB[rb][kk] = as_bf16x8(v);
            }
            mref[rb] = -INFINITY;
            lsum[rb] = 0.f;
#pragma unroll
            for (int db = 0; db < C::DB; ++db) acc[rb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        for (int off = 1; off < 64; off <<= 1) mn = min(mn, __shfl_xor(mn, off));
        nvis_min = mn;
        wait_vm_loads_visible();
    };
    auto end_segment = [&](int bq, int first_tile_of_seq) {
        if (!active) return;
        const int nseg = cur.ns;
        const int sl = cur.slot(worker);
#pragma unroll
        for (int rb = 0; rb < RBLK; ++rb) {
            const int r = rb * 16 + n;
            if (r >= R) continue;
            const int row = row_of(r);
            const float inv = lsum[rb] > 0.f ? 1.f / lsum[rb] : 0.f;
            const float lse2 = lsum[rb] > 0.f ? mref[rb] + fast_log2(lsum[rb]) : -INFINITY;
            // the result, or this segment's bf16 partial for the combine
            uint16_t *o = nseg == 1 ? out + ((size_t)bq * M + row) * DV + g * 4
                                    : part_out + ((size_t)sl * M + row) * DV + g * 4;
#pragma unroll
            for (int db = 0; db < C::DB; ++db) {
                u32x2 v;
                v[0] = pack_bf16x2(acc[rb][db][0] * inv, acc[rb][db][1] * inv);
                v[1] = pack_bf16x2(acc[rb][db][2] * inv, acc[rb][db][3] * inv);
                *(u32x2 *)(o + db * 16) = v;
            }
            if (g == 0) {
                if (nseg == 1)
                    lse[(size_t)bq * M + row] = lse2 * kLn2;
                else
                    part_lse[(size_t)sl * M + row] = lse2;
            }
        }
    };

    // ---- prologue (queries first: their wait then drains nothing else)
    int bcur = cur.b;
    int ts_cur = cur.ts;
    int te_cur = cur.te;
    int L = clamp_len(seqlens[bcur], t_max);
    begin_segment(bcur);
    for (int sg = 0; sg < min(C::NST - 1, nst); ++sg) issue_stage(sg);

    for (int sg = 0; sg < nst; ++sg) {
        const int tt = tile_lo + sg / SUB;
        if (tt >= te_cur) {  // first stage of a new sequence (stage sg % SUB == 0)
            end_segment(bcur, ts_cur);
            cur.seek(seqlens, tt);
            bcur = cur.b;
            ts_cur = cur.ts;
            te_cur = cur.te;
            L = clamp_len(seqlens[bcur], t_max);
            begin_segment(bcur);
        }
        // wait for this stage's copies (the later stages issued so far may stay in flight)
        wait_stage_copies<C::LW, C::NST - 2>(min(C::NST - 2, nst - 1 - sg));
        lds_barrier();
        if (sg + C::NST - 1 < nst) issue_stage(sg + C::NST - 1);

        const int tok0 = (tt - ts_cur) * kGqaTile + (sg % SUB) * C::T;
        if (!active || tok0 >= L) continue;
        const DA_LDS char *stg = lds + (sg % C::NST) * C::STAGE_BYTES;

        // scores
        f32x4 S[RBLK];
#pragma unroll
        for (int rb = 0; rb < RBLK; ++rb) S[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < C::KS; ++kk) {
            const int c = w * (D / 8) + kk * 4 + g;
            const bf16x8 a = *(const DA_LDS bf16x8 *)(stg + qk_base + ((c ^ sq) << 4));
#pragma unroll
            for (int rb = 0; rb < RBLK; ++rb) S[rb] = mfma16x16x32(a, qB[rb][kk], S[rb]);
        }
        // mask, online softmax, probabilities
        i16x4 pB[RBLK];
#pragma unroll
        for (int rb = 0; rb < RBLK; ++rb) {
            if (tok0 + C::T > nvis_min) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (tok0 + g * 4 + i >= nvis[rb]) S[rb][i] = -INFINITY;
            }
            float m = fmaxf(fmaxf(S[rb][0], S[rb][1]), fmaxf(S[rb][2], S[rb][3]));
            const float mt = wave_max_across_groups16(m) * scale_log2;
            if (__builtin_amdgcn_ballot_w64(mt > mref[rb] + kRescaleSlack)) {
                const float mnew = fmaxf(mref[rb], mt);
                const float alpha = mnew == -INFINITY ? 1.f : fast_exp2(mref[rb] - mnew);
                mref[rb] = mnew;
                lsum[rb] *= alpha;
#pragma unroll
                for (int db = 0; db < C::DB; ++db) acc[rb][db] *= alpha;
            }
            const float ms = mref[rb] == -INFINITY ? 0.f : mref[rb];
            float p[4], part = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                p[i] = fast_exp2(__builtin_fmaf(S[rb][i], scale_log2, -ms));
                part += p[i];
            }
            lsum[rb] += wave_sum_across_groups16(part);
            const u32x2 pk = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])};
            pB[rb] = __builtin_bit_cast(i16x4, pk);
        }
        // values
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
            const int c = w * (DV / 8) + 2 * db + hsel;
            const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (DA_LDS i16x4 *)(stg + tr_base + ((c ^ st) << 4)));
#pragma unroll
            for (int rb = 0; rb < RBLK; ++rb)
                acc[rb][db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, pB[rb], acc[rb][db], 0, 0, 0);
        }
    }
    end_segment(bcur, ts_cur);
}

}  // namespace da
