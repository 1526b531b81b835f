// Per-head projections on either side of absorbed MLA decode ("MLA Cost
// Analysis & Regime Guide", "Absorption Trick (FlashMLA)": the queries are
// taken into latent space with Wk^T before the attention, and the latent
// output is decompressed with Wv by a separate kernel after it).
//
//   C[m, hd, n] = sum_k A[m, hd, k] * B[hd, n, k]     for every head hd
//
// A: [M, H, K] bf16 (M = b*s query tokens), B: [H, N, K] bf16 (row n of head hd
// holds the length-K vector that output column n contracts with), C: [M, H, N]
// bf16 (round to nearest even), fp32 accumulation.
//   Q-absorption:          A = q_nope [b,s,h,d], B = Wk [h, k, d]  -> C = q_lat [b,s,h,k]
//   output decompression:  A = o_lat [b,s,h,k],  B = Wv^T [h, d, k] -> C = out [b,s,h,d]
//
// A block computes a 64 x BN tile of one head's C. Per stage of 128
// contraction values it copies its A rows (64 x 256 bytes) and B rows (BN x 256
// bytes) HBM -> LDS with 16-byte-per-lane copies (buffer_load ... lds; every
// copy instruction moves four whole 256-byte rows, so every request is a full
// run of two cache lines), two stages in flight. Rows past M or N, and
// contraction values past K, are copied as zeros (an out-of-range offset: no
// memory request). The LDS rows use the chunk swizzle of the grouped decode
// kernel's 256-byte token rows (gqa_swz), whose 16-row fragment reads are the
// ones made here: wave w reads the A fragments of all 64 rows and the B
// fragments of its BN / 4 columns, and issues v_mfma_f32_16x16x32_bf16 with B
// as the first operand (each lane ends with four consecutive columns of a C
// row). The finished tile passes through LDS once more so that every lane
// stores 16 contiguous bytes of a C row. Tiles are numbered in (head, row
// tile, column tile) order and every XCD takes a contiguous eighth of them, so
// the few heads an XCD works on at a time keep their A rows and weights in
// that XCD's L2.
#pragma once

#include "common.hpp"
#include "gqa_kernel.hpp"  // gqa_swz

namespace da {

template <int BN>
struct HeadGemmCfg {
    static constexpr int BM = 64;                // C rows (query tokens) per block
    static constexpr int BK = 128;               // contraction values per stage
    static constexpr int ROWB = BK * 2;          // bytes per LDS row
    static constexpr int A_BYTES = BM * ROWB;
    static constexpr int B_BYTES = BN * ROWB;
    static constexpr int STAGE = A_BYTES + B_BYTES;
    static constexpr int COPIES = STAGE / 1024;  // copy instructions per stage
    static constexpr int CPW = COPIES / 4;       // per wave
    static constexpr int ACOPY = A_BYTES / 1024 / 4;  // the first ACOPY of a wave's copies are A rows
    static constexpr int WC = BN / 4;            // C columns per wave
    static constexpr int NB = WC / 16;           // 16-column blocks per wave
    static constexpr int CROW = BN * 2 + 16;     // bytes per row of the output staging (padding spreads the banks)
    static_assert(BN == 64 || BN == 128, "tile width");
    static_assert(COPIES % 4 == 0 && A_BYTES % 4096 == 0, "copies split evenly over the four waves");
    static_assert(BM * CROW <= STAGE, "the output staging fits one stage buffer");
};

template <int BN>
__global__ void __launch_bounds__(256) head_gemm_lds_kernel(const uint16_t *__restrict__ A,
                                                            const uint16_t *__restrict__ B, uint16_t *__restrict__ C,
                                                            int M, int H, int N, int K, int ntm, int ntn, int tiles)
{
    using G = HeadGemmCfg<BN>;
    extern __shared__ __attribute__((aligned(1024))) char smem[];
    DA_LDS char *lds = (DA_LDS char *)smem;
    // tiles in (head, row tile, column tile) order, a contiguous share per XCD
    const int unit = xcd_linear_unit(blockIdx.x, gridDim.x);
    if (unit >= tiles) return;
    const int hd = unit / (ntm * ntn);
    const int r0 = unit - hd * ntm * ntn;
    const int mt = r0 / ntn;
    const int m0 = mt * G::BM, n0 = (r0 - mt * ntn) * BN;
    const int mrows = min(G::BM, M - m0), ncols = min(BN, N - n0);

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int n = lane & 15;
    const int g = lane >> 4;
    constexpr uint32_t kOut = 0x80000000u;  // an offset past the resources' range: reads zeros
    const u32x4 ra = raw_buffer_rsrc(A + ((size_t)m0 * H + hd) * K, kOut);
    const u32x4 rb = raw_buffer_rsrc(B + ((size_t)hd * N + n0) * K, kOut);
    const int nst = (K + G::BK - 1) / G::BK;

    // stage st into buffer st % 2: wave w issues copy instructions w, w + 4, ...; copy i
    // fills LDS rows 4i .. 4i + 3 (A rows first, then B rows), lane l row 4i + l / 16,
    // LDS chunk l % 16, which holds source chunk (l % 16) ^ gqa_swz(row)
    auto issue = [&](int st) {
        DA_LDS char *buf = lds + (st & 1) * G::STAGE;
        const int k0 = st * G::BK;
#pragma unroll
        for (int it = 0; it < G::CPW; ++it) {
            const int i = it * 4 + w;
            const int row = i * 4 + (lane >> 4);
            const int kc = k0 + 8 * ((lane & 15) ^ gqa_swz(row));
            uint32_t off;
            if (it < G::ACOPY)
                off = row < mrows && kc < K ? (uint32_t)(((size_t)row * H * K + kc) * 2) : kOut;
            else
                off = row - G::BM < ncols && kc < K ? (uint32_t)(((row - G::BM) * K + kc) * 2) : kOut;
            lds_dma16(it < G::ACOPY ? ra : rb, buf + i * 1024, off);
        }
    };

    f32x4 acc[4][G::NB];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < G::NB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int sw = gqa_swz(n);  // = gqa_swz of every row read below (16 i + n, 16 j + n)
    issue(0);
    if (nst > 1) issue(1);
    for (int st = 0; st < nst; ++st) {
        if (st + 1 < nst)
            wait_vmcnt<G::CPW>();  // this wave's copies of stage st have landed (st + 1 may fly)
        else
            wait_vmcnt<0>();
        lds_barrier();  // and every other wave's
        const DA_LDS char *abuf = lds + (st & 1) * G::STAGE;
        const DA_LDS char *bbuf = abuf + G::A_BYTES + w * G::WC * G::ROWB;
        const int nks = min(G::BK, K - st * G::BK) / 32;
#pragma unroll
        for (int kk = 0; kk < G::BK / 32; ++kk) {
            if (kk < nks) {
                const int co = ((kk * 4 + g) ^ sw) << 4;
                bf16x8 a[4], b[G::NB];
#pragma unroll
                for (int i = 0; i < 4; ++i) a[i] = *(const DA_LDS bf16x8 *)(abuf + (16 * i + n) * G::ROWB + co);
#pragma unroll
                for (int j = 0; j < G::NB; ++j) b[j] = *(const DA_LDS bf16x8 *)(bbuf + (16 * j + n) * G::ROWB + co);
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < G::NB; ++j) acc[i][j] = mfma16x16x32(b[j], a[i], acc[i][j]);
            }
        }
        if (st + 2 < nst) {
            lds_barrier();  // every wave is done with buffer st % 2
            issue(st + 2);
        }
    }

    // the tile through LDS: lane (n, g) holds C row 16 i + n, columns 16 j + 4 g .. + 3 of its share
    lds_barrier();
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < G::NB; ++j)
            *(DA_LDS u32x2 *)(lds + (16 * i + n) * G::CROW + (w * G::WC + 16 * j + 4 * g) * 2) =
                u32x2{pack_bf16x2(acc[i][j][0], acc[i][j][1]), pack_bf16x2(acc[i][j][2], acc[i][j][3])};
    lds_barrier();
    constexpr int CH = BN / 8;  // 16-byte chunks per C row of the tile
    const bool vec = (N & 7) == 0;
    for (int idx = tid; idx < mrows * CH; idx += 256) {
        const int r = idx / CH;
        const int col = (idx - r * CH) * 8;
        if (col >= ncols) continue;
        const u32x4 v = *(const DA_LDS u32x4 *)(lds + r * G::CROW + col * 2);
        uint16_t *dst = C + ((size_t)(m0 + r) * H + hd) * N + n0 + col;
        if (vec && col + 8 <= ncols) {
            *(u32x4 *)dst = v;
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (col + e < ncols) dst[e] = (uint16_t)(v[e >> 1] >> (16 * (e & 1)));
        }
    }
}

}  // namespace da
