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
// Each wave computes one 64 x 64 tile of one head's C (16 accumulators of
// 16 x 16): per 32-wide k-step it loads four A fragments (its 64 rows) and
// four B fragments (its 64 columns), 16 bytes per lane each, straight from
// global memory, two k-steps ahead, and issues sixteen v_mfma_f32_16x16x32_bf16
// (B as the MFMA's first operand, so each lane ends with four consecutive
// columns of a C row and writes them as one 8-byte store). The waves walk the
// tiles in (head, row tile, column tile) order, so the four waves of a block
// usually share their A fragments through the L1 cache.
#pragma once

#include "common.hpp"

namespace da {

constexpr int kGemmTile = 64;

// KSPLIT = 1: this wave computes the whole tile. KSPLIT = 4: the block's four
// waves take a quarter of the k-steps each and wave 0 adds the others' sums
// from LDS (red: 3 x 64 x 64 floats) before it writes the tile.
template <int KSPLIT>
__device__ __forceinline__ void head_gemm_tile(const uint16_t *__restrict__ A, const uint16_t *__restrict__ B,
                                               uint16_t *__restrict__ C, int M, int H, int N, int K, int hd, int m0,
                                               int n0, float *red)
{
    const int lane = threadIdx.x & 63;
    const int n = lane & 15;
    const int g = lane >> 4;
    const uint16_t *arow[4], *brow[4];
    bool a_ok[4], b_ok[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int am = m0 + 16 * i + n;
        a_ok[i] = am < M;
        arow[i] = A + ((size_t)(a_ok[i] ? am : 0) * H + hd) * K + 8 * g;
        const int bn = n0 + 16 * i + n;
        b_ok[i] = bn < N;
        brow[i] = B + ((size_t)hd * N + (b_ok[i] ? bn : 0)) * K + 8 * g;
    }
    struct Frag {
        bf16x8 a[4], b[4];
    };
    auto load = [&](int kk, Frag &f) {
        const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f.a[i] = as_bf16x8(a_ok[i] ? *(const u32x4 *)(arow[i] + kk) : z);
            f.b[i] = as_bf16x8(b_ok[i] ? *(const u32x4 *)(brow[i] + kk) : z);
        }
    };
    // acc[i][j]: lane (n, g) holds C row 16i + n of the tile, columns 16j + 4g .. + 3
    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int kall = K / 32;
    const int wv = KSPLIT > 1 ? (int)(threadIdx.x >> 6) : 0;
    const int kb = kall * wv / KSPLIT;        // this wave's k-steps [kb, ke)
    const int ksteps = kall * (wv + 1) / KSPLIT - kb;
    const uint16_t *ab[4], *bb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        ab[i] = arow[i] + kb * 32;
        bb[i] = brow[i] + kb * 32;
        arow[i] = ab[i];
        brow[i] = bb[i];
    }
    Frag f0, f1;
    if (ksteps > 0) load(0, f0);
    if (ksteps > 1) load(32, f1);
    for (int ks = 0; ks < ksteps; ks += 2) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = mfma16x16x32(f0.b[j], f0.a[i], acc[i][j]);
        if (ks + 2 < ksteps) load((ks + 2) * 32, f0);
        if (ks + 1 < ksteps) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = mfma16x16x32(f1.b[j], f1.a[i], acc[i][j]);
            if (ks + 3 < ksteps) load((ks + 3) * 32, f1);
        }
    }
    if constexpr (KSPLIT > 1) {
        if (wv > 0) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int e = 0; e < 4; ++e) red[(((wv - 1) * 16 + i * 4 + j) * 4 + e) * 64 + lane] = acc[i][j][e];
        }
        __syncthreads();
        if (wv == 0) {
#pragma unroll
            for (int w2 = 0; w2 < KSPLIT - 1; ++w2)
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
#pragma unroll
                        for (int e = 0; e < 4; ++e) acc[i][j][e] += red[((w2 * 16 + i * 4 + j) * 4 + e) * 64 + lane];
        }
        __syncthreads();  // red is reused by the block's next tile
        if (wv > 0) return;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if (!a_ok[i]) continue;
        uint16_t *crow = C + ((size_t)(m0 + 16 * i + n) * H + hd) * N;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int cn = n0 + 16 * j + 4 * g;
            if (cn + 3 < N && (N & 3) == 0) {
                *(u32x2 *)(crow + cn) =
                    u32x2{pack_bf16x2(acc[i][j][0], acc[i][j][1]), pack_bf16x2(acc[i][j][2], acc[i][j][3])};
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (cn + e < N) crow[cn + e] = to_bf16_bits(acc[i][j][e]);
            }
        }
    }
}

// KSPLIT = 1: each wave walks its own tiles (four per block at a time);
// KSPLIT = 4: each block walks tiles, its waves splitting every tile's k-steps.
template <int KSPLIT>
__global__ void __launch_bounds__(256) head_gemm_kernel(const uint16_t *__restrict__ A, const uint16_t *__restrict__ B,
                                                        uint16_t *__restrict__ C, int M, int H, int N, int K)
{
    __shared__ float red[KSPLIT > 1 ? (KSPLIT - 1) * 64 * 64 : 1];
    const int ntn = (N + kGemmTile - 1) / kGemmTile;
    const int ntm = (M + kGemmTile - 1) / kGemmTile;
    const long tiles = (long)H * ntm * ntn;
    const int per_block = KSPLIT > 1 ? 1 : 4;
    const long step = (long)gridDim.x * per_block;
    const long first = (long)blockIdx.x * per_block + (KSPLIT > 1 ? 0 : (threadIdx.x >> 6));
    // KSPLIT > 1: the loop bound is the same for the whole block (its barriers)
    for (long tile = first; tile < tiles; tile += step) {
        const int hd = (int)(tile / ((long)ntm * ntn));
        const int r = (int)(tile - (long)hd * ntm * ntn);
        head_gemm_tile<KSPLIT>(A, B, C, M, H, N, K, hd, (r / ntn) * kGemmTile, (r % ntn) * kGemmTile, red);
    }
}

}  // namespace da
