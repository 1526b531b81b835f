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
// Block = 4 waves = a 64 x 64 tile of one head's C; wave w owns rows 16w..16w+15
// of the tile. Per 32-wide k-step each lane loads its A fragment (16 bytes) and
// four B fragments straight from global memory (the operands are small and the
// same B fragments serve the block's four waves from the L1/L2 caches); a ring
// of four k-steps of loads runs ahead of the MFMAs. The MFMA takes B as its
// first operand, so each lane ends with four consecutive columns of one C row
// and writes them as one 8-byte store.
#pragma once

#include "common.hpp"

namespace da {

constexpr int kGemmTile = 64;

constexpr int kGemmRing = 4;  // k-steps of loads in flight

__global__ void __launch_bounds__(256) head_gemm_kernel(const uint16_t *__restrict__ A, const uint16_t *__restrict__ B,
                                                        uint16_t *__restrict__ C, int M, int H, int N, int K)
{
    // heads vary fastest over the grid, so the blocks in flight together cover
    // all heads of the same rows (contiguous in A and C) rather than rows far apart
    const int hd = blockIdx.x;
    const int n0 = blockIdx.y * kGemmTile;
    const int m0 = blockIdx.z * kGemmTile;
    const int w = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int n = lane & 15;
    const int g = lane >> 4;

    const int am = m0 + 16 * w + n;  // this lane's A row (and C row)
    const bool a_ok = am < M;
    const uint16_t *arow = A + ((size_t)(a_ok ? am : 0) * H + hd) * K + 8 * g;
    const uint16_t *brow[4];
    bool b_ok[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int bn = n0 + 16 * j + n;
        b_ok[j] = bn < N;
        brow[j] = B + ((size_t)hd * N + (b_ok[j] ? bn : 0)) * K + 8 * g;
    }
    struct Frag {
        bf16x8 a, b[4];
    };
    auto load = [&](int kk, Frag &f) {
        const u32x4 z = {0u, 0u, 0u, 0u};
        f.a = as_bf16x8(a_ok ? *(const u32x4 *)(arow + kk) : z);
#pragma unroll
        for (int j = 0; j < 4; ++j) f.b[j] = as_bf16x8(b_ok[j] ? *(const u32x4 *)(brow[j] + kk) : z);
    };

    // acc[j]: lane (n, g) holds C row 16w + n, columns 16j + 4g .. 16j + 4g + 3
    f32x4 acc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int ksteps = K / 32;
    Frag ring[kGemmRing];
#pragma unroll
    for (int r = 0; r < kGemmRing; ++r)
        if (r < ksteps) load(r * 32, ring[r]);
    for (int k0 = 0; k0 < ksteps; k0 += kGemmRing) {
#pragma unroll
        for (int r = 0; r < kGemmRing; ++r) {
            if (k0 + r < ksteps) {
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[j] = mfma16x16x32(ring[r].b[j], ring[r].a, acc[j]);
                if (k0 + r + kGemmRing < ksteps) load((k0 + r + kGemmRing) * 32, ring[r]);
            }
        }
    }
    if (!a_ok) return;
    uint16_t *crow = C + ((size_t)am * H + hd) * N;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int cn = n0 + 16 * j + 4 * g;
        if (cn + 3 < N && (N & 3) == 0) {
            *(u32x2 *)(crow + cn) = u32x2{pack_bf16x2(acc[j][0], acc[j][1]), pack_bf16x2(acc[j][2], acc[j][3])};
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (cn + i < N) crow[cn + i] = to_bf16_bits(acc[j][i]);
        }
    }
}

}  // namespace da
