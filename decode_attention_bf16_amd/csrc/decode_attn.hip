// C ABI of the gfx950 decode-attention library: argument checks, work-partition
// choice and kernel launches. See include/decode_attn.h for the contract.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <mutex>

#include "../../include/decode_attn.h"
#include "combine.hpp"
#include "head_gemm.hpp"
#include "common.hpp"
#include "gqa_kernel.hpp"
#include "mla_kernel.hpp"
#include "plan.hpp"

namespace {

constexpr int kMaxDevices = 64;

struct DeviceInfo {
    int cu_count = 0;
};

std::mutex g_mutex;
DeviceInfo g_dev[kMaxDevices];

int current_cu_count()
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
    std::lock_guard<std::mutex> lock(g_mutex);
    if (g_dev[dev].cu_count == 0) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            cus = 256;
        g_dev[dev].cu_count = cus;
    }
    return g_dev[dev].cu_count;
}

// The log-sum-exp combine for DV-wide rows (one wave per row, or a block per
// row when the sequences average more than 16 segments).
template <int DV>
void launch_combine(int b, int M, int workers, da::PlanHeader *hdr, const int *slot_start, const uint16_t *part_out,
                    const float *part_lse, uint16_t *out, float *lse, hipStream_t stream)
{
    const long rows = (long)b * M;
    const int cus = current_cu_count();
    if (da::combine_use_wide(b, workers))
        hipLaunchKernelGGL(da::combine_wide_kernel<DV>, dim3(da::combine_wide_grid(rows, cus)),
                           dim3(64 * da::kCombineWideWaves), 0, stream, b, M, hdr, slot_start, part_out, part_lse, out,
                           lse);
    else
        hipLaunchKernelGGL(da::combine_kernel<DV>, dim3(da::combine_grid(rows, cus)), dim3(256), 0, stream, b, M, hdr,
                           slot_start, part_out, part_lse, out, lse);
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

bool log_plan()
{
    static const bool on = [] {
        const char *e = getenv("DA_LOG");
        return e && e[0] == '1';
    }();
    return on;
}

// ------------------------------------------------------------------ MLA
int mla_row_blocks(int s, int h) { return (s * h + da::kMlaRows - 1) / da::kMlaRows; }

// Workers (split-KV segments over the tile sequence) for the MLA tile kernel.
// One block per CU is resident, so the units = workers x row blocks run in
// waves of `cus`; a block costs its fixed part (first loads and final stores,
// about kMlaFixedSteps tile steps) plus one step per tile. The count that
// minimises waves x (fixed + tiles per worker) is taken, with the tiles
// estimated from t_max (the lengths are on the device). For the power-of-two
// row-block counts this is cus / row_blocks; for others (e.g. 96 row blocks at
// s = 48, h = 128) it fills the CUs in several waves instead of leaving some idle.
// Within one wave count the cost falls as workers grow, so only the largest
// count of each wave count (up to four waves) and the cap are candidates.
constexpr int kMlaFixedSteps = 12;

int mla_workers(int b, int s, int h, int t_max, int requested)
{
    if (requested > 0) return requested;
    const int rb = mla_row_blocks(s, h);
    const int cus = current_cu_count();
    // never more workers than tiles could exist
    const long max_tiles = (long)b * ((t_max + da::kMlaTile - 1) / da::kMlaTile);
    const long w_hi = std::min<long>(max_tiles, std::max<long>(1, 4L * cus / rb));
    long best_w = 1;
    double best = -1.0;
    for (int k = 1; k <= 5; ++k) {
        const long w = k <= 4 ? std::min<long>(w_hi, std::max<long>(1, (long)k * cus / rb)) : w_hi;
        const long waves = (w * rb + cus - 1) / cus;
        const double cost = (double)waves * (kMlaFixedSteps + (double)((max_tiles + w - 1) / w));
        if (best < 0.0 || cost < best) {
            best = cost;
            best_w = w;
        }
    }
    return (int)best_w;
}

bool mla_supported(int k, int p)
{
    return (k == 512 && p == 64) || (k == 256 && p == 64) || (k == 128 && p == 64) || (k == 64 && p == 16);
}

template <int K, int P>
hipError_t launch_mla(const uint16_t *q_lat, const uint16_t *q_rope, const uint16_t *cache, const int32_t *seqlens,
                      int b, int s, int h, int t_max, float scale_log2, uint16_t *out, float *lse,
                      const da::WsLayout &ws, char *wsp, int workers, hipStream_t stream)
{
    using C = da::MlaCfg<K, P>;
    static std::once_flag attr_once;
    static hipError_t attr_err = hipSuccess;
    std::call_once(attr_once, [] {
        attr_err = hipFuncSetAttribute((const void *)da::mla_decode_kernel<K, P>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS_BYTES);
    });
    if (attr_err != hipSuccess) return attr_err;

    auto *hdr = (da::PlanHeader *)(wsp + ws.header);
    int *tile_start = (int *)(wsp + ws.tile_start);
    int *slot_start = (int *)(wsp + ws.slot_start);
    float *part_lse = (float *)(wsp + ws.part_lse);
    uint16_t *part_out = (uint16_t *)(wsp + ws.part_out);

    const int rb = mla_row_blocks(s, h);
    const int units = workers * rb;
    const int grid = (units + 7) / 8 * 8;
    if (log_plan())
        fprintf(stderr, "[decode_attn] mla k=%d p=%d b=%d s=%d h=%d t_max=%d workers=%d row_blocks=%d grid=%d lds=%d\n",
                K, P, b, s, h, t_max, workers, rb, grid, C::LDS_BYTES);
    hipLaunchKernelGGL((da::mla_decode_kernel<K, P>), dim3(grid), dim3(C::THREADS), C::LDS_BYTES, stream, q_lat, q_rope,
                       cache, seqlens, b, s, h, t_max, scale_log2, rb, units, hdr, tile_start, slot_start, out, lse,
                       part_out, part_lse);
    launch_combine<K>(b, s * h, workers, hdr, slot_start, part_out, part_lse, out, lse, stream);
    return hipGetLastError();
}

// ------------------------------------------------------------------ GQA
int gqa_head_blocks(int hkv) { return (hkv + 3) / 4; }
int gqa_choose_path(int rows, int path);

// Launch shape of the MFMA kernel per head dim: KV heads per block and ring depth.
#ifndef DA_GQA128_HPB
#define DA_GQA128_HPB 4
#endif
#ifndef DA_GQA128_NST
#define DA_GQA128_NST 4
#endif
template <int D>
struct GqaMfmaShape {
    static constexpr int HPB = D == 128 ? DA_GQA128_HPB : 512 / D;
    static constexpr int NST = D == 128 ? DA_GQA128_NST : 4;
};
template <int D, int RBLK>
using GqaMfmaCfgFor = da::GqaMfmaCfg<D, RBLK, GqaMfmaShape<D>::HPB, GqaMfmaShape<D>::NST>;

// (heads per block, resident blocks per CU) of the MFMA kernel for head dim d
void gqa_mfma_geometry(int d, int &hpb, int &per_cu)
{
    int lds = 0;
    if (d == 64) {
        hpb = GqaMfmaCfgFor<64, 1>::HPB;
        lds = GqaMfmaCfgFor<64, 1>::LDS_BYTES;
    } else if (d == 128) {
        hpb = GqaMfmaCfgFor<128, 1>::HPB;
        lds = GqaMfmaCfgFor<128, 1>::LDS_BYTES;
    } else {
        hpb = GqaMfmaCfgFor<256, 1>::HPB;
        lds = GqaMfmaCfgFor<256, 1>::LDS_BYTES;
    }
    per_cu = 163840 / lds;
    if (per_cu < 1) per_cu = 1;
}

int gqa_workers(int b, int hkv, int d, int rows, int path, int t_max, int requested)
{
    if (requested > 0) return requested;
    int w;
    if (gqa_choose_path(rows, path) == 0) {
        w = 2 * current_cu_count() / gqa_head_blocks(hkv);
    } else {
        int hpb, per_cu;
        gqa_mfma_geometry(d, hpb, per_cu);  // blocks stay resident through their LDS ring
        w = per_cu * current_cu_count() / ((hkv + hpb - 1) / hpb);
    }
    if (w < 1) w = 1;
    const long max_tiles = (long)b * ((t_max + da::kGqaTile - 1) / da::kGqaTile);
    if ((long)w > max_tiles) w = (int)max_tiles;
    return w < 1 ? 1 : w;
}

bool gqa_valu_ok(int rows) { return rows <= 16; }

template <int D, int R>
void launch_gqa_valu(const uint16_t *q, const uint16_t *k, const uint16_t *v, const int32_t *seqlens, int b, int s,
                     int hq, int hkv, int t_max, float scale_log2, uint16_t *out, float *lse, da::PlanHeader *hdr,
                     int *tile_start, int *slot_start, uint16_t *part_out, float *part_lse, int workers,
                     hipStream_t stream)
{
    const int hb = gqa_head_blocks(hkv);
    const int units = workers * hb;
    const int grid = (units + 7) / 8 * 8;
    hipLaunchKernelGGL((da::gqa_valu_kernel<D, R>), dim3(grid), dim3(256), 0, stream, q, k, v, seqlens, b, s, hq,
                       hkv, t_max, scale_log2, hb, units, hdr, tile_start, slot_start, out, lse, part_out,
                       part_lse);
}

template <int D>
bool dispatch_gqa_valu(int rows, const uint16_t *q, const uint16_t *k, const uint16_t *v, const int32_t *seqlens,
                       int b, int s, int hq, int hkv, int t_max, float scale_log2, uint16_t *out, float *lse,
                       da::PlanHeader *hdr, int *tile_start, int *slot_start, uint16_t *part_out, float *part_lse,
                       int workers, hipStream_t stream)
{
#define DA_GQA_CASE(RR)                                                                                            \
    if (rows <= RR) {                                                                                              \
        launch_gqa_valu<D, RR>(q, k, v, seqlens, b, s, hq, hkv, t_max, scale_log2, out, lse, hdr, tile_start,      \
                               slot_start, part_out, part_lse, workers, stream);                                  \
        return true;                                                                                               \
    }
    DA_GQA_CASE(2)
    DA_GQA_CASE(4)
    DA_GQA_CASE(8)
    DA_GQA_CASE(16)
#undef DA_GQA_CASE
    return false;
}

template <int D, int RBLK>
hipError_t launch_gqa_mfma(const uint16_t *q, const uint16_t *k, const uint16_t *v, const int32_t *seqlens, int b,
                           int s, int hq, int hkv, int t_max, float scale_log2, uint16_t *out, float *lse,
                           da::PlanHeader *hdr, int *tile_start, int *slot_start, uint16_t *part_out, float *part_lse,
                           int workers, hipStream_t stream)
{
    using C = GqaMfmaCfgFor<D, RBLK>;
    static std::once_flag attr_once;
    static hipError_t attr_err = hipSuccess;
    std::call_once(attr_once, [] {
        attr_err = hipFuncSetAttribute((const void *)da::gqa_mfma_kernel<D, RBLK, C::HPB, C::NST>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS_BYTES);
    });
    if (attr_err != hipSuccess) return attr_err;
    const int hb = (hkv + C::HPB - 1) / C::HPB;
    const int units = workers * hb;
    const int grid = (units + 7) / 8 * 8;
    hipLaunchKernelGGL((da::gqa_mfma_kernel<D, RBLK, C::HPB, C::NST>), dim3(grid), dim3(C::THREADS), C::LDS_BYTES, stream, q, k, v,
                       seqlens, b, s, hq, hkv, t_max, scale_log2, hb, units, hdr, tile_start, slot_start, out, lse,
                       part_out, part_lse);
    return hipSuccess;
}

template <int D>
hipError_t dispatch_gqa_mfma(int rows, const uint16_t *q, const uint16_t *k, const uint16_t *v,
                             const int32_t *seqlens, int b, int s, int hq, int hkv, int t_max, float scale_log2,
                             uint16_t *out, float *lse, da::PlanHeader *hdr, int *tile_start, int *slot_start,
                             uint16_t *part_out, float *part_lse, int workers, hipStream_t stream)
{
    if (rows <= 16)
        return launch_gqa_mfma<D, 1>(q, k, v, seqlens, b, s, hq, hkv, t_max, scale_log2, out, lse, hdr, tile_start,
                                     slot_start, part_out, part_lse, workers, stream);
    if (rows <= 32 || D == 256)
        return launch_gqa_mfma<D, 2>(q, k, v, seqlens, b, s, hq, hkv, t_max, scale_log2, out, lse, hdr, tile_start,
                                     slot_start, part_out, part_lse, workers, stream);
    if (rows <= 48)  // three 16-row blocks: 33..48 rows without padding to 64 (d = 256 stops at 32 rows)
        return launch_gqa_mfma<D, (D == 256 ? 2 : 3)>(q, k, v, seqlens, b, s, hq, hkv, t_max, scale_log2, out, lse,
                                                      hdr, tile_start, slot_start, part_out, part_lse, workers, stream);
    return launch_gqa_mfma<D, (D == 256 ? 2 : 4)>(q, k, v, seqlens, b, s, hq, hkv, t_max, scale_log2, out, lse, hdr,
                                                  tile_start, slot_start, part_out, part_lse, workers, stream);
}

// 0 = VALU dot kernel, 1 = MFMA kernel
int gqa_choose_path(int rows, int path)
{
    if (path == 1) return 0;
    if (path == 2) return 1;
    (void)rows;
    return 1;  // measured faster at every row count (see the design notes)
}

// ------------------------------------------------------------------ un-absorbed MLA
// The grouped MFMA kernel with one query head per KV head (g = 1): per-head
// key rows of 192 (128 decompressed + 64 rope) and value rows of 128.
constexpr int kUnabsDK = 192, kUnabsDV = 128, kUnabsHPB = 2, kUnabsNST = 4;
template <int RBLK>
using UnabsCfg = da::GqaMfmaCfg<kUnabsDK, RBLK, kUnabsHPB, kUnabsNST, kUnabsDV>;

int unabs_workers(int b, int h, int t_max, int requested)
{
    if (requested > 0) return requested;
    int per_cu = 163840 / UnabsCfg<1>::LDS_BYTES;
    if (per_cu < 1) per_cu = 1;
    int w = per_cu * current_cu_count() / ((h + kUnabsHPB - 1) / kUnabsHPB);
    if (w < 1) w = 1;
    const long max_tiles = (long)b * ((t_max + da::kGqaTile - 1) / da::kGqaTile);
    if ((long)w > max_tiles) w = (int)max_tiles;
    return w < 1 ? 1 : w;
}

template <int RBLK>
hipError_t launch_unabs(const uint16_t *q, const uint16_t *k, const uint16_t *v, const int32_t *seqlens, int b, int s,
                        int h, int t_max, float scale_log2, uint16_t *out, float *lse, da::PlanHeader *hdr,
                        int *tile_start, int *slot_start, uint16_t *part_out, float *part_lse, int workers,
                        hipStream_t stream)
{
    using C = UnabsCfg<RBLK>;
    static std::once_flag attr_once;
    static hipError_t attr_err = hipSuccess;
    std::call_once(attr_once, [] {
        attr_err = hipFuncSetAttribute(
            (const void *)da::gqa_mfma_kernel<kUnabsDK, RBLK, kUnabsHPB, kUnabsNST, kUnabsDV>,
            hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS_BYTES);
    });
    if (attr_err != hipSuccess) return attr_err;
    const int hb = (h + C::HPB - 1) / C::HPB;
    const int units = workers * hb;
    const int grid = (units + 7) / 8 * 8;
    if (log_plan())
        fprintf(stderr, "[decode_attn] mla-unabsorbed b=%d s=%d h=%d t_max=%d workers=%d grid=%d lds=%d\n", b, s, h,
                t_max, workers, grid, C::LDS_BYTES);
    hipLaunchKernelGGL((da::gqa_mfma_kernel<kUnabsDK, RBLK, kUnabsHPB, kUnabsNST, kUnabsDV>), dim3(grid),
                       dim3(C::THREADS), C::LDS_BYTES, stream, q, k, v, seqlens, b, s, h, h, t_max, scale_log2, hb,
                       units, hdr, tile_start, slot_start, out, lse, part_out, part_lse);
    return hipGetLastError();
}

}  // namespace

extern "C" {

int da_version(void) { return 100; }

const char *da_status_string(da_status status)
{
    switch (status) {
    case DA_OK:
        return "ok";
    case DA_ERR_INVALID_ARG:
        return "invalid argument";
    case DA_ERR_UNSUPPORTED:
        return "unsupported dimensions";
    case DA_ERR_WORKSPACE:
        return "workspace too small";
    case DA_ERR_HIP:
        return "HIP launch error";
    }
    return "unknown status";
}

static da_status mla_check(int b, int s, int h, int k, int p, int t_max, int num_workers)
{
    if (b <= 0 || s <= 0 || h <= 0 || k <= 0 || p <= 0 || t_max <= 0 || num_workers < 0) return DA_ERR_INVALID_ARG;
    if (s > t_max) return DA_ERR_INVALID_ARG;
    if (!mla_supported(k, p)) return DA_ERR_UNSUPPORTED;
    if ((long)s * h > 65536) return DA_ERR_UNSUPPORTED;
    // one sequence's cache rows must be addressable by a 32-bit buffer offset
    if ((long long)t_max * (k + p) * 2 >= (1LL << 31)) return DA_ERR_UNSUPPORTED;
    return DA_OK;
}

size_t mla_decode_workspace_size(int b, int s, int h, int k, int p, int t_max, int num_workers)
{
    if (mla_check(b, s, h, k, p, t_max, num_workers) != DA_OK) return 0;
    const int w = mla_workers(b, s, h, t_max, num_workers);
    return da::ws_layout(b, s * h, k, w).total;
}

da_status mla_decode(const uint16_t *q_lat, const uint16_t *q_rope, const uint16_t *cache, const int32_t *seqlens,
                     int b, int s, int h, int k, int p, int t_max, float scale, uint16_t *out_lat, float *lse,
                     void *workspace, size_t workspace_bytes, int num_workers, void *stream)
{
    da_status st = mla_check(b, s, h, k, p, t_max, num_workers);
    if (st != DA_OK) return st;
    if (!q_lat || !q_rope || !cache || !seqlens || !out_lat || !lse || !workspace) return DA_ERR_INVALID_ARG;
    if (!aligned16(q_lat) || !aligned16(q_rope) || !aligned16(cache) || !aligned16(out_lat))
        return DA_ERR_INVALID_ARG;
    if (((uintptr_t)workspace & 255u) != 0) return DA_ERR_INVALID_ARG;
    if (!std::isfinite(scale) || !(scale > 0.f)) return DA_ERR_INVALID_ARG;
    const int workers = mla_workers(b, s, h, t_max, num_workers);
    const da::WsLayout ws = da::ws_layout(b, s * h, k, workers);
    if (workspace_bytes < ws.total) return DA_ERR_WORKSPACE;

    const float sl2 = scale * da::kLog2e;
    hipStream_t st_ = (hipStream_t)stream;
    char *wsp = (char *)workspace;
    hipError_t e = hipSuccess;
    if (k == 512 && p == 64)
        e = launch_mla<512, 64>(q_lat, q_rope, cache, seqlens, b, s, h, t_max, sl2, out_lat, lse, ws, wsp, workers, st_);
    else if (k == 256 && p == 64)
        e = launch_mla<256, 64>(q_lat, q_rope, cache, seqlens, b, s, h, t_max, sl2, out_lat, lse, ws, wsp, workers, st_);
    else if (k == 128 && p == 64)
        e = launch_mla<128, 64>(q_lat, q_rope, cache, seqlens, b, s, h, t_max, sl2, out_lat, lse, ws, wsp, workers, st_);
    else
        e = launch_mla<64, 16>(q_lat, q_rope, cache, seqlens, b, s, h, t_max, sl2, out_lat, lse, ws, wsp, workers, st_);
    return e == hipSuccess ? DA_OK : DA_ERR_HIP;
}

static da_status gqa_check(int b, int s, int hq, int hkv, int d, int t_max, int num_workers, int path)
{
    if (b <= 0 || s <= 0 || hq <= 0 || hkv <= 0 || d <= 0 || t_max <= 0 || num_workers < 0) return DA_ERR_INVALID_ARG;
    if (hq % hkv != 0 || s > t_max) return DA_ERR_INVALID_ARG;
    if (path < 0 || path > 2) return DA_ERR_INVALID_ARG;
    if (!(d == 64 || d == 128 || d == 256)) return DA_ERR_UNSUPPORTED;
    const int rows = (hq / hkv) * s;
    if (rows > (d == 256 ? 32 : 64)) return DA_ERR_UNSUPPORTED;
    if (gqa_choose_path(rows, path) == 0 && !gqa_valu_ok(rows)) return DA_ERR_UNSUPPORTED;
    // one sequence's K (or V) rows must be addressable by a 32-bit buffer offset
    if ((long long)t_max * hkv * d * 2 >= (1LL << 31)) return DA_ERR_UNSUPPORTED;
    return DA_OK;
}

size_t gqa_decode_workspace_size(int b, int s, int hq, int hkv, int d, int t_max, int num_workers, int path)
{
    if (gqa_check(b, s, hq, hkv, d, t_max, num_workers, path) != DA_OK) return 0;
    const int w = gqa_workers(b, hkv, d, (hq / hkv) * s, path, t_max, num_workers);
    return da::ws_layout(b, s * hq, d, w).total;
}

da_status gqa_decode(const uint16_t *q, const uint16_t *k_cache, const uint16_t *v_cache, const int32_t *seqlens,
                     int b, int s, int hq, int hkv, int d, int t_max, float scale, uint16_t *out, float *lse,
                     void *workspace, size_t workspace_bytes, int num_workers, int path, void *stream)
{
    da_status st = gqa_check(b, s, hq, hkv, d, t_max, num_workers, path);
    if (st != DA_OK) return st;
    if (!q || !k_cache || !v_cache || !seqlens || !out || !lse || !workspace) return DA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out)) return DA_ERR_INVALID_ARG;
    if (((uintptr_t)workspace & 255u) != 0) return DA_ERR_INVALID_ARG;
    if (!std::isfinite(scale) || !(scale > 0.f)) return DA_ERR_INVALID_ARG;
    const int rows = (hq / hkv) * s;
    const int use_mfma = gqa_choose_path(rows, path);
    const int workers = gqa_workers(b, hkv, d, rows, path, t_max, num_workers);
    const da::WsLayout ws = da::ws_layout(b, s * hq, d, workers);
    if (workspace_bytes < ws.total) return DA_ERR_WORKSPACE;

    char *wsp = (char *)workspace;
    auto *hdr = (da::PlanHeader *)(wsp + ws.header);
    int *tile_start = (int *)(wsp + ws.tile_start);
    int *slot_start = (int *)(wsp + ws.slot_start);
    float *part_lse = (float *)(wsp + ws.part_lse);
    uint16_t *part_out = (uint16_t *)(wsp + ws.part_out);
    hipStream_t st_ = (hipStream_t)stream;
    const float sl2 = scale * da::kLog2e;

    if (log_plan())
        fprintf(stderr, "[decode_attn] gqa d=%d b=%d s=%d hq=%d hkv=%d t_max=%d workers=%d path=%s\n", d, b, s, hq,
                hkv, t_max, workers, use_mfma ? "mfma" : "valu");
    bool ok = false;
    if (use_mfma) {
        hipError_t e;
        if (d == 64)
            e = dispatch_gqa_mfma<64>(rows, q, k_cache, v_cache, seqlens, b, s, hq, hkv, t_max, sl2, out, lse, hdr,
                                      tile_start, slot_start, part_out, part_lse, workers, st_);
        else if (d == 128)
            e = dispatch_gqa_mfma<128>(rows, q, k_cache, v_cache, seqlens, b, s, hq, hkv, t_max, sl2, out, lse, hdr,
                                       tile_start, slot_start, part_out, part_lse, workers, st_);
        else
            e = dispatch_gqa_mfma<256>(rows, q, k_cache, v_cache, seqlens, b, s, hq, hkv, t_max, sl2, out, lse, hdr,
                                       tile_start, slot_start, part_out, part_lse, workers, st_);
        if (e != hipSuccess) return DA_ERR_HIP;
        ok = true;
    } else if (d == 64)
        ok = dispatch_gqa_valu<64>(rows, q, k_cache, v_cache, seqlens, b, s, hq, hkv, t_max, sl2, out, lse, hdr,
                                   tile_start, slot_start, part_out, part_lse, workers, st_);
    else if (d == 128)
        ok = dispatch_gqa_valu<128>(rows, q, k_cache, v_cache, seqlens, b, s, hq, hkv, t_max, sl2, out, lse, hdr,
                                    tile_start, slot_start, part_out, part_lse, workers, st_);
    else
        ok = dispatch_gqa_valu<256>(rows, q, k_cache, v_cache, seqlens, b, s, hq, hkv, t_max, sl2, out, lse, hdr,
                                    tile_start, slot_start, part_out, part_lse, workers, st_);
    if (!ok) return DA_ERR_UNSUPPORTED;
    if (d == 64)
        launch_combine<64>(b, s * hq, workers, hdr, slot_start, part_out, part_lse, out, lse, st_);
    else if (d == 128)
        launch_combine<128>(b, s * hq, workers, hdr, slot_start, part_out, part_lse, out, lse, st_);
    else
        launch_combine<256>(b, s * hq, workers, hdr, slot_start, part_out, part_lse, out, lse, st_);
    return hipGetLastError() == hipSuccess ? DA_OK : DA_ERR_HIP;
}

static da_status unabs_check(int b, int s, int h, int dqk, int dv, int t_max, int num_workers)
{
    if (b <= 0 || s <= 0 || h <= 0 || dqk <= 0 || dv <= 0 || t_max <= 0 || num_workers < 0) return DA_ERR_INVALID_ARG;
    if (s > t_max) return DA_ERR_INVALID_ARG;
    if (!(dqk == kUnabsDK && dv == kUnabsDV)) return DA_ERR_UNSUPPORTED;
    if (s > 64) return DA_ERR_UNSUPPORTED;
    // one sequence's K rows must be addressable by a 32-bit buffer offset
    if ((long long)t_max * h * dqk * 2 >= (1LL << 31)) return DA_ERR_UNSUPPORTED;
    return DA_OK;
}

size_t mla_decode_unabsorbed_workspace_size(int b, int s, int h, int dqk, int dv, int t_max, int num_workers)
{
    if (unabs_check(b, s, h, dqk, dv, t_max, num_workers) != DA_OK) return 0;
    return da::ws_layout(b, s * h, dv, unabs_workers(b, h, t_max, num_workers)).total;
}

da_status mla_decode_unabsorbed(const uint16_t *q, const uint16_t *k_cache, const uint16_t *v_cache,
                                const int32_t *seqlens, int b, int s, int h, int dqk, int dv, int t_max, float scale,
                                uint16_t *out, float *lse, void *workspace, size_t workspace_bytes, int num_workers,
                                void *stream)
{
    da_status st = unabs_check(b, s, h, dqk, dv, t_max, num_workers);
    if (st != DA_OK) return st;
    if (!q || !k_cache || !v_cache || !seqlens || !out || !lse || !workspace) return DA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out)) return DA_ERR_INVALID_ARG;
    if (((uintptr_t)workspace & 255u) != 0) return DA_ERR_INVALID_ARG;
    if (!std::isfinite(scale) || !(scale > 0.f)) return DA_ERR_INVALID_ARG;
    const int workers = unabs_workers(b, h, t_max, num_workers);
    const da::WsLayout ws = da::ws_layout(b, s * h, dv, workers);
    if (workspace_bytes < ws.total) return DA_ERR_WORKSPACE;

    char *wsp = (char *)workspace;
    auto *hdr = (da::PlanHeader *)(wsp + ws.header);
    int *tile_start = (int *)(wsp + ws.tile_start);
    int *slot_start = (int *)(wsp + ws.slot_start);
    float *part_lse = (float *)(wsp + ws.part_lse);
    uint16_t *part_out = (uint16_t *)(wsp + ws.part_out);
    hipStream_t st_ = (hipStream_t)stream;
    const float sl2 = scale * da::kLog2e;
    hipError_t e;
    if (s <= 16)
        e = launch_unabs<1>(q, k_cache, v_cache, seqlens, b, s, h, t_max, sl2, out, lse, hdr, tile_start, slot_start,
                            part_out, part_lse, workers, st_);
    else if (s <= 32)
        e = launch_unabs<2>(q, k_cache, v_cache, seqlens, b, s, h, t_max, sl2, out, lse, hdr, tile_start, slot_start,
                            part_out, part_lse, workers, st_);
    else if (s <= 48)  // three 16-row blocks: s = 33..48 without padding to 64 rows
        e = launch_unabs<3>(q, k_cache, v_cache, seqlens, b, s, h, t_max, sl2, out, lse, hdr, tile_start, slot_start,
                            part_out, part_lse, workers, st_);
    else
        e = launch_unabs<4>(q, k_cache, v_cache, seqlens, b, s, h, t_max, sl2, out, lse, hdr, tile_start, slot_start,
                            part_out, part_lse, workers, st_);
    if (e != hipSuccess) return DA_ERR_HIP;
    launch_combine<kUnabsDV>(b, s * h, workers, hdr, slot_start, part_out, part_lse, out, lse, st_);
    return hipGetLastError() == hipSuccess ? DA_OK : DA_ERR_HIP;
}

// ------------------------------------------------------------------ per-head projections
#ifndef PROJ_BLOCKS_PER_CU
#define PROJ_BLOCKS_PER_CU 2  // blocks per CU of the tile loop
#endif
static da_status head_gemm(const uint16_t *a, const uint16_t *bw, uint16_t *c, int m, int h, int n, int k,
                           void *stream)
{
    if (!a || !bw || !c || m <= 0 || h <= 0 || n <= 0 || k <= 0) return DA_ERR_INVALID_ARG;
    if (k % 32 != 0) return DA_ERR_UNSUPPORTED;
    if (!aligned16(a) || !aligned16(bw) || !aligned16(c)) return DA_ERR_INVALID_ARG;
    const long tiles = (long)h * ((n + da::kGemmTile - 1) / da::kGemmTile) * ((m + da::kGemmTile - 1) / da::kGemmTile);
    const int cus = current_cu_count();
    if (tiles < 2L * cus) {
        // few tiles: the four waves of a block split each tile's contraction
        const long want = 2L * cus;
        const unsigned grid = (unsigned)(tiles < want ? tiles : want);
        hipLaunchKernelGGL(da::head_gemm_kernel<4>, dim3(grid), dim3(256), 0, (hipStream_t)stream, a, bw, c, m, h, n,
                           k);
    } else {
        const long want = (long)PROJ_BLOCKS_PER_CU * cus;
        const long blocks = (tiles + 3) / 4;  // four tiles (one per wave) per block
        const unsigned grid = (unsigned)(blocks < want ? blocks : want);
        hipLaunchKernelGGL(da::head_gemm_kernel<1>, dim3(grid), dim3(256), 0, (hipStream_t)stream, a, bw, c, m, h, n,
                           k);
    }
    return hipGetLastError() == hipSuccess ? DA_OK : DA_ERR_HIP;
}

da_status mla_absorb_queries(const uint16_t *q_nope, const uint16_t *w_k, uint16_t *q_lat, int b, int s, int h,
                             int d, int k, void *stream)
{
    if (b <= 0 || s <= 0) return DA_ERR_INVALID_ARG;
    return head_gemm(q_nope, w_k, q_lat, b * s, h, k, d, stream);
}

da_status mla_decompress_output(const uint16_t *o_lat, const uint16_t *w_v_t, uint16_t *out, int b, int s, int h,
                                int k, int d, void *stream)
{
    if (b <= 0 || s <= 0) return DA_ERR_INVALID_ARG;
    return head_gemm(o_lat, w_v_t, out, b * s, h, d, k, stream);
}

// ------------------------------------------------------------------ split latent / decompressed cache
// Workspace of mla_decode_split_cache: the intermediates, then the inner calls'
// own workspaces.
struct SplitWs {
    size_t q_lat, q_full, o_lat, lse_old, out_old, out_new, lse_new, ws_abs, ws_unabs, total;
    size_t ws_abs_bytes, ws_unabs_bytes;
};
static SplitWs split_ws(int b, int s, int h, int o_max, int n_max, int num_workers)
{
    SplitWs w{};
    const size_t rows = (size_t)b * s * h;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off = da::align256(off + bytes);
        return at;
    };
    w.q_lat = take(rows * 512 * 2);
    w.q_full = take(rows * 192 * 2);
    w.o_lat = take(rows * 512 * 2);
    w.lse_old = take(rows * 4);
    w.out_old = take(rows * 128 * 2);
    w.out_new = take(rows * 128 * 2);
    w.lse_new = take(rows * 4);
    w.ws_abs_bytes = mla_decode_workspace_size(b, 1, s * h, 512, 64, o_max, num_workers);
    w.ws_unabs_bytes = mla_decode_unabsorbed_workspace_size(b, s, h, 192, 128, n_max, num_workers);
    w.ws_abs = take(w.ws_abs_bytes);
    w.ws_unabs = take(w.ws_unabs_bytes);
    w.total = off;
    return w;
}

static da_status split_check(int b, int s, int h, int o_max, int n_max, int num_workers)
{
    if (b <= 0 || s <= 0 || h <= 0 || o_max <= 0 || n_max <= 0 || num_workers < 0) return DA_ERR_INVALID_ARG;
    if (s > n_max) return DA_ERR_INVALID_ARG;
    if (mla_decode_workspace_size(b, 1, s * h, 512, 64, o_max, num_workers) == 0) return DA_ERR_UNSUPPORTED;
    if (mla_decode_unabsorbed_workspace_size(b, s, h, 192, 128, n_max, num_workers) == 0) return DA_ERR_UNSUPPORTED;
    return DA_OK;
}

size_t mla_decode_split_cache_workspace_size(int b, int s, int h, int o_max, int n_max, int num_workers)
{
    if (split_check(b, s, h, o_max, n_max, num_workers) != DA_OK) return 0;
    return split_ws(b, s, h, o_max, n_max, num_workers).total;
}

da_status mla_decode_split_cache(const uint16_t *q_nope, const uint16_t *q_rope, const uint16_t *w_k,
                                 const uint16_t *w_v_t, const uint16_t *latent, const int32_t *seqlens_old,
                                 const uint16_t *k_new, const uint16_t *v_new, const int32_t *seqlens_new, int b,
                                 int s, int h, int o_max, int n_max, float scale, uint16_t *out, float *lse,
                                 void *workspace, size_t workspace_bytes, int num_workers, void *stream)
{
    da_status st = split_check(b, s, h, o_max, n_max, num_workers);
    if (st != DA_OK) return st;
    if (!q_nope || !q_rope || !w_k || !w_v_t || !latent || !seqlens_old || !k_new || !v_new || !seqlens_new || !out ||
        !lse || !workspace)
        return DA_ERR_INVALID_ARG;
    if (!aligned16(q_nope) || !aligned16(q_rope) || !aligned16(out) || ((uintptr_t)workspace & 255u) != 0)
        return DA_ERR_INVALID_ARG;
    if (!std::isfinite(scale) || !(scale > 0.f)) return DA_ERR_INVALID_ARG;
    const SplitWs w = split_ws(b, s, h, o_max, n_max, num_workers);
    if (workspace_bytes < w.total) return DA_ERR_WORKSPACE;
    char *wsp = (char *)workspace;
    auto *q_lat = (uint16_t *)(wsp + w.q_lat);
    auto *q_full = (uint16_t *)(wsp + w.q_full);
    auto *o_lat = (uint16_t *)(wsp + w.o_lat);
    auto *lse_old = (float *)(wsp + w.lse_old);
    auto *out_old = (uint16_t *)(wsp + w.out_old);
    auto *out_new = (uint16_t *)(wsp + w.out_new);
    auto *lse_new = (float *)(wsp + w.lse_new);
    const long rows = (long)b * s * h;
    hipStream_t st_ = (hipStream_t)stream;
    // old rows, latent and absorbed: every draft sees all of them, so the s
    // drafts of a sequence are s*h independent query rows of one step
    if ((st = mla_absorb_queries(q_nope, w_k, q_lat, b, s, h, 128, 512, stream)) != DA_OK) return st;
    if ((st = mla_decode(q_lat, q_rope, latent, seqlens_old, b, 1, s * h, 512, 64, o_max, scale, o_lat, lse_old,
                         wsp + w.ws_abs, w.ws_abs_bytes, num_workers, stream)) != DA_OK)
        return st;
    if ((st = mla_decompress_output(o_lat, w_v_t, out_old, b, s, h, 512, 128, stream)) != DA_OK) return st;
    // new rows, decompressed: the drafts' causal mask applies here
    const unsigned cgrid = (unsigned)std::min<long>((rows * 24 + 255) / 256, 4L * current_cu_count());
    hipLaunchKernelGGL(da::concat_rows_kernel, dim3(cgrid), dim3(256), 0, st_, q_nope, 128, q_rope, 64, q_full, rows);
    if ((st = mla_decode_unabsorbed(q_full, k_new, v_new, seqlens_new, b, s, h, 192, 128, n_max, scale, out_new,
                                    lse_new, wsp + w.ws_unabs, w.ws_unabs_bytes, num_workers, stream)) != DA_OK)
        return st;
    hipLaunchKernelGGL(da::merge2_kernel<128>, dim3(da::combine_grid(rows, current_cu_count())), dim3(256), 0, st_,
                       rows, out_old, lse_old, out_new, lse_new, out, lse);
    return hipGetLastError() == hipSuccess ? DA_OK : DA_ERR_HIP;
}

}  // extern "C"
