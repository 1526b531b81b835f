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

// Device scratch of mla_decode_no_alloc (the split-KV plan and the partial
// results that mla_decode keeps in the caller's workspace). Every device the
// library runs on holds its own copy until the process ends. In host code the
// name is only a stand-in: the copy's device address comes from
// hipGetSymbolAddress, once per device, and only that address is used.
static __device__ __align__(256) unsigned char scratch[DA_NO_ALLOC_SCRATCH_BYTES];
void *g_scratch[kMaxDevices];  // device address of `scratch` per device (guarded by g_mutex)

// The current device's copy of `scratch` (nullptr on a HIP error).
void *current_scratch()
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_mutex);
    if (g_scratch[dev] == nullptr) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
            (void)hipGetLastError();
            return nullptr;
        }
        g_scratch[dev] = p;
    }
    return g_scratch[dev];
}

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

    // no workspace: one worker per sequence, no partials and no combine
    const bool per_seq = wsp == nullptr;
    auto *hdr = per_seq ? nullptr : (da::PlanHeader *)(wsp + ws.header);
    int *tile_start = per_seq ? nullptr : (int *)(wsp + ws.tile_start);
    int *slot_start = per_seq ? nullptr : (int *)(wsp + ws.slot_start);
    float *part_lse = per_seq ? nullptr : (float *)(wsp + ws.part_lse);
    uint16_t *part_out = per_seq ? nullptr : (uint16_t *)(wsp + ws.part_out);

    const int rb = mla_row_blocks(s, h);
    const int units = workers * rb;
    const int grid = (units + 7) / 8 * 8;
    if (log_plan())
        fprintf(stderr, "[decode_attn] mla k=%d p=%d b=%d s=%d h=%d t_max=%d workers=%d row_blocks=%d grid=%d lds=%d\n",
                K, P, b, s, h, t_max, workers, rb, grid, C::LDS_BYTES);
    hipLaunchKernelGGL((da::mla_decode_kernel<K, P>), dim3(grid), dim3(C::THREADS), C::LDS_BYTES, stream, q_lat, q_rope,
                       cache, seqlens, b, s, h, t_max, scale_log2, rb, units, hdr, tile_start, slot_start, out, lse,
                       part_out, part_lse);
    if (!per_seq) launch_combine<K>(b, s * h, workers, hdr, slot_start, part_out, part_lse, out, lse, stream);
    return hipGetLastError();
}

// ------------------------------------------------------------------ GQA
int gqa_head_blocks(int hkv) { return (hkv + 3) / 4; }
int gqa_choose_path(int rows, int path);
bool gqa_tg_ok(int d, int rows);
bool gqa_tg_auto(int d, int hkv, int rows);

// Launch shape of the head-block MFMA kernel (the shapes the token-group
// kernel does not take: more rows per KV head than one of its waves holds, and
// d = 64 with KV heads in whole eights under the automatic split): KV heads
// per block, row-group waves per head and 16-row blocks per wave. The default
// block holds kBase heads with
// one wave each (all rows of a head in that wave); when hkv is not a multiple
// of kBase, or a head has more rows than one wave holds, a block takes the
// fewest heads a whole LDS token row allows (kMin) and spreads each head's
// rows over up to RG waves that share its K/V stages.
#ifndef DA_GQA128_HPB
#define DA_GQA128_HPB 4
#endif
#ifndef DA_GQA128_NST
#define DA_GQA128_NST 4
#endif
template <int D>
struct GqaMfmaShape {
    static constexpr int kBase = D == 128 ? DA_GQA128_HPB : 512 / D;
    static constexpr int kNst = D == 128 ? DA_GQA128_NST : 4;
    static constexpr int kMin = D == 64 ? 2 : 1;           // a K token row of >= 256 bytes
    static constexpr int kMaxRblk = D == 256 ? 2 : 4;      // register budget of a wave
    static constexpr int kMaxRg = 4;
    static constexpr int kMaxRows = 16 * kMaxRblk * kMaxRg;
};

struct GqaGeom {
    int hpb = 0, rg = 0, rblk = 0;
};

int pow2ceil(int x)
{
    int p = 1;
    while (p < x) p <<= 1;
    return p;
}

template <int D>
GqaGeom gqa_mfma_geom(int hkv, int rows)
{
    using S = GqaMfmaShape<D>;
    const int nrb = (rows + 15) / 16;
    if (nrb <= S::kMaxRblk && hkv % S::kBase == 0) return {S::kBase, 1, nrb};
    int rg = std::min(S::kMaxRg, pow2ceil(nrb));
    int rblk = (nrb + rg - 1) / rg;
    if (rblk > S::kMaxRblk) return {};
    return {S::kMin, rg, rblk};
}

GqaGeom gqa_geom(int d, int hkv, int rows)
{
    return d == 64 ? gqa_mfma_geom<64>(hkv, rows) : d == 128 ? gqa_mfma_geom<128>(hkv, rows) : gqa_mfma_geom<256>(hkv, rows);
}

int gqa_max_rows(int d)
{
    return d == 64 ? GqaMfmaShape<64>::kMaxRows : d == 128 ? GqaMfmaShape<128>::kMaxRows : GqaMfmaShape<256>::kMaxRows;
}

template <int D, int RBLK, int HPB, int RG>
using GqaMfmaCfgFor = da::GqaMfmaCfg<D, RBLK, HPB, (HPB == GqaMfmaShape<D>::kBase ? GqaMfmaShape<D>::kNst : 4), D, RG>;

// LDS bytes of the MFMA kernel's block for a launch shape.
int gqa_mfma_lds(int d, const GqaGeom &g)
{
    const int nst = g.hpb == (d == 128 ? DA_GQA128_HPB : 512 / d) ? (d == 128 ? DA_GQA128_NST : 4) : 4;
    return nst * 16 * g.hpb * d * 2 * 2;
}

int gqa_workers(int b, int hkv, int d, int rows, int path, int t_max, int requested)
{
    if (requested > 0) return requested;
    int w;
    if (gqa_choose_path(rows, path) == 1 && gqa_tg_auto(d, hkv, rows)) {
        // token-group kernel: one block (worker, KV head) per CU
        w = current_cu_count() / hkv;
    } else if (gqa_choose_path(rows, path) == 0) {
        w = 2 * current_cu_count() / gqa_head_blocks(hkv);
    } else {
        const GqaGeom g = gqa_geom(d, hkv, rows);
        // resident blocks per CU: the LDS ring allows several; one per CU
        // measured fastest for both shapes (default heads per block, and one
        // head per block with its rows over several waves: MQA at hq = 64 on
        // this kernel, 512 workers 39.9 us, 256 workers 36.9 us)
        int per_cu = std::min(163840 / gqa_mfma_lds(d, g), 1);
        if (per_cu < 1) per_cu = 1;
        w = per_cu * current_cu_count() / ((hkv + g.hpb - 1) / g.hpb);
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

struct GqaArgs {
    const uint16_t *q, *k, *v;
    const int32_t *seqlens;
    int b, s, hq, hkv, t_max;
    float scale_log2;
    uint16_t *out;
    float *lse;
    da::PlanHeader *hdr;
    int *tile_start, *slot_start;
    uint16_t *part_out;
    float *part_lse;
    int workers;
    hipStream_t stream;
    int rsplit = 1;  // token-group kernel: blocks that split a KV head's query rows
};

template <int D, int RBLK, int HPB, int RG>
hipError_t launch_gqa_mfma(const GqaArgs &a)
{
    using C = GqaMfmaCfgFor<D, RBLK, HPB, RG>;
    auto kern = da::gqa_mfma_kernel<D, RBLK, HPB, C::NST, D, RG>;
    static std::once_flag attr_once;
    static hipError_t attr_err = hipSuccess;
    std::call_once(attr_once, [&] {
        attr_err = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS_BYTES);
    });
    if (attr_err != hipSuccess) return attr_err;
    const int hb = (a.hkv + HPB - 1) / HPB;
    const int units = a.workers * hb;
    const int grid = (units + 7) / 8 * 8;
    if (log_plan())
        fprintf(stderr, "[decode_attn] gqa-mfma d=%d heads/block=%d row groups=%d row blocks/wave=%d workers=%d grid=%d lds=%d\n",
                D, HPB, RG, RBLK, a.workers, grid, C::LDS_BYTES);
    hipLaunchKernelGGL(kern, dim3(grid), dim3(C::THREADS), C::LDS_BYTES, a.stream, a.q, a.k, a.v, a.seqlens, a.b, a.s,
                       a.hq, a.hkv, a.t_max, a.scale_log2, hb, units, a.hdr, a.tile_start, a.slot_start, a.out, a.lse,
                       a.part_out, a.part_lse);
    return hipSuccess;
}

// The instantiated launch shapes (see gqa_mfma_geom).
template <int D>
hipError_t dispatch_gqa_mfma(const GqaGeom &g, const GqaArgs &a)
{
    using S = GqaMfmaShape<D>;
    constexpr int B = S::kBase, M = S::kMin;
    if (g.hpb == B && g.rg == 1) {
        switch (g.rblk) {
        case 1: return launch_gqa_mfma<D, 1, B, 1>(a);
        case 2: return launch_gqa_mfma<D, 2, B, 1>(a);
        case 3: if constexpr (S::kMaxRblk >= 3) return launch_gqa_mfma<D, 3, B, 1>(a); break;
        case 4: if constexpr (S::kMaxRblk >= 4) return launch_gqa_mfma<D, 4, B, 1>(a); break;
        }
    } else if (g.hpb == M) {
        if (g.rg == 1 && g.rblk == 1) return launch_gqa_mfma<D, 1, M, 1>(a);
        if (g.rg == 2 && g.rblk == 1) return launch_gqa_mfma<D, 1, M, 2>(a);
        if (g.rg == 4) {
            switch (g.rblk) {
            case 1: return launch_gqa_mfma<D, 1, M, 4>(a);
            case 2: return launch_gqa_mfma<D, 2, M, 4>(a);
            case 3: if constexpr (S::kMaxRblk >= 3) return launch_gqa_mfma<D, 3, M, 4>(a); break;
            case 4: if constexpr (S::kMaxRblk >= 4) return launch_gqa_mfma<D, 4, M, 4>(a); break;
            }
        }
    }
    return hipErrorInvalidValue;  // not reached: gqa_check admits only these shapes
}

// ---- token-group kernel: one block per (sequence, KV head), no split-KV
constexpr int kGqaTgNst = 2;

bool gqa_tg_ok(int d, int rows) { return ((d == 64 || d == 128) && rows <= 64) || (d == 256 && rows <= 32); }

// The token-group kernel under the automatic worker count. At d = 64 with KV
// heads in whole eights the head-block kernel stays: its blocks copy all eight
// heads' 1 KB token rows whole, where a token-group block reads its own head's
// 128 bytes of every 1 KB (measured, hq = 32, hkv = 8: b = 64, t = 4096 84.5
// against 91.5 us; b = 8, t = 32768 84.5 against 95.3; b = 32, t = 4096 even).
// With four KV heads or fewer the token-group kernel is about twice as fast.
bool gqa_tg_auto(int d, int hkv, int rows) { return gqa_tg_ok(d, rows) && !(d == 64 && hkv % 8 == 0); }

// Row splits of the token-group kernel. With one KV head for all query heads
// (MQA) and more than 48 query rows (d = 64 or 128), the rows are split over
// two blocks that read the same K/V, consecutive units on one XCD: a wave then
// holds 32 rows at most, its registers allow two waves per SIMD, and those
// overlap one another's arithmetic and copy waits. Measured per call (b = 32,
// hq = 64, t = 4096): d = 128 25.2-25.8 against 27.7-28.1 us, d = 64 16.0-16.4
// against 18.2-18.6; at hq = 48 the split was slower (23.9-24.3 against
// 23.3-24.3). With several KV heads the two blocks of a pair drift apart over
// their longer streams and read the K/V twice from HBM: b = 8, s = 4, hq = 128,
// hkv = 8, t = 16384 126 against 93-97 us; b = 32, s = 8, hq = 64, hkv = 8,
// t = 2048 60 against 49-55.
int gqa_tg_rsplit(int d, int hkv, int rows) { return d <= 128 && hkv == 1 && rows > 48 ? 2 : 1; }

// Waves per block: about 32 KB of stage copies in flight per CU (one stage per
// wave, 8 KB at d = 64 and 128: four waves per CU; 16 KB at d = 256: two) measured
// fastest at every batch shape tried (per call, 0.54 GB of K/V unless noted):
//   d = 128, b*hkv =  256: 4 waves 82.5 us, 2 waves 100.7, 1 wave 176
//   d = 128, b*hkv =  512: 2 waves 87-89, 4 waves 91-93 (MHA, 1.07 GB: 165 vs 178)
//   d = 128, b*hkv = 1024: 1 wave 85-87, 2 waves 92, 4 waves 89
//   d = 256, b*hkv =  256: 2 waves 82.5-83, 4 waves 83, 1 wave 118
//   d = 256, b*hkv =  512: 1 wave 82.5, 2 waves 85.5, 4 waves 86.5
int gqa_tg_waves(int units, int d)
{
    const int per_cu = d == 256 ? 2 : 4;  // waves per CU for ~32 KB in flight
    const long budget = 3L * per_cu * current_cu_count();
    for (int tg = 4; tg > 1; tg >>= 1)
        if (2L * tg * units <= budget) return tg;
    return 1;
}

template <int D, int RBLK, int TG, bool SHARED = false>
hipError_t launch_gqa_tg(const GqaArgs &a)
{
    using C = da::GqaTgCfg<D, RBLK, TG, kGqaTgNst>;
    auto kern = da::gqa_tg_kernel<D, RBLK, TG, kGqaTgNst, SHARED>;
    static std::once_flag attr_once;
    static hipError_t attr_err = hipSuccess;
    std::call_once(attr_once, [&] {
        attr_err = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS_BYTES);
    });
    if (attr_err != hipSuccess) return attr_err;
    const int units = a.workers * a.hkv * a.rsplit;
    const int grid = (units + 7) / 8 * 8;
    if (log_plan())
        fprintf(stderr, "[decode_attn] gqa-token-groups d=%d row blocks=%d row splits=%d workers=%d blocks=%d waves=%d lds=%d\n",
                D, RBLK, a.rsplit, a.workers, units, TG, C::LDS_BYTES);
    hipLaunchKernelGGL(kern, dim3(grid), dim3(64 * TG), C::LDS_BYTES, a.stream, a.q, a.k, a.v, a.seqlens, a.b, a.s,
                       a.hq, a.hkv, a.t_max, a.scale_log2, a.rsplit, units, a.hdr, a.tile_start, a.slot_start, a.out,
                       a.lse, a.part_out, a.part_lse);
    return hipSuccess;
}

template <int D, int RBLK>
hipError_t launch_gqa_tg_waves(int tg, const GqaArgs &a)
{
    // split rows (MQA): at most 32 rows per block, two row blocks
    if constexpr (RBLK == 2 && D <= 128)
        if (a.rsplit > 1)
            return tg == 4   ? launch_gqa_tg<D, RBLK, 4, true>(a)
                   : tg == 2 ? launch_gqa_tg<D, RBLK, 2, true>(a)
                             : launch_gqa_tg<D, RBLK, 1, true>(a);
    return tg == 4 ? launch_gqa_tg<D, RBLK, 4>(a) : tg == 2 ? launch_gqa_tg<D, RBLK, 2>(a) : launch_gqa_tg<D, RBLK, 1>(a);
}

hipError_t dispatch_gqa_tg(int d, int rows, int tg, const GqaArgs &a)
{
    const int nrb = (rows + 15) / 16;
    if (d == 64) {
        switch (nrb) {
        case 1: return launch_gqa_tg_waves<64, 1>(tg, a);
        case 2: return launch_gqa_tg_waves<64, 2>(tg, a);
        case 3: return launch_gqa_tg_waves<64, 3>(tg, a);
        case 4: return launch_gqa_tg_waves<64, 4>(tg, a);
        }
    } else if (d == 128) {
        switch (nrb) {
        case 1: return launch_gqa_tg_waves<128, 1>(tg, a);
        case 2: return launch_gqa_tg_waves<128, 2>(tg, a);
        case 3: return launch_gqa_tg_waves<128, 3>(tg, a);
        case 4: return launch_gqa_tg_waves<128, 4>(tg, a);
        }
    } else if (d == 256) {
        switch (nrb) {
        case 1: return launch_gqa_tg_waves<256, 1>(tg, a);
        case 2: return launch_gqa_tg_waves<256, 2>(tg, a);
        }
    }
    return hipErrorInvalidValue;  // not reached: gqa_tg_ok admits only these shapes
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

// Per-head projection launch (one block per 64 x BN tile).
template <int BN>
hipError_t launch_head_gemm(const uint16_t *a, const uint16_t *bw, uint16_t *c, int m, int h, int n, int k,
                            hipStream_t stream)
{
    using G = da::HeadGemmCfg<BN>;
    auto kern = da::head_gemm_lds_kernel<BN>;
    static std::once_flag attr_once;
    static hipError_t attr_err = hipSuccess;
    std::call_once(attr_once, [&] {
        attr_err = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, 2 * G::STAGE);
    });
    if (attr_err != hipSuccess) return attr_err;
    const int ntm = (m + G::BM - 1) / G::BM, ntn = (n + BN - 1) / BN;
    const int tiles = h * ntm * ntn;
    const int lds = (k > G::BK ? 2 : 1) * G::STAGE;  // a second stage buffer only for longer contractions
    hipLaunchKernelGGL(kern, dim3((tiles + 7) / 8 * 8), dim3(256), lds, stream, a, bw, c, m, h, n, k, ntm, ntn,
                       tiles);
    return hipSuccess;
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
    if (!q_lat || !q_rope || !cache || !seqlens || !out_lat || !lse) return DA_ERR_INVALID_ARG;
    if (!aligned16(q_lat) || !aligned16(q_rope) || !aligned16(cache) || !aligned16(out_lat))
        return DA_ERR_INVALID_ARG;
    if (((uintptr_t)workspace & 255u) != 0) return DA_ERR_INVALID_ARG;
    if (!std::isfinite(scale) || !(scale > 0.f)) return DA_ERR_INVALID_ARG;
    // a null workspace: one worker per sequence (one split), num_workers ignored
    const int workers = workspace ? mla_workers(b, s, h, t_max, num_workers) : b;
    const da::WsLayout ws = da::ws_layout(b, s * h, k, workers);
    if (workspace && workspace_bytes < ws.total) return DA_ERR_WORKSPACE;
    // When the library's own choice is one worker per sequence (the batch's row
    // blocks fill the device, e.g. s = 4 at b = 32, h = 128), full-length
    // sequences are never split, so the call runs in the per-sequence mode: the
    // same blocks, no plan arrays and no combine launch (an empty combine still
    // costs its dispatch, ~4 us).
    const bool per_seq = !workspace || (num_workers == 0 && workers == b);

    const float sl2 = scale * da::kLog2e;
    hipStream_t st_ = (hipStream_t)stream;
    char *wsp = per_seq ? nullptr : (char *)workspace;
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

da_status mla_decode_no_alloc(const uint16_t *q_lat, const uint16_t *q_rope, const uint16_t *cache,
                              const int32_t *seqlens, int b, int s, int h, int k, int p, int t_max, float scale,
                              uint16_t *out_lat, float *lse, int num_workers, void *stream)
{
    const da_status st = mla_check(b, s, h, k, p, t_max, num_workers);
    if (st != DA_OK) return st;
    // the plan and partials this call needs must fit the device scratch
    const size_t need = mla_decode_workspace_size(b, s, h, k, p, t_max, num_workers);
    if (need > (size_t)DA_NO_ALLOC_SCRATCH_BYTES) return DA_ERR_WORKSPACE;
    void *ws = current_scratch();
    if (ws == nullptr) return DA_ERR_HIP;
    // nothing in the scratch has to start at zero: the tile kernel writes the
    // plan on every call and the combine reads only the slots that plan lists
    return mla_decode(q_lat, q_rope, cache, seqlens, b, s, h, k, p, t_max, scale, out_lat, lse, ws,
                      (size_t)DA_NO_ALLOC_SCRATCH_BYTES, num_workers, stream);
}

static da_status gqa_check(int b, int s, int hq, int hkv, int d, int t_max, int num_workers, int path)
{
    if (b <= 0 || s <= 0 || hq <= 0 || hkv <= 0 || d <= 0 || t_max <= 0 || num_workers < 0) return DA_ERR_INVALID_ARG;
    if (hq % hkv != 0 || s > t_max) return DA_ERR_INVALID_ARG;
    if (path < 0 || path > 2) return DA_ERR_INVALID_ARG;
    if (!(d == 64 || d == 128 || d == 256)) return DA_ERR_UNSUPPORTED;
    const int rows = (hq / hkv) * s;
    if (gqa_choose_path(rows, path) == 0) {
        if (!gqa_valu_ok(rows)) return DA_ERR_UNSUPPORTED;
    } else if (rows > gqa_max_rows(d) || gqa_geom(d, hkv, rows).hpb == 0) {
        return DA_ERR_UNSUPPORTED;
    }
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
    if (!q || !k_cache || !v_cache || !seqlens || !out || !lse) return DA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out)) return DA_ERR_INVALID_ARG;
    if (((uintptr_t)workspace & 255u) != 0) return DA_ERR_INVALID_ARG;
    if (!std::isfinite(scale) || !(scale > 0.f)) return DA_ERR_INVALID_ARG;
    const int rows = (hq / hkv) * s;
    const int use_mfma = gqa_choose_path(rows, path);
    // a null workspace: one worker per sequence (one split), num_workers ignored.
    // The token-group kernel takes that mode where its shapes allow, and also
    // the automatic one when the batch gives every CU a (sequence, KV head).
    const bool tg = use_mfma && (workspace != nullptr && num_workers == 0 ? gqa_tg_auto(d, hkv, rows)
                                                                          : gqa_tg_ok(d, rows));
    const bool per_seq =
        workspace == nullptr || (tg && num_workers == 0 && (long)b * hkv >= current_cu_count());
    const int workers = per_seq ? b : gqa_workers(b, hkv, d, rows, path, t_max, num_workers);
    const da::WsLayout ws = da::ws_layout(b, s * hq, d, workers);
    if (!per_seq && workspace_bytes < ws.total) return DA_ERR_WORKSPACE;

    char *wsp = (char *)workspace;
    auto *hdr = per_seq ? nullptr : (da::PlanHeader *)(wsp + ws.header);
    int *tile_start = per_seq ? nullptr : (int *)(wsp + ws.tile_start);
    int *slot_start = per_seq ? nullptr : (int *)(wsp + ws.slot_start);
    float *part_lse = per_seq ? nullptr : (float *)(wsp + ws.part_lse);
    uint16_t *part_out = per_seq ? nullptr : (uint16_t *)(wsp + ws.part_out);
    hipStream_t st_ = (hipStream_t)stream;
    const float sl2 = scale * da::kLog2e;

    if (log_plan())
        fprintf(stderr, "[decode_attn] gqa d=%d b=%d s=%d hq=%d hkv=%d t_max=%d workers=%d path=%s\n", d, b, s, hq,
                hkv, t_max, workers, use_mfma ? "mfma" : "valu");
    bool ok = false;
    if (use_mfma) {
        const int rsplit = tg ? gqa_tg_rsplit(d, hkv, rows) : 1;
        const GqaArgs a{q, k_cache, v_cache, seqlens, b, s, hq, hkv, t_max, sl2, out, lse, hdr,
                        tile_start, slot_start, part_out, part_lse, workers, st_, rsplit};
        const GqaGeom g = gqa_geom(d, hkv, rows);
        const hipError_t e = tg ? dispatch_gqa_tg(d, (rows + rsplit - 1) / rsplit, gqa_tg_waves(workers * hkv, d), a)
                             : d == 64 ? dispatch_gqa_mfma<64>(g, a)
                             : d == 128 ? dispatch_gqa_mfma<128>(g, a)
                                        : dispatch_gqa_mfma<256>(g, a);
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
    if (per_seq)
        ;
    else if (d == 64)
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
    if (!q || !k_cache || !v_cache || !seqlens || !out || !lse) return DA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out)) return DA_ERR_INVALID_ARG;
    if (((uintptr_t)workspace & 255u) != 0) return DA_ERR_INVALID_ARG;
    if (!std::isfinite(scale) || !(scale > 0.f)) return DA_ERR_INVALID_ARG;
    // a null workspace: one worker per sequence (one split), num_workers ignored
    const bool per_seq = workspace == nullptr;
    const int workers = per_seq ? b : unabs_workers(b, h, t_max, num_workers);
    const da::WsLayout ws = da::ws_layout(b, s * h, dv, workers);
    if (!per_seq && workspace_bytes < ws.total) return DA_ERR_WORKSPACE;

    char *wsp = (char *)workspace;
    auto *hdr = per_seq ? nullptr : (da::PlanHeader *)(wsp + ws.header);
    int *tile_start = per_seq ? nullptr : (int *)(wsp + ws.tile_start);
    int *slot_start = per_seq ? nullptr : (int *)(wsp + ws.slot_start);
    float *part_lse = per_seq ? nullptr : (float *)(wsp + ws.part_lse);
    uint16_t *part_out = per_seq ? nullptr : (uint16_t *)(wsp + ws.part_out);
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
    if (!per_seq) launch_combine<kUnabsDV>(b, s * h, workers, hdr, slot_start, part_out, part_lse, out, lse, st_);
    return hipGetLastError() == hipSuccess ? DA_OK : DA_ERR_HIP;
}

// ------------------------------------------------------------------ per-head projections
static da_status head_gemm(const uint16_t *a, const uint16_t *bw, uint16_t *c, int m, int h, int n, int k,
                           void *stream)
{
    if (!a || !bw || !c || m <= 0 || h <= 0 || n <= 0 || k <= 0) return DA_ERR_INVALID_ARG;
    if (k % 32 != 0) return DA_ERR_UNSUPPORTED;
    if (!aligned16(a) || !aligned16(bw) || !aligned16(c)) return DA_ERR_INVALID_ARG;
    // a tile's 64 A rows, and its B rows, must be addressable by a 32-bit buffer offset;
    // the tile count must fit an int
    if ((long long)64 * h * k * 2 >= (1LL << 31) || (long long)128 * k * 2 >= (1LL << 31)) return DA_ERR_UNSUPPORTED;
    const long long t128 = (long long)h * ((m + 63) / 64) * ((n + 127) / 128);
    if (2 * t128 >= (1LL << 31)) return DA_ERR_UNSUPPORTED;
    // 128-column tiles when they give every CU two blocks, else 64-column ones (twice as many)
    const hipError_t e = t128 >= 2LL * current_cu_count()
                             ? launch_head_gemm<128>(a, bw, c, m, h, n, k, (hipStream_t)stream)
                             : launch_head_gemm<64>(a, bw, c, m, h, n, k, (hipStream_t)stream);
    if (e != hipSuccess) return DA_ERR_HIP;
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
