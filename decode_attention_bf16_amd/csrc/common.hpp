// Shared device helpers for the gfx950 decode-attention kernels: vector types,
// bf16 packing, MFMA and LDS-transpose wrappers, DPP reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace da {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;

#define DA_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Lazy softmax rescale: the running reference maximum is only moved when a new
// score exceeds it by more than this many powers of two, so unnormalized
// probabilities stay below 2^kRescaleSlack (harmless in fp32/bf16 range) and
// the accumulator is rarely rescaled.
constexpr float kRescaleSlack = 8.0f;

__device__ __forceinline__ f32x4 mfma16x16x32(const bf16x8 &a, const bf16x8 &b, const f32x4 &c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4 &v) { return __builtin_bit_cast(bf16x8, v); }

typedef __attribute__((ext_vector_type(2))) float f32x2v;

// Two floats -> one dword of two bf16 (round to nearest even), lo in bits 0..15
// (a single v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2v{lo, hi}, bf16x2));
}

__device__ __forceinline__ uint16_t to_bf16_bits(float f)
{
    __bf16 a = (__bf16)f;
    return __builtin_bit_cast(unsigned short, a);
}

__device__ __forceinline__ float bf16lo_to_f32(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16hi_to_f32(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c)
{
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c,
                                           false);
}

// LDS transpose read (ds_read_b64_tr_b16). Within each group of 16 lanes, lane
// j supplies the address of four consecutive 16-bit elements R[j][0..3]; lane i
// receives element e = R[4e + i/4][i%4], e = 0..3.
__device__ __forceinline__ i16x4 lds_read_tr16(const void *p)
{
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((DA_LDS i16x4 *)(p));
}

// DPP cross-lane moves within a row of 16 lanes.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}
constexpr int kDppRowMirror = 0x140;      // lane i <-> 15 - i within 16
constexpr int kDppRowHalfMirror = 0x141;  // lane i <-> 7 - i within 8
constexpr int kDppQuadXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppQuadXor1 = 0xB1;        // quad_perm [1,0,3,2]

// Sum over aligned groups of N lanes (N in {8, 16, 32}); every lane of the
// group receives the full sum. Uses mirror butterflies (each step pairs lanes
// whose partial sums are disjoint) so the order is fixed.
template <int N>
__device__ __forceinline__ float group_sum(float v)
{
    static_assert(N == 8 || N == 16 || N == 32, "group size");
    if constexpr (N == 32) v += __shfl_xor(v, 16);
    if constexpr (N >= 16) v += dpp_f<kDppRowMirror>(v);
    v += dpp_f<kDppRowHalfMirror>(v);
    v += dpp_f<kDppQuadXor2>(v);
    v += dpp_f<kDppQuadXor1>(v);
    return v;
}

// Reductions over lanes l, l^16, l^32 and l^48 with the gfx950 lane-swap
// instructions (VALU, no LDS round trip). v_permlane16_swap applied to (v, v)
// returns two values whose pair, on every lane, is {v[l], v[l^16]} (in one
// order or the other), and v_permlane32_swap likewise {v[l], v[l^32]}; a
// commutative combine of the pair is therefore identical on both lanes.
struct LanePair {
    float a, b;
};
// The element copies into scalars matter: with this compiler a bit cast applied
// directly to a subscripted vector element reads element 0.
__device__ __forceinline__ LanePair swap16_pair(float v)
{
    const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, v), __builtin_bit_cast(uint32_t, v),
                                                    false, false);
    const uint32_t r0 = r[0], r1 = r[1];
    return {__builtin_bit_cast(float, r0), __builtin_bit_cast(float, r1)};
}
__device__ __forceinline__ LanePair swap32_pair(float v)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, v), __builtin_bit_cast(uint32_t, v),
                                                    false, false);
    const uint32_t r0 = r[0], r1 = r[1];
    return {__builtin_bit_cast(float, r0), __builtin_bit_cast(float, r1)};
}

__device__ __forceinline__ float wave_max_across_groups16(float v)
{
    const LanePair x = swap16_pair(v);
    const LanePair y = swap32_pair(fmaxf(x.a, x.b));
    return fmaxf(y.a, y.b);
}

__device__ __forceinline__ float wave_sum_across_groups16(float v)
{
    const LanePair x = swap16_pair(v);
    const LanePair y = swap32_pair(x.a + x.b);
    return y.a + y.b;
}

// Workgroup barrier for LDS traffic only: waits for this wave's own LDS
// operations, then s_barrier. Unlike __syncthreads() it does not drain
// outstanding global loads (vmcnt), so HBM->LDS copies issued for later tiles
// stay in flight across it; kernels wait for those copies explicitly (vmcnt)
// before the barrier that publishes them. The "memory" clobber keeps the
// compiler from moving memory accesses across the barrier.
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Wait until at most N of this wave's vector memory operations are in flight
// (loads return in issue order, so this retires all but the N newest).
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// s_waitcnt vmcnt(0) issued through the builtin, so that the compiler's own
// wait tracking sees it (encoding: vmcnt 0, expcnt 7 and lgkmcnt 15 = no wait).
// Used right after a wave's register loads that precede a long loop of copies
// issued with lds_dma16: the compiler does not know about those copies, and
// without this it would re-wait for the loads, hence for every copy in flight,
// at each use of the loaded registers inside the loop.
__device__ __forceinline__ void wait_vm_loads_visible() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// s_waitcnt lgkmcnt(0) through the builtin (vmcnt 63 and expcnt 7 = no wait).
// Placed at the end of a rarely taken branch that issues scalar loads, so that
// the join after the branch does not inherit their pending count: otherwise
// the compiler waits there for everything lgkmcnt covers, including the LDS
// reads the wave issued just before.
__device__ __forceinline__ void wait_lgkm_visible() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Buffer resource for raw (unswizzled, stride 0) byte addressing of
// [base, base + num_bytes): accesses at offsets >= num_bytes read as zero.
__device__ __forceinline__ u32x4 raw_buffer_rsrc(const void *base, uint32_t num_bytes)
{
    const uint64_t a = (uint64_t)(uintptr_t)base;
    return u32x4{(uint32_t)a, (uint32_t)(a >> 32) & 0xffffu, num_bytes, 0x00020000u};
}

// HBM -> LDS copy of 16 bytes per lane (buffer_load_dwordx4 ... lds): lane i
// reads rsrc bytes [voffset, voffset + 16) and writes LDS bytes
// [lds_base + 16 i, + 16). The copy has no register results; its LDS writes
// are ordered by the caller with wait_vmcnt (loads retire in issue order)
// followed by a barrier. Written as inline assembly because the compiler,
// which cannot tell the copy's LDS destination apart from the buffers the
// wave reads meanwhile, would otherwise wait for every copy in flight before
// the wave's next LDS read and so undo the multi-buffering. M0 carries the LDS
// base (an input operand, so the compiler writes it and knows it is live); one
// wait state separates writing M0 from the copy that reads it.
__device__ __forceinline__ void lds_dma16(const u32x4 &rsrc, const DA_LDS void *lds_base, uint32_t voffset)
{
    const uint32_t m0 = (uint32_t)(uintptr_t)lds_base;
    asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                 :
                 : "v"(voffset), "s"(rsrc), "{m0}"(m0)
                 : "memory");
}

// The same copy with the non-temporal hint (nt), for data that exactly one
// block reads once: the lines are not kept in the caches for reuse, which
// leaves the L2 and the last-level cache to the rest of the stream. Data that
// several blocks read (an MLA tile shared by the row blocks of a worker) keeps
// the default policy.
__device__ __forceinline__ void lds_dma16_stream(const u32x4 &rsrc, const DA_LDS void *lds_base, uint32_t voffset)
{
    const uint32_t m0 = (uint32_t)(uintptr_t)lds_base;
    asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen nt lds"
                 :
                 : "v"(voffset), "s"(rsrc), "{m0}"(m0)
                 : "memory");
}

__device__ __forceinline__ int clamp_len(int len, int t_max)
{
    return len < 0 ? 0 : (len > t_max ? t_max : len);
}

// Round-robin XCD dispatch: block id bid runs on XCD bid % 8. Map it to a
// linear unit id so that consecutive units share an XCD (and its L2).
__device__ __forceinline__ int xcd_linear_unit(int bid, int grid)
{
    const int per_xcd = grid >> 3;  // grid is a multiple of 8
    return (bid & 7) * per_xcd + (bid >> 3);
}

}  // namespace da
