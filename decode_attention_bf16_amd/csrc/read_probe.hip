// Ceiling probes for the benchmark, built as their own library (the decode
// path never loads it):
//  - the HBM read rate one streaming read of a large buffer attains, the
//    practical ceiling of a kernel bound by reading the KV cache (a copy moves
//    as many bytes out as in; decode attention's traffic is almost all reads).
//    Every thread XOR-reduces 16-byte non-temporal loads over a grid-stride
//    range, U loads in flight per thread;
//  - the bf16 matrix rate at the clock the chip sustains under a full matrix
//    load: every wave runs independent chains of 32x32x16 bf16 MFMAs on
//    register operands, with no memory traffic.
// Each result is stored only when it equals a value no input produces in
// practice, which keeps the work alive.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

template <int U>
__global__ void __launch_bounds__(256) read_kernel(const u32x4 *__restrict__ p, long n16, unsigned *__restrict__ sink)
{
    u32x4 acc = {0u, 0u, 0u, 0u};
    const long stride = (long)gridDim.x * blockDim.x;
    long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
    for (; i + (U - 1) * stride < n16; i += U * stride) {
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= v[u];
    }
    for (; i < n16; i += stride) acc ^= __builtin_nontemporal_load(p + i);
    const unsigned r = acc.x ^ acc.y ^ acc.z ^ acc.w;
    if (r == 0x9e3779b9u) sink[blockIdx.x * blockDim.x + threadIdx.x] = r;
}

// CH independent accumulation chains per wave, `iters` rounds of one MFMA per chain.
template <int CH>
__global__ void __launch_bounds__(256) mfma_kernel(int iters, float *__restrict__ sink)
{
    bf16x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = (__bf16)(0.001f * (float)((threadIdx.x + i) & 7));
        b[i] = (__bf16)(0.001f * (float)((threadIdx.x * 3 + i) & 7));
    }
    f32x16 acc[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[c][e] = 0.f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int c = 0; c < CH; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
    }
    float r = 0.f;
#pragma unroll
    for (int c = 0; c < CH; ++c)
#pragma unroll
        for (int e = 0; e < 16; ++e) r += acc[c][e];
    if (r == -1234.5f) sink[blockIdx.x * blockDim.x + threadIdx.x] = r;
}

}  // namespace

// Runs `blocks` blocks of 256 threads, each wave `iters` rounds of four
// independent 32x32x16 bf16 MFMAs (32768 FLOP each): blocks * 4 * iters * 4 *
// 32768 FLOP in all. `sink` is device memory of at least blocks * 256 floats.
// Returns 0, or the HIP error of the launch.
extern "C" int da_probe_mfma(int blocks, int iters, float *sink, void *stream)
{
    if (!sink || blocks < 1 || iters < 1) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(mfma_kernel<4>, dim3(blocks), dim3(256), 0, (hipStream_t)stream, iters, sink);
    return (int)hipGetLastError();
}

// Reads `bytes` (a multiple of 16) at device pointer `p` once on `stream`
// with `blocks` blocks of 256 threads and `unroll` (2, 4 or 8) loads in flight
// per thread. `sink` is device memory of at least blocks * 256 unsigned ints.
// Returns 0, or the HIP error of the launch.
extern "C" int da_probe_read(const void *p, long bytes, unsigned *sink, int blocks, int unroll, void *stream)
{
    if (!p || !sink || bytes < 16 || blocks < 1) return (int)hipErrorInvalidValue;
    const long n16 = bytes / 16;
    hipStream_t s = (hipStream_t)stream;
    const u32x4 *src = (const u32x4 *)p;
    if (unroll == 8)
        hipLaunchKernelGGL(read_kernel<8>, dim3(blocks), dim3(256), 0, s, src, n16, sink);
    else if (unroll == 4)
        hipLaunchKernelGGL(read_kernel<4>, dim3(blocks), dim3(256), 0, s, src, n16, sink);
    else
        hipLaunchKernelGGL(read_kernel<2>, dim3(blocks), dim3(256), 0, s, src, n16, sink);
    return (int)hipGetLastError();
}
