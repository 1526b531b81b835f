// HBM read-rate probe for the benchmark: the rate one streaming read of a
// large buffer attains on this GPU, the practical ceiling of a kernel bound by
// reading the KV cache (a copy moves as many bytes out as in; decode
// attention's traffic is almost all reads). Built as its own library; the
// decode path never loads it.
//
// Every thread XOR-reduces 16-byte non-temporal loads over a grid-stride
// range, U loads in flight per thread; the result is stored only when it
// equals a value no input produces in practice, which keeps the loads alive.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

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

}  // namespace

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
