// Streaming-bandwidth probe used by the benchmark to state the practical HBM
// ceiling next to the RMSNorm kernels: a copy (one read and one write stream)
// and a three-stream kernel (two reads, one write) over 16-byte elements,
// grid-stride, nontemporal.  Built as its own library; not part of the
// RMSNorm C ABI.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

template <int U>
__global__ void __launch_bounds__(256) copy_kernel(const u32x4_t *__restrict__ a, u32x4_t *__restrict__ c, int64_t n)
{
    const int64_t stride = (int64_t)gridDim.x * 256 * U;
    for (int64_t base = (int64_t)blockIdx.x * 256 * U + threadIdx.x; base < n; base += stride) {
        u32x4_t v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = base + (int64_t)u * 256;
            if (i < n)
                v[u] = __builtin_nontemporal_load(a + i);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = base + (int64_t)u * 256;
            if (i < n)
                __builtin_nontemporal_store(v[u], c + i);
        }
    }
}

template <int U>
__global__ void __launch_bounds__(256) three_stream_kernel(const u32x4_t *__restrict__ a, const u32x4_t *__restrict__ b,
                                                           u32x4_t *__restrict__ c, int64_t n)
{
    const int64_t stride = (int64_t)gridDim.x * 256 * U;
    for (int64_t base = (int64_t)blockIdx.x * 256 * U + threadIdx.x; base < n; base += stride) {
        u32x4_t v[U], w[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = base + (int64_t)u * 256;
            if (i < n) {
                v[u] = __builtin_nontemporal_load(a + i);
                w[u] = __builtin_nontemporal_load(b + i);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = base + (int64_t)u * 256;
            if (i < n)
                __builtin_nontemporal_store(v[u] ^ w[u], c + i);
        }
    }
}

} // namespace

// n16: number of 16-byte elements; unroll in {1, 2, 4}; returns a hipError_t.
extern "C" int stream_probe_copy(const void *a, void *c, int64_t n16, int blocks, int unroll, hipStream_t s)
{
    const dim3 g((unsigned)blocks), b(256);
    const u32x4_t *pa = static_cast<const u32x4_t *>(a);
    u32x4_t *pc = static_cast<u32x4_t *>(c);
    if (unroll == 1)
        hipLaunchKernelGGL((copy_kernel<1>), g, b, 0, s, pa, pc, n16);
    else if (unroll == 2)
        hipLaunchKernelGGL((copy_kernel<2>), g, b, 0, s, pa, pc, n16);
    else if (unroll == 4)
        hipLaunchKernelGGL((copy_kernel<4>), g, b, 0, s, pa, pc, n16);
    else
        return (int)hipErrorInvalidValue;
    return (int)hipGetLastError();
}

extern "C" int stream_probe_three(const void *a, const void *b, void *c, int64_t n16, int blocks, int unroll,
                                  hipStream_t s)
{
    const dim3 g((unsigned)blocks), bl(256);
    const u32x4_t *pa = static_cast<const u32x4_t *>(a);
    const u32x4_t *pb = static_cast<const u32x4_t *>(b);
    u32x4_t *pc = static_cast<u32x4_t *>(c);
    if (unroll == 1)
        hipLaunchKernelGGL((three_stream_kernel<1>), g, bl, 0, s, pa, pb, pc, n16);
    else if (unroll == 2)
        hipLaunchKernelGGL((three_stream_kernel<2>), g, bl, 0, s, pa, pb, pc, n16);
    else if (unroll == 4)
        hipLaunchKernelGGL((three_stream_kernel<4>), g, bl, 0, s, pa, pb, pc, n16);
    else
        return (int)hipErrorInvalidValue;
    return (int)hipGetLastError();
}
