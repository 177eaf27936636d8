// tri_probe.hip -- measurement aids: a streaming read and a plain copy of a byte range.
// The read is the size-matched floor for the weight stream of the GEMV kernels; the copy
// calibrates the hardware byte counters (bytes fetched / written per byte moved).
#include "tri_device.h"
#include "tri_internal.h"

namespace tri {

__global__ __launch_bounds__(256) void k_probe_read(const uint4 *__restrict__ p, int64_t n16, uint32_t *sink)
{
    uint32_t acc = 0;
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n16; i += (int64_t)gridDim.x * blockDim.x) {
        const uint4 v = p[i];
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    if (acc == 0x9E3779B9u && threadIdx.x == 0x3FF) sink[0] = acc;   // never true for blockDim 256
}

__global__ __launch_bounds__(256) void k_probe_copy(const uint4 *__restrict__ src, uint4 *__restrict__ dst, int64_t n16)
{
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n16; i += (int64_t)gridDim.x * blockDim.x)
        dst[i] = src[i];
}

static unsigned blocks_for(int64_t n16)
{
    int64_t b = (n16 + 255) / 256;   // one 16-byte load per thread when it fits
    if (b > (int64_t)1 << 20) b = (int64_t)1 << 20;
    return (unsigned)(b < 1 ? 1 : b);
}

int launch_probe_read(const void *src, int64_t bytes, uint32_t *sink, hipStream_t s)
{
    const int64_t n16 = bytes / 16;
    hipLaunchKernelGGL(k_probe_read, dim3(blocks_for(n16)), dim3(256), 0, s, (const uint4 *)src, n16, sink);
    return hipGetLastError() == hipSuccess ? TRI_OK : TRI_EHIP;
}

int launch_probe_copy(const void *src, void *dst, int64_t bytes, hipStream_t s)
{
    const int64_t n16 = bytes / 16;
    hipLaunchKernelGGL(k_probe_copy, dim3(blocks_for(n16)), dim3(256), 0, s, (const uint4 *)src, (uint4 *)dst, n16);
    return hipGetLastError() == hipSuccess ? TRI_OK : TRI_EHIP;
}

}  // namespace tri
