// tri_probe.hip -- measurement aids: a streaming read and a plain copy of a byte range, an empty
// kernel, the decode kernel's loads alone, and a resident-grid streaming read.  The reads are
// size-matched floors for the weight stream of the decode kernels; the empty kernel is the fixed
// cost of a launch; the copy calibrates the hardware byte counters (bytes fetched / written per
// byte moved).
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

// An empty kernel: the fixed cost of a launch of `grid` workgroups of a given size, with
// nothing to read or write (the store never happens: threadIdx.x < 1024).
__global__ void k_probe_empty(uint32_t *sink)
{
    if (threadIdx.x == 0xFFFFu) sink[0] = 1u;
}

constexpr uint32_t kRsrcWord3 = 0x00020000u;   // raw buffer resource, gfx9 family

__device__ __forceinline__ __amdgpu_buffer_rsrc_t probe_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, (int)kRsrcWord3);
}

// The loads of the one-row decode kernel and nothing else: a workgroup of NW waves owns 16
// rows of an N x S byte matrix (S = 16 C), wave w reads, for its steps s < CST, chunk
// c = 4 (s NW + w) + g of row j (lane = 16 g + j), and its activation pieces of a K-wide fp16
// row as whole-line loads (piece P = 64 i + lane is piece P % PIECES of the wave's local chunk
// P / PIECES; PIECES = 8 for 64-trit chunks, 10 for 80-trit chunks).  The words loaded are
// folded into one value per lane, which is stored (to the 16-element row of outputs of the
// workgroup, by the first wave's first 16 lanes) so the loads stay live.
template <int XH, int NW, int CST>
__global__ __launch_bounds__(64 * NW) void k_probe_rows(const uint16_t *__restrict__ X, const uint8_t *__restrict__ Wp,
                                                        int N, int K, int C, uint16_t *__restrict__ Y)
{
    constexpr int NCH = 4 * CST;
    constexpr int PIECES = XH / 8;
    constexpr int NLD = (NCH * PIECES + 63) / 64;
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4, j = lane & 15;
    const int n0 = (int)blockIdx.x * 16;
    const int64_t S = (int64_t)C * 16;
    const __amdgpu_buffer_rsrc_t xr = probe_rsrc(X, __builtin_amdgcn_readfirstlane((uint32_t)K * 2u));
    u32x4 xv[NLD];
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
        const int P = 64 * i + lane;
        const int l = P / PIECES;
        const int gc = 4 * ((l >> 2) * NW + wv) + (l & 3);
        const int k = gc * XH + 8 * (P % PIECES);
        const int off = (l < NCH && k < K) ? (int)((uint32_t)k * 2u) : (int)0x80000000u;
        xv[i] = __builtin_amdgcn_raw_buffer_load_b128(xr, off, 0, 0);
    }
    const int rows_here = min(16, N - n0);
    const __amdgpu_buffer_rsrc_t wr =
        probe_rsrc(Wp + (int64_t)n0 * S, __builtin_amdgcn_readfirstlane((uint32_t)(rows_here * S)));
    u32x4 wq[CST];
#pragma unroll
    for (int s = 0; s < CST; ++s) {
        const int c = 4 * (s * NW + wv) + g;
        wq[s] = __builtin_amdgcn_raw_buffer_load_b128(wr, c < C ? (int)(uint32_t)(j * S + c * 16) : (int)0x80000000u,
                                                      0, 0);
    }
    uint32_t acc = 0;
#pragma unroll
    for (int i = 0; i < NLD; ++i) acc ^= xv[i][0] ^ xv[i][1] ^ xv[i][2] ^ xv[i][3];
#pragma unroll
    for (int s = 0; s < CST; ++s) acc += wq[s][0] ^ wq[s][1] ^ wq[s][2] ^ wq[s][3];
    if (wv == 0 && lane < 16 && n0 + lane < N) Y[n0 + lane] = (uint16_t)(acc ^ (acc >> 16));
    else if (acc == 0x9E3779B9u && lane == 0) Y[n0] = 0;   // (keeps every wave's loads live)
}

// A resident-grid read: `gridDim.x` workgroups of 256 threads stream the range in rounds of U
// 16-byte loads per lane, all U issued before any is used (each load instruction of a wave
// reads 1 KB of consecutive bytes).
template <int U>
__global__ __launch_bounds__(256) void k_probe_stream(const uint4 *__restrict__ p, int64_t n16, uint32_t *sink)
{
    const __amdgpu_buffer_rsrc_t r = probe_rsrc(p, (uint32_t)min(n16 * 16, (int64_t)0x7FFFFFF0));
    const int64_t step = (int64_t)gridDim.x * 256 * U;
    uint32_t acc = 0;
    for (int64_t base = (int64_t)blockIdx.x * 256 * U + threadIdx.x; base < n16; base += step) {
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = base + 256 * u;
            v[u] = __builtin_amdgcn_raw_buffer_load_b128(r, i < n16 ? (int)(uint32_t)(i * 16) : (int)0x80000000u, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    }
    if (acc == 0x9E3779B9u && threadIdx.x == 0x3FF) sink[0] = acc;   // never true for 256 threads
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

int launch_probe_empty(int64_t workgroups, int threads, uint32_t *sink, hipStream_t s)
{
    hipLaunchKernelGGL(k_probe_empty, dim3((unsigned)workgroups), dim3(threads), 0, s, sink);
    return hipGetLastError() == hipSuccess ? TRI_OK : TRI_EHIP;
}

template <int XH, int NW>
static int rows_cst(const uint16_t *X, const uint8_t *Wp, int N, int K, int C, uint16_t *Y, hipStream_t s)
{
    const int steps = (C + 4 * NW - 1) / (4 * NW);
    const dim3 grid((unsigned)((N + 15) / 16)), block(64 * NW);
    switch (steps) {
    case 1: hipLaunchKernelGGL((k_probe_rows<XH, NW, 1>), grid, block, 0, s, X, Wp, N, K, C, Y); break;
    case 2: hipLaunchKernelGGL((k_probe_rows<XH, NW, 2>), grid, block, 0, s, X, Wp, N, K, C, Y); break;
    case 3: hipLaunchKernelGGL((k_probe_rows<XH, NW, 3>), grid, block, 0, s, X, Wp, N, K, C, Y); break;
    case 4: hipLaunchKernelGGL((k_probe_rows<XH, NW, 4>), grid, block, 0, s, X, Wp, N, K, C, Y); break;
    case 5: hipLaunchKernelGGL((k_probe_rows<XH, NW, 5>), grid, block, 0, s, X, Wp, N, K, C, Y); break;
    case 6: hipLaunchKernelGGL((k_probe_rows<XH, NW, 6>), grid, block, 0, s, X, Wp, N, K, C, Y); break;
    case 7: hipLaunchKernelGGL((k_probe_rows<XH, NW, 7>), grid, block, 0, s, X, Wp, N, K, C, Y); break;
    case 8: hipLaunchKernelGGL((k_probe_rows<XH, NW, 8>), grid, block, 0, s, X, Wp, N, K, C, Y); break;
    default: return TRI_EINVAL;
    }
    return hipGetLastError() == hipSuccess ? TRI_OK : TRI_EHIP;
}

int launch_probe_rows(const uint16_t *X, const uint8_t *Wp, int N, int K, int fmt, int waves, uint16_t *Y,
                      hipStream_t s)
{
    const int C = (int)(row_bytes(K, fmt) / 16);
    if (fmt == TRI_FMT_2BIT) return waves == 8 ? rows_cst<64, 8>(X, Wp, N, K, C, Y, s) : rows_cst<64, 4>(X, Wp, N, K, C, Y, s);
    return waves == 8 ? rows_cst<80, 8>(X, Wp, N, K, C, Y, s) : rows_cst<80, 4>(X, Wp, N, K, C, Y, s);
}

int launch_probe_stream(const void *src, int64_t bytes, int workgroups, int unroll, uint32_t *sink, hipStream_t s)
{
    const int64_t n16 = bytes / 16;
    const dim3 grid((unsigned)workgroups), block(256);
    const uint4 *p = (const uint4 *)src;
    switch (unroll) {
    case 1: hipLaunchKernelGGL(k_probe_stream<1>, grid, block, 0, s, p, n16, sink); break;
    case 2: hipLaunchKernelGGL(k_probe_stream<2>, grid, block, 0, s, p, n16, sink); break;
    case 4: hipLaunchKernelGGL(k_probe_stream<4>, grid, block, 0, s, p, n16, sink); break;
    case 8: hipLaunchKernelGGL(k_probe_stream<8>, grid, block, 0, s, p, n16, sink); break;
    default: return TRI_EINVAL;
    }
    return hipGetLastError() == hipSuccess ? TRI_OK : TRI_EHIP;
}

}  // namespace tri
