// tri_pack.hip -- packing and unpacking kernels of the two ternary weight formats.
//
// Formats (Pith review of "Spectra 1.1", sections "Core claim" and "What carries the
// argument"): 2-bit = base-4 digits, 4 trits per byte; 1.6-bit = base-3 digits,
// 5 trits per byte (3^5 = 243 < 256).  Digit of a trit t is t + 1; the lowest k is the
// least-significant digit; rows are padded with zero trits to 16-byte multiples.
// The unpack direction follows the repeated-division decode b'_i -> x_i that the
// review's referee report describes for the paper's section 3.2, extended to every byte.
#include "tri_device.h"
#include "tri_internal.h"

namespace tri {

__device__ __forceinline__ uint32_t digit_of(int8_t w) { return w > 0 ? 2u : (w < 0 ? 0u : 1u); }

// One thread per packed byte.
template <int FMT>
__global__ __launch_bounds__(256) void k_pack(const int8_t *__restrict__ W, int64_t N, int64_t K, int64_t S,
                                              uint8_t *__restrict__ Wp)
{
    constexpr int TPB = FMT == TRI_FMT_2BIT ? 4 : 5;   // trits per byte
    const int64_t total = N * S;
    for (int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int64_t n = idx / S;
        const int64_t b = idx - n * S;
        const int8_t *row = W + n * K;
        uint32_t value = 0;
#pragma unroll
        for (int j = TPB - 1; j >= 0; --j) {
            const int64_t k = b * TPB + j;
            const uint32_t d = (k < K) ? digit_of(row[k]) : 1u;
            value = value * (FMT == TRI_FMT_2BIT ? 4u : 3u) + d;
        }
        Wp[idx] = (uint8_t)value;
    }
}

// One thread per packed byte; writes the byte's trits that fall below K.
template <int FMT>
__global__ __launch_bounds__(256) void k_unpack(const uint8_t *__restrict__ Wp, int64_t N, int64_t K, int64_t S,
                                                int8_t *__restrict__ W)
{
    constexpr int TPB = FMT == TRI_FMT_2BIT ? 4 : 5;
    const int64_t total = N * S;
    for (int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int64_t n = idx / S;
        const int64_t b = idx - n * S;
        uint32_t v = Wp[idx];
        int8_t *row = W + n * K;
#pragma unroll
        for (int j = 0; j < TPB; ++j) {
            int t;
            if (FMT == TRI_FMT_2BIT) {
                const uint32_t code = (v >> (2 * j)) & 3u;
                t = code == 3u ? 0 : (int)code - 1;
            } else {
                const uint32_t q = v / 3u;            // b'_{j+1}
                t = (int)(v - 3u * q) - 1;            // x_j - 1 with x_j = b'_j mod 3
                v = q;
            }
            const int64_t k = b * TPB + j;
            if (k < K) row[k] = (int8_t)t;
        }
    }
}

static unsigned grid_for(int64_t items)
{
    int64_t blocks = (items + 255) / 256;
    if (blocks > 65536) blocks = 65536;   // grid-stride loops cover the rest
    return (unsigned)(blocks < 1 ? 1 : blocks);
}

int launch_pack(const int8_t *W, int64_t N, int64_t K, int fmt, uint8_t *Wp, hipStream_t s)
{
    const int64_t S = row_bytes(K, fmt);
    if (fmt == TRI_FMT_2BIT)
        hipLaunchKernelGGL(k_pack<TRI_FMT_2BIT>, dim3(grid_for(N * S)), dim3(256), 0, s, W, N, K, S, Wp);
    else
        hipLaunchKernelGGL(k_pack<TRI_FMT_1P6BIT>, dim3(grid_for(N * S)), dim3(256), 0, s, W, N, K, S, Wp);
    return hipGetLastError() == hipSuccess ? TRI_OK : TRI_EHIP;
}

int launch_unpack(const uint8_t *Wp, int64_t N, int64_t K, int fmt, int8_t *W, hipStream_t s)
{
    const int64_t S = row_bytes(K, fmt);
    if (fmt == TRI_FMT_2BIT)
        hipLaunchKernelGGL(k_unpack<TRI_FMT_2BIT>, dim3(grid_for(N * S)), dim3(256), 0, s, Wp, N, K, S, W);
    else
        hipLaunchKernelGGL(k_unpack<TRI_FMT_1P6BIT>, dim3(grid_for(N * S)), dim3(256), 0, s, Wp, N, K, S, W);
    return hipGetLastError() == hipSuccess ? TRI_OK : TRI_EHIP;
}

}  // namespace tri
