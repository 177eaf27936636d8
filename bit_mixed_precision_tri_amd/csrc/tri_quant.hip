// tri_quant.hip -- quantisation of latent float32 weights to trits and one scale, packed.
//
// A ternary linear layer keeps latent full-precision weights and rounds them on the fly to
// {-1, 0, +1} times one shared scale (Pith review of "Spectra 1.1", "What carries the
// argument"; the review's domain assumptions name the rounding as round-to-nearest).  The
// pages leave the scale rule open; the one taken here is the mean absolute value of the
// matrix:
//   scale = float32( sum_{n,k} |w| / (N*K) ),  summed in float64;
//   t     = round_half_even(w / scale) clipped to [-1, 1], and 0 when scale == 0.
// For scale > 0 the rounding reduces to one exact comparison: |w / scale| > 1/2, i.e.
// 2|w| > scale (both sides exact in float32), gives sign(w); anything else, the tie
// included, gives 0.  No division is evaluated.
//
// Three launches on the caller's stream:
//   k_absmean_part   each workgroup sums |w| over a fixed contiguous range in float64 and
//                    writes one partial sum to the workspace (fixed order, no atomics);
//   k_absmean_final  one workgroup adds the partial sums in a fixed order and writes the
//                    float32 scale to device memory;
//   k_quant_pack*    reads the scale, decides the trits and writes the packed bytes in the
//                    layout of tri_pack2 / tri_pack16 (digit t+1, lowest k least significant,
//                    rows padded with zero trits to whole 16-byte chunks): with 16-byte weight
//                    loads when K % 4 == 0 (one byte per thread for 2-bit, four for 1.6-bit),
//                    else one thread per byte with single loads.
// The result is deterministic: the same input gives the same scale and bytes on every run.
#include "tri_device.h"
#include "tri_internal.h"

namespace tri {

namespace {

constexpr int kThreads = 256;
constexpr int64_t kQuad = 4 * kThreads;          // floats one workgroup pass reads
constexpr int64_t kMaxParts = 2048;

// Elements per partial sum: a multiple of kQuad, so every range starts 16-byte aligned.
int64_t part_elems(int64_t E)
{
    int64_t per = (E + kMaxParts - 1) / kMaxParts;
    per = (per + kQuad - 1) / kQuad * kQuad;
    return per;
}

__device__ __forceinline__ double block_sum(double v, double *red)
{
    const int t = threadIdx.x;
    red[t] = v;
    __syncthreads();
#pragma unroll
    for (int st = kThreads / 2; st > 0; st >>= 1) {
        if (t < st) red[t] += red[t + st];
        __syncthreads();
    }
    return red[0];
}

}  // namespace

int64_t quant_workspace_bytes(int64_t E)
{
    const int64_t per = part_elems(E);
    return 8 * ((E + per - 1) / per);
}

__global__ __launch_bounds__(kThreads) void k_absmean_part(const float *__restrict__ W, int64_t E, int64_t per,
                                                           double *__restrict__ part)
{
    __shared__ double red[kThreads];
    const int64_t begin = (int64_t)blockIdx.x * per;
    const int64_t end = min(E, begin + per);
    const float4 *__restrict__ q = reinterpret_cast<const float4 *>(W);
    double acc = 0.0;
    int64_t i = begin + 4 * (int64_t)threadIdx.x;
#pragma unroll 4
    for (; i + 3 < end; i += kQuad) {
        const float4 v = q[i >> 2];
        acc += (double)fabsf(v.x) + (double)fabsf(v.y) + (double)fabsf(v.z) + (double)fabsf(v.w);
    }
    for (; i < end; ++i) acc += (double)fabsf(W[i]);   // the last 1..3 floats of the matrix
    const double s = block_sum(acc, red);
    if (threadIdx.x == 0) part[blockIdx.x] = s;
}

__global__ __launch_bounds__(kThreads) void k_absmean_final(const double *__restrict__ part, int P, int64_t E,
                                                            float *__restrict__ scale)
{
    __shared__ double red[kThreads];
    double acc = 0.0;
    for (int i = threadIdx.x; i < P; i += kThreads) acc += part[i];
    const double s = block_sum(acc, red);
    if (threadIdx.x == 0) scale[0] = (float)(s / (double)E);
}

template <int FMT>
__global__ __launch_bounds__(kThreads) void k_quant_pack(const float *__restrict__ W, int64_t N, int64_t K, int64_t S,
                                                         const float *__restrict__ scale, uint8_t *__restrict__ Wp)
{
    constexpr int TPB = FMT == TRI_FMT_2BIT ? 4 : 5;   // trits per byte
    constexpr uint32_t RADIX = FMT == TRI_FMT_2BIT ? 4u : 3u;
    const float g = scale[0];
    const int64_t total = N * S;
    for (int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int64_t n = idx / S;
        const int64_t b = idx - n * S;
        const float *row = W + n * K;
        uint32_t value = 0;
#pragma unroll
        for (int j = TPB - 1; j >= 0; --j) {
            const int64_t k = b * TPB + j;
            uint32_t d = 1u;                             // zero trit (also the row padding)
            if (k < K) {
                const float w = row[k];
                if (g > 0.f && 2.f * fabsf(w) > g) d = w > 0.f ? 2u : 0u;
            }
            value = value * RADIX + d;
        }
        Wp[idx] = (uint8_t)value;
    }
}

// The same with whole 16-byte weight loads, for K % 4 == 0 (every row starts 16-byte aligned):
// 2-bit, one thread per packed byte and one load per byte; 1.6-bit, one thread per four packed
// bytes (20 weights, five loads) written as one 32-bit word (a row's bytes are a multiple of 16,
// so a group never straddles two rows).
__device__ __forceinline__ uint32_t digit_of_weight(float w, float g)
{
    return (g > 0.f && 2.f * fabsf(w) > g) ? (w > 0.f ? 2u : 0u) : 1u;
}

__global__ __launch_bounds__(kThreads) void k_quant_pack2_v(const float *__restrict__ W, int64_t N, int64_t K,
                                                            int64_t S, const float *__restrict__ scale,
                                                            uint8_t *__restrict__ Wp)
{
    const float g = scale[0];
    const int64_t total = N * S;
    for (int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int64_t n = idx / S;
        const int64_t b = idx - n * S;
        uint32_t value = 1u | (1u << 2) | (1u << 4) | (1u << 6);   // four zero trits (row padding)
        if (4 * b < K) {
            const float4 v = *reinterpret_cast<const float4 *>(W + n * K + 4 * b);
            value = digit_of_weight(v.x, g) | (digit_of_weight(v.y, g) << 2) | (digit_of_weight(v.z, g) << 4) |
                    (digit_of_weight(v.w, g) << 6);
        }
        Wp[idx] = (uint8_t)value;
    }
}

__global__ __launch_bounds__(kThreads) void k_quant_pack16_v(const float *__restrict__ W, int64_t N, int64_t K,
                                                             int64_t S, const float *__restrict__ scale,
                                                             uint8_t *__restrict__ Wp)
{
    const float g = scale[0];
    const int64_t S4 = S / 4;
    const int64_t total = N * S4;
    for (int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int64_t n = idx / S4;
        const int64_t b0 = 4 * (idx - n * S4);      // first of the four bytes
        const int64_t k0 = 5 * b0;                  // its first trit
        float w[20];
        if (k0 + 20 <= K) {
            const float4 *q = reinterpret_cast<const float4 *>(W + n * K + k0);
#pragma unroll
            for (int i = 0; i < 5; ++i) {
                const float4 v = q[i];
                w[4 * i] = v.x; w[4 * i + 1] = v.y; w[4 * i + 2] = v.z; w[4 * i + 3] = v.w;
            }
        } else {
#pragma unroll
            for (int i = 0; i < 20; ++i) w[i] = (k0 + i < K) ? W[n * K + k0 + i] : 0.f;   // past K: zero trits
        }
        uint32_t word = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            uint32_t value = 0;
#pragma unroll
            for (int j = 4; j >= 0; --j) value = value * 3u + digit_of_weight(w[5 * q + j], g);
            word |= value << (8 * q);
        }
        *reinterpret_cast<uint32_t *>(Wp + n * S + b0) = word;
    }
}

// The partial sums of tri_quantize_noalloc: a file-scope device array (each device holds its own
// copy at its own address until the process ends).  In host code `scratch` names a host-side
// stand-in, never the device memory: kernels receive the address hipGetSymbolAddress returns.
static __device__ __align__(256) double scratch[kMaxParts];

static_assert(sizeof(scratch) == TRI_QUANTIZE_SCRATCH_BYTES, "the scratch size the header states");

int64_t quant_scratch_bytes() { return (int64_t)sizeof(scratch); }

void *quant_scratch()
{
    static std::atomic<void *> addr[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return nullptr;
    if (dev >= 0 && dev < kMaxDevices) {
        void *p = addr[dev].load(std::memory_order_acquire);
        if (p) return p;
    }
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    if (dev >= 0 && dev < kMaxDevices) addr[dev].store(p, std::memory_order_release);
    return p;
}

int launch_quantize(const float *W, int64_t N, int64_t K, int fmt, uint8_t *Wp, float *scale, void *workspace,
                    hipStream_t s)
{
    const int64_t E = N * K;
    const int64_t per = part_elems(E);
    const int P = (int)((E + per - 1) / per);
    double *part = static_cast<double *>(workspace);
    hipLaunchKernelGGL(k_absmean_part, dim3(P), dim3(kThreads), 0, s, W, E, per, part);
    hipLaunchKernelGGL(k_absmean_final, dim3(1), dim3(kThreads), 0, s, part, P, E, scale);
    const int64_t S = row_bytes(K, fmt);
    if (K % 4 == 0) {                                    // 16-byte aligned rows: vector loads
        const int64_t items = fmt == TRI_FMT_2BIT ? N * S : N * S / 4;
        int64_t vb = (items + kThreads - 1) / kThreads;
        if (vb > 65536) vb = 65536;                      // grid-stride loop covers the rest
        if (fmt == TRI_FMT_2BIT)
            hipLaunchKernelGGL(k_quant_pack2_v, dim3((unsigned)vb), dim3(kThreads), 0, s, W, N, K, S, scale, Wp);
        else
            hipLaunchKernelGGL(k_quant_pack16_v, dim3((unsigned)vb), dim3(kThreads), 0, s, W, N, K, S, scale, Wp);
        return hipGetLastError() == hipSuccess ? TRI_OK : TRI_EHIP;
    }
    int64_t blocks = (N * S + kThreads - 1) / kThreads;
    if (blocks > 65536) blocks = 65536;                  // grid-stride loop covers the rest
    if (fmt == TRI_FMT_2BIT)
        hipLaunchKernelGGL(k_quant_pack<TRI_FMT_2BIT>, dim3((unsigned)blocks), dim3(kThreads), 0, s, W, N, K, S, scale,
                           Wp);
    else
        hipLaunchKernelGGL(k_quant_pack<TRI_FMT_1P6BIT>, dim3((unsigned)blocks), dim3(kThreads), 0, s, W, N, K, S,
                           scale, Wp);
    return hipGetLastError() == hipSuccess ? TRI_OK : TRI_EHIP;
}

}  // namespace tri
