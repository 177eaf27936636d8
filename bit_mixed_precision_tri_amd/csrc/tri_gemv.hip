// tri_gemv.hip -- ternary GEMV for one activation row (M = 1), 2-bit weights, on the VALU.
//
// The layer (Pith review of "Spectra 1.1", "What carries the argument"):
//   y[n] = scale * sum_k t[n][k] * x[k],  t in {-1, 0, +1},  fp32 accumulation.
//
// Decode.  A 32-bit word of a 2-bit row holds 16 trits; trit 16w+p sits in bits 2p..2p+1
// (p < 8) and trit 16w+8+p in bits 16+2p..17+2p.  Masking the word with 0x00030003<<2p
// leaves the digit pair (d = t + 1) of trits (p, p+8) in place.  Read as two fp16 values
// the masked bits are d * 4^p * 2^-24 exactly: subnormals for 2p+1 <= 9, and for p = 5 the
// two lowest exponent bits, which still encode d * 2^10 * 2^-24 for d <= 2.  Positions 6
// and 7 are shifted down by 12 bits first.  v_dot2_f32_f16 multiplies such a pair with the
// matching activation pair (x[p], x[p+8]) exactly and adds in fp32, so one AND plus one
// dot2 handles two trits.  Each position class keeps its own fp32 accumulator.  Since
// t = d - 1, the same class sums of an all-zero-trit chunk (every digit 1) are subtracted
// class by class; then the classes are merged with exact power-of-two weights.
//
// Work split.  A workgroup is 4 waves; wave w owns RB consecutive rows and the whole K
// range of them.  Lane l owns 16-byte chunk l (64 trits) of every 64-chunk pass, so one
// load instruction reads 1 KB of one row, fully coalesced, and every weight byte of the
// wave is requested before any arithmetic waits on it.  The workgroup first stages the
// activations of PM passes in LDS, already permuted into (x[p], x[p+8]) pairs (loaded
// before the weights, so the staging overlaps the weight latency); each lane then reads
// its 64 activations from LDS once per pass and reuses them for its RB rows.  The RB
// per-lane partial sums are reduced across the wave with permlane swaps and DPP moves
// (no LDS, fixed order, no atomics).
#include "tri_device.h"
#include "tri_internal.h"

namespace tri {

// The 64 activations of one chunk (xr[q] = (x[2q], x[2q+1])), permuted into
// xp[8w+p] = (x[16w+p], x[16w+8+p]), the pairing of the masked weight words.
__device__ __forceinline__ void permute_x_chunk64(const uint32_t (&xr)[32], uint32_t (&xp)[32])
{
#pragma unroll
    for (int w = 0; w < 4; ++w) {
#pragma unroll
        for (int p = 0; p < 8; p += 2) {
            xp[8 * w + p] = pair_halves<0>(xr[8 * w + 4 + p / 2], xr[8 * w + p / 2]);
            xp[8 * w + p + 1] = pair_halves<1>(xr[8 * w + 4 + p / 2], xr[8 * w + p / 2]);
        }
    }
}

// Per position class c: sum over the chunk of d * x * 4^c * 2^-24, accumulated in a fixed order.
__device__ __forceinline__ void chunk_class_sums(const uint4 wv, const uint32_t (&xp)[32], float (&a)[6])
{
    const uint32_t words[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
    for (int c = 0; c < 6; ++c) a[c] = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const uint32_t v = words[w];
        const uint32_t u = v >> 12;
        a[0] = dot2(v & 0x00030003u, xp[8 * w + 0], a[0]);
        a[1] = dot2(v & 0x000C000Cu, xp[8 * w + 1], a[1]);
        a[2] = dot2(v & 0x00300030u, xp[8 * w + 2], a[2]);
        a[3] = dot2(v & 0x00C000C0u, xp[8 * w + 3], a[3]);
        a[4] = dot2(v & 0x03000300u, xp[8 * w + 4], a[4]);
        a[5] = dot2(v & 0x0C000C00u, xp[8 * w + 5], a[5]);
        a[0] = dot2(u & 0x00030003u, xp[8 * w + 6], a[0]);
        a[1] = dot2(u & 0x000C000Cu, xp[8 * w + 7], a[1]);
    }
}

// sum_k t_k * x_k * 2^-24 over one chunk: the class sums of the weights minus the class sums of
// an all-zero-trit chunk (every digit 1, bytes 0x55), evaluated by the same instruction
// sequence.  Where the weights are all zero the two agree bit for bit and cancel exactly.
__device__ __forceinline__ float chunk_dot_t(const uint4 wv, const uint32_t (&xp)[32], const float (&z)[6])
{
    float a[6];
    chunk_class_sums(wv, xp, a);
    return ((a[0] - z[0]) + 0.25f * (a[1] - z[1])) + (0.0625f * (a[2] - z[2]) + 0.015625f * (a[3] - z[3])) +
           (0.00390625f * (a[4] - z[4]) + 0.0009765625f * (a[5] - z[5]));
}

constexpr int kXSlot = 36;   // LDS dwords per staged chunk: 32 used, padded against bank conflicts

template <int RB, int PM>
__global__ __launch_bounds__(256) void k_gemv2(const uint16_t *__restrict__ X, const uint8_t *__restrict__ Wp,
                                               float scale, int N, int K, int C, uint16_t *__restrict__ Y)
{
    __shared__ __attribute__((aligned(16))) uint32_t xs[PM * 64 * kXSlot];
    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    const int row0 = (blockIdx.x * 4 + wv) * RB;
    const int64_t S = (int64_t)C * 16;
    const bool xvec = (K % 8) == 0;

    float acc[RB];
#pragma unroll
    for (int r = 0; r < RB; ++r) acc[r] = 0.f;

    for (int g0 = 0; g0 < C; g0 += 64 * PM) {   // groups of PM passes of 64 chunks; one group unless K is large
        // (a) activations of this group, one (chunk, 16-value word group) item per thread and pass;
        //     issued first so that their staging does not wait on the weights
        uint32_t xr[PM][8];
#pragma unroll
        for (int p = 0; p < PM; ++p) {
            const int item = p * 256 + threadIdx.x;
            const int chunk = g0 + (item >> 2);
            const int k0 = chunk * 64 + 16 * (item & 3);
            if (chunk < C) {
                load_x_span<16>(X, k0, K, xvec, xr[p]);
            } else {
#pragma unroll
                for (int q = 0; q < 8; ++q) xr[p][q] = 0u;
            }
        }
        // (b) weights: every 16-byte chunk of this wave's RB rows in the group, all in flight at once
        uint4 wq[PM][RB];
#pragma unroll
        for (int p = 0; p < PM; ++p) {
            const int chunk = g0 + 64 * p + lane;
#pragma unroll
            for (int r = 0; r < RB; ++r) {
                const int row = min(row0 + r, N - 1);   // rows past N repeat the last one; never stored
                wq[p][r] = chunk < C ? ld16(Wp + row * S + (int64_t)chunk * 16) : make_uint4(0, 0, 0, 0);
            }
        }
        // (c) stage the activations in LDS, permuted into the pairing of the masked weight words
        if (g0 > 0) __syncthreads();               // the previous group is no longer being read
#pragma unroll
        for (int p = 0; p < PM; ++p) {
            const int item = p * 256 + threadIdx.x;
            const int w = item & 3;
            uint32_t *dst = xs + (item >> 2) * kXSlot + 8 * w;
            uint4 lo, hi;
            lo.x = pair_halves<0>(xr[p][4], xr[p][0]); lo.y = pair_halves<1>(xr[p][4], xr[p][0]);
            lo.z = pair_halves<0>(xr[p][5], xr[p][1]); lo.w = pair_halves<1>(xr[p][5], xr[p][1]);
            hi.x = pair_halves<0>(xr[p][6], xr[p][2]); hi.y = pair_halves<1>(xr[p][6], xr[p][2]);
            hi.z = pair_halves<0>(xr[p][7], xr[p][3]); hi.w = pair_halves<1>(xr[p][7], xr[p][3]);
            reinterpret_cast<uint4 *>(dst)[0] = lo;
            reinterpret_cast<uint4 *>(dst)[1] = hi;
        }
        __syncthreads();
        // (d) each lane: its chunk of every pass, all RB rows
#pragma unroll
        for (int p = 0; p < PM; ++p) {
            if (g0 + 64 * p >= C) break;           // wave-uniform
            uint32_t xp[32];
            const uint4 *src = reinterpret_cast<const uint4 *>(xs + (64 * p + lane) * kXSlot);
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const uint4 v = src[q];
                xp[4 * q] = v.x; xp[4 * q + 1] = v.y; xp[4 * q + 2] = v.z; xp[4 * q + 3] = v.w;
            }
            float z[6];
            chunk_class_sums(make_uint4(0x55555555u, 0x55555555u, 0x55555555u, 0x55555555u), xp, z);
#pragma unroll
            for (int r = 0; r < RB; ++r) acc[r] += chunk_dot_t(wq[p][r], xp, z);
        }
    }

    const float total = wave_reduce_rows<RB>(acc, lane);
    constexpr int GROUP = 64 / RB;          // lanes holding the same row after the reduction
    const int r = lane / GROUP;
    // undo the 2^-24 of the decoded digits (exact), then apply the scale and round to fp16
    if ((lane % GROUP) == 0 && row0 + r < N)
        Y[row0 + r] = __builtin_bit_cast(uint16_t, (_Float16)((total * 16777216.0f) * scale));
}

template <int RB, int PM>
static void launch_cfg(const uint16_t *X, const uint8_t *Wp, float scale, int N, int K, int C, uint16_t *Y,
                       hipStream_t s)
{
    const int rows_per_block = 4 * RB;
    hipLaunchKernelGGL((k_gemv2<RB, PM>), dim3((N + rows_per_block - 1) / rows_per_block), dim3(256), 0, s, X, Wp,
                       scale, N, K, C, Y);
}

template <int PM>
static void launch_pm(const uint16_t *X, const uint8_t *Wp, float scale, int N, int K, int C, uint16_t *Y,
                      hipStream_t s)
{
    // rows per wave: measured best is 1 while that still gives >= ~4 waves per SIMD, else 2
    if (N > 4096 || PM > 1) launch_cfg<2, PM>(X, Wp, scale, N, K, C, Y, s);
    else launch_cfg<1, PM>(X, Wp, scale, N, K, C, Y, s);
}

int launch_gemv2(const uint16_t *X, const uint8_t *Wp, float scale, int N, int K, uint16_t *Y, hipStream_t s)
{
    const int C = (int)(row_bytes(K, TRI_FMT_2BIT) / 16);
    const int passes = (C + 63) / 64;
    if (passes <= 1) launch_pm<1>(X, Wp, scale, N, K, C, Y, s);
    else if (passes == 2) launch_pm<2>(X, Wp, scale, N, K, C, Y, s);
    else launch_pm<3>(X, Wp, scale, N, K, C, Y, s);   // longer rows take several groups of 3 passes
    return hipGetLastError() == hipSuccess ? TRI_OK : TRI_EHIP;
}

}  // namespace tri
