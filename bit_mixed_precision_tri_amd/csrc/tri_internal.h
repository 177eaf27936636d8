// tri_internal.h -- host-side declarations shared by the libtri translation units.
#pragma once
#include <stdint.h>
#include <atomic>
#include <hip/hip_runtime.h>
#include "../../include/tri.h"

namespace tri {

// What the library caches: per device (by its ordinal, up to kMaxDevices), the device's compute
// unit count and, per block-loop kernel variant, how many of its workgroups one CU holds.  Each
// entry is written once, by the first call that needs it on that device, with the value the HIP
// runtime reports; nothing else outlives a call.
constexpr int kMaxDevices = 64;

// Compute units of the calling thread's current device (256 on an MI355X).  Where no device can
// be queried (a host without a GPU, where only the host-side kernel choice runs) the MI355X
// figure is taken.
int cu_count();

// Workgroups of KERNEL, launched with `threads` threads, that one CU of the current device holds
// at once (at least 1).
template <auto KERNEL>
int resident_per_cu(int threads)
{
    static std::atomic<int> cache[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) dev = -1;
    if (dev >= 0 && dev < kMaxDevices) {
        const int c = cache[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, KERNEL, threads, 0) != hipSuccess || n < 1) n = 1;
    if (dev >= 0 && dev < kMaxDevices) cache[dev].store(n, std::memory_order_relaxed);
    return n;
}

inline int64_t row_bytes(int64_t K, int fmt)
{
    if (K < 1) return -1;
    if (fmt == TRI_FMT_2BIT) return 16 * ((K + 63) / 64);
    if (fmt == TRI_FMT_1P6BIT) return 16 * ((K + 79) / 80);
    return -1;
}

int launch_pack(const int8_t *W, int64_t N, int64_t K, int fmt, uint8_t *Wp, hipStream_t s);
int launch_unpack(const uint8_t *Wp, int64_t N, int64_t K, int fmt, int8_t *W, hipStream_t s);
// Quantiser (tri_quant.hip): workspace bytes for E = N*K weights, and the three launches.
int64_t quant_workspace_bytes(int64_t E);
int launch_quantize(const float *W, int64_t N, int64_t K, int fmt, uint8_t *Wp, float *scale, void *workspace,
                    hipStream_t s);
// The device scratch of tri_quantize_noalloc on the current device (its address from
// hipGetSymbolAddress, taken once per device; null if the runtime reports an error), and its size.
void *quant_scratch();
int64_t quant_scratch_bytes();

// Weight matrices that read the same activations, served by one launch (a grouped layer):
// matrix g has N[g] rows and owns the 16-row blocks blk[g] .. blk[g+1]-1 of the grid.  A
// single layer is the case G = 1.
constexpr int kMaxGroups = 4;
struct Groups {
    const uint8_t *Wp[kMaxGroups];
    uint16_t *Y[kMaxGroups];
    float scale[kMaxGroups];
    int N[kMaxGroups];
    int blk[kMaxGroups + 1];
    int G;
};

inline Groups make_groups(int G, const uint8_t *const *Wp, const float *scale, const int *N, uint16_t *const *Y)
{
    Groups gr{};
    gr.G = G;
    gr.blk[0] = 0;
    for (int g = 0; g < G; ++g) {
        gr.Wp[g] = Wp[g];
        gr.Y[g] = Y[g];
        gr.scale[g] = scale[g];
        gr.N[g] = N[g];
        gr.blk[g + 1] = gr.blk[g] + (N[g] + 15) / 16;
    }
    for (int g = G; g < kMaxGroups; ++g) gr.blk[g + 1] = gr.blk[G];
    return gr;
}

// The grid of RB-block workgroups: matrix g owns workgroups blk[g] .. blk[g+1]-1.
inline Groups regroup(const Groups &gr, int RB)
{
    Groups g = gr;
    for (int q = 0; q < gr.G; ++q) g.blk[q + 1] = g.blk[q] + (gr.N[q] + 16 * RB - 1) / (16 * RB);
    for (int q = gr.G; q < kMaxGroups; ++q) g.blk[q + 1] = g.blk[gr.G];
    return g;
}

// Blocks per workgroup (1..4).  A workgroup costs about one block's work on top of its blocks
// (it stages the activations of the whole K range once: measured at M = 4..64 on 4096 -> 11008,
// 11008 -> 4096 and 4096 -> 4096, 172 four-block workgroups beat 688 one-block ones by 15-25%,
// and 128 two-block ones lose to 256 one-block ones), and the grid runs in rounds of one
// workgroup per CU, so the busiest CU costs rounds * (1 + RB).  The cheapest RB is taken, the
// larger on a tie (fewer activation re-reads): 688 blocks take three per workgroup (230
// workgroups, one round), 256 blocks one.  At most max_rb blocks.
inline int choose_rb(const Groups &gr, int M, int max_rb = 4)
{
    const int64_t slices = (M + 15) / 16, cus = cu_count();
    int best = 1;
    int64_t best_cost = -1;
    for (int rb = max_rb; rb >= 1; --rb) {
        const int64_t w = (int64_t)regroup(gr, rb).blk[gr.G] * slices;
        const int64_t cost = (w + cus - 1) / cus * (1 + rb);
        if (best_cost < 0 || cost < best_cost) {
            best = rb;
            best_cost = cost;
        }
    }
    return best;
}

// Glue of a decode block folded around a (grouped) layer in the small-M kernels.  The
// residual (res[g] non-null: added to output g before rounding) is served by every variant;
// the others are compile-time variants of the kernels (template bits kGlueNorm, kGluePair):
//   norm: the activation rows are RMS-normalised, with an optional gain;
//   pair: matrices 0 and 1 (same N) are the gate and up projections of a gated MLP, served by
//         the same workgroups; only output 0 is written, fp16(silu(y0) * y1).
struct Fusion {
    const uint16_t *gain;                        // K fp16, or null (a gain of 1)
    const uint16_t *res[kMaxGroups];             // M x N[g] fp16 per matrix, or null
    float eps;
    int norm;
    int pair;
};
enum { kGlueNorm = 1, kGluePair = 2 };
inline int glue_bits(const Fusion *fu)
{
    return fu ? (fu->norm ? kGlueNorm : 0) | (fu->pair ? kGluePair : 0) : 0;
}

// The matrix of a grouped launch that a workgroup (by its block index) belongs to, with its
// fields.  ONE (a launch for one matrix) makes every field a constant-offset kernel argument;
// the kernels' single-matrix variants are measurably faster at the start of a short decode
// launch (0.2-0.35 us of 3-5 us, with the arguments in one batch of scalar loads either way).
struct GroupSel {
    const uint8_t *Wp;
    uint16_t *Y;
    const uint16_t *res;                         // the block glue's residual, or null
    float scale;
    int N;
    int first;                                   // the matrix's first block
};
template <bool ONE>
__device__ __forceinline__ GroupSel select_group(const Groups &gr, const Fusion &fu, int block)
{
    GroupSel s{gr.Wp[0], gr.Y[0], fu.res[0], gr.scale[0], gr.N[0], 0};
    if constexpr (!ONE) {
#pragma unroll
        for (int q = 1; q < kMaxGroups; ++q)
            if (q < gr.G && block >= gr.blk[q]) s = GroupSel{gr.Wp[q], gr.Y[q], fu.res[q], gr.scale[q], gr.N[q], gr.blk[q]};
    }
    return s;
}

// Kernel launchers of the layer; arguments are already validated.
int launch_gemv2(const uint16_t *X, const uint8_t *Wp, float scale, int N, int K, uint16_t *Y, hipStream_t s);
int launch_smallm(const uint16_t *X, const uint8_t *Wp, float scale, int M, int N, int K, int fmt, uint16_t *Y,
                  hipStream_t s);
// M = 1 on MFMA (tri_mv1.hip) and M >= 2 on MFMA (tri_mvm.hip; past 16 rows in 16-row slices,
// without glue), for one or several matrices, with the block glue `fu` folded in when it is
// non-null; false (nothing launched) if the shape is outside their range.
bool launch_mv1(const uint16_t *X, const Groups &gr, int K, int fmt, hipStream_t s, const Fusion *fu = nullptr);
// M = 2 (both formats) and M = 3, 4 (2-bit) on the M = 1 kernel's structure (of the glue, the
// residual only): all of a wave's activations of every row are staged at once, and A row i of
// the MFMA holds activation row i % MR (MR = 2 or 4).
bool launch_mvr(const uint16_t *X, const Groups &gr, int M, int K, int fmt, hipStream_t s, const Fusion *fu = nullptr);
bool launch_mvm(const uint16_t *X, const Groups &gr, int M, int K, int fmt, hipStream_t s, const Fusion *fu = nullptr);
// The small-M kernels for one matrix: the two above, else the LDS-staged kernel for short rows;
// false (nothing launched) if none of them takes the shape.
bool launch_decode(const uint16_t *X, const uint8_t *Wp, float scale, int M, int N, int K, int fmt, uint16_t *Y,
                   hipStream_t s);
int launch_gemm(const uint16_t *X, const uint8_t *Wp, float scale, int64_t M, int N, int K, int fmt, uint16_t *Y,
                hipStream_t s);
int launch_probe_read(const void *src, int64_t bytes, uint32_t *sink, hipStream_t s);
int launch_probe_copy(const void *src, void *dst, int64_t bytes, hipStream_t s);
int launch_probe_empty(int64_t workgroups, int threads, uint32_t *sink, hipStream_t s);
int launch_probe_rows(const uint16_t *X, const uint8_t *Wp, int N, int K, int fmt, int waves, uint16_t *Y,
                      hipStream_t s);
int launch_probe_stream(const void *src, int64_t bytes, int workgroups, int unroll, uint32_t *sink, hipStream_t s);

}  // namespace tri
