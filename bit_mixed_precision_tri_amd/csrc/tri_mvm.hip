// tri_mvm.hip -- ternary linear layer for a few activation rows (batched decode, up to 16 rows)
// on MFMA; more rows run as 16-row slices in one launch (a second grid dimension), the weights
// of a row block then being read once per slice.
//
// The layer (Pith review of "Spectra 1.1", "What carries the argument"):
//   Y[m][n] = scale * sum_k t[n][k] * X[m][k],  t in {-1, 0, +1},  fp32 accumulation.
// v_mfma_f32_16x16x32_f16 takes the (up to) 16 activation rows as its A operand and 16 weight
// rows, decoded in registers, as B.  The decode is the one of the M = 1 kernel (tri_mv1.hip):
// digits d = t + 1 read as exact fp16 values (2-bit: masked in place, d * 4^p * 2^-24, one
// accumulator per position class, merged with exact powers of two; 1.6-bit: the base-3
// quotients q_p, q * 2^-24, in two sums sum x_p q_p - 3 sum x_p q_{p+1} for tiles of 8 and 16
// rows, the digits d_p = q_p - 3 q_{p+1} themselves for tiles of 4 rows and the longest rows),
// and sum_k X[m][k] subtracted once per output at the end.
//
// Work split.  A workgroup of NW waves owns RB blocks of 16 weight rows; wave w takes chunk-steps
// s, where lane (g = lane/16, j = lane%16) reads 16-byte chunk c = 4*(s*NW + w) + g of row j of
// every block and supplies the activations of row j of X (as A operand) for the same chunk.  All weight chunks
// of the wave are requested at the start.  The activations of a step -- four consecutive
// chunks of every activation row -- are read with whole-line buffer loads that write straight
// into one of the wave's LDS slots (gfx950 loads to LDS: no registers, no LDS write
// instructions), up to two steps ahead; each lane then reads its row's pieces and permutes them
// into the pairing of the decoded weights (2-bit: trits (16v+p, 16v+8+p); 1.6-bit:
// (5q+p, 5q+40+p)).  The waves' partial tiles are added in LDS in a fixed order (no atomics).
//
// Block glue.  Every variant adds an optional residual to the fp32 results before rounding.
// Norm variant (GL & kGlueNorm): the sums of squares of the rows are the diagonal of the Gram
// matrix of the raw activations, formed on the matrix cores; each lane then multiplies its row's
// values by the norm gain (rounded to fp16), which is loaded into the same slot behind the
// activations; the 1/rms factor of each row scales its results.  Pair variant
// (GL & kGluePair): the workgroup also reads the same 16 rows of a second matrix, contracts
// them with the same A operands, and writes fp16(silu(y0) * y1) as its only output.
#include "tri_device.h"
#include "tri_internal.h"

namespace tri {

namespace {

constexpr uint32_t kRsrcWord3 = 0x00020000u;   // raw buffer resource, gfx9 family

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, (int)kRsrcWord3);
}

__device__ __forceinline__ float4_t mfma(const u32x4 a, const u32x4 b, float4_t c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, a), __builtin_bit_cast(half8_t, b), c, 0,
                                                  0, 0);
}

typedef __attribute__((address_space(3))) char *lds_ptr_t;

// Position of piece q of activation row r within its row of an LDS slot.  Rows of 32 pieces
// XOR the position with r, so the sixteen rows that one read instruction touches (one piece
// each) fall in sixteen distinct 16-byte bank groups; rows of 40 pieces do the same within
// their first 32 and last 8 pieces.  (The map is its own inverse.)
template <int RP>
__device__ __forceinline__ int swz(int r, int q)
{
    if constexpr (RP == 32) return q ^ (r & 15);
    else return q < 32 ? q ^ (r & 15) : 32 + ((q - 32) ^ (r & 7));
}

// s_waitcnt vmcnt(n): wait until at most n vector-memory loads of the wave are outstanding
// (the counter retires in issue order); n must fold to a constant.
template <int N>
__device__ __forceinline__ void wait_vm()
{
    __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | (((N >> 4) & 3) << 14));   // (expcnt, lgkmcnt: no wait)
}
template <int N = 0>
__device__ __forceinline__ void wait_vm_upto(int n)
{
    if constexpr (N < 63) {
        if (n <= N) wait_vm<N>();
        else wait_vm_upto<N + 1>(n);
    } else {
        wait_vm<63>();
    }
}

}  // namespace

template <int FMT, int MT, int NW, int CST, int GL, int RB, bool ONE>
__global__ __launch_bounds__(64 * NW) void k_mvm(const uint16_t *__restrict__ X, const Groups gr, int M, int K, int C,
                                                 const Fusion fu)
{
    constexpr bool NORM = (GL & kGlueNorm) != 0;
    constexpr bool PAIR = (GL & kGluePair) != 0;
    static_assert(!PAIR || RB <= 3, "the pair variant owns one to three 16-row blocks of each matrix per workgroup");
    const GroupSel grp = select_group<ONE>(gr, fu, (int)blockIdx.x);
    const uint8_t *__restrict__ Wp = grp.Wp;
    const float scale = grp.scale;
    const int N = grp.N;
    // more than 16 activation rows: workgroup row y of the grid takes rows 16y .. 16y+15 of X and Y
    const int64_t m_first = 16 * (int64_t)blockIdx.y;
    X += m_first * K;
    M = min(16, M - (int)m_first);
    uint16_t *__restrict__ Y = grp.Y + m_first * N;
    const uint16_t *__restrict__ R = grp.res ? grp.res + m_first * N : nullptr;
    constexpr bool TWO = FMT == TRI_FMT_2BIT;
    constexpr int XH = TWO ? 64 : 80;            // activations per chunk
    constexpr int NOP = TWO ? 8 : 10;            // A operands (MFMAs) per chunk
    // 1.6-bit from base-3 quotients (two sums by halves) where the registers allow it and
    // the tile has rows enough to keep the matrix cores' extra work off the critical path (at
    // four rows it measured slower); from the digits (one sum by halves) otherwise
    constexpr bool QT = !TWO && MT >= 8 && CST < 14;   // (not RB: grouped and single launches agree bitwise)
    constexpr int NCLS = TWO ? 6 : (QT ? 4 : 2);   // accumulators: position classes (2-bit), sums (1.6-bit)
    constexpr int RP = 4 * XH / 8;               // 16-byte pieces of one row per step (32 or 40)
    constexpr int NLD = (MT * RP + 63) / 64;     // whole-line activation loads per lane and step
    // per wave: PD slots of one step's activations each (piece q of row r at r * RP + swz(r, q);
    // every load instruction fills 64 pieces, so a slot holds NLD * 64, + 64 for the norm gain).
    // Two slots where eight waves' take at most 128 KB (at most 64 KB for four waves, which
    // share a CU two at a time), else one; one for the pair variant, whose fused launches have
    // grids of several workgroups per CU.  After the last step the same LDS holds the per-wave
    // partial tiles [row m][column (block r, row j)], + sum x (+ sum x^2).
    constexpr int SLOT = (NLD + (NORM ? 1 : 0)) * 64;
    constexpr int PD = !PAIR && NW * 2 * SLOT * 16 <= (NW <= 4 ? 64 : 128) * 1024 ? 2 : 1;
    constexpr int RCOL = 16 * RB + (NORM ? 2 : 1);
    constexpr int XS_B = NW * PD * SLOT * 16, RED_B = NW * 16 * RCOL * 4;
    __shared__ u32x4 smem[(XS_B > RED_B ? XS_B : RED_B) / 16];
    u32x4 (*xs)[PD][SLOT] = reinterpret_cast<u32x4 (*)[PD][SLOT]>(smem);
    float (*red)[16][RCOL] = reinterpret_cast<float (*)[16][RCOL]>(smem);
    __shared__ float red1[PAIR ? NW : 1][16][PAIR ? 16 * RB + 1 : 1];   // pair: the second matrix's partial tiles

    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform (scalar descriptors)
    const int g = lane >> 4;
    const int j = lane & 15;
    const int n0 = ((int)blockIdx.x - grp.first) * 16 * RB;
    const int64_t S = (int64_t)C * 16;

    // activations of step s: load instruction i, lane l fills slot position P = 64i + l, that is
    // row P / RP at position P % RP, with piece swz(row, P % RP) of the row's step (values
    // 8 q ... of the step's 4 XH): whole 128-byte lines per instruction
    const __amdgpu_buffer_rsrc_t xr = rsrc(X, __builtin_amdgcn_readfirstlane((uint32_t)((int64_t)M * K * 2)));
    // The lane's part of each load offset does not change from step to step (a step adds the
    // wave-uniform k of its first value); rows past M get an offset past the buffer, which
    // reads zeros.  Values past K occur only in a wave's last live step, the one step that
    // tests them per lane.  (The out-of-range offset is held in a register: as a literal it
    // would be rebuilt before every select.)
    uint32_t oob;
    asm volatile("v_mov_b32 %0, 0x80000000" : "=v"(oob));
    uint32_t xoff[NLD];
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
        const int P = 64 * i + lane;
        const int row = P / RP, q = swz<RP>(row, P % RP);
        xoff[i] = row < M ? (uint32_t)(row * K + 8 * q) * 2u : oob;
    }
    // step s into slot s % PD (norm: and piece `lane` of the step's gain behind it; without a
    // gain the resource is empty and the pieces read as zero, so every step issues the same
    // number of loads)
    const __amdgpu_buffer_rsrc_t gn = rsrc(fu.gain, NORM && fu.gain ? (uint32_t)K * 2u : 0u);
    auto load_x = [&](int s) {
        const int kb = 4 * (s * NW + wv) * XH;   // wave-uniform
        const lds_ptr_t dst = (lds_ptr_t)&xs[wv][s % PD][0];
        if (kb + 4 * XH <= K) {                  // (wave-uniform: only a wave's last live step tests K per lane)
#pragma unroll
            for (int i = 0; i < NLD; ++i)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, dst + 1024 * i, 16, (int)(xoff[i] + 2u * (uint32_t)kb), 0,
                                                        0, 0);
        } else {
#pragma unroll
            for (int i = 0; i < NLD; ++i) {
                const int P = 64 * i + lane;
                const int q = swz<RP>(P / RP, P % RP);
                const uint32_t off = kb + 8 * q < K ? xoff[i] + 2u * (uint32_t)kb : oob;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, dst + 1024 * i, 16, (int)off, 0, 0, 0);
            }
        }
        if constexpr (NORM) {
            const int k = kb + 8 * lane;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(gn, dst + 1024 * NLD, 16,
                                                    (lane < RP && k < K) ? (int)((uint32_t)k * 2u) : (int)0x80000000u,
                                                    0, 0, 0);
        }
    };

    const float4_t zero4 = {0.f, 0.f, 0.f, 0.f};
    float4_t acc[RB][NCLS];
#pragma unroll
    for (int r = 0; r < RB; ++r)
#pragma unroll
        for (int c = 0; c < NCLS; ++c) acc[r][c] = zero4;
    float4_t acc1[PAIR ? RB : 1][PAIR ? NCLS : 1];   // pair: the second matrix
#pragma unroll
    for (int r = 0; r < (PAIR ? RB : 1); ++r)
#pragma unroll
        for (int c = 0; c < (PAIR ? NCLS : 1); ++c) acc1[r][c] = zero4;
    auto contract = [&](const u32x4 (&a)[NOP], const u32x4 v, float4_t (&ac)[NCLS]) __attribute__((always_inline)) {
        if constexpr (TWO) {
            const u32x4 u = v >> 12u;
#pragma unroll
            for (int p = 0; p < 6; ++p) ac[p] = mfma(a[p], v & (0x00030003u << (2 * p)), ac[p]);
            ac[0] = mfma(a[6], u & 0x00030003u, ac[0]);
            ac[1] = mfma(a[7], u & 0x000C000Cu, ac[1]);
        } else {
            // register q: bytes q and q+8, position p pairs trits (5q+p, 5q+40+p).  From the
            // quotients q_p of the bytes: ac[0], ac[1] gather sum x_p q_p and ac[2], ac[3]
            // sum x_p q_{p+1}, by halves; from the digits: ac[0], ac[1] gather sum x_p d_p (every
            // quotient and digit carries the same scale)
            uint32_t qt[8][5];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                if constexpr (QT) base3_quotients_u16x2(byte_pair(v, q), qt[q]);
                else base3_digits_u16x2(byte_pair(v, q), qt[q]);
            }
#pragma unroll
            for (int p = 0; p < 5; ++p) {
                ac[0] = mfma(a[2 * p], u32x4{qt[0][p], qt[1][p], qt[2][p], qt[3][p]}, ac[0]);
                ac[1] = mfma(a[2 * p + 1], u32x4{qt[4][p], qt[5][p], qt[6][p], qt[7][p]}, ac[1]);
                if (QT && p < 4) {
                    ac[NCLS - 2] = mfma(a[2 * p], u32x4{qt[0][p + 1], qt[1][p + 1], qt[2][p + 1], qt[3][p + 1]}, ac[NCLS - 2]);
                    ac[NCLS - 1] = mfma(a[2 * p + 1], u32x4{qt[4][p + 1], qt[5][p + 1], qt[6][p + 1], qt[7][p + 1]}, ac[NCLS - 1]);
                }
            }
        }
    };
    float4_t accx = zero4;                       // sum_k X[m][k] in every column of the tile
    // norm: the Gram matrix D = X X^T of this wave's raw activations on the matrix cores (lane (g, j)
    // supplies row j's values of chunk g as both its A and its B operand), whose diagonal D[j][j] is
    // row j's sum of squares over the wave's chunks
    float4_t accq = {0.f, 0.f, 0.f, 0.f};
    // the activations of PD steps are in flight at once.  The first PD steps' activations are
    // requested before the weights: the load counter is in order, so the first steps'
    // permutation overlaps the weight stream instead of waiting behind it
#pragma unroll
    for (int t = 0; t < PD; ++t) load_x(t);
    // every weight chunk of the wave, all in flight at once
    const int rows_here = min(16 * RB, N - n0);
    const __amdgpu_buffer_rsrc_t wr =
        rsrc(Wp + (int64_t)n0 * S, __builtin_amdgcn_readfirstlane((uint32_t)(rows_here * S)));
    // (pair: the same chunks of the second matrix, requested in the order they are used)
    const __amdgpu_buffer_rsrc_t wr1 =
        rsrc(gr.Wp[PAIR ? 1 : 0] + (int64_t)n0 * S, __builtin_amdgcn_readfirstlane((uint32_t)(rows_here * S)));
    u32x4 wq[RB][CST], wq1[PAIR ? RB : 1][PAIR ? CST : 1];
#pragma unroll
    for (int s = 0; s < CST; ++s) {
        const int c = 4 * (s * NW + wv) + g;
#pragma unroll
        for (int r = 0; r < RB; ++r) {           // (rows past the matrix's end read as zero)
            const int off = c < C ? (int)(uint32_t)((16 * r + j) * S + c * 16) : (int)0x80000000u;
            wq[r][s] = __builtin_amdgcn_raw_buffer_load_b128(wr, off, 0, 0);
        }
        if constexpr (PAIR) {
#pragma unroll
            for (int r = 0; r < RB; ++r) {
                const int off = c < C ? (int)(uint32_t)((16 * r + j) * S + c * 16) : (int)0x80000000u;
                wq1[r][s] = __builtin_amdgcn_raw_buffer_load_b128(wr1, off, 0, 0);
            }
        }
    }
#pragma unroll
    for (int s = 0; s < CST; ++s) {
        // wave-uniform: no chunk of this step is live.  (Step 0 always runs -- a wave without a
        // live chunk contracts zeros -- so every accumulator's first MFMA takes a literal zero
        // instead of registers zeroed ahead of the loop.)
        if (s > 0 && 4 * (s * NW + wv) >= C) break;
        // wait for this step's pieces: loads issued after them are the later prefetched steps,
        // the weights (while s < PD) and the refills (issued at the ends of the earlier steps) of
        // the steps after s
        {
            constexpr int NWL = CST * RB * (PAIR ? 2 : 1), NX = NLD + (NORM ? 1 : 0);
            int after = 0;
            for (int u = s + 1; u < PD; ++u) after += NX;
            if (s < PD) after += NWL;
            for (int t = s - PD + 1 > 0 ? s - PD + 1 : 0; t < s; ++t) after += t + PD < CST ? NX : 0;
            wait_vm_upto(after);
        }
        // row j, chunk g of the step (tiles of fewer than 16 rows: A rows past the tile repeat its
        // rows, and the D rows they give are never read)
        const u32x4 *slot = &xs[wv][s % PD][0];
        const int row = j % MT;
        uint32_t x32[XH / 2];
#pragma unroll
        for (int q = 0; q < XH / 8; ++q) {
            const u32x4 v = slot[row * RP + swz<RP>(row, (XH / 8) * g + q)];
            x32[4 * q] = v[0]; x32[4 * q + 1] = v[1]; x32[4 * q + 2] = v[2]; x32[4 * q + 3] = v[3];
        }
        if constexpr (NORM) {
#pragma unroll
            for (int q = 0; q < XH / 8; ++q) {
                const u32x4 xq = {x32[4 * q], x32[4 * q + 1], x32[4 * q + 2], x32[4 * q + 3]};
                accq = mfma(xq, xq, accq);
            }
            if (fu.gain) {
#pragma unroll
                for (int q = 0; q < XH / 8; ++q) {
                    const u32x4 gq = slot[NLD * 64 + (XH / 8) * g + q];   // the same for every row
#pragma unroll
                    for (int e = 0; e < 4; ++e) x32[4 * q + e] = mul2(x32[4 * q + e], gq[e]);
                }
            }
        }
        u32x4 a[NOP];
        if constexpr (TWO) {
#pragma unroll
            for (int p = 0; p < 8; ++p)
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    a[p][v] = (p & 1) ? pair_halves<1>(x32[8 * v + 4 + p / 2], x32[8 * v + p / 2])
                                      : pair_halves<0>(x32[8 * v + 4 + p / 2], x32[8 * v + p / 2]);
        } else {
#pragma unroll
            for (int p = 0; p < 5; ++p)
#pragma unroll
                for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                    for (int qq = 0; qq < 4; ++qq) {
                        const int e = 5 * (4 * hh + qq) + p;   // value index; partner e + 40
                        a[2 * p + hh][qq] = (e & 1) ? pair_halves<1>(x32[(e >> 1) + 20], x32[e >> 1])
                                                    : pair_halves<0>(x32[(e >> 1) + 20], x32[e >> 1]);
                    }
        }
        // sum_k X[m][k] on the matrix cores: every A operand against a B of ones
        const u32x4 ones = {0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u};
#pragma unroll
        for (int p = 0; p < NOP; ++p) accx = mfma(a[p], ones, accx);
        // decode and contract
#pragma unroll
        for (int r = 0; r < RB; ++r) contract(a, wq[r][s], acc[r]);
        if constexpr (PAIR) {
#pragma unroll
            for (int r = 0; r < RB; ++r) contract(a, wq1[r][s], acc1[r]);
        }
        // refill the slot with step s + PD once its reads are done.  (Issued after the contraction:
        // the compiler's own waits for the weight registers do not count the loads to LDS, so a
        // refill issued earlier would be waited for with them -- measured 4% slower at 11008 -> 4096,
        // M = 16.)
        __builtin_amdgcn_s_waitcnt(0xC07F);      // lgkmcnt(0)
        if (s + PD < CST) load_x(s + PD);
    }

    // merge classes: lane (g, j) holds rows 4g + e of column j (of D and of the sums of X)
    auto merge = [&](const float4_t (&ac)[NCLS]) __attribute__((always_inline)) {
        if constexpr (!TWO) {
            if constexpr (QT) return (ac[0] + ac[1]) - 3.f * (ac[NCLS - 2] + ac[NCLS - 1]);   // d_p = q_p - 3 q_{p+1}
            else return ac[0] + ac[1];
        }
        float4_t t = ac[0] + 0.25f * ac[1];
        t += 0.0625f * ac[2] + 0.015625f * ac[3];
        t += 0.00390625f * ac[4] + 0.0009765625f * ac[5];
        return t;
    };
    __syncthreads();                             // every wave is done with its activation slot
#pragma unroll
    for (int r = 0; r < RB; ++r) {
        const float4_t t = merge(acc[r]);
#pragma unroll
        for (int e = 0; e < 4; ++e) red[wv][4 * g + e][16 * r + j] = t[e];
    }
    if (j == 0) {
#pragma unroll
        for (int e = 0; e < 4; ++e) red[wv][4 * g + e][16 * RB] = accx[e];
    }
    if constexpr (PAIR) {
#pragma unroll
        for (int r = 0; r < RB; ++r) {
            const float4_t t1 = merge(acc1[r]);
#pragma unroll
            for (int e = 0; e < 4; ++e) red1[wv][4 * g + e][16 * r + j] = t1[e];
        }
    }
    if constexpr (NORM) {                        // (D[j][j] is element j % 4 of lane (j / 4, j))
        if (g == (j >> 2)) red[wv][j][16 * RB + 1] = accq[j & 3];
    }
    __syncthreads();
    // thread (m, jj): output Y[m][n0 + jj], waves added in a fixed order
    for (int o = threadIdx.x; o < MT * 16 * RB; o += 64 * NW) {
        const int m = o / (16 * RB), jj = o % (16 * RB);
        if (m < M && n0 + jj < N) {
            float sd = 0.f, sx = 0.f;
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                sd += red[w][m][jj];
                sx += red[w][m][16 * RB];
            }
            float rinv = 1.f;
            if constexpr (NORM) {
                float sq = 0.f;
#pragma unroll
                for (int w = 0; w < NW; ++w) sq += red[w][m][16 * RB + 1];
                rinv = __builtin_amdgcn_rsqf(sq * __builtin_amdgcn_rcpf((float)K) + fu.eps);   // (v_rsq, v_rcp: about 1 ulp)
            }
            float y = (sd * 16777216.0f - sx) * scale * rinv;
            if constexpr (PAIR) {
                float sd1 = 0.f;
#pragma unroll
                for (int w = 0; w < NW; ++w) sd1 += red1[w][m][jj];
                const float y1 = (sd1 * 16777216.0f - sx) * gr.scale[1] * rinv;
                y = y / (1.f + __expf(-y)) * y1; // silu(gate) * up
            }
            if (R) y += h2f(R[(int64_t)m * N + n0 + jj]);
            Y[(int64_t)m * N + n0 + jj] = __builtin_bit_cast(uint16_t, (_Float16)y);
        }
    }
}

// Glue variants that exist: eight waves and up to eight steps only, and none whose registers
// would overflow (1.6-bit tiles of 16 rows past 6 steps; pairs of 16-row tiles past 4 steps).
template <int FMT, int MT, int NW, int CST, int GL>
constexpr bool has_glue()
{
    if (GL == 0) return true;
    if (NW != 8 || CST > 8) return false;
    if ((GL & kGlueNorm) && FMT == TRI_FMT_1P6BIT && MT == 16 && CST > 6) return false;
    if ((GL & kGluePair) && MT == 16 && CST > 4) return false;
    return true;
}

// Several 16-row blocks per workgroup (RB): every activation value a wave reads feeds RB
// blocks, so the activations are re-read from cache RB times less often.  Variants exist for
// eight waves, without glue or with the norm, and only where the registers do not spill (three
// blocks wherever four exist); the pair variant takes two or three blocks of each matrix for
// tiles of up to 8 rows and 2 steps (its two sets of accumulators).
template <int FMT, int MT, int CST, int RB, int GL>
constexpr bool has_rb()
{
    if (RB == 1) return true;
    if (GL & kGluePair) return (RB == 2 || RB == 3) && MT <= 8 && CST <= 2;
    const int c = CST + ((GL & kGlueNorm) ? 1 : 0);   // the norm takes about one more step's registers
    if (RB == 2) return FMT == TRI_FMT_2BIT ? (MT == 16 ? c <= 6 : c <= 8) : (MT == 16 ? c <= 5 : c <= 6);
    // (1.6-bit tiles of 4 rows: four blocks measured 4% slower than two, three are tried; of 8
    // rows, the quotient accumulators take one step's registers)
    if (RB == 3 && MT == 4 && FMT == TRI_FMT_1P6BIT) return c <= 4;   // (its digit sums: few accumulators)
    if (RB == 3 || RB == 4)
        return MT == 16 ? c <= 3 : MT == 8 ? c <= (FMT == TRI_FMT_2BIT ? 4 : 3) : (FMT == TRI_FMT_2BIT && c <= 5);
    return false;
}

template <int FMT, int MT, int NW, int CST, int GL, int RB>
static bool launch_gl(const uint16_t *X, const Groups &gr, int M, int K, int C, hipStream_t s, const Fusion &f)
{
    if constexpr (has_glue<FMT, MT, NW, CST, GL>() && has_rb<FMT, MT, CST, RB, GL>()) {
        Groups g = RB == 1 ? gr : regroup(gr, RB);
        if constexpr ((GL & kGluePair) != 0) {   // (the grid covers the first matrix's blocks only)
            for (int q = 2; q <= kMaxGroups; ++q) g.blk[q] = g.blk[1];
        }
        const dim3 grid(g.blk[g.G], (M + 15) / 16), block(64 * NW);
        // (single-matrix variants for the plain layer only: the glue variants serve grouped launches)
        if (GL == 0 && g.G == 1)
            hipLaunchKernelGGL((k_mvm<FMT, MT, NW, CST, GL, RB, GL == 0>), grid, block, 0, s, X, g, M, K, C, f);
        else
            hipLaunchKernelGGL((k_mvm<FMT, MT, NW, CST, GL, RB, false>), grid, block, 0, s, X, g, M, K, C, f);
        return true;
    }
    return false;
}

template <int FMT, int MT, int NW, int CST>
static bool launch_cfg(const uint16_t *X, const Groups &gr, int M, int K, int C, hipStream_t s, const Fusion *fu,
                       int rb = 1)
{
    const Fusion f = fu ? *fu : Fusion{};
    switch (glue_bits(fu)) {
    case kGlueNorm:
        if constexpr (NW == 8) {                 // the largest RB up to rb that has a variant
            if (rb >= 4 && launch_gl<FMT, MT, NW, CST, kGlueNorm, 4>(X, gr, M, K, C, s, f)) return true;
            if (rb >= 3 && launch_gl<FMT, MT, NW, CST, kGlueNorm, 3>(X, gr, M, K, C, s, f)) return true;
            if (rb >= 2 && launch_gl<FMT, MT, NW, CST, kGlueNorm, 2>(X, gr, M, K, C, s, f)) return true;
        }
        return launch_gl<FMT, MT, NW, CST, kGlueNorm, 1>(X, gr, M, K, C, s, f);
    case kGluePair:
        if (rb >= 3 && launch_gl<FMT, MT, NW, CST, kGluePair, 3>(X, gr, M, K, C, s, f)) return true;
        if (rb >= 2 && launch_gl<FMT, MT, NW, CST, kGluePair, 2>(X, gr, M, K, C, s, f)) return true;
        return launch_gl<FMT, MT, NW, CST, kGluePair, 1>(X, gr, M, K, C, s, f);
    case kGlueNorm | kGluePair:
        if (rb >= 3 && launch_gl<FMT, MT, NW, CST, kGlueNorm | kGluePair, 3>(X, gr, M, K, C, s, f)) return true;
        if (rb >= 2 && launch_gl<FMT, MT, NW, CST, kGlueNorm | kGluePair, 2>(X, gr, M, K, C, s, f)) return true;
        return launch_gl<FMT, MT, NW, CST, kGlueNorm | kGluePair, 1>(X, gr, M, K, C, s, f);
    default:
        if constexpr (NW == 8) {
            if (rb >= 4 && launch_gl<FMT, MT, NW, CST, 0, 4>(X, gr, M, K, C, s, f)) return true;
            if (rb >= 3 && launch_gl<FMT, MT, NW, CST, 0, 3>(X, gr, M, K, C, s, f)) return true;
            if (rb >= 2 && launch_gl<FMT, MT, NW, CST, 0, 2>(X, gr, M, K, C, s, f)) return true;
        }
        return launch_gl<FMT, MT, NW, CST, 0, 1>(X, gr, M, K, C, s, f);
    }
}

template <int FMT, int MT>
static bool launch_mt(const uint16_t *X, const Groups &gr, int M, int K, int C, hipStream_t s,
                      const Fusion *fu, int rb)
{
    // 1.6-bit tiles of 16 rows: an eight-wave workgroup's activation slots take about 93 KB of LDS,
    // so one workgroup fits a CU; with more row blocks than CUs (but too few for two blocks per
    // workgroup), four-wave workgroups (half the LDS) let two share a CU (measured 20% faster at
    // 4096 -> 11008 with one block per workgroup; slower where the grid fits)
    if constexpr (FMT == TRI_FMT_1P6BIT && MT == 16) {
        if (!glue_bits(fu) && rb == 1 && (int64_t)gr.blk[gr.G] * ((M + 15) / 16) > cu_count()) {
            switch ((C + 15) / 16) {
            case 1: return launch_cfg<FMT, MT, 4, 1>(X, gr, M, K, C, s, fu);
            case 2: return launch_cfg<FMT, MT, 4, 2>(X, gr, M, K, C, s, fu);
            case 3: return launch_cfg<FMT, MT, 4, 3>(X, gr, M, K, C, s, fu);
            case 4: return launch_cfg<FMT, MT, 4, 4>(X, gr, M, K, C, s, fu);
            case 5: return launch_cfg<FMT, MT, 4, 5>(X, gr, M, K, C, s, fu);
            case 6: return launch_cfg<FMT, MT, 4, 6>(X, gr, M, K, C, s, fu);
            case 7: return launch_cfg<FMT, MT, 4, 7>(X, gr, M, K, C, s, fu);
            case 8: return launch_cfg<FMT, MT, 4, 8>(X, gr, M, K, C, s, fu);
            default: break;
            }
        }
    }
    const int cst8 = (C + 31) / 32;              // chunk-steps with 8 waves (4 chunks per step and wave)
    switch (cst8) {
    case 1: return launch_cfg<FMT, MT, 8, 1>(X, gr, M, K, C, s, fu, rb);
    case 2: return launch_cfg<FMT, MT, 8, 2>(X, gr, M, K, C, s, fu, rb);
    case 3: return launch_cfg<FMT, MT, 8, 3>(X, gr, M, K, C, s, fu, rb);
    case 4: return launch_cfg<FMT, MT, 8, 4>(X, gr, M, K, C, s, fu, rb);
    case 5: return launch_cfg<FMT, MT, 8, 5>(X, gr, M, K, C, s, fu, rb);
    case 6: return launch_cfg<FMT, MT, 8, 6>(X, gr, M, K, C, s, fu, rb);
    case 7: return launch_cfg<FMT, MT, 8, 7>(X, gr, M, K, C, s, fu, rb);
    case 8: return launch_cfg<FMT, MT, 8, 8>(X, gr, M, K, C, s, fu, rb);
    default: break;
    }
    // longer rows (up to 16 steps): eight waves still, one block per workgroup and no glue.  (A
    // sixteen-wave workgroup has 128 registers per lane, too few for these steps: its variants
    // spilled and ran 1.2-3.5x slower.)
    if (!glue_bits(fu)) {
        switch (cst8) {
        case 9: case 10: return launch_cfg<FMT, MT, 8, 10>(X, gr, M, K, C, s, fu, 1);
        case 11: case 12: return launch_cfg<FMT, MT, 8, 12>(X, gr, M, K, C, s, fu, 1);
        case 13: case 14: return launch_cfg<FMT, MT, 8, 14>(X, gr, M, K, C, s, fu, 1);
        case 15: case 16:
            if constexpr (FMT == TRI_FMT_2BIT || MT <= 8) return launch_cfg<FMT, MT, 8, 16>(X, gr, M, K, C, s, fu, 1);
            break;
        default: break;
        }
    }
    return false;                                // longer rows: the streaming small-M kernel
}

// Sixteen waves of three steps for 2-bit tiles of 5..8 rows whose rows take five or six
// eight-wave steps (8192 < K <= 12288; 1.6-bit: 10240 < K <= 15360), where the matrix alone would
// run one block per workgroup and no glue but the residual applies: 11008 -> 4096 at M = 8
// 7.76 -> 7.33 us (sixteen-row tiles gain nothing).  1.6-bit, whose sixteen-wave variants spill,
// takes twelve waves of three or four steps, for tiles of 3..8 rows: 11008 -> 4096 at M = 8
// 8.30 -> 8.03 us, at M = 4 7.77 -> 7.58 us (sixteen-row tiles: 9.80 -> 9.87 us, not used).  The wave count changes the order of the sums, so the choice is made per
// matrix: a group whose matrices all qualify runs as one such launch, a mixed group as one
// launch per matrix, and every output stays bitwise equal to a single launch of its matrix.
static bool wide16(const Groups &gr, int g, int M, int C, int fmt, const Fusion *fu)
{
    if (M < (fmt == TRI_FMT_2BIT ? 5 : 3) || M > 8 || glue_bits(fu)) return false;
    const int cst8 = (C + 31) / 32;
    if (cst8 < 5 || cst8 > 6) return false;
    const Groups one = make_groups(1, &gr.Wp[g], &gr.scale[g], &gr.N[g], &gr.Y[g]);
    return choose_rb(one, M) == 1;
}

bool launch_mvm(const uint16_t *X, const Groups &gr, int M, int K, int fmt, hipStream_t s, const Fusion *fu)
{
    const int C = (int)(row_bytes(K, fmt) / 16);
    // 32-bit buffer offsets: one 16-row slice of the activations and one 16-row block of the
    // weights stay below 2^31 bytes; activations are read in pieces of 8 values, so K must be a
    // multiple of 8.  More than 16 rows run as 16-row slices (the second grid dimension).
    if (M < 2 || M > 16 * 65535 || (K % 8) != 0 || 16 * (int64_t)K * 2 >= ((int64_t)1 << 31) ||
        16 * (int64_t)C * 16 >= ((int64_t)1 << 31))
        return false;
    if (M > 16 && fu) return false;              // the block glue serves up to 16 rows
    int n16 = 0;
    for (int g = 0; g < gr.G; ++g) n16 += wide16(gr, g, M, C, fmt, fu);
    if (n16 == gr.G) {
        if (fmt == TRI_FMT_2BIT) return launch_cfg<TRI_FMT_2BIT, 8, 16, 3>(X, gr, M, K, C, s, fu, 1);
        if (M <= 4)
            return (C + 47) / 48 <= 3 ? launch_cfg<TRI_FMT_1P6BIT, 4, 12, 3>(X, gr, M, K, C, s, fu, 1)
                                      : launch_cfg<TRI_FMT_1P6BIT, 4, 12, 4>(X, gr, M, K, C, s, fu, 1);
        return (C + 47) / 48 <= 3 ? launch_cfg<TRI_FMT_1P6BIT, 8, 12, 3>(X, gr, M, K, C, s, fu, 1)
                                  : launch_cfg<TRI_FMT_1P6BIT, 8, 12, 4>(X, gr, M, K, C, s, fu, 1);
    }
    if (n16 > 0) {                               // (a mixed group: one launch per matrix)
        for (int g = 0; g < gr.G; ++g) {
            const Groups one = make_groups(1, &gr.Wp[g], &gr.scale[g], &gr.N[g], &gr.Y[g]);
            Fusion f1 = fu ? *fu : Fusion{};
            f1.res[0] = f1.res[g];
            for (int q = 1; q < kMaxGroups; ++q) f1.res[q] = nullptr;
            if (!launch_mvm(X, one, M, K, fmt, s, fu ? &f1 : nullptr)) return false;
        }
        return true;
    }
    // (the pair's grid covers the first matrix only: its block count decides, at most three blocks)
    Groups first = gr;
    first.G = 1;
    const int rb = (glue_bits(fu) & kGluePair) ? choose_rb(first, M, 3) : choose_rb(gr, M);
    if (fmt == TRI_FMT_2BIT) {
        if (M <= 4) return launch_mt<TRI_FMT_2BIT, 4>(X, gr, M, K, C, s, fu, rb);
        if (M <= 8) return launch_mt<TRI_FMT_2BIT, 8>(X, gr, M, K, C, s, fu, rb);
        return launch_mt<TRI_FMT_2BIT, 16>(X, gr, M, K, C, s, fu, rb);
    }
    if (M <= 4) return launch_mt<TRI_FMT_1P6BIT, 4>(X, gr, M, K, C, s, fu, rb);
    if (M <= 8) return launch_mt<TRI_FMT_1P6BIT, 8>(X, gr, M, K, C, s, fu, rb);
    return launch_mt<TRI_FMT_1P6BIT, 16>(X, gr, M, K, C, s, fu, rb);
}

}  // namespace tri
