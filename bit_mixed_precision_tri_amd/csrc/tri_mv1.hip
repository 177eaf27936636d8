// tri_mv1.hip -- ternary linear layer for one activation row (M = 1, decode) on MFMA, and for
// two rows with the same structure.
//
// The layer (Pith review of "Spectra 1.1", "What carries the argument"):
//   y[n] = scale * sum_k t[n][k] * x[k],  t in {-1, 0, +1},  fp32 accumulation.
// At M = 1 the work is a matrix-vector product bound by the weight stream.  It still runs on
// v_mfma_f32_16x16x32_f16: sixteen weight rows form the 16 columns of the B operand and the
// activation chunk is broadcast to the 16 rows of A (only one output row is kept).  That
// wastes matrix-core work but moves the multiply-adds off the vector ALU, which then only
// masks the packed words -- one instruction per register, against one per trit on the VALU
// path -- so the decode keeps pace with HBM.
//
// Decode.  Masking a packed register leaves each trit's digit d = t + 1 in the low bits of
// an fp16 half, which reads exactly as d * 4^p * 2^-24 (p = the digit's position in its
// 16-bit half): fp16 subnormals, or the two lowest exponent bits for p = 5.  One MFMA only
// mixes digits of one position, so it accumulates exact products into one accumulator per
// position class, and the classes are merged with exact powers of two.  That gives
// sum_k d*x; since t = d - 1, sum_k x is subtracted once per row at the end.
//   2-bit:   a register pairs trits (16v+p, 16v+8+p); positions 6, 7 are taken from the
//            word shifted right by 12, so they share the classes of 0 and 1.
//   1.6-bit: bytes q and q+8 of a chunk become the two 16-bit lanes of a register.  Their
//            base-3 digits are d_p = q_p - 3 q_{p+1} with q_p = floor(b / 3^p) (the repeated
//            division b'_i -> x_i that the review's referee report describes for the paper's
//            section 3.2), each quotient an exact multiply-shift; position p pairs trits
//            (5q+p, 5q+40+p).  The kernel contracts the quotients, not the digits:
//            sum_p x_p d_p = sum_p x_p q_p - 3 sum_p x_p q_{p+1}, two MFMA sums (each by halves
//            of the chunk) whose every quotient reads as q * 2^-24; that spares the VALU, which
//            bounds this format, four multiply-subtracts per register.
// The sum over k is order-free, so the activations are permuted into the same pairing.
//
// Work split.  A workgroup of NW waves owns 16 weight rows; wave w takes chunk-steps s,
// where lane (g = lane/16, j = lane%16) reads 16-byte chunk 4*(s*NW + w) + g of row j.  Every
// weight chunk of the wave is requested at the start (reads past the matrix return zero;
// chunks past a row's end meet zero activations).  The wave loads the activations of its own
// chunks with whole-line loads, permutes them into the A-operand order in LDS (no
// workgroup barrier), and adds them up for sum_k x.  The waves' partial sums meet in LDS and
// are added in a fixed order (no atomics).  With two activation rows (MR = 2) both rows are
// staged the same way and A row i holds activation row i % 2, so D rows 0 and 1 are the two
// outputs.
//
// Block glue.  Every variant adds an optional residual to the fp32 result before rounding.
// Norm variant (GL & kGlueNorm): the norm gain is read beside the activations; each lane adds
// the squares of its activations (gathered like sum_k x), multiplies them by the gain
// (rounded to fp16) and the 1/rms factor scales the result.  Pair variant (GL & kGluePair):
// the workgroup also reads the same 16 rows of a second matrix, contracts them with the same
// A operands, and writes fp16(silu(y0) * y1) -- the gated-MLP input -- as its only output.
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

}  // namespace

// LDS of the staged A operands of a workgroup (the layouts of k_mv1's xa and xb).
template <int FMT, int NW, int CST, int MR>
constexpr int xa_bytes()
{
    return FMT == TRI_FMT_2BIT ? NW * 4 * CST * MR * (8 + (MR == 4 ? 1 : 0)) * 16 : NW * MR * (4 * CST * 10 + 1) * 16;
}

// Block loop: outputs held in LDS before they are written (an even count), and the blocks per
// resident workgroup slot from which the loop pays.
constexpr int kPsOut = 16;
constexpr int kLoopBlocksPerSlot = 2;
// (a sixteen-wave loop for one-row 2-bit decode from three blocks per resident workgroup: at two
// it lost to the eight-wave one-shot grid, 11008 -> 8192: 7.19 -> 7.86 us)
constexpr int kTallBlocksPerSlot = 3;

template <int FMT, int NW, int CST, int GL, bool ONE, int MR, int RB, bool PS>
__global__ __launch_bounds__(64 * NW) void k_mv1(const uint16_t *__restrict__ X, const Groups gr, int M, int K, int C,
                                                 const Fusion fu)
{
    static_assert(MR == 1 || ((MR == 2 || MR == 4) && GL == 0), "several activation rows: the plain layer (and the residual) only");
    static_assert(RB == 1 || GL == 0, "several row blocks: the plain layer (and the residual) only");
    static_assert(!PS || (GL == 0 && RB == 1 && ONE), "block loop: one matrix, the plain layer (and the residual) only");
    constexpr bool NORM = (GL & kGlueNorm) != 0;
    constexpr bool PAIR = (GL & kGluePair) != 0;
    const GroupSel grp = select_group<ONE>(gr, fu, (int)blockIdx.x);
    const uint8_t *__restrict__ Wp = grp.Wp;
    uint16_t *__restrict__ Y = grp.Y;
    const float scale = grp.scale;
    const int N = grp.N;
    constexpr bool TWO = FMT == TRI_FMT_2BIT;
    constexpr int XH = TWO ? 64 : 80;            // activations per chunk
    constexpr int NOP = TWO ? 8 : 10;            // A operands (MFMAs) per chunk
    constexpr int NCLS = TWO ? 6 : 4;            // accumulators: position classes (2-bit); two sums by halves (1.6-bit)
    constexpr int NCH = 4 * CST;                 // chunks per wave
    constexpr int PIECES = XH / 8;               // 16-byte activation pieces per chunk
    constexpr int NLD = (NCH * PIECES + 63) / 64;   // whole-line activation loads per lane
    static_assert(NCH <= 64, "chunks per wave");
    // per wave: A operands of its chunks, per activation row.  2-bit: chunk-major (four rows: one
    // 16-byte pad per row, so the rows one read instruction touches fall in distinct banks).
    // 1.6-bit: row-major, chunk after chunk, each row padded by 16 bytes for the same reason; a
    // row is staged in place (the ten raw pieces of chunk l occupy the 160 bytes its ten A
    // operands will), so no separate bounce buffer is needed.
    constexpr int NOPP = MR == 4 ? NOP + 1 : NOP;
    constexpr int XBR = NCH * NOP + 1;           // 1.6-bit: 16-byte slots per row (+ pad)
    __shared__ u32x4 xa[TWO ? NW : 1][TWO ? NCH : 1][TWO ? MR : 1][TWO ? NOPP : 1];
    __shared__ u32x4 xb[TWO ? 1 : NW][TWO ? 1 : MR][TWO ? 1 : XBR];
    // per wave and activation row: the 16 outputs of each block, sum x (, sum x^2)
    __shared__ float red[PS ? 2 : 1][NW][MR][16 * RB + (NORM ? 2 : 1)];   // (block loop: two, alternating)
    __shared__ float yst[PS ? kPsOut : 1][MR][16];   // block loop: outputs not yet written
    __shared__ float red1[PAIR ? NW : 1][16];    // pair: the second matrix's rows

    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform (scalar descriptors)
    const int g = lane >> 4;
    const int j = lane & 15;
    const int n0 = ((int)blockIdx.x - grp.first) * 16 * RB;
    const int64_t S = (int64_t)C * 16;

    // (1) activations of this wave's chunks: local chunk l is global chunk
    //     4*((l/4)*NW + w) + l%4; piece P = 64i + lane of the wave's pieces is piece P % PIECES
    //     of local chunk P / PIECES, so a load instruction reads whole 128-byte lines
    //     (several activation rows: the same pieces of each row, rows past M reading as zero)
    const __amdgpu_buffer_rsrc_t xr =
        rsrc(X, __builtin_amdgcn_readfirstlane((uint32_t)min(M, MR) * (uint32_t)K * 2u));
    u32x4 xv[MR][NLD], nv[NORM ? NLD : 1];
#pragma unroll
    for (int r = 0; r < MR; ++r)
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
            const int P = 64 * i + lane;
            const int l = P / PIECES;
            const int gc = 4 * ((l >> 2) * NW + wv) + (l & 3);
            const int k = gc * XH + 8 * (P % PIECES);
            const int off = (l < NCH && k < K) ? (int)((uint32_t)(r * K + k) * 2u) : (int)0x80000000u;
            xv[r][i] = __builtin_amdgcn_raw_buffer_load_b128(xr, off, 0, 0);
            if constexpr (NORM) {                // the norm gain of the same activations
                if (fu.gain) nv[i] = __builtin_amdgcn_raw_buffer_load_b128(rsrc(fu.gain, (uint32_t)K * 2u), off, 0, 0);
            }
        }
    // (2) every weight chunk of the wave, all in flight at once.  Block loop (PS): the workgroup
    //     takes blocks blockIdx.x, + gridDim.x, ...; one resource spans the matrix, and the chunks
    //     of a block past its end read as zero
    const int rows_here = PS ? N : min(16 * RB, N - n0);
    const __amdgpu_buffer_rsrc_t wr =
        rsrc(Wp + (PS ? 0 : (int64_t)n0 * S), __builtin_amdgcn_readfirstlane((uint32_t)(rows_here * S)));
    // (pair: the same chunks of the second matrix, requested in the order they are used)
    const __amdgpu_buffer_rsrc_t wr1 =
        rsrc(gr.Wp[PAIR ? 1 : 0] + (int64_t)n0 * S, __builtin_amdgcn_readfirstlane((uint32_t)(rows_here * S)));
    const int nblk = (N + 15) / 16;
    auto load_block = [&](int b, u32x4 (&w)[RB][CST]) __attribute__((always_inline)) {
#pragma unroll
        for (int s = 0; s < CST; ++s) {
            const int c = 4 * (s * NW + wv) + g;
            const bool live = c < C && (!PS || b < nblk);
#pragma unroll
            for (int r = 0; r < RB; ++r)         // (rows past the matrix's end read as zero)
                w[r][s] = __builtin_amdgcn_raw_buffer_load_b128(
                    wr, live ? (int)(uint32_t)((16 * (PS ? b : r) + j) * S + c * 16) : (int)0x80000000u, 0, 0);
        }
    };
    u32x4 wq[RB][CST], wq1[PAIR ? CST : 1], wqb[PS ? RB : 1][PS ? CST : 1];
    load_block((int)blockIdx.x, wq);
    if constexpr (PAIR) {
#pragma unroll
        for (int s = 0; s < CST; ++s) {
            const int c = 4 * (s * NW + wv) + g;
            wq1[s] = __builtin_amdgcn_raw_buffer_load_b128(wr1, c < C ? (int)(uint32_t)(j * S + c * 16) : (int)0x80000000u, 0, 0);
        }
    }

    // (3) norm: sum of squares, then x -> fp16(x * gain); A operands in LDS and this lane's
    //     share of sum_k x
    float xsq = 0.f;
    if constexpr (NORM) {
#pragma unroll
        for (int i = 0; i < NLD; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                xsq = dot2(xv[0][i][e], xv[0][i][e], xsq);
                if (fu.gain) xv[0][i][e] = mul2(xv[0][i][e], nv[i][e]);
            }
    }
    float xsum[MR];
#pragma unroll
    for (int r = 0; r < MR; ++r) {
        xsum[r] = 0.f;
#pragma unroll
        for (int i = 0; i < NLD; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) xsum[r] = dot2(xv[r][i][e], 0x3C003C00u, xsum[r]);   // (x_lo, x_hi) . (1, 1)
    }
    if constexpr (TWO) {
        // lanes 2v, 2v+1 of a chunk's eight hold x[16v .. 16v+7] and x[16v+8 .. 16v+15]; the even
        // lane forms positions 0..3 from registers 0, 1 of both pieces, the odd one 4..7 from
        // registers 2, 3.  Each lane keeps the two registers it needs of its own piece and sends the
        // two its partner needs (DPP quad_perm [1,0,3,2]); one byte permute per A operand then puts
        // the value of trit 16v+p in the low half (the even lane's own, the odd lane's received)
        const bool odd = lane & 1;
        const int vv = (lane & 7) >> 1;
        const uint32_t sel0 = odd ? 0x05040100u : 0x01000504u;   // low halves: (received, own) / (own, received)
        const uint32_t sel1 = odd ? 0x07060302u : 0x03020706u;   // high halves, the same way
#pragma unroll
        for (int r = 0; r < MR; ++r)
#pragma unroll
            for (int i = 0; i < NLD; ++i) {
                const int l = (64 * i + lane) / PIECES;
                const u32x4 m = xv[r][i];
                uint32_t own[2], rcv[2];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    own[h] = odd ? m[2 + h] : m[h];
                    rcv[h] = (uint32_t)__builtin_amdgcn_mov_dpp((int)(odd ? m[h] : m[2 + h]), 0xB1, 0xF, 0xF, false);
                }
#pragma unroll
                for (int pp = 0; pp < 4; ++pp) {
                    const uint32_t v = perm(own[pp / 2], rcv[pp / 2], (pp & 1) ? sel1 : sel0);
                    if (l < NCH) reinterpret_cast<uint32_t *>(&xa[wv][l][r][pp + (odd ? 4 : 0)])[vv] = v;
                }
            }
    } else {
        // the pairing of a 40-value half spans ten pieces: bounce the raw pieces through the
        // row's own slots (piece P of the wave's pieces to slot P), then lane l reads the ten
        // pieces of chunk l and overwrites the same ten slots with its A operands (no other lane
        // reads them after the barrier)
#pragma unroll
        for (int r = 0; r < MR; ++r)
#pragma unroll
            for (int i = 0; i < NLD; ++i)
                if (64 * i + lane < NCH * PIECES) xb[wv][r][64 * i + lane] = xv[r][i];
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int r = 0; r < MR; ++r) {
            if (lane < NCH) {
                uint32_t x32[40];
#pragma unroll
                for (int q = 0; q < 10; ++q) {
                    const u32x4 v = xb[wv][r][10 * lane + q];
                    x32[4 * q] = v[0]; x32[4 * q + 1] = v[1]; x32[4 * q + 2] = v[2]; x32[4 * q + 3] = v[3];
                }
#pragma unroll
                for (int p = 0; p < 5; ++p)
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh) {
                        u32x4 av;
#pragma unroll
                        for (int qq = 0; qq < 4; ++qq) {
                            const int e = 5 * (4 * hh + qq) + p;   // value index; partner e + 40
                            av[qq] = (e & 1) ? pair_halves<1>(x32[(e >> 1) + 20], x32[e >> 1])
                                             : pair_halves<0>(x32[(e >> 1) + 20], x32[e >> 1]);
                        }
                        xb[wv][r][10 * lane + 2 * p + hh] = av;
                    }
            }
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // (4) decode and contract, one MFMA per position (and half, 1.6-bit)
    const float4_t zero4 = {0.f, 0.f, 0.f, 0.f};
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
            // sum x_p q_{p+1}, by halves (every quotient carries the same scale)
            uint32_t qt[8][5];
#pragma unroll
            for (int q = 0; q < 8; ++q) base3_quotients_u16x2(byte_pair(v, q), qt[q]);
#pragma unroll
            for (int p = 0; p < 5; ++p) {
                ac[0] = mfma(a[2 * p], u32x4{qt[0][p], qt[1][p], qt[2][p], qt[3][p]}, ac[0]);
                ac[1] = mfma(a[2 * p + 1], u32x4{qt[4][p], qt[5][p], qt[6][p], qt[7][p]}, ac[1]);
                if (p < 4) {
                    ac[2] = mfma(a[2 * p], u32x4{qt[0][p + 1], qt[1][p + 1], qt[2][p + 1], qt[3][p + 1]}, ac[2]);
                    ac[3] = mfma(a[2 * p + 1], u32x4{qt[4][p + 1], qt[5][p + 1], qt[6][p + 1], qt[7][p + 1]}, ac[3]);
                }
            }
        }
    };
    // (5) merge classes (D row i holds activation row i % MR; rows 0..MR-1 are elements 0..MR-1
    //     of lanes 0..15), add the waves' partial sums in a fixed order, subtract sum_k x, scale,
    //     round
    auto merge = [&](const float4_t (&ac)[NCLS]) __attribute__((always_inline)) {
        if constexpr (!TWO) return (ac[0] + ac[1]) - 3.f * (ac[2] + ac[3]);   // digits d_p = q_p - 3 q_{p+1}
        float4_t t = ac[0] + 0.25f * ac[1];
        t += 0.0625f * ac[2] + 0.015625f * ac[3];
        t += 0.00390625f * ac[4] + 0.0009765625f * ac[5];
        return t;
    };
    const float xs_wave = wave_reduce_rows<MR>(xsum, lane);   // lane group r (of 64 / MR lanes): row r
    float xq_wave = 0.f;
    if constexpr (NORM) {
        float xq[1] = {xsq};
        xq_wave = wave_reduce_rows<1>(xq, lane);
    }
    // steps (4) and (5) for the blocks whose weight chunks are in w, the first at row nb, through
    // partial-sum buffer rbuf
    auto run = [&](const u32x4 (&w)[RB][CST], int nb, int rbuf, int slot) __attribute__((always_inline)) {
        float4_t acc[RB][NCLS], acc1[PAIR ? NCLS : 1];
#pragma unroll
        for (int r = 0; r < RB; ++r)
#pragma unroll
            for (int c = 0; c < NCLS; ++c) acc[r][c] = zero4;
#pragma unroll
        for (int c = 0; c < (PAIR ? NCLS : 1); ++c) acc1[c] = zero4;
#pragma unroll
        for (int s = 0; s < CST; ++s) {
            // wave-uniform: no chunk of this step is live (the block loop contracts such steps,
            // whose activations are zero: a skipped step would leave its loads pending; step 0
            // always runs, so every accumulator's first MFMA takes a literal zero)
            if (!PS && s > 0 && 4 * (s * NW + wv) >= C) break;
            const u32x4 *asrc;                   // A row j: activation row j % MR
            if constexpr (TWO) asrc = &xa[wv][4 * s + g][j % MR][0];
            else asrc = &xb[wv][j % MR][(4 * s + g) * NOP];
            u32x4 a[NOP];
#pragma unroll
            for (int p = 0; p < NOP; ++p) a[p] = asrc[p];
#pragma unroll
            for (int r = 0; r < RB; ++r) contract(a, w[r][s], acc[r]);
            if constexpr (PAIR) contract(a, wq1[s], acc1);
        }
        auto &rd = red[rbuf];
#pragma unroll
        for (int r = 0; r < RB; ++r) {
            const float4_t t = merge(acc[r]);
            if (g == 0) {
#pragma unroll
                for (int e = 0; e < MR; ++e) rd[wv][e][16 * r + j] = t[e];
            }
        }
        if ((lane & (64 / MR - 1)) == 0) rd[wv][lane / (64 / MR)][16 * RB] = xs_wave;
        if constexpr (PAIR) {
            const float4_t t1 = merge(acc1);
            if (g == 0) red1[wv][j] = t1[0];
        }
        if constexpr (NORM) {
            if (lane == 0) rd[wv][0][16 * RB + 1] = xq_wave;
        }
        __syncthreads();
        const int e = threadIdx.x / (16 * RB), jj = threadIdx.x % (16 * RB);   // thread (e, jj): output Y[e][nb + jj]
        if (threadIdx.x < 16 * RB * MR && e < M && nb + jj < N) {
            float sd = 0.f, sx = 0.f;
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                sd += rd[w][e][jj];
                sx += rd[w][e][16 * RB];
            }
            float rinv = 1.f;
            if constexpr (NORM) {
                float sq = 0.f;
#pragma unroll
                for (int w = 0; w < NW; ++w) sq += rd[w][0][16 * RB + 1];
                rinv = __builtin_amdgcn_rsqf(sq * __builtin_amdgcn_rcpf((float)K) + fu.eps);   // (v_rsq, v_rcp: about 1 ulp)
            }
            float y = (sd * 16777216.0f - sx) * scale * rinv;
            if constexpr (PAIR) {
                float sd1 = 0.f;
#pragma unroll
                for (int w = 0; w < NW; ++w) sd1 += red1[w][jj];
                const float y1 = (sd1 * 16777216.0f - sx) * gr.scale[1] * rinv;
                y = y / (1.f + __expf(-y)) * y1;     // silu(gate) * up
            }
            if constexpr (PS) {
                yst[slot][e][jj] = y;            // (written out by the flush below)
            } else {
                const int64_t o = (int64_t)e * N + nb + jj;
                if (grp.res) y += h2f(grp.res[o]);
                Y[o] = __builtin_bit_cast(uint16_t, (_Float16)y);
            }
        }
    };
    if constexpr (!PS) {
        run(wq, n0, 0, 0);
    } else {
        // Two register sets in turn: the next block's chunks are in flight while one is
        // contracted, and the two partial-sum buffers alternate, so one barrier per block
        // suffices.  Outputs wait in LDS and are written kPsOut blocks at a time, away from the
        // loads in flight.
        const int G = (int)gridDim.x;
        int done = 0;                            // blocks of this workgroup whose outputs are written
        auto flush = [&](int upto) __attribute__((always_inline)) {
            __syncthreads();
            for (int t = (int)threadIdx.x; t < (upto - done) * MR * 16; t += 64 * NW) {
                const int i = t / (MR * 16), e = (t / 16) % MR, jj = t % 16;
                const int n = 16 * ((int)blockIdx.x + (done + i) * G) + jj;
                if (e < M && n < N) {
                    const int64_t o = (int64_t)e * N + n;
                    float y = yst[i][e][jj];
                    if (grp.res) y += h2f(grp.res[o]);
                    Y[o] = __builtin_bit_cast(uint16_t, (_Float16)y);
                }
            }
            __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): no store stays pending into the loop
            __syncthreads();
            done = upto;
        };
        // (The exit between the two halves costs a drain of the loads in flight at the top of
        // the loop, which the compiler inserts; contracting a phantom block past the matrix
        // instead measured slower.)
        int i = 0;                               // blocks of this workgroup contracted
        for (int b = (int)blockIdx.x; b < nblk; b += 2 * G, i += 2) {
            load_block(b + G, wqb);
            run(wq, 16 * b, 0, i - done);
            if (b + G >= nblk) {
                ++i;
                break;
            }
            load_block(b + 2 * G, wq);
            run(wqb, 16 * (b + G), 1, i + 1 - done);
            if (i + 2 - done == kPsOut) flush(i + 2);
        }
        flush(i);
    }
}

// One matrix of many blocks (at least kLoopBlocksPerSlot per resident workgroup): a resident
// grid that loops over the blocks.  Eight waves at most (sixteen would spill the second register
// set); no glue but the residual.
template <int FMT, int NW, int CST, int MR>
static bool launch_loop(const uint16_t *X, const Groups &gr, int M, int K, int C, hipStream_t s, const Fusion &f)
{
    constexpr int kXaBytes = xa_bytes<FMT, NW, CST, MR>();
    // (eight waves, or sixteen of up to four steps at one 2-bit row: more would spill the second
    // register set; the staged operands' LDS as below)
    if constexpr ((NW > 8 && !(NW == 16 && CST <= 4 && MR == 1 && FMT == TRI_FMT_2BIT)) ||
                  (MR > 1 && kXaBytes > (MR == 4 ? 120 : 100) * 1024)) {
        return false;
    } else {
        if (gr.G != 1 || (int64_t)gr.N[0] * C * 16 >= ((int64_t)1 << 31)) return false;
        const int resident = resident_per_cu<k_mv1<FMT, NW, CST, 0, true, MR, 1, true>>(64 * NW) * cu_count();
        if ((int64_t)gr.blk[1] < (int64_t)kLoopBlocksPerSlot * resident) return false;
        hipLaunchKernelGGL((k_mv1<FMT, NW, CST, 0, true, MR, 1, true>), dim3(resident), dim3(64 * NW), 0, s, X, gr, M, K,
                           C, f);
        return true;
    }
}

// Matrices of the group with at least kTallBlocksPerSlot 16-row blocks per workgroup of the NW-wave
// block loop that the device holds at once.
template <int FMT, int NW, int CST>
static int tall_count(const Groups &gr)
{
    const int64_t resident = (int64_t)resident_per_cu<k_mv1<FMT, NW, CST, 0, true, 1, 1, true>>(64 * NW) * cu_count();
    int n = 0;
    for (int g = 0; g < gr.G; ++g) n += (int64_t)(gr.blk[g + 1] - gr.blk[g]) >= kTallBlocksPerSlot * resident;
    return n;
}

template <int FMT, int NW, int CST, int GL, int MR, int RB>
static bool launch_gl(const uint16_t *X, const Groups &gr, int M, int K, int C, hipStream_t s, const Fusion &f)
{
    // several activation rows: only while the staged A operands of the workgroup stay below
    // 100 KB of LDS (120 KB at four rows, 136 KB at sixteen waves, whose registers hold one
    // workgroup per CU anyway)
    constexpr int kXaBytes = xa_bytes<FMT, NW, CST, MR>();
    if constexpr (MR > 1 && kXaBytes > (NW == 16 ? 136 : MR == 4 ? 120 : 100) * 1024) {
        return false;
    } else {
        const Groups g = RB == 1 ? gr : regroup(gr, RB);
        const dim3 grid(g.blk[g.G]), block(64 * NW);
        if constexpr (GL == 0 && RB == 1) {
            if (launch_loop<FMT, NW, CST, MR>(X, gr, M, K, C, s, f)) return true;
        }
        if constexpr (FMT == TRI_FMT_1P6BIT && MR == 4) return false;   // (1.6-bit, four rows: the block loop only)
        if (g.G == 1)
            hipLaunchKernelGGL((k_mv1<FMT, NW, CST, GL, true, MR, RB, false>), grid, block, 0, s, X, g, M, K, C, f);
        else
            hipLaunchKernelGGL((k_mv1<FMT, NW, CST, GL, false, MR, RB, false>), grid, block, 0, s, X, g, M, K, C, f);
        return true;
    }
}

// Four 16-row blocks per workgroup (2-bit, eight waves, no glue but the residual): every
// activation value a wave stages feeds four blocks.  At one or two rows it pays only while the
// grid of four-block workgroups fills most CUs once (4096 -> 14336, 224 of them: 5.48 -> 5.25 us
// at M = 1) and loses both below about 200 (4096 -> 11008: 5.03 -> 5.24 us) and past one per CU,
// where the last ones run alone (2 x 11008 grouped, 344: 7.01 -> 8.50 us).  At four rows the
// activation traffic weighs more and it wins from about 160 on (4096 -> 11008 at M = 4: 6.98 ->
// 5.89 us).  Two blocks lost wherever four did not win, so they are not used.  At four rows three
// blocks are taken where they cost less by rounds x (1 + blocks) of one workgroup per CU (688
// blocks: 230 workgroups in one round instead of 172; 4096 -> 11008 5.99 -> 5.86 us); at one row
// they lose like four (4096 -> 11008: 4.66 -> 5.02 us).  Returns 1, 3 or 4.
template <int FMT, int NW, int CST, int MR>
static int wide_rb(const Groups &gr, const Fusion *fu)
{
    if constexpr (FMT != TRI_FMT_2BIT || NW != 8 || (MR == 2 && CST > 6)) {
        return 1;
    } else {
        if (glue_bits(fu)) return 1;
        const int64_t cus = cu_count();
        const int w4 = regroup(gr, 4).blk[gr.G], w3 = regroup(gr, 3).blk[gr.G];
        if constexpr (MR == 4) {                 // (rounds of one workgroup per CU, each costing about 1 + RB blocks)
            if (w4 < 160) return 1;
            return (w3 + cus - 1) / cus * 4 < (w4 + cus - 1) / cus * 5 ? 3 : 4;
        } else {
            return w4 >= (MR == 1 ? 200 : 160) && w4 <= cus ? 4 : 1;
        }
    }
}

template <int FMT, int NW, int CST, int MR>
static bool launch_cfg(const uint16_t *X, const Groups &gr, int M, int K, int C, hipStream_t s, const Fusion *fu)
{
    const Fusion f = fu ? *fu : Fusion{};
    const int rbw = wide_rb<FMT, NW, CST, MR>(gr, fu);
    if constexpr (MR > 1) {                      // (no glue but the residual)
        if constexpr (FMT == TRI_FMT_2BIT && NW == 8 && (MR == 4 || CST <= 6)) {
            // (a tall matrix: the block loop before several-block workgroups)
            if (rbw > 1 && launch_loop<FMT, NW, CST, MR>(X, gr, M, K, C, s, f)) return true;
            if (rbw == 4) return launch_gl<FMT, NW, CST, 0, MR, 4>(X, gr, M, K, C, s, f);
            if constexpr (MR == 4) {             // (three blocks: four rows only)
                if (rbw == 3) return launch_gl<FMT, NW, CST, 0, MR, 3>(X, gr, M, K, C, s, f);
            }
        }
        return launch_gl<FMT, NW, CST, 0, MR, 1>(X, gr, M, K, C, s, f);
    } else {
        const int gl = glue_bits(fu);
        if constexpr (NW == 8) {                 // (pair variants: eight waves only, see launch_fmt)
            if (gl == kGluePair) return launch_gl<FMT, NW, CST, kGluePair, 1, 1>(X, gr, M, K, C, s, f);
            if (gl == (kGlueNorm | kGluePair))
                return launch_gl<FMT, NW, CST, kGlueNorm | kGluePair, 1, 1>(X, gr, M, K, C, s, f);
        }
        if constexpr (NW == 16) {                // (the norm serves rows of up to eight steps: eight waves)
            if (gl) return false;
        } else {
            if (gl & kGlueNorm) return launch_gl<FMT, NW, CST, kGlueNorm, 1, 1>(X, gr, M, K, C, s, f);
        }
        if constexpr (FMT == TRI_FMT_2BIT && NW == 8) {
            if (rbw == 4) return launch_gl<FMT, NW, CST, 0, 1, 4>(X, gr, M, K, C, s, f);
        }
        return launch_gl<FMT, NW, CST, 0, 1, 1>(X, gr, M, K, C, s, f);
    }
}

// Eight waves per 16 rows (measured best at K = 4096 and 11008 for 2-bit); sixteen for long rows.
template <int FMT, int MR>
static bool launch_fmt(const uint16_t *X, const Groups &gr, int M, int K, int C, hipStream_t s, const Fusion *fu)
{
    // 1.6-bit rows of up to 64 chunks: four waves with twice the steps each, so a wave's decode
    // of one step overlaps the arrival of the next (3-6% faster at K = 4096; equal at 11008, and
    // slower for 2-bit, whose decode is cheap)
    if constexpr (FMT == TRI_FMT_1P6BIT) {
        if (!glue_bits(fu) && C <= 64) {
            switch ((C + 15) / 16) {
            case 1: return launch_cfg<FMT, 4, 1, MR>(X, gr, M, K, C, s, fu);
            case 2: return launch_cfg<FMT, 4, 2, MR>(X, gr, M, K, C, s, fu);
            case 3: return launch_cfg<FMT, 4, 3, MR>(X, gr, M, K, C, s, fu);
            default: return launch_cfg<FMT, 4, 4, MR>(X, gr, M, K, C, s, fu);
            }
        }
    }
    const int cst8 = (C + 31) / 32;              // chunk-steps with 8 waves (4 chunks per step and wave)
    // Tall 2-bit matrices with rows of five to eight steps per wave of eight (8192 < K <= 16384) at one
    // row: sixteen waves of three or four steps, whose block loop over the matrix keeps four waves per
    // SIMD instead of two (11008 -> 14336: 12.9 -> 11.9 us, 16384 -> 16384: 20.5 -> 17.2 us; at two blocks
    // per resident workgroup it loses, 11008 -> 8192: 7.2 -> 7.9 us, and a one-shot grid gains nothing
    // on sixteen waves, so shorter matrices keep eight).  A matrix is tall when it has at least
    // kTallBlocksPerSlot blocks per resident sixteen-wave workgroup;
    // the choice is made per matrix, so a single, a grouped and a residual launch of it take the same
    // kernel (bitwise equal results), and a group that mixes tall and short matrices runs one launch per
    // matrix.  The norm and pair glue keep eight waves.
    if constexpr (FMT == TRI_FMT_2BIT && MR == 1) {
        if (!glue_bits(fu) && cst8 >= 5 && cst8 <= 8) {
            const int tall = cst8 <= 6 ? tall_count<FMT, 16, 3>(gr) : tall_count<FMT, 16, 4>(gr);
            if (tall == gr.G)
                return cst8 <= 6 ? launch_cfg<FMT, 16, 3, 1>(X, gr, M, K, C, s, fu)
                                 : launch_cfg<FMT, 16, 4, 1>(X, gr, M, K, C, s, fu);
            if (tall > 0) {                      // (tall and short matrices in one group: one launch each)
                for (int g = 0; g < gr.G; ++g) {
                    const Groups one = make_groups(1, &gr.Wp[g], &gr.scale[g], &gr.N[g], &gr.Y[g]);
                    Fusion f1 = fu ? *fu : Fusion{};
                    f1.res[0] = f1.res[g];
                    for (int q = 1; q < kMaxGroups; ++q) f1.res[q] = nullptr;
                    if (!launch_fmt<FMT, MR>(X, one, M, K, C, s, fu ? &f1 : nullptr)) return false;
                }
                return true;
            }
        }
    }
    // The other 2-bit one-row matrices with rows of five or six eight-wave steps (8192 < K <= 12288):
    // twelve waves of four steps, three waves per SIMD instead of two (11008 -> 4096: 4.99 -> 4.88 us;
    // sixteen waves of three measured equal to eight).  The choice depends on the matrix alone, so
    // single, grouped and residual launches of it take the same kernel.
    if constexpr (FMT == TRI_FMT_2BIT && MR == 1) {
        if (!glue_bits(fu) && (cst8 == 5 || cst8 == 6)) return launch_cfg<FMT, 12, 4, 1>(X, gr, M, K, C, s, fu);
    }
    switch (cst8) {
    case 1: return launch_cfg<FMT, 8, 1, MR>(X, gr, M, K, C, s, fu);
    case 2: return launch_cfg<FMT, 8, 2, MR>(X, gr, M, K, C, s, fu);
    case 3: return launch_cfg<FMT, 8, 3, MR>(X, gr, M, K, C, s, fu);
    case 4: return launch_cfg<FMT, 8, 4, MR>(X, gr, M, K, C, s, fu);
    case 5: return launch_cfg<FMT, 8, 5, MR>(X, gr, M, K, C, s, fu);
    case 6: return launch_cfg<FMT, 8, 6, MR>(X, gr, M, K, C, s, fu);
    case 7: return launch_cfg<FMT, 8, 7, MR>(X, gr, M, K, C, s, fu);
    case 8: return launch_cfg<FMT, 8, 8, MR>(X, gr, M, K, C, s, fu);
    default: break;
    }
    // sixteen waves (one or two activation rows); the staged activations of a workgroup must fit
    // in LDS.  (The pair variant would exceed the registers a wave has at sixteen waves: longer
    // rows are not paired.)
    if constexpr (MR <= 2) {
        if (fu && fu->pair) return false;
        const int cst16 = (C + 63) / 64;
        if (cst16 <= 6) return launch_cfg<FMT, 16, 6, MR>(X, gr, M, K, C, s, fu);
        if constexpr (FMT == TRI_FMT_2BIT) {
            if (cst16 <= 8) return launch_cfg<FMT, 16, 8, MR>(X, gr, M, K, C, s, fu);
            if constexpr (MR == 1) {
                if (cst16 <= 12) return launch_cfg<FMT, 16, 12, 1>(X, gr, M, K, C, s, fu);
            }
        }
    }
    return false;                                // longer rows: the streaming small-M kernel
}

bool launch_mv1(const uint16_t *X, const Groups &gr, int K, int fmt, hipStream_t s, const Fusion *fu)
{
    const int C = (int)(row_bytes(K, fmt) / 16);
    // 32-bit buffer offsets: the activation row and one 16-row block stay below 2^31 bytes;
    // activations are read in pieces of 8 values, so K must be a multiple of 8
    if ((K % 8) != 0 || (int64_t)K * 2 >= ((int64_t)1 << 31) || 16 * (int64_t)C * 16 >= ((int64_t)1 << 31))
        return false;
    return fmt == TRI_FMT_2BIT ? launch_fmt<TRI_FMT_2BIT, 1>(X, gr, 1, K, C, s, fu)
                             : launch_fmt<TRI_FMT_1P6BIT, 1>(X, gr, 1, K, C, s, fu);
}

bool launch_mvr(const uint16_t *X, const Groups &gr, int M, int K, int fmt, hipStream_t s, const Fusion *fu)
{
    const int C = (int)(row_bytes(K, fmt) / 16);
    // (as above, for up to four activation rows; of the glue, the residual only)
    if (M < 2 || M > 4 || glue_bits(fu) || (K % 8) != 0 || (int64_t)4 * K * 2 >= ((int64_t)1 << 31) ||
        16 * (int64_t)C * 16 >= ((int64_t)1 << 31))
        return false;
    if (fmt == TRI_FMT_2BIT)
        return M == 2 ? launch_fmt<TRI_FMT_2BIT, 2>(X, gr, M, K, C, s, fu)
                      : launch_fmt<TRI_FMT_2BIT, 4>(X, gr, M, K, C, s, fu);
    // 1.6-bit: two rows; three and four only as the block loop over a tall matrix (8192 -> 28672
    // at M = 4: 32.4 -> 22.5 us; a one-shot grid of four rows was 3-50% slower than the batched
    // kernel)
    return M == 2 ? launch_fmt<TRI_FMT_1P6BIT, 2>(X, gr, M, K, C, s, fu)
                  : launch_fmt<TRI_FMT_1P6BIT, 4>(X, gr, M, K, C, s, fu);
}

}  // namespace tri
