// tri_device.h -- device-side helpers shared by the libtri kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tri {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// Two fp16 lanes of a 32-bit register.
__device__ __forceinline__ half2_t as_h2(uint32_t v) { return __builtin_bit_cast(half2_t, v); }

// v_dot2_f32_f16: c + a.lo*b.lo + a.hi*b.hi with fp32 accumulation.  fp16 subnormal
// inputs are honoured (verified on gfx950), which the trit decoders below rely on.
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c)
{
    return __builtin_amdgcn_fdot2(as_h2(a), as_h2(b), c, false);
}

// An fp16 bit pattern as fp32.
__device__ __forceinline__ float h2f(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }

// fp16_rne(a * b) lane by lane: one packed fp16 multiply (IEEE, round to nearest even; the
// same result as rounding the exact fp32 product).
__device__ __forceinline__ uint32_t mul2(uint32_t a, uint32_t b)
{
    return __builtin_bit_cast(uint32_t, as_h2(a) * as_h2(b));
}

// v_perm_b32: byte i of the result is byte sel_i of the 8-byte value {hi:lo}.
__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel)
{
    return __builtin_amdgcn_perm(hi, lo, sel);
}

// fp16 lane `e` (0 = low half, 1 = high half) of `lo` and lane `e` of `hi`, packed as (lo, hi).
template <int E>
__device__ __forceinline__ uint32_t pair_halves(uint32_t hi, uint32_t lo)
{
    return perm(hi, lo, E == 0 ? 0x05040100u : 0x07060302u);
}

// v_mfma_f32_16x16x32_f16: D[16x16] += A[16x32] * B[32x16]; lane (g = lane/16, l = lane%16)
// supplies A[l][8g..8g+7] and B[8g..8g+7][l] as four registers of fp16 pairs and holds
// D[4g..4g+3][l] (layout and fp16-subnormal handling verified on gfx950).
__device__ __forceinline__ float4_t mfma16(const uint32_t a0, const uint32_t a1, const uint32_t a2, const uint32_t a3,
                                           const uint32_t b0, const uint32_t b1, const uint32_t b2, const uint32_t b3,
                                           float4_t c)
{
    const u32x4 av = {a0, a1, a2, a3};
    const u32x4 bv = {b0, b1, b2, b3};
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, av), __builtin_bit_cast(half8_t, bv), c,
                                                  0, 0, 0);
}

__device__ __forceinline__ float4_t mfma16(const uint4 a, const uint32_t b0, const uint32_t b1, const uint32_t b2,
                                           const uint32_t b3, float4_t c)
{
    return mfma16(a.x, a.y, a.z, a.w, b0, b1, b2, b3, c);
}

// The five base-3 digits of byte b (digit j = floor(b / 3^j) mod 3), two bits each at bits 2j:
// the table that turns a 1.6-bit byte into the 2-bit digit layout.
__device__ __forceinline__ uint32_t base3_digits_2bit(uint32_t b)
{
    uint32_t code = 0;
#pragma unroll
    for (int j = 0; j < 5; ++j) {
        const uint32_t q = b / 3u;
        code |= (b - 3u * q) << (2 * j);
        b = q;
    }
    return code;
}

// Base-3 digits of two bytes at once, for the 1.6-bit packing ("Spectra 1.1", Pith review,
// "Referee Report" minor comment 5: the decode is the repeated division b'_i -> x_i).  `b`
// holds one byte value per 16-bit lane; digit j of both is returned in d[j], one per lane:
// d[j] = q_j - 3 q_{j+1} with q_j = floor(b / 3^j), each quotient an exact multiply-shift
// (b*171 >> 9, b*57 >> 9, b*19 >> 9, b*203 >> 14; exact and below 2^16 for every b < 256).
// A lane's digit read as fp16 bits is the exact value d * 2^-24.
__device__ __forceinline__ void base3_digits_u16x2(uint32_t b, uint32_t (&d)[5])
{
    typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));
    const u16x2 v = __builtin_bit_cast(u16x2, b);
    const u16x2 q1 = (v * (uint16_t)171) >> (uint16_t)9;
    const u16x2 q2 = (v * (uint16_t)57) >> (uint16_t)9;
    const u16x2 q3 = (v * (uint16_t)19) >> (uint16_t)9;
    const u16x2 q4 = (v * (uint16_t)203) >> (uint16_t)14;
    d[0] = __builtin_bit_cast(uint32_t, (u16x2)(v - q1 * (uint16_t)3));
    d[1] = __builtin_bit_cast(uint32_t, (u16x2)(q1 - q2 * (uint16_t)3));
    d[2] = __builtin_bit_cast(uint32_t, (u16x2)(q2 - q3 * (uint16_t)3));
    d[3] = __builtin_bit_cast(uint32_t, (u16x2)(q3 - q4 * (uint16_t)3));
    d[4] = __builtin_bit_cast(uint32_t, q4);
}

// The quotients q_j = floor(b / 3^j), j = 0..4, of two bytes at once (q_0 = b), by the same
// multiply-shifts.  Since d_j = q_j - 3 q_{j+1} (q_5 = 0), a dot product with the digits is
//   sum_j x_j d_j = sum_j x_j q_j - 3 sum_{j<4} x_j q_{j+1},
// two dot products with the quotients, which saves the four multiply-subtracts of the digits.
// Every quotient is below 2^8, so its bits read as fp16 are the exact value q * 2^-24.
__device__ __forceinline__ void base3_quotients_u16x2(uint32_t b, uint32_t (&q)[5])
{
    typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));
    const u16x2 v = __builtin_bit_cast(u16x2, b);
    q[0] = b;
    q[1] = __builtin_bit_cast(uint32_t, (u16x2)((v * (uint16_t)171) >> (uint16_t)9));
    q[2] = __builtin_bit_cast(uint32_t, (u16x2)((v * (uint16_t)57) >> (uint16_t)9));
    q[3] = __builtin_bit_cast(uint32_t, (u16x2)((v * (uint16_t)19) >> (uint16_t)9));
    q[4] = __builtin_bit_cast(uint32_t, (u16x2)((v * (uint16_t)203) >> (uint16_t)14));
}

// Bytes q and q + 8 (q < 8) of a 16-byte chunk as the two 16-bit lanes of one register.
__device__ __forceinline__ uint32_t byte_pair(const u32x4 v, int q)
{
    const uint32_t sel = (uint32_t)(q & 3) | 0x0C00u | ((uint32_t)(4 + (q & 3)) << 16) | 0x0C000000u;
    return perm(v[2 + (q >> 2)], v[q >> 2], sel);
}

// 16-byte global load.
__device__ __forceinline__ uint4 ld16(const void *p) { return *reinterpret_cast<const uint4 *>(p); }

// NH consecutive fp16 values x[k0 .. k0+NH) of one activation row, as NH/2 registers
// (x[2q], x[2q+1]); zero beyond K.  `vec` says the row start is 16-byte aligned.
template <int NH>
__device__ __forceinline__ void load_x_span(const uint16_t *__restrict__ xrow, int k0, int K, bool vec,
                                            uint32_t (&out)[NH / 2])
{
    static_assert(NH % 8 == 0, "span must be whole 16-byte pieces");
    if (vec && k0 + NH <= K) {
#pragma unroll
        for (int q = 0; q < NH / 8; ++q) {
            uint4 v = ld16(xrow + k0 + 8 * q);
            out[4 * q + 0] = v.x; out[4 * q + 1] = v.y; out[4 * q + 2] = v.z; out[4 * q + 3] = v.w;
        }
    } else {
#pragma unroll
        for (int q = 0; q < NH / 2; ++q) {
            int k = k0 + 2 * q;
            uint32_t lo = (k < K) ? xrow[k] : 0u;
            uint32_t hi = (k + 1 < K) ? xrow[k + 1] : 0u;
            out[q] = lo | (hi << 16);
        }
    }
}

// Cross-lane moves of gfx950 used by the wave reductions.
// permlane32_swap(a, b): the upper 32 lanes of `a` trade places with the lower 32 lanes of `b`.
__device__ __forceinline__ void swap32(float &a, float &b)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
}
// permlane16_swap(a, b): the odd 16-lane rows of `a` trade places with the even rows of `b`.
__device__ __forceinline__ void swap16(float &a, float &b)
{
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
}
// v + (v of lane ^ 32) + (v of lane ^ 16) + (v of lane ^ 48): the sum over the four 16-lane
// rows, in every lane.
__device__ __forceinline__ float sum_over_rows(float v)
{
    float a = v, b = v;
    swap32(a, b);
    float s = a + b;
    a = s;
    b = s;
    swap16(a, b);
    return a + b;
}
template <int CTRL>
__device__ __forceinline__ float dpp(float v)
{
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sum RB (1, 2, 4 or 8) per-lane values over the 64 lanes of a wave, without LDS.  The
// first steps trade halves of the value list between partner lanes (32 apart, then 16
// apart, then mirrored inside a 16-lane row), so each lane keeps adding only the values of
// its own half; the rest is a butterfly inside the row over the lane masks 15
// (row_mirror), 7 (row_half_mirror), 2 and 1 (quad_perm).  The masks 32, 16, 15, 7, 2, 1
// span all six lane bits.  Afterwards every lane of group r = lane >> (6 - log2(RB)) holds
// the total of value r.  The order of the additions is fixed: results are deterministic.
template <int RB>
__device__ __forceinline__ float wave_reduce_rows(float (&v)[RB], int lane)
{
    static_assert(RB == 1 || RB == 2 || RB == 4 || RB == 8, "RB must be 1, 2, 4 or 8");
    float s;
    if constexpr (RB == 1) {
        float a = v[0], b = v[0];
        swap32(a, b);
        s = a + b;
        a = s;
        b = s;
        swap16(a, b);
        s = a + b;
    } else {
#pragma unroll
        for (int i = 0; i < RB / 2; ++i) {
            swap32(v[i], v[i + RB / 2]);
            v[i] += v[i + RB / 2];
        }
        if constexpr (RB == 2) {
            float a = v[0], b = v[0];
            swap16(a, b);
            s = a + b;
        } else {
#pragma unroll
            for (int i = 0; i < RB / 4; ++i) {
                swap16(v[i], v[i + RB / 4]);
                v[i] += v[i + RB / 4];
            }
            s = v[0];
            if constexpr (RB == 8) {
                const bool up = (lane & 8) != 0;
                const float send = up ? v[0] : v[1];
                const float keep = up ? v[1] : v[0];
                s = keep + dpp<0x140>(send);
            }
        }
    }
    if constexpr (RB <= 4) s += dpp<0x140>(s);   // row_mirror: lane ^ 15 within a row
    s += dpp<0x141>(s);                          // row_half_mirror: lane ^ 7 within 8 lanes
    s += dpp<0x4E>(s);                           // quad_perm [2,3,0,1]: lane ^ 2
    s += dpp<0xB1>(s);                           // quad_perm [1,0,3,2]: lane ^ 1
    return s;
}

}  // namespace tri
