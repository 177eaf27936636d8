// tri_internal.h -- host-side declarations shared by the libtri translation units.
#pragma once
#include <stdint.h>
#include <hip/hip_runtime.h>
#include "../../include/tri.h"

namespace tri {

inline int64_t row_bytes(int64_t K, int fmt)
{
    if (K < 1) return -1;
    if (fmt == TRI_FMT_2BIT) return 16 * ((K + 63) / 64);
    if (fmt == TRI_FMT_1P6BIT) return 16 * ((K + 79) / 80);
    return -1;
}

int launch_pack(const int8_t *W, int64_t N, int64_t K, int fmt, uint8_t *Wp, hipStream_t s);
int launch_unpack(const uint8_t *Wp, int64_t N, int64_t K, int fmt, int8_t *W, hipStream_t s);

// Kernel launchers of the layer; arguments are already validated.
int launch_gemv2(const uint16_t *X, const uint8_t *Wp, float scale, int N, int K, uint16_t *Y, hipStream_t s);
int launch_smallm(const uint16_t *X, const uint8_t *Wp, float scale, int M, int N, int K, int fmt, uint16_t *Y,
                  hipStream_t s);
// MFMA decode kernel with activations staged in LDS; false (nothing launched) if K is too long for it.
// M = 1 on MFMA (tri_mv1.hip); false if the shape is outside its range
bool launch_mv1(const uint16_t *X, const uint8_t *Wp, float scale, int N, int K, int fmt, uint16_t *Y, hipStream_t s);
// 2 <= M <= 16 on MFMA (tri_mvm.hip); false if the shape is outside its range
bool launch_mvm(const uint16_t *X, const uint8_t *Wp, float scale, int M, int N, int K, int fmt, uint16_t *Y,
                hipStream_t s);
bool launch_decode(const uint16_t *X, const uint8_t *Wp, float scale, int M, int N, int K, int fmt, uint16_t *Y,
                   hipStream_t s);
int launch_gemm(const uint16_t *X, const uint8_t *Wp, float scale, int64_t M, int N, int K, int fmt, uint16_t *Y,
                hipStream_t s);
int launch_probe_read(const void *src, int64_t bytes, uint32_t *sink, hipStream_t s);
int launch_probe_copy(const void *src, void *dst, int64_t bytes, hipStream_t s);

}  // namespace tri
