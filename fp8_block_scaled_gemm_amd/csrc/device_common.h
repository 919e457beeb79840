// Device helpers shared by the gfx950 kernels of this library: number-format
// conversions written from the formats' definitions, and MFMA operand types.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dg {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));  // 16-byte global/LDS chunk
typedef unsigned v2u __attribute__((ext_vector_type(2)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

// fp32 -> OCP E4M3FN code, round to nearest even, saturated to +-448, sign
// kept.  Normal results keep 3 of the 23 mantissa bits (carry into the
// exponent handled by the integer add); below 2^-6 the grid step is 2^-9.
__device__ __forceinline__ uint32_t e4m3_rne_sat(float v) {
    uint32_t u = __float_as_uint(v);
    uint32_t sign = (u >> 24) & 0x80u;
    uint32_t a = u & 0x7fffffffu;
    if (a > 0x7f800000u) return sign | 0x7fu;        // NaN
    if (a >= 0x43e00000u) return sign | 0x7eu;       // |v| >= 448
    if (a < 0x3c800000u) {                           // |v| < 2^-6
        float t = __uint_as_float(a) * 512.0f;       // exact power-of-two scaling
        return sign | (uint32_t)__builtin_rintf(t);  // 0..8; 8 is the code of 2^-6
    }
    uint32_t r = a + 0x7ffffu + ((a >> 20) & 1u);
    uint32_t code = (((r >> 23) - 120u) << 3) | ((r >> 20) & 7u);
    return sign | (code > 0x7eu ? 0x7eu : code);
}

}  // namespace dg
