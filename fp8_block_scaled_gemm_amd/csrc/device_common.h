// Device helpers shared by the gfx950 kernels of this library: vector types
// for MFMA operands and 16-byte accesses, and the e4m3 conversion.
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

// Four fp32 values -> four OCP E4M3FN codes (byte i = value i, sign kept)
// with the hardware conversion (v_cvt_pk_fp8_f32: round to nearest even,
// subnormal codes below 2^-6).  Inputs are clamped to +-448 first
// (v_med3_f32), so the conversion never sees a value past the largest finite
// e4m3: results saturate at +-448.
__device__ __forceinline__ uint32_t e4m3x4_hw(float a, float b, float c, float d) {
    const float lim = 448.0f;
    a = __builtin_amdgcn_fmed3f(a, -lim, lim);
    b = __builtin_amdgcn_fmed3f(b, -lim, lim);
    c = __builtin_amdgcn_fmed3f(c, -lim, lim);
    d = __builtin_amdgcn_fmed3f(d, -lim, lim);
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
    return (uint32_t)w;
}

}  // namespace dg
