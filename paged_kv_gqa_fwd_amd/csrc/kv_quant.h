// Device helpers of the quantising KV-cache write (fp8 cache): bf16 rows to
// OCP e4m3 codes of x * (1 / scale).  Shared by the write kernel and the
// split-decode kernels' fused write.  Internal to the library.
#pragma once

#include "attn_device.h"

namespace pa {

// |y| > 448 becomes +-448 (the largest e4m3 value); NaN stays NaN.  The
// conversion instruction alone does not saturate out-of-range inputs.
__device__ __forceinline__ float e4m3_saturate(float y) {
    return fabsf(y) > 448.f ? copysignf(448.f, y) : y;
}

// Sixteen bf16 (two 16-byte words) to sixteen e4m3 codes of x * inv: the
// product in f32, saturated to +-448, then v_cvt_pk_fp8_f32 (round to
// nearest even).
__device__ __forceinline__ u32x4 bf16x16_to_e4m3(const u32x4 a, const u32x4 b, float inv) {
    u32x4 r;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const u32x4 &src = w < 2 ? a : b;
        const uint32_t x0 = src[2 * (w & 1)], x1 = src[2 * (w & 1) + 1];
        const float f0 = e4m3_saturate(__uint_as_float(x0 << 16) * inv);
        const float f1 = e4m3_saturate(__uint_as_float(x0 & 0xFFFF0000u) * inv);
        const float f2 = e4m3_saturate(__uint_as_float(x1 << 16) * inv);
        const float f3 = e4m3_saturate(__uint_as_float(x1 & 0xFFFF0000u) * inv);
        int word = __builtin_amdgcn_cvt_pk_fp8_f32(f0, f1, 0, false);
        word = __builtin_amdgcn_cvt_pk_fp8_f32(f2, f3, word, true);
        r[w] = (uint32_t)word;
    }
    return r;
}

}  // namespace pa
