// Device helpers of the fp8 (OCP e4m3) KV cache: bf16 rows to codes of
// x * (1 / scale) (the quantising write, also fused into the split-decode
// kernels) and codes back to bf16, exactly.  Internal to the library.
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

// Four OCP e4m3 codes (one 32-bit word) to four bf16 (two words), exactly:
// every e4m3 value is a bf16 value (one conversion instruction per pair,
// with a unit scale).
__device__ __forceinline__ void e4m3x4_to_bf16x4(uint32_t w, uint32_t &lo, uint32_t &hi) {
    lo = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));  // bytes 0, 1
    hi = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true));   // bytes 2, 3
}

}  // namespace pa
