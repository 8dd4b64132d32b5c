// Argument block and layout constants of the quantised-attention kernels.
// Internal to the library (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

constexpr int kQuantD = 128;       // head_dim supported by the quantised path
constexpr int kQuantBlock = 64;    // tokens per int8 scale block and per key tile
constexpr int kQuantChunk = 256;   // tokens per statistics workgroup

// Stored position, within its 64-key tile, of key `key` in the fp8 V^T
// layout.  The Q.K MFMA leaves lane (row n, half hi) holding the scores of
// keys 32 kb + 8 (i / 4) + 4 hi + i % 4 for kb < 2, i < 16, in register
// order e = 16 kb + i; the P.V MFMA takes byte e of that lane's B operand as
// contraction index (hi, e).  Storing key(hi, e) at position 32 hi + e makes
// each lane's A operand (row d of V^T) 32 contiguous bytes.
__host__ __device__ constexpr int quant_pos_of_key(int key) {
    return 32 * (((key % 32) % 8) / 4) + 16 * (key / 32) + 4 * ((key % 32) / 8) + (key % 4);
}

struct QuantArgs {
    // inputs: bf16 [B, N, H, D] with element strides (batch, token, head)
    const uint16_t *q, *k, *v;
    int64_t q_sb, q_st, q_sh, k_sb, k_st, k_sh, v_sb, v_st, v_sh;
    // output: bf16 [B, N, H, D]
    uint16_t *out;
    int64_t o_sb, o_st, o_sh;
    int32_t b, n, h;
    int32_t blocks;   // ceil(N / 64)
    int32_t chunks;   // ceil(N / 256)
    int32_t vt_stride;   // blocks * 64: bytes per V^T row
    // workspace
    float *mk;            // f32 [B, H, D]      K channel means
    float *sv;            // f32 [B, H, D]      V channel scales
    float *sq, *sk;       // f32 [B, H, blocks] Q / K block scales
    int8_t *qi, *ki;      // int8 [B, N, H, D]  codes
    uint8_t *vt;          // e4m3 [B, H, D, vt_stride] codes, keys permuted per tile
    double *ksum_part;    // f64 [B, H, chunks, D]
    float *vmax_part;     // f32 [B, H, chunks, D]
    // attention
    float scale_log2_pos; // max(|scale| * log2(e), FLT_MIN)
    int32_t q_negate;     // scale < 0: Q codes are negated instead
    int32_t causal;
};

}  // namespace pa
