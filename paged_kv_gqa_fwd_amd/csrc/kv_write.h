// Arguments of the KV-cache write kernel (kv_write.hip).
#pragma once
#include <cstdint>

namespace pa {

struct KvWriteArgs {
    uint16_t *kv;                // bf16 pool (written)
    const uint16_t *k_new;       // bf16 [T, Hkv, D] (strided)
    const uint16_t *v_new;       // bf16 [T, Hkv, D] (strided)
    const int32_t *block_table;  // [B, MP] (row stride bt_stride)
    const int32_t *seq_lens;     // [B]
    const int32_t *cu_q;         // [B + 1]
    int64_t kv_sp, kv_ss, kv_sh, kv_skv;
    int64_t bt_stride;
    int64_t k_st, k_sh, v_st, v_sh;
    int32_t n_seqs, max_q, hkv, d;
    int32_t fp8;                 // pool holds OCP e4m3 codes (strides count bytes)
    float k_inv, v_inv;          // fp8: code = e4m3(x * (1 / scale)), product in f32
};

}  // namespace pa
