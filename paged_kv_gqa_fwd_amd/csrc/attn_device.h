// Device-side helpers and kernel argument blocks for the gfx950 paged
// attention kernels.  Internal to the library (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kPage = 64;      // keys per page (one KV tile)
constexpr int kThreads = 256;  // 4 wave64 per workgroup
constexpr int kBalMaxSeqs = 1024;  // sequences the balanced split path plans in one workgroup's LDS

// Split-decode tuning (compile-time knobs; the defaults are the measured best
// on MI355X): register stages = pages in flight per workgroup, and the
// resident waves per SIMD requested from the register allocator.  The host
// planner sizes splits from the same numbers.
#ifndef PA_DECODE_STAGES_128
#define PA_DECODE_STAGES_128 1
#endif
#ifndef PA_DECODE_STAGES_256
#define PA_DECODE_STAGES_256 1
#endif
#ifndef PA_DECODE_WAVES_128
#define PA_DECODE_WAVES_128 2
#endif
#ifndef PA_DECODE_WAVES_256
#define PA_DECODE_WAVES_256 1
#endif
// Prefill workgroups: wave64 count at each head_dim (two per SIMD at
// D = 128; one per SIMD at D = 256 by default) and packed query rows: 32
// rows per wave (4 x 64 at D = 128 with PA_PF_WAVES128 = 4).
#ifndef PA_PF_WAVES128
#define PA_PF_WAVES128 8
#endif
#ifndef PA_PF_WAVES256
#define PA_PF_WAVES256 4
#endif
constexpr int prefill_rows(int d) { return d == 128 ? 256 : 32 * PA_PF_WAVES256; }
constexpr int prefill_threads(int d) { return d == 128 ? 64 * PA_PF_WAVES128 : 64 * PA_PF_WAVES256; }
constexpr int decode_stages(int d) { return d == 128 ? PA_DECODE_STAGES_128 : PA_DECODE_STAGES_256; }
// Pages in flight per workgroup over an fp8 cache.  With non-temporal page
// loads fewer bytes in flight per workgroup read faster on MI355X (as for a
// plain read stream): one page, with two workgroups per CU at both head
// dims.  (At D = 256 one page and two workgroups per CU, which needs the
// vector-register MFMA form to fit 256 registers, ran long fp8 decode 13%
// faster than two pages and one workgroup per CU.)
#ifndef PA_DECODE_F8_STAGES_128
#define PA_DECODE_F8_STAGES_128 1
#endif
#ifndef PA_DECODE_F8_STAGES_256
#define PA_DECODE_F8_STAGES_256 1
#endif
constexpr int decode_stages_f8(int d) { return d == 128 ? PA_DECODE_F8_STAGES_128 : PA_DECODE_F8_STAGES_256; }
#ifndef PA_DECODE_F8_WAVES_128
#define PA_DECODE_F8_WAVES_128 2
#endif
#ifndef PA_DECODE_F8_WAVES_256
#define PA_DECODE_F8_WAVES_256 2
#endif
constexpr int decode_waves_per_simd_f8(int d) { return d == 128 ? PA_DECODE_F8_WAVES_128 : PA_DECODE_F8_WAVES_256; }
constexpr int decode_waves_per_simd(int d) { return d == 128 ? PA_DECODE_WAVES_128 : PA_DECODE_WAVES_256; }
// Resident waves per SIMD of the split-decode kernels (with rb blocks of 16
// packed rows a wave still holds one block's Q^T and O^T: the same count).
constexpr int decode_waves(int d, bool f8, int rb) {
    return rb > 0 && f8 ? decode_waves_per_simd_f8(d) : decode_waves_per_simd(d);
}
// Packed rows (G x query tokens of one sequence) the split-decode kernels
// take: blocks of 16, at most four (the short-sequence body).
constexpr int kDecodeRowBlock = 16;
constexpr int kMaxDecodeRowBlocks = 4;
constexpr int decode_row_blocks(int64_t rows) { return rows <= 16 ? 1 : rows <= 32 ? 2 : 4; }

// Arguments shared by the split-KV decode kernel and the prefill kernel.
struct AttnArgs {
    uint16_t *out;              // bf16 [T, Hq, D] (strided)
    const uint16_t *q;          // bf16 [T, Hq, D] (strided)
    const uint16_t *kv;         // bf16 pool
    const int32_t *block_table; // [B, MP] (row stride bt_stride)
    const int32_t *seq_lens;    // [B]
    const int32_t *cu_q;        // [B + 1]
    float *part_o;              // f32 [T, Hq, S, D] split partials (unnormalised)
    float *part_ml;             // f32 [T, Hq, S, 2] split (max in log2 units, sum)
    int32_t *counters;          // [B, Hkv] arrival counters of the in-kernel merge (zero between calls)
    int64_t q_st, q_sh, o_st, o_sh;
    int64_t kv_sp, kv_ss, kv_sh, kv_skv;
    int64_t bt_stride;
    int32_t n_seqs, max_q, hq, hkv, group;
    int32_t pages_per_split, max_splits;
    int32_t causal;
    float scale_log2;           // scale * log2(e): scores live in log2 units
    float scale_log2_pos;       // max(|scale| * log2(e), FLT_MIN) (prefill kernel)
    int32_t q_negate;           // scale < 0: the prefill kernel negates Q instead
    int32_t fuse_merge;         // split path: the last split of each (sequence, KV head) merges
    const float *sinks;         // [Hq] sink logits (units of the scaled scores), or null
    int32_t window;             // > 0: a query at pos sees only keys >= pos - window + 1; 0: no window
    int32_t kv_fp8;             // pool holds OCP e4m3 codes (split path only); strides count bytes
    float v_scale;              // V = v_scale * e4m3(code) (1 for a bf16 pool); k_scale is in scale_log2
    int32_t *seg_splits;        // balanced split path: [B] pieces per sequence (1 = written directly, 0 = no page)
    int32_t row_blocks;         // split paths: blocks of 16 packed rows per workgroup (1, 2 or 4)
    // Fused KV-cache write (split paths; null k_new = none): the step's new
    // K/V rows [T, Hkv, D] bf16, written into the pool by the workgroup that
    // streams their page, which attends to them in place of the slots' old bits.
    const uint16_t *k_new, *v_new;
    int64_t kn_st, kn_sh, vn_st, vn_sh;
    float k_inv, v_inv;         // fp8 cache: codes of x * (1 / scale)
    // Prefill over an fp8 cache: the pages the call reads are first decoded
    // (exactly) into a bf16 staging pool in the workspace, [n_seqs * MP]
    // pages of [P, Hkv, 2, D], with its own table [n_seqs, MP] (page b*MP + j
    // for page j of sequence b; -1 for pages not staged).  Null = none.
    uint16_t *stage_kv;
    int32_t *stage_bt;
    int32_t mp;                 // block-table columns (the staging pool's pages per sequence)
    // Prefill launch order (null = grid order, latest tiles first): entry i
    // is the (tile, KV head, sequence) index, in grid order, that workgroup i
    // computes; a permutation of the grid written by prefill_order_kernel.
    int32_t *pf_order;
    // Split-key prefill (> 1: small grids): splits per (sequence, KV head),
    // the page ranges and partial layout of the split-decode path
    // (pages_per_split, max_splits, part_o, part_ml); merged by the combine.
    int32_t pf_splits;
};

struct CombineArgs {
    uint16_t *out;
    const float *part_o;
    const float *part_ml;
    const int32_t *seq_lens;
    const int32_t *cu_q;
    const float *sinks;
    int64_t o_st, o_sh;
    int32_t n_seqs, max_q, hq, pages_per_split, max_splits, window;
    const int32_t *seg_splits;  // balanced split path: pieces per sequence (else null)
};

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
    return __uint_as_float(((uint32_t)b) << 16);
}

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
    __bf16 h = (__bf16)f;  // round to nearest even (v_cvt_pk_bf16_f32)
    return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ float shfl_xor_f32(float v, int mask) {
    return __shfl_xor(v, mask, 64);
}

constexpr float kLog2e = 1.4426950408889634f;

// First key a query at position pos may see under a left window of w keys
// (w > 0); 0 without a window.
__device__ __forceinline__ int window_start(int pos, int w) {
    if (w <= 0) return 0;
    const int64_t lo = (int64_t)pos - w + 1;
    return lo > 0 ? (int)lo : 0;
}

// Split-KV layout of one sequence: splits cover its pages from the first one
// inside row 0's window (row 0 has the earliest window) in runs of pps pages.
__device__ __forceinline__ int split_first_page(int L, int n, int w) { return window_start(L - n, w) / kPage; }
__device__ __forceinline__ int split_count(int npages, int p_lo, int pps, int max_splits) {
    const int ns = (npages - p_lo + pps - 1) / pps;
    return ns < 1 ? 1 : (ns > max_splits ? max_splits : ns);
}

// Number of keys visible to query i of a sequence with n queries and L keys
// (bottom-right causal alignment; all L keys when not causal).
__device__ __forceinline__ int visible_keys(int L, int n, int i, int causal) {
    if (!causal) return L;
    int v = L - n + i + 1;
    return v < 0 ? 0 : (v > L ? L : v);
}

// LDS transpose read (gfx950 ds_read_b64_tr_b16).  Within each group of 16
// lanes, lane s supplies the address of 4 consecutive bf16; lane j receives
// element (j % 4) of lanes 4r + j/4 for r = 0..3.  With lane s pointing at
// row (s / 4), columns 4*(s % 4) .. +3 of a row-major tile, lane j receives
// column j of the four rows.
__device__ __forceinline__ bf16x4 lds_read_tr16(const uint16_t *lds_ptr) {
    typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (lds_bf16x4 *)(const_cast<uint16_t *>(lds_ptr)));
}

}  // namespace pa
