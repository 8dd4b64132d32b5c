// KV-cache write (gfx950): the step's new K/V rows into the paged pool.
//
// What is computed: the cache write that the metrale blueprint graph.json
// runs just before attention (node l3.attn.kv_write, then l3.attn.attend),
// into the paged layout of the kern-kernels examples/decode.json manifest
// (buffers kv / table / seq / cuq).  New token i of sequence b (row
// t = cu_q[b] + i) is key position pos = L_b - n_b + i; its K and V rows of
// every KV head go to page block_table[b][pos / 64], slot pos % 64.  Tokens
// with pos < 0 (more new tokens than keys) have no slot and are skipped.
//
// Into an fp8 cache the rows are stored as OCP e4m3 codes of x * (1/scale)
// (one scale for K, one for V; the product in f32, round to nearest even,
// saturating), the quantised path's reading of "value / scale".
//
// Design (MI355X): one workgroup of 256 threads per (sequence, group of
// kWriteTok new tokens).  A token's rows are 2 * Hkv * D elements; thread c
// writes 16-byte output chunk c (chunk fastest, then K/V, then KV head, then
// token), so consecutive lanes read consecutive bytes of the new rows and
// write whole 16-byte runs of one slot.  HBM-bound: every new byte is read
// once and written once.
#include "attn_device.h"
#include "kv_quant.h"
#include "kv_write.h"

namespace pa {

constexpr int kWriteTok = 4;   // new tokens per workgroup

template <bool F8>
__global__ __launch_bounds__(kThreads) void paged_kv_write_kernel(const KvWriteArgs a) {
    const int b = blockIdx.y;
    const int i0 = blockIdx.x * kWriteTok;
    const int q0 = a.cu_q[b];
    int n = a.cu_q[b + 1] - q0;
    if (n > a.max_q) n = a.max_q;   // caller contract: n_b <= max_q
    if (i0 >= n) return;
    const int L = a.seq_lens[b];
    constexpr int EPC = F8 ? 16 : 8;             // pool elements per 16-byte output chunk
    const int chunks = a.d / EPC;                // output chunks per row
    const int per_head = 2 * chunks;             // K row then V row
    const int per_tok = a.hkv * per_head;
    const int total = (min(n, i0 + kWriteTok) - i0) * per_tok;
    const int32_t *bt_row = a.block_table + (int64_t)b * a.bt_stride;
    for (int c = threadIdx.x; c < total; c += kThreads) {
        const int ti = c / per_tok;
        const int r = c - ti * per_tok;
        const int i = i0 + ti;
        const int pos = L - n + i;
        if (pos < 0) continue;
        const int g = r / per_head;
        const int r2 = r - g * per_head;
        const int kv = r2 / chunks;              // 0 = K, 1 = V
        const int ch = r2 - kv * chunks;
        const int64_t t = q0 + i;
        const uint16_t *src = (kv ? a.v_new + t * a.v_st + (int64_t)g * a.v_sh
                                  : a.k_new + t * a.k_st + (int64_t)g * a.k_sh) + EPC * ch;
        const int64_t page = bt_row[pos / kPage];
        const int64_t off = page * a.kv_sp + (int64_t)(pos % kPage) * a.kv_ss + (int64_t)g * a.kv_sh +
                            kv * a.kv_skv + EPC * ch;   // pool elements
        if constexpr (!F8) {
            *reinterpret_cast<u32x4 *>(a.kv + off) = *reinterpret_cast<const u32x4 *>(src);
        } else {
            const u32x4 lo = *reinterpret_cast<const u32x4 *>(src);
            const u32x4 hi = *reinterpret_cast<const u32x4 *>(src + 8);
            *reinterpret_cast<u32x4 *>(reinterpret_cast<uint8_t *>(a.kv) + off) =
                bf16x16_to_e4m3(lo, hi, kv ? a.v_inv : a.k_inv);
        }
    }
}

hipError_t launch_kv_write(const KvWriteArgs &a, hipStream_t stream) {
    if (a.n_seqs == 0 || a.max_q == 0) return hipSuccess;
    const dim3 grid((a.max_q + kWriteTok - 1) / kWriteTok, a.n_seqs);
    if (a.fp8)
        hipLaunchKernelGGL(paged_kv_write_kernel<true>, grid, dim3(kThreads), 0, stream, a);
    else
        hipLaunchKernelGGL(paged_kv_write_kernel<false>, grid, dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace pa
