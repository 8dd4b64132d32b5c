// Paged prefill / chunked-prefill attention kernel (gfx950), one pass with
// online softmax and causal tile skipping.
//
// What is computed: the Mojo SM100MHA2Q docs' forward attention over a KV
// cache (UMMA0Type: S = Q K^T into f32; UMMA1Type: O += P V; MaskType:
// causal or unmasked; mask_status: per-tile mask classification that lets
// fully masked tiles be skipped; fuse_gqa / group: the q heads of one KV
// head share the K/V tiles), over the page layout of the kern-kernels
// examples/decode.json manifest (buffers.kv).
//
// Design (MI355X): one workgroup of 4 wave64 per (sequence, KV head, tile of
// 128 packed query rows).  Row r of a (sequence, KV head) is query token
// r / G, q head g*G + r % G, so the G heads sharing a KV head share every
// K/V tile.  Each wave owns 32 rows.  Per 64-key page: K and V rows are
// staged into LDS with coalesced 16-byte loads (two pages ahead in
// registers at D = 128, one at D = 256); S^T = K Q^T runs on v_mfma_f32_32x32x16_bf16 with keys on M,
// so every lane owns one query row and the row max / row sum are in-lane
// plus one cross-half exchange; the S^T C layout is directly the B operand
// of O^T += V^T P^T, whose V^T operand comes from the row-major V tile via
// the LDS transpose read.  Tiles past the causal frontier of the last row
// are never loaded; tiles below the first row's frontier skip the mask.
#include "attn_device.h"

namespace pa {

template <int D>
struct PrefillCfg {
    static constexpr int BM = 128;        // packed query rows per workgroup
    static constexpr int KROW = D + 8;
    static constexpr int VROW = D + 16;
    static constexpr int CH_PER_THREAD = 2 * kPage * D / 8 / kThreads;
    static constexpr int LDS_ELEMS = kPage * (KROW + VROW);
};

template <int D>
__device__ __forceinline__ void prefill_load_tile(u32x4 (&stage)[PrefillCfg<D>::CH_PER_THREAD],
                                                  const uint16_t *head_base, int64_t page_off,
                                                  int64_t kv_ss, int64_t kv_skv, int tid,
                                                  int valid) {
    // Slots at or past `valid` (past the sequence end) stage as zeros and are
    // never read: a non-finite V there would make 0 * V = NaN in P.V.
    constexpr int DC = D / 8;
#pragma unroll
    for (int it = 0; it < PrefillCfg<D>::CH_PER_THREAD; ++it) {
        const int c = it * kThreads + tid;
        const int dc = c % DC;
        const int kv = (c / DC) & 1;
        const int key = c / (2 * DC);
        stage[it] = key < valid ? *reinterpret_cast<const u32x4 *>(head_base + page_off +
                                                                   (int64_t)key * kv_ss +
                                                                   kv * kv_skv + dc * 8)
                                : u32x4{0u, 0u, 0u, 0u};
    }
}

template <int D>
__device__ __forceinline__ void prefill_store_tile(const u32x4 (&stage)[PrefillCfg<D>::CH_PER_THREAD],
                                                   uint16_t *ks, uint16_t *vs, int tid) {
    constexpr int DC = D / 8;
#pragma unroll
    for (int it = 0; it < PrefillCfg<D>::CH_PER_THREAD; ++it) {
        const int c = it * kThreads + tid;
        const int dc = c % DC;
        const int kv = (c / DC) & 1;
        const int key = c / (2 * DC);
        uint16_t *dst = kv ? (vs + key * PrefillCfg<D>::VROW + dc * 8)
                           : (ks + key * PrefillCfg<D>::KROW + dc * 8);
        *reinterpret_cast<u32x4 *>(dst) = stage[it];
    }
}

template <int D>
__global__ __launch_bounds__(kThreads) void paged_prefill_kernel(const AttnArgs a) {
    using C = PrefillCfg<D>;
    __shared__ __attribute__((aligned(16))) uint16_t smem[C::LDS_ELEMS];
    uint16_t *ks = smem;
    uint16_t *vs = smem + kPage * C::KROW;

    const int g = blockIdx.y;
    const int b = blockIdx.z;
    // Later query tiles see more keys under a causal mask: launch them first.
    const int tile = gridDim.x - 1 - blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int hi = lane >> 5;   // which half of the wave (0 / 1)

    const int L = a.seq_lens[b];
    const int q0 = a.cu_q[b];
    int n = a.cu_q[b + 1] - q0;
    if (n > a.max_q) n = a.max_q;
    const int G = a.group;
    const int R = n * G;
    const int r0 = tile * C::BM;
    if (r0 >= R) return;

    const int r = r0 + 32 * w + (lane & 31);
    const bool row_ok = r < R;
    const int qi = r / G;
    const int h = g * G + (r - qi * G);
    const int vis = row_ok ? visible_keys(L, n, qi, a.causal) : 0;
    const int r_last = min(R, r0 + C::BM) - 1;
    const int kv_end = visible_keys(L, n, r_last / G, a.causal);   // max over the tile's rows
    const int kv_full = visible_keys(L, n, r0 / G, a.causal);      // min over the tile's rows
    const int ntiles = (kv_end + kPage - 1) / kPage;

    // Q^T as the B operand of v_mfma_f32_32x32x16_bf16:
    // lane holds q[row, 16*ks + 8*hi .. +7] for ks = 0 .. D/16-1.
    bf16x8 qreg[D / 16];
    {
        const uint16_t *qp = a.q + (int64_t)(q0 + qi) * a.q_st + (int64_t)h * a.q_sh + 8 * hi;
#pragma unroll
        for (int ks_ = 0; ks_ < D / 16; ++ks_) {
            u32x4 v = {0u, 0u, 0u, 0u};
            if (row_ok) v = *reinterpret_cast<const u32x4 *>(qp + 16 * ks_);
            qreg[ks_] = __builtin_bit_cast(bf16x8, v);
        }
    }

    const uint16_t *head_base = a.kv + (int64_t)g * a.kv_sh;
    const int32_t *bt_row = a.block_table + (int64_t)b * a.bt_stride;

    f32x16 oacc[D / 32];
#pragma unroll
    for (int i = 0; i < D / 32; ++i) oacc[i] = f32x16{};
    float m_run = -INFINITY;
    float l_part = 0.f;

    auto compute_tile = [&](int kt) {
            // S^T = K Q^T for two 32-key blocks.
            f32x16 sacc[2] = {f32x16{}, f32x16{}};
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const uint16_t *kp = ks + (32 * kb + (lane & 31)) * C::KROW + 8 * hi;
#pragma unroll
                for (int ks_ = 0; ks_ < D / 16; ++ks_) {
                    const bf16x8 kop = *reinterpret_cast<const bf16x8 *>(kp + 16 * ks_);
                    sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qreg[ks_], sacc[kb], 0, 0, 0);
                }
            }
            // sacc[kb][i] = score of key kt*64 + 32kb + 8*(i/4) + 4*hi + i%4.
            const bool need_mask = (kt + 1) * kPage > kv_full;
            float mx = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    float sc = sacc[kb][i] * a.scale_log2;
                    if (need_mask) {
                        const int key = kt * kPage + 32 * kb + 8 * (i >> 2) + 4 * hi + (i & 3);
                        sc = key < vis ? sc : -INFINITY;
                    }
                    sacc[kb][i] = sc;
                    mx = fmaxf(mx, sc);
                }
            }
            mx = fmaxf(mx, shfl_xor_f32(mx, 32));
            const float m_new = fmaxf(m_run, mx);
            const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
            const float alpha = exp2_fast(m_run - m_use);
            m_run = m_new;
            bf16x8 pb[2][2];
            float psum = 0.f;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const __bf16 pr = (__bf16)exp2_fast(sacc[kb][i] - m_use);
                    pb[kb][i >> 3][i & 7] = pr;
                    psum += (float)pr;   // the sum uses the same rounded P as the P.V product
                }
            }
            l_part = l_part * alpha + psum;
            if (__any(alpha != 1.f)) {
#pragma unroll
                for (int i = 0; i < D / 32; ++i) oacc[i] *= alpha;
            }

            // O^T[d, row] += V^T[d, key] P^T[key, row]; 4 k-steps of 16 keys.
            // k-step (kb, jj), half hi holds keys 32kb+16jj + {4hi..4hi+3, 8+4hi..8+4hi+3}.
            const int q16 = lane >> 4;
            const int dsub = (q16 & 1) * 16;
            const int src_row = (lane & 15) >> 2;
            const int src_col = 4 * (lane & 3);
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
                for (int jj = 0; jj < 2; ++jj) {
                    const int kbase = 32 * kb + 16 * jj + 4 * hi;
                    const uint16_t *v1 = vs + (kbase + src_row) * C::VROW + dsub + src_col;
                    const uint16_t *v2 = v1 + 8 * C::VROW;
#pragma unroll
                    for (int db = 0; db < D / 32; ++db) {
                        const bf16x4 lo4 = lds_read_tr16(v1 + 32 * db);
                        const bf16x4 hi4 = lds_read_tr16(v2 + 32 * db);
                        const bf16x8 vop = __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
                        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pb[kb][jj], oacc[db], 0, 0, 0);
                    }
                }
            }
    };

    const int64_t sp = a.kv_sp;
    if constexpr (D == 128) {
        // Two tiles in flight: stage A holds even tiles, stage B odd ones; each
        // page id is read one compute phase before its loads issue.
        u32x4 stA[C::CH_PER_THREAD], stB[C::CH_PER_THREAD];
        if (ntiles > 0)
            prefill_load_tile<D>(stA, head_base, (int64_t)bt_row[0] * sp, a.kv_ss, a.kv_skv, tid, L);
        if (ntiles > 1)
            prefill_load_tile<D>(stB, head_base, (int64_t)bt_row[1] * sp, a.kv_ss, a.kv_skv, tid, L - kPage);
        int pid_a = (ntiles > 2) ? bt_row[2] : 0;
        for (int kt = 0; kt < ntiles; kt += 2) {
            __syncthreads();
            prefill_store_tile<D>(stA, ks, vs, tid);
            __syncthreads();
            if (kt + 2 < ntiles)
                prefill_load_tile<D>(stA, head_base, (int64_t)pid_a * sp, a.kv_ss, a.kv_skv, tid,
                                     L - (kt + 2) * kPage);
            const int pid_b = (kt + 3 < ntiles) ? bt_row[kt + 3] : 0;
            compute_tile(kt);
            if (kt + 1 >= ntiles) break;    // uniform across the workgroup
            __syncthreads();
            prefill_store_tile<D>(stB, ks, vs, tid);
            __syncthreads();
            if (kt + 3 < ntiles)
                prefill_load_tile<D>(stB, head_base, (int64_t)pid_b * sp, a.kv_ss, a.kv_skv, tid,
                                     L - (kt + 3) * kPage);
            pid_a = (kt + 4 < ntiles) ? bt_row[kt + 4] : 0;
            compute_tile(kt + 1);
        }
    } else {
        // One tile in flight (the register budget at D = 256 has no room for two).
        u32x4 st[C::CH_PER_THREAD];
        if (ntiles > 0)
            prefill_load_tile<D>(st, head_base, (int64_t)bt_row[0] * sp, a.kv_ss, a.kv_skv, tid, L);
        int pid = (ntiles > 1) ? bt_row[1] : 0;
        for (int kt = 0; kt < ntiles; ++kt) {
            __syncthreads();
            prefill_store_tile<D>(st, ks, vs, tid);
            __syncthreads();
            if (kt + 1 < ntiles)
                prefill_load_tile<D>(st, head_base, (int64_t)pid * sp, a.kv_ss, a.kv_skv, tid,
                                     L - (kt + 1) * kPage);
            pid = (kt + 2 < ntiles) ? bt_row[kt + 2] : 0;
            compute_tile(kt);
        }
    }

    // Epilogue: out = O / l, rounded to bf16.  oacc[db][i] holds
    // d = 32db + 8*(i/4) + 4*hi + i%4 of this lane's row.
    const float l_row = l_part + shfl_xor_f32(l_part, 32);
    if (!row_ok) return;
    const float inv = l_row > 0.f ? 1.f / l_row : 0.f;
    uint16_t *op = a.out + (int64_t)(q0 + qi) * a.o_st + (int64_t)h * a.o_sh;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4) {
            u32x2 pk;
            pk[0] = (uint32_t)f32_to_bf16_bits(oacc[db][4 * c4 + 0] * inv) |
                    ((uint32_t)f32_to_bf16_bits(oacc[db][4 * c4 + 1] * inv) << 16);
            pk[1] = (uint32_t)f32_to_bf16_bits(oacc[db][4 * c4 + 2] * inv) |
                    ((uint32_t)f32_to_bf16_bits(oacc[db][4 * c4 + 3] * inv) << 16);
            *reinterpret_cast<u32x2 *>(op + 32 * db + 8 * c4 + 4 * hi) = pk;
        }
    }
}

template <int D>
hipError_t launch_prefill(const AttnArgs &a, dim3 grid, hipStream_t stream) {
    hipLaunchKernelGGL(paged_prefill_kernel<D>, grid, dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_prefill_any(int D, const AttnArgs &a, dim3 grid, hipStream_t stream) {
    return D == 128 ? launch_prefill<128>(a, grid, stream) : launch_prefill<256>(a, grid, stream);
}

}  // namespace pa
