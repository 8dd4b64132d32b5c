// Split-KV paged decode kernel and log-sum-exp combine kernel (gfx950).
//
// What is computed follows the split-KV scheme of the kern-kernels
// examples/decode.json manifest (ops.decode.impl.scratch: per-split partial
// outputs and per-row (max, sum) statistics, grid.x = KV splits per
// (KV head, sequence)) and the Mojo SM100MHA2Q docs (PartitionType: KV-cache
// partition scheme; MaskType: causal or unmasked).  The splits are merged
// either by a second, separate kernel or, like the manifest's single launch
// with its i32 counter scratch (ops.decode.impl.scratch.counter), by the
// last workgroup of each (sequence, KV head) to finish its split.
//
// Design (MI355X): one workgroup of 4 wave64 per (KV head, sequence, split).
// The split's pages stream through LDS with 16-byte coalesced loads, staged
// in registers two pages ahead.  The G q heads x n query tokens of the KV
// head (<= 16 rows) form the N side of the MFMA and the keys the M side
// ("swap AB"), so the score tile's C layout is directly the B operand of the
// P.V MFMA.  Each wave owns 16 keys of every page and keeps its own online
// softmax state; the four waves merge in LDS at the end.
#include "attn_device.h"

namespace pa {

// Device-scope (all XCDs) relaxed store / load of a float.
__device__ __forceinline__ void store_coherent(float *p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(const float *p) {
    return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int D, bool F8>
struct DecodeCfg {
    static constexpr int STAGES = F8 ? decode_stages_f8(D) : decode_stages(D);
    static constexpr int WAVES_PER_SIMD = F8 ? decode_waves_per_simd_f8(D) : decode_waves_per_simd(D);
    static constexpr int KROW = D + 8;    // bf16 per LDS K row (16 B pad: conflict-free b128 reads)
    static constexpr int VROW = D + 16;   // bf16 per LDS V row (32 B pad: conflict-free tr reads)
    static constexpr int EB = F8 ? 1 : 2;                    // bytes per pool element
    static constexpr int EPC = 16 / EB;                      // pool elements per 16-byte chunk
    static constexpr int DC = D / EPC;                       // chunks per K or V row
    static constexpr int CHUNKS = 2 * kPage * DC;            // 16-byte chunks per K+V page
    static constexpr int CH_PER_THREAD = CHUNKS / kThreads;  // D/16 (bf16) or D/32 (fp8)
    static constexpr int LDS_ELEMS = kPage * (KROW + VROW);
};

// Issue the 16-byte loads of one page (K and V rows of one KV head) into
// registers.  Chunk c -> key = c / (2 DC), kv = (c / DC) % 2, dc = c % DC:
// consecutive threads read consecutive 16 bytes of one key's K row then V row.
// Slots at or past `valid` (the tail of a sequence's last page) are not read
// and stage as zeros: their memory may hold anything, and a non-finite V
// would turn the zero softmax weight of a masked key into NaN in P.V.
// `head_base` and the strides address pool elements (bf16 or fp8 bytes).
template <int D, bool F8>
__device__ __forceinline__ void load_page(u32x4 (&stage)[(DecodeCfg<D, F8>::CH_PER_THREAD)],
                                          const char *head_base, int64_t page_off,
                                          int64_t kv_ss, int64_t kv_skv, int tid, int valid) {
    using C = DecodeCfg<D, F8>;
#pragma unroll
    for (int it = 0; it < C::CH_PER_THREAD; ++it) {
        const int c = it * kThreads + tid;
        const int dc = c % C::DC;
        const int kv = (c / C::DC) & 1;
        const int key = c / (2 * C::DC);
        const char *src = head_base + (page_off + (int64_t)key * kv_ss + kv * kv_skv) * C::EB + dc * 16;
        stage[it] = key < valid ? *reinterpret_cast<const u32x4 *>(src) : u32x4{0u, 0u, 0u, 0u};
    }
}

// Four OCP e4m3 codes (one 32-bit word) to four bf16 (two words), exactly:
// every e4m3 value is a bf16 value (one conversion instruction per pair,
// with a unit scale).
__device__ __forceinline__ void e4m3x4_to_bf16x4(uint32_t w, uint32_t &lo, uint32_t &hi) {
    lo = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));  // bytes 0, 1
    hi = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true));   // bytes 2, 3
}

template <int D, bool F8>
__device__ __forceinline__ void store_page(const u32x4 (&stage)[(DecodeCfg<D, F8>::CH_PER_THREAD)],
                                           uint16_t *ks, uint16_t *vs, int tid) {
    using C = DecodeCfg<D, F8>;
#pragma unroll
    for (int it = 0; it < C::CH_PER_THREAD; ++it) {
        const int c = it * kThreads + tid;
        const int dc = c % C::DC;
        const int kv = (c / C::DC) & 1;
        const int key = c / (2 * C::DC);
        uint16_t *dst = kv ? (vs + key * C::VROW + dc * C::EPC) : (ks + key * C::KROW + dc * C::EPC);
        if constexpr (!F8) {
            *reinterpret_cast<u32x4 *>(dst) = stage[it];
        } else {
            // 16 codes -> 16 bf16 (dequantised; the scales are applied to
            // the scores and the output)
            uint32_t o[8];
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) e4m3x4_to_bf16x4(stage[it][q4], o[2 * q4], o[2 * q4 + 1]);
            *reinterpret_cast<u32x4 *>(dst) = u32x4{o[0], o[1], o[2], o[3]};
            *reinterpret_cast<u32x4 *>(dst + 8) = u32x4{o[4], o[5], o[6], o[7]};
        }
    }
}

template <int D, bool F8>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(DecodeCfg<D, F8>::WAVES_PER_SIMD)))
void paged_decode_split_kernel(const AttnArgs a) {
    using C = DecodeCfg<D, F8>;
    __shared__ __attribute__((aligned(16))) uint16_t smem[C::LDS_ELEMS];
    __shared__ float red_m[4][16];
    __shared__ float red_l[4][16];
    uint16_t *ks = smem;
    uint16_t *vs = smem + kPage * C::KROW;

    // Grid (KV head, sequence, split): splits vary slowest, so every
    // sequence's full-size first splits are dispatched before the shorter
    // remainder splits and the empty ones (which exit at once).
    const int g = blockIdx.x;
    const int b = blockIdx.y;
    const int s = blockIdx.z;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;

    const int L = a.seq_lens[b];
    const int q0 = a.cu_q[b];
    int n = a.cu_q[b + 1] - q0;
    if (n > a.max_q) n = a.max_q;  // caller contract: n_b <= max_q
    const int npages = (L + kPage - 1) / kPage;
    // Splits start at the first page inside row 0's window (page 0 without a
    // window), so pages no row can see are neither planned nor read.
    const int p_lo = split_first_page(L, n, a.window);
    const int p_begin = p_lo + s * a.pages_per_split;
    // Uniform across the workgroup.  A split past the sequence's last page
    // writes nothing (the combine never reads it); without splitting, an
    // empty sequence still runs the epilogue so its rows are written as zeros.
    if (n <= 0 || (s > 0 && p_begin >= npages)) return;
    const int p_end = min(npages, p_begin + a.pages_per_split);
    const int G = a.group;
    int rows = n * G;
    if (rows > 16) rows = 16;

    // This lane's query row (the N index of the MFMA tiles).
    const int row = lane & 15;
    const bool row_ok = row < rows;
    const int qi = row / G;
    const int h = g * G + (row - qi * G);
    const int vis = row_ok ? visible_keys(L, n, qi, a.causal) : 0;
    const int lo = row_ok ? window_start(L - n + qi, a.window) : 0;   // first key inside the window

    // Q^T as the B operand of v_mfma_f32_16x16x32_bf16: lane holds
    // q[row, 32*kk + 8*(lane/16) .. +7] for kk = 0 .. D/32-1.
    bf16x8 qreg[D / 32];
    {
        const uint16_t *qp = a.q + (int64_t)(q0 + qi) * a.q_st + (int64_t)h * a.q_sh + 8 * (lane >> 4);
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk) {
            u32x4 v = {0u, 0u, 0u, 0u};
            if (row_ok) v = *reinterpret_cast<const u32x4 *>(qp + 32 * kk);
            qreg[kk] = __builtin_bit_cast(bf16x8, v);
        }
    }

    const char *head_base = reinterpret_cast<const char *>(a.kv) + (int64_t)g * a.kv_sh * C::EB;
    const int32_t *bt_row = a.block_table + (int64_t)b * a.bt_stride;

    f32x4 oacc[D / 16];
#pragma unroll
    for (int i = 0; i < D / 16; ++i) oacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY;   // running max (log2 units) of this wave's keys, per row
    float l_part = 0.f;        // this lane's share of the running sum

    // Per-page work of one wave: keys 16w .. 16w+15 of page p (already in LDS).
    auto compute_page = [&](int p) {
        // S^T[16 keys x 16 rows] = K Q^T.
        f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
        {
            const uint16_t *kp = ks + (16 * w + (lane & 15)) * C::KROW + 8 * (lane >> 4);
#pragma unroll
            for (int kk = 0; kk < D / 32; ++kk) {
                bf16x8 kop = *reinterpret_cast<const bf16x8 *>(kp + 32 * kk);
                sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qreg[kk], sacc, 0, 0, 0);
            }
        }
        // sacc[i] = score of key p*64 + 16w + 4*(lane/16) + i for this lane's row.
        const int key0 = p * kPage + 16 * w + 4 * (lane >> 4);
        float sv[4];
        float mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            sv[i] = (key0 + i < vis && key0 + i >= lo) ? sacc[i] * a.scale_log2 : -INFINITY;
            mx = fmaxf(mx, sv[i]);
        }
        mx = fmaxf(mx, shfl_xor_f32(mx, 16));
        mx = fmaxf(mx, shfl_xor_f32(mx, 32));
        const float m_new = fmaxf(m_run, mx);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = exp2_fast(m_run - m_use);
        m_run = m_new;
        bf16x4 pb;
        float psum = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const __bf16 pr = (__bf16)exp2_fast(sv[i] - m_use);
            pb[i] = pr;
            psum += (float)pr;   // the sum uses the same rounded P as the P.V product
        }
        l_part = l_part * alpha + psum;
        if (__any(alpha != 1.f)) {
#pragma unroll
            for (int i = 0; i < D / 16; ++i) oacc[i] *= alpha;
        }
        // O^T[d, row] += V^T[d, key] P^T[key, row] over this wave's 16 keys.
        const i16x4 pop = __builtin_bit_cast(i16x4, pb);
        const uint16_t *vp = vs + (16 * w + 4 * (lane >> 4) + ((lane & 15) >> 2)) * C::VROW + 4 * (lane & 3);
#pragma unroll
        for (int db = 0; db < D / 16; ++db) {
            const i16x4 vop = __builtin_bit_cast(i16x4, lds_read_tr16(vp + 16 * db));
            oacc[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vop, pop, oacc[db], 0, 0, 0);
        }
    };

    const int64_t sp = a.kv_sp;
    if constexpr (C::STAGES >= 3) {
        // A ring of STAGES pages in flight: page p stages in slot (p - p_begin)
        // % STAGES, and its slot is refilled with page p + STAGES once the
        // page is in LDS.  Each page id is read before the LDS store so its
        // latency overlaps it.
        u32x4 st[C::STAGES][C::CH_PER_THREAD];
#pragma unroll
        for (int k = 0; k < C::STAGES; ++k)
            if (p_begin + k < p_end)
                load_page<D, F8>(st[k], head_base, (int64_t)bt_row[p_begin + k] * sp, a.kv_ss, a.kv_skv, tid,
                                 L - (p_begin + k) * kPage);
        for (int p0 = p_begin; p0 < p_end; p0 += C::STAGES) {
#pragma unroll
            for (int k = 0; k < C::STAGES; ++k) {
                const int p = p0 + k;
                if (p >= p_end) break;           // uniform across the workgroup
                const int pn = p + C::STAGES;
                const int pid = pn < p_end ? bt_row[pn] : 0;
                __syncthreads();                 // the previous page is fully consumed
                store_page<D, F8>(st[k], ks, vs, tid);
                __syncthreads();
                if (pn < p_end)
                    load_page<D, F8>(st[k], head_base, (int64_t)pid * sp, a.kv_ss, a.kv_skv, tid, L - pn * kPage);
                compute_page(p);
            }
        }
    } else if constexpr (C::STAGES == 2) {
        // Two pages in flight: stage A holds even pages of the split, stage B
        // odd ones.  Each page id is read one compute phase before its loads
        // issue, so the block-table latency stays off the critical path.
        u32x4 stA[C::CH_PER_THREAD], stB[C::CH_PER_THREAD];
        if (p_begin < p_end)
            load_page<D, F8>(stA, head_base, (int64_t)bt_row[p_begin] * sp, a.kv_ss, a.kv_skv, tid,
                         L - p_begin * kPage);
        if (p_begin + 1 < p_end)
            load_page<D, F8>(stB, head_base, (int64_t)bt_row[p_begin + 1] * sp, a.kv_ss, a.kv_skv, tid,
                         L - (p_begin + 1) * kPage);
        int pid_a = (p_begin + 2 < p_end) ? bt_row[p_begin + 2] : 0;
        for (int p = p_begin; p < p_end; p += 2) {
            __syncthreads();                 // the previous page is fully consumed
            store_page<D, F8>(stA, ks, vs, tid);
            __syncthreads();
            if (p + 2 < p_end)
                load_page<D, F8>(stA, head_base, (int64_t)pid_a * sp, a.kv_ss, a.kv_skv, tid,
                             L - (p + 2) * kPage);
            const int pid_b = (p + 3 < p_end) ? bt_row[p + 3] : 0;
            compute_page(p);
            if (p + 1 >= p_end) break;       // uniform across the workgroup
            __syncthreads();
            store_page<D, F8>(stB, ks, vs, tid);
            __syncthreads();
            if (p + 3 < p_end)
                load_page<D, F8>(stB, head_base, (int64_t)pid_b * sp, a.kv_ss, a.kv_skv, tid,
                             L - (p + 3) * kPage);
            pid_a = (p + 4 < p_end) ? bt_row[p + 4] : 0;
            compute_page(p + 1);
        }
    } else {
        // One page in flight per workgroup; several workgroups per CU overlap.
        u32x4 st[C::CH_PER_THREAD];
        if (p_begin < p_end)
            load_page<D, F8>(st, head_base, (int64_t)bt_row[p_begin] * sp, a.kv_ss, a.kv_skv, tid,
                         L - p_begin * kPage);
        int pid = (p_begin + 1 < p_end) ? bt_row[p_begin + 1] : 0;
        for (int p = p_begin; p < p_end; ++p) {
            __syncthreads();                 // the previous page is fully consumed
            store_page<D, F8>(st, ks, vs, tid);
            __syncthreads();
            if (p + 1 < p_end)
                load_page<D, F8>(st, head_base, (int64_t)pid * sp, a.kv_ss, a.kv_skv, tid,
                             L - (p + 1) * kPage);
            pid = (p + 2 < p_end) ? bt_row[p + 2] : 0;
            compute_page(p);
        }
    }

    // ---- merge the four waves' (m, l, O) in LDS --------------------------
    float l_row = l_part + shfl_xor_f32(l_part, 16);
    l_row += shfl_xor_f32(l_row, 32);
    if (lane < 16) {
        red_m[w][lane] = m_run;
        red_l[w][lane] = l_row;
    }
    __syncthreads();   // also: all waves are done with the K/V tiles
    float M = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) M = fmaxf(M, red_m[ww][row]);
    const float M_use = (M == -INFINITY) ? 0.f : M;
    const float wgt = exp2_fast(m_run - M_use);
    float *ored = reinterpret_cast<float *>(smem);   // [4 waves][16 rows][D] f32
    static_assert(4 * 16 * D * 4 <= C::LDS_ELEMS * 2, "LDS too small for the merge");
#pragma unroll
    for (int db = 0; db < D / 16; ++db) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int d = 16 * db + 4 * (lane >> 4) + i;
            ored[(w * 16 + row) * D + d] = oacc[db][i] * wgt;
        }
    }
    __syncthreads();

    const bool split = a.max_splits > 1;
    // Thread -> (rows r = tid / D + k * (256 / D), column d = tid % D).
    constexpr int RSTEP = kThreads / D;   // 1 (D=256) or 2 (D=128)
    const int d = tid % D;
    for (int r = tid / D; r < rows; r += RSTEP) {
        float Mr = -INFINITY;
#pragma unroll
        for (int ww = 0; ww < 4; ++ww) Mr = fmaxf(Mr, red_m[ww][r]);
        const float Mr_use = (Mr == -INFINITY) ? 0.f : Mr;
        float lsum = 0.f, osum = 0.f;
#pragma unroll
        for (int ww = 0; ww < 4; ++ww) {
            lsum += red_l[ww][r] * exp2_fast(red_m[ww][r] - Mr_use);
            osum += ored[(ww * 16 + r) * D + d];
        }
        if constexpr (F8) osum *= a.v_scale;   // V = v_scale * e4m3(code)
        const int ri = r / G;
        const int rh = g * G + (r - ri * G);
        const int64_t t = q0 + ri;
        if (split) {
            // partial rows are indexed by (sequence, query index), not token,
            // so the workspace scales with n_seqs * max_q
            const int64_t prow = (int64_t)b * a.max_q + ri;
            const int64_t slot = (prow * a.hq + rh) * a.max_splits + s;
            if (a.fuse_merge) {
                // read by another workgroup of this launch: device-coherent
                store_coherent(a.part_o + slot * D + d, osum);
                if (d == 0) {
                    store_coherent(a.part_ml + slot * 2 + 0, Mr);
                    store_coherent(a.part_ml + slot * 2 + 1, lsum);
                }
            } else {
                a.part_o[slot * D + d] = osum;
                if (d == 0) {
                    a.part_ml[slot * 2 + 0] = Mr;
                    a.part_ml[slot * 2 + 1] = lsum;
                }
            }
        } else {
            if (a.sinks) {
                // the row's sink logit joins the normaliser (no value row)
                const float sink2 = a.sinks[rh] * kLog2e;
                if (sink2 != -INFINITY) lsum += exp2_fast(sink2 - Mr_use);
            }
            const float o = lsum > 0.f ? osum / lsum : 0.f;
            a.out[t * a.o_st + (int64_t)rh * a.o_sh + d] = f32_to_bf16_bits(o);
        }
    }
    if (!split || !a.fuse_merge) return;

    // ---- in-kernel merge ---------------------------------------------------
    // Every split of (b, g) that ran takes a ticket once its partials are
    // visible device-wide; the one that draws the last ticket merges all of
    // them in split order (the combine kernel's arithmetic, so both forms
    // give the same bits) and returns the counter to zero for the next call.
    // Nothing waits on another workgroup, so no ordering of workgroups can
    // stall the grid.
    //
    // Visibility without cache-wide fences: the partials are written with
    // device-scope stores (written through each XCD's L2 to the device
    // coherence point) and read back with device-scope loads (served from
    // that point, not from a stale L2 copy), so waiting for this workgroup's
    // stores to complete before the ticket is taken is all the ordering the
    // merge needs.  A device-scope fence would write back and invalidate the
    // whole L2 of the XCD in every workgroup instead.
    __shared__ int s_last;
    const int ns = split_count(npages, p_lo, a.pages_per_split, a.max_splits);
    int32_t *counter = a.counters + (int64_t)b * a.hkv + g;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this wave's partial stores completed
    __syncthreads();                                    // ... and every wave's
    if (tid == 0)
        s_last = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == ns - 1;
    __syncthreads();
    if (!s_last) return;
    for (int r = tid / D; r < rows; r += RSTEP) {
        const int ri = r / G;
        const int rh = g * G + (r - ri * G);
        const int64_t base = (((int64_t)b * a.max_q + ri) * a.hq + rh) * a.max_splits;
        float M = -INFINITY;
        for (int s2 = 0; s2 < ns; ++s2) M = fmaxf(M, load_coherent(a.part_ml + (base + s2) * 2));
        const float sink2 = a.sinks ? a.sinks[rh] * kLog2e : -INFINITY;
        M = fmaxf(M, sink2);
        float acc = 0.f, lsum = 0.f;
        if (M != -INFINITY) {
            for (int s2 = 0; s2 < ns; ++s2) {
                const float ms = load_coherent(a.part_ml + (base + s2) * 2);
                const float ls = load_coherent(a.part_ml + (base + s2) * 2 + 1);
                const float wgt = exp2_fast(ms - M);   // ms = -inf gives 0
                lsum += wgt * ls;
                acc += wgt * load_coherent(a.part_o + (base + s2) * D + d);
            }
            if (sink2 != -INFINITY) lsum += exp2_fast(sink2 - M);
        }
        const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
        a.out[(q0 + ri) * a.o_st + (int64_t)rh * a.o_sh + d] = f32_to_bf16_bits(acc * inv);
    }
    if (tid == 0) __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Log-sum-exp merge of the split partials: per (token, q head) row,
// M = max(max_s m_s, sink), w_s = 2^(m_s - M),
// out = sum_s w_s O_s / (sum_s w_s l_s + 2^(sink - M)); no sink = -inf.
// One wave64 per row; splits that hold no page of the sequence are skipped.
template <int D>
__global__ __launch_bounds__(kThreads) void paged_combine_kernel(const CombineArgs a) {
    const int lane = threadIdx.x & 63;
    const int h = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int i = blockIdx.y;
    const int b = blockIdx.z;
    if (h >= a.hq) return;
    const int q0 = a.cu_q[b];
    int n = a.cu_q[b + 1] - q0;
    if (n > a.max_q) n = a.max_q;
    if (i >= n) return;
    const int L = a.seq_lens[b];
    const int npages = (L + kPage - 1) / kPage;
    const int ns = split_count(npages, split_first_page(L, n, a.window), a.pages_per_split, a.max_splits);
    const int64_t t = q0 + i;
    const int64_t base = (((int64_t)b * a.max_q + i) * a.hq + h) * a.max_splits;

    float M = -INFINITY;
    for (int s = lane; s < ns; s += 64) M = fmaxf(M, a.part_ml[(base + s) * 2]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, 64));
    // the row's sink logit (log2 units) joins the normaliser, with no value row
    const float sink2 = a.sinks ? a.sinks[h] * kLog2e : -INFINITY;
    M = fmaxf(M, sink2);
    constexpr int PER = D / 64;
    float acc[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] = 0.f;
    float lsum = 0.f;
    if (M != -INFINITY) {
        for (int s = 0; s < ns; ++s) {
            const float ms = a.part_ml[(base + s) * 2];
            const float ls = a.part_ml[(base + s) * 2 + 1];
            const float wgt = exp2_fast(ms - M);   // ms = -inf gives 0
            lsum += wgt * ls;
            const float *po = a.part_o + (base + s) * D;
#pragma unroll
            for (int e = 0; e < PER; ++e) acc[e] += wgt * po[lane + 64 * e];
        }
        if (sink2 != -INFINITY) lsum += exp2_fast(sink2 - M);
    }
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
    uint16_t *op = a.out + t * a.o_st + (int64_t)h * a.o_sh;
#pragma unroll
    for (int e = 0; e < PER; ++e) op[lane + 64 * e] = f32_to_bf16_bits(acc[e] * inv);
}

template <int D>
hipError_t launch_decode_split(const AttnArgs &a, dim3 grid, hipStream_t stream) {
    if (a.kv_fp8)
        hipLaunchKernelGGL((paged_decode_split_kernel<D, true>), grid, dim3(kThreads), 0, stream, a);
    else
        hipLaunchKernelGGL((paged_decode_split_kernel<D, false>), grid, dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

template <int D>
hipError_t launch_combine(const CombineArgs &a, hipStream_t stream) {
    dim3 grid((a.hq + 3) / 4, a.max_q, a.n_seqs);
    hipLaunchKernelGGL(paged_combine_kernel<D>, grid, dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

// Zero n 32-bit words (the merge counters of a workspace).
__global__ __launch_bounds__(kThreads) void workspace_clear_kernel(uint32_t *p, size_t n) {
    for (size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += (size_t)gridDim.x * kThreads)
        p[i] = 0u;
}

hipError_t launch_workspace_clear(uint32_t *p, size_t words, hipStream_t stream) {
    if (words == 0) return hipSuccess;
    const size_t blocks = std::min<size_t>((words + kThreads - 1) / kThreads, 1024);
    hipLaunchKernelGGL(workspace_clear_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, p, words);
    return hipGetLastError();
}

hipError_t launch_decode_split_any(int D, const AttnArgs &a, dim3 grid, hipStream_t stream) {
    return D == 128 ? launch_decode_split<128>(a, grid, stream) : launch_decode_split<256>(a, grid, stream);
}

hipError_t launch_combine_any(int D, const CombineArgs &a, hipStream_t stream) {
    return D == 128 ? launch_combine<128>(a, stream) : launch_combine<256>(a, stream);
}

}  // namespace pa
