// Split-KV paged decode kernels (gfx950).
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
// Design (MI355X): one workgroup of 4 wave64 per (KV head, split); the
// splits are either fixed runs of pages of one sequence or, by default,
// equal ranges of the whole batch's pages (the balanced kernel below).  The
// pages stream through LDS with 16-byte coalesced non-temporal loads, staged
// in registers one or two pages ahead.  The G q heads x n query tokens of
// the KV head form the N side of the MFMA in blocks of 16 rows and the keys
// the M side ("swap AB"), so the score tile's C layout is directly the B
// operand of the P.V MFMA.  With RB row blocks (one for decode; two or four
// for short multi-token runs, the short-sequence body: up to 64 packed
// rows) the four waves form RB groups of 4 / RB: wave w takes row block
// w / (4 / RB) and a slice of 16 RB keys of every page, and keeps its own
// online softmax state; the waves of a row block merge in LDS at the end.
// Per wave the registers are those of one row block whatever RB is.  The
// softmax keeps a reference max per row that moves only when the row's max
// passes it by more than 2^8, so the common page needs no cross-lane max
// and no rescale (the split partials carry that reference as their m).
#pragma once

#include "attn_device.h"
#include "kv_quant.h"

namespace pa {

// Device-scope (all XCDs) relaxed store / load of a float.
__device__ __forceinline__ void store_coherent(float *p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(const float *p) {
    return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Load of an int32 that stays constant for the whole launch, from an address
// uniform across the wave, through the scalar cache: the wait for it counts
// scalar loads only, so it never waits for the page loads in flight (vector
// loads complete in order, and waiting for a vector load issued after them
// would wait for all of them).
__device__ __forceinline__ int32_t load_invariant_i32(const int32_t *p) {
    return *(const __attribute__((address_space(4))) int32_t *)p;
}

#ifndef PA_DECODE_LAZY_MAX
#define PA_DECODE_LAZY_MAX 1
#endif
constexpr float kDecodeRescaleThreshold = 8.f;   // log2 units

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
    // Lazily moved reference max (the softmax with a common factor that
    // cancels; no cross-lane max on the common path): decode batch fp8
    // +2.5%, short batch +1.5%, long decode +0.6%; over an fp8 cache at
    // D = 256 it measured 2.5-3% slower, so that instance keeps the exact
    // running max.
    static constexpr bool LAZY = PA_DECODE_LAZY_MAX && !(D == 256 && F8);
};


// Row block and key slice of wave w with RB row blocks: waves
// KW rb .. KW rb + KW - 1 (KW = 4 / RB) share row block rb and take
// consecutive slices of 16 RB keys of every page.
template <int RB>
__device__ __forceinline__ int decode_row_block(int w) { return RB == 1 ? 0 : w / (4 / RB); }
template <int RB>
__device__ __forceinline__ int decode_key_offset(int w) { return RB == 1 ? 16 * w : (w % (4 / RB)) * 16 * RB; }

// Issue the 16-byte loads of one page (K and V rows of one KV head) into
// registers.  Chunk c -> key = c / (2 DC), kv = (c / DC) % 2, dc = c % DC:
// consecutive threads read consecutive 16 bytes of one key's K row then V row.
// Every slot of the page is read, also those past the sequence's last key
// (they lie inside the page, and store_page replaces them by zeros): loads
// that always issue let the compiler count them, so waiting for one stage
// of the ring does not wait for the stages issued after it.  The loads are
// non-temporal (each K/V byte is read once per launch): on MI355X that
// raised a plain read stream from 6.45 to 7.3 TB/s and the decode kernels
// by 2-13%.
// `head_base` and the strides address pool elements (bf16 or fp8 bytes).
template <int D, bool F8>
__device__ __forceinline__ void load_page(u32x4 (&stage)[(DecodeCfg<D, F8>::CH_PER_THREAD)],
                                          const char *head_base, int64_t page_off,
                                          int64_t kv_ss, int64_t kv_skv, int tid) {
    using C = DecodeCfg<D, F8>;
#pragma unroll
    for (int it = 0; it < C::CH_PER_THREAD; ++it) {
        const int c = it * kThreads + tid;
        const int dc = c % C::DC;
        const int kv = (c / C::DC) & 1;
        const int key = c / (2 * C::DC);
        const char *src = head_base + (page_off + (int64_t)key * kv_ss + kv * kv_skv) * C::EB + dc * 16;
        stage[it] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(src));
    }
}


// Write a staged page into the LDS K and V tiles.  Slots at or past `valid`
// (the tail of a sequence's last page) stage as zeros: their memory may hold
// anything, and a non-finite V would turn the zero softmax weight of a
// masked key into NaN in P.V.  Slots in [valid_old, valid) are skipped: they
// are the step's new tokens under a fused KV-cache write, whose rows the
// holders of the new rows write (valid_old = valid without one).
template <int D, bool F8, bool MASK>
__device__ __forceinline__ void store_page_impl(const u32x4 (&stage)[(DecodeCfg<D, F8>::CH_PER_THREAD)],
                                                uint16_t *ks, uint16_t *vs, int tid, int valid, int valid_old) {
    using C = DecodeCfg<D, F8>;
#pragma unroll
    for (int it = 0; it < C::CH_PER_THREAD; ++it) {
        const int c = it * kThreads + tid;
        const int dc = c % C::DC;
        const int kv = (c / C::DC) & 1;
        const int key = c / (2 * C::DC);
        uint16_t *dst = kv ? (vs + key * C::VROW + dc * C::EPC) : (ks + key * C::KROW + dc * C::EPC);
        if (MASK && key >= valid_old && key < valid) continue;
        const u32x4 v = (!MASK || key < valid) ? stage[it] : u32x4{0u, 0u, 0u, 0u};
        if constexpr (!F8) {
            *reinterpret_cast<u32x4 *>(dst) = v;
        } else {
            // 16 codes -> 16 bf16 (dequantised; the scales are applied to
            // the scores and the output)
            uint32_t o[8];
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) e4m3x4_to_bf16x4(v[q4], o[2 * q4], o[2 * q4 + 1]);
            *reinterpret_cast<u32x4 *>(dst) = u32x4{o[0], o[1], o[2], o[3]};
            *reinterpret_cast<u32x4 *>(dst + 8) = u32x4{o[4], o[5], o[6], o[7]};
        }
    }
}

// `valid` and `valid_old` are uniform across the workgroup: a full page
// without new tokens takes the branch without the per-chunk selects.
template <int D, bool F8>
__device__ __forceinline__ void store_page(const u32x4 (&stage)[(DecodeCfg<D, F8>::CH_PER_THREAD)],
                                           uint16_t *ks, uint16_t *vs, int tid, int valid, int valid_old) {
    if (valid >= kPage && valid_old >= kPage)
        store_page_impl<D, F8, false>(stage, ks, vs, tid, valid, valid_old);
    else
        store_page_impl<D, F8, true>(stage, ks, vs, tid, valid, min(valid_old, valid));
}

// One thread's share of a fused KV-cache write for one (sequence, KV head):
// chunk c = tid of its new rows, token i = c / (2 DC), K (kv = 0) or V
// (kv = 1) row, elements [EPC e, EPC e + EPC).  The bf16 input is loaded
// when the piece starts; when the page holding key position `pos` is staged
// the holder writes the value attention must see into the LDS tile (the
// bf16 row, or the decoded e4m3 codes over an fp8 cache), and after the
// piece its pool slot (bf16 or codes).  The host fuses the write only when
// every chunk has a holder (n 2 DC <= 256).
template <int D, bool F8>
struct NewKV {
    u32x4 val[F8 ? 2 : 1];   // the new row's EPC elements (bf16)
    char *pool;              // the chunk's pool address once its page is staged, else null
    int pos;                 // key position, or -1: no chunk (or a token with no slot)
    int kv, e;
};

template <int D, bool F8>
__device__ __forceinline__ void load_new_kv(const AttnArgs &a, int q0, int n, int L, int g, int tid,
                                            NewKV<D, F8> &nk) {
    using C = DecodeCfg<D, F8>;
    nk.pos = -1;
    nk.pool = nullptr;
    nk.kv = (tid / C::DC) & 1;
    nk.e = tid % C::DC;
    if (!a.k_new) return;   // uniform: no fused write
    const int i = tid / (2 * C::DC);
    const int pos = L - n + i;
    if (i < n && pos >= 0) {
        const int64_t t = q0 + i;
        const uint16_t *src = (nk.kv ? a.v_new + t * a.vn_st + (int64_t)g * a.vn_sh
                                     : a.k_new + t * a.kn_st + (int64_t)g * a.kn_sh) + C::EPC * nk.e;
#pragma unroll
        for (int w = 0; w < (F8 ? 2 : 1); ++w) nk.val[w] = *reinterpret_cast<const u32x4 *>(src + 8 * w);
        nk.pos = pos;
    }
}

// While page p (id pid) is staged: the holder of a new slot in it writes the
// slot's LDS row and remembers its pool address.
template <int D, bool F8>
__device__ __forceinline__ void new_kv_stage(const AttnArgs &a, NewKV<D, F8> &nk, uint16_t *ks, uint16_t *vs,
                                             const char *head_base, int p, int pid) {
    using C = DecodeCfg<D, F8>;
    const int key = nk.pos - p * kPage;
    if (key < 0 || key >= kPage) return;
    uint16_t *dst = nk.kv ? (vs + key * C::VROW + nk.e * C::EPC) : (ks + key * C::KROW + nk.e * C::EPC);
    if constexpr (!F8) {
        *reinterpret_cast<u32x4 *>(dst) = nk.val[0];
    } else {
        const u32x4 codes = bf16x16_to_e4m3(nk.val[0], nk.val[1], nk.kv ? a.v_inv : a.k_inv);
        uint32_t o[8];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) e4m3x4_to_bf16x4(codes[q4], o[2 * q4], o[2 * q4 + 1]);
        *reinterpret_cast<u32x4 *>(dst) = u32x4{o[0], o[1], o[2], o[3]};
        *reinterpret_cast<u32x4 *>(dst + 8) = u32x4{o[4], o[5], o[6], o[7]};
    }
    nk.pool = const_cast<char *>(head_base) +
              ((int64_t)pid * a.kv_sp + (int64_t)key * a.kv_ss + nk.kv * a.kv_skv) * C::EB + nk.e * 16;
}

// After the piece: the holder stores its slot into the pool (a 16-byte
// store; outside the page ring, so the ring's load counts stay exact).
template <int D, bool F8>
__device__ __forceinline__ void new_kv_commit(const AttnArgs &a, NewKV<D, F8> &nk) {
    if (!nk.pool) return;
    if constexpr (!F8)
        *reinterpret_cast<u32x4 *>(nk.pool) = nk.val[0];
    else
        *reinterpret_cast<u32x4 *>(nk.pool) = bf16x16_to_e4m3(nk.val[0], nk.val[1], nk.kv ? a.v_inv : a.k_inv);
    nk.pool = nullptr;
}

// Per-page work of one wave: the RB blocks of 16 keys starting at key kw0 of
// page p (already in LDS) against the 16 rows whose Q^T fragments are in
// qreg (lane row = lane % 16 of the wave's row block, visible keys
// [lo, vis)); updates the wave's online-softmax state.
template <int D, bool F8, int RB>
__device__ __forceinline__ void decode_compute_page(const uint16_t *ks, const uint16_t *vs,
                                                    const bf16x8 (&qreg)[D / 32], f32x4 (&oacc)[D / 16],
                                                    float &m_run, float &l_part, int p, int vis, int lo,
                                                    float scale_log2, int kw0, int lane) {
    using C = DecodeCfg<D, F8>;
    // S^T[16 keys x 16 rows] = K Q^T per key block.
    f32x4 sacc[RB];
#pragma unroll
    for (int kb = 0; kb < RB; ++kb) sacc[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
    {
        const uint16_t *kp = ks + (kw0 + (lane & 15)) * C::KROW + 8 * (lane >> 4);
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk) {
#pragma unroll
            for (int kb = 0; kb < RB; ++kb) {
                const bf16x8 kop = *reinterpret_cast<const bf16x8 *>(kp + 16 * kb * C::KROW + 32 * kk);
                sacc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qreg[kk], sacc[kb], 0, 0, 0);
            }
        }
    }
    // sacc[kb][i] = score of key p*64 + kw0 + 16 kb + 4*(lane/16) + i for this lane's row.
    const int key0 = p * kPage + kw0 + 4 * (lane >> 4);
    float sv[RB][4];
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < RB; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int key = key0 + 16 * kb + i;
            sv[kb][i] = (key < vis && key >= lo) ? sacc[kb][i] * scale_log2 : -INFINITY;
            mx = fmaxf(mx, sv[kb][i]);
        }
    // P = exp2(s - m_use) rounded to bf16, and the row-sum share of the same
    // rounded values (the sum uses the P of the P.V product)
    i16x4 pop[RB];
    float psum;
    auto weights = [&](float m_use) {
        psum = 0.f;
#pragma unroll
        for (int kb = 0; kb < RB; ++kb) {
            bf16x4 pb;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const __bf16 pr = (__bf16)exp2_fast(sv[kb][i] - m_use);
                pb[i] = pr;
                psum += (float)pr;
            }
            pop[kb] = __builtin_bit_cast(i16x4, pb);
        }
    };
    if constexpr (C::LAZY) {
        // m_run is a reference max that moves only when a row's max passes
        // it by more than 2^8 (P <= 256).  Each lane tests its own four
        // scores; only when some lane of the wave passes are the row's lanes
        // combined (two cross-lane exchanges), the reference moved and O, l
        // rescaled.
        if (__any(mx > m_run + kDecodeRescaleThreshold)) {
            mx = fmaxf(mx, shfl_xor_f32(mx, 16));
            mx = fmaxf(mx, shfl_xor_f32(mx, 32));
            const float m_new = mx > m_run + kDecodeRescaleThreshold ? mx : m_run;
            const float alpha = exp2_fast(m_run - ((m_new == -INFINITY) ? 0.f : m_new));
            m_run = m_new;
            l_part *= alpha;
#pragma unroll
            for (int i = 0; i < D / 16; ++i) oacc[i] *= alpha;
        }
        weights((m_run == -INFINITY) ? 0.f : m_run);
        l_part += psum;
    } else {
        // exact running max
        mx = fmaxf(mx, shfl_xor_f32(mx, 16));
        mx = fmaxf(mx, shfl_xor_f32(mx, 32));
        const float m_new = fmaxf(m_run, mx);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = exp2_fast(m_run - m_use);
        m_run = m_new;
        weights(m_use);
        l_part = l_part * alpha + psum;
        if (__any(alpha != 1.f)) {
#pragma unroll
            for (int i = 0; i < D / 16; ++i) oacc[i] *= alpha;
        }
    }
    // O^T[d, row] += V^T[d, key] P^T[key, row] over this wave's keys.
    const uint16_t *vp = vs + (kw0 + 4 * (lane >> 4) + ((lane & 15) >> 2)) * C::VROW + 4 * (lane & 3);
#pragma unroll
    for (int db = 0; db < D / 16; ++db) {
#pragma unroll
        for (int kb = 0; kb < RB; ++kb) {
            const i16x4 vop = __builtin_bit_cast(i16x4, lds_read_tr16(vp + 16 * kb * C::VROW + 16 * db));
            oacc[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vop, pop[kb], oacc[db], 0, 0, 0);
        }
    }
}

// Merge the (m, l, O) of the waves of each row block (4 / RB waves per
// block) of one (sequence, KV head) piece in LDS, then write each of its
// rows: the unnormalised partial and (max, sum) in split slot split_idx
// (device-coherent stores when another workgroup of the launch reads
// them), or, when the piece is the whole sequence, the normalised bf16
// output with the row's sink in the normaliser.  Starts with a barrier (all
// waves done with the K/V tiles); reuses the K/V LDS area.
template <int D, bool F8, int RB>
__device__ __forceinline__ void decode_merge_write(const AttnArgs &a, uint16_t *smem, float (&red_m)[4][16],
                                                   float (&red_l)[4][16], const f32x4 (&oacc)[D / 16],
                                                   float m_run, float l_part, int b, int g, int q0, int rows,
                                                   bool split, int split_idx, bool coherent, int tid) {
    using C = DecodeCfg<D, F8>;
    constexpr int KW = 4 / RB;   // waves per row block
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int row = lane & 15;
    const int w0 = KW == 4 ? 0 : w - w % KW;   // first wave of this wave's row block
    const int G = a.group;
    float l_row = l_part + shfl_xor_f32(l_part, 16);
    l_row += shfl_xor_f32(l_row, 32);
    if (lane < 16) {
        red_m[w][lane] = m_run;
        red_l[w][lane] = l_row;
    }
    __syncthreads();   // also: all waves are done with the K/V tiles
    float M = -INFINITY;
#pragma unroll
    for (int k = 0; k < KW; ++k) M = fmaxf(M, red_m[w0 + k][row]);
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

    // Thread -> (rows r = tid / D + k * (256 / D), column d = tid % D).
    // Packed row r is row r % 16 of row block r / 16, held by waves
    // KW (r / 16) .. + KW - 1.
    constexpr int RSTEP = kThreads / D;   // 1 (D=256) or 2 (D=128)
    const int d = tid % D;
    for (int r = tid / D; r < rows; r += RSTEP) {
        const int rw0 = KW == 4 ? 0 : (r / 16) * KW, rr = KW == 4 ? r : r % 16;
        float Mr = -INFINITY;
#pragma unroll
        for (int k = 0; k < KW; ++k) Mr = fmaxf(Mr, red_m[rw0 + k][rr]);
        const float Mr_use = (Mr == -INFINITY) ? 0.f : Mr;
        float lsum = 0.f, osum = 0.f;
#pragma unroll
        for (int k = 0; k < KW; ++k) {
            lsum += red_l[rw0 + k][rr] * exp2_fast(red_m[rw0 + k][rr] - Mr_use);
            osum += ored[((rw0 + k) * 16 + rr) * D + d];
        }
        if constexpr (F8) osum *= a.v_scale;   // V = v_scale * e4m3(code)
        const int ri = r / G;
        const int rh = g * G + (r - ri * G);
        const int64_t t = q0 + ri;
        if (split) {
            // partial rows are indexed by (sequence, query index), not token,
            // so the workspace scales with n_seqs * max_q
            const int64_t prow = (int64_t)b * a.max_q + ri;
            const int64_t slot = (prow * a.hq + rh) * a.max_splits + split_idx;
            if (coherent) {
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
}

// Stream pages [p_begin, p_end) of one (sequence, KV head) through LDS into
// the wave's online-softmax state: the ring of register stages (loads of
// the next pages in flight while a page is computed), STAGES deep.
//
// The compiler's wait for one stage is exact only if every path into it
// issued the same loads, so: page loads always issue (past the last page a
// stage reloads the last page, still in L2; the tail of a sequence's last
// page is read and zeroed in LDS), page ids come through the scalar cache,
// read a compute phase ahead, and the ring has one exit.  Otherwise the
// wait covers every load in flight and the ring drains at each page.
template <int D, bool F8, int RB, bool W>
__device__ __forceinline__ void decode_stream_pages(const AttnArgs &a, uint16_t *ks, uint16_t *vs,
                                                    const char *head_base, const int32_t *bt_row, int p_begin,
                                                    int p_end, int L, const bf16x8 (&qreg)[D / 32],
                                                    f32x4 (&oacc)[D / 16], float &m_run, float &l_part, int vis,
                                                    int lo, int tid,
                                                    u32x4 (&st1)[(DecodeCfg<D, F8>::CH_PER_THREAD)],
                                                    bool preloaded, int next_pid, NewKV<D, F8> &nk, int nv_lo) {
    using C = DecodeCfg<D, F8>;
    const int lane = tid & 63;
    const int kw0 = decode_key_offset<RB>(tid >> 6);
    auto compute_page = [&](int p) {
        decode_compute_page<D, F8, RB>(ks, vs, qreg, oacc, m_run, l_part, p, vis, lo, a.scale_log2, kw0, lane);
    };
    // Stage page p from a register stage; under a fused KV-cache write (W)
    // the slots of new tokens (key positions [nv_lo, L)) come from their holders.
    auto stage_page = [&](const u32x4 (&stg)[C::CH_PER_THREAD], int p) {
        if constexpr (W) {
            store_page<D, F8>(stg, ks, vs, tid, L - p * kPage, nv_lo - p * kPage);
            if (nv_lo < L && (p + 1) * kPage > nv_lo)   // uniform: the page holds new tokens
                new_kv_stage<D, F8>(a, nk, ks, vs, head_base, p, load_invariant_i32(bt_row + p));
        } else {
            store_page<D, F8>(stg, ks, vs, tid, L - p * kPage, L - p * kPage);
        }
    };
    const int64_t sp = a.kv_sp;
    const int p_last = p_end - 1;
    auto load_id = [&](u32x4 (&stg)[C::CH_PER_THREAD], int pid) {
        load_page<D, F8>(stg, head_base, (int64_t)pid * sp, a.kv_ss, a.kv_skv, tid);
    };
    auto refill = [&](u32x4 (&stg)[C::CH_PER_THREAD], int p) { load_id(stg, load_invariant_i32(bt_row + min(p, p_last))); };
    if (p_begin > p_last) {
        // no page
    } else if constexpr (C::STAGES >= 3) {
        // A ring of STAGES pages in flight: page p stages in slot (p - p_begin)
        // % STAGES, and its slot is refilled with page p + STAGES once the
        // page is in LDS.
        u32x4 st[C::STAGES][C::CH_PER_THREAD];
#pragma unroll
        for (int k = 0; k < C::STAGES; ++k)
            refill(st[k], p_begin + k);
        for (int p0 = p_begin; p0 < p_end; p0 += C::STAGES) {
#pragma unroll
            for (int k = 0; k < C::STAGES; ++k) {
                // Past the last page the group's remaining slots are skipped
                // (uniform) but the loop body keeps one exit, at its end, so
                // every path into the loop head has the same loads in flight.
                const int p = p0 + k;
                const bool live = p < p_end;
                if (live) {
                    __syncthreads();             // the previous page is fully consumed
                    stage_page(st[k], p);
                    __syncthreads();
                }
                refill(st[k], p + C::STAGES);
                if (live) compute_page(p);
            }
        }
    } else if constexpr (C::STAGES == 2) {
        // Two pages in flight: stage A holds even pages of the split, stage B
        // odd ones.  Each page id is read one compute phase before its loads
        // issue, so the block-table latency stays off the critical path.
        u32x4 stA[C::CH_PER_THREAD], stB[C::CH_PER_THREAD];
        refill(stA, p_begin);
        refill(stB, p_begin + 1);
        int pid_a = load_invariant_i32(bt_row + min(p_begin + 2, p_last));
        for (int p = p_begin; p < p_end; p += 2) {
            __syncthreads();                 // the previous page is fully consumed
            stage_page(stA, p);
            __syncthreads();
            load_id(stA, pid_a);
            const int pid_b = load_invariant_i32(bt_row + min(p + 3, p_last));
            compute_page(p);
            if (p + 1 >= p_end) break;       // uniform across the workgroup
            __syncthreads();
            stage_page(stB, p + 1);
            __syncthreads();
            load_id(stB, pid_b);
            pid_a = load_invariant_i32(bt_row + min(p + 4, p_last));
            compute_page(p + 1);
        }
    } else {
        // One page in flight per workgroup; several workgroups per CU overlap.
        // The stage st1 is the caller's: it may arrive holding page p_begin
        // (loaded during the previous piece's last page) and, given the next
        // piece's first page id, leave holding that page instead of a reload
        // of the last one, so a piece boundary does not restart the stream.
        auto pid_after = [&](int q) {   // id of the page to load once page q - 1 is stored
            const int id = load_invariant_i32(bt_row + min(q, p_last));
            return (q > p_last && next_pid >= 0) ? next_pid : id;
        };
        if (!preloaded) refill(st1, p_begin);
        int pid = pid_after(p_begin + 1);
        for (int p = p_begin; p < p_end; ++p) {
            __syncthreads();                 // the previous page is fully consumed
            stage_page(st1, p);
            __syncthreads();
            load_id(st1, pid);
            pid = pid_after(p + 2);
            compute_page(p);
        }
    }
}

// This lane's packed row (row lane % 16 of its wave's row block) of a
// (sequence, KV head) with n query tokens, L keys and `rows` packed rows:
// its visible key range [lo, vis) and Q^T fragments as the B operand of
// v_mfma_f32_16x16x32_bf16 (lane holds q[row, 32 kk + 8 (lane / 16) .. +7];
// zeros for rows past the end).
template <int D, int RB>
__device__ __forceinline__ void load_q_rows(const AttnArgs &a, int q0, int n, int L, int g, int rows, int tid,
                                            bf16x8 (&qreg)[D / 32], int &vis, int &lo) {
    const int G = a.group;
    const int lane = tid & 63;
    const int row = 16 * decode_row_block<RB>(tid >> 6) + (lane & 15);
    const bool row_ok = row < rows;
    const int qi = row / G;
    const int h = g * G + (row - qi * G);
    vis = row_ok ? visible_keys(L, n, qi, a.causal) : 0;
    lo = row_ok ? window_start(L - n + qi, a.window) : 0;   // first key inside the window
    const uint16_t *qp = a.q + (int64_t)(q0 + qi) * a.q_st + (int64_t)h * a.q_sh + 8 * (lane >> 4);
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) {
        u32x4 v = {0u, 0u, 0u, 0u};
        if (row_ok) v = *reinterpret_cast<const u32x4 *>(qp + 32 * kk);
        qreg[kk] = __builtin_bit_cast(bf16x8, v);
    }
}

template <int D, bool F8, int RB, bool W>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(decode_waves(D, F8, RB))))
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
    if (rows > 16 * RB) rows = 16 * RB;

    // This lane's query row (the N index of the MFMA tiles) and its Q^T.
    int vis, lo;
    bf16x8 qreg[D / 32];
    load_q_rows<D, RB>(a, q0, n, L, g, rows, tid, qreg, vis, lo);

    const char *head_base = reinterpret_cast<const char *>(a.kv) + (int64_t)g * a.kv_sh * C::EB;
    const int32_t *bt_row = a.block_table + (int64_t)b * a.bt_stride;

    f32x4 oacc[D / 16];
#pragma unroll
    for (int i = 0; i < D / 16; ++i) oacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY;   // running max (log2 units) of this wave's keys, per row
    float l_part = 0.f;        // this lane's share of the running sum

    NewKV<D, F8> nk;
    if constexpr (W) load_new_kv<D, F8>(a, q0, n, L, g, tid, nk);
    u32x4 st1[C::CH_PER_THREAD];
    decode_stream_pages<D, F8, RB, W>(a, ks, vs, head_base, bt_row, p_begin, p_end, L, qreg, oacc, m_run, l_part,
                                      vis, lo, tid, st1, false, -1, nk, W ? L - n : L);
    if constexpr (W) new_kv_commit<D, F8>(a, nk);

    // ---- merge the waves' (m, l, O) in LDS, write -------------------------
    const bool split = a.max_splits > 1;
    decode_merge_write<D, F8, RB>(a, smem, red_m, red_l, oacc, m_run, l_part, b, g, q0, rows, split, s,
                                  a.fuse_merge != 0, tid);
    constexpr int RSTEP = kThreads / D;
    const int d = tid % D;
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

// ---- balanced split decode --------------------------------------------------
// The pages the batch needs (each sequence's pages from the first one inside
// row 0's window, sequences in order) are dealt out as gridDim.y equal
// contiguous ranges of C = max(ceil(total / gridDim.y), pages_per_split)
// pages; workgroup (g, r) streams range r for KV head g, so every workgroup
// of the launch reads the same number of pages whatever the mix of lengths.
// A range may end inside one sequence and go on into the next: each
// (sequence, range) piece is streamed with its own online-softmax state.  A
// sequence held by one range is written out directly; otherwise its pieces
// go to split slots r - floor(F_b / C) (F_b = pages of the sequences before
// it) and the combine kernel merges them.  pages_per_split (the plan's
// minimum C) bounds a sequence's pieces by max_splits.
//
// Every workgroup derives the partition itself from seq_lens and cu_q (an
// LDS prefix sum over at most kBalMaxSeqs sequences), so nothing but the
// launch orders the two kernels.  Workgroup (0, 0) publishes each
// sequence's piece count for the combine kernel.
template <int D, bool F8, int RB, bool W>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(decode_waves(D, F8, RB))))
void paged_decode_balanced_kernel(const AttnArgs a) {
    using C = DecodeCfg<D, F8>;
    __shared__ __attribute__((aligned(16))) uint16_t smem[C::LDS_ELEMS];
    __shared__ float red_m[4][16];
    __shared__ float red_l[4][16];
    // s_F[b] = pages of the sequences before b.  A piece re-reads its
    // sequence's length and rows through the scalar cache: keeping them in
    // LDS too (12 KB more) left room for one workgroup per CU instead of two
    // over an fp8 cache at D = 256 (long fp8 decode 6050 -> 6650 GB/s).
    __shared__ int s_F[kBalMaxSeqs + 1];
    auto seq_L = [&](int bb) { return load_invariant_i32(a.seq_lens + bb); };
    __shared__ int s_wsum[4];
    __shared__ int s_first;
    uint16_t *ks = smem;
    uint16_t *vs = smem + kPage * C::KROW;

    const int g = blockIdx.x;
    const int r = blockIdx.y;
    const int R = gridDim.y;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int B = a.n_seqs;       // <= kBalMaxSeqs (the plan checks)
    const int G = a.group;

    // ---- the partition: pages per sequence and their prefix sum ----------
    int np4[4];
    int tsum = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int bb = 4 * tid + j;
        int np = 0;
        if (bb < B) {
            const int L = a.seq_lens[bb];
            const int q0 = a.cu_q[bb];
            int n = a.cu_q[bb + 1] - q0;
            if (n > a.max_q) n = a.max_q;   // caller contract: n_b <= max_q
            if (n > 0 && L > 0) np = (L + kPage - 1) / kPage - split_first_page(L, n, a.window);
        }
        np4[j] = np;
        tsum += np;
    }
    int incl = tsum;   // inclusive scan over the wave
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int v = __shfl_up(incl, off, 64);
        if (lane >= off) incl += v;
    }
    if (lane == 63) s_wsum[w] = incl;
    __syncthreads();
    int run = incl - tsum;
    for (int ww = 0; ww < w; ++ww) run += s_wsum[ww];
    if (tid == 0) s_F[0] = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        run += np4[j];
        s_F[4 * tid + j + 1] = run;   // entries past B repeat the total
    }
    __syncthreads();
    const int total = s_F[B];
    int Cr = (total + R - 1) / R;
    if (Cr < a.pages_per_split) Cr = a.pages_per_split;
    if (g == 0 && r == 0) {
        for (int bb = tid; bb < B; bb += kThreads) {
            const int F0 = s_F[bb], np = s_F[bb + 1] - F0;
            a.seg_splits[bb] = np > 0 ? (F0 + np - 1) / Cr - F0 / Cr + 1 : 0;
        }
    }
    if ((int64_t)r * Cr >= total) return;   // uniform: nothing left for this range
    const int u0 = r * Cr;
    const int nunits = min(total - u0, Cr);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int bb = 4 * tid + j;
        if (bb < B && s_F[bb] <= u0 && u0 < s_F[bb + 1]) s_first = bb;   // exactly one such sequence
    }
    __syncthreads();

    const char *head_base = reinterpret_cast<const char *>(a.kv) + (int64_t)g * a.kv_sh * C::EB;
    f32x4 oacc[D / 16];
    bf16x8 qreg[D / 32];

    // The range's pieces, in sequence order: sequence b from page p.
    int b = __builtin_amdgcn_readfirstlane(s_first);
    int p = __builtin_amdgcn_readfirstlane((seq_L(b) + kPage - 1) / kPage - (s_F[b + 1] - s_F[b]) + (u0 - s_F[b]));
    int left = nunits;
    // With one register stage the next piece's first page is loaded during
    // the current piece's last page (the stage is carried across pieces).
    constexpr bool kCarry = C::STAGES == 1;
    u32x4 st1[C::CH_PER_THREAD];
    bool preloaded = false;
    while (true) {   // uniform
        const int L = load_invariant_i32(a.seq_lens + b);
        const int q0 = load_invariant_i32(a.cu_q + b);
        const int n = min(load_invariant_i32(a.cu_q + b + 1) - q0, a.max_q);   // caller contract: n_b <= max_q
        const int F0 = __builtin_amdgcn_readfirstlane(s_F[b]);
        const int np = __builtin_amdgcn_readfirstlane(s_F[b + 1]) - F0;
        const int cnt = min(left, (L + kPage - 1) / kPage - p);
        // The next piece, if any: the next sequence with pages, from its first page.
        int b2 = b, p2 = 0, next_pid = -1;
        if (left > cnt) {
            do {
                ++b2;
            } while (s_F[b2 + 1] == s_F[b2]);   // a later sequence with pages exists: left > cnt
            b2 = __builtin_amdgcn_readfirstlane(b2);
            p2 = __builtin_amdgcn_readfirstlane((seq_L(b2) + kPage - 1) / kPage - (s_F[b2 + 1] - s_F[b2]));
            if constexpr (kCarry) next_pid = load_invariant_i32(a.block_table + (int64_t)b2 * a.bt_stride + p2);
        }
        const int rows = min(n * G, 16 * RB);
        int vis, lo;
        load_q_rows<D, RB>(a, q0, n, L, g, rows, tid, qreg, vis, lo);
#pragma unroll
        for (int i = 0; i < D / 16; ++i) oacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
        float m_run = -INFINITY;
        float l_part = 0.f;
        NewKV<D, F8> nk;
        if constexpr (W) load_new_kv<D, F8>(a, q0, n, L, g, tid, nk);
        decode_stream_pages<D, F8, RB, W>(a, ks, vs, head_base, a.block_table + (int64_t)b * a.bt_stride, p,
                                          p + cnt, L, qreg, oacc, m_run, l_part, vis, lo, tid, st1, preloaded,
                                          next_pid, nk, W ? L - n : L);
        if constexpr (W) new_kv_commit<D, F8>(a, nk);
        // The piece: the whole sequence (written out) or split slot
        // r - floor(F_b / C) of its ns pieces.
        const int ns = (F0 + np - 1) / Cr - F0 / Cr + 1;
        decode_merge_write<D, F8, RB>(a, smem, red_m, red_l, oacc, m_run, l_part, b, g, q0, rows, ns > 1,
                                      r - F0 / Cr, false, tid);
        left -= cnt;
        if (left <= 0) break;
        // Deeper rings wait for the piece's stores before the next piece's
        // loads: while stores are in flight the compiler cannot count loads
        // exactly (stores and loads share the counter) and would drain the
        // ring at every page.  A one-stage ring waits for all loads at each
        // page anyway, and its next page is already in flight.
        if constexpr (!kCarry) __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0); expcnt, lgkmcnt unchanged
        b = b2;
        p = p2;
        preloaded = kCarry;
    }
}

// Row blocks of 16 packed rows: one for decode (<= 16 rows), two or four for
// the short-sequence body (<= 32 / <= 64 rows).
template <int D, bool F8, bool W>
hipError_t launch_decode_split_rb(const AttnArgs &a, dim3 grid, hipStream_t stream) {
    if (a.row_blocks <= 1)
        hipLaunchKernelGGL((paged_decode_split_kernel<D, F8, 1, W>), grid, dim3(kThreads), 0, stream, a);
    else if (a.row_blocks == 2)
        hipLaunchKernelGGL((paged_decode_split_kernel<D, F8, 2, W>), grid, dim3(kThreads), 0, stream, a);
    else
        hipLaunchKernelGGL((paged_decode_split_kernel<D, F8, 4, W>), grid, dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

template <int D, bool F8, bool W>
hipError_t launch_decode_balanced_rb(const AttnArgs &a, dim3 grid, hipStream_t stream) {
    if (a.row_blocks <= 1)
        hipLaunchKernelGGL((paged_decode_balanced_kernel<D, F8, 1, W>), grid, dim3(kThreads), 0, stream, a);
    else if (a.row_blocks == 2)
        hipLaunchKernelGGL((paged_decode_balanced_kernel<D, F8, 2, W>), grid, dim3(kThreads), 0, stream, a);
    else
        hipLaunchKernelGGL((paged_decode_balanced_kernel<D, F8, 4, W>), grid, dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

// The kernels with the fused KV-cache write are separate instantiations, so
// the plain decode kernels carry none of its state.
template <int D, bool F8>
hipError_t launch_decode_split_w(const AttnArgs &a, dim3 grid, hipStream_t stream) {
    return a.k_new ? launch_decode_split_rb<D, F8, true>(a, grid, stream)
                   : launch_decode_split_rb<D, F8, false>(a, grid, stream);
}

template <int D, bool F8>
hipError_t launch_decode_balanced_w(const AttnArgs &a, dim3 grid, hipStream_t stream) {
    return a.k_new ? launch_decode_balanced_rb<D, F8, true>(a, grid, stream)
                   : launch_decode_balanced_rb<D, F8, false>(a, grid, stream);
}

}  // namespace pa
