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
// Design (MI355X):
//  * One workgroup of 4 wave64 per (sequence, KV head, tile of 256 packed
//    query rows).  Row r of a (sequence, KV head) is query token r / G,
//    q head g*G + r % G, so the G heads sharing a KV head share every K/V
//    tile.  Each wave owns 64 rows as two 32-row MFMA blocks, so every K or
//    V operand read from LDS feeds two MFMAs: 64 FLOP per LDS byte, half of
//    the LDS bandwidth the MFMA rate needs with 32 rows per wave.
//  * K/V pages (64 keys) stream HBM -> LDS with direct 16-byte loads
//    (global_load_lds_dwordx4), no register staging, through a ring of
//    STAGES page buffers (3 at D = 128, 2 at D = 256).  Rows are stored with
//    an XOR swizzle of their 16-byte chunks (chunk c of key k at c ^ 2(k&7))
//    so both the b128 K reads and the transposing V reads are bank-conflict
//    free without padding.
//  * S^T = K Q^T on v_mfma_f32_32x32x16_bf16 with keys on M: each lane owns
//    one query row per block, so row max / row sum are in-lane plus one
//    permlane32 swap.  The S^T C layout is directly the B operand of
//    O^T += V^T P^T, whose V^T operand comes from the row-major V tile via
//    the LDS transpose read (ds_read_b64_tr_b16).
//  * Online softmax in log2 units with a lazily moved reference max: the
//    reference only moves (and O, l are rescaled) when a row's max exceeds
//    it by more than 2^8, so P <= 256 and rescales are rare.  The result is
//    the same softmax; only the common factor cancelled at the end differs.
//  * Tiles past the causal frontier of the workgroup's last row are never
//    loaded; a wave skips the tiles past its own rows' frontier; tiles below
//    the first row's frontier skip the mask.
#include "attn_device.h"

namespace pa {

template <int D>
struct PfCfg {
    static constexpr int WAVES = 4;
    // 32-row MFMA blocks per wave: two at D = 128 (every LDS operand feeds
    // two MFMAs); one at D = 256, where two blocks' Q and O would not fit
    // the 512 registers of a lane.
    static constexpr int RB = D == 128 ? 2 : 1;
    static constexpr int BM = WAVES * RB * 32;      // packed query rows per workgroup
    static constexpr int CH = D / 8;                // 16-byte chunks per K or V row
    static constexpr int STAGES = D == 128 ? 3 : 2;
    static constexpr int TILE = kPage * D;          // bf16 elements of one K (or V) page tile
    static constexpr int KSTEP = 32;                // keys per softmax step
    static constexpr int KB = KSTEP / 32;           // 32-key MFMA blocks per softmax step
    static constexpr int LOADS = kPage * CH / kThreads;  // 16-byte loads per thread per K tile
};
static_assert(PfCfg<128>::BM == prefill_rows(128) && PfCfg<256>::BM == prefill_rows(256), "row tile");

constexpr float kRescaleThreshold = 8.f;   // log2 units: P stays <= 256

__device__ __forceinline__ float max_xor32(float x) {
    // lanes l and l ^ 32 exchange values (v_permlane32_swap)
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor32(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// LDS byte address of a __shared__ pointer (the value M0 takes).
__device__ __forceinline__ uint32_t lds_address(const void *p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}

// One direct 16-byte HBM -> LDS load per lane: lane l's 16 bytes at
// base + voff land at LDS byte lds + 16 l.  Written as inline assembly so
// the compiler does not serialise later LDS reads of other ring stages
// behind it; completion is waited for explicitly (vmcnt) before the
// barrier that publishes a stage.  M0 is not used for anything else here.
__device__ __forceinline__ void dma16(uint32_t lds, const void *base, uint32_t voff_bytes) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :: "s"(lds), "v"(voff_bytes), "s"(base) : "memory");
}

// Direct HBM -> LDS loads of one page (K and V rows of one KV head).  LDS
// position p = i*256 + tid of a tile holds key p / CH, physical chunk
// p % CH, i.e. logical chunk (p % CH) ^ 2(key & 7).  `off[i]` is this
// thread's byte offset of that chunk within a page; `off0[i]` the same
// chunk of key 0.  Keys at or past `valid` re-read key 0 (always valid when
// a page is loaded): their weight is exactly zero, but a poisoned
// (non-finite) V row there would turn 0 * V into NaN.
template <int D>
__device__ __forceinline__ void pf_load_page(uint16_t *lds_k, uint16_t *lds_v, const uint16_t *page_base,
                                             const uint32_t (&off)[PfCfg<D>::LOADS],
                                             const uint32_t (&off0)[PfCfg<D>::LOADS],
                                             const int (&key)[PfCfg<D>::LOADS], int64_t kv_skv,
                                             int w, int valid) {
    using C = PfCfg<D>;
    const uint16_t *vbase = page_base + kv_skv;
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) {
        const uint32_t o = key[i] < valid ? off[i] : off0[i];
        const int slot = (i * kThreads + w * 64) * 8;   // wave-uniform LDS element offset
        dma16(lds_address(lds_k + slot), page_base, o);
        dma16(lds_address(lds_v + slot), vbase, o);
    }
}

// Page id j of a block-table row, read through the scalar cache (the id is
// uniform across the workgroup).
__device__ __forceinline__ int load_page_id(const int32_t *bt_row, int j) {
    typedef __attribute__((address_space(4))) const int32_t const_i32;
    return *((const_i32 *)bt_row + j);
}

template <int D>
__global__ __launch_bounds__(kThreads, 1) void paged_prefill_kernel(const AttnArgs a) {
    using C = PfCfg<D>;
    // One LDS object per ring stage.
    constexpr int T2 = C::STAGES > 2 ? C::TILE : 8;
    __shared__ __attribute__((aligned(1024))) uint16_t sk0[C::TILE], sv0[C::TILE];
    __shared__ __attribute__((aligned(1024))) uint16_t sk1[C::TILE], sv1[C::TILE];
    __shared__ __attribute__((aligned(1024))) uint16_t sk2[T2], sv2[T2];
    auto kbuf = [&](int st) -> uint16_t * { return st == 0 ? sk0 : (st == 1 ? sk1 : sk2); };
    auto vbuf = [&](int st) -> uint16_t * { return st == 0 ? sv0 : (st == 1 ? sv1 : sv2); };

    const int g = blockIdx.y;
    const int b = blockIdx.z;
    // Later query tiles see more keys under a causal mask: launch them first.
    const int tile = gridDim.x - 1 - blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hi = lane >> 5;   // which half of the wave (0 / 1)

    const int L = a.seq_lens[b];
    const int q0 = a.cu_q[b];
    int n = a.cu_q[b + 1] - q0;
    if (n > a.max_q) n = a.max_q;
    const int G = a.group;
    const int R = n * G;
    const int r0 = tile * C::BM;
    if (r0 >= R) return;

    // This lane's rows: one per 32-row block.
    int vis[C::RB];
    bool row_ok[C::RB];
    int qi_[C::RB], h_[C::RB];
#pragma unroll
    for (int rb = 0; rb < C::RB; ++rb) {
        const int r = r0 + 32 * (C::RB * w + rb) + (lane & 31);
        row_ok[rb] = r < R;
        qi_[rb] = r / G;
        h_[rb] = g * G + (r - qi_[rb] * G);
        vis[rb] = row_ok[rb] ? visible_keys(L, n, qi_[rb], a.causal) : 0;
    }
    const int r_last = min(R, r0 + C::BM) - 1;
    const int kv_end = visible_keys(L, n, r_last / G, a.causal);   // max over the workgroup's rows
    const int ntiles = (kv_end + kPage - 1) / kPage;
    // this wave's own frontier: keys past it are masked for all its rows
    const int wr_last = min(R, r0 + 32 * C::RB * (w + 1)) - 1;
    const int w_end = (r0 + 32 * C::RB * w < R) ? visible_keys(L, n, wr_last / G, a.causal) : 0;
    const int w_full = visible_keys(L, n, min(R - 1, r0 + 32 * C::RB * w) / G, a.causal);

    const uint16_t *head_base = a.kv + (int64_t)g * a.kv_sh;
    const int32_t *bt_row = a.block_table + (int64_t)b * a.bt_stride;

    // This thread's page-relative load offsets (fixed for every page).
    uint32_t ld_off[C::LOADS], ld_off0[C::LOADS];
    int ld_key[C::LOADS];
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) {
        const int p = i * kThreads + tid;
        ld_key[i] = p / C::CH;
        const int c = (p % C::CH) ^ (2 * (ld_key[i] & 7));
        ld_off[i] = (uint32_t)(ld_key[i] * a.kv_ss + c * 8) * 2u;
        ld_off0[i] = (uint32_t)(c * 8) * 2u;
    }
    auto issue_page = [&](int j, int st) {
        const int pid = load_page_id(bt_row, j);
        pf_load_page<D>(kbuf(st), vbuf(st), head_base + (int64_t)pid * a.kv_sp, ld_off, ld_off0, ld_key,
                        a.kv_skv, w, L - j * kPage);
    };

    // Start the first pages streaming before anything else.
#pragma unroll
    for (int s = 0; s < C::STAGES - 1; ++s)
        if (s < ntiles) issue_page(s, s);

    // Q^T as the B operand of v_mfma_f32_32x32x16_bf16: lane holds
    // q[row, 16*ks + 8*hi .. +7]; a negative scale is applied by negating Q
    // (exact in bf16) so the kernel's scale is always positive.
    bf16x8 qreg[C::RB][D / 16];
    const uint32_t qflip = a.q_negate ? 0x80008000u : 0u;
#pragma unroll
    for (int rb = 0; rb < C::RB; ++rb) {
        const uint16_t *qp = a.q + (int64_t)(q0 + qi_[rb]) * a.q_st + (int64_t)h_[rb] * a.q_sh + 8 * hi;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
            u32x4 v = {0u, 0u, 0u, 0u};
            if (row_ok[rb]) v = *reinterpret_cast<const u32x4 *>(qp + 16 * ks);
            v ^= qflip;
            qreg[rb][ks] = __builtin_bit_cast(bf16x8, v);
        }
    }

    f32x16 oacc[C::RB][D / 32];
#pragma unroll
    for (int rb = 0; rb < C::RB; ++rb)
#pragma unroll
        for (int i = 0; i < D / 32; ++i) oacc[rb][i] = f32x16{};
    float m_ref[C::RB], l_part[C::RB];
#pragma unroll
    for (int rb = 0; rb < C::RB; ++rb) {
        m_ref[rb] = -INFINITY;
        l_part[rb] = 0.f;
    }
    const float sl2 = a.scale_log2_pos;   // > 0

    // Per-lane LDS offsets (elements) of the K operand (key = lane & 31 of a
    // 32-key block, chunk 2 ks + hi, swizzled) and of the transposing V reads.
    const int klane = (lane & 31) * D;
    const int kswz = 2 * (lane & 7);
    const int q16 = lane >> 4;
    const int src_row = (lane & 15) >> 2;
    const int vkey = 4 * hi + src_row;          // key within a 16-key step (plus 8 for the 2nd read)
    const int vswz = 2 * (vkey & 7);
    const int vcol_chunk = 2 * (q16 & 1) + ((4 * (lane & 3)) >> 3);
    const int vcol_in = (4 * (lane & 3)) & 7;

    // One softmax step over KSTEP keys starting at key kbase (tile-relative
    // offset koff) of the LDS tile (ks_t, vs_t).
    auto step = [&](const uint16_t *ks_t, const uint16_t *vs_t, int koff, int kbase, bool need_mask) {
        f32x16 sacc[C::RB][C::KB];
#pragma unroll
        for (int rb = 0; rb < C::RB; ++rb)
#pragma unroll
            for (int kb = 0; kb < C::KB; ++kb) sacc[rb][kb] = f32x16{};
#pragma unroll
        for (int kb = 0; kb < C::KB; ++kb) {
            const uint16_t *kp = ks_t + (koff + 32 * kb) * D + klane;
#pragma unroll
            for (int ks = 0; ks < D / 16; ++ks) {
                const int pc = (2 * ks + hi) ^ kswz;
                const bf16x8 kop = *reinterpret_cast<const bf16x8 *>(kp + pc * 8);
#pragma unroll
                for (int rb = 0; rb < C::RB; ++rb)
                    sacc[rb][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qreg[rb][ks], sacc[rb][kb], 0, 0, 0);
            }
        }
        // sacc[rb][kb][i] = raw score of key kbase + 32kb + 8(i/4) + 4hi + i%4.
        bf16x8 pb[C::RB][C::KB][2];
        float alpha[C::RB];
        bool any_upd = false;
#pragma unroll
        for (int rb = 0; rb < C::RB; ++rb) {
            float mx = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < C::KB; ++kb) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    float sc = sacc[rb][kb][i];
                    if (need_mask) {
                        const int key = kbase + 32 * kb + 8 * (i >> 2) + 4 * hi + (i & 3);
                        sc = key < vis[rb] ? sc : -INFINITY;
                        sacc[rb][kb][i] = sc;
                    }
                    mx = fmaxf(mx, sc);
                }
            }
            mx = max_xor32(mx);
            const float mt = mx * sl2;                 // -inf stays -inf (sl2 > 0)
            const bool upd = mt > m_ref[rb] + kRescaleThreshold;
            const float m_new = upd ? mt : m_ref[rb];
            alpha[rb] = upd ? exp2_fast(m_ref[rb] - m_new) : 1.f;
            any_upd |= upd;
            m_ref[rb] = m_new;
            const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
            float psum = 0.f;
#pragma unroll
            for (int kb = 0; kb < C::KB; ++kb) {
#pragma unroll
                for (int i = 0; i < 16; i += 2) {
                    const float p0 = exp2_fast(fmaf(sacc[rb][kb][i], sl2, -m_use));
                    const float p1 = exp2_fast(fmaf(sacc[rb][kb][i + 1], sl2, -m_use));
                    pb[rb][kb][i >> 3][i & 7] = (__bf16)p0;
                    pb[rb][kb][i >> 3][(i & 7) + 1] = (__bf16)p1;
                }
#pragma unroll
                for (int jj = 0; jj < 2; ++jj) {
                    // the row sum uses the same rounded P as the P.V product
                    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
                    const bf16x2 one2 = {(__bf16)1.f, (__bf16)1.f};
#pragma unroll
                    for (int e = 0; e < 8; e += 2) {
                        const bf16x2 pp = {pb[rb][kb][jj][e], pb[rb][kb][jj][e + 1]};
                        psum = __builtin_amdgcn_fdot2_f32_bf16(pp, one2, psum, false);
                    }
                }
            }
            l_part[rb] = l_part[rb] * alpha[rb] + psum;
        }
        if (__any(any_upd)) {
#pragma unroll
            for (int rb = 0; rb < C::RB; ++rb)
#pragma unroll
                for (int i = 0; i < D / 32; ++i) oacc[rb][i] *= alpha[rb];
        }

        // O^T[d, row] += V^T[d, key] P^T[key, row]; k-steps of 16 keys.
        // Half hi of k-step (kb, jj) holds keys 32kb + 16jj + {4hi..4hi+3, 8+4hi..8+4hi+3}.
#pragma unroll
        for (int kb = 0; kb < C::KB; ++kb) {
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
                const uint16_t *v1 = vs_t + (koff + 32 * kb + 16 * jj + vkey) * D + vcol_in;
                const uint16_t *v2 = v1 + 8 * D;
#pragma unroll
                for (int db = 0; db < D / 32; ++db) {
                    const int pc = (4 * db + vcol_chunk) ^ vswz;
                    const bf16x4 lo4 = lds_read_tr16(v1 + pc * 8);
                    const bf16x4 hi4 = lds_read_tr16(v2 + pc * 8);
                    const bf16x8 vop = __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
                    for (int rb = 0; rb < C::RB; ++rb)
                        oacc[rb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pb[rb][kb][jj], oacc[rb][db], 0, 0, 0);
                }
            }
        }
    };

    auto tile_body = [&](int kt, int s) {
        // Wait until this thread's loads of tile kt have landed (loads
        // complete in issue order; the pages issued after it may stay in
        // flight), then make the whole page visible to every wave.
        if (C::STAGES == 3 && kt + 1 < ntiles)
            asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * C::LOADS) : "memory");
        else
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        // Refill the stage freed by tile kt-1 with tile kt + STAGES - 1.
        const int nt = kt + C::STAGES - 1;
        if (nt < ntiles) issue_page(nt, (s + C::STAGES - 1) % C::STAGES);
        const int k0 = kt * kPage;
        if (k0 < w_end) {   // uniform per wave
#pragma unroll
            for (int kk = 0; kk < kPage; kk += C::KSTEP) {
                const bool need_mask = k0 + kk + C::KSTEP > w_full;
                step(kbuf(s), vbuf(s), kk, k0 + kk, need_mask);
            }
        }
    };

    int kt = 0;
    for (; kt + C::STAGES <= ntiles; kt += C::STAGES) {
#pragma unroll
        for (int s = 0; s < C::STAGES; ++s) tile_body(kt + s, s);
    }
#pragma unroll
    for (int s = 0; s < C::STAGES; ++s)
        if (kt + s < ntiles) tile_body(kt + s, s);

    // Epilogue: out = O / l, rounded to bf16.  oacc[rb][db][i] holds
    // d = 32db + 8(i/4) + 4hi + i%4 of this lane's row in block rb.
#pragma unroll
    for (int rb = 0; rb < C::RB; ++rb) {
        const float l_row = sum_xor32(l_part[rb]);
        if (!row_ok[rb]) continue;
        const float inv = l_row > 0.f ? 1.f / l_row : 0.f;
        uint16_t *op = a.out + (int64_t)(q0 + qi_[rb]) * a.o_st + (int64_t)h_[rb] * a.o_sh;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
#pragma unroll
            for (int c4 = 0; c4 < 4; ++c4) {
                u32x2 pk;
                pk[0] = (uint32_t)f32_to_bf16_bits(oacc[rb][db][4 * c4 + 0] * inv) |
                        ((uint32_t)f32_to_bf16_bits(oacc[rb][db][4 * c4 + 1] * inv) << 16);
                pk[1] = (uint32_t)f32_to_bf16_bits(oacc[rb][db][4 * c4 + 2] * inv) |
                        ((uint32_t)f32_to_bf16_bits(oacc[rb][db][4 * c4 + 3] * inv) << 16);
                *reinterpret_cast<u32x2 *>(op + 32 * db + 8 * c4 + 4 * hi) = pk;
            }
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
