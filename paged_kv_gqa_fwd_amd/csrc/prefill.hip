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
//  * One workgroup per (sequence, KV head, tile of packed query rows).  Row
//    r of a (sequence, KV head) is query token r / G, q head g*G + r % G,
//    so the G heads sharing a KV head share every K/V tile.  At D = 128 the
//    workgroup is 8 wave64 (two per SIMD) of 32 rows each: the SIMD
//    interleaves one wave's softmax VALU work and LDS waits with the other
//    wave's MFMAs, which one wave per SIMD cannot do for itself.  Each K or
//    V operand read from LDS then feeds one MFMA (32 FLOP per LDS byte, the
//    LDS rate the full MFMA rate would need); the variant with 4 waves of
//    64 rows (two MFMAs per operand, PA_PF_WAVES128=4) measured about 5%
//    slower.  At D = 256, 4 waves of 32 rows (Q and O of a second block
//    would not fit the registers).
//  * K/V pages (64 keys) stream HBM -> LDS with direct 16-byte loads
//    (global_load_lds_dwordx4), no register staging, through rings of K and
//    V page buffers with one or two pages in flight beyond the next one.
//    Rows are stored with an XOR swizzle of their 16-byte chunks (K: chunk c
//    of key k at c ^ (k&15); V: at c ^ 4(k&3)) so both the b128 K reads and
//    the transposing V reads are bank-conflict free without padding on
//    gfx950's 64-bank LDS (zero SQ_LDS_BANK_CONFLICT; the 32-bank layout
//    this replaced spent half of its LDS cycles in conflicts).
//  * The 32-key steps are software pipelined: the P.V MFMAs of step j-1
//    run while the VALU takes the row max of step j, and the Q.K MFMAs of
//    step j+1 run while the VALU exponentiates step j.  The first LDS
//    operands of each MFMA block are read during the block before it, and
//    the one workgroup barrier per page sits after the Q.K block of the
//    page's first step, so no block opens on an LDS round trip; the first
//    Q.K MFMA of a step goes out before the row-max reduction and rescale
//    that separate the two blocks.  At D = 256
//    (one page of lead) the barrier waits for the next page's K rows only,
//    and no loads go out there: the following page's K rows are issued one
//    load per four MFMAs over the next step and its V rows likewise over the
//    step after (a burst of a page's loads stalls the issuing waves until
//    the CU's vector-memory path has taken them).
//  * S^T = K Q^T on v_mfma_f32_32x32x16_bf16 with keys on M: each lane owns
//    one query row per block, so row max / row sum are in-lane plus one
//    permlane32 swap.  The S^T C layout is directly the B operand of
//    O^T += V^T P^T, whose V^T operand comes from the row-major V tile via
//    the LDS transpose read (ds_read_b64_tr_b16).
//  * Online softmax in log2 units with a lazily moved reference max: the
//    reference only moves (and O, l are rescaled) when a row's max exceeds
//    it by more than 2^8, so P <= 256 and rescales are rare.  The result is
//    the same softmax; only the common factor cancelled at the end differs.
//  * Keys past the causal frontier of the workgroup's last row are never
//    loaded; steps below the frontier of a wave's first row skip the mask.
#include "attn_device.h"
#include "kv_quant.h"
#include "lds_stream.h"

namespace pa {

#ifndef PA_PREFILL_PREFETCH
#define PA_PREFILL_PREFETCH 2
#endif
#ifndef PA_PF_SPREAD   // 0: D = 256 issues a page's K rows at the barrier (the former refill)
#define PA_PF_SPREAD 1
#endif
#ifndef PA_PF_SPREAD128   // 1: D = 128 spreads its tile refills the same way
#define PA_PF_SPREAD128 0
#endif
#ifndef PA_PF_Q_AGPR
#define PA_PF_Q_AGPR 1
#endif
#ifndef PA_PF_XCD_CHUNK   // grid-order launches: runs of 32 items per XCD
#define PA_PF_XCD_CHUNK 1
#endif
#ifndef PA_PF_PRIO   // D = 128 wave priority by phase: 1 = B high, 2 = A high, 0 = none
#define PA_PF_PRIO 1
#endif
#ifndef PA_PF_TILE_PAGES128
#define PA_PF_TILE_PAGES128 2
#endif

template <int D>
struct PfCfg {
    static constexpr int WAVES = D == 128 ? PA_PF_WAVES128 : PA_PF_WAVES256;
    static constexpr int THREADS = 64 * WAVES;
    // 32-row MFMA blocks per wave: two when one wave runs per SIMD (every
    // LDS operand feeds two MFMAs); one when two waves share a SIMD (their
    // registers are halved) and at D = 256, where two blocks' Q and O would
    // not fit the registers of a lane.
    static constexpr int RB = (D == 128 && WAVES == 4) ? 2 : 1;
    static constexpr int BM = WAVES * RB * 32;      // packed query rows per workgroup
    static constexpr int CH = D / 8;                // 16-byte chunks per K or V row
    static constexpr int TILE = kPage * D;          // bf16 elements of one K (or V) page
    static constexpr int LOADS = kPage * CH / THREADS;  // 16-byte loads per thread per K page
    static constexpr int KPL = THREADS / CH;            // keys per load
    static_assert(THREADS % CH == 0, "load layout");
    // The K/V ring's unit: a tile of TP pages (64 TP keys, SPT = 2 TP
    // 32-key steps), published by one workgroup barrier per tile.  At
    // D = 128 two pages per tile halve the barriers per key (and their wave
    // skew) at the LDS of the one-page ring with two pages of lead; at
    // D = 256 a page already fills the LDS.
    static constexpr int TP = D == 128 ? PA_PF_TILE_PAGES128 : 1;
    static constexpr int SPT = 2 * TP;
    // Tiles in flight beyond the next one, and the K / V ring depths that
    // allow it with the step pipeline below (K of tile t+1 and V of tile t
    // are read in the same step).
    static constexpr int LEAD = (D == 128 && TP == 1) ? 2 : 1;
    static constexpr int NK = LEAD + 1;
    static constexpr int NV = LEAD + 2;
    // D = 256 (one page of lead): a page's V rows are first read a page
    // after its K rows, so the refill issues K at the page barrier and
    // spreads V over the next two steps (VPH loads per MFMA phase); the
    // barrier then waits for K only.
    static constexpr bool SPLITV = D == 256;
    static constexpr bool Q_AGPR = PA_PF_Q_AGPR && D == 256;
    static constexpr int VPH = LOADS / 4;
    // SPREAD: no load burst at the barrier.  The tile that the barrier
    // after step SPT t + SPT - 2 frees slots for (tile t+2) has its K rows
    // issued one load per SP MFMAs over the next step (SPT t + SPT - 1) and
    // its V rows the same way over the step after (SPT t + SPT), so the
    // vector-memory path never queues more than one load per wave and the
    // issuing wave's wait hides under its running MFMA.  (At D = 256, K loads
    // packed into the first half of the step, or K and V over three-fifths /
    // two-fifths of the two steps, measured the same.)
    static constexpr bool SPREAD = PA_PF_SPREAD && (SPLITV || PA_PF_SPREAD128);
    static constexpr int SP = (2 * (D / 32) + D / 16) / (TP * LOADS);   // MFMA slots per step / loads per step
};
static_assert(PfCfg<128>::BM == prefill_rows(128) && PfCfg<256>::BM == prefill_rows(256), "row tile");


constexpr float kRescaleThreshold = 8.f;   // log2 units: P stays <= 256

// Direct HBM -> LDS loads of one page (K and V rows of one KV head).  LDS
// position p = i*THREADS + tid of a tile holds key p / CH, physical chunk
// p % CH.  The 16-byte chunks of a row are permuted so that the operand
// reads hit 64 distinct 4-byte banks per LDS cycle (256 bytes): K chunk c
// of key k is stored at c ^ (k & 15) (sixteen keys per b128 read cycle), V
// chunk c at c ^ 4(k & 3) (four keys x four chunks per transposing read
// cycle).
// kof / vof hold this thread's byte offsets within a page; load i carries
// key KPL i + kq (KPL = THREADS / CH).  Every slot of a page is read, also
// those past the sequence's last key: they lie inside the page, their scores
// are masked (a select, so any K there is harmless), and their V rows are
// zeroed in LDS once the page has landed (pf_zero_v_tail), since a
// non-finite V there would turn the zero weight into NaN.
template <int D>
struct PageLoad {
    uint32_t kof[PfCfg<D>::LOADS], vof[PfCfg<D>::LOADS];
    int kq;
};

template <int D>
__device__ __forceinline__ void pf_load_page(uint16_t *lds_k, uint16_t *lds_v, const uint16_t *page_base,
                                             const PageLoad<D> &pl, int64_t kv_skv, int w) {
    using C = PfCfg<D>;
    const uint16_t *vbase = page_base + kv_skv;
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) {
        const int slot = (i * C::THREADS + w * 64) * 8;   // wave-uniform LDS element offset
        dma16(lds_address(lds_k + slot), page_base, pl.kof[i]);
        dma16(lds_address(lds_v + slot), vbase, pl.vof[i]);
    }
}

// Zero this thread's 16-byte chunks of the V rows at or past `valid` in a
// page that has landed in LDS (the chunks its own loads wrote).
template <int D>
__device__ __forceinline__ void pf_zero_v_tail(uint16_t *lds_v, const PageLoad<D> &pl, int tid, int valid) {
    using C = PfCfg<D>;
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i)
        if (C::KPL * i + pl.kq >= valid)
            *reinterpret_cast<u32x4 *>(lds_v + (i * C::THREADS + tid) * 8) = u32x4{0u, 0u, 0u, 0u};
}

template <int D>
__device__ __forceinline__ void pf_load_k(uint16_t *lds_k, const uint16_t *page_base, const PageLoad<D> &pl,
                                          int w) {
    using C = PfCfg<D>;
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) {
        const int slot = (i * C::THREADS + w * 64) * 8;
        dma16(lds_address(lds_k + slot), page_base, pl.kof[i]);
    }
}

// V loads i0 .. i0+N-1 of a page (vbase = the page's V rows).
template <int D, int N>
__device__ __forceinline__ void pf_load_v(uint16_t *lds_v, const uint16_t *vbase, const PageLoad<D> &pl, int w,
                                          int i0) {
    using C = PfCfg<D>;
#pragma unroll
    for (int i = i0; i < i0 + N; ++i) {
        const int slot = (i * C::THREADS + w * 64) * 8;
        dma16(lds_address(lds_v + slot), vbase, pl.vof[i]);
    }
}

// At D = 256 (one wave per SIMD) O is accumulated in accumulation
// registers, which leaves the vector registers room to hold every K read
// address for the whole loop (below).  The library builds its MFMAs in
// vector-register form, so this P.V MFMA is written as asm, and the
// compiler's hazard tracking does not see it: vector code that reads or
// writes O first passes pf_o_fence (its P and V operands are written well
// before, and LDS returns are waited for as for any asm operand).
__device__ __forceinline__ void pf_mfma_pv_agpr(f32x16 &acc, const bf16x8 &a, const bf16x8 &b) {
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
// 20 wait states (an 8-pass MFMA's result may be read by vector
// instructions 11 after it) between the last asm MFMA into O and vector
// reads or writes of O, and between those and the next MFMA.
__device__ __forceinline__ void pf_o_fence(f32x16 (&o)[8]) {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3"
                 : "+a"(o[0]), "+a"(o[1]), "+a"(o[2]), "+a"(o[3]), "+a"(o[4]), "+a"(o[5]), "+a"(o[6]), "+a"(o[7]));
}

template <int D>
__global__ __launch_bounds__(PfCfg<D>::THREADS, 1) void paged_prefill_kernel(const AttnArgs a) {
    using C = PfCfg<D>;
    __shared__ __attribute__((aligned(1024))) uint16_t sk[C::NK][C::TP * C::TILE];
    __shared__ __attribute__((aligned(1024))) uint16_t sv[C::NV][C::TP * C::TILE];

    int g, b, tile, split = 0;
    if (a.pf_order) {
        // Launch order by decreasing work: workgroup i takes the i-th entry
        // of the order table, a (tile, KV head, sequence) index in grid order.
        const int item = a.pf_order[blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z)];
        tile = item % (int)gridDim.x;
        const int hb = item / (int)gridDim.x;
        g = hb % (int)gridDim.y;
        b = hb / (int)gridDim.y;
    } else {
        int x = blockIdx.x, y = blockIdx.y, z = blockIdx.z;
#if PA_PF_XCD_CHUNK
        {
            // Workgroups are dealt to the 8 XCDs in turn by linear id.  In
            // each full run of 256 ids, XCD c takes grid items 32c .. 32c + 31
            // (consecutive tiles, mostly of one head), so an XCD's L2 serves
            // one head's pages at a time.
            const int gx = (int)gridDim.x, gy = (int)gridDim.y;
            const int n = gx * gy * (int)gridDim.z;
            const int lin = x + gx * (y + gy * z);
            if (lin < n - n % 256) {
                const int w8 = lin % 256;
                const int item = lin - w8 + (w8 % 8) * 32 + w8 / 8;
                x = item % gx;
                y = (item / gx) % gy;
                z = item / (gx * gy);
            }
        }
#endif
        g = y;
        b = z;
        // Later query tiles see more keys under a causal mask: launch them
        // first.  Split-key launch: x = split * tiles + (reversed) tile.
        const int tiles = (int)gridDim.x / (a.pf_splits > 1 ? a.pf_splits : 1);
        split = x / tiles;
        tile = tiles - 1 - (x - split * tiles);
    }
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
    // Split-key launch (pf_splits > 1, small grids): this workgroup takes
    // the sequence's pages [ps, pe) of the split-decode layout (pages_per_split
    // pages from row 0's window start) and writes (O, m, l) partials that the
    // combine kernel merges.  A split past the last page writes nothing (the
    // combine never reads it); split 0 always runs, so that a row with no key
    // still gets its zero output.
    int ps = 0, pe = INT_MAX / kPage;
    if (a.pf_splits > 1) {
        const int np = (L + kPage - 1) / kPage;
        ps = split_first_page(L, n, a.window) + split * a.pages_per_split;
        if (split > 0 && ps >= np) return;
        pe = min(np, ps + a.pages_per_split);
    }

    // This lane's rows: one per 32-row block.  Row keys are [lo, vis).
    int vis[C::RB], lo[C::RB];
    bool row_ok[C::RB];
    int qi_[C::RB], h_[C::RB];
#pragma unroll
    for (int rb = 0; rb < C::RB; ++rb) {
        const int r = r0 + 32 * (C::RB * w + rb) + (lane & 31);
        row_ok[rb] = r < R;
        qi_[rb] = r / G;
        h_[rb] = g * G + (r - qi_[rb] * G);
        vis[rb] = row_ok[rb] ? min(visible_keys(L, n, qi_[rb], a.causal), kPage * pe) : 0;
        lo[rb] = row_ok[rb] ? max(window_start(L - n + qi_[rb], a.window), kPage * ps) : 0;
    }
    const int r_last = min(R, r0 + C::BM) - 1;
    // max over the workgroup's rows (and the split's last key)
    const int kv_end = min(visible_keys(L, n, r_last / G, a.causal), kPage * pe);
    // keys below this wave's first row's frontier are visible to all its rows
    const int w_full = min(visible_keys(L, n, min(R - 1, r0 + 32 * C::RB * w) / G, a.causal), kPage * pe);
    // keys at or above the window start of this wave's last row (and the
    // split's first key) are inside every row's window; pages below the
    // workgroup's first row's window start are never loaded (0 and page 0
    // without a window)
    const int w_lo = max(window_start(L - n + min(R - 1, r0 + 32 * C::RB * (w + 1) - 1) / G, a.window), kPage * ps);
    const int t0 = max(window_start(L - n + r0 / G, a.window) / kPage, ps) / C::TP;
    const int j0 = C::SPT * t0;                // first 32-key step
    const int nsteps = (kv_end + 31) / 32;     // 32-key softmax steps
    const int ntiles = (nsteps + C::SPT - 1) / C::SPT;   // ring tiles of TP pages
    const int npages = (kv_end + kPage - 1) / kPage;      // pages with a key some row sees
    // Ring slots count from the first tile, so that with the loop unrolled
    // by NK tiles the K slot of every step is a compile-time constant (its
    // LDS offset folds into the read instructions).
    auto kslot = [&](int t) { return (unsigned)(t - t0) % C::NK; };
    auto vslot = [&](int t) { return (unsigned)(t - t0) % C::NV; };

    const uint16_t *head_base = a.kv + (int64_t)g * a.kv_sh;
    const int32_t *bt_row = a.block_table + (int64_t)b * a.bt_stride;

    // Q^T as the B operand of v_mfma_f32_32x32x16_bf16: lane holds
    // q[row, 16*ks + 8*hi .. +7]; a negative scale is applied by negating Q
    // (exact in bf16) so the kernel's scale is always positive.  Issued
    // before the page loads so that waiting for page 0 also covers Q.
    bf16x8 qreg[C::RB][D / 16];
    {
        const uint32_t qflip = a.q_negate ? 0x80008000u : 0u;
        u32x4 qraw[C::RB][D / 16];
#pragma unroll
        for (int rb = 0; rb < C::RB; ++rb) {
            const int qrow = row_ok[rb] ? qi_[rb] : 0;   // rows past the end read token 0
            const uint16_t *qp = a.q + (int64_t)(q0 + qrow) * a.q_st + (int64_t)h_[rb] * a.q_sh + 8 * hi;
#pragma unroll
            for (int ks = 0; ks < D / 16; ++ks) qraw[rb][ks] = *reinterpret_cast<const u32x4 *>(qp + 16 * ks);
        }
#pragma unroll
        for (int rb = 0; rb < C::RB; ++rb) {
            const uint32_t keep = row_ok[rb] ? 0xFFFFFFFFu : 0u;
#pragma unroll
            for (int ks = 0; ks < D / 16; ++ks)
                qreg[rb][ks] = __builtin_bit_cast(bf16x8, (qraw[rb][ks] ^ qflip) & keep);
        }
        // Q is only ever an MFMA operand, which may sit in accumulation
        // registers: at D = 256 (one wave per SIMD, vector registers full)
        // placing it there leaves the vector registers to the softmax.
        // (At D = 128 two waves share a SIMD's registers and it spilled.)
        if constexpr (C::Q_AGPR) {
#pragma unroll
            for (int rb = 0; rb < C::RB; ++rb)
#pragma unroll
                for (int ks = 0; ks < D / 16; ++ks) asm volatile("" : "+a"(qreg[rb][ks]));
        }
    }

    // This thread's page-relative load offsets (fixed for every page).
    PageLoad<D> pl;
    pl.kq = tid / C::CH;
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) {
        const int p = i * C::THREADS + tid;
        const int key = p / C::CH;   // = KPL i + kq
        const int ck = (p % C::CH) ^ (key & 15);
        const int cv = (p % C::CH) ^ (4 * (key & 3));
        pl.kof[i] = (uint32_t)(key * a.kv_ss + ck * 8) * 2u;
        pl.vof[i] = (uint32_t)(key * a.kv_ss + cv * 8) * 2u;
    }
    // V rows past the last key of tile t (its last page, or a page of the
    // last tile that no row reaches) zeroed once the tile has landed
    auto zero_tile_tail = [&](int t) {
#pragma unroll
        for (int pp = 0; pp < C::TP; ++pp) {
            const int page = C::TP * t + pp;
            const int valid = page < npages ? L - page * kPage : 0;
            if (valid < kPage) pf_zero_v_tail<D>(sv[vslot(t)] + pp * C::TILE, pl, tid, valid);
        }
    };
    auto issue_page = [&](int t) {   // tile t: pages TP t .. TP t + TP - 1
        if constexpr (C::SPLITV) {   // all of K, then all of V
            const int pid = load_page_id(bt_row, t);
            pf_load_k<D>(sk[kslot(t)], head_base + (int64_t)pid * a.kv_sp, pl, w);
            pf_load_v<D, C::LOADS>(sv[vslot(t)], head_base + (int64_t)pid * a.kv_sp + a.kv_skv, pl, w, 0);
        } else {
#pragma unroll
            for (int pp = 0; pp < C::TP; ++pp) {
                // A page of the last tile past the workgroup's last visible
                // key is not named by the table: it re-reads the tile's first
                // page (its V rows are then zeroed), so every tile issues the
                // same loads.
                const int page = C::TP * t + pp;
                const int pid = load_page_id(bt_row, page < npages ? page : C::TP * t);
                pf_load_page<D>(sk[kslot(t)] + pp * C::TILE, sv[vslot(t)] + pp * C::TILE,
                                head_base + (int64_t)pid * a.kv_sp, pl, a.kv_skv, w);
            }
        }
    };
    // SPLITV: the page whose V rows are being issued over the two steps
    // after its K rows (part q of 4 during phase q of those steps).
    const uint16_t *vp_base = head_base;
    uint16_t *vp_slot = sv[0];
    bool vp_on = false;
    auto issue_v_part = [&](int q) {
        if (C::SPLITV && !C::SPREAD && vp_on) pf_load_v<D, C::VPH>(vp_slot, vp_base, pl, w, q * C::VPH);
    };
    // SPREAD: the tile being refilled (page bases) and its ring slots.  Its
    // loads always issue (a branch around each would split the step's basic
    // blocks, and the compiler then moves the exponentials away from the
    // MFMAs they overlap): with no tile to load they re-read an existing page
    // into free ring slots, and a vmcnt(0) before the epilogue drains them.
    const uint16_t *rp_base[C::TP];
    uint16_t *kp_slot = sk[0];
    // tile tn's pages (tile tv, which exists, lends a page id if tn does not)
    auto set_refill = [&](int tn, int tv) {
        kp_slot = sk[kslot(tn)];
        vp_slot = sv[vslot(tn)];
#pragma unroll
        for (int pp = 0; pp < C::TP; ++pp) {
            const int page = C::TP * tn + pp;
            const bool real = tn < ntiles && page < npages;
            const int pid = load_page_id(bt_row, real ? page : C::TP * (tn < ntiles ? tn : tv));
            rp_base[pp] = head_base + (int64_t)pid * a.kv_sp;
        }
    };
    // MFMA slot s of step j: K load s / SP of the refill tile in steps
    // SPT t + SPT - 1, V load s / SP in steps SPT t.
    auto spread_load = [&](int j, int s) {
        if constexpr (C::SPREAD) {
            const bool kstep = (unsigned)j % C::SPT == C::SPT - 1;
            const bool vstep = (unsigned)j % C::SPT == 0;
            if (s % C::SP == 0 && (kstep || vstep)) {
                const int q = s / C::SP;
                const int pp = q / C::LOADS, i = q % C::LOADS;
                const int slot = pp * C::TILE + (i * C::THREADS + w * 64) * 8;
                if (kstep)
                    dma16(lds_address(kp_slot + slot), rp_base[pp], pl.kof[i]);
                else
                    dma16(lds_address(vp_slot + slot), rp_base[pp] + a.kv_skv, pl.vof[i]);
            }
        }
    };
    // Wait until page t has landed in LDS: pages t+1 .. `issued` were
    // issued after it and may stay in flight (loads complete in issue order).
    int issued = -1;
    auto wait_page = [&](int t) {   // tile t; TP pages of K and V rows per tile
        const int younger = issued - t;
        if (C::LEAD == 2 && younger == 2)
            asm volatile("s_waitcnt vmcnt(%0)" ::"n"(4 * C::TP * C::LOADS) : "memory");
        else if (younger >= 1)
            asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * C::TP * C::LOADS) : "memory");
        else
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    };

#pragma unroll
    for (int tt = 0; tt <= C::LEAD; ++tt)
        if (t0 + tt < ntiles) {
            issue_page(t0 + tt);
            issued = t0 + tt;
        }

    f32x16 oacc[C::RB][D / 32];
#pragma unroll
    for (int rb = 0; rb < C::RB; ++rb)
#pragma unroll
        for (int i = 0; i < D / 32; ++i) oacc[rb][i] = f32x16{};
    if constexpr (D == 256) {
#pragma unroll
        for (int rb = 0; rb < C::RB; ++rb) pf_o_fence(oacc[rb]);
    }
    const float sl2 = a.scale_log2_pos;   // > 0
    const float inv_sl2 = 1.f / sl2;
    // m_ref: the row's reference max (log2 units), m_use the value P is taken
    // against (0 while no key of the row has been seen), thr the raw score
    // above which the reference moves: (m_ref + threshold) / sl2.
    float m_ref[C::RB], m_use[C::RB], thr[C::RB], l_part[C::RB];
#pragma unroll
    for (int rb = 0; rb < C::RB; ++rb) {
        m_ref[rb] = -INFINITY;
        m_use[rb] = 0.f;
        thr[rb] = -INFINITY;
        l_part[rb] = 0.f;
    }

    // Per-lane LDS element offsets.  K operand of a 32-key step: key
    // lane & 31, logical chunk 2 ks + hi, physical chunk (2 ks + hi) ^ (lane & 15).
    // V operand (transposing reads): key vkey (+8), columns of chunk
    // 4 db + vcol_chunk, physical chunk ^ 4(vkey & 3).
    const int klane = (lane & 31) * D;
    const int kswz = lane & 15;
    const int q16 = lane >> 4;
    const int vkey = 4 * hi + ((lane & 15) >> 2);
    const int vlane = vkey * D + ((4 * (lane & 3)) & 7);
    const int vswz = 4 * (vkey & 3);
    const int vcol_chunk = 2 * (q16 & 1) + ((4 * (lane & 3)) >> 3);

    constexpr int NKS = D / 16;            // Q.K MFMA k-steps per 32-key step
    constexpr int NPV = 2 * (D / 32);      // P.V (16-key half, 32-column block) pairs
    constexpr int NEL = C::RB * 16;        // scores per lane per step
    constexpr int EB = NEL / NKS;          // scores exponentiated per Q.K k-step
    constexpr int EA = NEL / NPV;          // scores max-reduced per P.V pair
    static_assert(EB * NKS == NEL && EA * NPV == NEL, "even split");
    static_assert(EB % C::RB == 0 && EA % C::RB == 0, "even split per MFMA");
    constexpr int PF = PA_PREFILL_PREFETCH;   // LDS operand reads in flight ahead of their MFMA

    auto vread = [&](const uint16_t *vt, int k) {
        const int jj = k / (D / 32), db = k % (D / 32);
        // the swizzle only moves chunks within each group of 16 (bits 2-3 of
        // the chunk index), so column blocks db and db + 4 share a lane's
        // address up to a constant 16 chunks: one address per block pair
        const uint16_t *v1 = vt + (16 * jj) * D + ((4 * (db & 3) + vcol_chunk) ^ vswz) * 8 + (db >> 2) * 128;
        const bf16x4 lo4 = lds_read_tr16(v1);
        const bf16x4 hi4 = lds_read_tr16(v1 + 8 * D);
        return __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
    };
    // The LDS byte address of every K chunk this lane reads, in ring slot 0
    // at the first step of a tile, held in registers for the whole loop (an
    // empty asm hides their origin, so the compiler cannot re-derive them
    // inside it); a read adds its slot and step as the instruction's offset.
    // cp: the step's position in the loop unrolled by NK tiles (j0 is a
    // multiple of SPT), a compile-time constant.  (At D = 128, where the
    // compiler kept no such registers, a change elsewhere in the kernel once
    // moved it to re-adding addresses in the loop: DiT -2.4%.)
    constexpr uint32_t SLOT_B = C::TP * C::TILE * 2;
    uint32_t kaddr[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
        kaddr[ks] = lds_address(sk[0]) + 2u * (klane + ((2 * ks + hi) ^ kswz) * 8);
        asm volatile("" : "+v"(kaddr[ks]));
    }
    auto kread_at = [&](int cp, int ks) -> bf16x8 {
        const uint32_t imm = (uint32_t)((cp / C::SPT) % C::NK) * SLOT_B + 64u * (uint32_t)(cp % C::SPT) * D;
        return *reinterpret_cast<const __attribute__((address_space(3))) bf16x8 *>((uintptr_t)(kaddr[ks] + imm));
    };
    auto vstage = [&](int j) {
        return sv[((unsigned)(j - j0) / C::SPT) % C::NV] + (32 * ((unsigned)j % C::SPT)) * D + vlane;
    };

    // S^T = K Q^T for the 32 keys of step j (raw scores, f32); no overlap
    // (pipeline prologue).  s[rb][i] = score of key 32j + 8(i/4) + 4hi + i%4
    // for this lane's row of block rb.
    auto qk = [&](int cp, f32x16 (&s)[C::RB]) {
#pragma unroll
        for (int rb = 0; rb < C::RB; ++rb) s[rb] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            const bf16x8 kop = kread_at(cp, ks);
#pragma unroll
            for (int rb = 0; rb < C::RB; ++rb)
                s[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qreg[rb][ks], s[rb], 0, 0, 0);
        }
    };
    // O^T[d, row] += V^T[d, key] P^T[key, row] over the 32 keys of step j;
    // no overlap (pipeline epilogue).  Half hi of k-step jj holds keys
    // 32j + 16jj + {4hi..4hi+3, 8+4hi..8+4hi+3}.
    auto pv = [&](int j, const bf16x8 (&p)[C::RB][2]) {
        const uint16_t *vt = vstage(j);
#pragma unroll
        for (int k = 0; k < NPV; ++k) {
            const bf16x8 vop = vread(vt, k);
#pragma unroll
            for (int rb = 0; rb < C::RB; ++rb)
                if constexpr (D == 256)
                    pf_mfma_pv_agpr(oacc[rb][k % (D / 32)], vop, p[rb][k / (D / 32)]);
                else
                    oacc[rb][k % (D / 32)] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        vop, p[rb][k / (D / 32)], oacc[rb][k % (D / 32)], 0, 0, 0);
        }
    };

    // The first PF operands of a section are read during the section before
    // it, so that neither MFMA block starts on an LDS round trip.
    bf16x8 vcar[PF], kcar[PF];
    bf16x8 pb[C::RB][2];
#pragma unroll
    for (int rb = 0; rb < C::RB; ++rb) pb[rb][0] = pb[rb][1] = bf16x8{};
    // One pipelined step: scur holds S_j on entry; snext receives S_{j+1}.
    auto step = [&](int j, int cp, f32x16 (&scur)[C::RB], f32x16 (&snext)[C::RB]) {
        // ---- mask (diagonal, tail and window-edge steps only)
        if (32 * j + 32 > w_full || 32 * j < w_lo) {
#pragma unroll
            for (int rb = 0; rb < C::RB; ++rb)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int key = 32 * j + 8 * (i >> 2) + 4 * hi + (i & 3);
                    scur[rb][i] = (key < vis[rb] && key >= lo[rb]) ? scur[rb][i] : -INFINITY;
                }
        }
        // ---- A(j): P_{j-1} V_{j-1} on the MFMA pipe, two V operands
        // ahead, with the row max of S_j on the VALU.  At the first step P
        // is zero and the first page's V (landed) is read.
        // (At D = 128 the two waves of a SIMD run this phase and B at
        // different priorities, B raised: DiT +0.3%, A raised +0.2%.)
        if constexpr (D == 128 && PA_PF_PRIO == 1) __builtin_amdgcn_s_setprio(0);
        if constexpr (D == 128 && PA_PF_PRIO == 2) __builtin_amdgcn_s_setprio(1);
        float mx[C::RB];
#pragma unroll
        for (int rb = 0; rb < C::RB; ++rb) mx[rb] = -INFINITY;
        {
            const uint16_t *vt = vstage(j > j0 ? j - 1 : j0);
            bf16x8 vop[PF + 1];
#pragma unroll
            // (at D = 256 the V page A(2t+1) reads is published by the
            // barrier just before it: no look-ahead into it)
            for (int k = 0; k < PF; ++k) vop[k] = (C::SPLITV && (j & 1)) ? vread(vt, k) : vcar[k];
#pragma unroll
            for (int k = 0; k < NPV; ++k) {
                if (k == NPV / 2) issue_v_part(2 * (1 - (j & 1)));   // A(2t+1): part 0, A(2t+2): part 2
                if (k + PF < NPV)
                    vop[(k + PF) % (PF + 1)] = vread(vt, k + PF);
                else
                    kcar[k + PF - NPV] = kread_at(cp + 1, k + PF - NPV);   // B(j)'s first operands
                // one MFMA, then its share of the VALU work
#pragma unroll
                for (int rb = 0; rb < C::RB; ++rb) {
                    if constexpr (D == 256)
                        pf_mfma_pv_agpr(oacc[rb][k % (D / 32)], vop[k % (PF + 1)], pb[rb][k / (D / 32)]);
                    else
                        oacc[rb][k % (D / 32)] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                            vop[k % (PF + 1)], pb[rb][k / (D / 32)], oacc[rb][k % (D / 32)], 0, 0, 0);
                    spread_load(j, k);
                    constexpr int EH = EA / C::RB;
#pragma unroll
                    for (int e = (k * C::RB + rb) * EH; e < (k * C::RB + rb + 1) * EH; ++e)
                        mx[e / 16] = fmaxf(mx[e / 16], scur[e / 16][e % 16]);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }
        // B(j)'s first Q.K MFMA (its operand was read during A(j)) goes to the
        // matrix unit now, overlapping the row-max reduction and rescale below.
#pragma unroll
        for (int rb = 0; rb < C::RB; ++rb)
            snext[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kcar[0], qreg[rb][0], f32x16{}, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        // ---- reference max and rescale.  Each lane first compares its
        // half-row max with the raw threshold; only when some lane of the
        // wave passes it (rare: a row's max rose by more than 2^8) are the
        // half-rows combined, the references moved and O, l rescaled.
        bool past = false;
#pragma unroll
        for (int rb = 0; rb < C::RB; ++rb) past |= mx[rb] > thr[rb];
        if (__any(past)) {
#pragma unroll
            for (int rb = 0; rb < C::RB; ++rb) {
                const float mt = max_xor32(mx[rb]) * sl2;   // -inf stays -inf (sl2 > 0)
                const bool upd = mt > m_ref[rb] + kRescaleThreshold;
                const float m_new = upd ? mt : m_ref[rb];
                const float alpha = upd ? exp2_fast(m_ref[rb] - m_new) : 1.f;
                m_ref[rb] = m_new;
                m_use[rb] = (m_new == -INFINITY) ? 0.f : m_new;
                thr[rb] = (m_new + kRescaleThreshold) * inv_sl2;
                l_part[rb] *= alpha;
                if constexpr (D == 256) pf_o_fence(oacc[rb]);
#pragma unroll
                for (int i = 0; i < D / 32; ++i) oacc[rb][i] *= alpha;
                if constexpr (D == 256) pf_o_fence(oacc[rb]);
            }
        }
        // ---- B(j): S_{j+1} = K_{j+1} Q^T on the MFMA pipe, two K operands
        // ahead, with P_j = exp2(S_j scale - m) on the VALU.  After the last
        // step the product reads a stale stage (in bounds) and is discarded.
        if constexpr (D == 128 && PA_PF_PRIO == 1) __builtin_amdgcn_s_setprio(1);
        if constexpr (D == 128 && PA_PF_PRIO == 2) __builtin_amdgcn_s_setprio(0);
        {
            bf16x8 kop[PF + 1];
#pragma unroll
            for (int k = 0; k < PF; ++k) kop[k] = kcar[k];
            float pf[NEL];
            float psum[C::RB];
#pragma unroll
            for (int rb = 0; rb < C::RB; ++rb) psum[rb] = 0.f;
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                if (ks == NKS / 2) issue_v_part(2 * (1 - (j & 1)) + 1);   // B(2t+1): part 1, B(2t+2): part 3
                if (ks + PF < NKS)
                    kop[(ks + PF) % (PF + 1)] = kread_at(cp + 1, ks + PF);
                else if (!C::SPLITV || (j & 1))
                    vcar[ks + PF - NKS] = vread(vstage(j), ks + PF - NKS);   // A(j+1)'s first operands
                // one MFMA, then its share of the VALU work
#pragma unroll
                for (int rb = 0; rb < C::RB; ++rb) {
                    if (ks > 0)
                        snext[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[ks % (PF + 1)], qreg[rb][ks], snext[rb], 0, 0, 0);
                    spread_load(j, NPV + ks);
                    constexpr int EH = EB / C::RB;
#pragma unroll
                    for (int e = (ks * C::RB + rb) * EH; e < (ks * C::RB + rb + 1) * EH; ++e) {
                        const int rr = e / 16, i = e % 16;
                        pf[e] = exp2_fast(fmaf(scur[rr][i], sl2, -m_use[rr]));
                        if (i & 1) {
                            // round the pair to bf16; the row sum uses the same
                            // rounded P as the P.V product
                            typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
                            const bf16x2 pp = {(__bf16)pf[e - 1], (__bf16)pf[e]};
                            pb[rr][i >> 3][(i & 7) - 1] = pp[0];
                            pb[rr][i >> 3][i & 7] = pp[1];
                            const bf16x2 one2 = {(__bf16)1.f, (__bf16)1.f};
                            psum[rr] = __builtin_amdgcn_fdot2_f32_bf16(pp, one2, psum[rr], false);
                        }
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
#pragma unroll
            for (int rb = 0; rb < C::RB; ++rb) {
                l_part[rb] += psum[rb];
                // An empty use of the weights here keeps their VALU work in
                // this block, interleaved with the Q.K MFMAs above: otherwise
                // the compiler may sink it below the loop's branch, after the
                // MFMAs, where nothing overlaps it.
                asm volatile("" ::"v"(pb[rb][0]), "v"(pb[rb][1]), "v"(l_part[rb]));
            }
        }
        // ---- page boundary after B(2t): publish page t+1 (first read by
        // A(2t+1)'s look-ahead into B(2t+1)'s K operands), then refill the
        // slots of K page t (last read by B(2t)) and V page t-1 (last read
        // by A(2t)) with page t+1+LEAD.
        const int t = j >> 1;
        if constexpr (C::SPLITV) {
            // K page t+1 has landed (only V page t+1, issued after it, may
            // be in flight; its first reader is A(2t+3), after the next
            // barrier); the refill of page t+2 issues its K rows over step
            // 2t+1 and its V rows over step 2t+2 (SPREAD; else K now and V
            // over the next two steps).  After the last page's first step
            // every load is waited for (its V rows are read next).
            if (!(j & 1)) {
                if (t + 1 < ntiles)
                    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(C::LOADS) : "memory");
                else
                    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                // V page t (issued before K page t+1) has landed; it is first
                // read by A(2t+1)
                if (t == ntiles - 1) zero_tile_tail(t);
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                __builtin_amdgcn_s_barrier();
                vp_on = t + 2 < ntiles;
                if constexpr (C::SPREAD) {
                    set_refill(t + 2, t);   // the slots page t+2 takes are free whether or not it exists
                } else if (vp_on) {
                    const int pid = load_page_id(bt_row, t + 2);
                    const uint16_t *pb2 = head_base + (int64_t)pid * a.kv_sp;
                    pf_load_k<D>(sk[kslot(t + 2)], pb2, pl, w);
                    vp_base = pb2 + a.kv_skv;
                    vp_slot = sv[vslot(t + 2)];
                }
            }
        } else if ((unsigned)j % C::SPT == C::SPT - 2 && (int)((unsigned)j / C::SPT) + 1 < ntiles) {
            // tile version of the same boundary: after B(SPT t + SPT - 2)
            // publish tile t+1, refill K tile t / V tile t-1's slots
            const int t = (unsigned)j / C::SPT;
            if constexpr (C::SPREAD) {
                // tile t+1's loads were the last issued (steps SPT t - 1, SPT t)
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                if (t + 1 == ntiles - 1) zero_tile_tail(t + 1);
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                __builtin_amdgcn_s_barrier();
                set_refill(t + 1 + C::LEAD, t);
            } else {
                wait_page(t + 1);
                if (t + 1 == ntiles - 1) zero_tile_tail(t + 1);
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                __builtin_amdgcn_s_barrier();
                if (t + 1 + C::LEAD < ntiles) {
                    issue_page(t + 1 + C::LEAD);
                    issued = t + 1 + C::LEAD;
                }
            }
        }
    };

    f32x16 sA[C::RB], sB[C::RB];
    if (j0 < nsteps) {
        wait_page(t0);
        // A(j0) reads tile t0's V (with zero weights) before any other barrier
        if (t0 == ntiles - 1) zero_tile_tail(t0);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        qk(0, sA);
        if constexpr (C::SPREAD) {
            // step j0 issues V loads before the first refill is set up: into
            // the free V slot tile t0+2 will take, from tile t0's first page;
            // K loads of a step before the first barrier (a single tile, no
            // barrier) go to the free slot of tile t0+1
            kp_slot = sk[kslot(t0 + 1)];
            vp_slot = sv[vslot(t0 + 2)];
#pragma unroll
            for (int pp = 0; pp < C::TP; ++pp)
                rp_base[pp] = head_base + (int64_t)load_page_id(bt_row, C::TP * t0) * a.kv_sp;
        }
#pragma unroll
        for (int k = 0; k < PF; ++k) vcar[k] = vread(vstage(j0), k);
        // SPT steps per tile, NK tiles per iteration; the S registers
        // alternate roles between steps.
        for (int u = 0; t0 + C::NK * u < ntiles; ++u) {
#pragma unroll
            for (int c = 0; c < C::NK * C::SPT; c += 2) {
                const int j = j0 + C::NK * C::SPT * u + c;
                if (c == 0 || j < nsteps) step(j, c, sA, sB);
                if (j + 1 < nsteps) step(j + 1, c + 1, sB, sA);
            }
        }
        pv(nsteps - 1, pb);
        if constexpr (C::SPREAD) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // no LDS load outlives the workgroup
    }

    // Epilogue: out = O / l, rounded to bf16.  oacc[rb][db][i] holds
    // d = 32db + 8(i/4) + 4hi + i%4 of this lane's row in block rb.
    if constexpr (D == 256) {
#pragma unroll
        for (int rb = 0; rb < C::RB; ++rb) pf_o_fence(oacc[rb]);
    }
    if (a.pf_splits > 1) {
        // split partials: O (f32, v_scale applied) and l against the
        // reference m (log2 units; -inf for a row that saw no key), the
        // split-decode kernels' layout; the sink joins in the combine
#pragma unroll
        for (int rb = 0; rb < C::RB; ++rb) {
            const float l_row = sum_xor32(l_part[rb]);
            if (!row_ok[rb]) continue;
            const int64_t prow = (((int64_t)b * a.max_q + qi_[rb]) * a.hq + h_[rb]) * a.max_splits + split;
            float *po = a.part_o + prow * D;
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
#pragma unroll
                for (int c4 = 0; c4 < 4; ++c4)
                    *reinterpret_cast<f32x4 *>(po + 32 * db + 8 * c4 + 4 * hi) =
                        f32x4{oacc[rb][db][4 * c4 + 0] * a.v_scale, oacc[rb][db][4 * c4 + 1] * a.v_scale,
                              oacc[rb][db][4 * c4 + 2] * a.v_scale, oacc[rb][db][4 * c4 + 3] * a.v_scale};
            if (hi == 0) {
                a.part_ml[prow * 2] = m_ref[rb];
                a.part_ml[prow * 2 + 1] = l_row;
            }
        }
        return;
    }
#pragma unroll
    for (int rb = 0; rb < C::RB; ++rb) {
        float l_row = sum_xor32(l_part[rb]);
        if (!row_ok[rb]) continue;
        if (a.sinks && l_row > 0.f) {
            // the row's sink logit joins the normaliser (no value row)
            const float sink2 = a.sinks[h_[rb]] * kLog2e;
            if (sink2 != -INFINITY) l_row += exp2_fast(sink2 - m_ref[rb]);
        }
        // v_scale: V = v_scale * e4m3(code) over an fp8 cache (1 for bf16)
        const float inv = l_row > 0.f ? a.v_scale / l_row : 0.f;
        uint16_t *op = a.out + (int64_t)(q0 + qi_[rb]) * a.o_st + (int64_t)h_[rb] * a.o_sh;
        // Lanes l and l + 32 hold the low and high four values of each
        // group of eight d.  One permlane32 swap per pair of groups gives
        // lane l both halves of the even group and lane l + 32 both halves
        // of the odd one, so every lane stores 16 contiguous bytes (half as
        // many stores, 32-byte runs per row).
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
            uint32_t w[4][2];
#pragma unroll
            for (int c4 = 0; c4 < 4; ++c4) {
                w[c4][0] = (uint32_t)f32_to_bf16_bits(oacc[rb][db][4 * c4 + 0] * inv) |
                           ((uint32_t)f32_to_bf16_bits(oacc[rb][db][4 * c4 + 1] * inv) << 16);
                w[c4][1] = (uint32_t)f32_to_bf16_bits(oacc[rb][db][4 * c4 + 2] * inv) |
                           ((uint32_t)f32_to_bf16_bits(oacc[rb][db][4 * c4 + 3] * inv) << 16);
            }
#pragma unroll
            for (int cp = 0; cp < 2; ++cp) {
                // upper lanes of the first operand <-> lower lanes of the second
                const auto s0 = __builtin_amdgcn_permlane32_swap(w[2 * cp][0], w[2 * cp + 1][0], false, false);
                const auto s1 = __builtin_amdgcn_permlane32_swap(w[2 * cp][1], w[2 * cp + 1][1], false, false);
                *reinterpret_cast<u32x4 *>(op + 32 * db + 16 * cp + 8 * hi) =
                    u32x4{(uint32_t)s0[0], (uint32_t)s1[0], (uint32_t)s0[1], (uint32_t)s1[1]};
            }
        }
    }
}

// ---- prefill over an fp8 cache: stage the pages as bf16 ---------------------
// Workgroup (j, b) decodes page j of sequence b, all KV heads, K and V, from
// e4m3 codes into bf16 (exactly: every e4m3 value is a bf16 value; the
// scales stay out, k_scale in the score scale and v_scale in the output) at
// staging page b * MP + j, and writes that index into the staging table.
// Pages the prefill kernel cannot read are not staged and keep -1: those of
// sequences with no query, those past the sequence's keys, and those below
// the window start of the sequence's first query (rounded down to a
// two-page ring tile).  The kernel then reads the staging pool exactly as
// a bf16 pool.
template <int D>
__global__ __launch_bounds__(kThreads) void fp8_stage_pages_kernel(const AttnArgs a) {
    const int j = blockIdx.x;
    const int b = blockIdx.y;
    const int L = a.seq_lens[b];
    const int q0 = a.cu_q[b];
    int n = a.cu_q[b + 1] - q0;
    if (n > a.max_q) n = a.max_q;
    const int npages = (L + kPage - 1) / kPage;
    const int p_lo = split_first_page(L, n, a.window) & ~1;
    const bool staged = n > 0 && j >= p_lo && j < npages;
    const int64_t si = (int64_t)b * a.mp + j;
    if (threadIdx.x == 0) a.stage_bt[si] = staged ? (int32_t)si : -1;
    if (!staged) return;
    const int pid = a.block_table[(int64_t)b * a.bt_stride + j];
    const uint8_t *src = reinterpret_cast<const uint8_t *>(a.kv) + (int64_t)pid * a.kv_sp;   // byte strides
    constexpr int dc = D / 16;                           // 16-code chunks per row
    const int per_slot = a.hkv * 2 * dc;
    const int total = kPage * per_slot;
    // chunk c = (slot, KV head, K/V, 16 codes) in the staging page's own
    // order, so its 16 bf16 land at element 16 c.  U loads in flight per
    // thread before the first conversion (each code is read once): one
    // round for a page of 4 KV heads at D = 256 (a kernel of 106 us on the
    // chunked prefill with one load at a time, 83 with 8, 74 with 32)
    uint16_t *dst = a.stage_kv + si * ((int64_t)kPage * a.hkv * 2 * D);
    constexpr int U = 32;
    for (int c0 = threadIdx.x; c0 < total; c0 += U * kThreads) {
        u32x4 w[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = c0 + u * kThreads;
            if (c < total) {
                const int slot = c / per_slot;
                const int r = c - slot * per_slot;
                const int h = r / (2 * dc);
                const int kv = (r / dc) & 1;
                const int ch = r % dc;
                w[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(
                    src + (int64_t)slot * a.kv_ss + (int64_t)h * a.kv_sh + kv * a.kv_skv + 16 * ch));
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = c0 + u * kThreads;
            if (c < total) {
                uint32_t o[8];
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) e4m3x4_to_bf16x4(w[u][q4], o[2 * q4], o[2 * q4 + 1]);
                uint16_t *op = dst + 16 * (int64_t)c;
                *reinterpret_cast<u32x4 *>(op) = u32x4{o[0], o[1], o[2], o[3]};
                *reinterpret_cast<u32x4 *>(op + 8) = u32x4{o[4], o[5], o[6], o[7]};
            }
        }
    }
}

hipError_t launch_fp8_stage_any(int D, const AttnArgs &a, hipStream_t stream) {
    if (D == 128)
        hipLaunchKernelGGL(fp8_stage_pages_kernel<128>, dim3(a.mp, a.n_seqs), dim3(kThreads), 0, stream, a);
    else
        hipLaunchKernelGGL(fp8_stage_pages_kernel<256>, dim3(a.mp, a.n_seqs), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

// ---- prefill launch order ----------------------------------------------------
// One workgroup sorts the prefill grid's (tile, KV head, sequence) items by
// the pages each streams, most first, and writes the permutation to
// a.pf_order: a counting sort on the page count (plus one for the start-up,
// clamped to kOrderBuckets - 1; items with no rows count 0).  Under a causal
// mask the last tiles of the longest sequences stream the most pages;
// launched first, they leave the short items to fill the tail of the grid
// (longest-processing-time-first list scheduling).  Every KV head of a
// (tile, sequence) pair has the same work, so pairs are sorted and their
// heads take adjacent places: the hardware deals workgroups to the eight
// XCDs in turn, so when Hkv divides 8 each XCD then works on fixed KV heads
// and its L2 holds only their pages (in grid order every XCD sees every
// head).  Pairs with equal counts land in any order: each item writes only
// its own output rows, so the order changes no bit of the result.
constexpr int kOrderThreads = 1024;
constexpr int kOrderBuckets = 2048;
constexpr int kOrderRegs = 8;       // pairs per thread whose bucket stays in registers

template <int D>
__device__ __forceinline__ int prefill_pair_bucket(const AttnArgs &a, int tile, int b) {
    using C = PfCfg<D>;
    const int L = a.seq_lens[b];
    const int q0 = a.cu_q[b];
    const int n = min(a.cu_q[b + 1] - q0, a.max_q);
    const int R = n * a.group;
    const int r0 = tile * C::BM;
    int work = 0;
    if (r0 < R) {
        // the pages the kernel streams for this tile: from its first ring
        // tile (window start of its first row) to the last visible key
        const int r_last = min(R, r0 + C::BM) - 1;
        const int kv_end = visible_keys(L, n, r_last / a.group, a.causal);
        const int first = window_start(L - n + r0 / a.group, a.window) / (kPage * C::TP) * C::TP;
        work = 1 + max(0, (int)(((int64_t)kv_end + kPage - 1) / kPage) - first);
    }
    return kOrderBuckets - 1 - min(work, kOrderBuckets - 1);
}

template <int D>
__global__ __launch_bounds__(kOrderThreads) void prefill_order_kernel(const AttnArgs a, int tiles) {
    constexpr int PER = kOrderBuckets / kOrderThreads;
    static_assert(kOrderBuckets % kOrderThreads == 0, "buckets per thread");
    __shared__ int hist[kOrderBuckets];
    __shared__ int wsum[kOrderThreads / 64];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = tid >> 6;
    const int hkv = a.hkv;
    const int pairs = tiles * a.n_seqs;
    auto bucket = [&](int p) { return prefill_pair_bucket<D>(a, p % tiles, p / tiles); };
    // hkv places per pair, the pair's heads side by side
    auto place = [&](int p, int pos) {
        const int tile = p % tiles;
        const int base = tile + tiles * hkv * (p / tiles);
        for (int g = 0; g < hkv; ++g) a.pf_order[pos + g] = base + tiles * g;
    };
    for (int i = tid; i < kOrderBuckets; i += kOrderThreads) hist[i] = 0;
    __syncthreads();
    int bk[kOrderRegs];
#pragma unroll
    for (int k = 0; k < kOrderRegs; ++k) {
        const int p = tid + k * kOrderThreads;
        bk[k] = p < pairs ? bucket(p) : -1;
        if (bk[k] >= 0) atomicAdd(&hist[bk[k]], hkv);
    }
    for (int p = tid + kOrderRegs * kOrderThreads; p < pairs; p += kOrderThreads) atomicAdd(&hist[bucket(p)], hkv);
    __syncthreads();
    // exclusive scan of the counts (bucket 0 = most pages): thread t owns
    // buckets [PER t, PER t + PER)
    int cnt[PER], own = 0;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        cnt[k] = hist[PER * tid + k];
        own += cnt[k];
    }
    int incl = own;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(incl, o, 64);
        if (lane >= o) incl += y;
    }
    if (lane == 63) wsum[wv] = incl;
    __syncthreads();
    int base = incl - own;
    for (int w = 0; w < wv; ++w) base += wsum[w];
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        hist[PER * tid + k] = base;   // each thread rewrites only the buckets it read
        base += cnt[k];
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kOrderRegs; ++k)
        if (bk[k] >= 0) place(tid + k * kOrderThreads, atomicAdd(&hist[bk[k]], hkv));
    for (int p = tid + kOrderRegs * kOrderThreads; p < pairs; p += kOrderThreads)
        place(p, atomicAdd(&hist[bucket(p)], hkv));
}

hipError_t launch_prefill_order_any(int D, const AttnArgs &a, dim3 grid, hipStream_t stream) {
    if (D == 128)
        hipLaunchKernelGGL(prefill_order_kernel<128>, dim3(1), dim3(kOrderThreads), 0, stream, a, (int)grid.x);
    else
        hipLaunchKernelGGL(prefill_order_kernel<256>, dim3(1), dim3(kOrderThreads), 0, stream, a, (int)grid.x);
    return hipGetLastError();
}

template <int D>
hipError_t launch_prefill(const AttnArgs &a, dim3 grid, hipStream_t stream) {
    static_assert(PfCfg<D>::THREADS == prefill_threads(D), "workgroup size");
    hipLaunchKernelGGL(paged_prefill_kernel<D>, grid, dim3(PfCfg<D>::THREADS), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_prefill_any(int D, const AttnArgs &a, dim3 grid, hipStream_t stream) {
    return D == 128 ? launch_prefill<128>(a, grid, stream) : launch_prefill<256>(a, grid, stream);
}

}  // namespace pa
