// Host side of libpaged_attn: argument validation, execution planning and
// kernel launches behind the C ABI declared in include/paged_attn.h.
//
// Validation and planning are pure host logic and touch no HIP API, so they
// run (and are tested) on machines without a GPU.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cfloat>
#include <cmath>
#include <cstdint>
#include <mutex>
#include <vector>

#include "attn_device.h"
#include "paged_attn.h"
#include "quant_device.h"
#include "kv_write.h"

namespace pa {
hipError_t launch_decode_split_any(int D, const AttnArgs &a, dim3 grid, hipStream_t stream);
hipError_t launch_decode_balanced_any(int D, const AttnArgs &a, dim3 grid, hipStream_t stream);
hipError_t launch_combine_any(int D, const CombineArgs &a, hipStream_t stream);
hipError_t launch_workspace_clear(uint32_t *p, size_t words, hipStream_t stream);
hipError_t launch_prefill_any(int D, const AttnArgs &a, dim3 grid, hipStream_t stream);
hipError_t launch_fp8_stage_any(int D, const AttnArgs &a, hipStream_t stream);
hipError_t launch_prefill_order_any(int D, const AttnArgs &a, dim3 grid, hipStream_t stream);
hipError_t launch_quant_prep(const QuantArgs &a, hipStream_t stream);
hipError_t launch_quant_attn(const QuantArgs &a, hipStream_t stream);
hipError_t launch_kv_write(const KvWriteArgs &a, hipStream_t stream);
}  // namespace pa

namespace {

constexpr int kVersion = 10000;          // 1.0.0
// G * max_q packed rows the split-decode kernels take (up to four 16-wide
// MFMA row blocks: the short-sequence body); more rows take the prefill kernel.
constexpr int kMaxDecodeRows = pa::kDecodeRowBlock * pa::kMaxDecodeRowBlocks;
constexpr int kGridYZMax = 65535;
constexpr size_t kWsAlign = 256;
// Split sizing for the decode path: aim for about this many rounds of
// resident workgroups (256 CUs x resident workgroups per CU), which balances
// the per-workgroup start-up cost against the tail of ragged sequences.
constexpr int64_t kComputeUnits = 256;
constexpr int64_t kSplitRounds = 4;
// Balanced split path: one round of resident workgroups (every workgroup
// streams the same number of pages, so there is no tail to fill), and a
// bound on the partial workspace that sets the least range size.
constexpr int64_t kBalRounds = 1;
constexpr size_t kBalPartialBudget = size_t(64) << 20;

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }
size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

int validate_dims(const attn_paged_dims *d, int32_t n_seqs, int32_t max_q) {
    if (!d) return ATTN_ERR_NULL;
    if (d->head_dim != 128 && d->head_dim != 256) return ATTN_ERR_UNSUPPORTED;
    if (d->page_size != pa::kPage) return ATTN_ERR_UNSUPPORTED;
    if (d->num_q_heads <= 0 || d->num_kv_heads <= 0) return ATTN_ERR_SHAPE;
    if (d->num_q_heads % d->num_kv_heads != 0) return ATTN_ERR_SHAPE;
    if (d->num_kv_heads > kGridYZMax) return ATTN_ERR_SHAPE;
    if (d->num_pages <= 0 || d->max_pages_per_seq <= 0) return ATTN_ERR_SHAPE;
    if (d->num_tokens < 0) return ATTN_ERR_SHAPE;
    if (n_seqs < 0 || n_seqs > kGridYZMax) return ATTN_ERR_SHAPE;
    if (n_seqs > 0 && (max_q <= 0 || (int64_t)max_q > d->num_tokens)) return ATTN_ERR_SHAPE;
    const int64_t D = d->head_dim, hq = d->num_q_heads;
    // Element strides: positive, multiples of 8 (16-byte aligned rows), rows disjoint.
    const int64_t strides[] = {d->q_stride_token, d->q_stride_head, d->o_stride_token,
                               d->o_stride_head, d->kv_stride_page, d->kv_stride_slot,
                               d->kv_stride_head, d->kv_stride_kv};
    for (int64_t s : strides)
        if (s <= 0 || (s & 7) != 0) return ATTN_ERR_STRIDE;
    if (d->q_stride_head < D || d->q_stride_token < hq * d->q_stride_head) return ATTN_ERR_STRIDE;
    if (d->o_stride_head < D || d->o_stride_token < hq * d->o_stride_head) return ATTN_ERR_STRIDE;
    if (d->kv_stride_kv < D) return ATTN_ERR_STRIDE;
    if (d->bt_stride < d->max_pages_per_seq) return ATTN_ERR_STRIDE;
    return ATTN_OK;
}

// A window that reaches past every key a table can hold changes nothing.
int32_t effective_window(const attn_paged_dims *d, int32_t window) {
    return (int64_t)window >= (int64_t)d->max_pages_per_seq * pa::kPage ? 0 : window;
}

// The balanced split path plans a batch in one workgroup's LDS (at most
// kBalMaxSeqs sequences) and counts its pages in int32.
bool balanced_fits(const attn_paged_dims *d, int32_t n_seqs, int64_t mq, int32_t window) {
    int64_t MP = d->max_pages_per_seq;
    if (window > 0) MP = std::min<int64_t>(MP, (window + mq + 62) / pa::kPage + 1);
    return n_seqs >= 0 && n_seqs <= pa::kBalMaxSeqs && (int64_t)n_seqs * MP <= INT32_MAX;
}

size_t bal_lead_bytes(int32_t n_seqs) { return align_up((size_t)std::max<int32_t>(n_seqs, 1) * 4, kWsAlign); }

// Prefill workspace: [fp8 staging pool | staging table] over an fp8 cache,
// then the launch-order table (one i32 per workgroup) when the grid holds
// several sequences and enough workgroups for their order to matter (fewer:
// the sort's launch costs more than a ragged tail); only if it fits ws_cap.
constexpr int64_t kPfOrderMinItems = 512;
constexpr int64_t kPfOrderMaxItems = int64_t(1) << 22;
// Split-key prefill: a grid of at most half as many items as CUs has its
// keys split into floor(kPfSplitTarget / items) runs, one round of
// workgroups (measured on MI355X: a 128-item grid over 8k-16k keys 18-32%
// faster with two splits, slower with three or four; a 16-item one 2.7x
// faster over 8k keys).
constexpr int64_t kPfSplitMaxItems = 128;
constexpr int64_t kPfSplitTarget = 256;
struct PrefillWs {
    size_t stage_pool = 0, stage_table = 0, order = 0, part_o = 0, part_ml = 0;
    size_t total() const { return stage_pool + stage_table + order + part_o + part_ml; }
};
// splits > 1: the split partials [rows * splits * D f32 | rows * splits * 2 f32]
// (rows = n_seqs * max_q * Hq) take the order table's place.
PrefillWs prefill_ws(const attn_paged_dims *d, int32_t n_seqs, int64_t mq, int64_t ss, bool f8, int64_t items,
                     int64_t splits, size_t ws_cap) {
    PrefillWs w;
    if (f8) {
        const size_t pages = (size_t)std::max<int32_t>(n_seqs, 1) * (size_t)d->max_pages_per_seq;
        w.stage_pool = align_up(pages * (size_t)pa::kPage * (size_t)ss * 2, kWsAlign);
        w.stage_table = align_up(pages * 4, kWsAlign);
    }
    if (splits > 1) {
        const size_t rows = (size_t)std::max<int32_t>(n_seqs, 1) * (size_t)mq * (size_t)d->num_q_heads * (size_t)splits;
        w.part_o = align_up(rows * (size_t)d->head_dim * 4, kWsAlign);
        w.part_ml = align_up(rows * 8, kWsAlign);
    } else if (n_seqs >= 2 && items >= kPfOrderMinItems && items <= kPfOrderMaxItems) {
        const size_t ob = align_up((size_t)items * 4, kWsAlign);
        if (w.total() + ob <= ws_cap) w.order = ob;
    }
    return w;
}

int make_plan(const attn_paged_dims *d, int32_t n_seqs, int32_t max_q, int32_t path_hint,
              int32_t pps, int32_t window, attn_paged_plan *plan, int32_t kv_dtype = ATTN_KV_BF16,
              size_t bal_budget = kBalPartialBudget, size_t ws_cap = SIZE_MAX) {
    int rc = validate_dims(d, n_seqs, max_q);
    if (rc != ATTN_OK) return rc;
    if (kv_dtype != ATTN_KV_BF16 && kv_dtype != ATTN_KV_FP8_E4M3) return ATTN_ERR_UNSUPPORTED;
    if (kv_dtype == ATTN_KV_FP8_E4M3) {
        // 16-byte aligned rows of D one-byte codes
        const int64_t kvs[] = {d->kv_stride_page, d->kv_stride_slot, d->kv_stride_head, d->kv_stride_kv};
        for (int64_t st : kvs)
            if ((st & 15) != 0) return ATTN_ERR_STRIDE;
    }
    if (!plan) return ATTN_ERR_NULL;
    if (path_hint < ATTN_PATH_AUTO || path_hint > ATTN_PATH_SPLIT_BALANCED) return ATTN_ERR_SHAPE;
    if (pps < 0 || window < 0) return ATTN_ERR_SHAPE;
    window = effective_window(d, window);
    const int G = d->num_q_heads / d->num_kv_heads;
    const int64_t mq = std::max<int32_t>(max_q, 1);
    int path = path_hint;
    if (path == ATTN_PATH_AUTO)
        // The two-kernel split form measured faster than the single-launch
        // merge on MI355X (the merge form makes every workgroup wait for its
        // write-through partial stores and the ticket atomic before it ends).
        // Among split forms, the balanced one (cuts placed by length) keeps a
        // ragged batch's workgroups equally busy; a forced split size asks
        // for the fixed-size form.
        path = (mq * G > kMaxDecodeRows) ? ATTN_PATH_PREFILL
               : (pps == 0 && balanced_fits(d, n_seqs, mq, window)) ? ATTN_PATH_SPLIT_BALANCED
                                                                    : ATTN_PATH_SPLIT_DECODE;
    const bool balanced = path == ATTN_PATH_SPLIT_BALANCED;
    const bool split_path = path == ATTN_PATH_SPLIT_DECODE || path == ATTN_PATH_SPLIT_FUSED || balanced;
    if (split_path && mq * G > kMaxDecodeRows) return ATTN_ERR_UNSUPPORTED;
    if (balanced && !balanced_fits(d, n_seqs, mq, window)) return ATTN_ERR_UNSUPPORTED;
    *plan = attn_paged_plan{};
    plan->path = path;
    plan->block_threads = pa::kThreads;
    // Pages the split path may have to read per sequence: all of them, or
    // with a window those from row 0's window start to the last key.
    int64_t MP = d->max_pages_per_seq;
    if (split_path && window > 0) MP = std::min<int64_t>(MP, (window + mq + 62) / pa::kPage + 1);
    if (balanced) {
        // Ranges: one per (resident workgroup slot / KV head).  The least
        // range size C_min bounds the pieces of one sequence by
        // floor((MP - 1) / C_min) + 2, which sizes the partial workspace.
        const int64_t waves = pa::decode_waves(d->head_dim, kv_dtype == ATTN_KV_FP8_E4M3,
                                               pa::decode_row_blocks(mq * G));
        const int64_t slots = kBalRounds * kComputeUnits * waves;
        const int64_t R = std::min<int64_t>(std::max<int64_t>((slots + d->num_kv_heads - 1) / d->num_kv_heads, 1),
                                            kGridYZMax);
        const size_t rows = (size_t)std::max<int32_t>(n_seqs, 1) * (size_t)mq * (size_t)d->num_q_heads;
        const size_t per_split = rows * ((size_t)d->head_dim + 2) * 4;
        const int64_t s_cap = std::max<int64_t>(1, std::min<int64_t>((int64_t)(bal_budget / per_split), R));
        int64_t c_min = (MP + s_cap - 1) / s_cap;
        c_min = std::max<int64_t>(c_min, pps);
        const int64_t S = (MP - 1) / c_min + 2;
        plan->pages_per_split = (int32_t)c_min;
        plan->max_splits = (int32_t)S;
        plan->grid_x = d->num_kv_heads;
        plan->grid_y = (int32_t)R;
        plan->grid_z = 1;
        // [pieces per sequence (i32) | partial O | partial (m, l)]
        plan->workspace_bytes = bal_lead_bytes(n_seqs) + align_up(rows * (size_t)S * (size_t)d->head_dim * 4, kWsAlign) +
                                align_up(rows * (size_t)S * 8, kWsAlign);
    } else if (split_path) {
        int64_t p = pps;
        if (p == 0) {
            // one workgroup per SIMD-wave slot: 4 waves = one per SIMD
            const int64_t target = kSplitRounds * kComputeUnits *
                                   pa::decode_waves(d->head_dim, kv_dtype == ATTN_KV_FP8_E4M3,
                                                    pa::decode_row_blocks(mq * G));
            const int64_t bound = MP * std::max<int64_t>(n_seqs, 1) * d->num_kv_heads;
            p = (bound + target - 1) / target;
        }
        // at most 65535 splits (grid z limit)
        p = std::max<int64_t>(p, (MP + kGridYZMax - 1) / kGridYZMax);
        p = std::min<int64_t>(std::max<int64_t>(p, 1), MP);
        const int64_t S = (MP + p - 1) / p;
        plan->pages_per_split = (int32_t)p;
        plan->max_splits = (int32_t)S;
        plan->grid_x = d->num_kv_heads;
        plan->grid_y = n_seqs;
        plan->grid_z = (int32_t)S;
        if (S > 1) {
            const size_t rows = (size_t)std::max<int32_t>(n_seqs, 1) * (size_t)mq * (size_t)d->num_q_heads * (size_t)S;
            if (path == ATTN_PATH_SPLIT_FUSED)
                plan->counter_bytes = align_up((size_t)std::max<int32_t>(n_seqs, 1) * (size_t)d->num_kv_heads * 4, kWsAlign);
            plan->workspace_bytes = plan->counter_bytes + align_up(rows * (size_t)d->head_dim * 4, kWsAlign) +
                                    align_up(rows * 8, kWsAlign);
        }
    } else {
        // The prefill kernel addresses a page's K/V rows with 32-bit byte
        // offsets from the page's base (one VGPR per direct-to-LDS load):
        // 63 slot strides plus one row must stay below 4 GiB.  Over an fp8
        // cache it reads the bf16 staging pool ([P, Hkv, 2, D] pages).
        const bool f8 = kv_dtype == ATTN_KV_FP8_E4M3;
        const int64_t ss = f8 ? (int64_t)d->num_kv_heads * 2 * d->head_dim : d->kv_stride_slot;
        if ((63 * ss + d->head_dim) * 2 > (int64_t)UINT32_MAX) return ATTN_ERR_UNSUPPORTED;
        const int64_t bm = pa::prefill_rows(d->head_dim);
        const int64_t tiles = (mq * G + bm - 1) / bm;
        if (tiles > INT32_MAX) return ATTN_ERR_SHAPE;
        const int64_t items = tiles * d->num_kv_heads * n_seqs;
        // Split-key prefill: forced by pages_per_split on the prefill path,
        // else for grids too small to fill the GPU.  Splits follow the
        // split-decode layout: runs of pps pages from row 0's window start,
        // at most the pages a row can see (the window's reach, else MP).
        int64_t MPw = MP;
        if (window > 0) MPw = std::min<int64_t>(MP, (window + mq + 62) / pa::kPage + 1);
        int64_t pp = MPw, S = 1;
        if (path_hint == ATTN_PATH_PREFILL && pps > 0) {
            pp = std::min<int64_t>(pps, MPw);
        } else if (items > 0 && items <= kPfSplitMaxItems && MPw >= 2) {
            const int64_t tp = d->head_dim == 128 ? 2 : 1;   // pages per ring tile
            const int64_t want = std::min<int64_t>(kPfSplitTarget / items, MPw);
            pp = ((MPw + want - 1) / want + tp - 1) / tp * tp;
        }
        S = (MPw + pp - 1) / pp;
        if (S > 1 && tiles * S > INT32_MAX) return ATTN_ERR_SHAPE;
        PrefillWs w = prefill_ws(d, n_seqs, mq, ss, f8, items, S, ws_cap);
        if (S > 1 && w.total() > ws_cap) {
            S = 1;   // the partials do not fit the caller's bound: one pass
            pp = MPw;
            w = prefill_ws(d, n_seqs, mq, ss, f8, items, S, ws_cap);
        }
        plan->block_threads = pa::prefill_threads(d->head_dim);
        plan->pages_per_split = (int32_t)(S > 1 ? pp : MP);
        plan->max_splits = (int32_t)S;
        plan->grid_x = (int32_t)(tiles * S);
        plan->grid_y = d->num_kv_heads;
        plan->grid_z = n_seqs;
        // [staging pool: n_seqs * MP pages of P * Hkv * 2 * D bf16 | staging
        // table: n_seqs * MP i32] over an fp8 cache, then the launch order or
        // the split partials
        plan->workspace_bytes = w.total();
    }
    return ATTN_OK;
}

// ---- kernel timing instrumentation ---------------------------------------
enum TimedKind { kTimedMain = 0, kTimedCombine = 1, kTimedPrep = 2, kTimedWrite = 3 };
struct TimedLaunch {
    hipEvent_t start, stop;
    int kind;
};
std::mutex g_timing_mu;
bool g_timing_on = false;
std::vector<TimedLaunch> g_timed;

int record_event(hipEvent_t *ev, hipStream_t stream) {
    if (hipEventCreate(ev) != hipSuccess) return ATTN_ERR_HIP;
    if (hipEventRecord(*ev, stream) != hipSuccess) return ATTN_ERR_HIP;
    return ATTN_OK;
}

bool timing_enabled() {
    std::lock_guard<std::mutex> lk(g_timing_mu);
    return g_timing_on;
}

void timing_push(const TimedLaunch &t) {
    std::lock_guard<std::mutex> lk(g_timing_mu);
    g_timed.push_back(t);
}

// Validate an attention call and build its kernel arguments (no launch).
int paged_prepare(void *out, const void *q, const void *kv_pool, const int32_t *block_table,
                  const int32_t *seq_lens, const int32_t *cu_q, int32_t n_seqs, int32_t max_q,
                  float scale, int32_t causal, const attn_paged_dims *dims, void *workspace,
                  size_t workspace_bytes, int32_t path_hint, int32_t pps, const float *sinks,
                  int32_t window, attn_paged_plan &plan, pa::AttnArgs &a, int32_t kv_dtype = ATTN_KV_BF16,
                  float k_scale = 1.f, float v_scale = 1.f, size_t bal_budget = kBalPartialBudget,
                  size_t ws_cap = SIZE_MAX) {
    int rc = make_plan(dims, n_seqs, max_q, path_hint, pps, window, &plan, kv_dtype, bal_budget, ws_cap);
    if (rc != ATTN_OK) return rc;
    if (!std::isfinite(scale)) return ATTN_ERR_SHAPE;
    if (kv_dtype == ATTN_KV_BF16) k_scale = v_scale = 1.f;   // the scales belong to an fp8 cache only
    if (!std::isfinite(k_scale) || !std::isfinite(v_scale)) return ATTN_ERR_SHAPE;
    if (n_seqs == 0) return ATTN_OK;
    if (!out || !q || !kv_pool || !block_table || !seq_lens || !cu_q) return ATTN_ERR_NULL;
    if (!aligned16(out) || !aligned16(q) || !aligned16(kv_pool)) return ATTN_ERR_ALIGN;
    if (!aligned4(block_table) || !aligned4(seq_lens) || !aligned4(cu_q)) return ATTN_ERR_ALIGN;
    if (sinks && !aligned4(sinks)) return ATTN_ERR_ALIGN;
    if (plan.workspace_bytes > 0) {
        if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & (kWsAlign - 1)) != 0)
            return ATTN_ERR_WORKSPACE;
        if (workspace_bytes < plan.workspace_bytes) return ATTN_ERR_WORKSPACE;
    }

    const int D = dims->head_dim;
    const int G = dims->num_q_heads / dims->num_kv_heads;
    a = pa::AttnArgs{};
    a.out = static_cast<uint16_t *>(out);
    a.q = static_cast<const uint16_t *>(q);
    a.kv = static_cast<const uint16_t *>(kv_pool);
    a.block_table = block_table;
    a.seq_lens = seq_lens;
    a.cu_q = cu_q;
    a.q_st = dims->q_stride_token;
    a.q_sh = dims->q_stride_head;
    a.o_st = dims->o_stride_token;
    a.o_sh = dims->o_stride_head;
    a.kv_sp = dims->kv_stride_page;
    a.kv_ss = dims->kv_stride_slot;
    a.kv_sh = dims->kv_stride_head;
    a.kv_skv = dims->kv_stride_kv;
    a.bt_stride = dims->bt_stride;
    a.n_seqs = n_seqs;
    a.max_q = max_q;
    a.hq = dims->num_q_heads;
    a.hkv = dims->num_kv_heads;
    a.group = G;
    a.pages_per_split = plan.pages_per_split;
    a.max_splits = plan.max_splits;
    a.causal = causal ? 1 : 0;
    a.scale_log2 = (float)((double)scale * 1.4426950408889634 * (double)k_scale);
    a.kv_fp8 = kv_dtype == ATTN_KV_FP8_E4M3 ? 1 : 0;
    a.v_scale = v_scale;
    // The prefill kernel takes the maximum of raw scores and applies the
    // scale afterwards, which needs a positive scale: a negative one is
    // applied by negating Q (exact), and zero as the smallest normal float
    // (every weight is then exactly 1 unless |q.k| exceeds about 1e30).  An
    // fp8 cache's k_scale joins the score scale (1 for bf16).
    const double eff_scale = (double)scale * (double)k_scale;
    a.scale_log2_pos = std::max((float)(std::fabs(eff_scale) * 1.4426950408889634), FLT_MIN);
    a.q_negate = eff_scale < 0.0 ? 1 : 0;
    a.sinks = sinks;
    a.window = effective_window(dims, window);
    a.row_blocks = pa::decode_row_blocks((int64_t)std::max<int32_t>(max_q, 1) * G);
    a.mp = dims->max_pages_per_seq;
    if (plan.path == ATTN_PATH_PREFILL) {
        // [staging pool | staging table] over an fp8 cache, then the launch order
        const int64_t ss = (int64_t)dims->num_kv_heads * 2 * D;
        const int64_t S = plan.max_splits;
        const PrefillWs w = prefill_ws(dims, n_seqs, std::max<int32_t>(max_q, 1), ss, a.kv_fp8 != 0,
                                       (int64_t)plan.grid_x / S * plan.grid_y * plan.grid_z, S, ws_cap);
        char *ws = static_cast<char *>(workspace);
        if (w.stage_pool > 0) {
            a.stage_kv = reinterpret_cast<uint16_t *>(ws);
            a.stage_bt = reinterpret_cast<int32_t *>(ws + w.stage_pool);
        }
        if (w.order > 0) a.pf_order = reinterpret_cast<int32_t *>(ws + w.stage_pool + w.stage_table);
        a.pf_splits = (int32_t)S;
        if (S > 1) {
            a.part_o = reinterpret_cast<float *>(ws + w.stage_pool + w.stage_table);
            a.part_ml = reinterpret_cast<float *>(ws + w.stage_pool + w.stage_table + w.part_o);
        }
    } else if (plan.workspace_bytes > 0) {
        // [merge counters or pieces per sequence | partial O | partial (m, l)],
        // each 256-byte aligned
        const size_t rows = (size_t)n_seqs * (size_t)max_q * (size_t)dims->num_q_heads * (size_t)plan.max_splits;
        char *ws = static_cast<char *>(workspace);
        size_t lead = plan.counter_bytes;
        if (plan.path == ATTN_PATH_SPLIT_BALANCED) {
            a.seg_splits = reinterpret_cast<int32_t *>(ws);
            lead = bal_lead_bytes(n_seqs);
        } else {
            a.counters = reinterpret_cast<int32_t *>(ws);
        }
        a.part_o = reinterpret_cast<float *>(ws + lead);
        a.part_ml = reinterpret_cast<float *>(ws + lead + align_up(rows * (size_t)D * 4, kWsAlign));
        a.fuse_merge = plan.path == ATTN_PATH_SPLIT_FUSED ? 1 : 0;
    }
    return ATTN_OK;
}

// Launch a prepared attention call (split kernel + combine, or prefill).
int paged_launch(const attn_paged_plan &plan, const pa::AttnArgs &a, int D, hipStream_t st) {
    const dim3 grid(plan.grid_x, plan.grid_y, plan.grid_z);
    const bool timing = timing_enabled();
    TimedLaunch t_main{}, t_comb{};
    hipError_t e;
    if (plan.path == ATTN_PATH_PREFILL && a.pf_order) {
        // Sort the grid's items by work (timed as preparation).
        TimedLaunch t_ord{};
        if (timing && record_event(&t_ord.start, st) != ATTN_OK) return ATTN_ERR_HIP;
        if (pa::launch_prefill_order_any(D, a, grid, st) != hipSuccess) return ATTN_ERR_HIP;
        if (timing) {
            if (record_event(&t_ord.stop, st) != ATTN_OK) return ATTN_ERR_HIP;
            t_ord.kind = kTimedPrep;
            timing_push(t_ord);
        }
    }
    if (plan.path == ATTN_PATH_PREFILL && a.stage_kv) {
        // Over an fp8 cache: decode the pages the prefill reads into the bf16
        // staging pool (timed as preparation), then prefill from it.
        TimedLaunch t_stage{};
        if (timing && record_event(&t_stage.start, st) != ATTN_OK) return ATTN_ERR_HIP;
        if (pa::launch_fp8_stage_any(D, a, st) != hipSuccess) return ATTN_ERR_HIP;
        if (timing) {
            if (record_event(&t_stage.stop, st) != ATTN_OK) return ATTN_ERR_HIP;
            t_stage.kind = kTimedPrep;
            timing_push(t_stage);
        }
        pa::AttnArgs b = a;
        b.kv = a.stage_kv;
        b.kv_ss = (int64_t)a.hkv * 2 * D;
        b.kv_sp = (int64_t)pa::kPage * b.kv_ss;
        b.kv_sh = 2 * D;
        b.kv_skv = D;
        b.block_table = a.stage_bt;
        b.bt_stride = a.mp;
        b.kv_fp8 = 0;
        if (timing && record_event(&t_main.start, st) != ATTN_OK) return ATTN_ERR_HIP;
        e = pa::launch_prefill_any(D, b, grid, st);
    } else {
        if (timing && record_event(&t_main.start, st) != ATTN_OK) return ATTN_ERR_HIP;
        e = plan.path == ATTN_PATH_PREFILL            ? pa::launch_prefill_any(D, a, grid, st)
            : plan.path == ATTN_PATH_SPLIT_BALANCED ? pa::launch_decode_balanced_any(D, a, grid, st)
                                                    : pa::launch_decode_split_any(D, a, grid, st);
    }
    if (e != hipSuccess) return ATTN_ERR_HIP;
    if (timing && record_event(&t_main.stop, st) != ATTN_OK) return ATTN_ERR_HIP;
    const bool need_combine = ((plan.path == ATTN_PATH_SPLIT_DECODE || plan.path == ATTN_PATH_PREFILL) &&
                               plan.max_splits > 1) ||
                              plan.path == ATTN_PATH_SPLIT_BALANCED;
    if (need_combine) {
        pa::CombineArgs c{};
        c.out = a.out;
        c.part_o = a.part_o;
        c.part_ml = a.part_ml;
        c.seq_lens = a.seq_lens;
        c.cu_q = a.cu_q;
        c.o_st = a.o_st;
        c.o_sh = a.o_sh;
        c.n_seqs = a.n_seqs;
        c.max_q = a.max_q;
        c.hq = a.hq;
        c.pages_per_split = plan.pages_per_split;
        c.max_splits = plan.max_splits;
        c.sinks = a.sinks;
        c.window = a.window;
        c.seg_splits = a.seg_splits;
        if (timing && record_event(&t_comb.start, st) != ATTN_OK) return ATTN_ERR_HIP;
        e = pa::launch_combine_any(D, c, st);
        if (e != hipSuccess) return ATTN_ERR_HIP;
        if (timing && record_event(&t_comb.stop, st) != ATTN_OK) return ATTN_ERR_HIP;
    }
    if (timing) {
        t_main.kind = kTimedMain;
        timing_push(t_main);
        if (need_combine) {
            t_comb.kind = kTimedCombine;
            timing_push(t_comb);
        }
    }
    return ATTN_OK;
}

// ---- quantised path -------------------------------------------------------
int paged_fwd_impl(void *out, const void *q, const void *kv_pool, const int32_t *block_table,
                   const int32_t *seq_lens, const int32_t *cu_q, int32_t n_seqs, int32_t max_q,
                   float scale, int32_t causal, const attn_paged_dims *dims, void *workspace,
                   size_t workspace_bytes, void *stream, int32_t path_hint, int32_t pps,
                   const float *sinks = nullptr, int32_t window = 0, int32_t kv_dtype = ATTN_KV_BF16,
                   float k_scale = 1.f, float v_scale = 1.f) {
    attn_paged_plan plan;
    pa::AttnArgs a;
    int rc = paged_prepare(out, q, kv_pool, block_table, seq_lens, cu_q, n_seqs, max_q, scale, causal,
                           dims, workspace, workspace_bytes, path_hint, pps, sinks, window, plan, a, kv_dtype,
                           k_scale, v_scale);
    if (rc != ATTN_OK || n_seqs == 0) return rc;
    return paged_launch(plan, a, dims->head_dim, static_cast<hipStream_t>(stream));
}

// Validate a KV-cache write and build its kernel arguments (no launch).
int kv_write_prepare(void *kv_pool, const void *k_new, const void *v_new, const int32_t *block_table,
                     const int32_t *seq_lens, const int32_t *cu_q, int32_t n_seqs, int32_t max_q,
                     const attn_paged_dims *dims, const attn_kv_new_dims *nd, pa::KvWriteArgs &w,
                     int32_t kv_dtype = ATTN_KV_BF16, float k_scale = 1.f, float v_scale = 1.f) {
    int rc = validate_dims(dims, n_seqs, max_q);
    if (rc != ATTN_OK) return rc;
    if (!nd) return ATTN_ERR_NULL;
    if (kv_dtype != ATTN_KV_BF16 && kv_dtype != ATTN_KV_FP8_E4M3) return ATTN_ERR_UNSUPPORTED;
    if (kv_dtype == ATTN_KV_FP8_E4M3) {
        const int64_t kvs[] = {dims->kv_stride_page, dims->kv_stride_slot, dims->kv_stride_head, dims->kv_stride_kv};
        for (int64_t st : kvs)
            if ((st & 15) != 0) return ATTN_ERR_STRIDE;
        // finite, nonzero scales (the codes are x * (1 / scale))
        if (!std::isfinite(k_scale) || !std::isfinite(v_scale) || k_scale == 0.f || v_scale == 0.f)
            return ATTN_ERR_SHAPE;
    }
    const int64_t D = dims->head_dim, hkv = dims->num_kv_heads;
    const int64_t strides[] = {nd->k_stride_token, nd->k_stride_head, nd->v_stride_token, nd->v_stride_head};
    for (int64_t st : strides)
        if (st <= 0 || (st & 7) != 0) return ATTN_ERR_STRIDE;
    if (nd->k_stride_head < D || nd->k_stride_token < hkv * nd->k_stride_head) return ATTN_ERR_STRIDE;
    if (nd->v_stride_head < D || nd->v_stride_token < hkv * nd->v_stride_head) return ATTN_ERR_STRIDE;
    if (n_seqs == 0) return ATTN_OK;
    if (!kv_pool || !k_new || !v_new || !block_table || !seq_lens || !cu_q) return ATTN_ERR_NULL;
    if (!aligned16(kv_pool) || !aligned16(k_new) || !aligned16(v_new)) return ATTN_ERR_ALIGN;
    if (!aligned4(block_table) || !aligned4(seq_lens) || !aligned4(cu_q)) return ATTN_ERR_ALIGN;
    w = pa::KvWriteArgs{};
    w.kv = static_cast<uint16_t *>(kv_pool);
    w.k_new = static_cast<const uint16_t *>(k_new);
    w.v_new = static_cast<const uint16_t *>(v_new);
    w.block_table = block_table;
    w.seq_lens = seq_lens;
    w.cu_q = cu_q;
    w.kv_sp = dims->kv_stride_page;
    w.kv_ss = dims->kv_stride_slot;
    w.kv_sh = dims->kv_stride_head;
    w.kv_skv = dims->kv_stride_kv;
    w.bt_stride = dims->bt_stride;
    w.k_st = nd->k_stride_token;
    w.k_sh = nd->k_stride_head;
    w.v_st = nd->v_stride_token;
    w.v_sh = nd->v_stride_head;
    w.n_seqs = n_seqs;
    w.max_q = max_q;
    w.hkv = dims->num_kv_heads;
    w.d = dims->head_dim;
    w.fp8 = kv_dtype == ATTN_KV_FP8_E4M3 ? 1 : 0;
    w.k_inv = w.fp8 ? 1.f / k_scale : 1.f;
    w.v_inv = w.fp8 ? 1.f / v_scale : 1.f;
    return ATTN_OK;
}

int kv_write_launch(const pa::KvWriteArgs &w, hipStream_t st) {
    const bool timing = timing_enabled();
    TimedLaunch tl{};
    if (timing && record_event(&tl.start, st) != ATTN_OK) return ATTN_ERR_HIP;
    if (pa::launch_kv_write(w, st) != hipSuccess) return ATTN_ERR_HIP;
    if (timing) {
        if (record_event(&tl.stop, st) != ATTN_OK) return ATTN_ERR_HIP;
        tl.kind = kTimedWrite;
        timing_push(tl);
    }
    return ATTN_OK;
}

int quant_layout(const attn_quant_dims *d, attn_quant_layout *lay) {
    if (!d || !lay) return ATTN_ERR_NULL;
    if (d->head_dim != pa::kQuantD) return ATTN_ERR_UNSUPPORTED;
    if (d->batch <= 0 || d->seq_len <= 0 || d->num_heads <= 0) return ATTN_ERR_SHAPE;
    if (d->batch > kGridYZMax || d->num_heads > kGridYZMax || 2 * (int64_t)d->batch > kGridYZMax)
        return ATTN_ERR_SHAPE;
    const int64_t *strides[] = {d->q_stride, d->k_stride, d->v_stride, d->o_stride};
    for (const int64_t *st : strides) {
        for (int i = 0; i < 3; ++i)
            if (st[i] <= 0 || (st[i] & 7) != 0) return ATTN_ERR_STRIDE;
        if (st[2] < d->head_dim || st[1] < (int64_t)d->num_heads * st[2] ||
            st[0] < (int64_t)d->seq_len * st[1])
            return ATTN_ERR_STRIDE;
    }
    const int64_t B = d->batch, N = d->seq_len, H = d->num_heads, D = d->head_dim;
    const int64_t blocks = (N + pa::kQuantBlock - 1) / pa::kQuantBlock;
    const int64_t chunks = (N + pa::kQuantChunk - 1) / pa::kQuantChunk;
    if (blocks > INT32_MAX || blocks * pa::kQuantBlock > INT32_MAX) return ATTN_ERR_SHAPE;
    // the attention kernel addresses one head's K codes and V^T with 32-bit offsets
    if (N * H * D > INT32_MAX || D * blocks * pa::kQuantBlock > INT32_MAX) return ATTN_ERR_SHAPE;
    *lay = attn_quant_layout{};
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off = align_up(off + bytes, kWsAlign);
        return o;
    };
    lay->off_mk = take((size_t)(B * H * D) * 4);
    lay->off_sv = take((size_t)(B * H * D) * 4);
    lay->off_sq = take((size_t)(B * H * blocks) * 4);
    lay->off_sk = take((size_t)(B * H * blocks) * 4);
    lay->off_qi = take((size_t)(B * N * H * D));
    lay->off_ki = take((size_t)(B * N * H * D));
    lay->off_vt = take((size_t)(B * H * D * blocks * pa::kQuantBlock));
    lay->off_ksum = take((size_t)(B * H * chunks * D) * 8);
    lay->off_vmax = take((size_t)(B * H * chunks * D) * 4);
    lay->workspace_bytes = off;
    lay->blocks = (int32_t)blocks;
    lay->chunks = (int32_t)chunks;
    lay->vt_stride = (int32_t)(blocks * pa::kQuantBlock);
    return ATTN_OK;
}

int quant_args(const attn_quant_dims *d, void *workspace, size_t bytes, pa::QuantArgs *a) {
    attn_quant_layout lay;
    int rc = quant_layout(d, &lay);
    if (rc != ATTN_OK) return rc;
    if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & (kWsAlign - 1)) != 0 ||
        bytes < lay.workspace_bytes)
        return ATTN_ERR_WORKSPACE;
    char *w = static_cast<char *>(workspace);
    *a = pa::QuantArgs{};
    a->b = d->batch;
    a->n = d->seq_len;
    a->h = d->num_heads;
    a->blocks = lay.blocks;
    a->chunks = lay.chunks;
    a->vt_stride = lay.vt_stride;
    a->mk = reinterpret_cast<float *>(w + lay.off_mk);
    a->sv = reinterpret_cast<float *>(w + lay.off_sv);
    a->sq = reinterpret_cast<float *>(w + lay.off_sq);
    a->sk = reinterpret_cast<float *>(w + lay.off_sk);
    a->qi = reinterpret_cast<int8_t *>(w + lay.off_qi);
    a->ki = reinterpret_cast<int8_t *>(w + lay.off_ki);
    a->vt = reinterpret_cast<uint8_t *>(w + lay.off_vt);
    a->ksum_part = reinterpret_cast<double *>(w + lay.off_ksum);
    a->vmax_part = reinterpret_cast<float *>(w + lay.off_vmax);
    return ATTN_OK;
}

int quant_prep_impl(const void *q, const void *k, const void *v, const attn_quant_dims *d,
                    void *workspace, size_t bytes, void *stream) {
    pa::QuantArgs a;
    int rc = quant_args(d, workspace, bytes, &a);
    if (rc != ATTN_OK) return rc;
    if (!q || !k || !v) return ATTN_ERR_NULL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v)) return ATTN_ERR_ALIGN;
    a.q = static_cast<const uint16_t *>(q);
    a.k = static_cast<const uint16_t *>(k);
    a.v = static_cast<const uint16_t *>(v);
    a.q_sb = d->q_stride[0]; a.q_st = d->q_stride[1]; a.q_sh = d->q_stride[2];
    a.k_sb = d->k_stride[0]; a.k_st = d->k_stride[1]; a.k_sh = d->k_stride[2];
    a.v_sb = d->v_stride[0]; a.v_st = d->v_stride[1]; a.v_sh = d->v_stride[2];
    hipStream_t st = static_cast<hipStream_t>(stream);
    const bool timing = timing_enabled();
    TimedLaunch tl{};
    if (timing && record_event(&tl.start, st) != ATTN_OK) return ATTN_ERR_HIP;
    if (pa::launch_quant_prep(a, st) != hipSuccess) return ATTN_ERR_HIP;
    if (timing) {
        if (record_event(&tl.stop, st) != ATTN_OK) return ATTN_ERR_HIP;
        tl.kind = kTimedPrep;
        timing_push(tl);
    }
    return ATTN_OK;
}

int quant_attend_impl(void *out, const attn_quant_dims *d, float scale, int32_t causal,
                      const void *workspace, size_t bytes, void *stream) {
    pa::QuantArgs a;
    int rc = quant_args(d, const_cast<void *>(workspace), bytes, &a);
    if (rc != ATTN_OK) return rc;
    if (!out) return ATTN_ERR_NULL;
    if (!aligned16(out)) return ATTN_ERR_ALIGN;
    if (!std::isfinite(scale)) return ATTN_ERR_SHAPE;
    a.out = static_cast<uint16_t *>(out);
    a.o_sb = d->o_stride[0]; a.o_st = d->o_stride[1]; a.o_sh = d->o_stride[2];
    a.scale_log2_pos = std::max((float)(std::fabs((double)scale) * 1.4426950408889634), FLT_MIN);
    a.q_negate = scale < 0.f ? 1 : 0;
    a.causal = causal ? 1 : 0;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const bool timing = timing_enabled();
    TimedLaunch tl{};
    if (timing && record_event(&tl.start, st) != ATTN_OK) return ATTN_ERR_HIP;
    if (pa::launch_quant_attn(a, st) != hipSuccess) return ATTN_ERR_HIP;
    if (timing) {
        if (record_event(&tl.stop, st) != ATTN_OK) return ATTN_ERR_HIP;
        tl.kind = kTimedMain;
        timing_push(tl);
    }
    return ATTN_OK;
}

// ---- KV-cache write fused into the split-decode launch ----------------------
// The split kernels can take the step's new K/V rows themselves when every
// 16-byte chunk of one (sequence, KV head)'s new rows has a holder thread:
// n * 2 * (D / elements per chunk) <= 256 (decode, and short runs of up to
// 8 tokens at D = 128, 4 at D = 256; twice that over an fp8 cache).
bool write_fusable(const attn_paged_plan &plan, const attn_paged_dims *d, int32_t max_q, int32_t kv_dtype) {
    const bool split = plan.path == ATTN_PATH_SPLIT_DECODE || plan.path == ATTN_PATH_SPLIT_FUSED ||
                       plan.path == ATTN_PATH_SPLIT_BALANCED;
    const int64_t epc = kv_dtype == ATTN_KV_FP8_E4M3 ? 16 : 8;
    return split && (int64_t)std::max<int32_t>(max_q, 1) * 2 * (d->head_dim / epc) <= pa::kThreads;
}

void fuse_write(pa::AttnArgs &a, const pa::KvWriteArgs &w) {
    a.k_new = w.k_new;
    a.v_new = w.v_new;
    a.kn_st = w.k_st;
    a.kn_sh = w.k_sh;
    a.vn_st = w.v_st;
    a.vn_sh = w.v_sh;
    a.k_inv = w.k_inv;
    a.v_inv = w.v_inv;
}

// ---- allocation-free entry point ------------------------------------------
// The split-KV partials of attn_paged_fwd_noalloc live in this library-owned
// device array (one copy per GPU, resident from the code object's load on
// that GPU until the process ends).  Host code never passes the array's name
// to a kernel: it is a host-side stand-in, not a device address.  The device
// address comes from hipGetSymbolAddress, taken once per device with that
// device current, and only that pointer is used.
constexpr size_t kScratchBytes = ATTN_NOALLOC_SCRATCH_BYTES;
// The balanced plan's partial budget under the scratch bound: the plan may
// exceed its budget by two splits' worth plus the piece counts, so half the
// scratch leaves room for that.
constexpr size_t kScratchBalBudget = kScratchBytes / 2;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
std::vector<void *> g_scratch_ptr;   // per device index; null until first use

// Device address of `scratch` on the device that owns `stream` (the current
// device for the null stream).
int scratch_pointer(hipStream_t stream, void **ptr) {
    int dev = -1;
    if (stream) {
        hipDevice_t sd;
        if (hipStreamGetDevice(stream, &sd) != hipSuccess) return ATTN_ERR_HIP;
        dev = (int)sd;
    } else if (hipGetDevice(&dev) != hipSuccess) {
        return ATTN_ERR_HIP;
    }
    if (dev < 0) return ATTN_ERR_HIP;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if ((size_t)dev >= g_scratch_ptr.size()) g_scratch_ptr.resize((size_t)dev + 1, nullptr);
    if (!g_scratch_ptr[dev]) {
        int cur = -1;
        if (hipGetDevice(&cur) != hipSuccess) return ATTN_ERR_HIP;
        if (cur != dev && hipSetDevice(dev) != hipSuccess) return ATTN_ERR_HIP;
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev && hipSetDevice(cur) != hipSuccess) return ATTN_ERR_HIP;
        if (e != hipSuccess || !p) return ATTN_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return ATTN_OK;
}

}  // namespace

extern "C" {

int attn_paged_make_plan(const attn_paged_dims *dims, int32_t n_seqs, int32_t max_q,
                         int32_t path_hint, int32_t pages_per_split, attn_paged_plan *plan) {
    return make_plan(dims, n_seqs, max_q, path_hint, pages_per_split, 0, plan);
}

int attn_paged_workspace_bytes(const attn_paged_dims *dims, int32_t n_seqs, int32_t max_q,
                               size_t *bytes) {
    if (!bytes) return ATTN_ERR_NULL;
    attn_paged_plan plan;
    int rc = make_plan(dims, n_seqs, max_q, ATTN_PATH_AUTO, 0, 0, &plan);
    if (rc != ATTN_OK) return rc;
    *bytes = plan.workspace_bytes;
    return ATTN_OK;
}

int attn_paged_fwd(void *out, const void *q, const void *kv_pool, const int32_t *block_table,
                   const int32_t *seq_lens, const int32_t *cu_q, int32_t n_seqs, int32_t max_q,
                   float scale, int32_t causal, const attn_paged_dims *dims, void *workspace,
                   size_t workspace_bytes, void *stream) {
    return paged_fwd_impl(out, q, kv_pool, block_table, seq_lens, cu_q, n_seqs, max_q, scale,
                          causal, dims, workspace, workspace_bytes, stream, ATTN_PATH_AUTO, 0);
}

int attn_paged_fwd_ex(void *out, const void *q, const void *kv_pool, const int32_t *block_table,
                      const int32_t *seq_lens, const int32_t *cu_q, int32_t n_seqs, int32_t max_q,
                      float scale, int32_t causal, const attn_paged_dims *dims, void *workspace,
                      size_t workspace_bytes, void *stream, int32_t path_hint,
                      int32_t pages_per_split) {
    return paged_fwd_impl(out, q, kv_pool, block_table, seq_lens, cu_q, n_seqs, max_q, scale,
                          causal, dims, workspace, workspace_bytes, stream, path_hint,
                          pages_per_split);
}

int attn_paged_make_plan_opt(const attn_paged_dims *dims, int32_t n_seqs, int32_t max_q,
                             const attn_paged_options *opt, attn_paged_plan *plan) {
    if (!opt) return ATTN_ERR_NULL;
    return make_plan(dims, n_seqs, max_q, opt->path_hint, opt->pages_per_split, opt->window, plan, opt->kv_dtype);
}

int attn_paged_fwd_opt(void *out, const void *q, const void *kv_pool, const int32_t *block_table,
                       const int32_t *seq_lens, const int32_t *cu_q, int32_t n_seqs, int32_t max_q,
                       float scale, int32_t causal, const attn_paged_dims *dims, const attn_paged_options *opt,
                       void *workspace, size_t workspace_bytes, void *stream) {
    if (!opt) return ATTN_ERR_NULL;
    return paged_fwd_impl(out, q, kv_pool, block_table, seq_lens, cu_q, n_seqs, max_q, scale, causal, dims,
                          workspace, workspace_bytes, stream, opt->path_hint, opt->pages_per_split, opt->sinks,
                          opt->window, opt->kv_dtype, opt->k_scale, opt->v_scale);
}

int attn_paged_fwd_noalloc(void *out, const void *q, const void *kv_pool, const int32_t *block_table,
                           const int32_t *seq_lens, const int32_t *cu_q, int32_t n_seqs, int32_t max_q,
                           float scale, int32_t causal, const attn_paged_dims *dims,
                           const attn_paged_options *opt, void *stream) {
    attn_paged_options o{nullptr, 0, ATTN_PATH_AUTO, 0, ATTN_KV_BF16, 1.f, 1.f};
    if (opt) o = *opt;
    // Everything is validated, and the plan's partials checked against the
    // scratch size, before any HIP call; a 256-aligned stand-in takes the
    // workspace's place until the scratch address is known.
    attn_paged_plan plan;
    pa::AttnArgs a;
    void *const stand_in = reinterpret_cast<void *>(uintptr_t(kWsAlign));
    int rc = make_plan(dims, n_seqs, max_q, o.path_hint, o.pages_per_split, o.window, &plan, o.kv_dtype,
                       kScratchBalBudget, kScratchBytes);
    if (rc != ATTN_OK) return rc;
    if (plan.workspace_bytes > kScratchBytes) return ATTN_ERR_WORKSPACE;
    rc = paged_prepare(out, q, kv_pool, block_table, seq_lens, cu_q, n_seqs, max_q, scale, causal, dims,
                       stand_in, kScratchBytes, o.path_hint, o.pages_per_split, o.sinks, o.window, plan, a,
                       o.kv_dtype, o.k_scale, o.v_scale, kScratchBalBudget, kScratchBytes);
    if (rc != ATTN_OK || n_seqs == 0) return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    void *ws = nullptr;
    if (plan.workspace_bytes > 0) {
        rc = scratch_pointer(st, &ws);
        if (rc != ATTN_OK) return rc;
        rc = paged_prepare(out, q, kv_pool, block_table, seq_lens, cu_q, n_seqs, max_q, scale, causal, dims, ws,
                           kScratchBytes, o.path_hint, o.pages_per_split, o.sinks, o.window, plan, a, o.kv_dtype,
                           o.k_scale, o.v_scale, kScratchBalBudget, kScratchBytes);
        if (rc != ATTN_OK) return rc;
        // The single-launch merge needs its counters at zero; earlier calls
        // on this GPU may have left partials in those bytes.  A kernel, not a
        // memset node, so that a captured graph replays it correctly.
        if (plan.counter_bytes > 0 &&
            pa::launch_workspace_clear(static_cast<uint32_t *>(ws), plan.counter_bytes / 4, st) != hipSuccess)
            return ATTN_ERR_HIP;
    }
    return paged_launch(plan, a, dims->head_dim, st);
}

int attn_paged_kv_write(void *kv_pool, const void *k_new, const void *v_new, const int32_t *block_table,
                        const int32_t *seq_lens, const int32_t *cu_q, int32_t n_seqs, int32_t max_q,
                        const attn_paged_dims *dims, const attn_kv_new_dims *new_dims, void *stream) {
    pa::KvWriteArgs w;
    int rc = kv_write_prepare(kv_pool, k_new, v_new, block_table, seq_lens, cu_q, n_seqs, max_q, dims,
                              new_dims, w);
    if (rc != ATTN_OK || n_seqs == 0) return rc;
    return kv_write_launch(w, static_cast<hipStream_t>(stream));
}

int attn_paged_fwd_write(void *out, const void *q, const void *k_new, const void *v_new, void *kv_pool,
                         const int32_t *block_table, const int32_t *seq_lens, const int32_t *cu_q,
                         int32_t n_seqs, int32_t max_q, float scale, int32_t causal,
                         const attn_paged_dims *dims, const attn_kv_new_dims *new_dims, void *workspace,
                         size_t workspace_bytes, void *stream) {
    // every argument of both steps is checked before anything is launched
    pa::KvWriteArgs w;
    int rc = kv_write_prepare(kv_pool, k_new, v_new, block_table, seq_lens, cu_q, n_seqs, max_q, dims,
                              new_dims, w);
    if (rc != ATTN_OK) return rc;
    attn_paged_plan plan;
    pa::AttnArgs a;
    rc = paged_prepare(out, q, kv_pool, block_table, seq_lens, cu_q, n_seqs, max_q, scale, causal, dims,
                       workspace, workspace_bytes, ATTN_PATH_AUTO, 0, nullptr, 0, plan, a);
    if (rc != ATTN_OK || n_seqs == 0) return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (write_fusable(plan, dims, max_q, ATTN_KV_BF16)) {
        fuse_write(a, w);   // one launch: the split kernel writes the new rows it streams
        return paged_launch(plan, a, dims->head_dim, st);
    }
    rc = kv_write_launch(w, st);
    if (rc != ATTN_OK) return rc;
    return paged_launch(plan, a, dims->head_dim, st);
}

int attn_paged_kv_write_opt(void *kv_pool, const void *k_new, const void *v_new, const int32_t *block_table,
                            const int32_t *seq_lens, const int32_t *cu_q, int32_t n_seqs, int32_t max_q,
                            const attn_paged_dims *dims, const attn_kv_new_dims *new_dims,
                            const attn_paged_options *opt, void *stream) {
    if (!opt) return ATTN_ERR_NULL;
    pa::KvWriteArgs w;
    int rc = kv_write_prepare(kv_pool, k_new, v_new, block_table, seq_lens, cu_q, n_seqs, max_q, dims,
                              new_dims, w, opt->kv_dtype, opt->k_scale, opt->v_scale);
    if (rc != ATTN_OK || n_seqs == 0) return rc;
    return kv_write_launch(w, static_cast<hipStream_t>(stream));
}

int attn_paged_fwd_write_opt(void *out, const void *q, const void *k_new, const void *v_new, void *kv_pool,
                             const int32_t *block_table, const int32_t *seq_lens, const int32_t *cu_q,
                             int32_t n_seqs, int32_t max_q, float scale, int32_t causal,
                             const attn_paged_dims *dims, const attn_kv_new_dims *new_dims,
                             const attn_paged_options *opt, void *workspace, size_t workspace_bytes,
                             void *stream) {
    if (!opt) return ATTN_ERR_NULL;
    pa::KvWriteArgs w;
    int rc = kv_write_prepare(kv_pool, k_new, v_new, block_table, seq_lens, cu_q, n_seqs, max_q, dims,
                              new_dims, w, opt->kv_dtype, opt->k_scale, opt->v_scale);
    if (rc != ATTN_OK) return rc;
    attn_paged_plan plan;
    pa::AttnArgs a;
    rc = paged_prepare(out, q, kv_pool, block_table, seq_lens, cu_q, n_seqs, max_q, scale, causal, dims,
                       workspace, workspace_bytes, opt->path_hint, opt->pages_per_split, opt->sinks, opt->window,
                       plan, a, opt->kv_dtype, opt->k_scale, opt->v_scale);
    if (rc != ATTN_OK || n_seqs == 0) return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (write_fusable(plan, dims, max_q, opt->kv_dtype)) {
        fuse_write(a, w);
        return paged_launch(plan, a, dims->head_dim, st);
    }
    rc = kv_write_launch(w, st);
    if (rc != ATTN_OK) return rc;
    return paged_launch(plan, a, dims->head_dim, st);
}

int attn_workspace_clear(void *workspace, size_t bytes, void *stream) {
    if (bytes == 0) return ATTN_OK;
    if (!workspace) return ATTN_ERR_NULL;
    if (!aligned4(workspace)) return ATTN_ERR_ALIGN;
    if (bytes % 4) return ATTN_ERR_SHAPE;
    if (pa::launch_workspace_clear(static_cast<uint32_t *>(workspace), bytes / 4,
                                   static_cast<hipStream_t>(stream)) != hipSuccess)
        return ATTN_ERR_HIP;
    return ATTN_OK;
}

int attn_kernel_timing_enable(int32_t enable) {
    std::lock_guard<std::mutex> lk(g_timing_mu);
    g_timing_on = enable != 0;
    return ATTN_OK;
}

int attn_kernel_timing_read(double *main_ms, int32_t *main_launches, double *combine_ms,
                            int32_t *combine_launches, double *prep_ms, int32_t *prep_launches,
                            double *write_ms, int32_t *write_launches) {
    std::vector<TimedLaunch> v;
    {
        std::lock_guard<std::mutex> lk(g_timing_mu);
        v.swap(g_timed);
    }
    double tms[4] = {0, 0, 0, 0};
    int32_t cnt[4] = {0, 0, 0, 0};
    int rc = ATTN_OK;
    for (auto &t : v) {
        float ms = 0.f;
        if (hipEventSynchronize(t.stop) != hipSuccess ||
            hipEventElapsedTime(&ms, t.start, t.stop) != hipSuccess)
            rc = ATTN_ERR_HIP;
        tms[t.kind] += ms;
        ++cnt[t.kind];
        (void)hipEventDestroy(t.start);
        (void)hipEventDestroy(t.stop);
    }
    if (main_ms) *main_ms = tms[kTimedMain];
    if (main_launches) *main_launches = cnt[kTimedMain];
    if (combine_ms) *combine_ms = tms[kTimedCombine];
    if (combine_launches) *combine_launches = cnt[kTimedCombine];
    if (prep_ms) *prep_ms = tms[kTimedPrep];
    if (prep_launches) *prep_launches = cnt[kTimedPrep];
    if (write_ms) *write_ms = tms[kTimedWrite];
    if (write_launches) *write_launches = cnt[kTimedWrite];
    return rc;
}

int attn_quant_layout_of(const attn_quant_dims *dims, attn_quant_layout *layout) {
    return quant_layout(dims, layout);
}

int attn_quant_prep(const void *q, const void *k, const void *v, const attn_quant_dims *dims,
                    void *workspace, size_t workspace_bytes, void *stream) {
    return quant_prep_impl(q, k, v, dims, workspace, workspace_bytes, stream);
}

int attn_quant_attend(void *out, const attn_quant_dims *dims, float scale, int32_t causal,
                      const void *workspace, size_t workspace_bytes, void *stream) {
    return quant_attend_impl(out, dims, scale, causal, workspace, workspace_bytes, stream);
}

int attn_quant_fwd(void *out, const void *q, const void *k, const void *v,
                   const attn_quant_dims *dims, float scale, int32_t causal, void *workspace,
                   size_t workspace_bytes, void *stream) {
    // validate everything before launching anything
    pa::QuantArgs a;
    int rc = quant_args(dims, workspace, workspace_bytes, &a);
    if (rc != ATTN_OK) return rc;
    if (!out || !q || !k || !v) return ATTN_ERR_NULL;
    if (!aligned16(out) || !aligned16(q) || !aligned16(k) || !aligned16(v)) return ATTN_ERR_ALIGN;
    if (!std::isfinite(scale)) return ATTN_ERR_SHAPE;
    rc = quant_prep_impl(q, k, v, dims, workspace, workspace_bytes, stream);
    if (rc != ATTN_OK) return rc;
    return quant_attend_impl(out, dims, scale, causal, workspace, workspace_bytes, stream);
}

const char *attn_status_string(int status) {
    switch (status) {
        case ATTN_OK: return "ok";
        case ATTN_ERR_NULL: return "a required pointer is NULL";
        case ATTN_ERR_SHAPE: return "inconsistent or out-of-range sizes";
        case ATTN_ERR_UNSUPPORTED: return "unsupported configuration (head_dim, page_size or rows)";
        case ATTN_ERR_STRIDE: return "invalid stride";
        case ATTN_ERR_ALIGN: return "pointer not aligned";
        case ATTN_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
        case ATTN_ERR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

int attn_version(void) { return kVersion; }

}  // extern "C"
