/*
 * paged_attn.h -- C ABI of the MI355X (gfx950) paged grouped-query attention
 * library (libpaged_attn.so).
 *
 * Operation (defined once, used by every entry point below).  For each
 * sequence b in [0, n_seqs), with n_b = cu_q[b+1] - cu_q[b] new query tokens
 * and L_b = seq_lens[b] cached keys, query token i (row t = cu_q[b] + i) of
 * q head h attends to the keys j in [0, vis) of KV head g = h / G, where
 * G = num_q_heads / num_kv_heads, pos = L_b - n_b + i and
 * vis = causal ? clamp(pos + 1, 0, L_b) : L_b:
 *
 *     out[t, h, :] = sum_j softmax_j(scale * <q[t, h, :], K_j>) * V_j
 *
 * Key j lives in page block_table[b, j / P], slot j % P of the pool.  Rows
 * with no visible key are written as zeros.  The slots of a sequence's last
 * page past L_b, and pages its table does not name, may hold any bits
 * (NaN and infinities included): none reaches the result.
 *   - Scaled dot-product attention over a paged KV cache, causal or unmasked,
 *     with ragged lengths and grouped q heads: Mojo SM100MHA2Q API docs
 *     (struct summary; parameters KVLUTType, MaskType, ValidLengthType,
 *     PartitionType; comptime members group, fuse_gqa, page_size).
 *   - Pool, block table, lengths and cumulative query offsets as separate
 *     device buffers, K and V as offsets into one pool: kern-kernels
 *     examples/decode.json (buffers; ops.decode.params; programs.decode).
 *   - The cache already holds the step's own tokens when attention runs:
 *     metrale blueprint graph.json (node l3.attn.kv_write precedes
 *     l3.attn.attend), hence queries sit at the tail (bottom-right causal).
 *
 * Conventions shared by every call:
 *   - All tensor pointers are DEVICE pointers owned by the caller; the library
 *     never allocates, frees or synchronises.  bf16 is IEEE bfloat16 stored in
 *     16 bits; int32 is little-endian two's complement.
 *   - Every call validates its arguments on the host before launching
 *     anything and returns an attn_status code (0 = success, negative =
 *     error).  A call that fails validation launches nothing and leaves `out`
 *     untouched.  Errors inside kernels (for example a page id outside
 *     [0, num_pages)) are not detected; they surface at the caller's next
 *     synchronisation as a HIP error.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL = the
 *     default stream).  Calls are re-entrant as long as concurrent calls use
 *     distinct workspaces.
 *   - Strides are in ELEMENTS; the head_dim axis must be contiguous.  Base
 *     pointers must be 16-byte aligned and every bf16 stride a multiple of 8.
 */
#ifndef PAGED_ATTN_H
#define PAGED_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum attn_status {
    ATTN_OK = 0,
    ATTN_ERR_NULL = -1,        /* a required pointer is NULL */
    ATTN_ERR_SHAPE = -2,       /* inconsistent or out-of-range sizes */
    ATTN_ERR_UNSUPPORTED = -3, /* head_dim not in {128, 256}, page_size != 64, ... */
    ATTN_ERR_STRIDE = -4,      /* bad stride (non-positive, not a multiple of 8, overlapping) */
    ATTN_ERR_ALIGN = -5,       /* base pointer not 16-byte aligned */
    ATTN_ERR_WORKSPACE = -6,   /* workspace missing, misaligned or too small */
    ATTN_ERR_HIP = -7          /* a HIP runtime call failed (launch error) */
} attn_status;

/* Sizes and element strides of the paged attention operands. */
typedef struct attn_paged_dims {
    int32_t num_q_heads;       /* Hq */
    int32_t num_kv_heads;      /* Hkv; Hq % Hkv == 0, G = Hq / Hkv */
    int32_t head_dim;          /* D: 128 or 256 */
    int32_t page_size;         /* P: 64 (slots per page) */
    int32_t num_pages;         /* NP >= 1: pages in the pool (valid ids are [0, NP)) */
    int32_t max_pages_per_seq; /* MP >= 1: block-table columns; every L_b <= MP * P */
    int64_t num_tokens;        /* rows of q and out (>= cu_q[n_seqs]) */
    int64_t q_stride_token;    /* q[t, h, d] at q + t*q_stride_token + h*q_stride_head + d */
    int64_t q_stride_head;
    int64_t o_stride_token;    /* out[t, h, d] likewise */
    int64_t o_stride_head;
    int64_t kv_stride_page;    /* K_j of head g: pool + page*kv_stride_page + slot*kv_stride_slot */
    int64_t kv_stride_slot;    /*                  + g*kv_stride_head;  V_j = that + kv_stride_kv */
    int64_t kv_stride_head;
    int64_t kv_stride_kv;
    int64_t bt_stride;         /* elements between block-table rows (>= MP) */
} attn_paged_dims;

/* Execution plan chosen for a call (host-side; no device access). */
typedef struct attn_paged_plan {
    int32_t path;              /* ATTN_PATH_SPLIT_DECODE or ATTN_PATH_PREFILL */
    int32_t pages_per_split;   /* KV pages one workgroup streams (split path); balanced
                                  path: the least pages of one range; split-key
                                  prefill: the pages of one key run */
    int32_t max_splits;        /* ceil(MP / pages_per_split); balanced path: the most
                                  pieces one sequence can be cut into; prefill: key
                                  runs per item (1 = one pass) */
    int32_t grid_x, grid_y, grid_z;
    int32_t block_threads;
    size_t workspace_bytes;    /* bytes of workspace the call needs (0 if none) */
    size_t counter_bytes;      /* leading workspace bytes holding merge counters (0 if none) */
} attn_paged_plan;

enum {
    ATTN_PATH_AUTO = 0,
    ATTN_PATH_SPLIT_DECODE = 1, /* split-KV partial kernel + log-sum-exp combine kernel; takes
                                   up to 64 packed rows G * max_q per (sequence, KV head), in
                                   blocks of 16 (more than 16 rows: the short-sequence body of
                                   the Mojo SM100MHA2Q docs' struct summary, short query runs
                                   routed to a cheaper body than the prefill tile) */
    ATTN_PATH_PREFILL = 2,      /* q-tile kernel with causal tile skipping; a grid of at
                                   most 128 (tile, KV head, sequence) items has each
                                   item's keys split into runs of the split-decode
                                   layout (page runs from row 0's window start),
                                   merged by the combine kernel, so that about one
                                   workgroup per CU runs */
    ATTN_PATH_SPLIT_FUSED = 3,  /* split-KV kernel whose last split per (sequence, KV head)
                                   merges the partials: one launch (decode.json's single
                                   launch with an i32 counter scratch, ops.decode.impl).
                                   Same bits as ATTN_PATH_SPLIT_DECODE; AUTO picks the
                                   two-kernel form, which measured faster on MI355X. */
    ATTN_PATH_SPLIT_BALANCED = 4 /* split-KV over an even division of the batch's pages:
                                   the pages every sequence needs, in sequence order,
                                   cut into grid_y equal ranges (at least pages_per_split
                                   pages each; a range may span sequences), one
                                   workgroup per (KV head, range), then the combine
                                   kernel for sequences cut into several pieces.  The
                                   same PartitionType split as ATTN_PATH_SPLIT_DECODE
                                   with the cuts placed by length, so ragged batches
                                   keep every workgroup equally busy.  At most
                                   1024 sequences.  AUTO's choice for decode-shaped
                                   and short calls (G * max_q <= 64, pages_per_split
                                   = 0, n_seqs <= 1024); longer query runs take
                                   ATTN_PATH_PREFILL. */
};

/*
 * attn_paged_make_plan -- choose path, split size and grid for a call with
 * these sizes.  path_hint: ATTN_PATH_AUTO or a forced path; pages_per_split:
 * 0 = automatic, otherwise forced (with ATTN_PATH_AUTO a forced value
 * selects ATTN_PATH_SPLIT_DECODE; on the balanced path it is the least range
 * size; with ATTN_PATH_PREFILL it splits every item's keys into runs of that
 * many pages, and a value of at least max_pages_per_seq keeps one pass).  Pure host logic: it
 * reads no device memory and may be called without a GPU.
 * Split-KV partial outputs and (max, sum) statistics per split follow the
 * decode.json manifest's scratch buffers partial / stats (ops.decode.impl
 * .scratch) and the Mojo docs' PartitionType (KV-cache partition scheme).
 * Returns ATTN_OK or a validation error.
 */
int attn_paged_make_plan(const attn_paged_dims *dims, int32_t n_seqs, int32_t max_q,
                         int32_t path_hint, int32_t pages_per_split, attn_paged_plan *plan);

/*
 * attn_paged_workspace_bytes -- device workspace (bytes) that attn_paged_fwd
 * needs for these sizes under the automatic plan; writes it to *bytes.
 * Host-only, may be called without a GPU.
 */
int attn_paged_workspace_bytes(const attn_paged_dims *dims, int32_t n_seqs, int32_t max_q,
                               size_t *bytes);

/*
 * attn_paged_fwd -- paged GQA attention forward (the operation above).
 *   out          bf16 [num_tokens, Hq, D] (strided); rows [0, cu_q[n_seqs])
 *                are written, other rows untouched.
 *   q            bf16 [num_tokens, Hq, D] (strided).
 *   kv_pool      bf16 pool; K/V rows addressed through dims' kv strides.
 *   block_table  int32 [n_seqs, MP] (row stride dims->bt_stride); only the
 *                first ceil(L_b / P) entries of row b are read.
 *   seq_lens     int32 [n_seqs]: L_b, the total KV length including this
 *                step's n_b tokens; 0 <= L_b <= MP * P.
 *   cu_q         int32 [n_seqs + 1]: cu_q[0] = 0, non-decreasing,
 *                cu_q[n_seqs] <= num_tokens.
 *   n_seqs       number of sequences (>= 0; 0 is a no-op).
 *   max_q        host-side upper bound on every n_b (sizes the grid without
 *                reading device memory); n_b > max_q is a caller error.
 *   scale        softmax scale applied to q.K (for example 1/sqrt(D)).
 *   causal       nonzero = bottom-right aligned causal mask.
 *   workspace    device buffer of >= attn_paged_workspace_bytes bytes,
 *                256-byte aligned (may be NULL when that size is 0); holds
 *                the split-KV partials and, on the fused split path, the
 *                merge counters in its first plan.counter_bytes bytes.  On
 *                the prefill path it holds the launch order when the grid
 *                has two or more sequences and 512 or more workgroups (one
 *                int32 per workgroup, written by the call before the
 *                prefill kernel reads it: the grid's items sorted by the KV
 *                pages each streams, most first, so that a ragged batch's
 *                longest items do not start last), or, for a split-key
 *                prefill, the split partials, after the fp8 staging pool
 *                and table over an fp8 cache.  Those
 *                counter bytes must be zero when the call starts; every call
 *                that runs to completion leaves them zero again.  A buffer
 *                from a zeroing allocator, or one cleared once with
 *                attn_workspace_clear, qualifies; after a call on another
 *                path or a larger plan has used the same bytes for partials,
 *                clear them again.  Calls that share a workspace must not
 *                overlap in time.
 *   stream       hipStream_t to enqueue on (NULL = default stream).
 */
int attn_paged_fwd(void *out, const void *q, const void *kv_pool, const int32_t *block_table,
                   const int32_t *seq_lens, const int32_t *cu_q, int32_t n_seqs, int32_t max_q,
                   float scale, int32_t causal, const attn_paged_dims *dims, void *workspace,
                   size_t workspace_bytes, void *stream);

/*
 * attn_paged_fwd_ex -- attn_paged_fwd with a forced path and split size
 * (path_hint / pages_per_split as in attn_paged_make_plan).  The workspace
 * must hold the workspace_bytes of that plan.  For tests and tuning.
 */
int attn_paged_fwd_ex(void *out, const void *q, const void *kv_pool, const int32_t *block_table,
                      const int32_t *seq_lens, const int32_t *cu_q, int32_t n_seqs, int32_t max_q,
                      float scale, int32_t causal, const attn_paged_dims *dims, void *workspace,
                      size_t workspace_bytes, void *stream, int32_t path_hint,
                      int32_t pages_per_split);

/* ---------------------------------------------------------------------------
 * Options of the paged call: attention sinks and a sliding window.
 *
 *   sinks   device f32 [Hq], 4-byte aligned, or NULL: one logit per q head in
 *           the units of the scaled scores (scale * q.k) that joins the softmax
 *           normalisation and carries no value row (Mojo SM100MHA2Q docs,
 *           SinkType: an optional pointer to attention-sink weights):
 *             out[t, h] = sum_j e^{s_j} V_j / (e^{sinks[h]} + sum_j e^{s_j}).
 *           -inf entries mean no sink for that head.
 *   window  0 = none; W > 0: a query at position pos sees only keys
 *           j >= pos - W + 1, besides the causal / length bound (decode.json's
 *           parameter pack carries an INT32_MAX field, read as "window
 *           disabled"; any W >= max_pages_per_seq * page_size changes
 *           nothing).  Negative values are a shape error.
 *   path_hint, pages_per_split: as for attn_paged_fwd_ex.
 * With a window the split path plans and reads only the pages from row 0's
 * window start on; rows with neither a visible key nor a sink give zeros, and
 * rows with only a sink give zeros too (all weight on the sink).
 */
typedef struct attn_paged_options {
    const float *sinks;
    int32_t window;
    int32_t path_hint;
    int32_t pages_per_split;
    int32_t kv_dtype;          /* ATTN_KV_BF16 (0) or ATTN_KV_FP8_E4M3 (1) */
    float k_scale, v_scale;    /* fp8 cache: K = k_scale * e4m3(code), V = v_scale * e4m3(code);
                                  ignored for a bf16 cache */
} attn_paged_options;

/*
 * KV-cache element types.  ATTN_KV_FP8_E4M3: the pool holds OCP e4m3 codes
 * (1 byte; dims' kv strides then count bytes and must be multiples of 16),
 * with one scale for all of K and one for all of V (the Mojo SM100MHA2Q docs
 * carry fp8 branches of the KV dtype; per-tensor scales are the reading taken
 * here).  Supported on every path.  The split-decode paths (packed rows
 * G * max_q <= 64) read the codes directly; the prefill path first decodes
 * the pages it reads (exactly: every e4m3 value is a bf16 value) into a
 * bf16 staging pool in the workspace, so its plan's workspace_bytes is
 * n_seqs * max_pages_per_seq * (P * Hkv * 2 * D * 2 + 4) bytes, plus the
 * launch order's 4 bytes per workgroup where the grid takes one or a split-key
 * prefill's partials (each part 256-byte aligned).  Scales must be finite.
 */
enum { ATTN_KV_BF16 = 0, ATTN_KV_FP8_E4M3 = 1 };

/* attn_paged_make_plan with options (the window shrinks the split plan). */
int attn_paged_make_plan_opt(const attn_paged_dims *dims, int32_t n_seqs, int32_t max_q,
                             const attn_paged_options *opt, attn_paged_plan *plan);

/* attn_paged_fwd with options; the workspace must hold the workspace_bytes of
 * attn_paged_make_plan_opt for the same options. */
int attn_paged_fwd_opt(void *out, const void *q, const void *kv_pool, const int32_t *block_table,
                       const int32_t *seq_lens, const int32_t *cu_q, int32_t n_seqs, int32_t max_q,
                       float scale, int32_t causal, const attn_paged_dims *dims, const attn_paged_options *opt,
                       void *workspace, size_t workspace_bytes, void *stream);

/* ---------------------------------------------------------------------------
 * attn_paged_fwd_noalloc -- attn_paged_fwd_opt for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  It takes no workspace.  The split-KV
 * partials (and the single-launch merge's counters) live in a library-owned
 * device array of ATTN_NOALLOC_SCRATCH_BYTES per GPU, part of the library's
 * code object: each GPU the library runs on holds it until the process ends.
 * The call itself allocates nothing (no hipMalloc, hipFree or allocating
 * library routine).
 *   opt     as for attn_paged_fwd_opt, or NULL for no options (automatic
 *           path, bf16 cache).
 *   Every other argument as for attn_paged_fwd_opt; the caller still owns
 *   q, out and the cache.
 * The plan is the automatic one except that the balanced split path budgets
 * its partials to half the array, so results can differ from
 * attn_paged_fwd_opt's by accumulation order (within the same tolerance),
 * that a prefill launch order that would not fit beside the fp8 staging
 * pool in the array is left out (grid order; same bits), and that a small
 * prefill grid whose split partials would not fit keeps one pass (within
 * the same tolerance).
 * A plan whose partials still exceed the array returns ATTN_ERR_WORKSPACE
 * before anything is launched.  Merge counters are cleared by a kernel
 * before each call that needs them (no memset node).  Every call on one GPU
 * shares that GPU's array: calls that overlap in time on one GPU (other
 * streams or threads) race and give wrong results; calls in stream order do
 * not.  The first call on a GPU looks up the array's device address with
 * that GPU current (ATTN_ERR_HIP if that fails).
 */
#define ATTN_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)   /* 64 MiB per GPU */

int attn_paged_fwd_noalloc(void *out, const void *q, const void *kv_pool, const int32_t *block_table,
                           const int32_t *seq_lens, const int32_t *cu_q, int32_t n_seqs, int32_t max_q,
                           float scale, int32_t causal, const attn_paged_dims *dims,
                           const attn_paged_options *opt, void *stream);

/* ---------------------------------------------------------------------------
 * KV-cache write: the step's new K and V rows into the paged pool, the step
 * that runs just before attention (metrale blueprint graph.json: node
 * l3.attn.kv_write precedes l3.attn.attend; page layout of kern-kernels
 * examples/decode.json, buffers kv / table / seq / cuq).
 *
 * For sequence b with n_b = cu_q[b+1] - cu_q[b] new tokens and L_b =
 * seq_lens[b] keys in all (the new ones included), new token i (row
 * t = cu_q[b] + i) is key position pos = L_b - n_b + i: k_new[t, g, :] and
 * v_new[t, g, :] of every KV head g are written to the K and V rows of page
 * block_table[b, pos / P], slot pos % P.  Tokens with pos < 0 (n_b > L_b) are
 * not written.  Nothing else in the pool changes.
 */
typedef struct attn_kv_new_dims {
    int64_t k_stride_token;    /* k_new[t, g, d] at k_new + t*k_stride_token + g*k_stride_head + d */
    int64_t k_stride_head;
    int64_t v_stride_token;    /* v_new likewise */
    int64_t v_stride_head;
} attn_kv_new_dims;

/*
 * attn_paged_kv_write -- the cache write alone.
 *   kv_pool        bf16 pool, written (addressed through dims' kv strides).
 *   k_new, v_new   bf16 [num_tokens, Hkv, D] (strides in new_dims; each a
 *                  multiple of 8, head stride >= D, token stride >= Hkv *
 *                  head stride), 16-byte aligned.  Views into a fused QKV
 *                  projection output qualify.
 *   block_table, seq_lens, cu_q, n_seqs, max_q, dims: as for attn_paged_fwd
 *                  (dims' q / out strides are checked, not used).
 * Pages written by two sequences at once, or a slot shared with a page that
 * another sequence reads, are the caller's race.  Returns ATTN_OK or a
 * validation error; nothing is launched on error.
 */
int attn_paged_kv_write(void *kv_pool, const void *k_new, const void *v_new, const int32_t *block_table,
                        const int32_t *seq_lens, const int32_t *cu_q, int32_t n_seqs, int32_t max_q,
                        const attn_paged_dims *dims, const attn_kv_new_dims *new_dims, void *stream);

/*
 * attn_paged_fwd_write -- the cache write followed by attn_paged_fwd in one
 * call (two launches in stream order; the attention sees the written rows).
 * Every argument of both steps is validated before either is launched.
 */
int attn_paged_fwd_write(void *out, const void *q, const void *k_new, const void *v_new, void *kv_pool,
                         const int32_t *block_table, const int32_t *seq_lens, const int32_t *cu_q,
                         int32_t n_seqs, int32_t max_q, float scale, int32_t causal,
                         const attn_paged_dims *dims, const attn_kv_new_dims *new_dims, void *workspace,
                         size_t workspace_bytes, void *stream);

/*
 * attn_paged_kv_write_opt / attn_paged_fwd_write_opt -- the same calls with
 * options (attn_paged_options above; the write uses kv_dtype, k_scale and
 * v_scale, the attention all of them).  Into an fp8 cache the new rows are
 * stored as OCP e4m3 codes of x * (1 / scale), with the reciprocal and the
 * product in f32, rounded to nearest even and saturating at +-448 (the
 * quantised path's reading of "value / scale"); the scales must be finite
 * and nonzero.
 */
int attn_paged_kv_write_opt(void *kv_pool, const void *k_new, const void *v_new, const int32_t *block_table,
                            const int32_t *seq_lens, const int32_t *cu_q, int32_t n_seqs, int32_t max_q,
                            const attn_paged_dims *dims, const attn_kv_new_dims *new_dims,
                            const attn_paged_options *opt, void *stream);
int attn_paged_fwd_write_opt(void *out, const void *q, const void *k_new, const void *v_new, void *kv_pool,
                             const int32_t *block_table, const int32_t *seq_lens, const int32_t *cu_q,
                             int32_t n_seqs, int32_t max_q, float scale, int32_t causal,
                             const attn_paged_dims *dims, const attn_kv_new_dims *new_dims,
                             const attn_paged_options *opt, void *workspace, size_t workspace_bytes,
                             void *stream);

/*
 * attn_workspace_clear -- enqueue a kernel that sets bytes [0, bytes) of a
 * device workspace to zero (the merge counters of the fused split path must
 * start at zero).  A kernel, not a memset node, so that graph capture of it
 * replays correctly.  workspace: 4-byte aligned device pointer (NULL only
 * with bytes == 0); bytes: a multiple of 4.  Returns ATTN_OK, ATTN_ERR_NULL,
 * ATTN_ERR_ALIGN, ATTN_ERR_SHAPE (bytes not a multiple of 4) or ATTN_ERR_HIP.
 */
int attn_workspace_clear(void *workspace, size_t bytes, void *stream);

/* ---------------------------------------------------------------------------
 * Quantised attention (int8 Q.K, fp8 P.V) over dense Q, K, V.
 *
 * Operation: softmax(scale * Q K^T) V per (batch b, head h) over the N tokens
 * of a sequence (queries and keys are the same N tokens; causal = query i
 * sees keys 0..i), computed through the quantisation steps named by the
 * SageAttention2 block-24 baseline page (h3-blackwell-runtime
 * benchmarks/gb10-sage2-block24-scheduler-baseline.json, phase_timings and
 * fused_mainloop_phases):
 *   1. K smoothing: mk = mean over tokens of K per (b, h, channel); K' = K - mk.
 *   2. Q and K' to int8 per (b, h, 64-token block): s = amax / 127 (1 for an
 *      all-zero block), code = clamp(rne(x / s), -127, 127).
 *   3. V to fp8 e4m3 per (b, h, channel): s_v = amax over tokens / 448,
 *      code = e4m3(V / s_v) (OCP e4m3, round to nearest even); stored
 *      transposed [b, h, channel, token] and padded to a multiple of 64
 *      tokens, with the tokens of every 64-token tile permuted.
 *   4. Fused loop over 64-key tiles: scores from the int8 products times the
 *      two block scales and scale; online softmax with the running maximum
 *      taken per tile; the weight w (<= 1) enters P.V as e4m3(448 w); the row
 *      sum uses the unrounded w; out = O s_v / (448 l), rounded to bf16.
 * Supported: head_dim 128.
 */
typedef struct attn_quant_dims {
    int32_t batch;        /* B */
    int32_t seq_len;      /* N: tokens per sequence (queries = keys) */
    int32_t num_heads;    /* H (one K/V head per q head) */
    int32_t head_dim;     /* D: 128 */
    int64_t q_stride[3];  /* element strides of (batch, token, head); D contiguous */
    int64_t k_stride[3];
    int64_t v_stride[3];
    int64_t o_stride[3];
} attn_quant_dims;

/* Byte offsets of the quantised intermediates inside the caller's workspace
 * (all 256-byte aligned).  Layouts: mk, sv f32 [B, H, D]; sq, sk f32
 * [B, H, blocks]; qi, ki int8 [B, N, H, D]; vt e4m3 codes [B, H, D, vt_stride]
 * where the token at offset j (< 64) of a 64-token tile is stored at position
 * 32 ((j % 8) / 4) + 16 (j / 32) + 4 ((j % 32) / 8) + j % 4 of the tile, and
 * padding tokens hold code 0; ksum (f64) and vmax (f32) [B, H, chunks, D] are
 * scratch. */
typedef struct attn_quant_layout {
    size_t workspace_bytes;
    size_t off_mk, off_sv, off_sq, off_sk, off_qi, off_ki, off_vt, off_ksum, off_vmax;
    int32_t blocks;       /* ceil(N / 64) */
    int32_t chunks;       /* ceil(N / 256) */
    int32_t vt_stride;    /* blocks * 64 */
} attn_quant_layout;

/* Workspace size and layout for these sizes (host only; no GPU needed).
 * Returns ATTN_OK or a validation error (head_dim != 128 is UNSUPPORTED). */
int attn_quant_layout_of(const attn_quant_dims *dims, attn_quant_layout *layout);

/* Steps 1-3: q, k, v bf16 device tensors (strides in dims) -> workspace. */
int attn_quant_prep(const void *q, const void *k, const void *v, const attn_quant_dims *dims,
                    void *workspace, size_t workspace_bytes, void *stream);

/* Step 4 from a workspace filled by attn_quant_prep: out bf16 [B, N, H, D]
 * (o_stride).  scale: finite; causal: nonzero = query i sees keys 0..i. */
int attn_quant_attend(void *out, const attn_quant_dims *dims, float scale, int32_t causal,
                      const void *workspace, size_t workspace_bytes, void *stream);

/* Steps 1-4 in one call (all arguments validated before anything launches). */
int attn_quant_fwd(void *out, const void *q, const void *k, const void *v,
                   const attn_quant_dims *dims, float scale, int32_t causal, void *workspace,
                   size_t workspace_bytes, void *stream);

/*
 * Kernel timing (instrumentation for benchmarks).  While enabled, every
 * launch is bracketed by HIP events recorded on the launch stream; elapsed
 * times are summed per kind: the main attention kernel (split-KV partials,
 * prefill or the quantised loop), the split-KV combine kernel, the other
 * work before the main kernel (the quantised path's preparation kernels,
 * the prefill launch-order sort, the fp8 page staging) and the KV-cache
 * write kernel (none when the write runs inside the split-decode launch).
 * attn_kernel_timing_read
 * synchronises on the recorded events, returns the totals (milliseconds)
 * and launch counts (any pointer may be NULL), and resets them.  Returns
 * ATTN_ERR_HIP if an event call fails.
 */
int attn_kernel_timing_enable(int32_t enable);
int attn_kernel_timing_read(double *main_ms, int32_t *main_launches, double *combine_ms,
                            int32_t *combine_launches, double *prep_ms, int32_t *prep_launches,
                            double *write_ms, int32_t *write_launches);

/*
 * attn_stream_read -- measurement utility: read `bytes` of device memory at
 * `buf` once with 16-byte non-temporal loads (grid-stride loop, `grid`
 * workgroups of 256 threads, `depth` = 4 or 8 loads in flight per thread)
 * and nothing else, asynchronously on `stream`.  The best rate over a few
 * grid sizes and depths is the on-box ceiling of a plain HBM read stream,
 * the practical denominator beside the 8 TB/s peak for the HBM-bound
 * attention kernels.  sink: device uint32 [grid * 256], overwritten (each
 * thread's XOR of what it read, so no load can be elided).  buf 16-byte
 * aligned, bytes a multiple of 16, 1 <= grid <= 65535; errors:
 * ATTN_ERR_NULL, ATTN_ERR_ALIGN, ATTN_ERR_SHAPE, ATTN_ERR_HIP.  Caller-owned
 * memory; nothing is allocated.
 */
int attn_stream_read(const void *buf, size_t bytes, uint32_t *sink, int32_t grid, int32_t depth, void *stream);

/* Human-readable text of a status code (static storage; never NULL). */
const char *attn_status_string(int status);

/* Library version as major * 10000 + minor * 100 + patch. */
int attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_ATTN_H */
