/*
 * Oracle for paged grouped-query attention -- TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow, fp64 CPU reference of what the GPU path computes.  Only the
 * test suite, the smoke check and the benchmark's CPU-baseline leg may load
 * this library; the product path never links, imports or calls it.  It shares
 * no code, header, table or helper with the HIP kernels.
 *
 * Sources (web pages, cited by title and section):
 *  - kern-kernels examples/decode.json (TRT-LLM-gen decode manifest):
 *      buffers q / out / kv / table / seq / cuq give the paged layout
 *      [pages, layer, slot, kv_head, {K,V}, head_dim]; programs.decode passes
 *      K and V as two byte offsets into the same kv buffer.
 *  - Mojo SM100MHA2Q API docs: "scaled dot-product attention over a KV cache",
 *      MaskType "causal or unmasked", group / fuse_gqa (several q heads share
 *      one KV head), ValidLengthType (ragged lengths), PartitionType (split-K).
 *  - metrale blueprint graph.json, node l3.attn.attend: paged decode
 *      attention with f32 scores, softmax and accumulation; node
 *      l3.attn.kv_write runs first, so the cache already holds the step's
 *      own tokens.
 *
 * What is computed (masked softmax attention, written out as its definition):
 *   for each sequence b, query token i (row t = cu_q[b] + i), q head h:
 *     n = cu_q[b+1] - cu_q[b], L = seq_lens[b], pos = L - n + i
 *     visible keys j in [0, vis), vis = causal ? clamp(pos + 1, 0, L) : L
 *     g = h / G (contiguous groups of G = Hq / Hkv q heads per KV head)
 *     K_j, V_j = pool rows of page block_table[b][j / P], slot j % P, head g
 *     s_j = scale * <q_t,h , K_j>
 *     out[t, h, :] = sum_j softmax(s)_j V_j,   lse = log sum_j exp(s_j)
 *   Rows with no visible key give out = 0 and lse = -inf.
 * Every bf16 input is widened exactly to fp64; nothing is rounded on output.
 *
 * Readings taken where the pages are silent (each one is listed in the
 * design notes): seq_lens counts the step's own tokens; causal alignment is
 * bottom-right (queries sit at the tail of the sequence); q head h uses KV
 * head h / G.
 *
 * Optional variants (oracle_paged_attn_ex):
 *  - attention sinks (Mojo SM100MHA2Q, SinkType: an optional pointer to
 *    attention-sink weights).  Reading: one logit per q head, in the units of
 *    the scaled scores, that joins the softmax normalisation and carries no
 *    value row:  out = sum_j e^{s_j} V_j / (e^{sink_h} + sum_j e^{s_j}),
 *    lse = log(e^{sink_h} + sum_j e^{s_j}).  A -inf sink changes nothing.
 *  - a sliding window (decode.json's parameter pack holds an INT32_MAX field,
 *    read as "window disabled").  Reading: with window W > 0 a query at
 *    position pos sees only keys j >= pos - W + 1 (besides the causal or
 *    length bound); W <= 0 means no window.
 *  - an fp8 KV cache (the Mojo SM100MHA2Q docs carry fp8 branches of the KV
 *    dtype): pool elements are OCP e4m3 codes with one scale for K and one
 *    for V, K_j = k_scale * e4m3(code), V_j = v_scale * e4m3(code), decoded
 *    exactly to fp64 by this oracle's own decoder (quant_oracle.c).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

double oracle_e4m3_decode(uint8_t c);   /* quant_oracle.c */

static double bf16_bits_to_f64(uint16_t bits)
{
    uint32_t u = ((uint32_t)bits) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

typedef struct {
    const uint16_t *q;
    int64_t q_stride_token, q_stride_head;
    const uint16_t *pool;
    int64_t s_page, s_slot, s_head, s_kv;
    const int32_t *block_table;
    int64_t bt_stride;
    int hq, hkv, d, page_size;
    double scale;
    int kv_fp8;                 /* pool elements: 0 = bf16, 1 = e4m3 codes */
    double k_scale, v_scale;    /* fp8 pool only */
} oracle_ctx;

/* Key (which = 0) or value (which = 1) row j of sequence b, KV head g,
   widened to fp64 into row[0 .. d). */
static void kv_row(const oracle_ctx *c, int b, int64_t j, int g, int which, double *row)
{
    int64_t page = c->block_table[(int64_t)b * c->bt_stride + j / c->page_size];
    int64_t slot = j % c->page_size;
    int64_t off = page * c->s_page + slot * c->s_slot + (int64_t)g * c->s_head + (int64_t)which * c->s_kv;
    if (!c->kv_fp8) {
        const uint16_t *p = c->pool + off;
        for (int e = 0; e < c->d; ++e) row[e] = bf16_bits_to_f64(p[e]);
    } else {
        const uint8_t *p = (const uint8_t *)c->pool + off;   /* strides count bytes */
        const double sc = which ? c->v_scale : c->k_scale;
        for (int e = 0; e < c->d; ++e) row[e] = sc * oracle_e4m3_decode(p[e]);
    }
}

/*
 * Attention of one (query token t of sequence b, q head h) over keys [j0, j1).
 * Returns the partial triple (m, l, o[]) with o unnormalised:
 *   m = max_j s_j, l = sum_j exp(s_j - m), o = sum_j exp(s_j - m) V_j.
 * An empty range gives m = -inf, l = 0, o = 0.
 */
static void attend_range(const oracle_ctx *c, int b, int64_t t, int h, int64_t j0, int64_t j1,
                         double *scores, double *m_out, double *l_out, double *o, double *row)
{
    const int d = c->d;
    const int g = h / (c->hq / c->hkv);
    const uint16_t *qrow = c->q + t * c->q_stride_token + (int64_t)h * c->q_stride_head;
    for (int e = 0; e < d; ++e) o[e] = 0.0;
    if (j1 <= j0) {
        *m_out = -INFINITY;
        *l_out = 0.0;
        return;
    }
    double m = -INFINITY;
    for (int64_t j = j0; j < j1; ++j) {
        kv_row(c, b, j, g, 0, row);
        double dot = 0.0;
        for (int e = 0; e < d; ++e) dot += bf16_bits_to_f64(qrow[e]) * row[e];
        double s = c->scale * dot;
        scores[j - j0] = s;
        if (s > m) m = s;
    }
    double l = 0.0;
    for (int64_t j = j0; j < j1; ++j) {
        double w = exp(scores[j - j0] - m);
        l += w;
        kv_row(c, b, j, g, 1, row);
        for (int e = 0; e < d; ++e) o[e] += w * row[e];
    }
    *m_out = m;
    *l_out = l;
}

/* Number of keys visible to query i of a sequence with n queries and L keys. */
static int64_t visible_keys(int64_t L, int64_t n, int64_t i, int causal)
{
    if (!causal) return L;
    int64_t vis = L - n + i + 1;
    if (vis < 0) vis = 0;
    if (vis > L) vis = L;
    return vis;
}

/*
 * out  : fp64 [num_tokens, hq, d] (rows outside [0, cu_q[n_seqs]) untouched)
 * sinks: fp64 [hq] sink logits, or NULL;  window: W > 0, or <= 0 for none
 * lse  : fp64 [num_tokens, hq] natural-log log-sum-exp, or NULL
 * row_mask : optional uint8 [num_tokens]; when given only rows with a nonzero
 *            entry are computed (sampled checks at large sizes)
 * n_chunks : 0 = single pass; otherwise the visible key range of every row is
 *            cut into chunks at the boundaries given by chunk_keys (keys per
 *            chunk, > 0) and the partial triples are merged by the
 *            log-sum-exp rule -- the split-KV reading, used for the
 *            "split + combine equals one pass" invariant.
 */
int oracle_paged_attn_ex(double *out, double *lse, const uint16_t *q, int64_t q_stride_token,
                         int64_t q_stride_head, const uint16_t *pool, int64_t s_page, int64_t s_slot,
                         int64_t s_head, int64_t s_kv, const int32_t *block_table, int64_t bt_stride,
                         const int32_t *seq_lens, const int32_t *cu_q, int n_seqs, int hq, int hkv,
                         int d, int page_size, double scale, int causal, const uint8_t *row_mask,
                         int64_t chunk_keys, int nthreads, const double *sinks, int64_t window,
                         int kv_fp8, double k_scale, double v_scale)
{
    if (hkv <= 0 || hq % hkv != 0 || d <= 0 || page_size <= 0 || n_seqs < 0) return -1;
    oracle_ctx c = {q, q_stride_token, q_stride_head, pool, s_page, s_slot, s_head, s_kv,
                    block_table, bt_stride, hq, hkv, d, page_size, scale, kv_fp8, k_scale, v_scale};
    int64_t max_l = 0;
    for (int b = 0; b < n_seqs; ++b)
        if (seq_lens[b] > max_l) max_l = seq_lens[b];
    const int64_t total = cu_q[n_seqs];
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    int status = 0;
#pragma omp parallel
    {
        double *scores = (double *)malloc(sizeof(double) * (size_t)(max_l > 0 ? max_l : 1));
        double *acc = (double *)malloc(sizeof(double) * (size_t)d);
        double *part = (double *)malloc(sizeof(double) * (size_t)d);
        double *row = (double *)malloc(sizeof(double) * (size_t)d);
        if (!scores || !acc || !part || !row) {
#pragma omp atomic write
            status = -2;
        } else {
#pragma omp for schedule(dynamic, 1) collapse(2)
            for (int64_t t = 0; t < total; ++t) {
                for (int h = 0; h < hq; ++h) {
                    if (row_mask && !row_mask[t]) continue;
                    int b = 0;
                    while (b + 1 <= n_seqs && cu_q[b + 1] <= t) ++b;
                    const int64_t n = cu_q[b + 1] - cu_q[b];
                    const int64_t i = t - cu_q[b];
                    const int64_t L = seq_lens[b];
                    const int64_t vis = visible_keys(L, n, i, causal);
                    int64_t lo = 0;                       /* first key inside the window */
                    if (window > 0) {
                        lo = L - n + i - window + 1;
                        if (lo < 0) lo = 0;
                    }
                    double *dst = out + (t * hq + h) * (int64_t)d;
                    double m = -INFINITY, l = 0.0;
                    if (chunk_keys <= 0) {
                        attend_range(&c, b, t, h, lo, vis, scores, &m, &l, acc, row);
                    } else {
                        /* merge partial triples chunk by chunk (log-sum-exp rule) */
                        for (int e = 0; e < d; ++e) acc[e] = 0.0;
                        for (int64_t j0 = lo; j0 < vis; j0 += chunk_keys) {
                            int64_t j1 = j0 + chunk_keys < vis ? j0 + chunk_keys : vis;
                            double ms, ls;
                            attend_range(&c, b, t, h, j0, j1, scores, &ms, &ls, part, row);
                            double mn = ms > m ? ms : m;
                            double a_old = (m == -INFINITY) ? 0.0 : exp(m - mn);
                            double a_new = (ms == -INFINITY) ? 0.0 : exp(ms - mn);
                            l = l * a_old + ls * a_new;
                            for (int e = 0; e < d; ++e) acc[e] = acc[e] * a_old + part[e] * a_new;
                            m = mn;
                        }
                    }
                    if (sinks && sinks[h] != -INFINITY) {
                        /* the sink joins the normalisation with no value row */
                        const double sk = sinks[h];
                        const double mn = sk > m ? sk : m;
                        const double a = (m == -INFINITY) ? 0.0 : exp(m - mn);
                        l = l * a + exp(sk - mn);
                        for (int e = 0; e < d; ++e) acc[e] *= a;
                        m = mn;
                    }
                    if (l > 0.0) {
                        for (int e = 0; e < d; ++e) dst[e] = acc[e] / l;
                        if (lse) lse[t * hq + h] = m + log(l);
                    } else {
                        for (int e = 0; e < d; ++e) dst[e] = 0.0;
                        if (lse) lse[t * hq + h] = -INFINITY;
                    }
                }
            }
        }
        free(scores);
        free(acc);
        free(part);
        free(row);
    }
    return status;
}

int oracle_paged_attn(double *out, double *lse, const uint16_t *q, int64_t q_stride_token,
                      int64_t q_stride_head, const uint16_t *pool, int64_t s_page, int64_t s_slot,
                      int64_t s_head, int64_t s_kv, const int32_t *block_table, int64_t bt_stride,
                      const int32_t *seq_lens, const int32_t *cu_q, int n_seqs, int hq, int hkv,
                      int d, int page_size, double scale, int causal, const uint8_t *row_mask,
                      int64_t chunk_keys, int nthreads)
{
    return oracle_paged_attn_ex(out, lse, q, q_stride_token, q_stride_head, pool, s_page, s_slot, s_head,
                                s_kv, block_table, bt_stride, seq_lens, cu_q, n_seqs, hq, hkv, d, page_size,
                                scale, causal, row_mask, chunk_keys, nthreads, NULL, 0, 0, 1.0, 1.0);
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
