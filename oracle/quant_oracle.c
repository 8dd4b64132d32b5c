/*
 * Oracle for quantised attention (int8 Q.K, fp8 P.V) -- TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow CPU reference of the quantised attention variant, emulating
 * every quantisation step.  Only the test suite and the benchmark's
 * CPU-baseline leg may load it; the product path never links, imports or
 * calls it, and it shares no code, header, table or helper with the HIP
 * kernels.
 *
 * Source: h3-blackwell-runtime benchmarks/gb10-sage2-block24-scheduler-baseline
 * .json (the SageAttention2 block-24 baseline on GB10): phase_timings names
 * the steps -- k_mean_and_smoothing_preparation, q_int8_quantization,
 * k_int8_subtract_mean_quantization, v_fp8_transpose_scale_quantization
 * (v_transpose_pad_permute + v_scale_fp8_quantization) -- and
 * fused_mainloop_phases lists int8_qk, scale_application, online_softmax,
 * pv_accumulation and final_normalization_and_output; the scheduler section
 * gives 64-key iterations (cta_k 64).  Q/K/V are dense [B, N, H, D] (q_shape,
 * k_shape, v_shape).
 *
 * What is computed, in the pages' order (the page names the steps only;
 * the readings below are the plainest ones that agree with them):
 *  1. K mean: mk[b,h,c] = (1/N) sum_j K[b,j,h,c], summed in fp64 (exact for
 *     bf16 inputs of ordinary range, so the order of summation does not
 *     matter), then rounded to f32.
 *  2. Smoothing: K'[j,c] = f32(K[j,c]) - mk[c] in f32.
 *  3. Per-block int8: for each (b, h) and 64-token block, s = amax / 127 in
 *     f32 (s = 1 when the block is all zero); code = clamp(rne(x * (1/s)),
 *     -127, 127) with 1/s and the product in f32.  Applied to Q and to K'.
 *  4. Per-channel fp8: s_v[b,h,c] = amax_j |V[b,j,h,c]| / 448 in f32 (1 when
 *     zero); code = e4m3(V * (1/s_v)) with 1/s_v and the product in f32,
 *     OCP E4M3 (bias 7, no infinities, largest finite 448), round to nearest
 *     even, saturating at 448.
 *  5. Scores: s_ij = (sum_d Qi_id Ki_jd, exact integer) * sq * sk * scale.
 *  6. Online softmax over 64-key tiles in ascending key order: the running
 *     max m takes the tile's max before the tile's weights are formed;
 *     w_j = exp(s_j - m) in (0, 1]; O and l are rescaled by exp(m_old - m).
 *  7. P.V: the weight enters the product as e4m3(448 w_j) (its fp8 code,
 *     decoded exactly) times the decoded V code; l sums the unquantised w_j.
 *     (quant_p = 0 skips the rounding of w: used to pin the rest against the
 *     plain attention oracle.)  Where this rounding happens is a reading:
 *     parity unpinned by the page, which names the fused steps but not
 *     their arithmetic.
 *  8. out = O * s_v / (448 l)  (or O * s_v / l when quant_p = 0), fp64.
 * Causal (square self-attention, n = N): query i sees keys [0, i].
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define QBLOCK 64   /* tokens per int8 scale block */
#define KTILE 64    /* keys per online-softmax tile */

static float bf16_to_f32(uint16_t bits)
{
    uint32_t u = ((uint32_t)bits) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Scale of a symmetric int8 block with largest magnitude amax (f32). */
static float int8_scale(float amax)
{
    return amax > 0.0f ? amax / 127.0f : 1.0f;
}

/* Round-to-nearest-even int8 code of x under inverse scale inv (f32). */
static int8_t int8_code(float x, float inv)
{
    float y = nearbyintf(x * inv);
    if (y > 127.0f) y = 127.0f;
    if (y < -127.0f) y = -127.0f;
    return (int8_t)y;
}

/* OCP E4M3 encoding of x: round to nearest even, saturate at +-448. */
uint8_t oracle_e4m3_encode(double x)
{
    if (isnan(x)) return 0x7F;
    const uint8_t sign = signbit(x) ? 0x80 : 0x00;
    const double a = fabs(x);
    int e;
    /* spacing of representable values around a: 2^-9 below the smallest
       normal 2^-6, else 2^(floor(log2 a) - 3) */
    double quantum;
    if (a < ldexp(1.0, -6)) {
        quantum = ldexp(1.0, -9);
    } else {
        frexp(a, &e);
        quantum = ldexp(1.0, (e - 1) - 3);
    }
    double r = nearbyint(a / quantum) * quantum;
    if (r > 448.0) r = 448.0;
    if (r == 0.0) return sign;
    frexp(r, &e);
    const int ub = (e - 1) + 7; /* biased exponent */
    if (ub <= 0) {
        /* subnormal: r = m * 2^-9, m in 1..7 */
        return sign | (uint8_t)(r / ldexp(1.0, -9));
    }
    const int mant = (int)((r / ldexp(1.0, e - 1) - 1.0) * 8.0);
    return sign | (uint8_t)((ub << 3) | mant);
}

/* Codes of n f32 values (the encoder above, element by element). */
void oracle_e4m3_encode_array(const float *x, uint8_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_e4m3_encode((double)x[i]);
}

double oracle_e4m3_decode(uint8_t c)
{
    const int s = c >> 7, ub = (c >> 3) & 15, m = c & 7;
    if (ub == 15 && m == 7) return NAN;
    double v = ub == 0 ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, ub - 7);
    return s ? -v : v;
}

static int64_t idx4(int64_t b, int64_t j, int64_t h, int64_t c, int N, int H, int D)
{
    return ((b * N + j) * H + h) * D + c;
}

/*
 * Steps 1-4.  Inputs bf16 [B, N, H, D] contiguous.  Outputs (logical layouts):
 *   mk  f32 [B, H, D]          qi, ki int8 [B, N, H, D]
 *   sq, sk f32 [B, H, NB] with NB = ceil(N / 64)
 *   vq  uint8 [B, H, D, N] (e4m3 codes, channel-major)    sv f32 [B, H, D]
 */
int oracle_quant_prep(const uint16_t *q, const uint16_t *k, const uint16_t *v, int B, int N, int H,
                      int D, float *mk, int8_t *qi, float *sq, int8_t *ki, float *sk, uint8_t *vq,
                      float *sv, int nthreads)
{
    if (B <= 0 || N <= 0 || H <= 0 || D <= 0) return -1;
    const int NB = (N + QBLOCK - 1) / QBLOCK;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int b = 0; b < B; ++b) {
        for (int h = 0; h < H; ++h) {
            /* 1. K mean over tokens, per channel */
            for (int c = 0; c < D; ++c) {
                double sum = 0.0;
                for (int j = 0; j < N; ++j) sum += (double)bf16_to_f32(k[idx4(b, j, h, c, N, H, D)]);
                mk[((int64_t)b * H + h) * D + c] = (float)(sum / (double)N);
            }
            /* 2-3. per-block int8 of Q and of K - mk */
            for (int blk = 0; blk < NB; ++blk) {
                const int j0 = blk * QBLOCK, j1 = j0 + QBLOCK < N ? j0 + QBLOCK : N;
                float aq = 0.0f, ak = 0.0f;
                for (int j = j0; j < j1; ++j)
                    for (int c = 0; c < D; ++c) {
                        const float xq = fabsf(bf16_to_f32(q[idx4(b, j, h, c, N, H, D)]));
                        const float xk = fabsf(bf16_to_f32(k[idx4(b, j, h, c, N, H, D)]) -
                                               mk[((int64_t)b * H + h) * D + c]);
                        if (xq > aq) aq = xq;
                        if (xk > ak) ak = xk;
                    }
                const float sq_ = int8_scale(aq), sk_ = int8_scale(ak);
                const float iq = 1.0f / sq_, ik = 1.0f / sk_;
                sq[((int64_t)b * H + h) * NB + blk] = sq_;
                sk[((int64_t)b * H + h) * NB + blk] = sk_;
                for (int j = j0; j < j1; ++j)
                    for (int c = 0; c < D; ++c) {
                        const int64_t i = idx4(b, j, h, c, N, H, D);
                        qi[i] = int8_code(bf16_to_f32(q[i]), iq);
                        ki[i] = int8_code(bf16_to_f32(k[i]) - mk[((int64_t)b * H + h) * D + c], ik);
                    }
            }
            /* 4. per-channel fp8 of V */
            for (int c = 0; c < D; ++c) {
                float a = 0.0f;
                for (int j = 0; j < N; ++j) {
                    const float x = fabsf(bf16_to_f32(v[idx4(b, j, h, c, N, H, D)]));
                    if (x > a) a = x;
                }
                const float s = a > 0.0f ? a / 448.0f : 1.0f;
                const float inv = 1.0f / s;
                sv[((int64_t)b * H + h) * D + c] = s;
                uint8_t *dst = vq + (((int64_t)b * H + h) * D + c) * N;
                for (int j = 0; j < N; ++j) dst[j] = oracle_e4m3_encode((double)(bf16_to_f32(v[idx4(b, j, h, c, N, H, D)]) * inv));
            }
        }
    }
    return 0;
}

/*
 * Steps 5-8 from the prep outputs.  out fp64 [B, N, H, D].  row_mask
 * (optional, uint8 [N]) restricts the computed query tokens.
 */
int oracle_quant_attn(const int8_t *qi, const float *sq, const int8_t *ki, const float *sk,
                      const uint8_t *vq, const float *sv, int B, int N, int H, int D, double scale,
                      int causal, int quant_p, const uint8_t *row_mask, double *out, int nthreads)
{
    if (B <= 0 || N <= 0 || H <= 0 || D <= 0) return -1;
    const int NB = (N + QBLOCK - 1) / QBLOCK;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    int status = 0;
#pragma omp parallel
    {
        double *vdec = (double *)malloc(sizeof(double) * 256);   /* fp8 decode table */
        double *o = (double *)malloc(sizeof(double) * (size_t)D);
        double *s = (double *)malloc(sizeof(double) * KTILE);
        if (!vdec || !o || !s) {
#pragma omp atomic write
            status = -2;
        } else {
            for (int c = 0; c < 256; ++c) vdec[c] = oracle_e4m3_decode((uint8_t)c);
#pragma omp for collapse(3) schedule(dynamic, 4)
            for (int b = 0; b < B; ++b)
                for (int h = 0; h < H; ++h)
                    for (int i = 0; i < N; ++i) {
                        if (row_mask && !row_mask[i]) continue;
                        const int vis = causal ? i + 1 : N;
                        const int8_t *qrow = qi + idx4(b, i, h, 0, N, H, D);
                        const double qs = (double)sq[((int64_t)b * H + h) * NB + i / QBLOCK];
                        double m = -INFINITY, l = 0.0;
                        for (int c = 0; c < D; ++c) o[c] = 0.0;
                        for (int t0 = 0; t0 < vis; t0 += KTILE) {
                            const int t1 = t0 + KTILE < vis ? t0 + KTILE : vis;
                            double mt = -INFINITY;
                            for (int j = t0; j < t1; ++j) {
                                const int8_t *krow = ki + idx4(b, j, h, 0, N, H, D);
                                int64_t dot = 0;
                                for (int c = 0; c < D; ++c) dot += (int64_t)qrow[c] * (int64_t)krow[c];
                                s[j - t0] = (double)dot * qs *
                                            (double)sk[((int64_t)b * H + h) * NB + j / QBLOCK] * scale;
                                if (s[j - t0] > mt) mt = s[j - t0];
                            }
                            const double mn = mt > m ? mt : m;
                            const double alpha = (m == -INFINITY) ? 0.0 : exp(m - mn);
                            l *= alpha;
                            for (int c = 0; c < D; ++c) o[c] *= alpha;
                            m = mn;
                            for (int j = t0; j < t1; ++j) {
                                const double w = exp(s[j - t0] - m);
                                l += w;
                                const double pw = quant_p ? vdec[oracle_e4m3_encode(448.0 * w)] : w;
                                for (int c = 0; c < D; ++c)
                                    o[c] += pw * vdec[vq[(((int64_t)b * H + h) * D + c) * N + j]];
                            }
                        }
                        double *dst = out + idx4(b, i, h, 0, N, H, D);
                        const double denom = quant_p ? 448.0 * l : l;
                        for (int c = 0; c < D; ++c)
                            dst[c] = l > 0.0 ? o[c] * (double)sv[((int64_t)b * H + h) * D + c] / denom : 0.0;
                    }
        }
        free(vdec);
        free(o);
        free(s);
    }
    return status;
}
