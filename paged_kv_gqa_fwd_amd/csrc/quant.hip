// Quantised attention (gfx950): K-mean smoothing, per-block int8 Q and K,
// per-channel fp8 (e4m3) V, and the fused int8 Q.K / fp8 P.V attention loop.
//
// What is computed follows the SageAttention2 block-24 baseline page
// (h3-blackwell-runtime benchmarks/gb10-sage2-block24-scheduler-baseline
// .json): phase_timings names the preparation steps (K mean for smoothing,
// Q int8, K-minus-mean int8, V transpose / pad / permute and per-channel fp8
// scaling) and fused_mainloop_phases the fused loop (int8 Q.K, scale
// application, online softmax, P.V accumulation, final normalisation); the
// scheduler section iterates over 64-key tiles.  The arithmetic of each step
// (scales amax/127 and amax/448, round to nearest even, fp8 weights 448 w)
// is the plainest reading of those names.
//
// Design (MI355X):
//  * Statistics: one pass over K and V per (batch, head, 256-token chunk)
//    writes fp64 partial channel sums of K and f32 partial channel maxima of
//    |V|; a finalize kernel reduces the chunks in a fixed order.  fp64 sums
//    of bf16 values are exact for ordinary ranges, so the mean does not
//    depend on the reduction order.
//  * Q / K int8: one workgroup per (batch, head, 64-token block): block amax
//    in LDS, then codes written in the input's [B, N, H, D] order.
//  * V fp8: one workgroup per (batch, head, 64-token tile) scales, converts
//    (v_cvt_pk_fp8_f32) and transposes through LDS into V^T [B, H, D, Npad]
//    with the keys of each tile permuted so that every lane's P.V operand is
//    32 contiguous bytes (the permutation matches the score layout of the
//    Q.K MFMA, see quant_pos_of_key).
//  * Attention: 4 wave64 per (batch, head, 128-query tile), 32 rows per wave.
//    K (int8) and V^T (fp8) tiles stream HBM -> LDS with direct 16-byte loads
//    through a 3-stage ring, swizzled so the operand reads are bank-conflict
//    free.  S^T = K Q^T on v_mfma_i32_32x32x32_i8 (keys on M); dequantised
//    by one f32 factor per (row, tile); exact running max per tile; weights
//    448 w = exp2(s - m + log2 448) rounded to fp8 by v_cvt_pk_fp8_f32 and
//    used directly as the B operand of v_mfma_scale_f32_32x32x64_f8f6f4
//    (unit scales); l sums the unrounded 448 w.
#include "attn_device.h"
#include "quant_device.h"
#include "lds_stream.h"

namespace pa {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x16 __attribute__((ext_vector_type(16)));

// ---------------------------------------------------------------- statistics
// Grid (chunks, H, B), 256 threads.  Thread t owns channels 8 (t % 16) .. +7
// and tokens chunk*256 + t/16 + 16 i.
__global__ __launch_bounds__(256) void quant_stats_kernel(const QuantArgs a) {
    constexpr int D = kQuantD;
    __shared__ double s_sum[16][D];
    __shared__ float s_max[16][D];
    const int chunk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int t = threadIdx.x, cg = t % 16, rg = t / 16;
    double sum[8];
    float vmax[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        sum[e] = 0.0;
        vmax[e] = 0.f;
    }
    const int j0 = chunk * kQuantChunk;
    for (int i = 0; i < kQuantChunk / 16; ++i) {
        const int j = j0 + rg + 16 * i;
        if (j >= a.n) break;
        const u32x4 kv = *reinterpret_cast<const u32x4 *>(a.k + (int64_t)b * a.k_sb + (int64_t)j * a.k_st +
                                                         (int64_t)h * a.k_sh + 8 * cg);
        const u32x4 vv = *reinterpret_cast<const u32x4 *>(a.v + (int64_t)b * a.v_sb + (int64_t)j * a.v_st +
                                                         (int64_t)h * a.v_sh + 8 * cg);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint16_t kb = (uint16_t)(kv[e / 2] >> (16 * (e & 1)));
            const uint16_t vb = (uint16_t)(vv[e / 2] >> (16 * (e & 1)));
            sum[e] += (double)bf16_bits_to_f32(kb);
            vmax[e] = fmaxf(vmax[e], fabsf(bf16_bits_to_f32(vb)));
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        s_sum[rg][8 * cg + e] = sum[e];
        s_max[rg][8 * cg + e] = vmax[e];
    }
    __syncthreads();
    if (t < D) {
        double s = 0.0;
        float m = 0.f;
        for (int r = 0; r < 16; ++r) {
            s += s_sum[r][t];
            m = fmaxf(m, s_max[r][t]);
        }
        const int64_t o = (((int64_t)b * a.h + h) * a.chunks + chunk) * D + t;
        a.ksum_part[o] = s;
        a.vmax_part[o] = m;
    }
}

// Grid (H, B), D threads: reduce the chunk partials in chunk order.
__global__ __launch_bounds__(kQuantD) void quant_finalize_kernel(const QuantArgs a) {
    constexpr int D = kQuantD;
    const int h = blockIdx.x, b = blockIdx.y, c = threadIdx.x;
    const int64_t base = ((int64_t)b * a.h + h) * a.chunks * D + c;
    double s = 0.0;
    float m = 0.f;
    for (int ch = 0; ch < a.chunks; ++ch) {
        s += a.ksum_part[base + (int64_t)ch * D];
        m = fmaxf(m, a.vmax_part[base + (int64_t)ch * D]);
    }
    const int64_t o = ((int64_t)b * a.h + h) * D + c;
    a.mk[o] = (float)(s / (double)a.n);
    a.sv[o] = m > 0.f ? m / 448.0f : 1.0f;
}

// ---------------------------------------------------------------- Q / K int8
// Grid (blocks, H, 2B): z = 2b + which (0 = Q, 1 = K minus mean).  Thread t
// owns channels 8 (t % 16) .. +7 of tokens blk*64 + t/16 + 16 i, i < 4.
__global__ __launch_bounds__(256) void quant_qk_kernel(const QuantArgs a) {
    constexpr int D = kQuantD;
    __shared__ float s_red[4];
    const int blk = blockIdx.x, h = blockIdx.y, b = blockIdx.z >> 1, which = blockIdx.z & 1;
    const int t = threadIdx.x, cg = t % 16, rg = t / 16;
    const uint16_t *src = which ? a.k : a.q;
    const int64_t sb = which ? a.k_sb : a.q_sb, st = which ? a.k_st : a.q_st, sh = which ? a.k_sh : a.q_sh;
    float mean[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) mean[e] = which ? a.mk[((int64_t)b * a.h + h) * D + 8 * cg + e] : 0.f;
    float x[4][8];
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int j = blk * kQuantBlock + rg + 16 * i;
        u32x4 raw = {0u, 0u, 0u, 0u};
        if (j < a.n) raw = *reinterpret_cast<const u32x4 *>(src + (int64_t)b * sb + (int64_t)j * st + (int64_t)h * sh + 8 * cg);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float f = bf16_bits_to_f32((uint16_t)(raw[e / 2] >> (16 * (e & 1))));
            x[i][e] = j < a.n ? f - mean[e] : 0.f;
            amax = fmaxf(amax, fabsf(x[i][e]));
        }
    }
    // block amax: wave reduction, then across the four waves
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
    if ((t & 63) == 0) s_red[t >> 6] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
    const float scale = amax > 0.f ? amax / 127.0f : 1.0f;
    const float inv = 1.0f / scale;
    if (t == 0) (which ? a.sk : a.sq)[((int64_t)b * a.h + h) * a.blocks + blk] = scale;
    int8_t *dst = which ? a.ki : a.qi;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int j = blk * kQuantBlock + rg + 16 * i;
        if (j >= a.n) break;
        u32x2 packed = {0u, 0u};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float y = __builtin_rintf(x[i][e] * inv);
            y = fminf(fmaxf(y, -127.f), 127.f);
            packed[e / 4] |= ((uint32_t)(uint8_t)(int8_t)(int)y) << (8 * (e & 3));
        }
        *reinterpret_cast<u32x2 *>(dst + (((int64_t)b * a.n + j) * a.h + h) * D + 8 * cg) = packed;
    }
}

// ---------------------------------------------------------------- V fp8 (transposed)
// Grid (blocks, H, B), 256 threads: one 64-token tile.  Thread t converts
// channels 8 (t % 16) .. +7 of tokens t/16 + 16 i, i < 4, into LDS [c][pos]
// (pos = stored position of the token within the tile), then the tile is
// written as 128 rows of 64 bytes.  Tokens past N are stored as code 0.
__global__ __launch_bounds__(256) void quant_v_kernel(const QuantArgs a) {
    constexpr int D = kQuantD;
    __shared__ __attribute__((aligned(16))) uint8_t s_t[D][kQuantBlock];
    const int tile = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int t = threadIdx.x, cg = t % 16, rg = t / 16;
    float inv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) inv[e] = 1.0f / a.sv[((int64_t)b * a.h + h) * D + 8 * cg + e];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int key = rg + 16 * i;
        const int j = tile * kQuantBlock + key;
        u32x4 raw = {0u, 0u, 0u, 0u};
        if (j < a.n) raw = *reinterpret_cast<const u32x4 *>(a.v + (int64_t)b * a.v_sb + (int64_t)j * a.v_st + (int64_t)h * a.v_sh + 8 * cg);
        const int pos = quant_pos_of_key(key);
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
            const float f0 = bf16_bits_to_f32((uint16_t)(raw[e / 2])) * inv[e];
            const float f1 = bf16_bits_to_f32((uint16_t)(raw[e / 2] >> 16)) * inv[e + 1];
            const int pk = __builtin_amdgcn_cvt_pk_fp8_f32(f0, f1, 0, false);
            s_t[8 * cg + e][pos] = (uint8_t)(pk & 0xFF);
            s_t[8 * cg + e + 1][pos] = (uint8_t)((pk >> 8) & 0xFF);
        }
    }
    __syncthreads();
    // 128 rows x 64 bytes = 512 chunks of 16 bytes: two per thread
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int c16 = t + 256 * r;
        const int d = c16 / 4, part = c16 % 4;
        const u32x4 val = *reinterpret_cast<const u32x4 *>(&s_t[d][16 * part]);
        *reinterpret_cast<u32x4 *>(a.vt + (((int64_t)b * a.h + h) * D + d) * a.vt_stride + tile * kQuantBlock + 16 * part) = val;
    }
}

// ---------------------------------------------------------------- attention
// Wave-uniform f32 read through the scalar cache.
__device__ __forceinline__ float load_scalar_f32(const float *p) {
    typedef __attribute__((address_space(4))) const float const_f32;
    return *(const_f32 *)p;
}

constexpr int kQStages = 3;
constexpr int kQRows = 128;   // query rows per workgroup (4 waves x 32)
constexpr int kQXcdRun = 64;  // consecutive grid items per XCD (its resident workgroups)

__global__ __launch_bounds__(256, 2) void quant_attn_kernel(const QuantArgs a) {
    constexpr int D = kQuantD;
    constexpr int TB = kQuantBlock * D;   // bytes of one K (or V^T) tile
    __shared__ __attribute__((aligned(1024))) uint8_t sk[kQStages][TB];
    __shared__ __attribute__((aligned(1024))) uint8_t sv[kQStages][TB];

    int bx = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    {
        // Workgroups are dealt to the 8 XCDs in turn by linear id; in each
        // full run of 8 QXCD ids, XCD c takes QXCD consecutive grid items
        // (query tiles of one head), so an XCD's L2 serves one head at a time.
        const int gx = (int)gridDim.x, gy = (int)gridDim.y;
        const int n = gx * gy * (int)gridDim.z;
        const int lin = (int)blockIdx.x + gx * ((int)blockIdx.y + gy * (int)blockIdx.z);
        if (lin < n - n % (8 * kQXcdRun)) {
            const int w8 = lin % (8 * kQXcdRun);
            const int item = lin - w8 + (w8 % 8) * kQXcdRun + w8 / 8;
            bx = item % gx;
            h = (item / gx) % gy;
            b = item / (gx * gy);
        }
    }
    const int qt = gridDim.x - 1 - bx;   // later query tiles first (longer under causal)
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hi = lane >> 5;
    const int N = a.n;
    const int r0 = qt * kQRows;
    const int row = r0 + 32 * w + (lane & 31);   // this lane's query token
    const bool row_ok = row < N;
    const int vis = row_ok ? (a.causal ? row + 1 : N) : 0;
    const int last_row = min(N, r0 + kQRows) - 1;
    const int kv_end = a.causal ? last_row + 1 : N;
    const int ntiles = (kv_end + kQuantBlock - 1) / kQuantBlock;
    const int w_full = a.causal ? min(N, r0 + 32 * w + 1) : N;   // keys below it are visible to all of the wave's rows

    // Q codes (B operand of the int8 MFMA): lane holds row `row`,
    // d = 32 ks + 16 hi .. +15 for ks < 4.
    // A negative scale is applied by negating the Q codes (exact for
    // -127..127), so the kernel's scale factor is always positive.
    i32x4 qreg[D / 32];
    {
        typedef signed char i8x16 __attribute__((ext_vector_type(16)));
        const int qrow = row_ok ? row : 0;
        const int8_t *qp = a.qi + (((int64_t)b * N + qrow) * a.h + h) * D + 16 * hi;
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks) {
            i8x16 v = *reinterpret_cast<const i8x16 *>(qp + 32 * ks);
            if (a.q_negate) v = -v;
            qreg[ks] = row_ok ? __builtin_bit_cast(i32x4, v) : i32x4{0, 0, 0, 0};
        }
    }
    const float qscale = a.sq[((int64_t)b * a.h + h) * a.blocks + (row_ok ? row : 0) / kQuantBlock];

    // per-thread DMA offsets: K tile chunk p = i*256 + tid (16-byte units,
    // 8 per key row): key p/8, physical chunk p%8, logical chunk ^ ((key>>1) & 7).
    // V^T tile: row d = p/4, physical chunk p%4, logical chunk ^ ((d>>2)&3).
    // With 64 four-byte banks (256 bytes per LDS cycle) the sixteen lanes of
    // one b128 read cycle then hit sixteen distinct 16-byte bank groups.
    uint32_t koff[2], voff[2];
    int kkey[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int p = i * 256 + tid;
        const int key = p / 8, ck = (p % 8) ^ ((key >> 1) & 7);
        kkey[i] = key;
        koff[i] = (uint32_t)(key * a.h * D + ck * 16);
        const int d = p / 4, cv = (p % 4) ^ ((d >> 2) & 3);
        voff[i] = (uint32_t)(d * a.vt_stride + cv * 16);
    }
    const int8_t *kbase = a.ki + ((int64_t)b * N * a.h + h) * D;
    const uint8_t *vbase = a.vt + ((int64_t)b * a.h + h) * D * (int64_t)a.vt_stride;
    auto issue_tile = [&](int t) {
        const int st = t % kQStages;
        const int valid = N - t * kQuantBlock;
        const int8_t *kt = kbase + (int64_t)t * kQuantBlock * a.h * D;
        const uint8_t *vt = vbase + t * kQuantBlock;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int slot = (i * 256 + w * 64) * 16;
            // keys past the end re-read key 0 of the tile (always valid)
            const uint32_t ko = kkey[i] < valid ? koff[i] : koff[i] - (uint32_t)(kkey[i] * a.h * D);
            dma16(lds_address(&sk[st][slot]), kt, ko);
            dma16(lds_address(&sv[st][slot]), vt, voff[i]);
        }
    };
    int issued = -1;
    auto wait_tile = [&](int t) {
        const int younger = issued - t;
        if (younger >= 2)
            asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
        else if (younger == 1)
            asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
        else
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    };
#pragma unroll
    for (int t = 0; t < kQStages - 1; ++t)
        if (t < ntiles) {
            issue_tile(t);
            issued = t;
        }

    f32x16 oacc[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) oacc[db] = f32x16{};
    float m_run = -INFINITY, l_part = 0.f;
    const float fbase = a.scale_log2_pos * qscale;   // times the key block's scale
    const float log2_448 = 8.807354922057604f;

    // operand offsets
    const int klane = (lane & 31) * D;
    const int kswz = ((lane & 31) >> 1) & 7;
    const int vrow = (lane & 31);
    const int vswz = (vrow >> 2) & 3;

    for (int t = 0; t < ntiles; ++t) {
        const int st = t % kQStages;
        wait_tile(t);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        if (t + kQStages - 1 < ntiles) {
            issue_tile(t + kQStages - 1);
            issued = t + kQStages - 1;
        }
        // S^T = K Q^T: two 32-key blocks
        i32x16 sacc[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            sacc[kb] = i32x16{};
            const uint8_t *kp = &sk[st][0] + (32 * kb) * D + klane;
#pragma unroll
            for (int ks = 0; ks < D / 32; ++ks) {
                const i32x4 kop = *reinterpret_cast<const i32x4 *>(kp + ((2 * ks + hi) ^ kswz) * 16);
                sacc[kb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(kop, qreg[ks], sacc[kb], 0, 0, 0);
            }
        }
        // scores (raw, f32) with the mask; sacc[kb][i] is key 64t + 32kb + 8(i/4) + 4hi + i%4
        float sf[2][16];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) sf[kb][i] = (float)sacc[kb][i];
        // Only the diagonal and tail tiles need the mask: one wave-uniform
        // branch around the whole loop, so that the other tiles do not pay
        // for it (a per-element select costs three VALU instructions a score).
        if ((t + 1) * kQuantBlock > w_full) {
            const int lim = vis - (t * kQuantBlock + 4 * hi);   // key offset o is visible iff o < lim
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    sf[kb][i] = (32 * kb + 8 * (i >> 2) + (i & 3)) < lim ? sf[kb][i] : -INFINITY;
        }
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sf[kb][i]);
        mx = max_xor32(mx);
        const float f = fbase * load_scalar_f32(a.sk + ((int64_t)b * a.h + h) * a.blocks + t);
        const float mt = mx * f;   // -inf stays -inf (f > 0)
        const float m_new = fmaxf(m_run, mt);
        const float alpha = (m_new == -INFINITY) ? 1.f : exp2_fast(m_run - m_new);
        m_run = m_new;
        if (__any(alpha != 1.f)) {
            l_part *= alpha;
#pragma unroll
            for (int db = 0; db < D / 32; ++db) oacc[db] *= alpha;
        }
        const float c0 = log2_448 - ((m_new == -INFINITY) ? 0.f : m_new);
        // 448 w rounded to fp8: the B operand (32 keys of this lane's row)
        i32x8 pq;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 16; i += 4) {
                const float p0 = exp2_fast(fmaf(sf[kb][i], f, c0));
                const float p1 = exp2_fast(fmaf(sf[kb][i + 1], f, c0));
                const float p2 = exp2_fast(fmaf(sf[kb][i + 2], f, c0));
                const float p3 = exp2_fast(fmaf(sf[kb][i + 3], f, c0));
                l_part += (p0 + p1) + (p2 + p3);
                int word = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, 0, false);
                word = __builtin_amdgcn_cvt_pk_fp8_f32(p2, p3, word, true);
                pq[(16 * kb + i) / 4] = word;
            }
        // O^T += V^T P^T: V^T rows d = 32 db + lane % 32, stored positions 32 hi .. +31
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
            const uint8_t *vp = &sv[st][0] + (32 * db + vrow) * kQuantBlock;
            const i32x4 v0 = *reinterpret_cast<const i32x4 *>(vp + ((2 * hi) ^ vswz) * 16);
            const i32x4 v1 = *reinterpret_cast<const i32x4 *>(vp + ((2 * hi + 1) ^ vswz) * 16);
            const i32x8 vop = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
            oacc[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vop, pq, oacc[db], 0, 0, 0, 127, 0, 127);
        }
    }

    // out = O * s_v / (448 l) = O * s_v / l_part (l_part sums 448 w)
    const float l_row = sum_xor32(l_part);
    if (!row_ok) return;
    const float inv = l_row > 0.f ? 1.f / l_row : 0.f;
    const float *svp = a.sv + ((int64_t)b * a.h + h) * D;
    uint16_t *op = a.out + (int64_t)b * a.o_sb + (int64_t)row * a.o_st + (int64_t)h * a.o_sh;
    // lanes l and l + 32 hold the low and high four values of each group of
    // eight d: one permlane32 swap per pair of groups lets every lane store
    // 16 contiguous bytes (as in the prefill kernel's epilogue)
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
        uint32_t w[4][2];
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4) {
            const int d0 = 32 * db + 8 * c4 + 4 * hi;
            const f32x4 s4 = *reinterpret_cast<const f32x4 *>(svp + d0);
            w[c4][0] = (uint32_t)f32_to_bf16_bits(oacc[db][4 * c4 + 0] * s4[0] * inv) |
                       ((uint32_t)f32_to_bf16_bits(oacc[db][4 * c4 + 1] * s4[1] * inv) << 16);
            w[c4][1] = (uint32_t)f32_to_bf16_bits(oacc[db][4 * c4 + 2] * s4[2] * inv) |
                       ((uint32_t)f32_to_bf16_bits(oacc[db][4 * c4 + 3] * s4[3] * inv) << 16);
        }
#pragma unroll
        for (int cp = 0; cp < 2; ++cp) {
            const auto s0 = __builtin_amdgcn_permlane32_swap(w[2 * cp][0], w[2 * cp + 1][0], false, false);
            const auto s1 = __builtin_amdgcn_permlane32_swap(w[2 * cp][1], w[2 * cp + 1][1], false, false);
            *reinterpret_cast<u32x4 *>(op + 32 * db + 16 * cp + 8 * hi) =
                u32x4{(uint32_t)s0[0], (uint32_t)s1[0], (uint32_t)s0[1], (uint32_t)s1[1]};
        }
    }
}

hipError_t launch_quant_prep(const QuantArgs &a, hipStream_t stream) {
    hipLaunchKernelGGL(quant_stats_kernel, dim3(a.chunks, a.h, a.b), dim3(256), 0, stream, a);
    hipLaunchKernelGGL(quant_finalize_kernel, dim3(a.h, a.b), dim3(kQuantD), 0, stream, a);
    hipLaunchKernelGGL(quant_qk_kernel, dim3(a.blocks, a.h, 2 * a.b), dim3(256), 0, stream, a);
    hipLaunchKernelGGL(quant_v_kernel, dim3(a.blocks, a.h, a.b), dim3(256), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_quant_attn(const QuantArgs &a, hipStream_t stream) {
    const int qtiles = (a.n + kQRows - 1) / kQRows;
    hipLaunchKernelGGL(quant_attn_kernel, dim3(qtiles, a.h, a.b), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace pa
