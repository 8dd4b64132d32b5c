// Launchers of the split-decode kernels (bf16 cache at both head dims, fp8
// cache at head_dim 128) and the log-sum-exp combine kernel.  The kernels
// themselves are in decode_kernels.h.
#include <algorithm>

#include "decode_kernels.h"

namespace pa {

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
    // The row's metadata loads are independent of each other: issued together.
    const int q0 = a.cu_q[b];
    const int q1 = a.cu_q[b + 1];
    const int pieces = a.seg_splits ? a.seg_splits[b] : 0;
    int n = q1 - q0;
    if (n > a.max_q) n = a.max_q;
    if (i >= n) return;
    int ns;
    if (a.seg_splits) {
        // balanced split path: a sequence in one piece was written directly;
        // one with no page (L = 0) is written as zeros below
        ns = pieces;
        if (ns == 1) return;
    } else {
        const int L = a.seq_lens[b];
        ns = split_count((L + kPage - 1) / kPage, split_first_page(L, n, a.window), a.pages_per_split,
                         a.max_splits);
    }
    const int64_t t = q0 + i;
    const int64_t base = (((int64_t)b * a.max_q + i) * a.hq + h) * a.max_splits;

    // Lane s keeps split s's (m, l) for the first 64 splits, so the merge
    // below takes them from a register instead of a second global round trip.
    float m_l = -INFINITY, l_l = 0.f;
    if (lane < ns) {
        m_l = a.part_ml[(base + lane) * 2];
        l_l = a.part_ml[(base + lane) * 2 + 1];
    }
    float M = m_l;
    for (int s = lane + 64; s < ns; s += 64) M = fmaxf(M, a.part_ml[(base + s) * 2]);
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
        // Splits in order, each with the same arithmetic as before (the
        // single-launch merge uses it too, so both forms stay bitwise
        // equal); four splits' O loads are issued before their products.
        const int ns64 = ns < 64 ? ns : 64;
        int s = 0;
        for (; s + 4 <= ns64; s += 4) {
            float po4[4][PER];
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int e = 0; e < PER; ++e) po4[u][e] = a.part_o[(base + s + u) * D + lane + 64 * e];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const float ms = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, m_l), s + u));
                const float ls = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, l_l), s + u));
                const float wgt = exp2_fast(ms - M);   // ms = -inf gives 0
                lsum += wgt * ls;
#pragma unroll
                for (int e = 0; e < PER; ++e) acc[e] += wgt * po4[u][e];
            }
        }
        for (; s < ns; ++s) {
            float ms, ls;
            if (s < 64) {
                ms = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, m_l), s));
                ls = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, l_l), s));
            } else {
                ms = a.part_ml[(base + s) * 2];
                ls = a.part_ml[(base + s) * 2 + 1];
            }
            const float wgt = exp2_fast(ms - M);
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

// The fp8-cache kernels at head_dim 256 live in decode_f8_256.hip.
hipError_t launch_decode_split_f8_256(const AttnArgs &a, dim3 grid, hipStream_t stream);
hipError_t launch_decode_balanced_f8_256(const AttnArgs &a, dim3 grid, hipStream_t stream);

template <int D>
hipError_t launch_decode_split(const AttnArgs &a, dim3 grid, hipStream_t stream) {
    if (!a.kv_fp8) return launch_decode_split_w<D, false>(a, grid, stream);
    if constexpr (D == 256) return launch_decode_split_f8_256(a, grid, stream);
    else return launch_decode_split_w<D, true>(a, grid, stream);
}

template <int D>
hipError_t launch_decode_balanced(const AttnArgs &a, dim3 grid, hipStream_t stream) {
    if (!a.kv_fp8) return launch_decode_balanced_w<D, false>(a, grid, stream);
    if constexpr (D == 256) return launch_decode_balanced_f8_256(a, grid, stream);
    else return launch_decode_balanced_w<D, true>(a, grid, stream);
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

hipError_t launch_decode_balanced_any(int D, const AttnArgs &a, dim3 grid, hipStream_t stream) {
    return D == 128 ? launch_decode_balanced<128>(a, grid, stream) : launch_decode_balanced<256>(a, grid, stream);
}

hipError_t launch_combine_any(int D, const CombineArgs &a, hipStream_t stream) {
    return D == 128 ? launch_combine<128>(a, stream) : launch_combine<256>(a, stream);
}

}  // namespace pa
