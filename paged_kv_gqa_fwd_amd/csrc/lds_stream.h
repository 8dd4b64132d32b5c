// Device helpers shared by the LDS-streaming kernels (prefill and the
// quantised loop): wave-half exchanges, direct HBM -> LDS loads and scalar
// block-table reads.  Internal to the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

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

// Page id j of a block-table row, read through the scalar cache (the id is
// uniform across the workgroup).
__device__ __forceinline__ int load_page_id(const int32_t *bt_row, int j) {
    typedef __attribute__((address_space(4))) const int32_t const_i32;
    return *((const_i32 *)bt_row + j);
}

}  // namespace pa
