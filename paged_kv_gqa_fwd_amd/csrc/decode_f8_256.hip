// The split-decode kernels over an fp8 cache at head_dim 256, in a
// translation unit of their own: it is built with vector-register MFMA
// accumulators, which fit these kernels in 256 registers so that two
// workgroups share a CU (the other instances keep the default form; the
// bf16 D = 256 kernel ran 0.7% slower in the vector form).
#include "decode_kernels.h"

namespace pa {

hipError_t launch_decode_split_f8_256(const AttnArgs &a, dim3 grid, hipStream_t stream) {
    return launch_decode_split_w<256, true>(a, grid, stream);
}

hipError_t launch_decode_balanced_f8_256(const AttnArgs &a, dim3 grid, hipStream_t stream) {
    return launch_decode_balanced_w<256, true>(a, grid, stream);
}

}  // namespace pa
