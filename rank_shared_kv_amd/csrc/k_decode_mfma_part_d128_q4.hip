// Instances of the bf16 MFMA split kernel for d_h = 128 serving 4 query tokens per workgroup (multi-token
// decode; all H and r, one wave per SIMD).
#include "k_decode_mfma.hpp"

namespace lrkv {

hipError_t launch_split_mfma_d128_q4(const DecodeArgs& a, hipStream_t stream) {
    return launch_h<128, false, 4>(a, 1, stream);
}

}  // namespace lrkv
