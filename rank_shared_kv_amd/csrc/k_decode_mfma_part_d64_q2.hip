// Instances of the bf16 MFMA split kernel for d_h = 64 serving 2 query tokens per workgroup (multi-token
// decode; all H and r, one wave per SIMD).
#include "k_decode_mfma.hpp"

namespace lrkv {

hipError_t launch_split_mfma_d64_q2(const DecodeArgs& a, hipStream_t stream) {
    return launch_h<64, false, 2>(a, 1, stream);
}

}  // namespace lrkv
