// Instances of the bf16 MFMA split kernel for d_h = 64 in the fused decode step (all H, r, occupancies).
#include "k_decode_mfma.hpp"

namespace lrkv {

hipError_t launch_step_mfma_d64(const DecodeArgs& a, int occupancy, hipStream_t stream) {
    return launch_step_h<64>(a, occupancy, stream);
}

}  // namespace lrkv
