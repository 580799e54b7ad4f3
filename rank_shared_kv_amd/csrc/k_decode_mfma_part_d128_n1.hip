// Instances of the bf16 MFMA split kernel for d_h = 128, normalised variant (all H, r, occupancies).
#include "k_decode_mfma.hpp"

namespace lrkv {

hipError_t launch_split_mfma_d128_n1(const DecodeArgs& a, int occupancy, hipStream_t stream) {
    return launch_h<128, true>(a, occupancy, stream);
}

}  // namespace lrkv
