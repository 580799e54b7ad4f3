// MFMA split kernel for bf16 LRKV decode (gfx950).  Filled in below.
#include "lrkv_device.hpp"
#include "lrkv_internal.hpp"

namespace lrkv {

bool mfma_path_supports(int H, int d_h, int r, int dtype) { return false; }

hipError_t launch_split_mfma(const DecodeArgs& a, int waves, hipStream_t stream) { return hipErrorInvalidValue; }

}  // namespace lrkv
