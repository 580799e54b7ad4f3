// Instances of the bf16 MFMA split kernel for the head counts and ranks of the reading notes' model table
// ("Low-Rank Key Value Attention: Chinese reading notes", sec. 2.5, the ranks of Table 7 recomputed with
// Eq. (9)): d_h = 128 with (H, r) = (6, 46), (12, 51), (18, 55), (32, 54).  Heads fill 8-head octets only
// partly and a head's last latent lanes hold fewer coordinates; plain (and paged) single-token decode, both
// occupancies.
#include "k_decode_mfma.hpp"

namespace lrkv {

bool mfma_table_shape(int H, int d_h, int r) {
    return d_h == 128 && ((H == 6 && r == 46) || (H == 12 && r == 51) || (H == 18 && r == 55) || (H == 32 && r == 54));
}

hipError_t launch_split_mfma_d128_t7(const DecodeArgs& a, int occupancy, hipStream_t stream) {
    if (a.d_h != 128) return hipErrorInvalidValue;
    if (a.H == 6 && a.r == 46) return launch_dhr<128, 46, 6, false, 1>(a, occupancy, stream);
    if (a.H == 12 && a.r == 51) return launch_dhr<128, 51, 12, false, 1>(a, occupancy, stream);
    if (a.H == 18 && a.r == 55) return launch_dhr<128, 55, 18, false, 1>(a, occupancy, stream);
    if (a.H == 32 && a.r == 54) return launch_dhr<128, 54, 32, false, 1>(a, occupancy, stream);
    return hipErrorInvalidValue;
}

}  // namespace lrkv
