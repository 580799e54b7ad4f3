// Dispatch of the bf16 MFMA split kernel (k_decode_mfma.hpp) over its
// per-(d_h, variant) instance sets, and the shapes it covers.
#include "lrkv_internal.hpp"

namespace lrkv {

hipError_t launch_split_mfma_d64_n0(const DecodeArgs& a, int occupancy, hipStream_t stream);
hipError_t launch_split_mfma_d64_n1(const DecodeArgs& a, int occupancy, hipStream_t stream);
hipError_t launch_split_mfma_d128_n0(const DecodeArgs& a, int occupancy, hipStream_t stream);
hipError_t launch_split_mfma_d128_n1(const DecodeArgs& a, int occupancy, hipStream_t stream);

namespace {
constexpr int kRows = 32;   // rows per block (k_decode_mfma.hpp)
constexpr int kWaves = 4;   // waves per workgroup
}  // namespace

bool mfma_path_supports(int H, int d_h, int r, int dtype, int L_cap) {
    if (dtype != 1) return false;
    // rows of a block never leave the allocation when L_cap is a multiple of 32; buffer offsets are 32-bit
    if (L_cap % kRows != 0) return false;
    if ((long long)L_cap * d_h * 2 >= (1LL << 31) || (long long)H * L_cap * r * 2 >= (1LL << 31)) return false;
    if (d_h != 64 && d_h != 128) return false;
    if (!(r == 0 || r == 8 || r == 16 || r == 32 || r == 48 || r == 64)) return false;
    return H == 8 || H == 16 || H == 32;
}

int mfma_rows_per_tile(int H) { return kRows * (kWaves / ((H + 15) / 16)); }

hipError_t launch_split_mfma(const DecodeArgs& a, int occupancy, hipStream_t stream) {
    const bool norm = a.rho != nullptr;
    if (a.d_h == 64) return norm ? launch_split_mfma_d64_n1(a, occupancy, stream) : launch_split_mfma_d64_n0(a, occupancy, stream);
    if (a.d_h == 128) return norm ? launch_split_mfma_d128_n1(a, occupancy, stream) : launch_split_mfma_d128_n0(a, occupancy, stream);
    return hipErrorInvalidValue;
}

}  // namespace lrkv
