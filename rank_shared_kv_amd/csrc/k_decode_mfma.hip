// Dispatch of the bf16 MFMA split kernel (k_decode_mfma.hpp) over its
// per-(d_h, variant) instance sets, and the shapes it covers.
#include "lrkv_internal.hpp"

namespace lrkv {

hipError_t launch_split_mfma_d64_n0(const DecodeArgs& a, int occupancy, hipStream_t stream);
hipError_t launch_split_mfma_d64_n1(const DecodeArgs& a, int occupancy, hipStream_t stream);
hipError_t launch_split_mfma_d128_n0(const DecodeArgs& a, int occupancy, hipStream_t stream);
hipError_t launch_split_mfma_d128_n1(const DecodeArgs& a, int occupancy, hipStream_t stream);
hipError_t launch_split_mfma_d64_q2(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_split_mfma_d64_q4(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_split_mfma_d128_q2(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_split_mfma_d128_q4(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_split_mfma_d128_t7(const DecodeArgs& a, int occupancy, hipStream_t stream);
hipError_t launch_step_mfma_d64(const DecodeArgs& a, int occupancy, hipStream_t stream);
hipError_t launch_step_mfma_d128(const DecodeArgs& a, int occupancy, hipStream_t stream);
bool mfma_table_shape(int H, int d_h, int r);

namespace {
constexpr int kRows = 32;   // rows per block (k_decode_mfma.hpp)
constexpr int kWaves = 4;   // waves per workgroup
}  // namespace

bool mfma_path_supports(int H, int d_h, int r, int dtype, int L_cap) {
    if (dtype != 1) return false;
    // rows of a block never leave the allocation when L_cap is a multiple of 32; buffer offsets are 32-bit
    if (L_cap % kRows != 0) return false;
    if ((long long)L_cap * d_h * 2 >= (1LL << 31) || (long long)H * L_cap * r * 2 >= (1LL << 31)) return false;
    if (mfma_table_shape(H, d_h, r)) return true;
    if (d_h != 64 && d_h != 128) return false;
    if (!(r == 0 || r == 8 || r == 16 || r == 32 || r == 48 || r == 64)) return false;
    return H == 8 || H == 16 || H == 32;
}

// the normalised-variant and several-query instances exist for the regular shapes only (the model table's
// shapes have plain and paged single-token decode)
bool mfma_all_variants(int H, int d_h, int r) { return !mfma_table_shape(H, d_h, r); }

int mfma_rows_per_tile(int H) { return kRows * (kWaves / ((H + 15) / 16)); }

// query tokens one workgroup can serve in multi-token decode: 4, except at d_h = 128 and r = 64, where four
// queries' accumulators do not fit the register file next to the load ring (k_decode_mfma.hpp)
int mfma_max_query_width(int H, int d_h, int r) { return (d_h == 128 && r == 64) ? 2 : 4; }

hipError_t launch_split_mfma(const DecodeArgs& a, int occupancy, hipStream_t stream) {
    if (a.qw == 2 || a.qw == 4) {  // several query tokens per workgroup (plain decode only, one wave per SIMD)
        if (a.rho != nullptr || a.block_table != nullptr) return hipErrorInvalidValue;
        if (a.d_h == 64) return a.qw == 2 ? launch_split_mfma_d64_q2(a, stream) : launch_split_mfma_d64_q4(a, stream);
        if (a.d_h == 128) return a.qw == 2 ? launch_split_mfma_d128_q2(a, stream) : launch_split_mfma_d128_q4(a, stream);
        return hipErrorInvalidValue;
    }
    if (a.qw != 1) return hipErrorInvalidValue;
    const bool norm = a.rho != nullptr;
    if (mfma_table_shape(a.H, a.d_h, a.r)) return norm ? hipErrorInvalidValue : launch_split_mfma_d128_t7(a, occupancy, stream);
    if (a.d_h == 64) return norm ? launch_split_mfma_d64_n1(a, occupancy, stream) : launch_split_mfma_d64_n0(a, occupancy, stream);
    if (a.d_h == 128) return norm ? launch_split_mfma_d128_n1(a, occupancy, stream) : launch_split_mfma_d128_n0(a, occupancy, stream);
    return hipErrorInvalidValue;
}

// Fused decode step: single query, plain contiguous cache, the regular shapes (the model-table ranks are outside
// the absorb's one-wave vector path, so their steps run as separate launches).
hipError_t launch_step_mfma(const DecodeArgs& a, int occupancy, hipStream_t stream) {
    if (a.qw != 1 || a.qgroup != 1 || a.rho != nullptr || a.block_table != nullptr || a.sync == nullptr ||
        mfma_table_shape(a.H, a.d_h, a.r))
        return hipErrorInvalidValue;
    if (a.d_h == 64) return launch_step_mfma_d64(a, occupancy, stream);
    if (a.d_h == 128) return launch_step_mfma_d128(a, occupancy, stream);
    return hipErrorInvalidValue;
}

}  // namespace lrkv
