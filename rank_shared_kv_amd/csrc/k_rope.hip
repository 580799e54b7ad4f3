// Rotary position table of the rotary variant ("Low-Rank Key Value Attention |
// What a shared cache can preserve", sec. 8, "Full RoPE needs a stronger
// identity"; "Low-Rank Key Value Attention: Chinese reading notes", sec.
// 2.7): coordinate pair k = (2k, 2k + 1) of a row at position t turns by
// phi = t * theta_k, theta_k = base^(-2k / d_h).  The angle and its cosine
// and sine are computed in fp64 (t * theta_k reaches tens of thousands of
// radians at long context, where fp32 would lose the angle's low bits) and
// stored in fp32 as table[t][k] = (cos phi, sin phi).
#include "lrkv_device.hpp"
#include "lrkv_internal.hpp"

namespace lrkv {
namespace {

__global__ void __launch_bounds__(256) rope_table_kernel(int half_d, int n_pos, double base, float* __restrict__ table) {
    const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (size_t)n_pos * half_d) return;
    const int t = (int)(idx / half_d), k = (int)(idx - (size_t)t * half_d);
    const double theta = pow(base, -2.0 * (double)k / (double)(2 * half_d));
    const double phi = (double)t * theta;
    table[2 * idx] = (float)cos(phi);
    table[2 * idx + 1] = (float)sin(phi);
}

}  // namespace

hipError_t launch_rope_table(int d_h, int n_pos, float base, float* table, hipStream_t stream) {
    const size_t n = (size_t)n_pos * (d_h / 2);
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, d_h / 2, n_pos,
                       (double)base, table);
    return hipGetLastError();
}

}  // namespace lrkv
