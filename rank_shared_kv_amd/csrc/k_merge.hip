// Split merge and epilogue of LRKV decode.
//
// For one (sequence b, head h) the per-split states (m_s, l_s, numerators)
// are combined: M = max_s m_s, w_s = 2^(m_s - M), l = sum_s w_s l_s,
// numerators = sum_s w_s num_s -- the same joint rescale of both accumulators
// and the denominator that the fused online softmax applies per tile ("Low-Rank
// Key Value Attention | What a shared cache can preserve", sec. 3, paragraph
// after Algorithm 2).  The epilogue divides by the denominator and maps the
// private value sum through B^V once per head:
//   out = (shared_num + private_num (B^V_h)^T) / l
// ("Low-Rank Key Value Attention: Chinese reading notes", sec. 2.4 Eq. (7)).
// A sequence with no live rows gets out = 0.
//
// Split s of sequence b is the partial record of workgroup W_b + s of the
// split launch (splits dealt to sequences by length; see lrkv_device.hpp);
// only splits with s * granule < L_b hold live rows.
//
// One workgroup of 1024 threads per (b, h): thread (column c, split group j)
// sums splits s = j, j + 4, ... of column c with four independent partial sums
// (memory-level parallelism), then the four groups are added in LDS in a fixed
// order -- results are bitwise reproducible.
#include "lrkv_device.hpp"
#include "lrkv_internal.hpp"

namespace lrkv {
namespace {

constexpr int kMergeThreads = 1024;
constexpr int kCols = 256;                       // columns handled per pass
constexpr int kGroups = kMergeThreads / kCols;   // split groups

__device__ __forceinline__ float block_max(float v, float* red) {
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    if (lane == 0) red[wave] = v;
    __syncthreads();
    float m = red[0];
    for (int w = 1; w < kMergeThreads / 64; ++w) m = fmaxf(m, red[w]);
    __syncthreads();
    return m;
}

template <typename T>
__global__ void __launch_bounds__(kMergeThreads) merge_kernel(int batch, int H, int D, int R, int max_len, int chunk,
                                                              int S,
                                                              const int32_t* __restrict__ seq_lens,
                                                              const T* __restrict__ B_v, float* __restrict__ out,
                                                              const float* __restrict__ ws) {
    extern __shared__ float sm[];
    float* w = sm;                          // [S - batch + 1] split weights
    float* part = w + (S - batch + 1);      // [kGroups][kCols] per-group column sums
    float* sums = part + kGroups * kCols;   // [D + R] merged numerators
    float* red = sums + D + R;              // [16] reduction scratch
    const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
    const int rec = partial_record_floats(D, R);
    float* o = out + ((size_t)b * H + h) * D;
    const int Lb = clamped_len(seq_lens, b, max_len);
    int W_b, S_b;
    sequence_splits(seq_lens, batch, max_len, S, b, &W_b, &S_b);  // every wave computes the same values
    const int Sb = min(S_b, (Lb + chunk - 1) / chunk);  // splits s with s * granule < L_b hold live rows
    if (Sb == 0) {
        for (int c = tid; c < D; c += kMergeThreads) o[c] = 0.f;
        return;
    }
    const float* base = ws + ((size_t)W_b * H + h) * rec;  // split s at base + s * H * rec
    const size_t sstride = (size_t)H * rec;

    float mloc = -INFINITY;
    for (int s = tid; s < Sb; s += kMergeThreads) mloc = fmaxf(mloc, base[s * sstride + D + R]);
    const float M = block_max(mloc, red);
    for (int s = tid; s < Sb; s += kMergeThreads) w[s] = fast_exp2(base[s * sstride + D + R] - M);
    __syncthreads();

    // numerators (columns 0 .. D+R-1) and the denominator (column D+R+1) in passes of kCols columns
    const int ncols = D + R + 2;
    float l = 0.f;
    for (int c0 = 0; c0 < ncols; c0 += kCols) {
        const int c = c0 + (tid % kCols), j = tid / kCols;
        float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
        if (c < ncols && c != D + R) {
            int s = j;
            for (; s + 3 * kGroups < Sb; s += 4 * kGroups) {
                a0 = fmaf(w[s], base[(size_t)s * sstride + c], a0);
                a1 = fmaf(w[s + kGroups], base[(size_t)(s + kGroups) * sstride + c], a1);
                a2 = fmaf(w[s + 2 * kGroups], base[(size_t)(s + 2 * kGroups) * sstride + c], a2);
                a3 = fmaf(w[s + 3 * kGroups], base[(size_t)(s + 3 * kGroups) * sstride + c], a3);
            }
            for (; s < Sb; s += kGroups) a0 = fmaf(w[s], base[(size_t)s * sstride + c], a0);
        }
        part[j * kCols + (tid % kCols)] = (a0 + a1) + (a2 + a3);
        __syncthreads();
        if (j == 0 && c < ncols) {
            float v = part[tid % kCols];
            for (int g = 1; g < kGroups; ++g) v += part[g * kCols + (tid % kCols)];
            if (c < D + R) sums[c] = v;
            else if (c == D + R + 1) red[15] = v;
        }
        __syncthreads();
    }
    l = red[15];
    const float inv_l = 1.0f / l;
    const float* u = sums + D;
    const T* Bh = B_v + (size_t)h * D * R;
    for (int c = tid; c < D; c += kMergeThreads) {
        float pr = 0.f;
        for (int i = 0; i < R; ++i) pr = fmaf(u[i], elem<T>::load(Bh, (size_t)c * R + i), pr);
        o[c] = (sums[c] + pr) * inv_l;
    }
}

}  // namespace

hipError_t launch_merge(int batch, int H, int d_h, int r, int dtype, int max_len, int chunk, int num_splits,
                        const int32_t* seq_lens, const void* B_v, float* out, const float* ws, hipStream_t stream) {
    dim3 grid(H, batch), block(kMergeThreads);
    // a sequence has at most num_splits - batch + 1 splits (every other sequence holds at least one)
    const size_t max_sb = (size_t)(num_splits - batch + 1);
    const size_t lds = sizeof(float) * (max_sb + kGroups * kCols + (size_t)d_h + r + 16);
    if (dtype == 0)
        hipLaunchKernelGGL(merge_kernel<float>, grid, block, lds, stream, batch, H, d_h, r, max_len, chunk, num_splits,
                           seq_lens, (const float*)B_v, out, ws);
    else
        hipLaunchKernelGGL(merge_kernel<uint16_t>, grid, block, lds, stream, batch, H, d_h, r, max_len, chunk,
                           num_splits,
                           seq_lens, (const uint16_t*)B_v, out, ws);
    return hipGetLastError();
}

}  // namespace lrkv
