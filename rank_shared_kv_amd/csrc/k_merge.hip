// Split merge and epilogue of LRKV decode.
//
// For one (sequence b, head h) the per-split states (m_s, l_s, numerators)
// are combined in split order: M = max_s m_s, w_s = 2^(m_s - M),
// l = sum_s w_s l_s, numerators = sum_s w_s num_s -- the same joint rescale of
// both accumulators and the denominator that the fused online softmax applies
// per tile ("Low-Rank Key Value Attention | What a shared cache can
// preserve", sec. 3, paragraph after Algorithm 2).  The epilogue divides by
// the denominator and maps the private value sum through B^V once per head:
//   out = (shared_num + private_num (B^V_h)^T) / l
// ("Low-Rank Key Value Attention: Chinese reading notes", sec. 2.4 Eq. (7)).
// A sequence with no live rows gets out = 0.
#include "lrkv_device.hpp"
#include "lrkv_internal.hpp"

namespace lrkv {
namespace {

constexpr int kMergeThreads = 128;

template <typename T>
__global__ void __launch_bounds__(kMergeThreads) merge_kernel(int H, int D, int R, int max_len, int chunk, int S,
                                                              const int32_t* __restrict__ seq_lens,
                                                              const T* __restrict__ B_v, float* __restrict__ out,
                                                              const float* __restrict__ ws) {
    extern __shared__ float sm[];  // w[S], private sum[R]
    float* w = sm;
    float* u = sm + S;
    const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
    const int rec = partial_record_floats(D, R);
    float* o = out + ((size_t)b * H + h) * D;
    int Lb = seq_lens[b];
    Lb = Lb < 0 ? 0 : (Lb > max_len ? max_len : Lb);
    const int Sb = (Lb + chunk - 1) / chunk;
    if (Sb == 0) {
        for (int c = tid; c < D; c += kMergeThreads) o[c] = 0.f;
        return;
    }
    const float* base = ws + ((size_t)b * S * H + h) * rec;  // split s at base + s * H * rec
    const size_t sstride = (size_t)H * rec;
    float M = -INFINITY;
    for (int s = 0; s < Sb; ++s) M = fmaxf(M, base[s * sstride + D + R]);
    for (int s = tid; s < Sb; s += kMergeThreads) w[s] = fast_exp2(base[s * sstride + D + R] - M);
    __syncthreads();
    float l = 0.f;
    for (int s = 0; s < Sb; ++s) l = fmaf(w[s], base[s * sstride + D + R + 1], l);
    for (int i = tid; i < R; i += kMergeThreads) {
        float acc = 0.f;
        for (int s = 0; s < Sb; ++s) acc = fmaf(w[s], base[s * sstride + D + i], acc);
        u[i] = acc;
    }
    __syncthreads();
    const float inv_l = 1.0f / l;
    const T* Bh = B_v + (size_t)h * D * R;
    for (int c = tid; c < D; c += kMergeThreads) {
        float acc = 0.f;
        for (int s = 0; s < Sb; ++s) acc = fmaf(w[s], base[s * sstride + c], acc);
        float pr = 0.f;
        for (int i = 0; i < R; ++i) pr = fmaf(u[i], elem<T>::load(Bh, (size_t)c * R + i), pr);
        o[c] = (acc + pr) * inv_l;
    }
}

}  // namespace

hipError_t launch_merge(int batch, int H, int d_h, int r, int dtype, int max_len, int chunk, int num_splits,
                        const int32_t* seq_lens, const void* B_v, float* out, const float* ws, hipStream_t stream) {
    dim3 grid(H, batch), block(kMergeThreads);
    const size_t lds = sizeof(float) * ((size_t)num_splits + (size_t)r);
    if (dtype == 0)
        hipLaunchKernelGGL(merge_kernel<float>, grid, block, lds, stream, H, d_h, r, max_len, chunk, num_splits,
                           seq_lens, (const float*)B_v, out, ws);
    else
        hipLaunchKernelGGL(merge_kernel<uint16_t>, grid, block, lds, stream, H, d_h, r, max_len, chunk, num_splits,
                           seq_lens, (const uint16_t*)B_v, out, ws);
    return hipGetLastError();
}

}  // namespace lrkv
