// Streaming-read probe: the measured read bandwidth that the decode's achieved
// bandwidth is also compared with (besides the published HBM peak).  Every
// 16-byte chunk of a buffer is read once with non-temporal loads: each
// workgroup sweeps a contiguous slice, 16 loads in flight per lane (the best of
// 4, 8 and 16 measured; non-temporal loads read 7.0 TB/s where ordinary ones
// read 6.3); each workgroup folds what it read into one XOR checksum so the
// loads cannot be dropped.  Not part of the attention method.
#include "lrkv_device.hpp"
#include "lrkv_internal.hpp"

namespace lrkv {
namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 16;

__global__ void __launch_bounds__(kProbeThreads) read_probe_kernel(const u32x4_t* __restrict__ p, size_t n16,
                                                                   uint32_t* __restrict__ sink) {
    __shared__ uint32_t part[kProbeThreads / 64];
    // workgroup w sweeps its own contiguous slice; one load instruction of the workgroup covers 4 KiB
    const size_t per = (n16 + gridDim.x - 1) / gridDim.x;
    const size_t begin = min(n16, (size_t)blockIdx.x * per), end = min(n16, begin + per);
    size_t i = begin + threadIdx.x;
    uint32_t acc = 0;
    for (; i + (kProbeUnroll - 1) * kProbeThreads < end; i += kProbeUnroll * kProbeThreads) {
        u32x4_t v[kProbeUnroll];
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) v[u] = __builtin_nontemporal_load(p + i + u * kProbeThreads);
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < end; i += kProbeThreads) {
        const u32x4_t v = __builtin_nontemporal_load(p + i);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) sink[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

}  // namespace

int read_probe_workgroups() { return 1024; }  // 4 per CU on 256 CUs

hipError_t launch_read_probe(const void* src, size_t bytes, uint32_t* sink, hipStream_t stream) {
    hipLaunchKernelGGL(read_probe_kernel, dim3(read_probe_workgroups()), dim3(kProbeThreads), 0, stream,
                       (const u32x4_t*)src, bytes / 16, sink);
    return hipGetLastError();
}

}  // namespace lrkv
