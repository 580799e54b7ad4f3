// Projections around the attention core of an LRKV layer decode step.
//
// project + append: the new token x_t of every sequence is projected by one
//   stacked weight matrix, y = x W_in^T with the rows of W_in ordered
//   [W_q (H*d_h) | W_S^K (d_h) | W_S^V (d_h) | U^K (H*r) | U^V (H*r)], and the
//   outputs go straight to their destinations: q to the query buffer, the
//   shared key/value rows and every head's latents to row seq_lens[b] of the
//   cache ("Low-Rank Key Value Attention | What a shared cache can preserve",
//   sec. 3, Algorithm 1; "Low-Rank Key Value Attention: Chinese reading
//   notes", sec. 2.1 Eqs. (2)-(5), sec. 2.3).  A second, tiny kernel then
//   advances seq_lens (every projection workgroup reads it first).
// output projection: y = concat_h(o_h) W_o^T (review, Algorithm 2's last step).
//
// Both are skinny products (M = batch rows, K = d_model or H*d_h, N features)
// bound by streaming the weights once.  Matrix-core path (bf16 weights): a
// workgroup of 16 (or 8, 4) waves owns 16 output features; the waves split K
// into equal slices and each runs v_mfma_f32_16x16x32_bf16 over its slice for
// every 16-row tile of the batch (weights read once, reused by all rows).  Operands
// are 16-byte global loads: weight row n, 8 consecutive k per lane; batch row
// m likewise.  An fp32 left operand (the decode output o) enters as a bf16
// high part plus a bf16 low part (two products), about 16 significant bits.
// The waves' partial products are added in LDS in a fixed order.  Other shapes
// and fp32 weights use a plain fp32 kernel.
#include "lrkv_device.hpp"
#include "lrkv_internal.hpp"

namespace lrkv {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;  // plain kernel
constexpr int kMaxMTiles = 4;  // at most 64 rows per workgroup pass
constexpr int kUnroll = 4;     // k-steps of 32 whose loads are issued together

// Where output feature n of row m goes.
struct ProjectSink {
    int H, d_h, r, L_cap, dtype;
    void* q;                 // [batch][H*d_h]
    void* k_shared;          // [batch][L_cap][d_h]
    void* v_shared;
    void* z_k;               // [batch][L_cap][H][r]
    void* z_v;
    const int32_t* seq_lens;
    __device__ void put(int m, int n, float v) const {
        const int nq = H * d_h;
        size_t off;
        void* base;
        if (n < nq) {
            base = q;
            off = (size_t)m * nq + n;
        } else {
            const int j = seq_lens[m];
            if (j < 0 || j >= L_cap) return;  // full sequence: nothing is written
            int c = n - nq;
            if (c < d_h) {
                base = k_shared;
                off = ((size_t)m * L_cap + j) * d_h + c;
            } else if ((c -= d_h) < d_h) {
                base = v_shared;
                off = ((size_t)m * L_cap + j) * d_h + c;
            } else if ((c -= d_h) < H * r) {
                base = z_k;
                off = ((size_t)m * L_cap + j) * H * r + c;  // token-major: head c / r, coordinate c % r
            } else {
                c -= H * r;
                base = z_v;
                off = ((size_t)m * L_cap + j) * H * r + c;
            }
        }
        if (dtype == 0) ((float*)base)[off] = v;
        else ((uint16_t*)base)[off] = (uint16_t)f32_to_bf16_bits(v);
    }
};

struct DenseSink {
    float* y;  // [M][N]
    int N;
    __device__ void put(int m, int n, float v) const { y[(size_t)m * N + n] = v; }
};

// left operand fragment of 8 consecutive k for one row: bf16 rows load directly; fp32 rows are split
template <typename AT>
struct AFrag;
template <>
struct AFrag<uint16_t> {
    static constexpr int kParts = 1;
    u32x4_t w;
    __device__ void load(const uint16_t* row, int k) { w = *(const u32x4_t*)(row + k); }
    __device__ void zero() { w = u32x4_t{0u, 0u, 0u, 0u}; }
    __device__ u32x4_t part(int) const { return w; }
};
template <>
struct AFrag<float> {
    static constexpr int kParts = 2;
    u32x4_t a, b;  // 8 fp32 values
    __device__ void load(const float* row, int k) {
        a = *(const u32x4_t*)(row + k);
        b = *(const u32x4_t*)(row + k + 4);
    }
    __device__ void zero() { a = b = u32x4_t{0u, 0u, 0u, 0u}; }
    __device__ u32x4_t part(int p) const {  // p = 0: bf16 high parts, 1: bf16 low parts (x - high)
        u32x4_t out;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float x0 = __uint_as_float(i < 2 ? a[2 * i] : b[2 * i - 4]);
            const float x1 = __uint_as_float(i < 2 ? a[2 * i + 1] : b[2 * i - 3]);
            uint32_t h0 = f32_to_bf16_bits(x0), h1 = f32_to_bf16_bits(x1);
            if (p == 1) {
                h0 = f32_to_bf16_bits(x0 - __uint_as_float(h0 << 16));
                h1 = f32_to_bf16_bits(x1 - __uint_as_float(h1 << 16));
            }
            out[i] = h0 | (h1 << 16);
        }
        return out;
    }
};

// MT row tiles of 16 per workgroup pass; KW waves split K into equal slices, so K must be a multiple of
// KW * 32 * kUnroll.  Many waves per workgroup keep many weight loads in flight per CU.
template <typename AT, int MT, int KW, typename Sink>
__global__ void __launch_bounds__(KW * 64) linear_mfma_kernel(int M, int K, int N, const AT* __restrict__ A,
                                                              const uint16_t* __restrict__ W, Sink sink) {
    __shared__ float red[KW][MT * 16][17];
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n16 = lane & 15, g4 = lane >> 4;
    const int n0 = blockIdx.x * 16;
    const int m_base = blockIdx.y * (MT * 16);
    const int mt_count = min(MT, (M - m_base + 15) / 16);
    const int kq = K / KW, k_begin = wave * kq;  // this wave's slice of K
    const int n = min(n0 + n16, N - 1);           // features past N re-read the last row; results dropped
    const uint16_t* wrow = W + (size_t)n * K + 8 * g4;

    f32x4_t acc[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    for (int k0 = k_begin; k0 < k_begin + kq; k0 += 32 * kUnroll) {
        u32x4_t wv[kUnroll];
        AFrag<AT> af[kUnroll][MT];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            wv[u] = *(const u32x4_t*)(wrow + k0 + 32 * u);
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                const int m = min(m_base + 16 * t + n16, M - 1);  // rows past M re-read the last row
                if (t < mt_count) af[u][t].load(A + (size_t)m * K + 8 * g4, k0 + 32 * u);
            }
        }
        __builtin_amdgcn_sched_barrier(0);  // every load of the group ahead of the products
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                if (t >= mt_count) continue;
                if (m_base + 16 * t + n16 >= M) af[u][t].zero();
#pragma unroll
                for (int p = 0; p < AFrag<AT>::kParts; ++p)
                    acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, af[u][t].part(p)),
                                                                     __builtin_bit_cast(bf16x8_t, wv[u]), acc[t], 0,
                                                                     0, 0);
            }
    }
    mfma_result_fence();  // the K loop ends with products; their results are read next
    // D layout: lane (n16, g4) holds rows 4 g4 + i of the tile, feature n0 + n16
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) red[wave][16 * t + 4 * g4 + i][n16] = acc[t][i];
    __syncthreads();
    for (int idx = tid; idx < mt_count * 16 * 16; idx += KW * 64) {
        const int ml = idx / 16, nl = idx % 16;
        const int m = m_base + ml, nn = n0 + nl;
        if (m >= M || nn >= N) continue;
        float v = red[0][ml][nl];
#pragma unroll
        for (int w = 1; w < KW; ++w) v += red[w][ml][nl];  // fixed order
        sink.put(m, nn, v);
    }
}

// Plain fp32 path: one thread per (row, feature), fixed-order sum over K.
template <typename AT, typename WT, typename Sink>
__global__ void __launch_bounds__(kThreads) linear_simple_kernel(int M, int K, int N, const AT* __restrict__ A,
                                                                 const WT* __restrict__ W, Sink sink) {
    const int idx = blockIdx.x * kThreads + threadIdx.x;
    if (idx >= M * N) return;
    const int m = idx / N, n = idx % N;
    float s = 0.f;
    for (int k = 0; k < K; ++k) s = fmaf(elem<AT>::load(A, (size_t)m * K + k), elem<WT>::load(W, (size_t)n * K + k), s);
    sink.put(m, n, s);
}

__global__ void commit_kernel(int batch, int L_cap, int32_t* __restrict__ seq_lens) {
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= batch) return;
    const int L = seq_lens[b];
    if (L >= 0 && L < L_cap) seq_lens[b] = L + 1;
}

template <typename AT, int MT, int KW, typename Sink>
void launch_mfma(int M, int K, int N, const AT* A, const void* W, Sink sink, hipStream_t stream) {
    dim3 grid((N + 15) / 16, (M + MT * 16 - 1) / (MT * 16));
    hipLaunchKernelGGL((linear_mfma_kernel<AT, MT, KW, Sink>), grid, dim3(KW * 64), 0, stream, M, K, N, A,
                       (const uint16_t*)W, sink);
}

// K slices per workgroup: as many waves as the shape allows (16, 8 or 4); four row tiles use at most 8
// (the LDS of the final reduction)
template <typename AT, int MT, typename Sink>
bool launch_mfma_kw(int M, int K, int N, const AT* A, const void* W, Sink sink, hipStream_t stream) {
    constexpr int step = 32 * kUnroll;
    if (MT < 4 && K % (16 * step) == 0) launch_mfma<AT, MT, (MT < 4 ? 16 : 8)>(M, K, N, A, W, sink, stream);
    else if (K % (8 * step) == 0) launch_mfma<AT, MT, 8>(M, K, N, A, W, sink, stream);
    else if (K % (4 * step) == 0) launch_mfma<AT, MT, 4>(M, K, N, A, W, sink, stream);
    else return false;
    return true;
}

template <typename AT, typename Sink>
hipError_t launch_linear(int dtype, int M, int K, int N, const AT* A, const void* W, Sink sink, hipStream_t stream) {
    bool done = false;
    if (dtype == 1) {
        if (M <= 16) done = launch_mfma_kw<AT, 1>(M, K, N, A, W, sink, stream);
        else if (M <= 32) done = launch_mfma_kw<AT, 2>(M, K, N, A, W, sink, stream);
        else done = launch_mfma_kw<AT, kMaxMTiles>(M, K, N, A, W, sink, stream);
    }
    if (!done) {
        const long total = (long)M * N;
        dim3 grid((unsigned)((total + kThreads - 1) / kThreads));
        if (dtype == 1)
            hipLaunchKernelGGL((linear_simple_kernel<AT, uint16_t, Sink>), grid, dim3(kThreads), 0, stream, M, K, N,
                               A, (const uint16_t*)W, sink);
        else
            hipLaunchKernelGGL((linear_simple_kernel<AT, float, Sink>), grid, dim3(kThreads), 0, stream, M, K, N, A,
                               (const float*)W, sink);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_project_append(int batch, int H, int d_h, int r, int L_cap, int dtype, int d_model, void* k_shared,
                                 void* v_shared, void* z_k, void* z_v, int32_t* seq_lens, const void* x,
                                 const void* W_in, void* q_out, hipStream_t stream) {
    ProjectSink sink{H, d_h, r, L_cap, dtype, q_out, k_shared, v_shared, z_k, z_v, seq_lens};
    const int N = H * d_h + 2 * d_h + 2 * H * r;
    hipError_t e = (dtype == 1)
                       ? launch_linear<uint16_t>(dtype, batch, d_model, N, (const uint16_t*)x, W_in, sink, stream)
                       : launch_linear<float>(dtype, batch, d_model, N, (const float*)x, W_in, sink, stream);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(commit_kernel, dim3((batch + 255) / 256), dim3(256), 0, stream, batch, L_cap, seq_lens);
    return hipGetLastError();
}

hipError_t launch_output_project(int batch, int H, int d_h, int dtype, int d_model, const float* o, const void* W_o,
                                 float* y, hipStream_t stream) {
    DenseSink sink{y, d_model};
    return launch_linear<float>(dtype, batch, H * d_h, d_model, o, W_o, sink, stream);
}

}  // namespace lrkv
