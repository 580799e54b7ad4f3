// Query absorption and cache append.
//
// absorb:  p_h = q_h B^K_h, one d_h x r product per (sequence, head) and step
//          ("Low-Rank Key Value Attention: Chinese reading notes", sec. 2.4
//          Eq. (6); "Low-Rank Key Value Attention | What a shared cache can
//          preserve", sec. 3, Algorithm 2).  fp32 result, fp32 accumulation in
//          a fixed order over d_h.
// append:  write one token's shared rows and per-head latents at index
//          seq_lens[b] and advance seq_lens[b] (review sec. 3, Algorithm 1;
//          reading notes sec. 2.3).  Latents are token-major, so one token's
//          H x r latents land in one contiguous row.  With a block table the
//          row goes to its pool page instead (paged cache).
// append + absorb: both in one launch (a decode step's per-token work).
// multi-token lengths: query i of Q at the end of sequence b sees
//          max(0, L_b - Q + 1 + i) rows (the causal mask inside the chunk);
//          the multi-token decode runs one virtual sequence per set of qw
//          consecutive query tokens, with the length of the set's last token.
#include "lrkv_device.hpp"
#include "lrkv_internal.hpp"
#include "lrkv_step.hpp"

namespace lrkv {
namespace {

// One workgroup per (b, h): thread (i, quarter) sums a quarter of the d_h terms
// for coordinate i, the four quarters are added in a fixed order in LDS.
constexpr int kAbsorbThreads = 256;

template <typename T>
__global__ void __launch_bounds__(kAbsorbThreads) absorb_kernel(int H, int d_h, int r, const T* __restrict__ q,
                                                                const T* __restrict__ B_k, float* __restrict__ p) {
    __shared__ float part[kAbsorbThreads];
    const int bh = blockIdx.x;  // b * H + h
    const int h = bh % H;
    const T* qrow = q + (size_t)bh * d_h;
    const T* basis = B_k + (size_t)h * d_h * r;
    const int tid = threadIdx.x, i0 = tid & 63, quarter = tid >> 6;
    const int c_per = (d_h + 3) / 4;
    const int c_lo = quarter * c_per, c_hi = min(d_h, c_lo + c_per);
    // every thread runs the same number of iterations (barriers inside)
    for (int ib = 0; ib < r; ib += 64) {
        const int i = ib + i0;
        float a0 = 0.f, a1 = 0.f;
        if (i < r) {
            int c = c_lo;
            for (; c + 1 < c_hi; c += 2) {
                a0 = fmaf(elem<T>::load(qrow, c), elem<T>::load(basis, (size_t)c * r + i), a0);
                a1 = fmaf(elem<T>::load(qrow, c + 1), elem<T>::load(basis, (size_t)(c + 1) * r + i), a1);
            }
            if (c < c_hi) a0 = fmaf(elem<T>::load(qrow, c), elem<T>::load(basis, (size_t)c * r + i), a0);
        }
        part[tid] = a0 + a1;
        __syncthreads();
        if (quarter == 0 && i < r) p[(size_t)bh * r + i] = ((part[i0] + part[64 + i0]) + part[128 + i0]) + part[192 + i0];
        __syncthreads();
    }
}

// Vector path (rows of B^K a multiple of 16 bytes, r / VE <= 64): one wave per (b, h) unit, four units per
// workgroup (absorb_wave, lrkv_step.hpp; the fused decode step runs the same body).
constexpr int kAbsorbUnitsPerWg = kAbsorbThreads / 64;
constexpr int kAbsorbPartFloats = 64 * 8;  // 64 * VE floats per wave (VE <= 8)

template <typename T>
__device__ __forceinline__ void absorb_wg_units(int wg, int n_units, int H, int d_h, int r, const T* __restrict__ q,
                                                const T* __restrict__ B_k, float* __restrict__ p) {
    __shared__ float qs[kAbsorbUnitsPerWg][256];
    __shared__ float part[kAbsorbUnitsPerWg][kAbsorbPartFloats];
    const int wave = threadIdx.x >> 6;
    const int u = wg * kAbsorbUnitsPerWg + wave;
    if (u < n_units) absorb_wave<T>(u, H, d_h, r, q, B_k, p, qs[wave], part[wave]);
}

template <typename T>
__global__ void __launch_bounds__(kAbsorbThreads) absorb_vec_kernel(int n_units, int H, int d_h, int r,
                                                                    const T* __restrict__ q,
                                                                    const T* __restrict__ B_k,
                                                                    float* __restrict__ p) {
    absorb_wg_units<T>(blockIdx.x, n_units, H, d_h, r, q, B_k, p);
}

// block_table NULL: contiguous cache [batch][L_cap][...]; else page pools [n_pages][1 << page_shift][...]
// with logical page m of sequence b at pool page block_table[b * max_pages + m] (L_cap = max_pages pages)
template <typename T>
__device__ __forceinline__ void append_body(int b, int H, int d_h, int r, int L_cap, T* __restrict__ k_shared,
                                            T* __restrict__ v_shared, T* __restrict__ z_k, T* __restrict__ z_v,
                                            int32_t* __restrict__ seq_lens, const T* __restrict__ k_new,
                                            const T* __restrict__ v_new, const T* __restrict__ zk_new,
                                            const T* __restrict__ zv_new, const int32_t* __restrict__ block_table,
                                            int page_shift, int max_pages) {
    __shared__ int row;
    if (threadIdx.x == 0) {
        const int L = seq_lens[b];
        row = (L >= 0 && L < L_cap) ? L : -1;
    }
    __syncthreads();
    const int j = row;
    if (j < 0) return;  // full or invalid: nothing written, length unchanged
    append_row_copy<T>(b, j, H, d_h, r, L_cap, k_shared, v_shared, z_k, z_v, k_new, v_new, zk_new, zv_new,
                       block_table, page_shift, max_pages);
    __syncthreads();
    if (threadIdx.x == 0) seq_lens[b] = j + 1;
}

template <typename T>
__global__ void __launch_bounds__(256) append_kernel(int H, int d_h, int r, int L_cap, T* __restrict__ k_shared,
                                                     T* __restrict__ v_shared, T* __restrict__ z_k,
                                                     T* __restrict__ z_v, int32_t* __restrict__ seq_lens,
                                                     const T* __restrict__ k_new, const T* __restrict__ v_new,
                                                     const T* __restrict__ zk_new, const T* __restrict__ zv_new,
                                                     const int32_t* __restrict__ block_table, int page_shift,
                                                     int max_pages) {
    append_body<T>(blockIdx.x, H, d_h, r, L_cap, k_shared, v_shared, z_k, z_v, seq_lens, k_new, v_new, zk_new,
                   zv_new, block_table, page_shift, max_pages);
}

// One launch for the two per-token operations of a decode step: workgroups 0 .. batch-1 append (as
// append_kernel), the rest absorb four (b, h) units each (as absorb_vec_kernel).  The two touch
// disjoint memory, so they run side by side; each workgroup's arithmetic is the separate kernels', so the
// results are bitwise the same.
template <typename T>
__global__ void __launch_bounds__(256) append_absorb_kernel(int batch, int H, int d_h, int r, int L_cap,
                                                            T* __restrict__ k_shared, T* __restrict__ v_shared,
                                                            T* __restrict__ z_k, T* __restrict__ z_v,
                                                            int32_t* __restrict__ seq_lens,
                                                            const T* __restrict__ k_new, const T* __restrict__ v_new,
                                                            const T* __restrict__ zk_new,
                                                            const T* __restrict__ zv_new, const T* __restrict__ q,
                                                            const T* __restrict__ B_k, float* __restrict__ p) {
    const int w = blockIdx.x;
    if (w < batch)
        append_body<T>(w, H, d_h, r, L_cap, k_shared, v_shared, z_k, z_v, seq_lens, k_new, v_new, zk_new, zv_new,
                       nullptr, 0, 0);
    else
        absorb_wg_units<T>(w - batch, batch * H, H, d_h, r, q, B_k, p);
}

}  // namespace

// The vector path needs 16-byte rows of B^K (r a multiple of 16 / element bytes), a q row that fits its LDS
// stage (d_h <= 256) and at least one row group: each lane of a unit's wave owns one 16-byte vector of a row,
// so r / (16 / element bytes) must not exceed 64 (r <= 512 for bf16, 256 for fp32).  Other shapes take the
// scalar kernel.
static bool absorb_vec_ok(int d_h, int r, int dtype) { return absorb_wave_ok(d_h, r, dtype == 0 ? 4 : 2); }

static int absorb_workgroups(int n_units) { return (n_units + kAbsorbUnitsPerWg - 1) / kAbsorbUnitsPerWg; }

hipError_t launch_absorb(int batch, int H, int d_h, int r, int dtype, const void* q, const void* B_k, float* p,
                         hipStream_t stream) {
    const bool vec = absorb_vec_ok(d_h, r, dtype);
    dim3 grid(vec ? absorb_workgroups(batch * H) : batch * H), block(kAbsorbThreads);
    if (dtype == 0) {
        if (vec)
            hipLaunchKernelGGL(absorb_vec_kernel<float>, grid, block, 0, stream, batch * H, H, d_h, r, (const float*)q,
                               (const float*)B_k, p);
        else
            hipLaunchKernelGGL(absorb_kernel<float>, grid, block, 0, stream, H, d_h, r, (const float*)q,
                               (const float*)B_k, p);
    } else {
        if (vec)
            hipLaunchKernelGGL(absorb_vec_kernel<uint16_t>, grid, block, 0, stream, batch * H, H, d_h, r,
                               (const uint16_t*)q, (const uint16_t*)B_k, p);
        else
            hipLaunchKernelGGL(absorb_kernel<uint16_t>, grid, block, 0, stream, H, d_h, r, (const uint16_t*)q,
                               (const uint16_t*)B_k, p);
    }
    return hipGetLastError();
}

bool append_absorb_supported(int H, int d_h, int r, int dtype) {
    return kAbsorbThreads == 256 && absorb_vec_ok(d_h, r, dtype);  // the absorb's vector path
}

hipError_t launch_append_absorb(int batch, int H, int d_h, int r, int L_cap, int dtype, void* k_shared,
                                void* v_shared, void* z_k, void* z_v, int32_t* seq_lens, const void* k_new,
                                const void* v_new, const void* zk_new, const void* zv_new, const void* q,
                                const void* B_k, float* p, hipStream_t stream) {
    if (!append_absorb_supported(H, d_h, r, dtype)) return hipErrorInvalidValue;
    dim3 grid(batch + absorb_workgroups(batch * H)), block(256);
    if (dtype == 0)
        hipLaunchKernelGGL(append_absorb_kernel<float>, grid, block, 0, stream, batch, H, d_h, r, L_cap,
                           (float*)k_shared, (float*)v_shared, (float*)z_k, (float*)z_v, seq_lens,
                           (const float*)k_new, (const float*)v_new, (const float*)zk_new, (const float*)zv_new,
                           (const float*)q, (const float*)B_k, p);
    else
        hipLaunchKernelGGL(append_absorb_kernel<uint16_t>, grid, block, 0, stream, batch, H, d_h, r, L_cap,
                           (uint16_t*)k_shared, (uint16_t*)v_shared, (uint16_t*)z_k, (uint16_t*)z_v, seq_lens,
                           (const uint16_t*)k_new, (const uint16_t*)v_new, (const uint16_t*)zk_new,
                           (const uint16_t*)zv_new, (const uint16_t*)q, (const uint16_t*)B_k, p);
    return hipGetLastError();
}

namespace {
template <typename T>
void launch_append_t(int batch, int H, int d_h, int r, int L_cap, void* k_shared, void* v_shared, void* z_k,
                     void* z_v, int32_t* seq_lens, const void* k_new, const void* v_new, const void* zk_new,
                     const void* zv_new, const int32_t* block_table, int page_shift, int max_pages,
                     hipStream_t stream) {
    hipLaunchKernelGGL(append_kernel<T>, dim3(batch), dim3(256), 0, stream, H, d_h, r, L_cap, (T*)k_shared,
                       (T*)v_shared, (T*)z_k, (T*)z_v, seq_lens, (const T*)k_new, (const T*)v_new, (const T*)zk_new,
                       (const T*)zv_new, block_table, page_shift, max_pages);
}
}  // namespace

hipError_t launch_append(int batch, int H, int d_h, int r, int L_cap, int dtype, void* k_shared, void* v_shared,
                         void* z_k, void* z_v, int32_t* seq_lens, const void* k_new, const void* v_new,
                         const void* zk_new, const void* zv_new, hipStream_t stream) {
    if (dtype == 0)
        launch_append_t<float>(batch, H, d_h, r, L_cap, k_shared, v_shared, z_k, z_v, seq_lens, k_new, v_new, zk_new,
                               zv_new, nullptr, 0, 0, stream);
    else
        launch_append_t<uint16_t>(batch, H, d_h, r, L_cap, k_shared, v_shared, z_k, z_v, seq_lens, k_new, v_new,
                                  zk_new, zv_new, nullptr, 0, 0, stream);
    return hipGetLastError();
}

namespace {
__global__ void __launch_bounds__(256) multi_lengths_kernel(int n, int Q, int qw, const int32_t* __restrict__ seq_lens,
                                                            int32_t* __restrict__ lens_out) {
    const int v = blockIdx.x * 256 + threadIdx.x;
    if (v >= n) return;
    const int nc = (Q + qw - 1) / qw;
    const int b = v / nc, c = v - b * nc;
    const int last = min((c + 1) * qw, Q) - 1;  // the set's last token
    lens_out[v] = max(0, seq_lens[b] - Q + 1 + last);
}
}  // namespace

hipError_t launch_multi_lengths(int batch, int Q, int qw, const int32_t* seq_lens, int32_t* lens_out,
                                hipStream_t stream) {
    const int n = batch * ((Q + qw - 1) / qw);
    hipLaunchKernelGGL(multi_lengths_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, n, Q, qw, seq_lens,
                       lens_out);
    return hipGetLastError();
}

namespace {
// dst[b][j][h][i] = src[b][h][j][i]: one workgroup per (sequence, 8-row tile); thread t of a tile walks the
// tile's destination elements (8 rows x H x r, contiguous in dst) with stride 256, so the writes are
// coalesced and the reads come in runs of r elements of one head's rows.
template <typename T>
__global__ void __launch_bounds__(256) latents_token_major_kernel(int H, int L_cap, int r, const T* __restrict__ src,
                                                                  T* __restrict__ dst) {
    constexpr int kTile = 8;
    const int b = blockIdx.y, j0 = blockIdx.x * kTile;
    const int rows = min(kTile, L_cap - j0);
    const size_t hr = (size_t)H * r;
    const T* s = src + (size_t)b * H * L_cap * r;
    T* d = dst + ((size_t)b * L_cap + j0) * hr;
    const size_t n = (size_t)rows * hr;
    for (size_t e = threadIdx.x; e < n; e += 256) {
        const size_t jj = e / hr, rem = e - jj * hr;
        const size_t h = rem / r, i = rem - h * r;
        d[e] = s[(h * L_cap + j0 + jj) * r + i];
    }
}
}  // namespace

hipError_t launch_latents_token_major(int batch, int H, int L_cap, int r, int dtype, const void* src, void* dst,
                                      hipStream_t stream) {
    dim3 grid((L_cap + 7) / 8, batch), block(256);
    if (dtype == 0)
        hipLaunchKernelGGL(latents_token_major_kernel<float>, grid, block, 0, stream, H, L_cap, r, (const float*)src,
                           (float*)dst);
    else
        hipLaunchKernelGGL(latents_token_major_kernel<uint16_t>, grid, block, 0, stream, H, L_cap, r,
                           (const uint16_t*)src, (uint16_t*)dst);
    return hipGetLastError();
}

hipError_t launch_paged_append(int batch, int H, int d_h, int r, int dtype, int page_shift, int max_pages,
                              void* k_pages, void* v_pages, void* zk_pages, void* zv_pages,
                              const int32_t* block_table, int32_t* seq_lens, const void* k_new, const void* v_new,
                              const void* zk_new, const void* zv_new, hipStream_t stream) {
    const int L_cap = max_pages << page_shift;
    if (dtype == 0)
        launch_append_t<float>(batch, H, d_h, r, L_cap, k_pages, v_pages, zk_pages, zv_pages, seq_lens, k_new, v_new,
                               zk_new, zv_new, block_table, page_shift, max_pages, stream);
    else
        launch_append_t<uint16_t>(batch, H, d_h, r, L_cap, k_pages, v_pages, zk_pages, zv_pages, seq_lens, k_new,
                                  v_new, zk_new, zv_new, block_table, page_shift, max_pages, stream);
    return hipGetLastError();
}

}  // namespace lrkv
