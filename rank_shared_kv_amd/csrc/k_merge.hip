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
// only splits with s * granule < L_b hold live rows.  Multi-token decode with
// Q query tokens per sequence runs virtual sequences of qw tokens each
// (ceil(Q / qw) per sequence); a workgroup then holds qw records per head, and
// token i of sequence b reads record i % qw of the splits of its virtual
// sequence, live up to its own causal length.
//
// One workgroup per (b, h) of 256 threads times 1 or 4 split groups: thread (column c, split group j)
// walks splits s = j, j + 4, ... of column c once, in batches of 16 whose
// loads are issued together, keeping its own running maximum and rescaling
// its sum once per batch (no separate pass for the maxima).  The four groups
// are then combined in LDS in a fixed order, so results are bitwise
// reproducible.  The B^V row
// fragments the epilogue needs are loaded at kernel start, off the critical
// path.  The fused decode step merges with merge_body (lrkv_step.hpp), whose
// arithmetic per column is this kernel's, so both give the same bits.
#include "lrkv_device.hpp"
#include "lrkv_internal.hpp"
#include "lrkv_step.hpp"

namespace lrkv {
namespace {

constexpr int kCols = 256;                       // columns handled per pass
constexpr int kMaxCols = 512;                    // d_h + r <= 512
constexpr int kBatch = 16;                       // splits per thread loaded together

typedef step_u32x4_t u32x4_t;

// kGroups split groups of kCols threads each: 4 groups when sequences hold many splits, 1 when they
// hold few (then the extra threads would only wait).
template <typename T, int kGroups>
__global__ void __launch_bounds__(kGroups * kCols) merge_kernel(int nv, int Q, int qw, int H, int D, int R,
                                                                int max_len, int chunk, int S,
                                                                const int32_t* __restrict__ seq_lens,
                                                                const T* __restrict__ B_v, float* __restrict__ out,
                                                                const float* __restrict__ ws) {
    constexpr int kMergeThreads = kGroups * kCols;
    constexpr int VE = 16 / (int)sizeof(T);  // B^V elements per 16-byte vector
    __shared__ float gmax[kGroups][kCols];   // per-group running maxima
    __shared__ float gsum[kGroups][kCols];   // per-group rescaled sums
    __shared__ float sums[kMaxCols + 2];     // merged numerators, then l at [D + R]
    __shared__ float epi[kMergeThreads];     // epilogue partial products
    const int h = blockIdx.x, row = blockIdx.y, tid = threadIdx.x;  // output row = sequence * Q + token
    const int rec = partial_record_floats(D, R);
    float* o = out + ((size_t)row * H + h) * D;
    // the virtual sequence v holding token i of sequence b, the token's slot qi in it and its causal length
    const int nc = (Q + qw - 1) / qw;
    const int b = row / Q, i = row - b * Q;
    const int c = i / qw, qi = i - c * qw;
    const int v = b * nc + c;
    const int nreal = min(qw, Q - c * qw);

    // epilogue operand: thread (c, vi) holds B^V[h][c][vi*VE, vi*VE + VE) as one 16-byte vector
    const int nvv = (R > 0 && (R % VE) == 0) ? R / VE : 0;
    const bool vec_epi = merge_epilogue_in_parts(D, nvv, kMergeThreads);
    u32x4_t bv = {0u, 0u, 0u, 0u};
    const int ec = vec_epi ? tid / nvv : 0, evi = vec_epi ? tid % nvv : 0;
    if (vec_epi && ec < D) bv = *(const u32x4_t*)(B_v + ((size_t)h * D + ec) * R + evi * VE);

    const int Lb = max(0, clamped_len(seq_lens, v, max_len) - (nreal - 1 - qi));
    int W_b, S_b;
    sequence_splits(seq_lens, nv, max_len, S, chunk, nc, v, &W_b, &S_b);  // every wave computes the same values
    const int Sb = min(S_b, (Lb + chunk - 1) / chunk);  // splits s with s * granule < L_b hold rows
    if (Sb == 0) {
        for (int c = tid; c < D; c += kMergeThreads) o[c] = 0.f;
        return;
    }
    const float* base = ws + (((size_t)W_b * qw + qi) * H + h) * rec;  // split s at base + s * qw * H * rec
    const int sstride = qw * H * rec;  // the workspace is below 2^31 floats

    // numerators (columns 0 .. D+R-1) and the denominator (column D+R+1) in passes of kCols columns
    const int ncols = D + R + 2;
    for (int c0 = 0; c0 < ncols; c0 += kCols) {
        const int cl = tid % kCols, j = tid / kCols, c = c0 + cl;
        float mj = -INFINITY, sj = 0.f;
        if (c < ncols && c != D + R) {
            // batches of kBatch splits: all loads of a batch are issued together, one rescale per batch
            for (int s0 = j; s0 < Sb; s0 += kGroups * kBatch) {
                float mr[kBatch], xr[kBatch];
#pragma unroll
                for (int k = 0; k < kBatch; ++k) {
                    // unconditional loads (splits past the end re-read split s0), all issued before any use
                    const int s = s0 + kGroups * k;
                    const int o = (s < Sb ? s : s0) * sstride;
                    mr[k] = base[o + D + R];
                    xr[k] = base[o + c];
                }
                __builtin_amdgcn_sched_barrier(0);  // keep every load of the batch ahead of the arithmetic
#pragma unroll
                for (int k = 0; k < kBatch; ++k) {
                    if (s0 + kGroups * k >= Sb) {
                        mr[k] = -INFINITY;
                        xr[k] = 0.f;
                    }
                }
                float mc = mr[0];
#pragma unroll
                for (int k = 1; k < kBatch; ++k) mc = fmaxf(mc, mr[k]);
                const float mn = fmaxf(mj, mc);  // finite: split s0 < Sb holds live rows
                float t = 0.f;
#pragma unroll
                for (int k = 0; k < kBatch; ++k) t = fmaf(fast_exp2(mr[k] - mn), xr[k], t);  // absent: 0 * 0
                sj = fmaf(sj, fast_exp2(mj - mn), t);  // mj = -inf at first: 0
                mj = mn;
            }
        }
        gmax[j][cl] = mj;
        gsum[j][cl] = sj;
        __syncthreads();
        if (j == 0 && c < ncols && c != D + R) {
            float M = gmax[0][cl];
            for (int g = 1; g < kGroups; ++g) M = fmaxf(M, gmax[g][cl]);
            float v = 0.f;
            for (int g = 0; g < kGroups; ++g)  // fixed order; empty groups (max -inf) add nothing
                v += (gmax[g][cl] == -INFINITY) ? 0.f : fast_exp2(gmax[g][cl] - M) * gsum[g][cl];
            sums[c < D + R ? c : D + R] = v;
        }
        __syncthreads();
    }
    // Every column saw the same split maxima, so all of them are scaled by the same 2^-M.
    const float inv_l = 1.0f / sums[D + R];
    const float* u = sums + D;
    if (R == 0) {
        for (int c = tid; c < D; c += kMergeThreads) o[c] = sums[c] * inv_l;
    } else if (vec_epi) {
        float pr = 0.f;
        if (ec < D) {
#pragma unroll
            for (int e = 0; e < VE; ++e) pr = fmaf(u[evi * VE + e], vec_elem<T>(bv, e), pr);
        }
        epi[tid] = pr;
        __syncthreads();
        for (int c = tid; c < D; c += kMergeThreads) {
            float t = 0.f;
            for (int k = 0; k < nvv; ++k) t += epi[c * nvv + k];  // fixed order
            o[c] = (sums[c] + t) * inv_l;
        }
    } else if (nvv > 0) {  // row c of B^V_h read as 16-byte vectors by thread c
        for (int c = tid; c < D; c += kMergeThreads) {
            const T* row = B_v + ((size_t)h * D + c) * R;
            float pr = 0.f;
            for (int vi = 0; vi < nvv; ++vi) {
                const u32x4_t v = *(const u32x4_t*)(row + vi * VE);
#pragma unroll
                for (int e = 0; e < VE; ++e) pr = fmaf(u[vi * VE + e], vec_elem<T>(v, e), pr);
            }
            o[c] = (sums[c] + pr) * inv_l;
        }
    } else {
        const T* Bh = B_v + (size_t)h * D * R;
        for (int c = tid; c < D; c += kMergeThreads) {
            float pr = 0.f;
            for (int i = 0; i < R; ++i) pr = fmaf(u[i], elem<T>::load(Bh, (size_t)c * R + i), pr);
            o[c] = (sums[c] + pr) * inv_l;
        }
    }
}

}  // namespace

// KG = 4 when sequences average more than 32 splits (two batches per group otherwise)
bool merge_wide(int num_splits, int n_virtual) { return num_splits > 32 * n_virtual; }

hipError_t launch_merge(int batch, int Q, int qw, int H, int d_h, int r, int dtype, int max_len, int chunk,
                        int num_splits, const int32_t* seq_lens, const void* B_v, float* out, const float* ws,
                        hipStream_t stream) {
    if (d_h + r > kMaxCols || Q < 1 || qw < 1) return hipErrorInvalidValue;
    const int nv = batch * ((Q + qw - 1) / qw);  // sequences of the split launch
    // one split group per column when sequences average at most 32 splits (two batches per thread), four
    // otherwise (4-token decode at long context, 32 splits per token set: 8.0 us with one group, 11.1 us
    // with four)
    const bool wide = merge_wide(num_splits, nv);
    dim3 grid(H, batch * Q), block(wide ? 4 * kCols : kCols);
    if (dtype == 0) {
        auto k = wide ? merge_kernel<float, 4> : merge_kernel<float, 1>;
        hipLaunchKernelGGL(k, grid, block, 0, stream, nv, Q, qw, H, d_h, r, max_len, chunk, num_splits, seq_lens,
                           (const float*)B_v, out, ws);
    } else {
        auto k = wide ? merge_kernel<uint16_t, 4> : merge_kernel<uint16_t, 1>;
        hipLaunchKernelGGL(k, grid, block, 0, stream, nv, Q, qw, H, d_h, r, max_len, chunk, num_splits, seq_lens,
                           (const uint16_t*)B_v, out, ws);
    }
    return hipGetLastError();
}

// The split plan on its own: one wave per sequence b writes W_b (its first workgroup, the index of its first
// partial record) and S_b (its split count), as the split and merge kernels of a launch with these arguments
// compute them.
__global__ void __launch_bounds__(64) split_plan_kernel(int batch, int max_len, int append_cap, int chunk, int S,
                                                       const int32_t* __restrict__ seq_lens,
                                                       int32_t* __restrict__ first_wg, int32_t* __restrict__ splits) {
    int W_b, S_b;
    sequence_splits(seq_lens, batch, max_len, S, chunk, 1, (int)blockIdx.x, &W_b, &S_b, append_cap);
    if (threadIdx.x == 0) {
        first_wg[blockIdx.x] = W_b;
        splits[blockIdx.x] = S_b;
    }
}

hipError_t launch_split_plan(int batch, int max_len, int append_cap, int chunk, int num_splits,
                             const int32_t* seq_lens, int32_t* first_wg, int32_t* splits, hipStream_t stream) {
    hipLaunchKernelGGL(split_plan_kernel, dim3(batch), dim3(64), 0, stream, batch, max_len, append_cap, chunk,
                       num_splits, seq_lens, first_wg, splits);
    return hipGetLastError();
}

}  // namespace lrkv
