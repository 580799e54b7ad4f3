// General split kernel for LRKV decode: any supported (d_h, r, H), fp32 or
// bf16 inputs, fp32 arithmetic.  Used for fp32 problems and for shapes the
// MFMA kernel does not cover.
//
// One workgroup owns one (sequence b, split) for all H heads; splits are dealt
// to sequences by length and a split takes every S_b-th tile of kTile tokens
// of its sequence.  Per tile the shared key/value rows are staged once
// in LDS (as fp32) and reused by every head; each head then
//   scores  s_j = (q_h . k_j + p_h . z^K_{h,j}) * log2(e)/sqrt(d_h)
//   updates its running max, denominator and both numerators (online softmax)
// -- the fused single-softmax form of "Low-Rank Key Value Attention | What a
// shared cache can preserve", sec. 3 (paragraph after Algorithm 2), of the
// summed-logit score in "Low-Rank Key Value Attention: Chinese reading notes",
// sec. 2.4 Eqs. (6)-(7).  The running state of all heads lives in LDS; the
// split's final state is written to the workspace for the merge kernel.
// Normalised variant (rho set): each logit is also multiplied by the cached
// reciprocal RMS of its (head, token) key ("Low-Rank Key Value Attention |
// What a shared cache can preserve", sec. 8, post-projection normalisation).
#include "lrkv_device.hpp"
#include "lrkv_internal.hpp"

namespace lrkv {
namespace {

constexpr int kTile = 32;     // tokens per tile (lanes 0..31 and 32..63 split each dot product)
constexpr int kThreads = 256;  // 4 waves

__host__ __device__ inline size_t general_lds_floats(int H, int d_h, int r, bool rope) {
    return (size_t)kTile * (d_h + 1)      // K tile, padded rows
           + (size_t)kTile * d_h          // V tile
           + (size_t)H * (d_h + r)        // numerators
           + 2 * (size_t)H                // running max, denominator
           + 4 * (size_t)kTile            // per-wave weights
           + (rope ? (size_t)H * d_h : 0);  // rotated queries
}

template <typename T, bool ROPE>
__global__ void __launch_bounds__(kThreads) split_general_kernel(DecodeArgs a) {
    extern __shared__ float smem[];
    const int H = a.H, D = a.d_h, R = a.r, rec = partial_record_floats(D, R);
    float* Kt = smem;                          // [kTile][D + 1]
    float* Vt = Kt + kTile * (D + 1);          // [kTile][D]
    float* acc = Vt + kTile * D;               // [H][D + R]
    float* mrow = acc + (size_t)H * (D + R);   // [H]
    float* lrow = mrow + H;                    // [H]
    float* ebuf = lrow + H;                    // [4][kTile]
    float* qrot = ebuf + 4 * kTile;            // [H][D] rotated queries (rotary variant)

    // which sequence and split (splits dealt to sequences by length); split s of sequence b takes the
    // tiles s, s + S_b, s + 2 S_b, ... of the sequence
    const SplitSlot wslot = split_slot(a.seq_lens, a.batch, a.max_len, a.num_splits, a.chunk, a.qgroup, blockIdx.x);
    const int b = wslot.b, split = wslot.s;
    if (b < 0) return;
    const int Lb = clamped_len(a.seq_lens, b, a.max_len);
    if (split * kTile >= Lb) return;  // no live rows in this split; the merge skips it
    const int bc = b / a.qgroup;      // the cached sequence this (virtual) sequence reads

    const T* ks = (const T*)a.k_shared;  // rows addressed by their row in the tensor (or page pool)
    const T* vs = (const T*)a.v_shared;
    const T* zk = (const T*)a.z_k;
    const T* zv = (const T*)a.z_v;
    const T* q = (const T*)a.q;
    const T* rho = (const T*)a.rho;  // [batch][L_cap][H] or NULL
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const float scale = kLog2e / sqrtf((float)D);

    if constexpr (ROPE) {
        // the query sits at position L_b - 1: q D_{L_b - 1}, pair by pair, in fp32
        const float* cs = a.rope_cs + (size_t)(Lb - 1) * D;
        for (int idx = tid; idx < H * (D / 2); idx += kThreads) {
            const int h = idx / (D / 2), k = idx - h * (D / 2);
            const float x0 = elem<T>::load(q, ((size_t)b * H + h) * D + 2 * k);
            const float x1 = elem<T>::load(q, ((size_t)b * H + h) * D + 2 * k + 1);
            const float co = cs[2 * k], si = cs[2 * k + 1];
            qrot[h * D + 2 * k] = x0 * co - x1 * si;
            qrot[h * D + 2 * k + 1] = x0 * si + x1 * co;
        }
    }
    for (int i = tid; i < H * (D + R); i += kThreads) acc[i] = 0.f;
    for (int i = tid; i < H; i += kThreads) {
        mrow[i] = -INFINITY;
        lrow[i] = 0.f;
    }

    for (int t0 = split * kTile; t0 < Lb; t0 += wslot.S_b * kTile) {
        const int nvalid = min(kTile, Lb - t0);
        // first row of the tile in the cache tensors: contiguous, or the pool row of its page (a page holds
        // whole tiles)
        const size_t r0 = a.block_table ? (size_t)paged_row(a, bc, t0) : (size_t)bc * a.L_cap + t0;
        __syncthreads();  // previous tile fully consumed (and state initialised)
        for (int idx = tid; idx < kTile * D; idx += kThreads) {
            const int t = idx / D, c = idx - t * D;
            const size_t row = r0 + (t < nvalid ? t : nvalid - 1);  // stay on live rows
            Kt[t * (D + 1) + c] = elem<T>::load(ks, row * D + c);
            Vt[t * D + c] = elem<T>::load(vs, row * D + c);
        }
        __syncthreads();

        const int t = lane & 31, half = lane >> 5;
        const bool live = t < nvalid;
        const int c_lo = half * ((D + 1) / 2), c_hi = min(D, (half + 1) * ((D + 1) / 2));
        const int i_lo = half * ((R + 1) / 2), i_hi = min(R, (half + 1) * ((R + 1) / 2));
        for (int h = wave; h < H; h += kThreads / 64) {
            const size_t bh = (size_t)b * H + h;  // q and p row of (sequence, head)
            // latents are token-major: row t of sequence b holds every head's r coordinates
            const size_t zrow = ((r0 + (size_t)(live ? t : 0)) * H + h) * R;
            // score: shared part on the LDS tile, private part on the latent row
            float sc = 0.f;
            if constexpr (ROPE) {
                // rotary variant: rebuild the key's columns of this half (shared row + latent times B^K_h),
                // turn each pair at the row's position, dot with the rotated query (the halves hold whole
                // pairs: d_h is a multiple of 4)
                const T* bkh = (const T*)a.rope_bk + (size_t)h * D * R;
                const float* cs = a.rope_cs + (size_t)(t0 + (live ? t : 0)) * D;
                for (int c = c_lo; c < c_hi; c += 2) {
                    float u0 = Kt[t * (D + 1) + c], u1 = Kt[t * (D + 1) + c + 1];
                    for (int i = 0; i < R; ++i) {
                        const float z = elem<T>::load(zk, zrow + i);
                        u0 = fmaf(z, elem<T>::load(bkh, (size_t)c * R + i), u0);
                        u1 = fmaf(z, elem<T>::load(bkh, (size_t)(c + 1) * R + i), u1);
                    }
                    const float co = cs[c], si = cs[c + 1];
                    sc = fmaf(qrot[h * D + c], u0 * co - u1 * si, sc);
                    sc = fmaf(qrot[h * D + c + 1], u0 * si + u1 * co, sc);
                }
            } else {
                for (int c = c_lo; c < c_hi; ++c) sc = fmaf(elem<T>::load(q, bh * D + c), Kt[t * (D + 1) + c], sc);
                for (int i = i_lo; i < i_hi; ++i) sc = fmaf(a.p[bh * R + i], elem<T>::load(zk, zrow + i), sc);
            }
            sc += __shfl_xor(sc, 32);
            // normalised variant: the cached scale of (row, head) multiplies the summed logit
            float f = scale;
            if (rho) f *= elem<T>::load(rho, ((size_t)bc * a.L_cap + (size_t)(t0 + (live ? t : 0))) * H + h);
            const float s2 = live ? sc * f : -INFINITY;
            float tmax = s2;
            for (int o = 16; o >= 1; o >>= 1) tmax = fmaxf(tmax, __shfl_xor(tmax, o));
            const float m_old = mrow[h];
            const float m_new = fmaxf(m_old, tmax);
            const float alpha = (m_new == -INFINITY) ? 1.f : fast_exp2(m_old - m_new);  // nothing seen yet
            const float e = live ? fast_exp2(s2 - m_new) : 0.f;
            float esum = e;
            for (int o = 16; o >= 1; o >>= 1) esum += __shfl_xor(esum, o);
            if (lane < kTile) ebuf[wave * kTile + lane] = e;
            wave_lds_sync();
            if (lane == 0) {
                mrow[h] = m_new;
                lrow[h] = alpha * lrow[h] + esum;
            }
            float* acc_h = acc + (size_t)h * (D + R);
            for (int c = lane; c < D; c += 64) {
                float sum = 0.f;
                for (int u = 0; u < nvalid; ++u) sum = fmaf(ebuf[wave * kTile + u], Vt[u * D + c], sum);
                acc_h[c] = alpha * acc_h[c] + sum;
            }
            for (int i = lane; i < R; i += 64) {
                float sum = 0.f;
                const size_t z0 = (r0 * H + h) * R + i;
                for (int u = 0; u < nvalid; ++u)
                    sum = fmaf(ebuf[wave * kTile + u], elem<T>::load(zv, z0 + (size_t)u * H * R), sum);
                acc_h[D + i] = alpha * acc_h[D + i] + sum;
            }
            wave_lds_sync();  // ebuf reused by this wave's next head
        }
    }
    __syncthreads();
    float* out = a.ws + (size_t)blockIdx.x * H * rec;  // record of workgroup w = W_b + split
    for (int idx = tid; idx < H * rec; idx += kThreads) {
        const int v = idx / rec, k = idx - v * rec;
        float x = 0.f;
        if (k < D + R) x = acc[(size_t)v * (D + R) + k];
        else if (k == D + R) x = mrow[v];
        else if (k == D + R + 1) x = lrow[v];
        out[idx] = x;
    }
}

}  // namespace

int general_rows_per_tile() { return kTile; }

size_t general_lds_bytes(int H, int d_h, int r, bool rope) { return general_lds_floats(H, d_h, r, rope) * sizeof(float); }

// gfx950 gives a workgroup up to 160 KiB of LDS
bool general_path_supports(int H, int d_h, int r) {
    return d_h >= 1 && d_h <= 256 && r >= 0 && r <= 256 && H >= 1 && general_lds_bytes(H, d_h, r) <= 160 * 1024;
}

template <typename T, bool ROPE>
hipError_t launch_general_t(const DecodeArgs& a, hipStream_t stream) {
    const size_t lds = general_lds_bytes(a.H, a.d_h, a.r, ROPE);
    auto kern = split_general_kernel<T, ROPE>;
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(a.num_splits), dim3(kThreads), lds, stream, a);
    return hipGetLastError();
}

hipError_t launch_split_general(const DecodeArgs& a, hipStream_t stream) {
    const bool rope = a.rope_cs != nullptr;
    if (a.dtype == 0) return rope ? launch_general_t<float, true>(a, stream) : launch_general_t<float, false>(a, stream);
    return rope ? launch_general_t<uint16_t, true>(a, stream) : launch_general_t<uint16_t, false>(a, stream);
}

}  // namespace lrkv
