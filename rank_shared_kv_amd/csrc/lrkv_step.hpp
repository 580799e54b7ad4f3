// Device bodies shared by the separate per-step kernels and the fused decode step.
//
// absorb_wave:  p_h = q_h B^K_h for one (sequence, head) unit on one wave
//               ("Low-Rank Key Value Attention: Chinese reading notes", sec. 2.4 Eq. (6)).
// merge_body:   the combination of one (sequence, head)'s split records and the epilogue
//               ("Low-Rank Key Value Attention | What a shared cache can preserve", sec. 3, the fused
//               online-softmax paragraph after Algorithm 2; reading notes Eq. (7)).
// step_*:       the counters through which the workgroups of one fused decode-step launch hand work on.
//
// The separate kernels (absorb_vec_kernel, append_absorb_kernel, merge_kernel) and the fused decode step
// call the same bodies, so the two ways of running a step give bitwise the same p and outputs.
#pragma once

#include "lrkv_device.hpp"

namespace lrkv {

typedef uint32_t step_u32x4_t __attribute__((ext_vector_type(4)));

// Loads and stores coherent across the GPU's XCDs (relaxed atomics at agent scope: they bypass the non-coherent
// per-XCD L2 copies), for data one workgroup of a launch hands to another.
__device__ __forceinline__ float ld_agent(const float* p) {
    return __uint_as_float(__hip_atomic_load((uint32_t*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}
__device__ __forceinline__ void st_agent(float* p, float v) {
    __hip_atomic_store((uint32_t*)p, __float_as_uint(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <bool COH>
__device__ __forceinline__ float ld_f32(const float* p) {
    if constexpr (COH) return ld_agent(p);
    else return *p;
}
template <bool COH>
__device__ __forceinline__ void st_f32(float* p, float v) {
    if constexpr (COH) st_agent(p, v);
    else *p = v;
}

template <typename T>
__device__ __forceinline__ float vec_elem(const step_u32x4_t& v, int e) {
    if constexpr (sizeof(T) == 4) {
        return __uint_as_float(v[e]);
    } else {
        const uint32_t w = v[e >> 1];
        return (e & 1) ? bf16_hi(w) : bf16_lo(w);
    }
}

// ---------------------------------------------------------------------------------------------------------
// Absorb on one wave.  Unit u = b * H + h: p[u][i] = sum_c q[u][c] B^K[h][c][i], fp32, in a fixed order.
// B^K rows are read as 16-byte vectors (VE elements): with nv = r / VE vectors per row, lane (row group rg,
// vector vi) takes vector vi of rows c = rg, rg + rpw, ... (rpw = 64 / nv row groups), keeps VE partial sums,
// and the row groups are added in order through LDS.  All of a lane's B^K loads are issued before its q
// values are read (one memory round trip).  Needs r % VE == 0, r / VE <= 64 and d_h <= 256; qs holds d_h
// floats and part 64 * VE floats of this wave's LDS.  COH: p is written with agent-coherent stores (the fused
// step hands it to other workgroups of the launch).
// ---------------------------------------------------------------------------------------------------------
constexpr int kAbsorbChunk = 16;  // B^K vectors a lane loads before it uses them

template <typename T>
__host__ __device__ constexpr int absorb_ve() {
    return 16 / (int)sizeof(T);
}

inline bool absorb_wave_ok(int d_h, int r, int elem_bytes) {
    const int ve = 16 / elem_bytes;
    return r > 0 && (r % ve) == 0 && r / ve <= 64 && d_h <= 256;
}

template <typename T, bool COH = false>
__device__ __forceinline__ void absorb_wave(int u, int H, int d_h, int r, const T* __restrict__ q,
                                            const T* __restrict__ B_k, float* __restrict__ p, float* qs,
                                            float* part) {
    constexpr int VE = absorb_ve<T>();
    const int lane = threadIdx.x & 63, h = u % H;
    const int nv = r / VE, rpw = 64 / nv;
    const int vi = lane % nv, rg = lane / nv;
    const int groups = min(rpw, d_h);
    const T* basis = B_k + (size_t)h * d_h * r + vi * VE;
    float acc[VE];
#pragma unroll
    for (int e = 0; e < VE; ++e) acc[e] = 0.f;
    // rows c = rg + rpw * k; chunks of kAbsorbChunk rows per lane, every load of a chunk issued before its use
    for (int c0 = 0; c0 < d_h; c0 += kAbsorbChunk * rpw) {
        step_u32x4_t v[kAbsorbChunk];
#pragma unroll
        for (int k = 0; k < kAbsorbChunk; ++k) {
            const int c = c0 + rg + rpw * k;
            v[k] = *(const step_u32x4_t*)(basis + (size_t)(c < d_h ? c : 0) * r);  // row 0 stands in past d_h
        }
        if (c0 == 0) {
            for (int c = lane; c < d_h; c += 64) qs[c] = elem<T>::load(q, (size_t)u * d_h + c);
            wave_lds_sync();
        }
        if (rg < groups) {
#pragma unroll
            for (int k = 0; k < kAbsorbChunk; ++k) {
                const int c = c0 + rg + rpw * k;
                if (c < d_h) {
                    const float qc = qs[c];
#pragma unroll
                    for (int e = 0; e < VE; ++e) acc[e] = fmaf(qc, vec_elem<T>(v[k], e), acc[e]);
                }
            }
        }
    }
    if (rg < groups) {
#pragma unroll
        for (int e = 0; e < VE; ++e) part[rg * r + vi * VE + e] = acc[e];
    }
    wave_lds_sync();
    for (int i = lane; i < r; i += 64) {
        float sum = 0.f;
        for (int g = 0; g < groups; ++g) sum += part[g * r + i];  // fixed order
        st_f32<COH>(p + (size_t)u * r + i, sum);
    }
    wave_lds_sync();  // part and qs free for the next unit of this wave
}

// ---------------------------------------------------------------------------------------------------------
// Append: token b's shared rows and per-head latents written at row j of sequence b (review sec. 3,
// Algorithm 1; reading notes sec. 2.3), by every thread of the calling workgroup.  Latents are token-major, so
// one token's H x r latents form one contiguous row.  block_table NULL: contiguous cache [batch][L_cap][...];
// else page pools [n_pages][1 << page_shift][...] with logical page m of sequence b at pool page
// block_table[b * max_pages + m].
// ---------------------------------------------------------------------------------------------------------
template <typename T>
__device__ __forceinline__ void append_row_copy(int b, int j, int H, int d_h, int r, int L_cap,
                                                T* __restrict__ k_shared, T* __restrict__ v_shared,
                                                T* __restrict__ z_k, T* __restrict__ z_v,
                                                const T* __restrict__ k_new, const T* __restrict__ v_new,
                                                const T* __restrict__ zk_new, const T* __restrict__ zv_new,
                                                const int32_t* __restrict__ block_table, int page_shift,
                                                int max_pages) {
    // the row's index in the cache tensors (contiguous) or page pools (paged)
    const size_t grow = block_table ? ((size_t)block_table[(size_t)b * max_pages + (j >> page_shift)] << page_shift) +
                                          (size_t)(j & ((1 << page_shift) - 1))
                                    : (size_t)b * L_cap + j;
    const size_t srow = grow * d_h;
    const size_t zrow = grow * H * r, zsrc = (size_t)b * H * r;
    constexpr int VE = absorb_ve<T>();
    if ((d_h % VE) == 0 && ((H * r) % VE) == 0) {
        for (int c = threadIdx.x; c < d_h / VE; c += blockDim.x) {
            ((step_u32x4_t*)(k_shared + srow))[c] = ((const step_u32x4_t*)(k_new + (size_t)b * d_h))[c];
            ((step_u32x4_t*)(v_shared + srow))[c] = ((const step_u32x4_t*)(v_new + (size_t)b * d_h))[c];
        }
        for (int c = threadIdx.x; c < H * r / VE; c += blockDim.x) {
            ((step_u32x4_t*)(z_k + zrow))[c] = ((const step_u32x4_t*)(zk_new + zsrc))[c];
            ((step_u32x4_t*)(z_v + zrow))[c] = ((const step_u32x4_t*)(zv_new + zsrc))[c];
        }
    } else {
        for (int c = threadIdx.x; c < d_h; c += blockDim.x) {
            k_shared[srow + c] = k_new[(size_t)b * d_h + c];
            v_shared[srow + c] = v_new[(size_t)b * d_h + c];
        }
        for (int idx = threadIdx.x; idx < H * r; idx += blockDim.x) {
            z_k[zrow + idx] = zk_new[zsrc + idx];
            z_v[zrow + idx] = zv_new[zsrc + idx];
        }
    }
}

// ---------------------------------------------------------------------------------------------------------
// Merge of one (output row, head) on a workgroup of kStepMergeThreads threads (the fused decode step).
//
// Split s of sequence v is the partial record of workgroup W_v + s of the split launch (splits dealt to
// sequences by length, lrkv_device.hpp); splits with s * chunk < L_v hold live rows.  For every column c
// (numerators [0, d_h + r) and the denominator d_h + r + 1) the splits are taken in KG interleaved groups,
// group j holding splits j, j + KG, ..., each group in batches of kMergeBatch splits with one rescale per
// batch; then the groups are combined in a fixed order:
//   M = max_g m_g,  value = sum_g 2^(m_g - M) sum_g'
// Thread t handles column c0 + t of each pass and all KG groups of it, issuing the loads of one batch of every
// group together.  Per column this is the arithmetic of the standalone merge kernel (k_merge.hip), which gives
// each group a thread of its own.  Multi-token decode (Q query tokens per sequence in virtual sequences of qw tokens): token i
// of sequence b reads record i % qw of the splits of its virtual sequence, live up to its causal length.
// Epilogue: out = (shared numerator + (private numerator) (B^V_h)^T) / l, the product summed as
// merge_epilogue_in_parts decides for a KG * 256-thread standalone workgroup.  A sequence with no live rows
// gets 0.
// wait(S_b) runs after every address is known and before the first record is read, with the number of split
// workgroups of the sequence (the fused step waits there for all of them).  COH: the records are read with
// agent-coherent loads (the fused step's split workgroups wrote them in the same launch).  sums: LDS of kMergeMaxCols + 2 floats.
// ---------------------------------------------------------------------------------------------------------
constexpr int kMergeMaxCols = 512;  // d_h + r <= 512
constexpr int kStepMergeThreads = 256;
constexpr int kMergeBatch = 16;
constexpr int kMergeBvVecs = 8;     // B^V row vectors held from the start (r <= 8 VE)

// The epilogue's product (private numerator) (B^V_h)^T is summed as r / VE partial dot products of VE terms
// when the standalone merge kernel, with `threads` threads per workgroup, gives each (column, vector) pair a
// thread of its own (r a multiple of VE and d_h * r / VE <= threads); otherwise as one running sum over the r
// coordinates.  The fused step's merge takes the same choice for the same split grouping, so both agree bit for
// bit.
__host__ __device__ inline bool merge_epilogue_in_parts(int D, int nvv, int threads) {
    return nvv > 0 && D * nvv <= threads;
}

template <typename T, int KG, bool COH, typename Wait>
__device__ __forceinline__ void merge_body(int h, int row, int nv, int Q, int qw, int H, int D, int R, int max_len,
                                           int append_cap, int chunk, int S, const int32_t* __restrict__ seq_lens,
                                           const T* __restrict__ B_v, float* __restrict__ out,
                                           const float* __restrict__ ws, float* sums, Wait wait) {
    constexpr int VE = absorb_ve<T>();
    const int tid = threadIdx.x;
    const int rec = partial_record_floats(D, R);
    float* o = out + ((size_t)row * H + h) * D;
    // the virtual sequence v holding token i of sequence b, the token's slot qi in it and its causal length
    const int nc = (Q + qw - 1) / qw;
    const int b = row / Q, i = row - b * Q;
    const int c = i / qw, qi = i - c * qw;
    const int v = b * nc + c;
    const int nreal = min(qw, Q - c * qw);

    // epilogue operand: row tid of B^V_h, as VE-element vectors, loaded now (off the critical path); every
    // load reads a valid vector of the row
    const int nvv = (R > 0 && (R % VE) == 0) ? R / VE : 0;
    const bool bv_pre = nvv > 0 && nvv <= kMergeBvVecs;
    step_u32x4_t bv[kMergeBvVecs];
    if (bv_pre && tid < D) {
        const T* brow = B_v + ((size_t)h * D + tid) * R;
#pragma unroll
        for (int k = 0; k < kMergeBvVecs; ++k) bv[k] = *(const step_u32x4_t*)(brow + (k < nvv ? k : 0) * VE);
    }

    const int Lb = max(0, clamped_len(seq_lens, v, max_len, append_cap) - (nreal - 1 - qi));
    int W_b, S_b;
    sequence_splits(seq_lens, nv, max_len, S, chunk, nc, v, &W_b, &S_b, append_cap);  // every wave: the same values
    const int Sb = min(S_b, (Lb + chunk - 1) / chunk);  // splits s with s * granule < L_b hold rows
    wait(S_b);
    if (Sb == 0) {
        for (int cc = tid; cc < D; cc += kStepMergeThreads) o[cc] = 0.f;
        return;
    }
    const float* base = ws + (((size_t)W_b * qw + qi) * H + h) * rec;  // split s at base + s * qw * H * rec
    const int sstride = qw * H * rec;  // the workspace is below 2^31 floats

    const int ncols = D + R + 2;
    for (int c0 = 0; c0 < ncols; c0 += kStepMergeThreads) {
        const int cc = c0 + tid;
        float mj[KG], sj[KG];
#pragma unroll
        for (int g = 0; g < KG; ++g) {
            mj[g] = -INFINITY;
            sj[g] = 0.f;
        }
        if (cc < ncols && cc != D + R) {
            // round r0: batch (r0 / (KG * kMergeBatch)) of every group; group g's batch starts at split r0 + g
            for (int r0 = 0; r0 < Sb; r0 += KG * kMergeBatch) {
                float mr[KG][kMergeBatch], xr[KG][kMergeBatch];
#pragma unroll
                for (int g = 0; g < KG; ++g) {
#pragma unroll
                    for (int k = 0; k < kMergeBatch; ++k) {
                        // unconditional loads (absent splits re-read split r0), all issued before any use
                        const int s = r0 + g + KG * k;
                        const int off = (s < Sb ? s : r0) * sstride;
                        mr[g][k] = ld_f32<COH>(base + off + D + R);
                        xr[g][k] = ld_f32<COH>(base + off + cc);
                    }
                }
                __builtin_amdgcn_sched_barrier(0);  // keep every load of the round ahead of the arithmetic
#pragma unroll
                for (int g = 0; g < KG; ++g) {
                    if (r0 + g >= Sb) continue;  // group g has no batch in this round
#pragma unroll
                    for (int k = 0; k < kMergeBatch; ++k) {
                        if (r0 + g + KG * k >= Sb) {
                            mr[g][k] = -INFINITY;
                            xr[g][k] = 0.f;
                        }
                    }
                    float mc = mr[g][0];
#pragma unroll
                    for (int k = 1; k < kMergeBatch; ++k) mc = fmaxf(mc, mr[g][k]);
                    const float mn = fmaxf(mj[g], mc);  // finite: split r0 + g < Sb holds live rows
                    float t = 0.f;
#pragma unroll
                    for (int k = 0; k < kMergeBatch; ++k) t = fmaf(fast_exp2(mr[g][k] - mn), xr[g][k], t);  // absent: 0 * 0
                    sj[g] = fmaf(sj[g], fast_exp2(mj[g] - mn), t);  // mj = -inf at first: 0
                    mj[g] = mn;
                }
            }
            float M = mj[0];
#pragma unroll
            for (int g = 1; g < KG; ++g) M = fmaxf(M, mj[g]);
            float val = 0.f;
#pragma unroll
            for (int g = 0; g < KG; ++g)  // fixed order; empty groups (max -inf) add nothing
                val += (mj[g] == -INFINITY) ? 0.f : fast_exp2(mj[g] - M) * sj[g];
            sums[cc < D + R ? cc : D + R] = val;
        }
    }
    __syncthreads();
    // Every column saw the same split maxima, so all of them are scaled by the same 2^-M.
    const float inv_l = 1.0f / sums[D + R];
    const float* u = sums + D;
    if (R == 0) {
        for (int cc = tid; cc < D; cc += kStepMergeThreads) o[cc] = sums[cc] * inv_l;
    } else if (merge_epilogue_in_parts(D, nvv, KG * 256)) {
        // r / VE partial products of VE terms each, added in order
        for (int cc = tid; cc < D; cc += kStepMergeThreads) {
            float t = 0.f;
            if (bv_pre && cc == tid) {  // the row loaded at the start
#pragma unroll
                for (int k = 0; k < kMergeBvVecs; ++k) {
                    if (k < nvv) {
                        float pr = 0.f;
#pragma unroll
                        for (int e = 0; e < VE; ++e) pr = fmaf(u[k * VE + e], vec_elem<T>(bv[k], e), pr);
                        t += pr;
                    }
                }
            } else {
                const T* brow = B_v + ((size_t)h * D + cc) * R;
                for (int k = 0; k < nvv; ++k) {
                    const step_u32x4_t w = *(const step_u32x4_t*)(brow + k * VE);
                    float pr = 0.f;
#pragma unroll
                    for (int e = 0; e < VE; ++e) pr = fmaf(u[k * VE + e], vec_elem<T>(w, e), pr);
                    t += pr;
                }
            }
            o[cc] = (sums[cc] + t) * inv_l;
        }
    } else {
        // one running sum over the r coordinates, in order
        const T* Bh = B_v + (size_t)h * D * R;
        for (int cc = tid; cc < D; cc += kStepMergeThreads) {
            float pr = 0.f;
            if (bv_pre && cc == tid) {  // the row loaded at the start
#pragma unroll
                for (int k = 0; k < kMergeBvVecs; ++k) {
                    if (k < nvv) {
#pragma unroll
                        for (int e = 0; e < VE; ++e) pr = fmaf(u[k * VE + e], vec_elem<T>(bv[k], e), pr);
                    }
                }
            } else {
                for (int k = 0; k < R; ++k) pr = fmaf(u[k], elem<T>::load(Bh, (size_t)cc * R + k), pr);
            }
            o[cc] = (sums[cc] + pr) * inv_l;
        }
    }
}

// ---------------------------------------------------------------------------------------------------------
// Fused decode step: one launch of n_absorb absorb workgroups, then the split workgroups, then the merge
// workgroups.  Work is handed on through 32-bit counters in the workspace (kStep* words below).  A producer
// writes what it hands on (p rows, split records) with agent-coherent stores, waits until they are done, then
// raises the counter; a consumer reads the counter, then reads the data with agent-coherent loads.  No cache
// is written back or invalidated as a whole (agent-scope fences do that, and a few thousand of them per launch
// cost more than the launches the fusion saves).  Each role waits only on roles placed earlier in the launch:
// split workgroups on the absorb of their sequence, merge workgroups on the splits of their sequence.
// Workgroups are dispatched in index order (on each XCD), so whatever a waiting workgroup waits for has been
// dispatched already and does not itself wait on anything later: every wait ends.  Waits are bounded all the
// same (kStepSpinLimit polls); one that runs out counts itself in the error word and goes on, so no launch can
// hang.  The last merge workgroup to finish grows the sequence lengths and clears the counters, so the counters
// start at zero for the next launch (the workspace's counter area must be zero before the first one).
// ---------------------------------------------------------------------------------------------------------
constexpr int kStepFinished = 0;  // merge workgroups that have finished
constexpr int kStepError = 1;     // nonzero: a bounded wait ran out (results of that launch are not valid)
constexpr int kStepHeader = 4;    // then ready[batch] (absorb units done), done[batch] (split workgroups done)
constexpr int kStepSpinLimit = 1 << 20;

__host__ __device__ inline int step_sync_words(int batch) { return kStepHeader + 2 * batch; }

// Thread 0 polls *ctr until it reaches target (or the poll bound runs out); then the workgroup goes on.
__device__ __forceinline__ void step_wait(uint32_t* ctr, uint32_t target, uint32_t* sync) {
    if (threadIdx.x == 0) {
        int n = 0;
        while (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
            if (++n > kStepSpinLimit) {
                __hip_atomic_fetch_add(sync + kStepError, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                break;
            }
            __builtin_amdgcn_s_sleep(2);
        }
    }
    __syncthreads();
}

// Every thread waits for its stores to complete; then thread 0 raises *ctr (ctr NULL: the wait only).
__device__ __forceinline__ void step_publish(uint32_t* ctr) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (ctr && threadIdx.x == 0) __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// End of a merge workgroup of the fused step: counts it as finished; the last of the `total` grows every
// sequence that took the appended token and clears the counters (every workgroup of the launch has read the
// lengths by then, and every merge workgroup has passed its wait, so no counter is read any more).  The count
// comes after the merge: taken right after the wait instead, the merge workgroups of a sequence, which pass
// their waits together, queued on the one counter address, and their record loads (which return in order after
// the count) waited for the queue.  flag: one int of LDS.
__device__ __forceinline__ void step_finish(uint32_t* sync, int total, int batch, int L_cap, int32_t* seq_lens,
                                            int* flag) {
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t old = __hip_atomic_fetch_add(sync + kStepFinished, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *flag = (old + 1 == (uint32_t)total) ? 1 : 0;
    }
    __syncthreads();
    if (*flag) {
        for (int b = threadIdx.x; b < batch; b += blockDim.x) seq_lens[b] = grown_len(seq_lens[b], L_cap);
        for (int k = threadIdx.x; k < step_sync_words(batch); k += blockDim.x)
            if (k != kStepError) sync[k] = 0u;
    }
}

}  // namespace lrkv
