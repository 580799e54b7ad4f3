// Device-side helpers shared by the LRKV kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lrkv {

// Partial softmax state of one (sequence, split, head), as written by the
// split kernels and read by the merge kernel:
//   [0, d_h)         sum_j e_j v_shared[j]          (shared-value numerator)
//   [d_h, d_h + r)   sum_j e_j z_v[h][j]            (private-value numerator)
//   d_h + r          running max m, in log2 units (scores scaled by log2(e)/sqrt(d_h))
//   d_h + r + 1      denominator sum_j e_j, with e_j = 2^(s_j - m)
// Records are padded to a multiple of 4 floats.
__host__ __device__ inline int partial_record_floats(int d_h, int r) { return ((d_h + r + 2) + 3) & ~3; }

// bf16 <-> fp32.  A bf16 value is the upper half of its fp32 value, so
// widening is exact.
__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t v) { return __uint_as_float(uint32_t(v) << 16); }

// fp32 -> bf16, round to nearest even (inputs here are finite).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

template <typename T> struct elem;
template <> struct elem<float> {
    __device__ __forceinline__ static float load(const float* p, size_t i) { return p[i]; }
    __device__ __forceinline__ static void store(float* p, size_t i, float v) { p[i] = v; }
};
template <> struct elem<uint16_t> {
    __device__ __forceinline__ static float load(const uint16_t* p, size_t i) { return bf16_to_f32(p[i]); }
};

// Orders LDS traffic between lanes of one wave: stores before the call are
// visible to loads after it (a wave executes its LDS operations in order; the
// fences keep the compiler from moving memory operations across the point).
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Wait states between matrix-core products and the first read of their results, for code where the
// products end a loop with a run-time trip count and the results are read after it: at such a loop exit
// the compiler was seen to read accumulators too early.  24 wait states cover the longest result latency
// of the 16x16 products used here.  Costs a few dozen cycles per use.
__device__ __forceinline__ void mfma_result_fence() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7");
    __builtin_amdgcn_sched_barrier(0);
}

// log2(e): scores are carried in log2 units so that exp2 (v_exp_f32) applies.
constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------------------
// Length-proportional split plan, evaluated on the device from seq_lens.
//
// A decode launches G workgroups for the whole batch.  They are dealt to the
// sequences in proportion to each sequence's number of 32-row blocks, at
// least one each: with G' = G - batch, C_b = blocks of sequences 0..b and
// T = C_{batch-1},
//   W_b = b + floor(G' * C_{b-1} / T)      first workgroup of sequence b
//   S_b = W_{b+1} - W_b                    its number of splits
// (with T = 0 every sequence gets one workgroup, W_b = b).  Workgroup
// w = W_b + s handles split s of sequence b and writes partial record w.
// Split s of sequence b holds live rows iff s * granule < L_b.  The split
// kernels and the merge kernel evaluate the same integer formulas, so they
// agree on every W_b and S_b.  All helpers below are wave-level: every lane
// of the calling wave must call them, and they return wave-uniform values.
//
// append_cap: 0 for a plain decode; L_cap for the fused decode step, which
// appends one token per sequence in the same launch and so sees a sequence
// of stored length L with 0 <= L < L_cap at length L + 1 (a full sequence,
// or a negative length, does not grow), as lrkv_cache_append followed by a
// decode would.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int grown_len(int L, int append_cap) { return (L >= 0 && L < append_cap) ? L + 1 : L; }
__device__ __forceinline__ int clamped_len(const int32_t* seq_lens, int b, int max_len, int append_cap = 0) {
    const int L = grown_len(seq_lens[b], append_cap);
    return L < 0 ? 0 : (L > max_len ? max_len : L);
}
__device__ __forceinline__ int len_blocks(int L) { return (L + 31) >> 5; }

// floor(n * k / d) for 0 <= k < d < 2^16, in 32-bit arithmetic (n * k may not fit 32 bits)
__device__ __forceinline__ int mul_div_floor(int n, int k, int d) {
    const uint32_t q = (uint32_t)n / (uint32_t)d, r = (uint32_t)n % (uint32_t)d;
    return (int)(q * (uint32_t)k + (r * (uint32_t)k) / (uint32_t)d);
}

__device__ __forceinline__ int wave_sum_i32(int v) {
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
    return __builtin_amdgcn_readfirstlane(v);  // equal in every lane
}

// total blocks T of the batch
__device__ inline int batch_blocks(const int32_t* seq_lens, int batch, int max_len, int append_cap = 0) {
    int t = 0;
    for (int i = (int)(threadIdx.x & 63); i < batch; i += 64)
        t += len_blocks(clamped_len(seq_lens, i, max_len, append_cap));
    return wave_sum_i32(t);
}

// b + floor(extra * blocks_before / total), the quotient in double precision: exact here (the product is below
// 2^53 and so exact; a quotient that is not an integer lies at least 1 / total > 2^-31 from one, and the
// division, correctly rounded, errs by less than 2^-39 at these magnitudes), and much cheaper than the 64-bit
// integer division it replaces (which every split and merge workgroup ran before its first load)
__device__ __forceinline__ int first_workgroup(int b, int blocks_before, int extra, int total) {
    return b + (total > 0 ? (int)floor((double)extra * (double)blocks_before / (double)total) : 0);
}

struct SplitSlot {
    int b;    // sequence, or -1 if workgroup w has none
    int s;    // split index within the sequence
    int S_b;  // splits of the sequence
};

// The (sequence, split) that workgroup w of a G-workgroup launch handles.
__device__ inline SplitSlot split_slot(const int32_t* seq_lens, int batch, int max_len, int G, int w,
                                      int append_cap = 0) {
    const int lane = threadIdx.x & 63;
    const int T = batch_blocks(seq_lens, batch, max_len, append_cap);
    const int extra = G - batch;
    int carry = 0;
    for (int c0 = 0; c0 < batch; c0 += 64) {
        const int b = c0 + lane;
        const int nbk = (b < batch) ? len_blocks(clamped_len(seq_lens, b, max_len, append_cap)) : 0;
        int incl = nbk;  // inclusive scan over the lanes of this chunk of 64 sequences
        for (int o = 1; o < 64; o <<= 1) {
            const int y = __shfl_up(incl, o);
            if (lane >= o) incl += y;
        }
        const int before = carry + incl - nbk;
        const int W0 = first_workgroup(b, before, extra, T);
        const int W1 = first_workgroup(b + 1, before + nbk, extra, T);
        const unsigned long long hit = __ballot(b < batch && w >= W0 && w < W1);
        if (hit) {
            // the values are wave-uniform; readfirstlane lets the compiler keep them (and every block
            // offset derived from them) in scalar registers
            const int src = __builtin_ctzll(hit);
            return SplitSlot{__builtin_amdgcn_readfirstlane(__shfl(b, src)),
                             __builtin_amdgcn_readfirstlane(w - __shfl(W0, src)),
                             __builtin_amdgcn_readfirstlane(__shfl(W1 - W0, src))};
        }
        carry += __shfl(incl, 63);
    }
    return SplitSlot{-1, 0, 0};
}

// First workgroup W_b and split count S_b of sequence b.
__device__ inline void sequence_splits(const int32_t* seq_lens, int batch, int max_len, int G, int b, int* W_b,
                                       int* S_b, int append_cap = 0) {
    const int T = batch_blocks(seq_lens, batch, max_len, append_cap);
    int before = 0;
    for (int i = (int)(threadIdx.x & 63); i < b; i += 64)
        before += len_blocks(clamped_len(seq_lens, i, max_len, append_cap));
    before = wave_sum_i32(before);
    const int nbk = len_blocks(clamped_len(seq_lens, b, max_len, append_cap));
    const int W0 = first_workgroup(b, before, G - batch, T);
    *W_b = __builtin_amdgcn_readfirstlane(W0);
    *S_b = __builtin_amdgcn_readfirstlane(first_workgroup(b + 1, before + nbk, G - batch, T) - W0);
}

}  // namespace lrkv
