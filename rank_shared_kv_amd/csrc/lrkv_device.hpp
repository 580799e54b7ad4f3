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
// Split plan, evaluated on the device from seq_lens.
//
// A decode launches G workgroups for the whole batch (G >= batch); sequence b
// gets S_b >= 1 of them (its splits), and a split deals the sequence's nb_b
// 32-row blocks round robin over its ntl row lanes (ntl = granule / 32), so
// its busiest lane reads ceil(nb_b / (S_b ntl)) blocks.  Two plans:
//  - fewest splits: the least cap M for which S_b = max(1, ceil(nb_b / (M ntl)))
//    add up to at most G, and those S_b (workgroups past their sum have no
//    split and leave).  No split of any sequence has a lane longer than M,
//    and no other choice of S_b gives a shorter busiest lane; the lanes are
//    nearly even, so the pass does not end with a few lanes streaming alone.
//  - proportional: S_b in proportion to nb_b, at least one each: with
//    G' = G - batch, C_b = blocks of sequences 0..b and T = C_{batch-1},
//      W_b = b + floor(G' * C_{b-1} / T),   S_b = W_{b+1} - W_b
//    (with T = 0 every sequence gets one workgroup, W_b = b).  Every
//    workgroup has a split, but where nb_b does not divide evenly over the
//    S_b ntl lanes a few lanes read one block more than the rest.
// The fewest-splits plan is used when its cap M is at least kPlanFewestCap
// blocks, each cached sequence is one virtual sequence (qgroup == 1) and the
// batch holds at most kPlanMaxBatch sequences; otherwise the proportional one.
// Long lanes gain from the even lanes; with short ones (4 or 5 blocks at
// 16 x 8192 rows) the workgroups the fewest-splits plan leaves idle cost more
// than the evening saves, and the virtual sequences of a multi-token decode,
// which read the same rows together when their plans agree, can get
// different split counts.
// Workgroup w = W_b + s handles split s of sequence b and writes partial
// record w.  Split s of sequence b holds live rows iff s * granule < L_b.  The
// split kernels and the merge kernels evaluate the same integer formulas, so
// they agree on every W_b and S_b.  All helpers below are wave-level: every
// lane of the calling wave must call them, and they return wave-uniform values.
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

// Wave-wide integer scans and reductions for the split plan, which every split and merge workgroup evaluates
// before its first load of the cache: DPP row shifts within each row of 16 lanes (a source lane outside the row
// reads 0), then the row totals read from lanes 15, 31, 47 and 63 -- a few cycles per step where a lane shuffle
// (ds_bpermute) waits on the LDS crossbar.  Every lane of the wave must be active.
template <bool kMax>
__device__ __forceinline__ int row_incl_scan(int v) {  // inclusive scan (sum or max) within each row of 16 lanes
    const auto op = [](int a, int b) { return kMax ? max(a, b) : a + b; };
    v = op(v, __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true));  // row_shr:1
    v = op(v, __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true));  // row_shr:2
    v = op(v, __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true));  // row_shr:4
    v = op(v, __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true));  // row_shr:8
    return v;
}
// inclusive prefix sum over the wave's lanes
__device__ __forceinline__ int wave_incl_scan_i32(int v) {
    v = row_incl_scan<false>(v);
    const int r0 = __builtin_amdgcn_readlane(v, 15), r1 = __builtin_amdgcn_readlane(v, 31),
              r2 = __builtin_amdgcn_readlane(v, 47);
    const int row = (int)(threadIdx.x & 63) >> 4;
    return v + (row >= 1 ? r0 : 0) + (row >= 2 ? r1 : 0) + (row >= 3 ? r2 : 0);
}
// sum over the wave's lanes, equal in every lane (a scalar)
__device__ __forceinline__ int wave_sum_i32(int v) {
    v = row_incl_scan<false>(v);
    return __builtin_amdgcn_readlane(v, 15) + __builtin_amdgcn_readlane(v, 31) + __builtin_amdgcn_readlane(v, 47) +
           __builtin_amdgcn_readlane(v, 63);
}
// maximum over the wave's lanes of values >= 0, equal in every lane (a scalar)
__device__ __forceinline__ int wave_max_i32(int v) {
    v = row_incl_scan<true>(v);
    return max(max(__builtin_amdgcn_readlane(v, 15), __builtin_amdgcn_readlane(v, 31)),
               max(__builtin_amdgcn_readlane(v, 47), __builtin_amdgcn_readlane(v, 63)));
}

// b + floor(extra * blocks_before / total), the quotient in double precision: exact here (the product is below
// 2^53 and so exact; a quotient that is not an integer lies at least 1 / total > 2^-31 from one, and the
// division, correctly rounded, errs by less than 2^-39 at these magnitudes), and much cheaper than a 64-bit
// integer division
__device__ __forceinline__ int first_workgroup(int b, int blocks_before, int extra, int total) {
    return b + (total > 0 ? (int)floor((double)extra * (double)blocks_before / (double)total) : 0);
}

constexpr int kPlanFewestCap = 8;  // blocks per row lane from which the fewest-splits plan is used
constexpr int kPlanRegs = 1;       // block counts per lane held in registers while planning (more unrolled slots
                                   // change the register allocation of the kernels' main loops and spill some)
constexpr int kPlanMaxBatch = 64 * kPlanRegs;  // larger batches take the proportional plan

// splits a sequence of nb blocks needs at `per` blocks per split (per = M * ntl)
__device__ __forceinline__ int plan_splits(int nb, int per) { return nb > per ? (nb + per - 1) / per : 1; }

// The batch's block counts, read once: lane l, slot k holds sequence 64 k + l (0 past the batch).  All planning
// below works on these registers, so the plan costs one round trip to memory however many caps it tries.
struct PlanBlocks {
    int nb[kPlanRegs];
};
__device__ __forceinline__ PlanBlocks plan_blocks(const int32_t* seq_lens, int batch, int max_len, int append_cap) {
    PlanBlocks pb;
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int k = 0; k < kPlanRegs; ++k) {
        const int i = 64 * k + lane;
        pb.nb[k] = i < batch ? len_blocks(clamped_len(seq_lens, i, max_len, append_cap)) : 0;
    }
    return pb;
}

// sum over the batch of plan_splits at `per`
__device__ __forceinline__ int plan_need(const PlanBlocks& pb, int batch, int per) {
    const int lane = threadIdx.x & 63;
    int t = 0;
#pragma unroll
    for (int k = 0; k < kPlanRegs; ++k)
        if (64 * k + lane < batch) t += plan_splits(pb.nb[k], per);
    return wave_sum_i32(t);
}

// The plan of a launch of batch <= kPlanMaxBatch sequences: per > 0, the fewest-splits plan at `per` blocks per
// split (per = M ntl); per = 0, the proportional plan over T blocks.  If cap kPlanFewestCap - 1 fits, M is below
// kPlanFewestCap and the plan is proportional.  Otherwise M lies between max(kPlanFewestCap, ceil(T / (G ntl)))
// (the answer when the lengths are even) and ceil(Bmax / ntl) (one split each; batch <= G, so it fits):
// exponential, then binary search.
struct SplitPlanDev {
    int per, T;
};
__device__ inline SplitPlanDev split_plan(const PlanBlocks& pb, int batch, int G, int ntl, int qgroup) {
    int t = 0, bmax = 0;
#pragma unroll
    for (int k = 0; k < kPlanRegs; ++k) {
        t += pb.nb[k];
        bmax = max(bmax, pb.nb[k]);
    }
    const int T = wave_sum_i32(t);
    if (qgroup != 1 || plan_need(pb, batch, (kPlanFewestCap - 1) * ntl) <= G) return SplitPlanDev{0, T};
    bmax = wave_max_i32(bmax);
    const uint32_t gn = (uint32_t)G * ntl;  // (block counts fit 31 bits)
    int lo = max(kPlanFewestCap, (int)(((uint32_t)T + gn - 1) / gn));
    int good = max(lo, (bmax + ntl - 1) / ntl);  // fits; the least M that fits lies in [lo, good]
    if (plan_need(pb, batch, lo * ntl) <= G) {
        good = lo;
    } else {  // lo does not fit
        for (int step = 1; lo + step < good; step *= 2) {
            if (plan_need(pb, batch, (lo + step) * ntl) <= G) {
                good = lo + step;
                break;
            }
            lo += step;
        }
        while (good - lo > 1) {
            const int mid = lo + (good - lo) / 2;
            if (plan_need(pb, batch, mid * ntl) <= G) good = mid;
            else lo = mid;
        }
    }
    return SplitPlanDev{__builtin_amdgcn_readfirstlane(good * ntl), T};
}

struct SplitSlot {
    int b;    // sequence, or -1 if workgroup w has none
    int s;    // split index within the sequence
    int S_b;  // splits of the sequence
};

// Workgroups W0 .. W1 - 1 of the sequence whose count (splits, or blocks for the proportional plan) is x and
// whose predecessors' counts add up to `before`.
__device__ __forceinline__ void plan_range(const SplitPlanDev& pl, int b, int x, int before, int extra, int* W0,
                                           int* W1) {
    *W0 = pl.per ? before : first_workgroup(b, before, extra, pl.T);
    *W1 = pl.per ? before + x : first_workgroup(b + 1, before + x, extra, pl.T);
}

// Scan step over one chunk of 64 sequences (sequence c0 + lane, count x): the slot of workgroup w if it lies in
// the chunk; `carry` is the counts of the sequences before the chunk and grows by the chunk's.
__device__ __forceinline__ bool plan_scan_chunk(const SplitPlanDev& pl, int c0, int batch, int x, int extra, int w,
                                                int* carry, SplitSlot* out) {
    const int lane = threadIdx.x & 63, b = c0 + lane;
    const int incl = wave_incl_scan_i32(x);  // inclusive scan over the lanes of this chunk
    int W0, W1;
    plan_range(pl, b, x, *carry + incl - x, extra, &W0, &W1);
    const unsigned long long hit = __ballot(b < batch && w >= W0 && w < W1);
    if (hit) {
        const int src = __builtin_ctzll(hit);
        *out = SplitSlot{__builtin_amdgcn_readlane(b, src), w - __builtin_amdgcn_readlane(W0, src),
                         __builtin_amdgcn_readlane(W1 - W0, src)};
        return true;
    }
    *carry += __builtin_amdgcn_readlane(incl, 63);
    return false;
}

// the slot's values are wave-uniform; readfirstlane lets the compiler keep them (and every block offset derived
// from them) in scalar registers
__device__ __forceinline__ SplitSlot uniform_slot(SplitSlot x) {
    return SplitSlot{__builtin_amdgcn_readfirstlane(x.b), __builtin_amdgcn_readfirstlane(x.s),
                     __builtin_amdgcn_readfirstlane(x.S_b)};
}

// The (sequence, split) that workgroup w of a G-workgroup launch handles.
__device__ inline SplitSlot split_slot(const int32_t* seq_lens, int batch, int max_len, int G, int granule,
                                      int qgroup, int w, int append_cap = 0) {
    const int lane = threadIdx.x & 63, extra = G - batch;
    SplitSlot out{-1, 0, 0};
    int carry = 0;
    if (batch <= kPlanMaxBatch) {
        const PlanBlocks pb = plan_blocks(seq_lens, batch, max_len, append_cap);
        const SplitPlanDev pl = split_plan(pb, batch, G, max(1, granule >> 5), qgroup);
#pragma unroll
        for (int k = 0; k < kPlanRegs; ++k) {
            if (64 * k >= batch) break;
            const int x = pl.per ? (64 * k + lane < batch ? plan_splits(pb.nb[k], pl.per) : 0) : pb.nb[k];
            if (plan_scan_chunk(pl, 64 * k, batch, x, extra, w, &carry, &out)) break;
        }
        return uniform_slot(out);
    }
    // larger batches: the proportional plan, the lengths read once for the total and once for the scan
    int t = 0;
    for (int i = lane; i < batch; i += 64) t += len_blocks(clamped_len(seq_lens, i, max_len, append_cap));
    const SplitPlanDev pl{0, wave_sum_i32(t)};
    for (int c0 = 0; c0 < batch; c0 += 64) {
        const int b = c0 + lane;
        const int x = (b < batch) ? len_blocks(clamped_len(seq_lens, b, max_len, append_cap)) : 0;
        if (plan_scan_chunk(pl, c0, batch, x, extra, w, &carry, &out)) break;
    }
    return uniform_slot(out);
}

// First workgroup W_b and split count S_b of sequence b.
__device__ inline void sequence_splits(const int32_t* seq_lens, int batch, int max_len, int G, int granule,
                                       int qgroup, int b, int* W_b, int* S_b, int append_cap = 0) {
    const int lane = threadIdx.x & 63, extra = G - batch;
    const int nbk = len_blocks(clamped_len(seq_lens, b, max_len, append_cap));
    SplitPlanDev pl;
    int before = 0;
    if (batch <= kPlanMaxBatch) {
        const PlanBlocks pb = plan_blocks(seq_lens, batch, max_len, append_cap);
        pl = split_plan(pb, batch, G, max(1, granule >> 5), qgroup);
#pragma unroll
        for (int k = 0; k < kPlanRegs; ++k)
            if (64 * k + lane < b) before += pl.per ? plan_splits(pb.nb[k], pl.per) : pb.nb[k];
    } else {
        int t = 0;
        for (int i = lane; i < batch; i += 64) {
            const int nb = len_blocks(clamped_len(seq_lens, i, max_len, append_cap));
            t += nb;
            if (i < b) before += nb;
        }
        pl = SplitPlanDev{0, wave_sum_i32(t)};
    }
    before = wave_sum_i32(before);
    int W0, W1;
    plan_range(pl, b, pl.per ? plan_splits(nbk, pl.per) : nbk, before, extra, &W0, &W1);
    *W_b = __builtin_amdgcn_readfirstlane(W0);
    *S_b = __builtin_amdgcn_readfirstlane(W1 - W0);
}

}  // namespace lrkv
