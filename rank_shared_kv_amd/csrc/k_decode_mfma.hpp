// MFMA split kernel for bf16 LRKV decode on gfx950 (CDNA4, wave64).
//
// What one step computes, per sequence b and head h (fp32 arithmetic):
//   s_j = (q_h . k_j + p_h . z^K_{h,j}) / sqrt(d_h)    p_h = q_h B^K_h (absorbed)
//   a   = softmax(s) over the live rows j < L_b          (one softmax, summed logits)
//   o_h = sum_j a_j v_j + (sum_j a_j z^V_{h,j}) (B^V_h)^T
// ("Low-Rank Key Value Attention: Chinese reading notes", sec. 2.4,
// Eqs. (6)-(7); "Low-Rank Key Value Attention | What a shared cache can
// preserve", sec. 3, Algorithm 2 and the fused online-softmax paragraph after
// it).  This kernel produces, for every (b, split of `chunk` rows, h), the
// online-softmax state of that split: running max m (log2 units), denominator
// l, shared numerator sum_j e_j v_j (d_h) and private numerator
// sum_j e_j z^V_{h,j} (r).  The merge kernel combines splits and applies B^V.
//
// Work decomposition.  A workgroup of 4 waves owns one (b, split).  Each wave
// handles one group of 16 heads (the MFMA N dimension) on one "row lane": the
// 32-row blocks tl, tl + NTL, ... of the split, where NTL = 4 / head groups.
// Shared key/value rows of a block are read from HBM once per block and serve
// every head of the group; with two head groups the second wave of the same
// row lane re-reads them from the L2 of the same CU.  At the end the waves of
// a head group merge their states in LDS in a fixed order and the workgroup
// writes one record per head.
//
// Per 32-row block (one wave, 16 heads):
//   * shared scores S^T[row][head] = K_s[32 x d_h] Q^T[d_h x 16] on MFMA
//     (v_mfma_f32_16x16x32_bf16, exact bf16 products, fp32 accumulation); the
//     key fragments are loaded from HBM straight into the MFMA A layout;
//   * the value tile is transposed into LDS (V^T[d_h][32 rows]);
//   * private scores p_h . z^K_{h,j} on the VALU: latent rows are read from HBM
//     into registers, 8 lanes per head (each lane owns r/8 coordinates); the
//     latents are stored token-major, so one load instruction reads one token's
//     latents of 8 consecutive heads, 8*r*2 contiguous bytes; the 8 partial dots
//     of 8 rows are combined by a 3-stage transpose-reduce over lanes (DPP half
//     mirror, xor 2, xor 1) that leaves each lane with one finished score;
//   * scores meet in the MFMA result layout (lane = one head, 8 rows) through a
//     small LDS exchange; online softmax there (max across lanes xor 16, 32);
//   * shared values O^T[d_h x 16] += V^T[d_h x 32] P^T[32 x 16] on MFMA, with P
//     split into bf16 hi + lo parts (two MFMAs) so the weights keep ~16 bits;
//   * private values acc_pr[h] += e_j z^V_{h,j} on the VALU in the latent layout,
//     the weights read back from the LDS exchange.
// All global loads of a block -- key fragments, value tile, latent units --
// form one sequence of equal-sized "units" that runs through a ring of NSLOT
// register slots, NSLOT - 1 units ahead of the arithmetic (across blocks too).
// Loads are buffer loads: the lane-dependent part of an address is a 32-bit
// VGPR offset fixed for the whole kernel, the block/octet part is a scalar
// offset and the row within the block an immediate, so no vector arithmetic is
// spent on addresses.  Rows are kept inside the allocation by construction
// (L_cap is a multiple of 32 and blocks start on multiples of 32); rows past a
// sequence's length inside its last block are masked (scores) or zeroed
// (values), never used.
//
// Several query tokens (QW = 2 or 4, multi-token decode): a workgroup serves
// QW consecutive query tokens of one sequence from a single pass over its rows.
// Every loaded unit feeds all of them: the key fragments go into QW score
// products, the V^T tile into QW value products, and each latent register
// into QW private dots and QW private-value updates.  Each token keeps its own
// softmax state and is causally masked at its own length; the padding slots of
// a last, partial set see no row.  Records are [workgroup][QW][H].
//
// Normalised variant (NORM): the key of every (head, token) is RMS-normalised
// as a whole, and its cached reciprocal scale multiplies the summed logit
// ("Low-Rank Key Value Attention | What a shared cache can preserve", sec. 8,
// post-projection normalisation; the gain is already folded into q).  Each
// lane reads the 8 scales of its scores (2 bytes each) at the top of a block;
// they are used at the combine step, half a block of loads later.
//
// The template is instantiated in k_decode_mfma_part*.hip, one (d_h, NORM)
// set per translation unit so they compile in parallel.
#pragma once

#include "lrkv_device.hpp"
#include "lrkv_internal.hpp"
#include "lrkv_step.hpp"

namespace lrkv {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4_t;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2_t;

constexpr int kRows = 32;   // rows per block
constexpr int kWaves = 4;   // waves per workgroup
// Cache-policy bits of the streamed loads: 2 = non-temporal.  When a launch reads every latent row once
// (one query set per cached sequence: single-token decode, or multi-token decode with Q <= qw), marking
// those loads non-temporal raises the stream rate (long context: split pass 177 us against 195 us; a plain
// streaming read of 1 GiB goes from 6.3 to 7.0 TB/s the same way).  With several query sets per sequence
// the sets re-read the same rows through L2, so those launches keep ordinary loads (the NTL template flag
// of the kernel, chosen per launch).  Shared key/value rows are re-read through L2 (split key lines,
// second head group) and keep ordinary loads.
// Waves of a workgroup advance block by block together (one barrier per block) in single-token decode: the
// second head-group wave's shared-row loads then hit more often in L2 (long context: HBM read 1.176 GB per
// launch instead of 1.188 GB, split pass 1.3% faster)
#ifndef LRKV_LOCKSTEP
#define LRKV_LOCKSTEP 1
#endif
#ifndef LRKV_NT_LATENT
#define LRKV_NT_LATENT 1
#endif
#ifndef LRKV_NT_SHARED
#define LRKV_NT_SHARED 0
#endif
template <bool NTL>
constexpr int kNTLat = (LRKV_NT_LATENT && NTL) ? 2 : 0;
constexpr int kNTSh = LRKV_NT_SHARED ? 2 : 0;

template <int D, int R, int H, int OCC, int QW = 1>
struct Cfg {
    // Latent slices: 8 lanes per head, lane sl owns the EPL coordinates from sl*EPL (the last lane: the rest,
    // TAIL of them).  In the plain form (R a multiple of 8, H a multiple of 8) a lane's coordinates start on a
    // dword and fill LDW dwords.  In the general form (GEN) every lane loads a window of LDL dwords from a
    // token's latent row that holds its coordinates and lies inside the row: lanes 0..6 from the even element
    // at or below their first coordinate, the last lane ending at its head's end (rounded up to an even
    // element); a lane's coordinates then sit at window positions off .. off + own - 1, and the positions
    // around them (neighbouring lanes' or heads' values) are masked out of the private score.
    static constexpr int EPL = (R + 7) / 8;             // latent coordinates per lane
    static constexpr bool REAL = EPL > 1 && !(R % 2 == 0 && EPL % 2 == 0);  // lanes may start on an odd element
    static constexpr int LDW = (EPL + 1) / 2;           // dwords per lane and row (EPL = 1 uses one dword)
    static constexpr int LDL = REAL ? (EPL + 2) / 2 : LDW;  // dwords per latent load
    static constexpr int NHG = (H + 15) / 16;           // head groups (16 heads: MFMA N)
    static constexpr int NTL = kWaves / NHG;            // row lanes per workgroup
    static constexpr int OCTS = (H >= 16) ? 2 : (H + 7) / 8;  // octets (8 head slots) per head group
    static constexpr int HS = 16 * (NHG - 1) + 8 * OCTS;     // head slots the octets cover (padding slots: >= H)
    // GEN: head slots past H or a partial last slice -- the general form of the addressing and masks
    // (shapes with H a multiple of 8 and R a multiple of 8 compile to the plain form)
    static constexpr bool GEN = (HS != H) || (8 * EPL != R);
    static constexpr int TAIL = (R - 7 * EPL > 0) ? R - 7 * EPL : 0;  // coordinates of a head's last lane
    static constexpr int NPOS = GEN ? 2 * LDL : EPL;   // latent values a lane accumulates per row (window positions)
    static constexpr int KSTEPS = D / 32;               // k-steps of the score MFMA
    static constexpr int CB = D / 16;                   // 16-column blocks of the value MFMA
    static constexpr int LPR = D / 8;                   // lanes per shared row (16 B each)
    static constexpr int RPI = 64 / LPR;                // shared rows per load instruction
    static constexpr int NINS = kRows / RPI;            // load instructions per value tile
    static constexpr int NLU = (R > 0) ? 8 * OCTS : 0;  // latent units per block (K then V)
    static constexpr int NU = 2 + NLU;                  // + key-fragment unit + value-tile unit
    static constexpr int KDW = 8 * KSTEPS;              // dwords of the key unit
    static constexpr int VDW = 4 * NINS;                // dwords of the value unit
    static constexpr int LUDW = 8 * LDL;                // dwords of a latent unit
    static constexpr int SLOT_DW = (KDW > VDW ? (KDW > LUDW ? KDW : LUDW) : (VDW > LUDW ? VDW : LUDW));
    // ring depth: as deep as the register budget allows.  OCC = waves per SIMD (2: 256 registers per
    // wave, 1: 512); each query a wave serves takes (d_h + r) / 2 + 16 accumulator registers from it.
    // The depth must divide the per-block unit count so slots repeat every block.
    static constexpr int pick_slots() {
        const int budget = (OCC == 2) ? 96 : (QW == 1) ? 200 : (QW == 2) ? 160 : (H <= 16) ? 96 : 64;  // ring registers
        const int cand[6] = {9, 6, 5, 4, 3, 2};
        for (int i = 0; i < 6; ++i)
            if (NU % cand[i] == 0 && cand[i] * SLOT_DW <= budget) return cand[i];
        return (NU % 2 == 0) ? 2 : 1;
    }
    static constexpr int NSLOT = pick_slots();
    static constexpr int QROW = D + 8;                  // bf16 per q row in LDS (16 B pad)
    // floats per p row in LDS: 8 slices of LDL high and LDL low pairs (matrix-core dot path), or R floats
    static constexpr int PROW = (EPL >= 2 ? 16 * LDL : R) + 4;
    static constexpr int VTS = kRows + 4;               // bf16 per V^T row in LDS (72 B: conflict-free reads)
    static constexpr int XS = 36;                       // floats per exchange row (32 rows + alpha + pad)
    static constexpr int REC = ((D + R + 2) + 3) & ~3;
    static constexpr int Q_BYTES = QW * NHG * 16 * QROW * 2;        // q rows of each query, head-group padded
    static constexpr int P_BYTES = ((QW * HS * PROW * 4) + 15) & ~15;
    static constexpr int MW_BYTES = kWaves * 16 * 4;
    static constexpr int VT_BYTES = ((D * VTS * 2) + 15) & ~15;
    static constexpr int X_BYTES = QW * 16 * XS * 4;                   // one exchange area per query
    static constexpr int WAVE_BYTES = VT_BYTES + X_BYTES;
    static constexpr int LDS_BYTES = Q_BYTES + P_BYTES + MW_BYTES + kWaves * WAVE_BYTES;
    static constexpr int MERGE_BYTES = H * REC * 4;
    static_assert(MERGE_BYTES <= kWaves * WAVE_BYTES, "merge area must fit in the per-wave tiles");
    static_assert(NU % NSLOT == 0, "ring must divide the unit sequence");
    static_assert(H % 2 == 0 && H <= 32 && (H % 8 == 0 || GEN), "head count");
    // general form: the windows of lanes 0..6 end inside their head's coordinates or the next head's, never past
    // the row (the last lane's window ends at its head's end), and the last lane has coordinates of its own
    static_assert(!GEN || (EPL >= 2 && 6 * EPL + 2 * LDL <= R && TAIL >= 1 && 2 * LDL >= TAIL + (R % 2)),
                  "latent windows");
    static_assert(QW == 1 || QW == 2 || QW == 4, "queries per wave");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS");
};

__device__ __forceinline__ uint32_t pack_lo(uint32_t a, uint32_t b) {  // (a.lo16, b.lo16)
    return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) {  // (a.hi16, b.hi16)
    return __builtin_amdgcn_perm(b, a, 0x07060302u);
}
__device__ __forceinline__ float lat_at(const uint32_t* w, int e) {
    return (e & 1) ? bf16_hi(w[e >> 1]) : bf16_lo(w[e >> 1]);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t v4u_t __attribute__((ext_vector_type(4)));
typedef uint32_t v3u_t __attribute__((ext_vector_type(3)));
typedef uint32_t v2u_t __attribute__((ext_vector_type(2)));

// DPP lane exchanges within rows of 16 lanes (no LDS traffic)
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7 - i within each 8 lanes
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// dot of two bf16 pairs accumulated into fp32 (v_dot2_f32_bf16); operands are plain
// scalars, never vector subscripts, before the bit casts
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c, false);
}

// raw buffer descriptor over [base, base + bytes)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// General form: the latent window of lane sl of a real head h (its first coordinate, its element offset in the
// row, the window position of that coordinate, the number of its coordinates); see Cfg.
struct LatWindow {
    int first, start, off, own;
};
template <int R, int EPL, int LDL>
__device__ __forceinline__ LatWindow lat_window(int h, int sl) {
    LatWindow w;
    if (sl < 7) {
        w.first = sl * EPL;
        w.own = EPL;
        const int e0 = h * R + w.first;
        w.start = e0 & ~1;
        w.off = e0 & 1;
    } else {
        w.first = 7 * EPL;
        w.own = R - 7 * EPL;
        int end = (h + 1) * R;
        end += end & 1;
        w.start = end - 2 * LDL;
        w.off = h * R + w.first - w.start;
    }
    return w;
}

// Fused decode step (STEP): LDS of the absorb workgroups (per wave: q staged as floats, then the row-group
// partial sums) and the byte offset of the finish flag, past them.
constexpr int kStepAbsorbWaveFloats = 256 + 64 * 8;
constexpr int kStepFlagByte = kWaves * kStepAbsorbWaveFloats * 4;
constexpr int kStepLdsMin = kStepFlagByte + 16;

// Absorb and merge roles of the fused step.
template <int D, int R, int H>
__device__ __forceinline__ void step_absorb_role(const DecodeArgs& a, unsigned char* lds, int wave, int lane) {
    if constexpr (R > 0) {
        // four (sequence, head) units per workgroup, one per wave; each wave releases its p row, then counts it in
        // ready[b]
        const int u = (int)blockIdx.x * kWaves + wave;
        if (u < a.batch * H) {
            float* qs = (float*)lds + wave * kStepAbsorbWaveFloats;
            absorb_wave<uint16_t, true>(u, H, D, R, (const uint16_t*)a.q, (const uint16_t*)a.B_k, a.p_out, qs,
                                        qs + 256);
            __builtin_amdgcn_s_waitcnt(0);  // this wave's p stores are done before the count
            if (lane == 0)
                __hip_atomic_fetch_add(a.sync + kStepHeader + u / H, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

template <int D, int R, int H>
__device__ __forceinline__ void step_merge_role(const DecodeArgs& a, unsigned char* lds) {
    // one (sequence, head) per workgroup, once every split workgroup of the sequence is done
    const int m = (int)blockIdx.x - a.n_absorb - a.num_splits;
    const int mb = m / H, mh = m - mb * H;
    uint32_t* done = a.sync + kStepHeader + a.batch + mb;
    uint32_t* sync = a.sync;
    auto wait = [=](int S_b) { step_wait(done, (uint32_t)S_b, sync); };
    float* sums = (float*)lds;
    if (a.merge_wide)
        merge_body<uint16_t, 4, true>(mh, mb, a.batch, 1, 1, H, D, R, a.max_len, a.append_cap, a.chunk, a.num_splits,
                                      a.seq_lens, (const uint16_t*)a.B_v, a.out, a.ws, sums, wait);
    else
        merge_body<uint16_t, 1, true>(mh, mb, a.batch, 1, 1, H, D, R, a.max_len, a.append_cap, a.chunk, a.num_splits,
                                      a.seq_lens, (const uint16_t*)a.B_v, a.out, a.ws, sums, wait);
    step_finish(a.sync, a.n_merge, a.batch, a.L_cap, a.seq_lens_rw, (int*)(lds + kStepFlagByte));
}

template <int D, int R, int H, int OCC, bool NORM, int QW, bool NTL, bool STEP = false>
__global__ void __launch_bounds__(kWaves * 64, OCC) split_mfma_kernel(DecodeArgs a) {
    using C = Cfg<D, R, H, OCC, QW>;
    static_assert(!(NORM && QW > 1), "the normalised variant serves one query per sequence");
    static_assert(!STEP || (QW == 1 && !NORM), "the fused step serves one query per sequence, plain decode");
    constexpr int EPL = C::EPL, LDW = C::LDW, LDL = C::LDL, OCTS = C::OCTS, NU = C::NU, NSLOT = C::NSLOT,
                  SDW = C::SLOT_DW, HS = C::HS, NPOS = C::NPOS;
    constexpr bool kDot2 = EPL >= 2;  // private score on v_dot2 (p split into bf16 hi + lo)
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    uint16_t* q_lds = (uint16_t*)lds;
    uint32_t* p_lds = (uint32_t*)(lds + C::Q_BYTES);
    float* mw_lds = (float*)(lds + C::Q_BYTES + C::P_BYTES);
    unsigned char* wave_base = lds + C::Q_BYTES + C::P_BYTES + C::MW_BYTES;

    // the wave index is uniform across a wave; saying so keeps every block offset in SGPRs
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hg = wave % C::NHG, tl = wave / C::NHG;  // head group, row lane
    unsigned char* my = wave_base + wave * C::WAVE_BYTES;
    uint16_t* vt = (uint16_t*)my;
    float* xb = (float*)(my + C::VT_BYTES);

    // Fused decode step: workgroups [0, n_absorb) absorb, the next num_splits split, the rest merge.  The
    // absorb and merge workgroups run their bodies (lrkv_step.hpp) here and leave.  Only the merge workgroups
    // count themselves finished: the last of them finishes after every split workgroup has read the lengths
    // (each merge waited for every split of its sequence) and after every absorb count was seen (by the splits).
    int wid = blockIdx.x;  // this workgroup's index among the split workgroups
    if constexpr (STEP) {
        if ((int)blockIdx.x < a.n_absorb) {
            step_absorb_role<D, R, H>(a, lds, wave, lane);
            return;
        }
        if ((int)blockIdx.x >= a.n_absorb + a.num_splits) {
            step_merge_role<D, R, H>(a, lds);
            return;
        }
        wid = (int)blockIdx.x - a.n_absorb;
    }

    // Which sequence and split this workgroup handles (splits dealt to sequences by length), and
    // which 32-row blocks its row lanes take: blocks are dealt round-robin over the (split, row lane)
    // slots of the sequence, slot (split, tl) takes blocks split*NTL + tl + k*S_b*NTL.
    const SplitSlot wslot = split_slot(a.seq_lens, a.batch, a.max_len, a.num_splits, a.chunk, a.qgroup, wid,
                                         a.append_cap);
    const int b = wslot.b, split = wslot.s;
    // fused step: after the records are out (stores done), count this workgroup in done[b]
    auto step_end = [&]() {
        if constexpr (STEP) step_publish(b >= 0 ? a.sync + kStepHeader + a.batch + b : nullptr);
    };
    if (b < 0) {
        step_end();
        return;
    }
    // uniform: readfirstlane keeps it (and every loop bound and block offset derived from it) in SGPRs also where
    // the compiler cannot prove the lengths unwritten (the fused step writes global memory before the loop)
    const int Lb = __builtin_amdgcn_readfirstlane(clamped_len(a.seq_lens, b, a.max_len, a.append_cap));
    if constexpr (STEP) {
        // The appended token's rows (row L0 = stored length, when below L_cap), written before anything reads
        // them: by the workgroup whose slot owns their block when the decode sees them, else by split 0.
        const int L0 = __builtin_amdgcn_readfirstlane(a.seq_lens[b]);
        if (L0 >= 0 && L0 < a.L_cap) {
            const int owner = (L0 < Lb) ? ((L0 / kRows) % (wslot.S_b * C::NTL)) / C::NTL : 0;
            if (split == owner) {
                append_row_copy<uint16_t>(b, L0, H, D, R, a.L_cap, (uint16_t*)a.k_shared, (uint16_t*)a.v_shared,
                                          (uint16_t*)a.z_k, (uint16_t*)a.z_v, (const uint16_t*)a.k_new,
                                          (const uint16_t*)a.v_new, (const uint16_t*)a.zk_new,
                                          (const uint16_t*)a.zv_new, nullptr, 0, 0);
                __builtin_amdgcn_s_waitcnt(0);  // the rows are in this XCD's L2 before any wave loads them
                __syncthreads();
            }
        }
    }
    if (split * a.chunk >= Lb) {  // whole workgroup: no live rows in this split
        step_end();
        return;
    }
    const int nb = (Lb + kRows - 1) / kRows;  // blocks of this sequence
    const int bc = b / a.qgroup;  // the cached sequence this (virtual) sequence reads

    // Query rows served by this workgroup.  QW == 1: the row of sequence b (virtual sequence b of a
    // multi-token decode).  QW > 1 (multi-token decode of n_queries tokens per sequence): virtual sequence b
    // is token set c = b % qgroup of cached sequence bc, tokens c*QW .. c*QW + nreal - 1; token qi of the set
    // sees Lq[qi] rows, the set's last token Lb of them (the virtual length), each earlier token one row
    // fewer.  Padding slots qi >= nreal see no row and their records are never read.
    int q_row0 = b, nreal = 1;
    int Lq[QW];
    Lq[0] = Lb;
    if constexpr (QW > 1) {
        const int c = b - bc * a.qgroup;
        nreal = min(QW, a.n_queries - c * QW);
        q_row0 = bc * a.n_queries + c * QW;
#pragma unroll
        for (int qi = 0; qi < QW; ++qi) Lq[qi] = (qi < nreal) ? max(0, Lb - (nreal - 1 - qi)) : 0;
    }
    const uint16_t* qg = (const uint16_t*)a.q + (size_t)q_row0 * H * D;

    // ---- q (zero rows pad a partial head group and the padding query slots) and p into LDS ----
    // LDS q row (qi, head) sits at qi * 16 * NHG + head; p row (qi, head) at qi * H + head
    auto stage_q = [&]() {
        for (int i = tid; i < QW * C::NHG * 16 * D; i += kWaves * 64) {
            const int hq = i / D, c = i - hq * D;
            const int qi = (QW == 1) ? 0 : hq / (C::NHG * 16), h = hq - qi * (C::NHG * 16);
            q_lds[hq * C::QROW + c] = (h < H && qi < nreal) ? qg[(qi * H + h) * D + c] : (uint16_t)0;
        }
    };
    // the fused step stages q after the first cache loads have been issued (their round trip then covers the q
    // loads; 0.8 us per step at the long-context shape), except at two waves per SIMD, where q's registers
    // would spill
    constexpr bool kQLate = STEP && OCC == 1;
    if constexpr (!kQLate) stage_q();
    auto stage_p = [&]() {
    if constexpr (R > 0) {
        const float* pg = a.p + (size_t)q_row0 * H * R;
        if constexpr (C::GEN) {
            // per (query, head slot) and lane: LDL pairs of high parts, then LDL of low parts, in the order of the
            // lane's latent window (position j holds p of coordinate first + j - off, or 0 where the position is
            // not one of the lane's coordinates, or the slot is a padding head or query)
            for (int i = tid; i < QW * HS * 8 * LDL; i += kWaves * 64) {
                const int h = i / (8 * LDL), rem = i - h * (8 * LDL);
                const int slice = rem / LDL, t = rem - slice * LDL;
                const int qi = h / HS, hl = h - qi * HS;
                const bool live = hl < H && (QW == 1 || qi < nreal);
                const LatWindow lw = lat_window<R, EPL, LDL>(live ? hl : 0, slice);
                const int j0 = 2 * t - lw.off, j1 = j0 + 1;  // the positions' coordinates within the lane's own
                const bool ok0 = live && j0 >= 0 && j0 < lw.own, ok1 = live && j1 >= 0 && j1 < lw.own;
                const float* prow = pg + (size_t)(qi * H + (live ? hl : 0)) * R + lw.first;
                const float x0 = ok0 ? ld_f32<STEP>(prow + j0) : 0.f, x1 = ok1 ? ld_f32<STEP>(prow + j1) : 0.f;
                const uint32_t h0 = f32_to_bf16_bits(x0), h1 = f32_to_bf16_bits(x1);
                const uint32_t l0 = f32_to_bf16_bits(x0 - __uint_as_float(h0 << 16));
                const uint32_t l1 = f32_to_bf16_bits(x1 - __uint_as_float(h1 << 16));
                uint32_t* row = p_lds + h * C::PROW + slice * 2 * LDL;
                row[t] = h0 | (h1 << 16);
                row[LDL + t] = l0 | (l1 << 16);
            }
        } else if constexpr (kDot2) {
            // per head and r-slice of EPL coordinates: EPL/2 pairs of high parts, then EPL/2 of low parts
            for (int i = tid; i < QW * H * (R / 2); i += kWaves * 64) {
                const int h = i / (R / 2), pr = i - h * (R / 2);  // pair index within the (query, head) row
                const int slice = pr / (EPL / 2), j = pr - slice * (EPL / 2);
                const bool live = QW == 1 || h < nreal * H;
                const float x0 = live ? ld_f32<STEP>(pg + h * R + 2 * pr) : 0.f;
                const float x1 = live ? ld_f32<STEP>(pg + h * R + 2 * pr + 1) : 0.f;
                const uint32_t h0 = f32_to_bf16_bits(x0), h1 = f32_to_bf16_bits(x1);
                const uint32_t l0 = f32_to_bf16_bits(x0 - __uint_as_float(h0 << 16));
                const uint32_t l1 = f32_to_bf16_bits(x1 - __uint_as_float(h1 << 16));
                uint32_t* row = p_lds + h * C::PROW + slice * EPL;
                row[j] = h0 | (h1 << 16);
                row[EPL / 2 + j] = l0 | (l1 << 16);
            }
        } else {
            for (int i = tid; i < QW * H * R; i += kWaves * 64) {
                const int h = i / R, k = i - h * R;
                p_lds[h * C::PROW + k] = (QW == 1 || h < nreal * H) ? __float_as_uint(ld_f32<STEP>(pg + i)) : 0u;
            }
        }
    }
    };
    // fused step: p is staged after the first cache loads are on their way and the absorb of this sequence
    // is done (below)
    if constexpr (!STEP) stage_p();
    for (int i = lane; i < QW * 16 * C::XS; i += 64) xb[i] = 0.f;
    if constexpr (!STEP) __syncthreads();

    const int n16 = lane & 15, g4 = lane >> 4;  // MFMA layout: column (head or value column), row group
    const int hh = lane >> 3, sl = lane & 7;    // latent layout: head within octet, coordinate slice
    const bool sb0 = sl & 1, sb1 = (sl >> 1) & 1, sb2 = (sl >> 2) & 1;
    const int srow = lane / C::LPR, schunk = lane % C::LPR;  // value-tile load layout
    const float scale = kLog2e / sqrtf((float)D);

    f32x4_t acc_sh[QW][C::CB];
    float acc_pr[QW][OCTS][NPOS > 0 ? NPOS : 1];
    float m_run[QW], l_run[QW];
#pragma unroll
    for (int qi = 0; qi < QW; ++qi) {
        m_run[qi] = -INFINITY;
        l_run[qi] = 0.f;
#pragma unroll
        for (int cb = 0; cb < C::CB; ++cb) acc_sh[qi][cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int o = 0; o < OCTS; ++o)
#pragma unroll
            for (int e = 0; e < NPOS; ++e) acc_pr[qi][o][e] = 0.f;
    }

    // ---- buffer descriptors of this sequence and fixed per-lane byte offsets ----
    // latents are token-major ([L_cap][H][r] per sequence): one latent row holds every head
    const uint32_t row_bytes_sh = D * 2, row_bytes_lat = H * R * 2;
    // contiguous cache: descriptors over this sequence's rows, a block addressed by its row t0; paged cache:
    // descriptors over the whole page pools, a block addressed by its pool row (pages hold whole blocks)
    const bool paged = a.block_table != nullptr;  // never in the fused step (its launches pass no block table)
    // pool row of logical row t of this sequence (t when contiguous), uniform
    // pool row of logical row t of this sequence (t when contiguous).  readfirstlane: the row is uniform, and
    // where the kernel writes global memory before the loop (the fused step) the compiler cannot tell that the
    // block table is unchanged and would otherwise keep the row, and every block offset, in VGPRs
    auto prow = [&](int t) { return __builtin_amdgcn_readfirstlane(paged_row(a, bc, t)); };
    const size_t seq_rows = paged ? 0 : (size_t)bc * a.L_cap;
    const uint32_t n_rows = paged ? (uint32_t)a.n_pages << a.page_shift : (uint32_t)a.L_cap;
    const __amdgpu_buffer_rsrc_t rs_k = buf_rsrc((const uint16_t*)a.k_shared + seq_rows * D, n_rows * row_bytes_sh);
    const __amdgpu_buffer_rsrc_t rs_v = buf_rsrc((const uint16_t*)a.v_shared + seq_rows * D, n_rows * row_bytes_sh);
    __amdgpu_buffer_rsrc_t rs_zk = rs_k, rs_zv = rs_v;
    uint32_t vo_zv = 0;  // lane offset of (head 16*hg + hh, coordinate slice sl) in the latent tensors
    // general form: the lane's window offset in a latent row per octet (a padding head slot gets an offset out
    // of every descriptor's range, so its loads return zeros and touch no memory), and per-pair masks that keep
    // the lane's own coordinates of the window
    uint32_t vo_oct[OCTS];
    uint32_t lat_mask[LDL > 0 ? LDL : 1];
    if constexpr (R > 0) {
        const uint32_t lat_bytes = n_rows * row_bytes_lat;
        rs_zk = buf_rsrc((const uint16_t*)a.z_k + seq_rows * H * R, lat_bytes);
        rs_zv = buf_rsrc((const uint16_t*)a.z_v + seq_rows * H * R, lat_bytes);
        if constexpr (C::GEN) {
#pragma unroll
            for (int oi = 0; oi < OCTS; ++oi) {
                const int h = 16 * hg + 8 * oi + hh;
                vo_oct[oi] = (h < H) ? (uint32_t)lat_window<R, EPL, LDL>(h, sl).start * 2 : 0x80000000u;
            }
            // a lane's window positions depend on its head only through the parity of head * R
            const LatWindow lw = lat_window<R, EPL, LDL>(hh & 1, sl);
#pragma unroll
            for (int t = 0; t < LDL; ++t) {
                const int j0 = 2 * t - lw.off, j1 = j0 + 1;
                lat_mask[t] = ((j0 >= 0 && j0 < lw.own) ? 0x0000ffffu : 0u) | ((j1 >= 0 && j1 < lw.own) ? 0xffff0000u : 0u);
            }
        } else {
            vo_zv = (uint32_t)(16 * hg + hh) * R * 2 + sl * EPL * 2;
        }
    }
    const uint32_t vo_kf = (uint32_t)n16 * row_bytes_sh + 16 * g4;              // key fragment rows n16, 16 + n16
    const uint32_t vo_vt = (uint32_t)(4 * srow) * row_bytes_sh + 16 * schunk;  // value tile rows 4*srow + 0..3
    const uint32_t oct_bytes = 8u * R * 2;  // next head octet within a latent row
    // normalised variant: the cached scale of (row, head) multiplies the summed logit; this lane's scores are
    // head 16*hg + n16 at rows 4*g4 + i and 16 + 4*g4 + i of a block (scales token-major: [L_cap][H])
    __amdgpu_buffer_rsrc_t rs_rho = rs_k;
    uint32_t vo_rho = 0;
    if constexpr (NORM) {
        rs_rho = buf_rsrc((const uint16_t*)a.rho + (size_t)bc * a.L_cap * H, (uint32_t)a.L_cap * H * 2);
        vo_rho = (uint32_t)(4 * g4 * H + 16 * hg + n16) * 2;
    }

    // ---- the load ring ----
    uint32_t ring[NSLOT][SDW];
    // a descriptor of no bytes: every load through it is out of range, returns zeros and touches no memory.
    // During a row lane's last block there is no next block to prefetch; its latent units (non-temporal, so a
    // re-read would go back to memory) then go through this descriptor, while the key and value units re-read
    // the current block from L2.
    const __amdgpu_buffer_rsrc_t rs_none = buf_rsrc(a.k_shared, 0);

    // unit u of the block whose first row sits at (pool) row pr, into ring slot `slot`; live = false sends
    // the latent loads through the empty descriptor
    auto issue = [&](int u, int pr, int slot, bool live) {
        if (u == 0) {  // key fragments in the MFMA A layout: rows 16*half + n16, chunk 4*kk + g4
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const int so = (pr + 16 * half) * (int)row_bytes_sh;
#pragma unroll
                for (int kk = 0; kk < C::KSTEPS; ++kk) {
                    const v4u_t v = __builtin_amdgcn_raw_buffer_load_b128(rs_k, vo_kf + 64 * kk, so, kNTSh);
                    const int o = 4 * (half * C::KSTEPS + kk);
                    ring[slot][o] = v.x;
                    ring[slot][o + 1] = v.y;
                    ring[slot][o + 2] = v.z;
                    ring[slot][o + 3] = v.w;
                }
            }
        } else if (u == 1) {  // value tile, rows 4*srow + (ins & 3) + 4*RPI*(ins >> 2)
#pragma unroll
            for (int grp = 0; grp < C::NINS / 4; ++grp) {
                const int so = (pr + 4 * C::RPI * grp) * (int)row_bytes_sh;
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int ins = 4 * grp + jj;
                    const v4u_t v = __builtin_amdgcn_raw_buffer_load_b128(rs_v, vo_vt + jj * row_bytes_sh, so, kNTSh);
                    ring[slot][4 * ins] = v.x;
                    ring[slot][4 * ins + 1] = v.y;
                    ring[slot][4 * ins + 2] = v.z;
                    ring[slot][4 * ins + 3] = v.w;
                }
            }
        } else if constexpr (R > 0) {  // latent unit: phase (K, V), octet, 8-row sub-block
            const int v = u - 2;
            const int phase = v / (4 * OCTS);
            const int oi = (v % (4 * OCTS)) / 4, sub = v % 4;
            // general form: the octet is in the lane's window offset; plain form: in the scalar offset
            const int so = pr * (int)row_bytes_lat + (C::GEN ? 0 : oi * (int)oct_bytes);
            const __amdgpu_buffer_rsrc_t rs = !live ? rs_none : (phase == 0) ? rs_zk : rs_zv;
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                // one instruction reads row 8*sub + k of 8 consecutive heads: 8*r*2 contiguous bytes
                const uint32_t vo = (C::GEN ? vo_oct[oi] : vo_zv) + (k + 8 * sub) * row_bytes_lat;
                if constexpr (LDL == 4) {
                    const v4u_t w = __builtin_amdgcn_raw_buffer_load_b128(rs, vo, so, kNTLat<NTL>);
                    ring[slot][4 * k] = w.x;
                    ring[slot][4 * k + 1] = w.y;
                    ring[slot][4 * k + 2] = w.z;
                    ring[slot][4 * k + 3] = w.w;
                } else if constexpr (LDL == 3) {
                    const v3u_t w = __builtin_amdgcn_raw_buffer_load_b96(rs, vo, so, kNTLat<NTL>);
                    ring[slot][3 * k] = w.x;
                    ring[slot][3 * k + 1] = w.y;
                    ring[slot][3 * k + 2] = w.z;
                } else if constexpr (LDL == 2) {
                    const v2u_t w = __builtin_amdgcn_raw_buffer_load_b64(rs, vo, so, kNTLat<NTL>);
                    ring[slot][2 * k] = w.x;
                    ring[slot][2 * k + 1] = w.y;
                } else if constexpr (EPL == 2) {
                    ring[slot][k] = __builtin_amdgcn_raw_buffer_load_b32(rs, vo, so, kNTLat<NTL>);
                } else {  // EPL == 1
                    ring[slot][k] = __builtin_amdgcn_raw_buffer_load_b16(rs, vo, so, kNTLat<NTL>);
                }
            }
        }
    };

    const int first_blk = split * C::NTL + tl, step_blk = wslot.S_b * C::NTL, last_blk = nb;
    const int nmine = (last_blk > first_blk) ? (last_blk - first_blk + step_blk - 1) / step_blk : 0;
    // Sequence b walks its blocks starting b/batch of the way along (the same blocks, rotated order).
    // Otherwise every sequence reads the same relative position of its cache region at the same time,
    // and with some region strides those concurrent streams crowd the same HBM channels.
    // (the virtual sequences of one cached sequence share its rotation, so they read the same rows together)
    const int rot = mul_div_floor(nmine, bc, a.batch / a.qgroup);
    if (nmine > 0) {
        const int pr_first = prow(kRows * (first_blk + rot * step_blk));
#pragma unroll
        for (int u = 0; u < NSLOT - 1; ++u) {
            issue(u, pr_first, u, true);
            // in unit order, as the loop issues them: the wait counts at the loop head then hold for both ways
            // into it (scheduled freely, the loads forced waits that left less than half the ring in flight)
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    if constexpr (STEP) {
        // the absorb workgroups' p rows of this sequence (H units), then p into LDS; the barrier inside the
        // wait also orders the q rows staged above
        if constexpr (kQLate) stage_q();
        if constexpr (R > 0) step_wait(a.sync + kStepHeader + b, (uint32_t)H, a.sync);
        stage_p();
        __syncthreads();
    }

#if LRKV_LOCKSTEP
    // Every wave runs row lane 0's trip count, which depends only on (split, length, S_b) and so is the same
    // across the workgroup: the barrier at the top of an iteration is reached equally often by every wave
    // (a wave past its own blocks only takes the barrier).  The waves then move block by block together,
    // and the two head-group waves of a row lane read the same shared rows at nearly the same time.
    // Only with two head groups (no duplicate fetch to save otherwise: one group measured 0.5-4% slower
    // with it) and without virtual sequences (multi-token decode: the barrier cost 7-11%).
    const bool lockstep = C::NHG > 1 && a.qgroup == 1;  // compile-time and a kernel argument: the same for every wave
    const int n_all = !lockstep ? nmine
                      : (last_blk > split * C::NTL) ? (last_blk - split * C::NTL + step_blk - 1) / step_blk : 0;
    for (int it = 0; it < n_all; ++it) {
        if (lockstep) __syncthreads();
        if (it >= nmine) continue;
#else
    for (int it = 0; it < nmine; ++it) {
#endif
        int itr = it + rot;
        if (itr >= nmine) itr -= nmine;
        const int blk = first_blk + itr * step_blk;
        const int t0 = kRows * blk;
        const int nvalid = min(kRows, Lb - t0);
        // next block of this row lane; on the last block there is none, and the prefetch goes through the
        // empty descriptor (same addresses as this block, no memory traffic)
        const int itn = (itr + 1 < nmine) ? itr + 1 : 0;
        const bool pf_live = it + 1 < nmine;
        const int t0_pf = pf_live ? kRows * (first_blk + itn * step_blk) : t0;
        const int pr = prow(t0), pr_pf = prow(t0_pf);  // pool rows (t0 when contiguous)
        f32x4_t s_sh[QW][2];
        uint32_t rho_w[8];  // scales of this lane's 8 scores (bf16 bits), read at the top of the block
        if constexpr (NORM) {
            const int so = t0 * H * 2;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                rho_w[i] = __builtin_amdgcn_raw_buffer_load_b16(rs_rho, vo_rho + i * H * 2, so, 0);
                rho_w[4 + i] = __builtin_amdgcn_raw_buffer_load_b16(rs_rho, vo_rho + (16 + i) * H * 2, so, 0);
            }
        }

#pragma unroll
        for (int u = 0; u < NU; ++u) {
            // keep NSLOT - 1 units in flight ahead of this one
            {
                const int un = u + NSLOT - 1;
                if (un < NU) issue(un, pr, un % NSLOT, true);
                else issue(un - NU, pr_pf, un % NSLOT, pf_live);
            }
            // fence the scheduler at unit boundaries: loads stay NSLOT - 1 units ahead, no further
            __builtin_amdgcn_sched_barrier(0);
            const uint32_t* cur = ring[u % NSLOT];
            if (u == 0) {
                // shared scores on MFMA (both 16-row halves)
#pragma unroll
                for (int half = 0; half < 2; ++half) {
#pragma unroll
                    for (int qi = 0; qi < QW; ++qi) {  // every query against the same key fragments
                        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int kk = 0; kk < C::KSTEPS; ++kk) {
                            const int o = 4 * (half * C::KSTEPS + kk);
                            const u32x4_t av = {cur[o], cur[o + 1], cur[o + 2], cur[o + 3]};
                            const u32x4_t bv = *(const u32x4_t*)(q_lds + (qi * C::NHG * 16 + 16 * hg + n16) * C::QROW +
                                                                 32 * kk + 8 * g4);
                            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                __builtin_bit_cast(bf16x8_t, av), __builtin_bit_cast(bf16x8_t, bv), acc, 0, 0, 0);
                        }
                        s_sh[qi][half] = acc;
                    }
                }
            } else if (u == 1) {
                // value tile -> V^T in LDS: vt[c][row], 4 consecutive rows per 8-byte store;
                // rows past the sequence end are zeroed (their weight is 0, their content arbitrary)
#pragma unroll
                for (int grp = 0; grp < C::NINS / 4; ++grp) {
                    const int t4 = 4 * srow + 4 * C::RPI * grp;
                    const bool ok0 = t4 < nvalid, ok1 = t4 + 1 < nvalid, ok2 = t4 + 2 < nvalid, ok3 = t4 + 3 < nvalid;
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const int c = 8 * schunk + j;
                        const uint32_t w0 = ok0 ? cur[4 * (4 * grp + 0) + (j >> 1)] : 0u;
                        const uint32_t w1 = ok1 ? cur[4 * (4 * grp + 1) + (j >> 1)] : 0u;
                        const uint32_t w2 = ok2 ? cur[4 * (4 * grp + 2) + (j >> 1)] : 0u;
                        const uint32_t w3 = ok3 ? cur[4 * (4 * grp + 3) + (j >> 1)] : 0u;
                        u32x2_t pk;
                        pk[0] = (j & 1) ? pack_hi(w0, w1) : pack_lo(w0, w1);
                        pk[1] = (j & 1) ? pack_hi(w2, w3) : pack_lo(w2, w3);
                        *(u32x2_t*)(vt + c * C::VTS + t4) = pk;
                    }
                }
                if constexpr (R == 0) {
                    // no private branch: zero private scores
#pragma unroll
                    for (int qi = 0; qi < QW; ++qi)
#pragma unroll
                        for (int oi = 0; oi < OCTS; ++oi)
#pragma unroll
                            for (int sub = 0; sub < 4; ++sub)
                                xb[(qi * 16 + 8 * oi + hh) * C::XS + 8 * sub + sl] = 0.f;
                }
            } else if constexpr (R > 0) {
                const int v = u - 2;
                const int phase = v / (4 * OCTS);
                const int oi = (v % (4 * OCTS)) / 4, sub = v % 4;
                if (phase == 0) {
#pragma unroll
                    for (int qi = 0; qi < QW; ++qi) {  // every query against the same latent registers
                        constexpr int NPW = kDot2 ? 2 * LDL : EPL;  // p dwords of a lane slice
                        uint32_t pw[NPW];
#pragma unroll
                        for (int e = 0; e < NPW; ++e)
                            pw[e] = p_lds[(qi * HS + 16 * hg + 8 * oi + hh) * C::PROW + sl * NPW + e];
                        float part[8];
#pragma unroll
                        for (int k = 0; k < 8; ++k) {
                            float acc = 0.f;
                            if constexpr (kDot2) {
#pragma unroll
                                for (int pr = 0; pr < LDL; ++pr) {
                                    uint32_t z = cur[LDL * k + pr];
                                    // window positions that are not the lane's coordinates (a neighbouring lane's
                                    // or head's values) have p = 0 but are zeroed too: nothing there is assumed
                                    if constexpr (C::GEN) z &= lat_mask[pr];
                                    acc = dot2_bf16(z, pw[LDL + pr], acc);  // low parts of p
                                    acc = dot2_bf16(z, pw[pr], acc);        // high parts of p
                                }
                            } else {
#pragma unroll
                                for (int e = 0; e < EPL; ++e)
                                    acc = fmaf(__uint_as_float(pw[e]), lat_at(cur + LDW * k, e), acc);
                            }
                            part[k] = acc;
                        }
                        // transpose-reduce across the 8 lanes of a head: part[k] is this lane's slice of
                        // row k.  Stage 1 pairs lanes sl, 7-sl (half mirror) and each keeps the rows whose
                        // bit 2 equals its own; stages 2 and 3 do the same on bits 1 and 0 with lanes
                        // sl^2 and sl^1.  Lane sl ends with the whole score of row 8*sub + sl.
                        float q4[4], q2[2];
#pragma unroll
                        for (int k = 0; k < 4; ++k) {
                            const float keep = sb2 ? part[k + 4] : part[k];
                            const float send = sb2 ? part[k] : part[k + 4];
                            q4[k] = keep + dpp<kDppHalfMirror>(send);
                        }
#pragma unroll
                        for (int k = 0; k < 2; ++k) {
                            const float keep = sb1 ? q4[k + 2] : q4[k];
                            const float send = sb1 ? q4[k] : q4[k + 2];
                            q2[k] = keep + dpp<kDppXor2>(send);
                        }
                        const float keep = sb0 ? q2[1] : q2[0];
                        const float send = sb0 ? q2[0] : q2[1];
                        xb[(qi * 16 + 8 * oi + hh) * C::XS + 8 * sub + sl] = keep + dpp<kDppXor1>(send);
                    }
                } else {
                    if (sub == 0) {
#pragma unroll
                        for (int qi = 0; qi < QW; ++qi) {
                            const float al = xb[(qi * 16 + 8 * oi + hh) * C::XS + 32];
#pragma unroll
                            for (int e = 0; e < NPOS; ++e) acc_pr[qi][oi][e] *= al;
                        }
                    }
                    f32x4_t e0[QW], e1[QW];
#pragma unroll
                    for (int qi = 0; qi < QW; ++qi) {
                        e0[qi] = *(const f32x4_t*)(xb + (qi * 16 + 8 * oi + hh) * C::XS + 8 * sub);
                        e1[qi] = *(const f32x4_t*)(xb + (qi * 16 + 8 * oi + hh) * C::XS + 8 * sub + 4);
                    }
#pragma unroll
                    for (int k = 0; k < 8; ++k) {
                        // rows past the sequence end: weight 0, content arbitrary (rows a query token does not
                        // see are live rows of the sequence with weight 0)
                        if (8 * sub + k < nvalid) {
#pragma unroll
                            for (int e = 0; e < NPOS; ++e) {
                                const float z = lat_at(cur + LDL * k, e);
#pragma unroll
                                for (int qi = 0; qi < QW; ++qi)
                                    acc_pr[qi][oi][e] = fmaf((k < 4) ? e0[qi][k] : e1[qi][k - 4], z, acc_pr[qi][oi][e]);
                            }
                        }
                    }
                }
            }

            // after the last key unit: combine, online softmax, shared values
            if (u == 1 + C::NLU / 2) {
                wave_lds_sync();
                // one query at a time: softmax of its scores, its weights and alpha into its exchange area (for
                // the private values), then its shared-value products; each lane reads and rewrites only its
                // own score slots, so no exchange between the queries' passes is needed
#pragma unroll
                for (int qi = 0; qi < QW; ++qi) {
                    // rows of this block that query qi sees (the sequence's rows when QW == 1)
                    const int nvq = (QW == 1) ? nvalid : Lq[qi] - t0;
                    float* xq = xb + qi * 16 * C::XS;
                    float sc[8];
                    const f32x4_t pa = *(const f32x4_t*)(xq + n16 * C::XS + 4 * g4);
                    const f32x4_t pb = *(const f32x4_t*)(xq + n16 * C::XS + 16 + 4 * g4);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int r0 = 4 * g4 + i, r1 = 16 + 4 * g4 + i;
                        float f0 = scale, f1 = scale;
                        if constexpr (NORM) {
                            f0 = scale * __uint_as_float(rho_w[i] << 16);
                            f1 = scale * __uint_as_float(rho_w[4 + i] << 16);
                        }
                        sc[i] = (r0 < nvq) ? (s_sh[qi][0][i] + pa[i]) * f0 : -INFINITY;
                        sc[4 + i] = (r1 < nvq) ? (s_sh[qi][1][i] + pb[i]) * f1 : -INFINITY;
                    }
                    float tmax = sc[0];
#pragma unroll
                    for (int i = 1; i < 8; ++i) tmax = fmaxf(tmax, sc[i]);
                    tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
                    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
                    const float m_new = fmaxf(m_run[qi], tmax);
                    // with several queries a block can hold no row for an earlier token (m_new = -inf while
                    // nothing was seen yet): subtract 0 instead so that alpha and the weights are 0, not NaN
                    const float m_sub = (QW > 1 && m_new == -INFINITY) ? 0.f : m_new;
                    const float alpha = fast_exp2(m_run[qi] - m_sub);
                    m_run[qi] = m_new;
                    float ev[8];
                    float esum = 0.f;
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        ev[i] = fast_exp2(sc[i] - m_sub);
                        esum += ev[i];
                    }
                    l_run[qi] = fmaf(alpha, l_run[qi], esum);
                    wave_lds_sync();  // every lane has read its private scores
                    *(f32x4_t*)(xq + n16 * C::XS + 4 * g4) = f32x4_t{ev[0], ev[1], ev[2], ev[3]};
                    *(f32x4_t*)(xq + n16 * C::XS + 16 + 4 * g4) = f32x4_t{ev[4], ev[5], ev[6], ev[7]};
                    if (g4 == 0) xq[n16 * C::XS + 32] = alpha;

                    // shared values on MFMA: O^T += V^T P^T with P = hi + lo (bf16)
                    u32x4_t phi, plo;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const uint32_t h0 = f32_to_bf16_bits(ev[2 * i]), h1 = f32_to_bf16_bits(ev[2 * i + 1]);
                        const float r0 = ev[2 * i] - __uint_as_float(h0 << 16);
                        const float r1 = ev[2 * i + 1] - __uint_as_float(h1 << 16);
                        phi[i] = h0 | (h1 << 16);
                        plo[i] = f32_to_bf16_bits(r0) | (f32_to_bf16_bits(r1) << 16);
                    }
#pragma unroll
                    for (int cb = 0; cb < C::CB; ++cb) {
                        acc_sh[qi][cb] *= alpha;
                        const int c = 16 * cb + n16;
                        const u32x2_t v0 = *(const u32x2_t*)(vt + c * C::VTS + 4 * g4);
                        const u32x2_t v1 = *(const u32x2_t*)(vt + c * C::VTS + 16 + 4 * g4);
                        const uint32_t a0 = v0[0], a1 = v0[1], a2 = v1[0], a3 = v1[1];
                        const u32x4_t av = {a0, a1, a2, a3};
                        const bf16x8_t a8 = __builtin_bit_cast(bf16x8_t, av);
                        acc_sh[qi][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a8, __builtin_bit_cast(bf16x8_t, phi),
                                                                                acc_sh[qi][cb], 0, 0, 0);
                        acc_sh[qi][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a8, __builtin_bit_cast(bf16x8_t, plo),
                                                                                acc_sh[qi][cb], 0, 0, 0);
                    }
                }
                wave_lds_sync();  // weights and alphas visible to the private-value units
            }
        }
        wave_lds_sync();  // V^T and weights consumed before the next block rewrites them
    }
    // the block loop has a run-time trip count and can end on a value product: wait for the matrix cores
    // before the accumulators are read below
    mfma_result_fence();

    // ---- merge the row lanes of each head group (fixed order), one record per (query, head) ----
    // (records of workgroup w = W_b + split: [QW][H] at (w * QW + qi) * H; the next query's pass starts
    // with a barrier after every wave has copied this one's records out)
#pragma unroll
    for (int qi = 0; qi < QW; ++qi) {
        float l_q = l_run[qi];
        l_q += __shfl_xor(l_q, 16);
        l_q += __shfl_xor(l_q, 32);
        if (g4 == 0) mw_lds[wave * 16 + n16] = m_run[qi];
        __syncthreads();  // all waves done with their tiles (or the previous query's copy); maxima visible
        float* mg = (float*)wave_base;  // [H][REC], aliases the per-wave areas
        float M = -INFINITY;
        for (int t = 0; t < C::NTL; ++t) M = fmaxf(M, mw_lds[(t * C::NHG + hg) * 16 + n16]);
        const float fsh = (m_run[qi] == -INFINITY) ? 0.f : fast_exp2(m_run[qi] - M);
        float fpr[OCTS];
#pragma unroll
        for (int oi = 0; oi < OCTS; ++oi) {
            const int n = 8 * oi + hh;
            float Mo = -INFINITY;
            for (int t = 0; t < C::NTL; ++t) Mo = fmaxf(Mo, mw_lds[(t * C::NHG + hg) * 16 + n]);
            const float mine = mw_lds[wave * 16 + n];
            fpr[oi] = (mine == -INFINITY) ? 0.f : fast_exp2(mine - Mo);
        }
        const int head = 16 * hg + n16;
        for (int t = 0; t < C::NTL; ++t) {
            if (tl == t && head < H) {
                float* row = mg + head * C::REC;
#pragma unroll
                for (int cb = 0; cb < C::CB; ++cb) {
                    const f32x4_t v = acc_sh[qi][cb] * fsh;
                    f32x4_t* dst = (f32x4_t*)(row + 16 * cb + 4 * g4);
                    *dst = (t == 0) ? v : (*dst + v);
                }
                if (g4 == 0) {
                    const float lv = l_q * fsh;
                    row[D + R + 1] = (t == 0) ? lv : row[D + R + 1] + lv;
                    if (t == 0) row[D + R] = M;
                }
            }
            if (tl == t) {
                // general form: window position j holds coordinate first + j - off of the lane's own
                LatWindow lw{sl * EPL, 0, 0, EPL};
                if constexpr (C::GEN) lw = lat_window<R, EPL, LDL>(hh & 1, sl);
#pragma unroll
                for (int oi = 0; oi < OCTS; ++oi) {
                    const int hs = 16 * hg + 8 * oi + hh;
                    if (C::GEN && hs >= H) continue;  // padding head slot
                    float* row = mg + hs * C::REC + D + lw.first;
#pragma unroll
                    for (int e = 0; e < NPOS; ++e) {
                        if (C::GEN && (e < lw.off || e >= lw.off + lw.own)) continue;  // not the lane's coordinate
                        const float v = acc_pr[qi][oi][e] * fpr[oi];
                        const int c = e - lw.off;
                        row[c] = (t == 0) ? v : row[c] + v;
                    }
                }
            }
            __syncthreads();
        }
        float* out = a.ws + ((size_t)wid * QW + qi) * H * C::REC;
        // fused step: agent-coherent stores, for the merge workgroups of the same launch
        for (int i = tid; i < H * C::REC; i += kWaves * 64) st_f32<STEP>(out + i, mg[i]);
    }
    step_end();
}

template <int D, int R, int H, int OCC, bool NORM, int QW, bool NTL = true>
hipError_t launch_one(const DecodeArgs& a, hipStream_t stream) {
    using C = Cfg<D, R, H, OCC, QW>;
    auto kern = split_mfma_kernel<D, R, H, OCC, NORM, QW, NTL>;
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS_BYTES);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(a.num_splits), dim3(kWaves * 64), C::LDS_BYTES, stream, a);
    return hipGetLastError();
}

// Fused decode step: absorb workgroups, split workgroups and merge workgroups in one launch.
template <int D, int R, int H, int OCC>
hipError_t launch_step_one(const DecodeArgs& a, hipStream_t stream) {
    using C = Cfg<D, R, H, OCC, 1>;
    auto kern = split_mfma_kernel<D, R, H, OCC, false, 1, true, true>;
    constexpr int kLds = C::LDS_BYTES > kStepLdsMin ? C::LDS_BYTES : kStepLdsMin;
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, kLds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(a.n_absorb + a.num_splits + a.n_merge), dim3(kWaves * 64), kLds, stream, a);
    return hipGetLastError();
}

template <int D, int R, int H>
hipError_t launch_step_dhr(const DecodeArgs& a, int occ, hipStream_t stream) {
    return occ == 1 ? launch_step_one<D, R, H, 1>(a, stream) : launch_step_one<D, R, H, 2>(a, stream);
}

template <int D, int H>
hipError_t launch_step_r(const DecodeArgs& a, int occ, hipStream_t stream) {
    switch (a.r) {
        case 0: return launch_step_dhr<D, 0, H>(a, occ, stream);
        case 8: return launch_step_dhr<D, 8, H>(a, occ, stream);
        case 16: return launch_step_dhr<D, 16, H>(a, occ, stream);
        case 32: return launch_step_dhr<D, 32, H>(a, occ, stream);
        case 48: return launch_step_dhr<D, 48, H>(a, occ, stream);
        case 64: return launch_step_dhr<D, 64, H>(a, occ, stream);
    }
    return hipErrorInvalidValue;
}

template <int D>
hipError_t launch_step_h(const DecodeArgs& a, int occ, hipStream_t stream) {
    switch (a.H) {
        case 8: return launch_step_r<D, 8>(a, occ, stream);
        case 16: return launch_step_r<D, 16>(a, occ, stream);
        case 32: return launch_step_r<D, 32>(a, occ, stream);
    }
    return hipErrorInvalidValue;
}

// Four queries per wave do not fit the register file at d_h = 128, r = 64 (the compiled kernel spills in its
// main loop); those shapes serve at most two (mfma_max_query_width, k_decode_mfma.hip).
template <int D, int R, int H>
constexpr bool query_width_fits(int qw) {
    return qw <= 2 || !(D == 128 && R == 64);
}

// the normalised variant and the several-query instances are built for one wave per SIMD only
template <int D, int R, int H, bool NORM, int QW>
hipError_t launch_dhr(const DecodeArgs& a, int occ, hipStream_t stream) {
    if constexpr (!query_width_fits<D, R, H>(QW)) return hipErrorInvalidValue;
    else if constexpr (QW > 1)  // non-temporal latent loads only with one query set per cached sequence
        return a.qgroup == 1 ? launch_one<D, R, H, 1, false, QW, true>(a, stream)
                             : launch_one<D, R, H, 1, false, QW, false>(a, stream);
    else if constexpr (NORM) return launch_one<D, R, H, 1, NORM, 1>(a, stream);
    else return occ == 1 ? launch_one<D, R, H, 1, false, 1>(a, stream) : launch_one<D, R, H, 2, false, 1>(a, stream);
}

template <int D, int H, bool NORM, int QW>
hipError_t launch_r(const DecodeArgs& a, int occ, hipStream_t stream) {
    switch (a.r) {
        case 0: return launch_dhr<D, 0, H, NORM, QW>(a, occ, stream);
        case 8: return launch_dhr<D, 8, H, NORM, QW>(a, occ, stream);
        case 16: return launch_dhr<D, 16, H, NORM, QW>(a, occ, stream);
        case 32: return launch_dhr<D, 32, H, NORM, QW>(a, occ, stream);
        case 48: return launch_dhr<D, 48, H, NORM, QW>(a, occ, stream);
        case 64: return launch_dhr<D, 64, H, NORM, QW>(a, occ, stream);
    }
    return hipErrorInvalidValue;
}

template <int D, bool NORM, int QW = 1>
hipError_t launch_h(const DecodeArgs& a, int occ, hipStream_t stream) {
    switch (a.H) {
        case 8: return launch_r<D, 8, NORM, QW>(a, occ, stream);
        case 16: return launch_r<D, 16, NORM, QW>(a, occ, stream);
        case 32: return launch_r<D, 32, NORM, QW>(a, occ, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace
}  // namespace lrkv
