// MFMA split kernel for fp32 decode with r = 0 on gfx950 (CDNA4, wave64).
//
// With rank 0 the factored cache holds only the shared key and value rows, and
// every head attends over them: the MQA special case of LRKV ("Low-Rank Key
// Value Attention: Chinese reading notes", sec. 2.1 and the cache table of
// sec. 1; "Low-Rank Key Value Attention | What a shared cache can preserve",
// sec. 3, where rank 0 removes the private branch).  Per sequence b and head h:
//   s_j = q_h . k_j / sqrt(d_h),  a = softmax(s),  o_h = sum_j a_j v_j.
// Both products are dense contractions over all heads of a group at once, so
// both run on the matrix cores with fp32 accumulation.  The value product uses
// v_mfma_f32_16x16x4f32 (fp32 products).  The score product takes its fp32
// operands to the bf16 matrix cores: every key and query value x is split
// exactly into three bf16 parts, x = x1 + x2 + x3 (x1 is x with the low 16
// bits of its pattern cleared, x2 the same of x - x1, x3 the rest, at most 8
// significant bits), and k q is taken as the six terms k1q1 + k1q2 + k2q1 +
// k1q3 + k2q2 + k3q1 on v_mfma_f32_16x16x32_bf16; the three left out are below
// 2^-21 |k q| together, against the 2^-24 of an fp32 product's rounding and
// the accumulation error of a 128-term dot product.  That is 16 matrix-core
// cycles per 32-column chunk and term, 96 for what takes 256 on the fp32
// matrix cores, at about five VALU operations per key value for the split.
// The kernel writes the same per-split online-softmax records as the bf16
// kernel; the merge kernel combines them.
//
// Decode step (STEP): the split pass also appends the new token.  Every
// sequence is seen at its appended length, and the workgroup whose split owns
// the appended row's block writes the row before its first load (the others
// never read that block).  Every workgroup counts itself finished at its end;
// the last of the launch, after every workgroup has read the lengths, grows
// them and clears the counter.  The merge kernel then runs on the grown
// lengths, which give it the plan this pass used, so the two launches give the
// results of lrkv_append_absorb followed by lrkv_decode bit for bit; no
// workgroup waits for another.  (Merging inside this launch, by the last split
// of each sequence, made the step slower: one workgroup per sequence then
// merges every head while the merge kernel spreads them over the GPU.)
//
// Work decomposition: a workgroup of 4 waves owns one (b, split), splits dealt
// to sequences by length; each wave is one row lane of 32-row blocks (blocks
// dealt round-robin over the sequence's (split, row lane) slots) and handles
// every head, in groups of 16 (MFMA N), so each key/value row is loaded by
// exactly one wave.  Per block and head group:
//   S^T[32 rows x 16 heads] = K[32 x d_h] Q^T         (two 16-row halves)
//   online softmax on S^T in the MFMA result layout (lane = head, 8 rows)
//   O^T[d_h x 16 heads]    += V^T[d_h x 32 rows] P^T
// The contraction index of each product is permuted so that every lane loads
// 16 contiguous bytes per global load and no cache operand goes through LDS:
//   * score product, 32-column chunk j of a half: lane (row n, group g)
//     supplies the parts of K[n][32 j + 4 g + e] and K[n][32 j + 16 + 4 g + e]
//     (e < 4; two 16-byte loads) and, from LDS where they are split once, of
//     q[head n][the same columns];
//   * value product, k-step t (rows of half t/4): lane (column slot n, group g)
//     supplies V[16 (t/4) + 4 g + t%4][64 p + 4 n + s] for column block
//     cb = 4 p + s, and P^T[that row][head] is exactly the softmax weight the
//     lane already holds from the score layout.
// The accumulator of column block cb = 4 p + s then holds, in lane (head n,
// group g) and register i, o_h at column 64 p + 16 g + 4 i + s.
#include "lrkv_device.hpp"
#include "lrkv_internal.hpp"
#include "lrkv_step.hpp"

// Cache policy of the value-row loads: non-temporal (2).  Each value row is read once, as whole 256-byte
// pieces; the split pass runs 240-242 us against 245-249 us with ordinary loads.  The key loads read half
// cache lines (the other half comes with the next instruction) and keep ordinary loads: non-temporal key
// and value loads together made the pass slower (254 us).
constexpr int kNTValue = 2;

namespace lrkv {
namespace {

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t v4u_t __attribute__((ext_vector_type(4)));
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;

// (a.hi16, b.hi16): the high halves of two fp32 bit patterns, packed as two bf16 values
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x07060302u); }

// Exact three-way bf16 split of 8 fp32 values x = x1 + x2 + x3: x1 is x with its low 16 bits cleared, x2 the same
// of x - x1 (exact), x3 = x - x1 - x2 (exact, at most 8 significant bits); packed as three bf16x8 operands.
__device__ __forceinline__ void split3(const float* x, v4u_t& p1, v4u_t& p2, v4u_t& p3) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t u0 = __float_as_uint(x[2 * j]), u1 = __float_as_uint(x[2 * j + 1]);
        const float r0 = x[2 * j] - __uint_as_float(u0 & 0xffff0000u);
        const float r1 = x[2 * j + 1] - __uint_as_float(u1 & 0xffff0000u);
        const uint32_t w0 = __float_as_uint(r0), w1 = __float_as_uint(r1);
        const float t0 = r0 - __uint_as_float(w0 & 0xffff0000u);
        const float t1 = r1 - __uint_as_float(w1 & 0xffff0000u);
        p1[j] = pack_hi(u0, u1);
        p2[j] = pack_hi(w0, w1);
        p3[j] = pack_hi(__float_as_uint(t0), __float_as_uint(t1));
    }
}

__device__ __forceinline__ f32x4_t mfma_bf(const v4u_t& a, const v4u_t& b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                   0, 0, 0);
}

constexpr int kRows = 32;
constexpr int kWaves = 4;

template <int D, int H, int OCC>
struct CfgF32 {
    static constexpr int NHG = (H + 15) / 16;        // head groups of 16 (MFMA N), all handled by every wave
    static constexpr int NTL = kWaves;                // row lanes per workgroup: one per wave
    static constexpr int KLD = D / 16;                // 16-byte loads per lane per key half
    static constexpr int VP = D / 64;                 // 64-column blocks of a value row
    static constexpr int KPH = D == 128 ? 4 : 2;      // key units per 16-row half
    static constexpr int LK = KLD / KPH;              // 16-byte key loads per lane and unit (even: whole chunks)
    static constexpr int VPU = D == 128 ? 4 : 2;      // value units per half
    static constexpr int TTU = 4 / VPU;               // row offsets tt per value unit
    static constexpr int UDW = 4 * LK;                // dwords per unit
    static constexpr int NU = 2 * KPH + 2 * VPU;      // units per block: the key units, then the value units
    // ring depth (divides NU), 64 dwords at two waves per SIMD, 128 at one: at d_h = 128 the ring holds 8 or 16
    // units of two loads, 14 or 30 loads ahead (units of four loads in 4 slots kept 12 ahead: 196.8 against
    // 193.4 us on the ragged fp32 pass); a 16-unit ring at two waves per SIMD spills
    static constexpr int NSLOT = D == 128 ? (OCC == 2 ? 8 : 16) : (OCC == 2 ? 4 : 8);
    static_assert(UDW == 4 * TTU * (D / 64) && LK % 2 == 0 && NU % NSLOT == 0, "unit shape");
    static constexpr int CB = D / 16;                 // column blocks of the value product
    static constexpr int KB = D / 32;                 // 32-column chunks of the score contraction
    static constexpr int REC = ((D + 2) + 3) & ~3;
    static constexpr int Q_BYTES = 3 * NHG * KB * 64 * 16;  // q's three bf16 parts in each lane's operand order
    static constexpr int MW_BYTES = kWaves * NHG * 16 * 4;
    static constexpr int LDS_BYTES = Q_BYTES + MW_BYTES + H * REC * 4;
    static_assert(D % 64 == 0, "head width");
    static_assert(H % 8 == 0 && H <= 32, "head count");
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// End of a decode-step workgroup: it counts itself finished; the last of the launch's workgroups grows the
// lengths and clears the counters (every workgroup has read the lengths by then).  flag: one int of LDS.
__device__ __forceinline__ void step_tail(const DecodeArgs& a, int* flag) {
    __syncthreads();  // the workgroup is done with its LDS and its lengths
    step_finish(a.sync, a.num_splits, a.batch, a.L_cap, a.seq_lens_rw, flag);
}

template <int D, int H, int OCC, bool STEP = false>
__global__ void __launch_bounds__(kWaves * 64, OCC) split_mfma_f32_kernel(DecodeArgs a) {
    using C = CfgF32<D, H, OCC>;
    constexpr int NSLOT = C::NSLOT, NU = C::NU, UDW = C::UDW, NHG = C::NHG;
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    v4u_t* qp_lds = (v4u_t*)lds;                             // [3][NHG][KB][64 lanes] q's bf16 parts
    float* mw_lds = (float*)(lds + C::Q_BYTES);              // [waves][NHG * 16] running maxima
    float* mg = (float*)(lds + C::Q_BYTES + C::MW_BYTES);   // [H][REC] merged records

    const int tid = threadIdx.x, lane = tid & 63, tl = __builtin_amdgcn_readfirstlane(tid >> 6);
    const SplitSlot wslot = split_slot(a.seq_lens, a.batch, a.max_len, a.num_splits, a.chunk, a.qgroup, blockIdx.x,
                                       a.append_cap);
    const int b = wslot.b, split = wslot.s;
    if (b < 0) {
        if constexpr (STEP) step_tail(a, (int*)lds);
        return;
    }
    const int Lb = __builtin_amdgcn_readfirstlane(clamped_len(a.seq_lens, b, a.max_len, a.append_cap));
    if constexpr (STEP) {
        // the appended token's rows (row L0 = stored length, when below L_cap), written before anything reads
        // them: by the workgroup whose split owns their block when the decode sees them, else by split 0
        const int L0 = __builtin_amdgcn_readfirstlane(a.seq_lens[b]);
        if (L0 >= 0 && L0 < a.L_cap) {
            const int owner = (L0 < Lb) ? ((L0 / kRows) % (wslot.S_b * C::NTL)) / C::NTL : 0;
            if (split == owner) {
                append_row_copy<float>(b, L0, H, D, 0, a.L_cap, (float*)a.k_shared, (float*)a.v_shared, nullptr,
                                       nullptr, (const float*)a.k_new, (const float*)a.v_new, nullptr, nullptr,
                                       nullptr, 0, 0);
                __builtin_amdgcn_s_waitcnt(0);  // the rows are in this XCD's L2 before any wave loads them
                __syncthreads();
            }
        }
    }
    if (split * a.chunk >= Lb) {  // whole workgroup: no live rows in this split
        if constexpr (STEP) step_tail(a, (int*)lds);
        return;
    }
    const int nb = (Lb + kRows - 1) / kRows;

    const int n16 = lane & 15, g4 = lane >> 4;
    const float scale = kLog2e / sqrtf((float)D);

    {
        // lane (head n, group g) of chunk j supplies q[head][32 j + 4 g + e] and q[head][32 j + 16 + 4 g + e], e < 4,
        // the columns the key operand's lane (row n, g) holds
        const float* qg = (const float*)a.q + (size_t)b * H * D;
        for (int i = tid; i < NHG * C::KB * 64; i += kWaves * 64) {
            const int ln = i & 63, gk = i >> 6;
            const int g = gk / C::KB, j = gk - g * C::KB;
            const int head = 16 * g + (ln & 15), gg = ln >> 4;
            float x[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                x[e] = head < H ? qg[(size_t)head * D + 32 * j + 4 * gg + e] : 0.f;
                x[4 + e] = head < H ? qg[(size_t)head * D + 32 * j + 16 + 4 * gg + e] : 0.f;
            }
            v4u_t p1, p2, p3;
            split3(x, p1, p2, p3);
            qp_lds[(0 * NHG * C::KB + gk) * 64 + ln] = p1;
            qp_lds[(1 * NHG * C::KB + gk) * 64 + ln] = p2;
            qp_lds[(2 * NHG * C::KB + gk) * 64 + ln] = p3;
        }
    }
    __syncthreads();

    const uint32_t row_bytes = D * 4;
    const int bc = b / a.qgroup;  // the cached sequence this (virtual) sequence reads
    const __amdgpu_buffer_rsrc_t rs_k = buf_rsrc((const float*)a.k_shared + (size_t)bc * a.L_cap * D,
                                                 (uint32_t)a.L_cap * row_bytes);
    const __amdgpu_buffer_rsrc_t rs_v = buf_rsrc((const float*)a.v_shared + (size_t)bc * a.L_cap * D,
                                                 (uint32_t)a.L_cap * row_bytes);
    const uint32_t vo_k = (uint32_t)n16 * row_bytes + 16 * g4;       // row n16 of the half, columns 4 g4 + 16 m
    const uint32_t vo_v = (uint32_t)(4 * g4) * row_bytes + 16 * n16;  // rows 4 g4 + tt, columns 64 p + 4 n16

    // Units of a block (NU, equal size, LK 16-byte loads per lane):
    //   u < 2 KPH        key half u / KPH, 16-column blocks m = LK (u % KPH) .. LK (u % KPH) + LK - 1
    //   u = 2 KPH + w    value half w / VPU, rows 4 g4 + tt with tt = TTU (w % VPU) .. TTU (w % VPU) + TTU - 1
    constexpr int KPH = C::KPH, LK = C::LK, VPU = C::VPU, TTU = C::TTU, NKU = 2 * KPH;
    uint32_t ring[NSLOT][UDW];
    // a descriptor of no bytes: loads through it are out of range, return zeros and touch no memory (the
    // prefetch issued during a row lane's last block, which has no next block)
    const __amdgpu_buffer_rsrc_t rs_none = buf_rsrc(a.k_shared, 0);
    auto issue = [&](int u, int t0, int slot, bool live) {
        if (u < NKU) {
            const int so = (t0 + 16 * (u / KPH)) * (int)row_bytes;
#pragma unroll
            for (int mm = 0; mm < LK; ++mm) {
                const int m = LK * (u % KPH) + mm;
                const v4u_t v = __builtin_amdgcn_raw_buffer_load_b128(live ? rs_k : rs_none, vo_k + 64 * m, so, 0);
                ring[slot][4 * mm] = v.x;
                ring[slot][4 * mm + 1] = v.y;
                ring[slot][4 * mm + 2] = v.z;
                ring[slot][4 * mm + 3] = v.w;
            }
        } else {
            const int so = (t0 + 16 * ((u - NKU) / VPU)) * (int)row_bytes;
#pragma unroll
            for (int k = 0; k < TTU; ++k) {
                const int tt = TTU * ((u - NKU) % VPU) + k;
#pragma unroll
                for (int p = 0; p < C::VP; ++p) {
                    const v4u_t v = __builtin_amdgcn_raw_buffer_load_b128(live ? rs_v : rs_none,
                                                                          vo_v + tt * row_bytes + 256 * p, so, kNTValue);
                    const int o = 4 * (k * C::VP + p);
                    ring[slot][o] = v.x;
                    ring[slot][o + 1] = v.y;
                    ring[slot][o + 2] = v.z;
                    ring[slot][o + 3] = v.w;
                }
            }
        }
    };

    f32x4_t acc[NHG][C::CB];
    float m_run[NHG], l_run[NHG];
#pragma unroll
    for (int g = 0; g < NHG; ++g) {
        m_run[g] = -INFINITY;
        l_run[g] = 0.f;
#pragma unroll
        for (int cb = 0; cb < C::CB; ++cb) acc[g][cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }

    // row lane tl of split s takes blocks s*NTL + tl + k*S_b*NTL of the sequence
    const int first_blk = split * C::NTL + tl, step_blk = wslot.S_b * C::NTL, last_blk = nb;
    const int nmine = (last_blk > first_blk) ? (last_blk - first_blk + step_blk - 1) / step_blk : 0;
    // sequence b walks its blocks starting b/batch of the way along (same blocks, rotated order; the
    // virtual sequences of one cached sequence share its rotation)
    const int rot = mul_div_floor(nmine, bc, a.batch / a.qgroup);
    if (nmine > 0) {
#pragma unroll
        for (int u = 0; u < NSLOT - 1; ++u) {
            issue(u, kRows * (first_blk + rot * step_blk), u, true);
            __builtin_amdgcn_sched_barrier(0);  // in unit order, as the loop issues them
        }
    }

    for (int it = 0; it < nmine; ++it) {
        int itr = it + rot;
        if (itr >= nmine) itr -= nmine;
        const int t0 = kRows * (first_blk + itr * step_blk);
        const int nvalid = min(kRows, Lb - t0);
        const int itn = (itr + 1 < nmine) ? itr + 1 : 0;
        const bool pf_live = it + 1 < nmine;  // the last block prefetches nothing (the empty descriptor)
        const int t0_pf = pf_live ? kRows * (first_blk + itn * step_blk) : t0;
        constexpr int NCH = (NHG == 1) ? 2 : 1;
        f32x4_t s_sh[NHG][2], s_acc[NHG][NCH];
        float ev[NHG][8];

#pragma unroll
        for (int u = 0; u < NU; ++u) {
            {
                const int un = u + NSLOT - 1;
                if (un < NU) issue(un, t0, un % NSLOT, true);
                else issue(un - NU, t0_pf, un % NSLOT, pf_live);
            }
            __builtin_amdgcn_sched_barrier(0);
            uint32_t* cur = ring[u % NSLOT];
            if (u < NKU) {
                // S^T of key half u/2 on the matrix cores, 16-column blocks of part u%2; q fragments from
                // LDS.  Two independent accumulation chains are interleaved (the head groups, or with one
                // group its even and odd column blocks) so consecutive MFMAs never wait on each other.
                if (u % KPH == 0) {
#pragma unroll
                    for (int g = 0; g < NHG; ++g)
#pragma unroll
                        for (int c = 0; c < NCH; ++c) s_acc[g][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                }
#pragma unroll
                for (int pp = 0; pp < LK / 2; ++pp) {
                    // loads 2 pp and 2 pp + 1 of the unit: columns 32 j + 4 g4 + e and 32 j + 16 + 4 g4 + e
                    const int j = (LK / 2) * (u % KPH) + pp;
                    float x[8];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        x[e] = __uint_as_float(cur[4 * (2 * pp) + e]);
                        x[4 + e] = __uint_as_float(cur[4 * (2 * pp + 1) + e]);
                    }
                    v4u_t k1, k2, k3;
                    split3(x, k1, k2, k3);
#pragma unroll
                    for (int g = 0; g < NHG; ++g) {
                        const int gk = g * C::KB + j;
                        const v4u_t q1 = qp_lds[(0 * NHG * C::KB + gk) * 64 + lane];
                        const v4u_t q2 = qp_lds[(1 * NHG * C::KB + gk) * 64 + lane];
                        const v4u_t q3 = qp_lds[(2 * NHG * C::KB + gk) * 64 + lane];
                        f32x4_t c = s_acc[g][pp % NCH];
                        c = mfma_bf(k3, q1, c);  // the six leading terms, smallest first
                        c = mfma_bf(k2, q2, c);
                        c = mfma_bf(k1, q3, c);
                        c = mfma_bf(k2, q1, c);
                        c = mfma_bf(k1, q2, c);
                        s_acc[g][pp % NCH] = mfma_bf(k1, q1, c);
                    }
                }
                if (u % KPH == KPH - 1) {
#pragma unroll
                    for (int g = 0; g < NHG; ++g)
                        s_sh[g][u / KPH] = (NCH == 2) ? s_acc[g][0] + s_acc[g][NCH - 1] : s_acc[g][0];
                }
                if (u == NKU - 1) {
                    // online softmax: lane (head n16 of group g, g4) holds rows 4 g4 + i and 16 + 4 g4 + i
#pragma unroll
                    for (int g = 0; g < NHG; ++g) {
                        float sc[8];
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            sc[i] = (4 * g4 + i < nvalid) ? s_sh[g][0][i] * scale : -INFINITY;
                            sc[4 + i] = (16 + 4 * g4 + i < nvalid) ? s_sh[g][1][i] * scale : -INFINITY;
                        }
                        float tmax = sc[0];
#pragma unroll
                        for (int i = 1; i < 8; ++i) tmax = fmaxf(tmax, sc[i]);
                        tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
                        tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
                        const float m_new = fmaxf(m_run[g], tmax);
                        const float alpha = fast_exp2(m_run[g] - m_new);
                        m_run[g] = m_new;
                        float esum = 0.f;
#pragma unroll
                        for (int i = 0; i < 8; ++i) {
                            ev[g][i] = fast_exp2(sc[i] - m_new);
                            esum += ev[g][i];
                        }
                        l_run[g] = fmaf(alpha, l_run[g], esum);
#pragma unroll
                        for (int cb = 0; cb < C::CB; ++cb) acc[g][cb] *= alpha;
                    }
                }
            } else {
                const int h = (u - NKU) / VPU;            // value half: rows 16 h + 4 g4 + tt
                const int tp = TTU * ((u - NKU) % VPU);  // this unit holds tt = tp .. tp + TTU - 1
                if (nvalid < kRows) {
                    // last block of the sequence: rows past the end hold arbitrary values; zero them
#pragma unroll
                    for (int k = 0; k < TTU; ++k)
                        if (16 * h + 4 * g4 + tp + k >= nvalid) {
#pragma unroll
                            for (int e = 0; e < 4 * C::VP; ++e) cur[4 * k * C::VP + e] = 0u;
                        }
                }
#pragma unroll
                for (int g = 0; g < NHG; ++g)
#pragma unroll
                    for (int k = 0; k < TTU; ++k)
#pragma unroll
                        for (int p = 0; p < C::VP; ++p)
#pragma unroll
                            for (int s = 0; s < 4; ++s) {
                                const int cb = 4 * p + s;
                                acc[g][cb] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                                    __uint_as_float(cur[4 * (k * C::VP + p) + s]), ev[g][4 * h + tp + k],
                                    acc[g][cb], 0, 0, 0);
                            }
            }
        }
    }

    // the block loop has a run-time trip count and ends on value products: wait for the matrix cores before
    // the accumulators are read below
    mfma_result_fence();

    // ---- merge the row lanes (fixed order), one record per head ----
#pragma unroll
    for (int g = 0; g < NHG; ++g) {
        l_run[g] += __shfl_xor(l_run[g], 16);  // every lane of a head holds the same partial sum of its rows
        l_run[g] += __shfl_xor(l_run[g], 32);
        if (g4 == 0) mw_lds[(tl * NHG + g) * 16 + n16] = m_run[g];
    }
    __syncthreads();
    float f[NHG], M[NHG];
#pragma unroll
    for (int g = 0; g < NHG; ++g) {
        M[g] = -INFINITY;
        for (int t = 0; t < C::NTL; ++t) M[g] = fmaxf(M[g], mw_lds[(t * NHG + g) * 16 + n16]);
        f[g] = (m_run[g] == -INFINITY) ? 0.f : fast_exp2(m_run[g] - M[g]);
    }
    for (int t = 0; t < C::NTL; ++t) {
        if (tl == t) {
#pragma unroll
            for (int g = 0; g < NHG; ++g) {
                const int head = 16 * g + n16;
                if (head < H) {
                    float* row = mg + head * C::REC;
#pragma unroll
                    for (int p = 0; p < C::VP; ++p)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const f32x4_t v = f32x4_t{acc[g][4 * p][i], acc[g][4 * p + 1][i], acc[g][4 * p + 2][i],
                                                      acc[g][4 * p + 3][i]} * f[g];
                            f32x4_t* dst = (f32x4_t*)(row + 64 * p + 16 * g4 + 4 * i);
                            *dst = (t == 0) ? v : (*dst + v);
                        }
                    if (g4 == 0) {
                        const float lv = l_run[g] * f[g];
                        row[D + 1] = (t == 0) ? lv : row[D + 1] + lv;
                        if (t == 0) row[D] = M[g];
                    }
                }
            }
        }
        __syncthreads();
    }
    float* out = a.ws + (size_t)blockIdx.x * H * C::REC;  // record of workgroup w = W_b + split
    for (int i = tid; i < H * C::REC; i += kWaves * 64) out[i] = mg[i];
    if constexpr (STEP) step_tail(a, (int*)lds);
}

template <int D, int H, int OCC, bool STEP>
hipError_t launch_one(const DecodeArgs& a, hipStream_t stream) {
    using C = CfgF32<D, H, OCC>;
    auto kern = split_mfma_f32_kernel<D, H, OCC, STEP>;
    hipLaunchKernelGGL(kern, dim3(a.num_splits), dim3(kWaves * 64), C::LDS_BYTES, stream, a);
    return hipGetLastError();
}

template <int D, bool STEP>
hipError_t launch_h(const DecodeArgs& a, int occ, hipStream_t stream) {
    switch (a.H) {
        case 8: return occ == 1 ? launch_one<D, 8, 1, STEP>(a, stream) : launch_one<D, 8, 2, STEP>(a, stream);
        case 16: return occ == 1 ? launch_one<D, 16, 1, STEP>(a, stream) : launch_one<D, 16, 2, STEP>(a, stream);
        case 32: return occ == 1 ? launch_one<D, 32, 1, STEP>(a, stream) : launch_one<D, 32, 2, STEP>(a, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace

int mfma_f32_rows_per_tile() { return kRows * kWaves; }

bool mfma_f32_path_supports(int H, int d_h, int r, int dtype, int L_cap) {
    if (dtype != 0 || r != 0) return false;
    if (L_cap % kRows != 0) return false;  // blocks never leave the allocation
    if ((long long)L_cap * d_h * 4 >= (1LL << 31)) return false;  // 32-bit buffer offsets
    if (d_h != 64 && d_h != 128) return false;
    return H == 8 || H == 16 || H == 32;
}

hipError_t launch_split_mfma_f32(const DecodeArgs& a, int occupancy, hipStream_t stream) {
    if (a.d_h == 64) return launch_h<64, false>(a, occupancy, stream);
    if (a.d_h == 128) return launch_h<128, false>(a, occupancy, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_step_mfma_f32(const DecodeArgs& a, int occupancy, hipStream_t stream) {
    if (a.d_h == 64) return launch_h<64, true>(a, occupancy, stream);
    if (a.d_h == 128) return launch_h<128, true>(a, occupancy, stream);
    return hipErrorInvalidValue;
}

}  // namespace lrkv
