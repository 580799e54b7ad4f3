// Matrix-core split kernel of the rotary variant, bf16 ("Low-Rank Key Value
// Attention | What a shared cache can preserve", sec. 8, "Full RoPE needs a
// stronger identity"; "Low-Rank Key Value Attention: Chinese reading notes",
// sec. 2.7).  Every head's whole key is turned at its own position,
//   ktilde_{h,j} = (k_s[j] + z^K_{h,j} (B^K_h)^T) D_j,   qtilde = q D_{L_b - 1},
// which no rank-space rotation reproduces for a generic B_h, so the private
// part of every (row, head) key is rebuilt: d_h * r multiply-adds per row and
// head, the cost the review names for the exact contraction.  The rotation is
// linear, so the score splits into a shared part, qtilde_h . (k_s[j] D_j), and
// a private part, qtilde_h . ((z^K_{h,j} (B^K_h)^T) D_j).
//
// A workgroup of 8 waves owns one (sequence, split) and walks its 128-row tiles
// (tile s, s + S_b, ... of the sequence); one workgroup per CU.  Per tile:
//   1. stage: the (cos, sin) rows go to LDS as fp32, the value rows as V^T
//      (bf16); each wave also loads the shared-key fragments of its 16-row
//      group for step 2a into registers;
//   2a. shared scores of all heads on the matrix cores (v_mfma_f32_16x16x32_bf16):
//      wave w turns the key rows of row group w (fp32) and splits them into
//      bf16 high and low parts, and computes S[16 rows x 16 heads] = Ktilde
//      Qtilde^T for every head group with both operands split (hi*hi + hi*lo
//      + lo*hi; about 16 significant bits of each operand);
//   2b. private scores: wave w takes heads w, w + 8, ...; per head it loads
//      the B^K_h fragments once for the tile's two 64-row halves and, per
//      16-row group, rebuilds the private key 16 columns at a time,
//      Out^T[16 cols x 16 rows] = B_h[16 x r] Z^T[r x 16] (exact bf16
//      products, fp32 sums).  Lane (row n16, g4) then holds columns
//      16 cb + 4 g4 + i of its row: it turns the two coordinate pairs (fp32)
//      and dots them with the rotated query; the four lanes of a row sum in a
//      fixed order;
//   3. softmax: one wave per head, two rows per lane, online max and
//      denominator in LDS;
//   4. values: the shared sum O^T[d_h x 16 heads] += V^T[d_h x 128] P^T on the
//      matrix cores (P split into bf16 high + low parts), one or two
//      (column block, head group) blocks per wave; the private sum on the VALU:
//      a thread owns one 16-byte chunk (8 coordinates of one head) of the
//      latent rows in one part of the tile, reads 16 rows at a time, and the
//      parts' sums are added in a fixed order at the end.
// The workgroup writes the usual partial record per head (running max in
// log2 units, denominator, shared sum, private sum); the merge kernel combines
// splits and applies B^V.
#include "lrkv_device.hpp"
#include "lrkv_internal.hpp"

namespace lrkv {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kTileRows = 128;  // 8 groups of 16 rows
constexpr int kHalfRows = 64;   // rows of one private-score pass (4 groups of 16)
constexpr int kMaxHeads = 32;
constexpr int kBatchRows = 16;  // private-value rows whose latent loads are issued together

template <int D, int R>
struct RopeCfg {
    static constexpr int CB = D / 16;                 // 16-column blocks of a key or value row
    static constexpr int KSD = D / 32;                // k-steps of the shared-score product
    static constexpr int NKS = (R + 31) / 32;         // k-steps of 32 latent coordinates
    static constexpr int CS_STRIDE = D + 4;           // floats per staged (cos, sin) row
    static constexpr int VT_STRIDE = kTileRows + 8;   // bf16 per V^T row (one value column, 128 rows)
    static constexpr int E_STRIDE = kTileRows + 4;    // floats per head of the score / weight rows
    static constexpr int NCH = R / 8;                 // 16-byte chunks (8 coordinates) of a head's latent row
    static constexpr int SVB = (CB * 2 + kWaves - 1) / kWaves;  // shared-value blocks per wave (H <= 32)
    static constexpr size_t CS_BYTES = (size_t)kTileRows * CS_STRIDE * 4;
    static constexpr size_t VT_BYTES = (size_t)D * VT_STRIDE * 2;
    // the weight rows come last but for the 96 floats of running state, which a masked read past the last
    // head's row (private values, at most 31 floats) may touch
    static constexpr size_t lds_bytes(int H) {
        return CS_BYTES + VT_BYTES + (size_t)H * D * 4 + 2 * (size_t)kMaxHeads * E_STRIDE * 4 +
               3 * (size_t)kMaxHeads * 4;
    }
};

// (hi, lo) bf16 parts of x: hi = bf16(x), lo = bf16(x - hi); hi + lo carries about 16 significant bits
__device__ __forceinline__ void split_bf16(float x, uint32_t& hi, uint32_t& lo) {
    hi = f32_to_bf16_bits(x);
    lo = f32_to_bf16_bits(x - __uint_as_float(hi << 16));
}

template <int D, int R>
__global__ void __launch_bounds__(kThreads, 1) split_rope_mfma_kernel(DecodeArgs a) {
    using C = RopeCfg<D, R>;
    constexpr int CB = C::CB, NKS = C::NKS, KSD = C::KSD;
    static_assert(R <= 64, "a head's latent row is at most 8 chunks, so a tile part holds at most 64 rows");
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    const int H = a.H;
    float* cs_l = (float*)lds;                                // [128][D + 4]
    uint16_t* vt = (uint16_t*)(lds + C::CS_BYTES);            // [D][128 + 8]
    float* qr_l = (float*)(lds + C::CS_BYTES + C::VT_BYTES);  // [H][D]
    float* es_l = qr_l + (size_t)H * D;                       // [32][128 + 4] shared scores
    float* ep_l = es_l + (size_t)kMaxHeads * C::E_STRIDE;     // [32][128 + 4] private, then weights
    float* m_l = ep_l + (size_t)kMaxHeads * C::E_STRIDE;      // [32] running max (log2 units)
    float* l_l = m_l + kMaxHeads;                             // [32] denominator
    float* al_l = l_l + kMaxHeads;                            // [32] this tile's rescale

    const SplitSlot wslot = split_slot(a.seq_lens, a.batch, a.max_len, a.num_splits, a.chunk, a.qgroup, blockIdx.x);
    const int b = wslot.b, split = wslot.s;
    if (b < 0) return;
    const int Lb = clamped_len(a.seq_lens, b, a.max_len);
    if (split * kTileRows >= Lb) return;
    const int bc = b / a.qgroup;
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n16 = lane & 15, g4 = lane >> 4;
    const int NHG = (H + 15) / 16;  // head groups of the matrix-core products
    const float scale = kLog2e / sqrtf((float)D);

    const uint16_t* ksg = (const uint16_t*)a.k_shared + (size_t)bc * a.L_cap * D;
    const uint16_t* vsg = (const uint16_t*)a.v_shared + (size_t)bc * a.L_cap * D;
    const uint16_t* zkg = (const uint16_t*)a.z_k + (size_t)bc * a.L_cap * H * R;
    const uint16_t* zvg = (const uint16_t*)a.z_v + (size_t)bc * a.L_cap * H * R;
    const uint16_t* bkg = (const uint16_t*)a.rope_bk;

    // the rotated query (position L_b - 1) of every head, fp32; score and weight rows of absent heads stay
    // zero, so the shared-value product reads finite weights for them
    {
        const float* cs = a.rope_cs + (size_t)(Lb - 1) * D;
        const uint16_t* qg = (const uint16_t*)a.q + (size_t)b * H * D;
        for (int idx = tid; idx < H * (D / 2); idx += kThreads) {
            const int h = idx / (D / 2), k = idx - h * (D / 2);
            const float x0 = bf16_to_f32(qg[h * D + 2 * k]), x1 = bf16_to_f32(qg[h * D + 2 * k + 1]);
            const float co = cs[2 * k], si = cs[2 * k + 1];
            qr_l[h * D + 2 * k] = x0 * co - x1 * si;
            qr_l[h * D + 2 * k + 1] = x0 * si + x1 * co;
        }
        for (int i = tid; i < 2 * kMaxHeads * C::E_STRIDE; i += kThreads) es_l[i] = 0.f;
        for (int h = tid; h < kMaxHeads; h += kThreads) {
            m_l[h] = -INFINITY;
            l_l[h] = 0.f;
            al_l[h] = 0.f;
        }
    }
    __syncthreads();

    // shared-value blocks of this wave: block blk = wave + 8 k is (column block blk % CB, head group blk / CB)
    f32x4_t acc_sv[C::SVB];
#pragma unroll
    for (int k = 0; k < C::SVB; ++k) acc_sv[k] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // private-value ownership: a latent row holds H * NCH chunks of 16 bytes (cells); thread t takes cell
    // t % cells over the rows of tile part t / cells (parts * cells <= 512, parts a power of two, at most 16),
    // so consecutive threads read consecutive chunks of a row; the parts' sums are added at the end
    const int cells = H * C::NCH;
    int parts = 1;
    while (cells > 0 && parts < 16 && 2 * parts * cells <= kThreads) parts *= 2;
    const int rpp = kTileRows / parts;  // rows per part: 8 .. 64
    const int cell = cells > 0 ? tid % cells : 0, part = cells > 0 ? tid / cells : 0;
    const bool own_pr = R > 0 && part < parts;
    const int hv = cell / (C::NCH > 0 ? C::NCH : 1);  // the cell's head
    float acc_pr[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc_pr[j] = 0.f;

    // Latent fragments of one head over 64 rows (four 16-row groups) of a tile; rows past the tile's end
    // re-read its last live row.  Two register sets are used in turn, so that the next 64 rows load while
    // the current ones compute; the first half of the next tile's first head is loaded at the end of a
    // tile's private-score phase.  Vector loads retire in order, so every load here is issued
    // unconditionally (a stand-in head or row where there is none): a load issued on one branch only would
    // make the compiler wait for it wherever an older load is waited for after the branches join.
    constexpr int NKS1 = NKS > 0 ? NKS : 1;
    typedef u32x4_t ZFrag[4][NKS1];
    typedef u32x4_t BFrag[CB][NKS1];
    auto load_z = [&](ZFrag& zf, int h, int tb, int nv, int half) {
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
            const size_t row = (size_t)(tb + min(kHalfRows * half + 16 * rg + n16, nv - 1));
#pragma unroll
            for (int ks = 0; ks < NKS1; ++ks) {
                const int k = 32 * ks + 8 * g4;
                zf[rg][ks] = (k < R) ? *(const u32x4_t*)(zkg + (row * H + h) * R + k) : u32x4_t{0u, 0u, 0u, 0u};
            }
        }
    };
    const int hw0 = min(wave, H - 1);  // this wave's first head (a stand-in for a wave without heads)
    ZFrag za, zb;
    if constexpr (NKS > 0) load_z(za, hw0, split * kTileRows, min(kTileRows, Lb - split * kTileRows), 0);

    // private-value latent rows of this thread's part, 16 at a time in two register sets; the first set is
    // loaded before the softmax (rows past the part's end re-read its last live row)
    const int rbeg = own_pr ? part * rpp : 0;
    u32x4_t va[kBatchRows], vb[kBatchRows];
    auto load_v = [&](u32x4_t (&zv)[kBatchRows], int tb, int r0, int rend) {
        const uint16_t* zbase = zvg + (size_t)tb * H * R + 8 * cell;
#pragma unroll
        for (int k = 0; k < kBatchRows; ++k)
            zv[k] = *(const u32x4_t*)(zbase + (size_t)max(min(r0 + k, rend - 1), 0) * H * R);
    };

    for (int t0 = split * kTileRows; t0 < Lb; t0 += wslot.S_b * kTileRows) {
        const int nvalid = min(kTileRows, Lb - t0);
        __syncthreads();  // the previous tile's staged rows and weights are consumed
        // ---- 1. stage the tile.  This wave's shared-key fragments (row group `wave`, for step 2a) go to
        //         registers.  Key and (cos, sin) rows past the end re-read the last live row (their scores are
        //         masked); value rows past the end are zero (weight 0 must not meet arbitrary contents) ----
        const int rk = 16 * wave + n16;  // this lane's key row in the tile (step 2a)
        u32x4_t kf[KSD];
        {
            const size_t row = (size_t)(t0 + min(rk, nvalid - 1));
#pragma unroll
            for (int ks = 0; ks < KSD; ++ks) kf[ks] = *(const u32x4_t*)(ksg + row * D + 32 * ks + 8 * g4);
        }
#pragma unroll
        for (int it = 0; it < kTileRows * (D / 4) / kThreads; ++it) {
            const int idx = tid + it * kThreads;
            const int r = idx / (D / 4), c4 = idx - r * (D / 4);
            const size_t row = (size_t)(t0 + min(r, nvalid - 1));
            *(f32x4_t*)(cs_l + r * C::CS_STRIDE + 4 * c4) = *(const f32x4_t*)(a.rope_cs + row * D + 4 * c4);
        }
        for (int idx = tid; idx < (kTileRows / 4) * (D / 8); idx += kThreads) {
            // V^T: 4 consecutive rows x 8 columns per thread, one 8-byte store per column
            const int r4 = idx / (D / 8), c8 = idx - r4 * (D / 8);
            uint32_t w[4][4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int r = 4 * r4 + k;
                const u32x4_t v = *(const u32x4_t*)(vsg + (size_t)(t0 + min(r, nvalid - 1)) * D + 8 * c8);
#pragma unroll
                for (int e = 0; e < 4; ++e) w[k][e] = (r < nvalid) ? v[e] : 0u;  // loaded anyway: no branch
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;  // high or low halves
                u32x2_t pk;
                pk[0] = __builtin_amdgcn_perm(w[1][j >> 1], w[0][j >> 1], sel);  // (row 4 r4, row 4 r4 + 1)
                pk[1] = __builtin_amdgcn_perm(w[3][j >> 1], w[2][j >> 1], sel);
                *(u32x2_t*)(vt + (8 * c8 + j) * C::VT_STRIDE + 4 * r4) = pk;
            }
        }
        __syncthreads();

        // ---- 2a. shared scores: rows 16 wave .., every head group.  The key fragment is turned by its row's
        //          (cos, sin) pairs once and split into (hi, lo) bf16 parts ----
        {
            u32x4_t khi[KSD], klo[KSD];
#pragma unroll
            for (int ks = 0; ks < KSD; ++ks) {
                const int c = 32 * ks + 8 * g4;
                const f32x4_t c0 = *(const f32x4_t*)(cs_l + rk * C::CS_STRIDE + c);      // pairs c/2, c/2 + 1
                const f32x4_t c1 = *(const f32x4_t*)(cs_l + rk * C::CS_STRIDE + c + 4);  // pairs c/2 + 2, + 3
#pragma unroll
                for (int p = 0; p < 4; ++p) {  // pair p of the 8 columns: (x0, x1) turned by (cos, sin)
                    const float x0 = bf16_lo(kf[ks][p]), x1 = bf16_hi(kf[ks][p]);
                    const float co = p < 2 ? c0[2 * p] : c1[2 * p - 4], si = p < 2 ? c0[2 * p + 1] : c1[2 * p - 3];
                    uint32_t h0, l0, h1, l1;
                    split_bf16(x0 * co - x1 * si, h0, l0);
                    split_bf16(x0 * si + x1 * co, h1, l1);
                    khi[ks][p] = h0 | (h1 << 16);
                    klo[ks][p] = l0 | (l1 << 16);
                }
            }
            for (int hg = 0; hg < NHG; ++hg) {
                f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
                const int hq = 16 * hg + n16;  // the query row of the B operand (zero past H)
#pragma unroll
                for (int ks = 0; ks < KSD; ++ks) {
                    const int c = 32 * ks + 8 * g4;
                    // the rotated query's 8 values split into (hi, lo) bf16 parts
                    f32x4_t q0 = {0.f, 0.f, 0.f, 0.f}, q1 = {0.f, 0.f, 0.f, 0.f};
                    if (hq < H) {
                        q0 = *(const f32x4_t*)(qr_l + hq * D + c);
                        q1 = *(const f32x4_t*)(qr_l + hq * D + c + 4);
                    }
                    u32x4_t qh4, ql4;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        uint32_t h0, l0, h1, l1;
                        split_bf16(i < 2 ? q0[2 * i] : q1[2 * i - 4], h0, l0);
                        split_bf16(i < 2 ? q0[2 * i + 1] : q1[2 * i - 3], h1, l1);
                        qh4[i] = h0 | (h1 << 16);
                        ql4[i] = l0 | (l1 << 16);
                    }
                    const bf16x8_t khv = __builtin_bit_cast(bf16x8_t, khi[ks]);
                    const bf16x8_t klv = __builtin_bit_cast(bf16x8_t, klo[ks]);
                    const bf16x8_t qhi = __builtin_bit_cast(bf16x8_t, qh4);
                    const bf16x8_t qlo = __builtin_bit_cast(bf16x8_t, ql4);
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(khv, qhi, acc, 0, 0, 0);
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(khv, qlo, acc, 0, 0, 0);
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(klv, qhi, acc, 0, 0, 0);
                }
                // lane (head n16, g4) holds rows 16 wave + 4 g4 + i
                if (hq < H) *(f32x4_t*)(es_l + hq * C::E_STRIDE + 16 * wave + 4 * g4) = acc;
            }
        }

        // ---- 2b. private scores of this wave's heads: per head, the B^K_h fragments (from L2) once, then the
        //          tile's two 64-row halves (h, 0) in za and (h, 1) in zb.  The B^K_h loads are issued before
        //          the next half's latent loads (from HBM), so the first product waits for the former only ----
        const int rbeg_end = min(rbeg + rpp, nvalid);  // end of this thread's private-value rows
        if constexpr (NKS > 0) {
            auto score_half = [&](const ZFrag& zf, const u32x4_t (&bf)[CB][NKS1], int h, int half) {
                const float* qh = qr_l + (size_t)h * D;
#pragma unroll
                for (int rg = 0; rg < 4; ++rg) {
                    const int rl = kHalfRows * half + 16 * rg + n16;  // this lane's row in the tile
                    float part = 0.f;
#pragma unroll
                    for (int cb = 0; cb < CB; ++cb) {
                        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int ks = 0; ks < NKS; ++ks)
                            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, bf[cb][ks]),
                                                                          __builtin_bit_cast(bf16x8_t, zf[rg][ks]),
                                                                          acc, 0, 0, 0);
                        const int c0 = 16 * cb + 4 * g4;
                        const f32x4_t cs = *(const f32x4_t*)(cs_l + rl * C::CS_STRIDE + c0);
                        const f32x4_t qv = *(const f32x4_t*)(qh + c0);
                        part = fmaf(qv[0], acc[0] * cs[0] - acc[1] * cs[1], part);
                        part = fmaf(qv[1], acc[0] * cs[1] + acc[1] * cs[0], part);
                        part = fmaf(qv[2], acc[2] * cs[2] - acc[3] * cs[3], part);
                        part = fmaf(qv[3], acc[2] * cs[3] + acc[3] * cs[2], part);
                    }
                    part += __shfl_xor(part, 16);  // the row's four column groups: (0 + 1) + (2 + 3)
                    part += __shfl_xor(part, 32);
                    if (g4 == 0) ep_l[(size_t)h * C::E_STRIDE + rl] = part;
                }
            };
            auto load_bk = [&](BFrag& bf, int h) {
#pragma unroll
                for (int cb = 0; cb < CB; ++cb)
#pragma unroll
                    for (int ks = 0; ks < NKS; ++ks) {
                        const int k = 32 * ks + 8 * g4;
                        bf[cb][ks] = (k < R) ? *(const u32x4_t*)(bkg + ((size_t)h * D + 16 * cb + n16) * R + k)
                                             : u32x4_t{0u, 0u, 0u, 0u};
                    }
            };
            // the next tile of this split (this tile again when there is none: the loads are then stand-ins)
            const int t0n = t0 + wslot.S_b * kTileRows;
            const int tbn = t0n < Lb ? t0n : t0, nvn = t0n < Lb ? min(kTileRows, Lb - t0n) : nvalid;
            BFrag bf;
            for (int h = wave; h < H; h += kWaves) {
                const bool last = h + kWaves >= H;  // the next unit is the next tile's first head
                load_bk(bf, h);
                load_z(zb, h, t0, nvalid, 1);
                score_half(za, bf, h, 0);
                load_z(za, last ? hw0 : h + kWaves, last ? tbn : t0, last ? nvn : nvalid, 0);
                score_half(zb, bf, h, 1);
            }
        }
        if constexpr (R > 0) load_v(va, t0, rbeg, rbeg_end);  // the first private-value batch
        __syncthreads();

        // ---- 3. online softmax, one wave per head, rows lane and lane + 64 ----
        for (int h = wave; h < H; h += kWaves) {
            float* eh = ep_l + (size_t)h * C::E_STRIDE;
            const float* sh = es_l + (size_t)h * C::E_STRIDE;
            const bool live0 = lane < nvalid, live1 = lane + 64 < nvalid;
            const float s0 = live0 ? (sh[lane] + (NKS > 0 ? eh[lane] : 0.f)) * scale : -INFINITY;
            const float s1 = live1 ? (sh[lane + 64] + (NKS > 0 ? eh[lane + 64] : 0.f)) * scale : -INFINITY;
            float tmax = fmaxf(s0, s1);
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1) tmax = fmaxf(tmax, __shfl_xor(tmax, o));
            const float m_old = m_l[h];
            const float m_new = fmaxf(m_old, tmax);  // finite: the tile holds a live row
            const float alpha = fast_exp2(m_old - m_new);
            const float e0 = live0 ? fast_exp2(s0 - m_new) : 0.f;
            const float e1 = live1 ? fast_exp2(s1 - m_new) : 0.f;
            float esum = e0 + e1;
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1) esum += __shfl_xor(esum, o);
            eh[lane] = e0;
            eh[lane + 64] = e1;
            wave_lds_sync();
            if (lane == 0) {
                m_l[h] = m_new;
                l_l[h] = fmaf(alpha, l_l[h], esum);
                al_l[h] = alpha;
            }
        }
        __syncthreads();

        // ---- 4a. shared values on the matrix cores: O^T[16 cols x 16 heads] += V^T[16 x 128] P^T[128 x 16] ----
#pragma unroll
        for (int k = 0; k < C::SVB; ++k) {
            const int blk = wave + kWaves * k;
            const int cb = blk % CB, hg = blk / CB;
            if (hg < NHG) {
                const int h = 16 * hg + n16;
                acc_sv[k] *= al_l[h];  // absent heads: alpha 0 on zero sums
#pragma unroll
                for (int ks = 0; ks < kTileRows / 32; ++ks) {
                    const int r0 = 32 * ks + 8 * g4;
                    const bf16x8_t av =
                        __builtin_bit_cast(bf16x8_t, *(const u32x4_t*)(vt + (16 * cb + n16) * C::VT_STRIDE + r0));
                    const f32x4_t e0 = *(const f32x4_t*)(ep_l + h * C::E_STRIDE + r0);
                    const f32x4_t e1 = *(const f32x4_t*)(ep_l + h * C::E_STRIDE + r0 + 4);
                    u32x4_t phi, plo;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        uint32_t h0, l0, h1, l1;
                        split_bf16(i < 2 ? e0[2 * i] : e1[2 * i - 4], h0, l0);
                        split_bf16(i < 2 ? e0[2 * i + 1] : e1[2 * i - 3], h1, l1);
                        phi[i] = h0 | (h1 << 16);
                        plo[i] = l0 | (l1 << 16);
                    }
                    acc_sv[k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(bf16x8_t, phi),
                                                                        acc_sv[k], 0, 0, 0);
                    acc_sv[k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(bf16x8_t, plo),
                                                                        acc_sv[k], 0, 0, 0);
                }
            }
        }

        // ---- 4b. private values: chunk `cell` of the latent rows of this thread's part, in batches of 16
        //          rows, two register sets used in turn; the first batch was loaded before the softmax ----
        if constexpr (R > 0) {
            const float al = al_l[hv];
#pragma unroll
            for (int j = 0; j < 8; ++j) acc_pr[j] *= al;  // threads without a part: sums never stored
            // Branch-free.  Rows past the tile's end have weight 0 in LDS; rows past the part are masked by a
            // uniform test.  Their latents are re-read live rows, so finite.  The weight read for such a row
            // can lie up to 31 floats past this head's row, inside the workgroup's LDS, and is discarded.  A
            // thread without a part reads part 0 and never stores its sums.
            const float* ep = ep_l + (size_t)hv * C::E_STRIDE + rbeg;
            auto consume = [&](const u32x4_t (&zv)[kBatchRows], int kb) {
#pragma unroll
                for (int k = 0; k < kBatchRows; ++k) {
                    const float ek = ep[kb + k];
                    const float e = (kb + k < rpp) ? ek : 0.f;
#pragma unroll
                    for (int j = 0; j < 8; ++j)
                        acc_pr[j] = fmaf(e, (j & 1) ? bf16_hi(zv[k][j >> 1]) : bf16_lo(zv[k][j >> 1]), acc_pr[j]);
                }
            };
            // batches 2 i (in va) and 2 i + 1 (in vb); the load after the last pair is a stand-in
            for (int kb = 0; kb < rpp; kb += 2 * kBatchRows) {
                load_v(vb, t0, rbeg + kb + kBatchRows, rbeg_end);
                consume(va, kb);
                load_v(va, t0, rbeg + kb + 2 * kBatchRows, rbeg_end);
                consume(vb, kb + kBatchRows);
            }
        }
    }

    // ---- the split's record of every head ----
    mfma_result_fence();  // the shared-value products end a loop with a run-time trip count
    __syncthreads();
    const int rec = partial_record_floats(D, R);
    float* out = a.ws + (size_t)blockIdx.x * H * rec;
#pragma unroll
    for (int k = 0; k < C::SVB; ++k) {
        const int blk = wave + kWaves * k;
        const int cb = blk % CB, hg = blk / CB;
        const int h = 16 * hg + n16;
        if (hg < NHG && h < H) *(f32x4_t*)(out + (size_t)h * rec + 16 * cb + 4 * g4) = acc_sv[k];
    }
    if constexpr (R > 0) {  // the parts' private sums, added in part order (the staged (cos, sin) area is free now)
        float* pr_l = (float*)lds;  // [512][8]
        if (own_pr) {
#pragma unroll
            for (int j = 0; j < 8; ++j) pr_l[tid * 8 + j] = acc_pr[j];
        }
        __syncthreads();
        for (int i = tid; i < cells * 8; i += kThreads) {
            const int c = i >> 3, j = i & 7;
            float sum = 0.f;
            for (int p = 0; p < parts; ++p) sum += pr_l[(p * cells + c) * 8 + j];
            const int h = c / C::NCH, ch = c - h * C::NCH;
            out[(size_t)h * rec + D + 8 * ch + j] = sum;
        }
    }
    for (int h = tid; h < H; h += kThreads) {
        out[(size_t)h * rec + D + R] = m_l[h];
        out[(size_t)h * rec + D + R + 1] = l_l[h];
    }
}

template <int D, int R>
hipError_t launch_dr(const DecodeArgs& a, hipStream_t stream) {
    const size_t lds = RopeCfg<D, R>::lds_bytes(a.H);
    auto kern = split_rope_mfma_kernel<D, R>;
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(a.num_splits), dim3(kThreads), lds, stream, a);
    return hipGetLastError();
}

template <int D>
hipError_t launch_d(const DecodeArgs& a, hipStream_t stream) {
    switch (a.r) {
        case 0: return launch_dr<D, 0>(a, stream);
        case 8: return launch_dr<D, 8>(a, stream);
        case 16: return launch_dr<D, 16>(a, stream);
        case 32: return launch_dr<D, 32>(a, stream);
        case 48: return launch_dr<D, 48>(a, stream);
        case 64: return launch_dr<D, 64>(a, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace

bool rope_mfma_path_supports(int H, int d_h, int r, int dtype) {
    if (dtype != 1 || H < 1 || H > kMaxHeads) return false;
    if (d_h != 64 && d_h != 128) return false;
    return r == 0 || r == 8 || r == 16 || r == 32 || r == 48 || r == 64;
}

int rope_mfma_rows_per_tile() { return kTileRows; }
int rope_mfma_workgroups() { return 256; }  // one per CU

hipError_t launch_split_rope_mfma(const DecodeArgs& a, hipStream_t stream) {
    static_assert(RopeCfg<128, 64>::lds_bytes(kMaxHeads) <= 160 * 1024, "LDS");
    if (a.d_h == 64) return launch_d<64>(a, stream);
    if (a.d_h == 128) return launch_d<128>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace lrkv
