// Matrix-core split kernel of the rotary variant, bf16 ("Low-Rank Key Value
// Attention | What a shared cache can preserve", sec. 8, "Full RoPE needs a
// stronger identity"; "Low-Rank Key Value Attention: Chinese reading notes",
// sec. 2.7).  Every head's whole key is turned at its own position,
//   ktilde_{h,j} = (k_s[j] + z^K_{h,j} (B^K_h)^T) D_j,   qtilde = q D_{L_b - 1},
// which no rank-space rotation reproduces for a generic B_h, so the key of
// every (row, head) is rebuilt: d_h * r multiply-adds per row and head, the
// cost the review names for the exact contraction.  They run on the matrix
// cores, the rest on the VALU.
//
// A workgroup of 4 waves owns one (sequence, split) and walks its 64-row
// tiles (tile s, s + S_b, ... of the sequence).  Per tile:
//   1. stage: shared key rows (bf16) and their (cos, sin) rows (fp32) in LDS;
//   2. scores: wave w takes heads w*HPW .. w*HPW + HPW - 1.  Per head it loads
//      the B^K_h fragments once (the next head's are loaded while this one
//      computes) and, per 16-row group, rebuilds the key 16 columns at a time,
//      Out^T[16 cols x 16 rows] = B_h[16 x r] Z^T[r x 16], on
//      v_mfma_f32_16x16x32_bf16 (exact bf16 products, fp32 sums).  Lane
//      (row n16, g4) then holds columns 16 cb + 4 g4 + i of its row: it adds
//      the shared row, turns the two coordinate pairs, dots them with the
//      rotated query (fp32) and the four lanes of a row sum in a fixed order;
//   3. softmax: one wave per head, lanes = the tile's rows, online max and
//      denominator in LDS;
//   4. values: thread (head, g) of 8 groups accumulates the shared sum over
//      columns g*d_h/8 .. and the private sum over latent coordinates g*r/8 ..,
//      reading value and latent rows 8 at a time (the lanes of a wave that
//      read the same value columns share one access).
// Two workgroups are resident per CU (LDS 75 KB, at most 256 registers per
// lane), so one workgroup's barriers and load latency overlap the other's work.
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

constexpr int kWaves = 4;
constexpr int kTileRows = 64;  // 4 groups of 16 rows

template <int D, int R>
struct RopeCfg {
    static constexpr int CB = D / 16;              // 16-column blocks of a key
    static constexpr int NKS = (R + 31) / 32;      // k-steps of 32 latent coordinates
    static constexpr int KS_STRIDE = D + 8;        // bf16 per staged shared-key row
    static constexpr int CS_STRIDE = D + 4;        // floats per staged (cos, sin) row
    static constexpr int E_STRIDE = kTileRows + 4; // floats per head of the score / weight rows
    static constexpr int SHC = D / 8;              // shared-value columns per thread
    static constexpr int PRC = R / 8;              // latent coordinates per thread
    static constexpr size_t lds_bytes(int H) {
        return (size_t)kTileRows * KS_STRIDE * 2 + (size_t)kTileRows * CS_STRIDE * 4 + (size_t)H * D * 4 +
               (size_t)H * E_STRIDE * 4 + 3 * (size_t)H * 4;
    }
};

constexpr int kBatchRows = 8;  // value-phase rows whose value and latent loads are issued together

// N consecutive bf16 values (latent coordinates: N = r / 8 in {0, 1, 2, 4, 6, 8}; value columns: N = d_h / 8
// in {8, 16}), loaded with as few instructions as their alignment allows
template <int N>
struct LatVec {
    uint32_t w[N > 1 ? (N + 1) / 2 : 1];
    __device__ __forceinline__ void load(const uint16_t* p) {
        if constexpr (N == 16) {
            const u32x4_t v0 = *(const u32x4_t*)p, v1 = *(const u32x4_t*)(p + 8);
            w[0] = v0[0]; w[1] = v0[1]; w[2] = v0[2]; w[3] = v0[3];
            w[4] = v1[0]; w[5] = v1[1]; w[6] = v1[2]; w[7] = v1[3];
        } else if constexpr (N == 8) {
            const u32x4_t v = *(const u32x4_t*)p;
            w[0] = v[0]; w[1] = v[1]; w[2] = v[2]; w[3] = v[3];
        } else if constexpr (N == 6) {
            const uint32_t* d = (const uint32_t*)p;  // 12 bytes at 4-byte alignment
            w[0] = d[0]; w[1] = d[1]; w[2] = d[2];
        } else if constexpr (N == 4) {
            const u32x2_t v = *(const u32x2_t*)p;
            w[0] = v[0]; w[1] = v[1];
        } else if constexpr (N == 2) {
            w[0] = *(const uint32_t*)p;
        } else if constexpr (N == 1) {
            w[0] = *p;
        }
    }
    __device__ __forceinline__ float at(int j) const {  // j < N, a compile-time index after unrolling
        return (j & 1) ? bf16_hi(w[j >> 1]) : bf16_lo(w[j >> 1]);
    }
};

template <int D, int R>
struct Frags {  // one head's B^K fragments and the latent fragments of the tile's 4 row groups
    u32x4_t b[RopeCfg<D, R>::CB][RopeCfg<D, R>::NKS > 0 ? RopeCfg<D, R>::NKS : 1];
    u32x4_t z[4][RopeCfg<D, R>::NKS > 0 ? RopeCfg<D, R>::NKS : 1];
};

template <int D, int R>
__global__ void __launch_bounds__(kWaves * 64, 2) split_rope_mfma_kernel(DecodeArgs a) {
    using C = RopeCfg<D, R>;
    constexpr int CB = C::CB, NKS = C::NKS;
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    const int H = a.H;
    uint16_t* ks_l = (uint16_t*)lds;                                           // [64][D + 8]
    float* cs_l = (float*)(lds + (size_t)kTileRows * C::KS_STRIDE * 2);        // [64][D + 4]
    float* qr_l = (float*)((unsigned char*)cs_l + (size_t)kTileRows * C::CS_STRIDE * 4);  // [H][D]
    float* e_l = qr_l + (size_t)H * D;                                         // [H][64 + 4]
    float* m_l = e_l + (size_t)H * C::E_STRIDE;                                // [H] running max (log2 units)
    float* l_l = m_l + H;                                                      // [H] denominator
    float* al_l = l_l + H;                                                     // [H] this tile's rescale

    const SplitSlot wslot = split_slot(a.seq_lens, a.batch, a.max_len, a.num_splits, blockIdx.x);
    const int b = wslot.b, split = wslot.s;
    if (b < 0) return;
    const int Lb = clamped_len(a.seq_lens, b, a.max_len);
    if (split * kTileRows >= Lb) return;
    const int bc = b / a.qgroup;
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n16 = lane & 15, g4 = lane >> 4;
    const int HPW = (H + kWaves - 1) / kWaves;  // heads per wave (scores) and per wave in the value phase
    const float scale = kLog2e / sqrtf((float)D);

    const uint16_t* ksg = (const uint16_t*)a.k_shared + (size_t)bc * a.L_cap * D;
    const uint16_t* vsg = (const uint16_t*)a.v_shared + (size_t)bc * a.L_cap * D;
    const uint16_t* zkg = (const uint16_t*)a.z_k + (size_t)bc * a.L_cap * H * R;
    const uint16_t* zvg = (const uint16_t*)a.z_v + (size_t)bc * a.L_cap * H * R;
    const uint16_t* bkg = (const uint16_t*)a.rope_bk;

    // the rotated query (position L_b - 1) of every head, fp32
    {
        const float* cs = a.rope_cs + (size_t)(Lb - 1) * D;
        const uint16_t* qg = (const uint16_t*)a.q + (size_t)b * H * D;
        for (int idx = tid; idx < H * (D / 2); idx += kWaves * 64) {
            const int h = idx / (D / 2), k = idx - h * (D / 2);
            const float x0 = bf16_to_f32(qg[h * D + 2 * k]), x1 = bf16_to_f32(qg[h * D + 2 * k + 1]);
            const float co = cs[2 * k], si = cs[2 * k + 1];
            qr_l[h * D + 2 * k] = x0 * co - x1 * si;
            qr_l[h * D + 2 * k + 1] = x0 * si + x1 * co;
        }
        for (int h = tid; h < H; h += kWaves * 64) {
            m_l[h] = -INFINITY;
            l_l[h] = 0.f;
        }
    }

    // value-phase ownership: thread (head hv, group g)
    const int hv = wave * HPW + (lane >> 3), gv = lane & 7;
    const bool own = (lane >> 3) < HPW && hv < H;
    float acc_sh[C::SHC], acc_pr[C::PRC > 0 ? C::PRC : 1];
#pragma unroll
    for (int j = 0; j < C::SHC; ++j) acc_sh[j] = 0.f;
#pragma unroll
    for (int j = 0; j < C::PRC; ++j) acc_pr[j] = 0.f;

    const int h_first = wave * HPW, h_end = min(H, h_first + HPW);

    for (int t0 = split * kTileRows; t0 < Lb; t0 += wslot.S_b * kTileRows) {
        const int nvalid = min(kTileRows, Lb - t0);
        __syncthreads();  // the previous tile's weights and value rows are consumed
        // ---- 1. stage the tile (rows past the end re-read the last live row) ----
        for (int idx = tid; idx < kTileRows * (D / 8); idx += kWaves * 64) {
            const int r = idx / (D / 8), c8 = idx - r * (D / 8);
            const size_t row = (size_t)(t0 + min(r, nvalid - 1));
            *(u32x4_t*)(ks_l + r * C::KS_STRIDE + 8 * c8) = *(const u32x4_t*)(ksg + row * D + 8 * c8);
        }
        for (int idx = tid; idx < kTileRows * (D / 4); idx += kWaves * 64) {
            const int r = idx / (D / 4), c4 = idx - r * (D / 4);
            const size_t pos = (size_t)(t0 + min(r, nvalid - 1));
            *(f32x4_t*)(cs_l + r * C::CS_STRIDE + 4 * c4) = *(const f32x4_t*)(a.rope_cs + pos * D + 4 * c4);
        }
        __syncthreads();

        // ---- 2. scores of this wave's heads ----
        auto load_frags = [&](Frags<D, R>& f, int h) {
            if constexpr (NKS > 0) {
#pragma unroll
                for (int cb = 0; cb < CB; ++cb)
#pragma unroll
                    for (int ks = 0; ks < NKS; ++ks) {
                        const int k = 32 * ks + 8 * g4;
                        const int kc = k < R ? k : 0;
                        f.b[cb][ks] = *(const u32x4_t*)(bkg + ((size_t)h * D + 16 * cb + n16) * R + kc);
                        if (k >= R) f.b[cb][ks] = u32x4_t{0u, 0u, 0u, 0u};
                    }
#pragma unroll
                for (int rg = 0; rg < 4; ++rg) {
                    const size_t row = (size_t)(t0 + min(16 * rg + n16, nvalid - 1));
#pragma unroll
                    for (int ks = 0; ks < NKS; ++ks) {
                        const int k = 32 * ks + 8 * g4;
                        const int kc = k < R ? k : 0;
                        f.z[rg][ks] = *(const u32x4_t*)(zkg + (row * H + h) * R + kc);
                        if (k >= R) f.z[rg][ks] = u32x4_t{0u, 0u, 0u, 0u};
                    }
                }
            }
        };
        auto score_head = [&](const Frags<D, R>& f, int h) {
            const float* qh = qr_l + (size_t)h * D;
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                const int rl = 16 * rg + n16;  // this lane's row in the tile
                float part = 0.f;
#pragma unroll
                for (int cb = 0; cb < CB; ++cb) {
                    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
                    if constexpr (NKS > 0) {
#pragma unroll
                        for (int ks = 0; ks < NKS; ++ks)
                            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, f.b[cb][ks]),
                                                                          __builtin_bit_cast(bf16x8_t, f.z[rg][ks]),
                                                                          acc, 0, 0, 0);
                    }
                    const int c0 = 16 * cb + 4 * g4;
                    const u32x2_t kv = *(const u32x2_t*)(ks_l + rl * C::KS_STRIDE + c0);
                    const f32x4_t cs = *(const f32x4_t*)(cs_l + rl * C::CS_STRIDE + c0);
                    const f32x4_t qv = *(const f32x4_t*)(qh + c0);
                    const float u0 = acc[0] + bf16_lo(kv[0]), u1 = acc[1] + bf16_hi(kv[0]);
                    const float u2 = acc[2] + bf16_lo(kv[1]), u3 = acc[3] + bf16_hi(kv[1]);
                    part = fmaf(qv[0], u0 * cs[0] - u1 * cs[1], part);
                    part = fmaf(qv[1], u0 * cs[1] + u1 * cs[0], part);
                    part = fmaf(qv[2], u2 * cs[2] - u3 * cs[3], part);
                    part = fmaf(qv[3], u2 * cs[3] + u3 * cs[2], part);
                }
                part += __shfl_xor(part, 16);  // the row's four column groups: (0 + 1) + (2 + 3)
                part += __shfl_xor(part, 32);
                if (g4 == 0) e_l[(size_t)h * C::E_STRIDE + rl] = part;
            }
        };
        for (int h = h_first; h < h_end; ++h) {  // the other resident workgroup covers these loads' latency
            Frags<D, R> f;
            load_frags(f, h);
            score_head(f, h);
        }
        __syncthreads();

        // ---- 3. online softmax, one wave per head, lanes = rows ----
        for (int h = wave; h < H; h += kWaves) {
            float* eh = e_l + (size_t)h * C::E_STRIDE;
            const bool live = lane < nvalid;
            const float s = live ? eh[lane] * scale : -INFINITY;
            float tmax = s;
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1) tmax = fmaxf(tmax, __shfl_xor(tmax, o));
            const float m_old = m_l[h];
            const float m_new = fmaxf(m_old, tmax);  // finite: the tile holds a live row
            const float alpha = fast_exp2(m_old - m_new);
            const float e = live ? fast_exp2(s - m_new) : 0.f;
            float esum = e;
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1) esum += __shfl_xor(esum, o);
            eh[lane] = e;
            wave_lds_sync();
            if (lane == 0) {
                m_l[h] = m_new;
                l_l[h] = fmaf(alpha, l_l[h], esum);
                al_l[h] = alpha;
            }
        }
        __syncthreads();

        // ---- 4. values: shared columns gv*SHC.., latent coordinates gv*PRC.. of head hv ----
        // Rows go in batches of 16: the batch's latent loads are all issued before any of its arithmetic, so
        // their latency is paid once per batch (rows past the tile's end re-read the last live row, unused).
        if (own) {
            const float al = al_l[hv];
#pragma unroll
            for (int j = 0; j < C::SHC; ++j) acc_sh[j] *= al;
#pragma unroll
            for (int j = 0; j < C::PRC; ++j) acc_pr[j] *= al;
            const float* eh = e_l + (size_t)hv * C::E_STRIDE;
            const uint16_t* zbase = zvg + ((size_t)t0 * H + hv) * R + gv * C::PRC;
            const uint16_t* vbase = vsg + (size_t)t0 * D + gv * C::SHC;
            for (int r0 = 0; r0 < nvalid; r0 += kBatchRows) {
                LatVec<C::SHC> vb[kBatchRows];
                LatVec<C::PRC> zb[kBatchRows];
#pragma unroll
                for (int k = 0; k < kBatchRows; ++k) {
                    const size_t r = (size_t)min(r0 + k, nvalid - 1);
                    vb[k].load(vbase + r * D);
                    zb[k].load(zbase + r * H * R);
                }
#pragma unroll
                for (int k = 0; k < kBatchRows; ++k) {
                    if (r0 + k < nvalid) {
                        const float e = eh[r0 + k];
#pragma unroll
                        for (int j = 0; j < C::SHC; ++j) acc_sh[j] = fmaf(e, vb[k].at(j), acc_sh[j]);
#pragma unroll
                        for (int j = 0; j < C::PRC; ++j) acc_pr[j] = fmaf(e, zb[k].at(j), acc_pr[j]);
                    }
                }
            }
        }
    }

    // ---- the split's record of every head ----
    __syncthreads();
    if (own) {
        const int rec = partial_record_floats(D, R);
        float* out = a.ws + ((size_t)blockIdx.x * H + hv) * rec;
#pragma unroll
        for (int j = 0; j < C::SHC; ++j) out[gv * C::SHC + j] = acc_sh[j];
#pragma unroll
        for (int j = 0; j < C::PRC; ++j) out[D + gv * C::PRC + j] = acc_pr[j];
        if (gv == 0) {
            out[D + R] = m_l[hv];
            out[D + R + 1] = l_l[hv];
        }
    }
}

template <int D, int R>
hipError_t launch_dr(const DecodeArgs& a, hipStream_t stream) {
    const size_t lds = RopeCfg<D, R>::lds_bytes(a.H);
    auto kern = split_rope_mfma_kernel<D, R>;
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(a.num_splits), dim3(kWaves * 64), lds, stream, a);
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
    if (dtype != 1 || H < 1 || H > 32) return false;
    if (d_h != 64 && d_h != 128) return false;
    if (!(r == 0 || r == 8 || r == 16 || r == 32 || r == 48 || r == 64)) return false;
    return RopeCfg<128, 64>::lds_bytes(H) <= 160 * 1024;
}

int rope_mfma_rows_per_tile() { return kTileRows; }

hipError_t launch_split_rope_mfma(const DecodeArgs& a, hipStream_t stream) {
    if (a.d_h == 64) return launch_d<64>(a, stream);
    if (a.d_h == 128) return launch_d<128>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace lrkv
