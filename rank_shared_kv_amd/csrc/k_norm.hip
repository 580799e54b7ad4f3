// Kernels of the normalised variant ("Low-Rank Key Value Attention | What a
// shared cache can preserve", sec. 8, post-projection normalisation and its
// cache cost; "Low-Rank Key Value Attention: Chinese reading notes", sec. 2.7,
// last paragraph).  The key of head h at token j is the summed key
//   k_{h,j} = k_s[j] + z^K_{h,j} (B^K_h)^T,
// RMS-normalised as a whole; what the cache keeps besides the factors is its
// reciprocal RMS, one scalar per (token, head):
//   rho_{h,j} = 1 / sqrt(|k_{h,j}|^2 / d_h + eps)         [batch][L_cap][H], cache dtype
// The per-head key gain moves to the query side, so the decode only multiplies
// the summed logit of (h, j) by rho_{h,j}:
//   q_eff_h = g^K_h * g^Q_h * q_h / sqrt(|q_h|^2 / d_h + eps)
//
// bf16, r a multiple of 8 up to 64: the keys are rebuilt 16 columns x 16 rows
// at a time on v_mfma_f32_16x16x32_bf16 (Out^T = B_h Z^T, as the materialise
// kernel does), the shared row is added and the squares accumulated; the four
// lanes that hold one row's columns then sum in a fixed order.  The keys
// themselves are never written.  With d_h = 64 or 128 (key_scales_rows_kernel)
// the eight waves of a workgroup take eight heads of the same rows (up to 1024), in
// chunks of 64 whose shared rows the workgroup stages in LDS; each wave fetches
// its B_h fragments once, and the next chunk's loads are in flight while a chunk
// computes.  Other d_h (key_scales_mfma_kernel) take a wave per 16 rows.  Other
// shapes: one thread per (row, head).
#include <algorithm>
#include <cstdlib>
#include <type_traits>

#include "lrkv_device.hpp"
#include "lrkv_internal.hpp"

namespace lrkv {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;  // 64 rows of one head per workgroup

__device__ __forceinline__ float rms_scale(float sum_sq, int D, float eps) { return 1.f / sqrtf(sum_sq / (float)D + eps); }

// rows max(0, L_b - n_last) .. L_b - 1 of sequence b; NKS k-steps of 32 rank coordinates, a compile-time
// count so the matrix-core results are read after their wait states (see materialize_mfma_kernel)
template <int NKS>
__global__ void __launch_bounds__(kWaves * 64) key_scales_mfma_kernel(int H, int D, int R, int L_cap, int max_len,
                                                                      int n_last, float eps,
                                                                      const int32_t* __restrict__ seq_lens,
                                                                      const uint16_t* __restrict__ shared,
                                                                      const uint16_t* __restrict__ z,
                                                                      const uint16_t* __restrict__ basis,
                                                                      uint16_t* __restrict__ rho) {
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n16 = lane & 15, g4 = lane >> 4;
    const int h = blockIdx.y, b = blockIdx.z;
    const int Lb = clamped_len(seq_lens, b, max_len);
    const int start = max(0, Lb - n_last);
    const int t0 = start + (blockIdx.x * kWaves + wave) * 16;
    if (t0 >= Lb) return;
    const int row = t0 + n16;                       // this lane's row (B operand column, result column)
    const int row_c = min(row, Lb - 1);             // rows past the end re-read the last live row
    const uint16_t* zrow = z + (((size_t)b * L_cap + row_c) * H + h) * R;  // token-major latents
    const uint16_t* srow = shared + ((size_t)b * L_cap + row_c) * D;
    const uint16_t* bh = basis + (size_t)h * D * R;
    float ss = 0.f;
    for (int cb = 0; cb < D / 16; ++cb) {
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            const int k = 32 * ks + 8 * g4;
            const bool in = k < R;                   // R is a multiple of 8: whole 8-coordinate groups
            const int kc = in ? k : 0;
            u32x4_t zv = *(const u32x4_t*)(zrow + kc);
            u32x4_t bv = *(const u32x4_t*)(bh + (size_t)(16 * cb + n16) * R + kc);
            if (!in) zv = bv = u32x4_t{0u, 0u, 0u, 0u};
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, bv),
                                                          __builtin_bit_cast(bf16x8_t, zv), acc, 0, 0, 0);
        }
        mfma_result_fence();
        // lane (row n16, g4) holds columns 16 cb + 4 g4 + i of its row's key
        const u32x2_t s = *(const u32x2_t*)(srow + 16 * cb + 4 * g4);
        const float v0 = acc[0] + bf16_lo(s[0]), v1 = acc[1] + bf16_hi(s[0]);
        const float v2 = acc[2] + bf16_lo(s[1]), v3 = acc[3] + bf16_hi(s[1]);
        ss = fmaf(v0, v0, ss);
        ss = fmaf(v1, v1, ss);
        ss = fmaf(v2, v2, ss);
        ss = fmaf(v3, v3, ss);
    }
    ss += __shfl_xor(ss, 16);  // the four column groups of a row: (g4 0 + 1) + (2 + 3)
    ss += __shfl_xor(ss, 32);
    if (g4 == 0 && row < Lb) rho[((size_t)b * L_cap + row) * H + h] = (uint16_t)f32_to_bf16_bits(rms_scale(ss, D, eps));
}

constexpr int kChunkRows = 64;  // rows per chunk in the d_h = 64 / 128 kernel

// f(integral_constant<int, 0>), f(..1), ... in order while f returns true
template <class F, int... Cs>
__device__ __forceinline__ void for_each_while(F&& f, std::integer_sequence<int, Cs...>) {
    (void)((f(std::integral_constant<int, Cs>{})) && ...);
}
constexpr int kRowWaves = 8;    // waves (heads) per workgroup in the d_h = 64 / 128 kernel

// A buffer resource over `bytes` bytes at base (bytes >= 0): a load whose lane offset (the offset from
// the vector register; the scalar offset is not range-checked) is past the end returns zeros and touches no
// memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t ks_rsrc(const void* base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}
constexpr uint32_t kOutOfRange = 0x80000000u;  // a lane offset past every resource of this kernel

// rows max(0, L_b - n_last) .. L_b - 1 of sequence b; heads 8 y .. 8 y + 7 in the workgroup's waves.  The
// workgroup walks CH chunks of 64 rows (past L_b: zeros, computed, not stored); each wave loads its head's B^K_h
// fragments once.  The chunk's shared rows are staged in LDS by the whole workgroup.  Every byte read through
// the L1 caches costs about as much as one from memory here (measured: the kernel moved 1.08 GB through them
// for 579 MB of data when 4 heads shared a chunk and B^K_h was fetched per 256 rows), so eight heads share each
// staged chunk and B^K_h serves CH * 64 rows.  The shared rows are widened to fp32 when they are staged (once
// per workgroup instead of once per head) and enter each product as its accumulator, so the key k_s + z B^T
// comes out of the matrix cores whole and the VALU only squares it.  The loads run two chunks ahead: chunk
// c + 2's latents and shared rows are issued before chunk c is computed (three latent register sets, two
// staging sets for the shared rows, two LDS buffers).  The chunks are unrolled at compile time, so that
// whether a chunk has a successor to load is known to the compiler: with those loads under a run-time condition
// (and a loop back edge), the wait counts it derived were conservative, and most chunks waited for nearly every
// load in flight.  Each latent load reads whole rows of the wave's head (a head's r coordinates are contiguous),
// which the wave passes through its own LDS rows into the operand layout, where a row's coordinates are spread
// over four lanes (loaded directly in that layout, every load instruction read 16 rows x 64 bytes, and the
// kernel ran 8% slower).  The cache is read through buffer resources that start at a load's first row (latents)
// or a chunk (shared rows) and end at row L_b, so that the row offsets are scalar and rows past L_b (and coordinates past
// r, through an offset past every resource) read as zeros without per-lane clamps; the
// four partial sums of a row are reduced so that lane (row n16, group g4) ends with the whole sum of row
// 16 g4 + n16 of the chunk, and each lane computes and stores one scale per chunk.  (The VALU issued more
// instructions than the matrix cores took cycles before: per 64-row chunk and wave about 480, 130 of them the
// squares, the rest address arithmetic, clamps and four full-precision scales per lane.)  FULL: r = 32 NKS.
template <int D, int NKS, int CH, bool FULL>
__global__ void __launch_bounds__(kRowWaves * 64) key_scales_rows_kernel(int H, int R, int L_cap, int max_len, int n_last,
                                                                      float eps, const int32_t* __restrict__ seq_lens,
                                                                      const uint16_t* __restrict__ shared,
                                                                      const uint16_t* __restrict__ z,
                                                                      const uint16_t* __restrict__ basis,
                                                                      uint16_t* __restrict__ rho) {
    constexpr int CB = D / 16;
    constexpr int SROW = D + 4;                               // floats per staged shared row
    constexpr int PPT = kChunkRows * (D / 8) / (kRowWaves * 64);  // 16-byte pieces of a chunk per thread
    constexpr int RB = 64 * NKS;           // bytes of a head's latent row that the loads cover (r <= 32 NKS)
    constexpr int LR = RB / 16;            // lanes per latent row in a load
    constexpr int RPI = 64 / LR;           // latent rows per load instruction
    constexpr int NZI = kChunkRows / RPI;  // latent load instructions per chunk
    constexpr int ZS = RB + 16;            // bytes per latent row staged in LDS (padded)
    __shared__ __attribute__((aligned(16))) float sh_l[2][kChunkRows * SROW];
    __shared__ __attribute__((aligned(16))) unsigned char zs_l[kRowWaves][kChunkRows * ZS];
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n16 = lane & 15, g4 = lane >> 4;
    const int h = blockIdx.y * kRowWaves + wave, b = blockIdx.z;
    const int hc = min(h, H - 1);  // waves past the last head compute a stand-in and store nothing
    const int Lb = __builtin_amdgcn_readfirstlane(clamped_len(seq_lens, b, max_len));
    const int start = max(0, Lb - n_last);
    const int r0 = start + blockIdx.x * kChunkRows * CH;
    if (r0 >= Lb) return;  // the whole workgroup
    const int zrow = H * R * 2, srow = D * 2;  // bytes per cache row (every head), per shared row
    const uint16_t* zb = z + (size_t)b * L_cap * H * R;
    const uint16_t* sb = shared + (size_t)b * L_cap * D;
    // latent loads: lane (zi, zj) reads 16-byte piece zj (coordinates 8 zj ..) of head hc in row zi of the
    // instruction's RPI rows (past r: out of range), so that each instruction reads whole rows of the head
    const int zi = lane / LR, zj = lane % LR;
    const uint32_t vz = (FULL || 8 * zj < R) ? (uint32_t)(zi * zrow + (hc * R + 8 * zj) * 2) : kOutOfRange;
    const uint16_t* bh = basis + (size_t)hc * D * R;
    typedef u32x4_t ZFrag[NZI];
    typedef u32x4_t SFrag[PPT];
    auto load_z = [&](ZFrag& zf, int c) {  // latents of rows r0 + 64 c + RPI m + zi (past L_b: zeros)
#pragma unroll
        for (int m = 0; m < NZI; ++m) {
            const int t = r0 + kChunkRows * c + RPI * m;  // the instruction's first row
            const __amdgpu_buffer_rsrc_t rs = ks_rsrc(zb + (size_t)t * H * R, Lb > t ? (Lb - t) * zrow : 0);
            zf[m] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, vz, 0, 0));
        }
    };
    auto load_sh = [&](SFrag& v, int c) {  // piece p: row p / (D / 8), 8 columns at 8 (p % (D / 8))
        const int t = r0 + kChunkRows * c;  // the chunk's first row
        const __amdgpu_buffer_rsrc_t rs = ks_rsrc(sb + (size_t)t * D, Lb > t ? (Lb - t) * srow : 0);
#pragma unroll
        for (int i = 0; i < PPT; ++i) {
            const int p = tid + kRowWaves * 64 * i;
            const uint32_t vo = (uint32_t)((p / (D / 8)) * srow + 16 * (p % (D / 8)));
            v[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, vo, 0, 0));
        }
    };
    auto store_sh = [&](const SFrag& v, int buf) {  // widened to fp32 (exact)
#pragma unroll
        for (int i = 0; i < PPT; ++i) {
            const int p = tid + kRowWaves * 64 * i;
            float* dst = sh_l[buf] + (p / (D / 8)) * SROW + 8 * (p % (D / 8));
            *(f32x4_t*)dst = f32x4_t{bf16_lo(v[i][0]), bf16_hi(v[i][0]), bf16_lo(v[i][1]), bf16_hi(v[i][1])};
            *(f32x4_t*)(dst + 4) = f32x4_t{bf16_lo(v[i][2]), bf16_hi(v[i][2]), bf16_lo(v[i][3]), bf16_hi(v[i][3])};
        }
    };
    u32x4_t bf[CB][NKS];  // B_h rows 16 cb + n16, coordinates 32 ks + 8 g4 (past r: zero)
    SFrag sv[2];          // shared rows of chunk k in sv[k & 1] until staged
    ZFrag zr[3];          // latents of chunk k in zr[k % 3]
    // prologue: B^K_h, then chunks 0 and 1 (shared rows and latents), in the order they are needed
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            const int k = 32 * ks + 8 * g4;
            bf[cb][ks] = *(const u32x4_t*)(bh + (size_t)(16 * cb + n16) * R + (FULL || k < R ? k : 0));
        }
    load_sh(sv[0], 0);
    load_z(zr[0], 0);
    if constexpr (CH > 1) {
        load_sh(sv[1], 1);
        load_z(zr[1], 1);
    }
    if constexpr (!FULL) {
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
            if (32 * ks + 8 * g4 >= R) {
#pragma unroll
                for (int cb = 0; cb < CB; ++cb) bf[cb][ks] = u32x4_t{0u, 0u, 0u, 0u};
            }
    }
    store_sh(sv[0], 0);
    __syncthreads();
    // chunk C (compile time): chunk C + 2's loads first, then this chunk's keys, then chunk C + 1's shared rows
    // into LDS; false once no later chunk holds a live row
    auto chunk = [&](auto c_tag) -> bool {
        constexpr int C = decltype(c_tag)::value, K = C;
        constexpr int c = C;
        if constexpr (C + 2 < CH) {
            load_sh(sv[K & 1], c + 2);
            load_z(zr[(K + 2) % 3], c + 2);
        }
        // the chunk's latents through this wave's LDS rows into the operand layout: lane (row n16, g4) takes
        // coordinates 32 ks + 8 g4 .. of row 16 rg + n16 (a wave's LDS operations complete in order)
        unsigned char* zw = zs_l[wave];
#pragma unroll
        for (int m = 0; m < NZI; ++m) *(u32x4_t*)(zw + (RPI * m + zi) * ZS + 16 * zj) = zr[K % 3][m];
        u32x4_t zc[4][NKS];
#pragma unroll
        for (int rg = 0; rg < 4; ++rg)
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) zc[rg][ks] = *(const u32x4_t*)(zw + (16 * rg + n16) * ZS + 16 * (g4 + 4 * ks));
        const float* shc = sh_l[c % 2];
        float ss[4];
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
            ss[rg] = 0.f;
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) {
                // lane (row n16, g4) holds columns 16 cb + 4 g4 + i of its row's key: the shared row's values
                // there are the accumulator the latent part is added to
                f32x4_t acc = *(const f32x4_t*)(shc + (16 * rg + n16) * SROW + 16 * cb + 4 * g4);
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks)
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, bf[cb][ks]),
                                                                  __builtin_bit_cast(bf16x8_t, zc[rg][ks]), acc, 0, 0, 0);
                ss[rg] = fmaf(acc[0], acc[0], ss[rg]);
                ss[rg] = fmaf(acc[1], acc[1], ss[rg]);
                ss[rg] = fmaf(acc[2], acc[2], ss[rg]);
                ss[rg] = fmaf(acc[3], acc[3], ss[rg]);
            }
        }
        // the four column groups of a row (lanes g4 = 0..3 of its n16) into lane g4 = rg of the row's group rg:
        // groups (0 + 2) and (1 + 3) of the rows of groups rg with bit 1 equal to g4's, then the two of them
        const bool hi2 = (g4 & 2) != 0, hi1 = (g4 & 1) != 0;
        const float k0 = hi2 ? ss[2] : ss[0], k1 = hi2 ? ss[3] : ss[1];  // kept
        const float s0 = hi2 ? ss[0] : ss[2], s1 = hi2 ? ss[1] : ss[3];  // sent
        const float t0 = k0 + __shfl_xor(s0, 32), t1 = k1 + __shfl_xor(s1, 32);
        const float kt = hi1 ? t1 : t0, st = hi1 ? t0 : t1;
        const float tot = kt + __shfl_xor(st, 16);
        const int row = r0 + kChunkRows * c + 16 * g4 + n16;
        if (h < H && row < Lb)
            rho[((size_t)b * L_cap + row) * H + h] = (uint16_t)f32_to_bf16_bits(rms_scale(tot, D, eps));
        if constexpr (C + 1 >= CH) {
            return false;
        } else {
            // chunk c + 1's buffer last held chunk c - 1, which every wave finished before the last barrier
            store_sh(sv[(K + 1) & 1], (c + 1) % 2);
            __syncthreads();
            return r0 + kChunkRows * (c + 1) < Lb;  // (workgroup-uniform)
        }
    };
    for_each_while(chunk, std::make_integer_sequence<int, CH>{});
}

template <typename T>
__global__ void __launch_bounds__(256) key_scales_simple_kernel(int batch, int H, int D, int R, int L_cap, int max_len,
                                                                int n_last, int n_rows, float eps,
                                                                const int32_t* __restrict__ seq_lens,
                                                                const T* __restrict__ shared, const T* __restrict__ z,
                                                                const T* __restrict__ basis, T* __restrict__ rho) {
    const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (size_t)batch * n_rows * H) return;
    const int h = (int)(idx % H);
    const int k = (int)((idx / H) % n_rows);
    const int b = (int)(idx / ((size_t)H * n_rows));
    const int Lb = clamped_len(seq_lens, b, max_len);
    const int row = max(0, Lb - n_last) + k;
    if (row >= Lb) return;
    const size_t zr = (((size_t)b * L_cap + row) * H + h) * R;
    float ss = 0.f;
    for (int c = 0; c < D; ++c) {
        float v = elem<T>::load(shared, ((size_t)b * L_cap + row) * D + c);
        for (int i = 0; i < R; ++i) v = fmaf(elem<T>::load(z, zr + i), elem<T>::load(basis, ((size_t)h * D + c) * R + i), v);
        ss = fmaf(v, v, ss);
    }
    const float s = rms_scale(ss, D, eps);
    const size_t o = ((size_t)b * L_cap + row) * H + h;
    if constexpr (sizeof(T) == 4) rho[o] = s;
    else rho[o] = (T)f32_to_bf16_bits(s);
}

// one wave per (b, h): q_eff = g_k * ((g_q * q) * inv_rms(q)), rounded once to the storage dtype
template <typename T>
__global__ void __launch_bounds__(64) norm_query_kernel(int H, int D, float eps, const T* __restrict__ q,
                                                        const T* __restrict__ g_q, const T* __restrict__ g_k,
                                                        T* __restrict__ q_eff) {
    const int h = blockIdx.x, b = blockIdx.y, lane = threadIdx.x;
    const size_t row = ((size_t)b * H + h) * D;
    float ss = 0.f;
    for (int c = lane; c < D; c += 64) {
        const float x = elem<T>::load(q, row + c);
        ss = fmaf(x, x, ss);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) ss += __shfl_xor(ss, o);
    const float inv = rms_scale(ss, D, eps);
    for (int c = lane; c < D; c += 64) {
        const float x = elem<T>::load(q, row + c);
        const float v = elem<T>::load(g_k, (size_t)h * D + c) * ((elem<T>::load(g_q, (size_t)h * D + c) * x) * inv);
        if constexpr (sizeof(T) == 4) q_eff[row + c] = v;
        else q_eff[row + c] = (T)f32_to_bf16_bits(v);
    }
}

}  // namespace

hipError_t launch_key_scales(int batch, int H, int d_h, int r, int L_cap, int dtype, int max_len, int n_last,
                             float eps, const int32_t* seq_lens, const void* k_shared, const void* z_k,
                             const void* B_k, void* rho, hipStream_t stream) {
    const int n_rows = std::min(n_last, max_len);
    if (n_rows <= 0) return hipSuccess;
    // (the rows kernel sizes its buffer resources in 31-bit byte counts)
    const bool rows_fit = (size_t)L_cap * H * r * 2 < ((size_t)1 << 31);
    if (dtype == 1 && (d_h == 64 || d_h == 128) && r % 8 == 0 && r > 0 && r <= 64 && rows_fit) {
        // chunks of 64 rows per workgroup: B^K_h serves that many rows; a long history takes 32 (2048 rows: the
        // long-context whole history runs as one resident round of 256 workgroups, 153 us against 158 with 16),
        // a short pass (an append's single row) 1; LRKV_KS_CHUNKS overrides (tuning, read at every call).
        // (Eight chunks spilled registers with two chunks ahead, so that count is not built.)
        int ch = n_rows >= 16384 ? 32 : n_rows >= 4096 ? 16 : n_rows >= 1024 ? 4 : 1;
        if (const char* e = getenv("LRKV_KS_CHUNKS")) ch = atoi(e);
        ch = (ch >= 32) ? 32 : (ch >= 16) ? 16 : (ch >= 4) ? 4 : 1;
        dim3 grid((n_rows + kChunkRows * ch - 1) / (kChunkRows * ch), (H + kRowWaves - 1) / kRowWaves, batch);
        const bool full = r == 32 || r == 64;
        auto pick_f = [&](auto d_tag, auto k_tag, auto f_tag) {
            constexpr int DD = decltype(d_tag)::value, KK = decltype(k_tag)::value;
            constexpr bool FF = decltype(f_tag)::value;
            return ch == 32 ? key_scales_rows_kernel<DD, KK, 32, FF> : ch == 16 ? key_scales_rows_kernel<DD, KK, 16, FF>
                   : ch == 4 ? key_scales_rows_kernel<DD, KK, 4, FF> : key_scales_rows_kernel<DD, KK, 1, FF>;
        };
        auto pick = [&](auto d_tag, auto k_tag) {
            return full ? pick_f(d_tag, k_tag, std::true_type{}) : pick_f(d_tag, k_tag, std::false_type{});
        };
        using I64 = std::integral_constant<int, 64>;
        using I128 = std::integral_constant<int, 128>;
        using K1 = std::integral_constant<int, 1>;
        using K2 = std::integral_constant<int, 2>;
        auto kern = (d_h == 64) ? (r <= 32 ? pick(I64{}, K1{}) : pick(I64{}, K2{}))
                                : (r <= 32 ? pick(I128{}, K1{}) : pick(I128{}, K2{}));
        hipLaunchKernelGGL(kern, grid, dim3(kRowWaves * 64), 0, stream, H, r, L_cap, max_len, n_last, eps, seq_lens,
                           (const uint16_t*)k_shared, (const uint16_t*)z_k, (const uint16_t*)B_k, (uint16_t*)rho);
    } else if (dtype == 1 && d_h % 16 == 0 && r % 8 == 0 && r > 0 && r <= 64) {
        dim3 grid((n_rows + 16 * kWaves - 1) / (16 * kWaves), H, batch);
        auto kern = (r <= 32) ? key_scales_mfma_kernel<1> : key_scales_mfma_kernel<2>;
        hipLaunchKernelGGL(kern, grid, dim3(kWaves * 64), 0, stream, H, d_h, r, L_cap, max_len, n_last, eps, seq_lens,
                           (const uint16_t*)k_shared, (const uint16_t*)z_k, (const uint16_t*)B_k, (uint16_t*)rho);
    } else {
        const size_t total = (size_t)batch * n_rows * H;
        dim3 grid((unsigned)((total + 255) / 256));
        if (dtype == 0)
            hipLaunchKernelGGL(key_scales_simple_kernel<float>, grid, dim3(256), 0, stream, batch, H, d_h, r, L_cap,
                               max_len, n_last, n_rows, eps, seq_lens, (const float*)k_shared, (const float*)z_k,
                               (const float*)B_k, (float*)rho);
        else
            hipLaunchKernelGGL(key_scales_simple_kernel<uint16_t>, grid, dim3(256), 0, stream, batch, H, d_h, r, L_cap,
                               max_len, n_last, n_rows, eps, seq_lens, (const uint16_t*)k_shared,
                               (const uint16_t*)z_k, (const uint16_t*)B_k, (uint16_t*)rho);
    }
    return hipGetLastError();
}

hipError_t launch_norm_query(int batch, int H, int d_h, int dtype, float eps, const void* q, const void* g_q,
                             const void* g_k, void* q_eff, hipStream_t stream) {
    dim3 grid(H, batch);
    if (dtype == 0)
        hipLaunchKernelGGL(norm_query_kernel<float>, grid, dim3(64), 0, stream, H, d_h, eps, (const float*)q,
                           (const float*)g_q, (const float*)g_k, (float*)q_eff);
    else
        hipLaunchKernelGGL(norm_query_kernel<uint16_t>, grid, dim3(64), 0, stream, H, d_h, eps, (const uint16_t*)q,
                           (const uint16_t*)g_q, (const uint16_t*)g_k, (uint16_t*)q_eff);
    return hipGetLastError();
}

}  // namespace lrkv
