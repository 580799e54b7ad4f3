// Materialised per-head keys and values from the factored cache:
//   K_h[j] = k_shared[j] + z^K_{h,j} (B^K_h)^T,   V_h[j] = v_shared[j] + z^V_{h,j} (B^V_h)^T
// for every live row j < seq_lens[b] ("Low-Rank Key Value Attention: Chinese
// reading notes", sec. 2.1 Eqs. (2)-(5); "Low-Rank Key Value Attention | What
// a shared cache can preserve", sec. 3: the rebuilt form training and prefill
// use).  Output [batch][H][L_cap][d_h] in the cache dtype.
//
// bf16 path (r <= 64): per 16-column block of d_h and 16 rows,
// Out^T[16 cols x 16 rows] = B_h[16 x r] Z^T[r x 16] on v_mfma_f32_16x16x32_bf16
// (k-steps of 32 rank coordinates; coordinates past r enter as zeros).  In that
// layout each lane holds four consecutive columns of one row, so the shared row
// is added and the result stored 8 bytes at a time.  With d_h = 64 or 128 the
// four waves of a workgroup take four heads of the same 256 rows, in chunks of
// 64 rows whose shared rows the workgroup stages in LDS; each wave fetches its
// B_h fragments (16 KB at d_h = 128, r = 64, from L2) once, the next chunk's
// loads are in flight while a chunk computes, and the products of 16 rows pass
// through LDS so that whole rows are written out (16 bytes per lane, 256
// contiguous bytes per row at d_h = 128), the shared row added before the
// single rounding.  Other d_h: a wave per 16 rows, one column block at a time.
// fp32 (or shapes off the grid): one thread per output element.
#include "lrkv_device.hpp"
#include "lrkv_internal.hpp"

namespace lrkv {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;  // 64 rows of one head per workgroup

// NKS k-steps of 32 rank coordinates (1 for r <= 32, 2 for r <= 64), a compile-time count: the products
// and the reads of their results then sit in one straight-line block, where the compiler places the wait
// states between a matrix-core result and its first read (with a run-time loop count those waits were
// missing at the loop exit and three of the four result registers were read too early).
template <int NKS>
__global__ void __launch_bounds__(kWaves * 64) materialize_mfma_kernel(int H, int D, int R, int L_cap, int max_len,
                                                                       const int32_t* __restrict__ seq_lens,
                                                                       const uint16_t* __restrict__ shared,
                                                                       const uint16_t* __restrict__ z,
                                                                       const uint16_t* __restrict__ basis,
                                                                       uint16_t* __restrict__ out) {
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n16 = lane & 15, g4 = lane >> 4;
    const int h = blockIdx.y, b = blockIdx.z;
    const int Lb = clamped_len(seq_lens, b, max_len);
    const int t0 = (blockIdx.x * kWaves + wave) * 16;
    if (t0 >= Lb) return;
    const int row = t0 + n16;                       // this lane's row (B operand column, result column)
    const int row_c = min(row, L_cap - 1);          // clamped: loads stay inside the allocation
    const uint16_t* zrow = z + (((size_t)b * L_cap + row_c) * H + h) * R;  // token-major latents
    const uint16_t* bh = basis + (size_t)h * D * R;
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
        // lane (row n16, g4) holds columns 16 cb + 4 g4 + i of its row
        if (row < Lb) {
            const int c0 = 16 * cb + 4 * g4;
            const u32x2_t s = *(const u32x2_t*)(shared + ((size_t)b * L_cap + row) * D + c0);
            const float v0 = acc[0] + bf16_lo(s[0]), v1 = acc[1] + bf16_hi(s[0]);
            const float v2 = acc[2] + bf16_lo(s[1]), v3 = acc[3] + bf16_hi(s[1]);
            u32x2_t o;
            o[0] = f32_to_bf16_bits(v0) | (f32_to_bf16_bits(v1) << 16);
            o[1] = f32_to_bf16_bits(v2) | (f32_to_bf16_bits(v3) << 16);
            *(u32x2_t*)(out + (((size_t)b * H + h) * L_cap + row) * D + c0) = o;
        }
    }
}

// the operands of one rebuilt matrix (keys or values)
struct MatOperands {
    const uint16_t* shared;  // [batch][L_cap][d_h]
    const uint16_t* z;       // [batch][L_cap][H][r]
    const uint16_t* basis;   // [H][d_h][r]
    uint16_t* out;           // [batch][H][L_cap][d_h]
};

constexpr int kChunkRows = 64;  // rows per chunk in the d_h = 64 / 128 kernel
constexpr int kChunks = 4;      // chunks per workgroup: 256 rows, one B_h fetch per wave

// Keys and values in one launch: blockIdx.z = batch * (0 for keys, 1 for values) + b.  The workgroup's
// waves take heads 4 y .. 4 y + 3 of the same 256 rows, in 4 chunks of 64 (rows past L_b: stand-ins,
// computed, not stored).  Each wave loads its head's B_h fragments once.  The chunk's shared rows are staged
// in LDS by the whole workgroup (two buffers: the next chunk's rows and latents load while the current chunk
// computes), and the products of 16 rows pass through a per-wave LDS tile so that whole rows are written.
template <int D, int NKS>
__global__ void __launch_bounds__(kWaves * 64) materialize_rows_kernel(int batch, int H, int R, int L_cap,
                                                                       int max_len,
                                                                       const int32_t* __restrict__ seq_lens,
                                                                       MatOperands kop, MatOperands vop) {
    constexpr int CB = D / 16;
    constexpr int SROW = D + 8;                               // bf16 per staged shared row
    constexpr int PPT = kChunkRows * (D / 8) / (kWaves * 64);  // 16-byte pieces of a chunk per thread
    constexpr int XS = D + 4;                                 // floats per staged product row
    constexpr int LPR = D / 8;                                // lanes per row in the write-out (8 columns each)
    constexpr int RPI = 64 / LPR;                             // rows per write-out instruction
    __shared__ __attribute__((aligned(16))) uint16_t sh_l[2][kChunkRows * SROW];
    __shared__ __attribute__((aligned(16))) float xs_all[kWaves][16 * XS];
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    float* xs = xs_all[wave];
    const int n16 = lane & 15, g4 = lane >> 4;
    const int h = blockIdx.y * kWaves + wave;
    const int hc = min(h, H - 1);  // waves past the last head compute a stand-in and store nothing
    const bool is_v = (int)blockIdx.z >= batch;
    const int b = (int)blockIdx.z - (is_v ? batch : 0);
    const MatOperands op = is_v ? vop : kop;
    const uint16_t* __restrict__ shared = op.shared;
    const uint16_t* __restrict__ z = op.z;
    const uint16_t* __restrict__ basis = op.basis;
    const int Lb = clamped_len(seq_lens, b, max_len);
    const int r0 = blockIdx.x * kChunkRows * kChunks;
    if (r0 >= Lb) return;  // the whole workgroup
    uint16_t* outh = op.out + ((size_t)b * H + hc) * L_cap * D;
    const uint16_t* bh = basis + (size_t)hc * D * R;
    typedef u32x4_t ZFrag[4][NKS];
    auto load_z = [&](ZFrag& zf, int c) {  // latents of rows r0 + 64 c + 16 rg + n16 (past L_b: row L_b - 1)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
            const size_t row = (size_t)min(r0 + kChunkRows * c + 16 * rg + n16, Lb - 1);
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                const int k = 32 * ks + 8 * g4;
                zf[rg][ks] = *(const u32x4_t*)(z + (((size_t)b * L_cap + row) * H + hc) * R + (k < R ? k : 0));
            }
        }
    };
    auto load_sh = [&](u32x4_t (&v)[PPT], int c) {  // piece p: row p / (D / 8), 8 columns at 8 (p % (D / 8))
#pragma unroll
        for (int i = 0; i < PPT; ++i) {
            const int p = tid + kWaves * 64 * i;
            const size_t row = (size_t)min(r0 + kChunkRows * c + p / (D / 8), Lb - 1);
            v[i] = *(const u32x4_t*)(shared + ((size_t)b * L_cap + row) * D + 8 * (p % (D / 8)));
        }
    };
    auto store_sh = [&](const u32x4_t (&v)[PPT], int buf) {
#pragma unroll
        for (int i = 0; i < PPT; ++i) {
            const int p = tid + kWaves * 64 * i;
            *(u32x4_t*)(sh_l[buf] + (p / (D / 8)) * SROW + 8 * (p % (D / 8))) = v[i];
        }
    };
    u32x4_t bf[CB][NKS];  // B_h rows 16 cb + n16 (columns of the key), coordinates 32 ks + 8 g4 (past r: zero)
    u32x4_t sv[PPT];
    ZFrag za, zb;
    load_sh(sv, 0);
    load_z(za, 0);
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            const int k = 32 * ks + 8 * g4;
            bf[cb][ks] = *(const u32x4_t*)(bh + (size_t)(16 * cb + n16) * R + (k < R ? k : 0));
        }
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
        if (32 * ks + 8 * g4 >= R) {
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) bf[cb][ks] = u32x4_t{0u, 0u, 0u, 0u};
        }
    store_sh(sv, 0);
    __syncthreads();
    const int wr = lane / LPR, wc = 8 * (lane % LPR);  // write-out: row within RPI rows, first column
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
        ZFrag& zc = (c & 1) ? zb : za;
        ZFrag& zn = (c & 1) ? za : zb;
        if (c + 1 < kChunks) {  // the next chunk's loads first
            load_sh(sv, c + 1);
            load_z(zn, c + 1);
        }
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
            if (32 * ks + 8 * g4 >= R) {
#pragma unroll
                for (int rg = 0; rg < 4; ++rg) zc[rg][ks] = u32x4_t{0u, 0u, 0u, 0u};
            }
        const uint16_t* shc = sh_l[c & 1];
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
            // the products of 16 rows: lane (row n16, g4) holds columns 16 cb + 4 g4 .. + 3, staged as fp32
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) {
                f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks)
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, bf[cb][ks]),
                                                                  __builtin_bit_cast(bf16x8_t, zc[rg][ks]), acc, 0, 0, 0);
                *(f32x4_t*)(xs + n16 * XS + 16 * cb + 4 * g4) = acc;
            }
            wave_lds_sync();
            // write-out: RPI whole rows per instruction, 8 columns per lane, the shared row added before rounding
#pragma unroll
            for (int it = 0; it < 16 / RPI; ++it) {
                const int rl = RPI * it + wr;  // row within the 16
                const f32x4_t a0 = *(const f32x4_t*)(xs + rl * XS + wc);
                const f32x4_t a1 = *(const f32x4_t*)(xs + rl * XS + wc + 4);
                const u32x4_t sr = *(const u32x4_t*)(shc + (16 * rg + rl) * SROW + wc);
                u32x4_t o;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float lo = (i < 2 ? a0[2 * i] : a1[2 * i - 4]) + bf16_lo(sr[i]);
                    const float hi = (i < 2 ? a0[2 * i + 1] : a1[2 * i - 3]) + bf16_hi(sr[i]);
                    o[i] = f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
                }
                const int row = r0 + kChunkRows * c + 16 * rg + rl;
                if (h < H && row < Lb) *(u32x4_t*)(outh + (size_t)row * D + wc) = o;
            }
            wave_lds_sync();  // the product tile is rewritten by the next row group
        }
        if (c + 1 < kChunks) {
            store_sh(sv, (c + 1) & 1);  // that buffer's chunk finished before the previous barrier
            __syncthreads();
        }
    }
}

template <typename T>
__global__ void __launch_bounds__(256) materialize_simple_kernel(int batch, int H, int D, int R, int L_cap,
                                                                 int max_len, const int32_t* __restrict__ seq_lens,
                                                                 const T* __restrict__ shared,
                                                                 const T* __restrict__ z, const T* __restrict__ basis,
                                                                 T* __restrict__ out) {
    const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
    const size_t total = (size_t)batch * H * max_len * D;
    if (idx >= total) return;
    const int c = (int)(idx % D);
    const int row = (int)((idx / D) % max_len);
    const int h = (int)((idx / ((size_t)D * max_len)) % H);
    const int b = (int)(idx / ((size_t)D * max_len * H));
    if (row >= clamped_len(seq_lens, b, max_len)) return;
    float s = elem<T>::load(shared, ((size_t)b * L_cap + row) * D + c);
    const size_t zr = (((size_t)b * L_cap + row) * H + h) * R;
    for (int i = 0; i < R; ++i) s = fmaf(elem<T>::load(z, zr + i), elem<T>::load(basis, ((size_t)h * D + c) * R + i), s);
    const size_t o = (((size_t)b * H + h) * L_cap + row) * D + c;
    if constexpr (sizeof(T) == 4) out[o] = s;
    else out[o] = (T)f32_to_bf16_bits(s);
}

hipError_t launch_one(int batch, int H, int d_h, int r, int L_cap, int dtype, int max_len, const int32_t* seq_lens,
                      const void* shared, const void* z, const void* basis, void* out, hipStream_t stream) {
    if (max_len == 0) return hipSuccess;
    if (dtype == 1 && d_h % 16 == 0 && r % 8 == 0 && r > 0 && r <= 64) {
        dim3 grid((max_len + 16 * kWaves - 1) / (16 * kWaves), H, batch);
        auto kern = (r <= 32) ? materialize_mfma_kernel<1> : materialize_mfma_kernel<2>;
        hipLaunchKernelGGL(kern, grid, dim3(kWaves * 64), 0, stream, H, d_h, r, L_cap, max_len, seq_lens,
                           (const uint16_t*)shared, (const uint16_t*)z, (const uint16_t*)basis, (uint16_t*)out);
    } else {
        const size_t total = (size_t)batch * H * max_len * d_h;
        dim3 grid((unsigned)((total + 255) / 256));
        if (dtype == 0)
            hipLaunchKernelGGL(materialize_simple_kernel<float>, grid, dim3(256), 0, stream, batch, H, d_h, r, L_cap,
                               max_len, seq_lens, (const float*)shared, (const float*)z, (const float*)basis,
                               (float*)out);
        else
            hipLaunchKernelGGL(materialize_simple_kernel<uint16_t>, grid, dim3(256), 0, stream, batch, H, d_h, r,
                               L_cap, max_len, seq_lens, (const uint16_t*)shared, (const uint16_t*)z,
                               (const uint16_t*)basis, (uint16_t*)out);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_materialize(int batch, int H, int d_h, int r, int L_cap, int dtype, int max_len,
                              const int32_t* seq_lens, const void* k_shared, const void* v_shared, const void* z_k,
                              const void* z_v, const void* B_k, const void* B_v, void* K_out, void* V_out,
                              hipStream_t stream) {
    if (max_len > 0 && dtype == 1 && (d_h == 64 || d_h == 128) && r % 8 == 0 && r > 0 && r <= 64 &&
        2 * (long)batch <= 65535) {  // grid z: keys and values of every sequence
        dim3 grid((max_len + kChunkRows * kChunks - 1) / (kChunkRows * kChunks), (H + kWaves - 1) / kWaves,
                  2 * batch);
        auto kern = (d_h == 64) ? (r <= 32 ? materialize_rows_kernel<64, 1> : materialize_rows_kernel<64, 2>)
                                : (r <= 32 ? materialize_rows_kernel<128, 1> : materialize_rows_kernel<128, 2>);
        const MatOperands kop{(const uint16_t*)k_shared, (const uint16_t*)z_k, (const uint16_t*)B_k, (uint16_t*)K_out};
        const MatOperands vop{(const uint16_t*)v_shared, (const uint16_t*)z_v, (const uint16_t*)B_v, (uint16_t*)V_out};
        hipLaunchKernelGGL(kern, grid, dim3(kWaves * 64), 0, stream, batch, H, r, L_cap, max_len, seq_lens, kop, vop);
        return hipGetLastError();
    }
    hipError_t e = launch_one(batch, H, d_h, r, L_cap, dtype, max_len, seq_lens, k_shared, z_k, B_k, K_out, stream);
    if (e != hipSuccess) return e;
    return launch_one(batch, H, d_h, r, L_cap, dtype, max_len, seq_lens, v_shared, z_v, B_v, V_out, stream);
}

}  // namespace lrkv
