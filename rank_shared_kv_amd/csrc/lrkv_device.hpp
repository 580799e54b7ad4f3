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

// log2(e): scores are carried in log2 units so that exp2 (v_exp_f32) applies.
constexpr float kLog2e = 1.4426950408889634f;

}  // namespace lrkv
