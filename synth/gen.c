/*
 * Seeded synthetic input generator shared by the tests, the benchmark and the
 * CPU reference.  It holds no attention arithmetic: it only turns
 * (seed, element index) into numbers with a stated distribution.
 *
 * Generator: counter based.  Element k of a stream with seed S uses two 64-bit
 * words  w = mix64(S ^ mix64(2k + c)), c in {0, 1}, where mix64 is the
 * SplitMix64 output function (Steele, Lea, Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014).  The top 53 bits of each word
 * give a uniform u in (0, 1); the pair goes through the Box-Muller transform
 * (Box and Muller, 1958), cosine branch only, to give one N(0, 1) sample.
 * Because every element depends only on (S, k), any slice of a tensor can be
 * regenerated on its own and the result does not depend on the thread count.
 *
 * Rounding: the fp64 sample times the standard deviation is rounded to fp32
 * (round to nearest even, by the C conversion), and for bf16 the fp32 value is
 * rounded again to bf16 (round to nearest even on the 16 dropped bits).
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>
#include <string.h>

static inline uint64_t mix64(uint64_t z) {
    z += 0x9e3779b97f4a7c15ull;
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    return z ^ (z >> 31);
}

/* uniform in (0, 1): (top 53 bits + 0.5) * 2^-53, never 0 or 1 */
static inline double unit_open(uint64_t seed, uint64_t counter) {
    uint64_t w = mix64(seed ^ mix64(counter));
    return ((double)(w >> 11) + 0.5) * (1.0 / 9007199254740992.0);
}

static inline double normal_at(uint64_t seed, uint64_t k) {
    const double two_pi = 6.283185307179586476925286766559;
    double u1 = unit_open(seed, 2 * k);
    double u2 = unit_open(seed, 2 * k + 1);
    return sqrt(-2.0 * log(u1)) * cos(two_pi * u2);
}

static inline uint16_t f32_to_bf16_rne(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7f800000u) == 0x7f800000u) /* inf / nan: truncate, keep a nan quiet */
        return (uint16_t)((u >> 16) | ((u & 0xffffu) ? 0x40u : 0u));
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

/* out[k] = fp32(std * N(0,1) at counter offset + k), k in [0, n) */
void synth_normal_f32(uint64_t seed, double stddev, uint64_t offset, float* out, size_t n, int nthreads) {
#pragma omp parallel for num_threads(nthreads) schedule(static)
    for (size_t k = 0; k < n; ++k) out[k] = (float)(stddev * normal_at(seed, offset + k));
}

/* out[k] = bf16 bits of fp32(std * N(0,1) at counter offset + k) */
void synth_normal_bf16(uint64_t seed, double stddev, uint64_t offset, uint16_t* out, size_t n, int nthreads) {
#pragma omp parallel for num_threads(nthreads) schedule(static)
    for (size_t k = 0; k < n; ++k) out[k] = f32_to_bf16_rne((float)(stddev * normal_at(seed, offset + k)));
}

/* out[k] = fp64 std * N(0,1) at counter offset + k (no rounding) */
void synth_normal_f64(uint64_t seed, double stddev, uint64_t offset, double* out, size_t n, int nthreads) {
#pragma omp parallel for num_threads(nthreads) schedule(static)
    for (size_t k = 0; k < n; ++k) out[k] = stddev * normal_at(seed, offset + k);
}

/* out[k] uniform integer in [lo, hi] (inclusive) at counter offset + k */
void synth_uniform_int(uint64_t seed, int32_t lo, int32_t hi, uint64_t offset, int32_t* out, size_t n) {
    double span = (double)hi - (double)lo + 1.0;
    for (size_t k = 0; k < n; ++k) {
        int64_t v = (int64_t)lo + (int64_t)floor(unit_open(seed, offset + k) * span);
        if (v > hi) v = hi;
        out[k] = (int32_t)v;
    }
}
