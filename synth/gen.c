/*
 * Seeded synthetic input generator shared by the tests, the benchmark and the
 * CPU reference.  It holds no attention arithmetic: it only turns
 * (seed, element index) into numbers with a stated distribution.
 *
 * Generator: counter based.  Elements 2k and 2k+1 of a stream with seed S
 * share two 64-bit words  w_c = mix64(S ^ mix64(2k + c)), c in {0, 1}, where
 * mix64 is the SplitMix64 output function (Steele, Lea, Flood, "Fast
 * splittable pseudorandom number generators", OOPSLA 2014).  The top 53 bits
 * of each word give uniforms u1, u2 in (0, 1); the Box-Muller transform (Box
 * and Muller, 1958) turns them into two independent N(0, 1) samples:
 * element 2k = sqrt(-2 ln u1) cos(2 pi u2), element 2k+1 = the same with sin.
 * Because every element depends only on (S, k), any slice of a tensor can be
 * regenerated on its own and the result does not depend on the thread count.
 *
 * Rounding: the fp64 sample times the standard deviation is rounded to fp32
 * (round to nearest even, by the C conversion), and for bf16 the fp32 value is
 * rounded again to bf16 (round to nearest even on the 16 dropped bits).
 */
#define _GNU_SOURCE
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
    const uint64_t pair = k >> 1;
    double u1 = unit_open(seed, 2 * pair);
    double u2 = unit_open(seed, 2 * pair + 1);
    double rad = sqrt(-2.0 * log(u1));
    return (k & 1) ? rad * sin(two_pi * u2) : rad * cos(two_pi * u2);
}

/* Fill out[0..n) with elements offset .. offset+n-1, computing each pair once. */
#define FILL_PAIRS(CONVERT)                                                              \
    do {                                                                                 \
        const double two_pi = 6.283185307179586476925286766559;                         \
        uint64_t first = offset, last = offset + n; /* [first, last) */                 \
        uint64_t p0 = first >> 1, p1 = (last + 1) >> 1;                                 \
        _Pragma("omp parallel for num_threads(nthreads) schedule(static)")              \
        for (uint64_t p = p0; p < p1; ++p) {                                             \
            double u1 = unit_open(seed, 2 * p), u2 = unit_open(seed, 2 * p + 1);        \
            double rad = sqrt(-2.0 * log(u1)), sn, cs;                                   \
            sincos(two_pi * u2, &sn, &cs);                                               \
            uint64_t e0 = 2 * p, e1 = 2 * p + 1;                                         \
            if (e0 >= first && e0 < last) out[e0 - first] = CONVERT(stddev * (rad * cs)); \
            if (e1 >= first && e1 < last) out[e1 - first] = CONVERT(stddev * (rad * sn)); \
        }                                                                                \
    } while (0)

#define CONV_F32(x) ((float)(x))
#define CONV_BF16(x) f32_to_bf16_rne((float)(x))
#define CONV_F64(x) (x)

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
    FILL_PAIRS(CONV_F32);
}

/* out[k] = bf16 bits of fp32(std * N(0,1) at counter offset + k) */
void synth_normal_bf16(uint64_t seed, double stddev, uint64_t offset, uint16_t* out, size_t n, int nthreads) {
    FILL_PAIRS(CONV_BF16);
}

/* out[k] = fp64 std * N(0,1) at counter offset + k (no rounding) */
void synth_normal_f64(uint64_t seed, double stddev, uint64_t offset, double* out, size_t n, int nthreads) {
    FILL_PAIRS(CONV_F64);
}

/* one element (for checks of the bulk fill) */
double synth_normal_one(uint64_t seed, uint64_t k) { return normal_at(seed, k); }

/* out[k] uniform integer in [lo, hi] (inclusive) at counter offset + k */
void synth_uniform_int(uint64_t seed, int32_t lo, int32_t hi, uint64_t offset, int32_t* out, size_t n) {
    double span = (double)hi - (double)lo + 1.0;
    for (size_t k = 0; k < n; ++k) {
        int64_t v = (int64_t)lo + (int64_t)floor(unit_open(seed, offset + k) * span);
        if (v > hi) v = hi;
        out[k] = (int32_t)v;
    }
}
