/*
 * CPU reference ("oracle") for LRKV decode attention, fp64 throughout.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links or calls
 * this file; only the tests, the smoke check and the benchmark's CPU-baseline
 * leg load it.  It shares no code with the GPU path.
 *
 * What it computes (for every requested (sequence b, head h)):
 *   the plain definition of one decode step of low-rank key-value attention
 *   with the per-head keys and values rebuilt in full:
 *     K_h = K_shared + Z^K_h (B^K_h)^T,   V_h = V_shared + Z^V_h (B^V_h)^T
 *       -- "Low-Rank Key Value Attention: reading notes" (zh), sec. 2.1,
 *          Eqs. (2)-(5); "Low-Rank Key Value Attention | What a shared cache
 *          can preserve", sec. 3 (weight factorisation to token coordinates)
 *     s_j = q_h . K_h[j] / sqrt(d_h)  for every live row j < L_b
 *     a   = softmax(s)             (max-shifted exponentials over their sum)
 *     o_h = sum_j a_j V_h[j]
 *       -- same review, sec. 2 (attention as routing and retrieval: score,
 *          weight and output equations); reading notes sec. 2.4.
 *   Single-query decode: the query's own row is already in the cache, every
 *   live row is visible, rows at or beyond seq_lens[b] are not read.
 *   A sequence with no live rows gives o_h = 0.
 *
 * Also provided:
 *   oracle_mqa_decode      K_h = K_shared, V_h = V_shared (r = 0 sharing;
 *                          reading notes sec. 1 cache table, MQA row)
 *   oracle_factored_decode the associative evaluation of reading notes
 *                          sec. 2.4, Eqs. (6)-(7): p = q B^K, score =
 *                          q.k_s + p.z^K, o = a V_s + (a Z^V)(B^V)^T.  Used
 *                          only to check the associativity identity.
 *
 * Input element types (dtype argument): 0 = fp32, 1 = bf16 bit patterns
 * (uint16), 2 = fp64.  Every element is widened exactly to double.
 *
 * Layouts (row-major):  q [batch][H][d_h];  k_s, v_s [batch][L_cap][d_h];
 *   z_k, z_v [batch][H][L_cap][r];  B_k, B_v [H][d_h][r];  seq_lens [batch].
 * Output: out[p][d_h] for pair p = (pair_b[p], pair_h[p]); optionally the
 *   attention weights weights[p][L_cap] (entries past L_b are set to 0).
 *
 * ORACLE_PLANT (compile-time, default 0) plants one known mistake so the tests
 * can show that the pins catch it; the shipped build never sets it.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifndef ORACLE_PLANT
#define ORACLE_PLANT 0
#endif

typedef struct {
    int32_t batch, H, d_h, r, L_cap, dtype;
} oracle_dims;

static double elem(const void* base, int dtype, size_t i) {
    if (dtype == 0) return (double)((const float*)base)[i];
    if (dtype == 2) return ((const double*)base)[i];
    uint32_t u = (uint32_t)((const uint16_t*)base)[i] << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

static int check_dims(const oracle_dims* d) {
    if (!d || d->batch < 0 || d->H <= 0 || d->d_h <= 0 || d->r < 0 || d->L_cap < 0) return -1;
    if (d->dtype < 0 || d->dtype > 2) return -1;
    return 0;
}

/* softmax over n scores into a (fp64), returns 0 */
static void softmax(const double* s, int n, double* a) {
    double m = -INFINITY;
    for (int j = 0; j < n; ++j)
        if (s[j] > m) m = s[j];
    double z = 0.0;
    for (int j = 0; j < n; ++j) {
        a[j] = exp(s[j] - m);
        z += a[j];
    }
    for (int j = 0; j < n; ++j) a[j] = a[j] / z;
}

static int live_rows(const oracle_dims* d, const int32_t* seq_lens, int b) {
    int L = seq_lens[b];
    if (L < 0) L = 0;
    if (L > d->L_cap) L = d->L_cap;
    return L;
}

/* One (b, h): rebuild K_h and V_h, then attend. */
static void lrkv_pair(const oracle_dims* d, const void* q, const void* k_s, const void* v_s, const void* z_k,
                      const void* z_v, const void* B_k, const void* B_v, int L, int b, int h, double* out,
                      double* weights) {
    const int D = d->d_h, R = d->r, T = d->dtype;
    const size_t cap = (size_t)d->L_cap;
    for (int c = 0; c < D; ++c) out[c] = 0.0;
    if (weights)
        for (size_t j = 0; j < cap; ++j) weights[j] = 0.0;
    if (L == 0) return;

    double* Kh = (double*)malloc(sizeof(double) * (size_t)L * D);
    double* Vh = (double*)malloc(sizeof(double) * (size_t)L * D);
    double* s = (double*)malloc(sizeof(double) * (size_t)L);
    double* a = (double*)malloc(sizeof(double) * (size_t)L);
    const size_t shared0 = (size_t)b * cap * D;
    const size_t lat0 = ((size_t)b * d->H + h) * cap * R;
    const size_t basis0 = (size_t)h * D * R;

    /* K_h[j][c] = k_s[j][c] + sum_i z_k[j][i] * B_k[c][i]; V_h likewise */
    for (int j = 0; j < L; ++j) {
        for (int c = 0; c < D; ++c) {
            double kk = 0.0, vv = 0.0;
            for (int i = 0; i < R; ++i) {
                kk += elem(z_k, T, lat0 + (size_t)j * R + i) * elem(B_k, T, basis0 + (size_t)c * R + i);
                vv += elem(z_v, T, lat0 + (size_t)j * R + i) * elem(B_v, T, basis0 + (size_t)c * R + i);
            }
#if ORACLE_PLANT == 1 /* planted: private key term dropped */
            kk = 0.0;
#endif
#if ORACLE_PLANT == 2 /* planted: wrong sign on the private value term */
            vv = -vv;
#endif
            Kh[(size_t)j * D + c] = elem(k_s, T, shared0 + (size_t)j * D + c) + kk;
            Vh[(size_t)j * D + c] = elem(v_s, T, shared0 + (size_t)j * D + c) + vv;
        }
    }
    /* s_j = q . K_h[j] / sqrt(d_h) */
    const size_t q0 = ((size_t)b * d->H + h) * D;
    double scale = 1.0 / sqrt((double)D);
#if ORACLE_PLANT == 3 /* planted: scale by 1/sqrt(r) instead of 1/sqrt(d_h) */
    scale = 1.0 / sqrt((double)(R > 0 ? R : 1));
#endif
    for (int j = 0; j < L; ++j) {
        double dot = 0.0;
        for (int c = 0; c < D; ++c) dot += elem(q, T, q0 + c) * Kh[(size_t)j * D + c];
        s[j] = dot * scale;
    }
#if ORACLE_PLANT == 4 /* planted: last visible row masked out */
    if (L > 1) s[L - 1] = -INFINITY;
#endif
    softmax(s, L, a);
    /* o = sum_j a_j V_h[j] */
    for (int j = 0; j < L; ++j)
        for (int c = 0; c < D; ++c) out[c] += a[j] * Vh[(size_t)j * D + c];
    if (weights)
        for (int j = 0; j < L; ++j) weights[j] = a[j];
    free(Kh);
    free(Vh);
    free(s);
    free(a);
}

int oracle_lrkv_decode(const oracle_dims* d, const void* q, const void* k_s, const void* v_s, const void* z_k,
                       const void* z_v, const void* B_k, const void* B_v, const int32_t* seq_lens, int npairs,
                       const int32_t* pair_b, const int32_t* pair_h, double* out, double* weights, int nthreads) {
    if (check_dims(d) || npairs < 0) return -1;
    if (d->r > 0 && (!z_k || !z_v || !B_k || !B_v)) return -1;
    for (int p = 0; p < npairs; ++p)
        if (pair_b[p] < 0 || pair_b[p] >= d->batch || pair_h[p] < 0 || pair_h[p] >= d->H) return -1;
    if (nthreads < 1) nthreads = 1;
#pragma omp parallel for num_threads(nthreads) schedule(dynamic, 1)
    for (int p = 0; p < npairs; ++p) {
        int b = pair_b[p], h = pair_h[p];
        lrkv_pair(d, q, k_s, v_s, z_k, z_v, B_k, B_v, live_rows(d, seq_lens, b), b, h, out + (size_t)p * d->d_h,
                  weights ? weights + (size_t)p * d->L_cap : NULL);
    }
    return 0;
}

/* MQA: every head reads the same shared keys and values. */
int oracle_mqa_decode(const oracle_dims* d, const void* q, const void* k_s, const void* v_s, const int32_t* seq_lens,
                      int npairs, const int32_t* pair_b, const int32_t* pair_h, double* out, int nthreads) {
    if (check_dims(d) || npairs < 0) return -1;
    for (int p = 0; p < npairs; ++p)
        if (pair_b[p] < 0 || pair_b[p] >= d->batch || pair_h[p] < 0 || pair_h[p] >= d->H) return -1;
    if (nthreads < 1) nthreads = 1;
    const int D = d->d_h, T = d->dtype;
    const size_t cap = (size_t)d->L_cap;
#pragma omp parallel for num_threads(nthreads) schedule(dynamic, 1)
    for (int p = 0; p < npairs; ++p) {
        int b = pair_b[p], h = pair_h[p];
        int L = live_rows(d, seq_lens, b);
        double* o = out + (size_t)p * D;
        for (int c = 0; c < D; ++c) o[c] = 0.0;
        if (L == 0) continue;
        double* s = (double*)malloc(sizeof(double) * (size_t)L);
        double* a = (double*)malloc(sizeof(double) * (size_t)L);
        const size_t shared0 = (size_t)b * cap * D;
        const size_t q0 = ((size_t)b * d->H + h) * D;
        const double scale = 1.0 / sqrt((double)D);
        for (int j = 0; j < L; ++j) {
            double dot = 0.0;
            for (int c = 0; c < D; ++c) dot += elem(q, T, q0 + c) * elem(k_s, T, shared0 + (size_t)j * D + c);
            s[j] = dot * scale;
        }
        softmax(s, L, a);
        for (int j = 0; j < L; ++j)
            for (int c = 0; c < D; ++c) o[c] += a[j] * elem(v_s, T, shared0 + (size_t)j * D + c);
        free(s);
        free(a);
    }
    return 0;
}

/* Associative (factored) evaluation, reading notes sec. 2.4 Eqs. (6)-(7). */
int oracle_factored_decode(const oracle_dims* d, const void* q, const void* k_s, const void* v_s, const void* z_k,
                           const void* z_v, const void* B_k, const void* B_v, const int32_t* seq_lens, int npairs,
                           const int32_t* pair_b, const int32_t* pair_h, double* out, int nthreads) {
    if (check_dims(d) || npairs < 0) return -1;
    if (d->r > 0 && (!z_k || !z_v || !B_k || !B_v)) return -1;
    for (int p = 0; p < npairs; ++p)
        if (pair_b[p] < 0 || pair_b[p] >= d->batch || pair_h[p] < 0 || pair_h[p] >= d->H) return -1;
    if (nthreads < 1) nthreads = 1;
    const int D = d->d_h, R = d->r, T = d->dtype;
    const size_t cap = (size_t)d->L_cap;
#pragma omp parallel for num_threads(nthreads) schedule(dynamic, 1)
    for (int p = 0; p < npairs; ++p) {
        int b = pair_b[p], h = pair_h[p];
        int L = live_rows(d, seq_lens, b);
        double* o = out + (size_t)p * D;
        for (int c = 0; c < D; ++c) o[c] = 0.0;
        if (L == 0) continue;
        double* s = (double*)malloc(sizeof(double) * (size_t)L);
        double* a = (double*)malloc(sizeof(double) * (size_t)L);
        double* pq = (double*)calloc((size_t)(R > 0 ? R : 1), sizeof(double));
        double* u = (double*)calloc((size_t)(R > 0 ? R : 1), sizeof(double));
        const size_t shared0 = (size_t)b * cap * D;
        const size_t lat0 = ((size_t)b * d->H + h) * cap * R;
        const size_t basis0 = (size_t)h * D * R;
        const size_t q0 = ((size_t)b * d->H + h) * D;
        /* p = q B^K  (1 x d_h times d_h x r) */
        for (int i = 0; i < R; ++i)
            for (int c = 0; c < D; ++c) pq[i] += elem(q, T, q0 + c) * elem(B_k, T, basis0 + (size_t)c * R + i);
        const double scale = 1.0 / sqrt((double)D);
        for (int j = 0; j < L; ++j) {
            double sh = 0.0, pr = 0.0;
            for (int c = 0; c < D; ++c) sh += elem(q, T, q0 + c) * elem(k_s, T, shared0 + (size_t)j * D + c);
            for (int i = 0; i < R; ++i) pr += pq[i] * elem(z_k, T, lat0 + (size_t)j * R + i);
            s[j] = (sh + pr) * scale;
        }
        softmax(s, L, a);
        /* o = a V_s + (a Z^V) (B^V)^T */
        for (int j = 0; j < L; ++j) {
            for (int c = 0; c < D; ++c) o[c] += a[j] * elem(v_s, T, shared0 + (size_t)j * D + c);
            for (int i = 0; i < R; ++i) u[i] += a[j] * elem(z_v, T, lat0 + (size_t)j * R + i);
        }
        for (int c = 0; c < D; ++c) {
            double acc = 0.0;
            for (int i = 0; i < R; ++i) acc += u[i] * elem(B_v, T, basis0 + (size_t)c * R + i);
            o[c] += acc;
        }
        free(s);
        free(a);
        free(pq);
        free(u);
    }
    return 0;
}
