/*
 * synth.c — host implementation of the seeded input generator (see synth.h).
 * Input generation only; no quantisation or other arithmetic of the method.
 */
#include "synth.h"
#include <math.h>

#define PHILOX_M0 0xD2511F53u
#define PHILOX_M1 0xCD9E8D57u
#define PHILOX_W0 0x9E3779B9u
#define PHILOX_W1 0xBB67AE85u

void synth_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4])
{
    uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
    uint32_t k0 = key[0], k1 = key[1];
    for (int round = 0; round < 10; ++round) {
        if (round > 0) { k0 += PHILOX_W0; k1 += PHILOX_W1; }
        uint64_t p0 = (uint64_t)PHILOX_M0 * c0;
        uint64_t p1 = (uint64_t)PHILOX_M1 * c2;
        uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
        uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
        uint32_t n0 = hi1 ^ c1 ^ k0;
        uint32_t n2 = hi0 ^ c3 ^ k1;
        c0 = n0; c1 = lo1; c2 = n2; c3 = lo0;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

float synth_normal_scale(double sigma)
{
    return (float)(sigma / (65536.0 * sqrt(8.0 / 3.0)));
}

uint32_t synth_stream_expert(int layer, int expert, int matrix)
{
    return (0u << 30) | ((uint32_t)(layer & 0x3FFF) << 16) | ((uint32_t)(expert & 0x3FFF) << 2)
         | (uint32_t)(matrix & 3);
}

uint32_t synth_stream_layer(int layer, int what)
{
    return (1u << 30) | ((uint32_t)(layer & 0xFFFFF) << 4) | (uint32_t)(what & 15);
}

uint32_t synth_stream_tokens(int set, int what)
{
    return (2u << 30) | ((uint32_t)(set & 0xFFFFF) << 4) | (uint32_t)(what & 15);
}

static inline int32_t irwin_hall8(const uint32_t w[4])
{
    int32_t z = 0;
    for (int i = 0; i < 4; ++i) {
        z += 2 * (int32_t)(w[i] & 0xFFFFu) - 65535;
        z += 2 * (int32_t)(w[i] >> 16) - 65535;
    }
    return z;
}

int32_t synth_normal_int(uint32_t seed, uint32_t stream, uint64_t n)
{
    uint32_t ctr[4] = {(uint32_t)n, (uint32_t)(n >> 32), 0u, 0u};
    uint32_t key[2] = {seed, stream};
    uint32_t w[4];
    synth_philox4x32_10(ctr, key, w);
    return irwin_hall8(w);
}

uint32_t synth_outlier_threshold(double outlier_rate)
{
    if (!(outlier_rate > 0.0)) return 0u;
    double t = floor(outlier_rate * 4294967296.0);
    return t >= 4294967295.0 ? 4294967295u : (uint32_t)t;
}

int64_t synth_outlier_col(uint32_t seed, uint32_t stream, int64_t row, int64_t cols, double outlier_rate)
{
    uint32_t thr = synth_outlier_threshold(outlier_rate);
    if (thr == 0u) return -1;
    uint32_t ctr[4] = {(uint32_t)row, (uint32_t)((uint64_t)row >> 32), 1u, 0u};
    uint32_t key[2] = {seed, stream};
    uint32_t w[4];
    synth_philox4x32_10(ctr, key, w);
    if (w[0] >= thr) return -1;
    return (int64_t)(((uint64_t)w[1] * (uint64_t)cols) >> 32);
}

void synth_fill_matrix(uint32_t seed, uint32_t stream, int64_t row0, int64_t nrows, int64_t cols,
                       double sigma, double outlier_rate, float outlier_mult, float *out)
{
    const float c = synth_normal_scale(sigma);
#pragma omp parallel for schedule(static)
    for (int64_t rr = 0; rr < nrows; ++rr) {
        const int64_t r = row0 + rr;
        float *dst = out + rr * cols;
        for (int64_t col = 0; col < cols; ++col) {
            int32_t z = synth_normal_int(seed, stream, (uint64_t)(r * cols + col));
            dst[col] = (float)z * c;
        }
        int64_t oc = synth_outlier_col(seed, stream, r, cols, outlier_rate);
        if (oc >= 0) dst[oc] = dst[oc] * outlier_mult;
    }
}

double synth_uniform(uint32_t seed, uint32_t stream, uint64_t n)
{
    uint32_t ctr[4] = {(uint32_t)n, (uint32_t)(n >> 32), 2u, 0u};
    uint32_t key[2] = {seed, stream};
    uint32_t w[4];
    synth_philox4x32_10(ctr, key, w);
    uint64_t bits = ((uint64_t)w[0] << 21) ^ (uint64_t)(w[1] >> 11);
    bits &= ((uint64_t)1 << 53) - 1;
    return (double)bits * (1.0 / 9007199254740992.0);
}

void synth_permutation(uint32_t seed, uint32_t stream, int n, int32_t *perm)
{
    for (int i = 0; i < n; ++i) perm[i] = i;
    for (int i = n - 1; i > 0; --i) {
        int j = (int)floor(synth_uniform(seed, stream, (uint64_t)i) * (double)(i + 1));
        if (j > i) j = i;
        int32_t t = perm[i]; perm[i] = perm[j]; perm[j] = t;
    }
}
