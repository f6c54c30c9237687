/*
 * oracle.c — the plain CPU reference (see oracle.h for the sources and the
 * readings). TEST INFRASTRUCTURE ONLY: loaded by the tests, the smoke check
 * and the benchmark's CPU-baseline leg; never by the GPU library.
 *
 * Style: straight loops in the order the method states its steps, double
 * for every sum, no blocking, no fusion, no vector intrinsics. Compiled -O2
 * without -ffast-math and without FMA contraction.
 */
#include "oracle.h"
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int oracle_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Shared rounding rule of both quantisers: round half to even, clamp to
 * [lo, hi]; a NaN product (0 * inf) gives 0. */
static int round_clamp(float v, float lo, float hi)
{
    if (isnan(v)) return 0;
    float r = rintf(v);
    if (r < lo) r = lo;
    if (r > hi) r = hi;
    return (int)r;
}

/* ------------------------------------------------------------ O1 / O2 ---- */
void oracle_pack_int4_rows(const float *w, int rows, int cols, uint8_t *q, float *s)
{
#pragma omp parallel for schedule(static)
    for (int r = 0; r < rows; ++r) {
        const float *row = w + (size_t)r * cols;
        float amax = 0.0f;
        for (int c = 0; c < cols; ++c) {
            float a = fabsf(row[c]);
            if (a > amax) amax = a;
        }
        float d = amax / 7.0f;
        float id = (d != 0.0f) ? 1.0f / d : 0.0f;
        s[r] = d;
        uint8_t *dst = q + (size_t)r * (cols / 2);
        for (int j = 0; j < cols / 2; ++j) {
            int lo = round_clamp(row[2 * j] * id, -8.0f, 7.0f);
            int hi = round_clamp(row[2 * j + 1] * id, -8.0f, 7.0f);
            dst[j] = (uint8_t)((lo & 0xF) | ((hi & 0xF) << 4));
        }
    }
}

int oracle_nibble(uint8_t byte, int hi)
{
    int v = hi ? (byte >> 4) & 0xF : byte & 0xF;
    return v >= 8 ? v - 16 : v;   /* 4-bit two's complement */
}

void oracle_unpack_int4_rows(const uint8_t *q, const float *s, int rows, int cols, double *w)
{
    for (int r = 0; r < rows; ++r) {
        for (int c = 0; c < cols; ++c) {
            uint8_t byte = q[(size_t)r * (cols / 2) + c / 2];
            w[(size_t)r * cols + c] = (double)s[r] * (double)oracle_nibble(byte, c & 1);
        }
    }
}

/* ------------------------------------------------------------------ O3 --- */
void oracle_quant_q8(const float *x, int n, int8_t *q, float *d)
{
    for (int b = 0; b < n / 32; ++b) {
        const float *blk = x + 32 * b;
        float amax = 0.0f;
        for (int k = 0; k < 32; ++k) {
            float a = fabsf(blk[k]);
            if (a > amax) amax = a;
        }
        float db = amax / 127.0f;
        float id = (db != 0.0f) ? 1.0f / db : 0.0f;
        d[b] = db;
        for (int k = 0; k < 32; ++k)
            q[32 * b + k] = (int8_t)round_clamp(blk[k] * id, -127.0f, 127.0f);
    }
}

/* ------------------------------------------------------------- O4 / O5 --- */
/* S_b of one packed row: the exact int32 dot of block b's 32 int4 codes with
 * the 32 Q8 codes of the same block. */
static int32_t block_dot_i4(const uint8_t *row, const int8_t *q8, int b)
{
    int32_t acc = 0;
    for (int k = 32 * b; k < 32 * b + 32; ++k)
        acc += oracle_nibble(row[k / 2], k & 1) * (int32_t)q8[k];
    return acc;
}

void oracle_block_dots(const uint8_t *q4, const int8_t *q8, int rows, int cols, int32_t *S)
{
    for (int r = 0; r < rows; ++r) {
        const uint8_t *row = q4 + (size_t)r * (cols / 2);
        for (int b = 0; b < cols / 32; ++b)
            S[(size_t)r * (cols / 32) + b] = block_dot_i4(row, q8, b);
    }
}

void oracle_rowdot(const uint8_t *q4, const float *s4, const int8_t *q8, const float *d8,
                   int rows, int cols, float *out)
{
    const int nb = cols / 32;
#pragma omp parallel for schedule(static)
    for (int r = 0; r < rows; ++r) {
        const uint8_t *row = q4 + (size_t)r * (cols / 2);
        double acc = 0.0;
        for (int b = 0; b < nb; ++b) acc += (double)d8[b] * (double)block_dot_i4(row, q8, b);
        out[r] = (float)((double)s4[r] * acc);
    }
}

/* ----------------------------------------------------------- O16 / O17 --- */
void oracle_pack_int4_groups(const float *w, int rows, int cols, int group, uint8_t *q, float *s)
{
    const int ng = cols / group;
#pragma omp parallel for schedule(static)
    for (int r = 0; r < rows; ++r) {
        const float *row = w + (size_t)r * cols;
        uint8_t *dst = q + (size_t)r * (cols / 2);
        for (int g = 0; g < ng; ++g) {
            const float *grp = row + (size_t)g * group;
            float amax = 0.0f;
            for (int c = 0; c < group; ++c) {
                float a = fabsf(grp[c]);
                if (a > amax) amax = a;
            }
            float d = amax / 7.0f;
            float id = (d != 0.0f) ? 1.0f / d : 0.0f;
            s[(size_t)r * ng + g] = d;
            for (int j = 0; j < group / 2; ++j) {
                int lo = round_clamp(grp[2 * j] * id, -8.0f, 7.0f);
                int hi = round_clamp(grp[2 * j + 1] * id, -8.0f, 7.0f);
                dst[(size_t)g * (group / 2) + j] = (uint8_t)((lo & 0xF) | ((hi & 0xF) << 4));
            }
        }
    }
}

void oracle_unpack_int4_groups(const uint8_t *q, const float *s, int rows, int cols, int group, double *w)
{
    const int ng = cols / group;
    for (int r = 0; r < rows; ++r) {
        for (int c = 0; c < cols; ++c) {
            uint8_t byte = q[(size_t)r * (cols / 2) + c / 2];
            w[(size_t)r * cols + c] = (double)s[(size_t)r * ng + c / group] * (double)oracle_nibble(byte, c & 1);
        }
    }
}

void oracle_rowdot_groups(const uint8_t *q4, const float *s4, int group, const int8_t *q8, const float *d8,
                          int rows, int cols, float *out)
{
    const int nb = cols / 32, ng = cols / group;
#pragma omp parallel for schedule(static)
    for (int r = 0; r < rows; ++r) {
        const uint8_t *row = q4 + (size_t)r * (cols / 2);
        double acc = 0.0;
        for (int b = 0; b < nb; ++b) {
            double sg = (double)s4[(size_t)r * ng + (32 * b) / group];
            acc += sg * ((double)d8[b] * (double)block_dot_i4(row, q8, b));
        }
        out[r] = (float)acc;
    }
}

/* ----------------------------------------------------------- O18 / O19 --- */
void oracle_pack_int2_rows(const float *w, int rows, int cols, uint8_t *q, float *s)
{
#pragma omp parallel for schedule(static)
    for (int r = 0; r < rows; ++r) {
        const float *row = w + (size_t)r * cols;
        float amax = 0.0f;
        for (int c = 0; c < cols; ++c) {
            float a = fabsf(row[c]);
            if (a > amax) amax = a;
        }
        float d = amax / 1.0f;
        float id = (d != 0.0f) ? 1.0f / d : 0.0f;
        s[r] = d;
        uint8_t *dst = q + (size_t)r * (cols / 4);
        for (int j = 0; j < cols / 4; ++j) {
            int byte = 0;
            for (int i = 0; i < 4; ++i)
                byte |= (round_clamp(row[4 * j + i] * id, -2.0f, 1.0f) & 0x3) << (2 * i);
            dst[j] = (uint8_t)byte;
        }
    }
}

int oracle_crumb(uint8_t byte, int i)
{
    int v = (byte >> (2 * i)) & 0x3;
    return v >= 2 ? v - 4 : v;    /* 2-bit two's complement */
}

void oracle_unpack_int2_rows(const uint8_t *q, const float *s, int rows, int cols, double *w)
{
    for (int r = 0; r < rows; ++r)
        for (int c = 0; c < cols; ++c)
            w[(size_t)r * cols + c] = (double)s[r] * (double)oracle_crumb(q[(size_t)r * (cols / 4) + c / 4], c & 3);
}

/* S_b of one int2 row: the exact int32 dot of block b's 32 two-bit codes with
 * the block's 32 Q8 codes. */
static int32_t block_dot_i2(const uint8_t *row, const int8_t *q8, int b)
{
    int32_t acc = 0;
    for (int k = 32 * b; k < 32 * b + 32; ++k)
        acc += oracle_crumb(row[k / 4], k & 3) * (int32_t)q8[k];
    return acc;
}

void oracle_block_dots_i2(const uint8_t *q2, const int8_t *q8, int rows, int cols, int32_t *S)
{
    for (int r = 0; r < rows; ++r) {
        const uint8_t *row = q2 + (size_t)r * (cols / 4);
        for (int b = 0; b < cols / 32; ++b)
            S[(size_t)r * (cols / 32) + b] = block_dot_i2(row, q8, b);
    }
}

void oracle_rowdot_i2(const uint8_t *q2, const float *s2, const int8_t *q8, const float *d8,
                      int rows, int cols, float *out)
{
    const int nb = cols / 32;
#pragma omp parallel for schedule(static)
    for (int r = 0; r < rows; ++r) {
        const uint8_t *row = q2 + (size_t)r * (cols / 4);
        double acc = 0.0;
        for (int b = 0; b < nb; ++b) acc += (double)d8[b] * (double)block_dot_i2(row, q8, b);
        out[r] = (float)((double)s2[r] * acc);
    }
}

/* ----------------------------------------------------------- O11 - O13 --- */
void oracle_pack_int8_rows(const float *w, int rows, int cols, int8_t *q, float *s)
{
#pragma omp parallel for schedule(static)
    for (int r = 0; r < rows; ++r) {
        const float *row = w + (size_t)r * cols;
        float amax = 0.0f;
        for (int c = 0; c < cols; ++c) {
            float a = fabsf(row[c]);
            if (a > amax) amax = a;
        }
        float d = amax / 127.0f;
        float id = (d != 0.0f) ? 1.0f / d : 0.0f;
        s[r] = d;
        for (int c = 0; c < cols; ++c)
            q[(size_t)r * cols + c] = (int8_t)round_clamp(row[c] * id, -127.0f, 127.0f);
    }
}

/* S_b of one int8 row: the exact int32 dot of block b's 32 weight codes with
 * the block's 32 Q8 codes. */
static int32_t block_dot_i8(const int8_t *row, const int8_t *q8, int b)
{
    int32_t acc = 0;
    for (int k = 32 * b; k < 32 * b + 32; ++k) acc += (int32_t)row[k] * (int32_t)q8[k];
    return acc;
}

void oracle_block_dots_i8(const int8_t *qw, const int8_t *q8, int rows, int cols, int32_t *S)
{
    for (int r = 0; r < rows; ++r) {
        const int8_t *row = qw + (size_t)r * cols;
        for (int b = 0; b < cols / 32; ++b) S[(size_t)r * (cols / 32) + b] = block_dot_i8(row, q8, b);
    }
}

void oracle_rowdot_i8(const int8_t *qw, const float *sw, const int8_t *q8, const float *d8,
                      int rows, int cols, float *out)
{
    const int nb = cols / 32;
#pragma omp parallel for schedule(static)
    for (int r = 0; r < rows; ++r) {
        const int8_t *row = qw + (size_t)r * cols;
        double acc = 0.0;
        for (int b = 0; b < nb; ++b) acc += (double)d8[b] * (double)block_dot_i8(row, q8, b);
        out[r] = (float)((double)sw[r] * acc);
    }
}

/* ------------------------------------------------------------------ O6 --- */
int oracle_route(const float *W, const float *b, const float *x, int T, int H, int E, int top_k,
                 int n_group, int topk_group, float route_scale, int32_t *idx, float *w,
                 double *keys)
{
    if (T < 0 || H <= 0 || E <= 0 || top_k < 1 || top_k > E) return -1;
    if (n_group < 1 || E % n_group != 0 || topk_group < 1 || topk_group > n_group) return -1;
    const int gsize = E / n_group;
    if (n_group > 1 && top_k > topk_group * gsize) return -1;
    double *s = (double *)malloc(sizeof(double) * (size_t)E);
    double *key = (double *)malloc(sizeof(double) * (size_t)E);
    int *eligible = (int *)malloc(sizeof(int) * (size_t)E);
    int *taken = (int *)malloc(sizeof(int) * (size_t)(E > n_group ? E : n_group));
    double *gscore = (double *)malloc(sizeof(double) * (size_t)n_group);

    for (int t = 0; t < T; ++t) {
        const float *xt = x + (size_t)t * H;
        for (int e = 0; e < E; ++e) {
            double z = 0.0;
            for (int h = 0; h < H; ++h) z += (double)W[(size_t)e * H + h] * (double)xt[h];
            s[e] = 1.0 / (1.0 + exp(-z));
            key[e] = s[e] + (double)b[e];
            if (keys) keys[(size_t)t * E + e] = key[e];
            eligible[e] = 1;
        }
        if (n_group > 1) {
            for (int g = 0; g < n_group; ++g) {
                /* sum of the two largest keys of the group */
                double m1 = -INFINITY, m2 = -INFINITY;
                for (int e = g * gsize; e < (g + 1) * gsize; ++e) {
                    if (key[e] > m1) { m2 = m1; m1 = key[e]; }
                    else if (key[e] > m2) { m2 = key[e]; }
                }
                gscore[g] = gsize >= 2 ? m1 + m2 : m1;
                taken[g] = 0;
            }
            for (int pick = 0; pick < topk_group; ++pick) {
                int best = -1;
                for (int g = 0; g < n_group; ++g)
                    if (!taken[g] && (best < 0 || gscore[g] > gscore[best])) best = g;
                taken[best] = 1;
            }
            for (int e = 0; e < E; ++e) eligible[e] = taken[e / gsize];
        }
        for (int e = 0; e < E; ++e) taken[e] = 0;
        double ssum = 0.0;
        int32_t *it = idx + (size_t)t * top_k;
        for (int j = 0; j < top_k; ++j) {
            int best = -1;
            for (int e = 0; e < E; ++e)
                if (eligible[e] && !taken[e] && (best < 0 || key[e] > key[best])) best = e;
            taken[best] = 1;
            it[j] = best;
            ssum += s[best];
        }
        for (int j = 0; j < top_k; ++j)
            w[(size_t)t * top_k + j] = (float)((double)route_scale * s[it[j]] / ssum);
    }
    free(s); free(key); free(eligible); free(taken); free(gscore);
    return 0;
}

/* ------------------------------------------------------------------ O7 --- */
/* The IDOT row product of either weight format (O5 for 4 bits, O13 for 8). */
/* group > 0: int4 rows with one scale per group of that many columns (O17). */
static void rowdot_w(int wbits, int group, const void *q, const float *s, const int8_t *q8, const float *d8,
                     int rows, int cols, float *out)
{
    if (wbits == 8) oracle_rowdot_i8((const int8_t *)q, s, q8, d8, rows, cols, out);
    else if (wbits == 2) oracle_rowdot_i2((const uint8_t *)q, s, q8, d8, rows, cols, out);
    else if (group > 0) oracle_rowdot_groups((const uint8_t *)q, s, group, q8, d8, rows, cols, out);
    else oracle_rowdot((const uint8_t *)q, s, q8, d8, rows, cols, out);
}

static void expert_impl(int wbits, int group, const void *gate_q, const float *gate_s, const void *up_q,
                        const float *up_s, const void *down_q, const float *down_s, int H, int I,
                        const int8_t *xq, const float *xs, float *y,
                        float *g_out, float *u_out, float *h_out, int8_t *hq_out, float *hs_out)
{
    float *g = (float *)malloc(sizeof(float) * (size_t)I);
    float *u = (float *)malloc(sizeof(float) * (size_t)I);
    float *h = (float *)malloc(sizeof(float) * (size_t)I);
    int8_t *hq = (int8_t *)malloc((size_t)I);
    float *hs = (float *)malloc(sizeof(float) * (size_t)(I / 32));

    rowdot_w(wbits, group, gate_q, gate_s, xq, xs, I, H, g);
    rowdot_w(wbits, group, up_q, up_s, xq, xs, I, H, u);
    for (int i = 0; i < I; ++i) {
        double gd = (double)g[i];
        double silu = gd / (1.0 + exp(-gd));
        h[i] = (float)(silu * (double)u[i]);
    }
    oracle_quant_q8(h, I, hq, hs);
    rowdot_w(wbits, group, down_q, down_s, hq, hs, H, I, y);

    if (g_out) memcpy(g_out, g, sizeof(float) * (size_t)I);
    if (u_out) memcpy(u_out, u, sizeof(float) * (size_t)I);
    if (h_out) memcpy(h_out, h, sizeof(float) * (size_t)I);
    if (hq_out) memcpy(hq_out, hq, (size_t)I);
    if (hs_out) memcpy(hs_out, hs, sizeof(float) * (size_t)(I / 32));
    free(g); free(u); free(h); free(hq); free(hs);
}

void oracle_expert_w(int wbits, const void *gate_q, const float *gate_s, const void *up_q, const float *up_s,
                     const void *down_q, const float *down_s, int H, int I,
                     const int8_t *xq, const float *xs, float *y,
                     float *g_out, float *u_out, float *h_out, int8_t *hq_out, float *hs_out)
{
    expert_impl(wbits, 0, gate_q, gate_s, up_q, up_s, down_q, down_s, H, I, xq, xs, y, g_out, u_out, h_out,
                hq_out, hs_out);
}

void oracle_expert_groups(int group, const uint8_t *gate_q, const float *gate_s, const uint8_t *up_q,
                          const float *up_s, const uint8_t *down_q, const float *down_s, int H, int I,
                          const int8_t *xq, const float *xs, float *y,
                          float *g_out, float *u_out, float *h_out, int8_t *hq_out, float *hs_out)
{
    expert_impl(4, group, gate_q, gate_s, up_q, up_s, down_q, down_s, H, I, xq, xs, y, g_out, u_out, h_out,
                hq_out, hs_out);
}

void oracle_expert(const uint8_t *gate_q, const float *gate_s, const uint8_t *up_q, const float *up_s,
                   const uint8_t *down_q, const float *down_s, int H, int I,
                   const int8_t *xq, const float *xs, float *y,
                   float *g_out, float *u_out, float *h_out, int8_t *hq_out, float *hs_out)
{
    oracle_expert_w(4, gate_q, gate_s, up_q, up_s, down_q, down_s, H, I, xq, xs, y,
                    g_out, u_out, h_out, hq_out, hs_out);
}

/* O7 for n tokens of one expert (the rows of xq/xs and of every output are
 * the tokens): each token is oracle_expert_w on its own row; the OpenMP
 * build spreads the tokens over threads. Outputs as oracle_expert_w, one row
 * per token (y [n][H]; g, u, h [n][I]; hq [n][I]; hs [n][I/32]; any may be
 * NULL except y). group > 0: int4 rows with O16 group scales (as
 * oracle_expert_groups). */
void oracle_expert_tokens(int wbits, int group, const void *gate_q, const float *gate_s, const void *up_q,
                          const float *up_s, const void *down_q, const float *down_s, int H, int I, int n,
                          const int8_t *xq, const float *xs, float *y,
                          float *g_out, float *u_out, float *h_out, int8_t *hq_out, float *hs_out)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int t = 0; t < n; ++t) {
        const size_t ti = (size_t)t * I;
        expert_impl(wbits, group, gate_q, gate_s, up_q, up_s, down_q, down_s, H, I, xq + (size_t)t * H,
                    xs + (size_t)t * (H / 32), y + (size_t)t * H, g_out ? g_out + ti : NULL,
                    u_out ? u_out + ti : NULL, h_out ? h_out + ti : NULL, hq_out ? hq_out + ti : NULL,
                    hs_out ? hs_out + (size_t)t * (I / 32) : NULL);
    }
}

/* ------------------------------------------------------------------ O8 --- */
void oracle_combine(const float *y_routed, const float *w, int k, const float *y_shared, int H,
                    float *y)
{
    for (int r = 0; r < H; ++r) {
        double acc = 0.0;
        for (int j = 0; j < k; ++j) acc += (double)w[j] * (double)y_routed[(size_t)j * H + r];
        if (y_shared) acc += (double)y_shared[r];
        y[r] = (float)acc;
    }
}

/* ------------------------------------------------------------------ O9 --- */
void oracle_rmsnorm(const float *x, const float *gamma, int T, int H, float eps, float *out)
{
    for (int t = 0; t < T; ++t) {
        const float *xt = x + (size_t)t * H;
        double ss = 0.0;
        for (int i = 0; i < H; ++i) ss += (double)xt[i] * (double)xt[i];
        double r = 1.0 / sqrt(ss / (double)H + (double)eps);
        for (int i = 0; i < H; ++i)
            out[(size_t)t * H + i] = (float)((double)xt[i] * r * (double)gamma[i]);
    }
}

/* ----------------------------------------------------------------- O10 --- */
void oracle_expert_dense(const uint8_t *gate_q, const float *gate_s, const uint8_t *up_q,
                         const float *up_s, const uint8_t *down_q, const float *down_s, int H, int I,
                         const float *x, double *y)
{
    double *h = (double *)malloc(sizeof(double) * (size_t)I);
    for (int i = 0; i < I; ++i) {
        double g = 0.0, u = 0.0;
        for (int c = 0; c < H; ++c) {
            size_t byte = (size_t)i * (H / 2) + c / 2;
            g += (double)gate_s[i] * oracle_nibble(gate_q[byte], c & 1) * (double)x[c];
            u += (double)up_s[i] * oracle_nibble(up_q[byte], c & 1) * (double)x[c];
        }
        h[i] = g / (1.0 + exp(-g)) * u;
    }
    for (int r = 0; r < H; ++r) {
        double acc = 0.0;
        for (int i = 0; i < I; ++i) {
            size_t byte = (size_t)r * (I / 2) + i / 2;
            acc += (double)down_s[r] * oracle_nibble(down_q[byte], i & 1) * h[i];
        }
        y[r] = acc;
    }
    free(h);
}

/* ----------------------------------------------------------------- O14 --- */
void oracle_expert_dense_i8(const int8_t *gate_q, const float *gate_s, const int8_t *up_q,
                            const float *up_s, const int8_t *down_q, const float *down_s, int H, int I,
                            const float *x, double *y)
{
    double *h = (double *)malloc(sizeof(double) * (size_t)I);
    for (int i = 0; i < I; ++i) {
        double g = 0.0, u = 0.0;
        for (int c = 0; c < H; ++c) {
            g += (double)gate_s[i] * (double)gate_q[(size_t)i * H + c] * (double)x[c];
            u += (double)up_s[i] * (double)up_q[(size_t)i * H + c] * (double)x[c];
        }
        h[i] = g / (1.0 + exp(-g)) * u;
    }
    for (int r = 0; r < H; ++r) {
        double acc = 0.0;
        for (int i = 0; i < I; ++i) acc += (double)down_s[r] * (double)down_q[(size_t)r * I + i] * h[i];
        y[r] = acc;
    }
    free(h);
}

/* --------------------------------------------------------- whole layer --- */
int oracle_moe_forward(const oracle_layer *L, const float *x, int T, float *y, int32_t *idx_out,
                       float *w_out)
{
    const int H = L->H, I = L->I, E = L->E, k = L->top_k;
    if (H <= 0 || I <= 0 || H % 32 || I % 32 || T < 0) return -1;
    if (L->weight_bits != 0 && L->weight_bits != 2 && L->weight_bits != 4 && L->weight_bits != 8) return -1;
    const int G = L->group_size;
    if (G < 0 || (G > 0 && (L->weight_bits == 8 || L->weight_bits == 2 || G % 32 || H % G || I % G))) return -1;
    int32_t *idx = (int32_t *)malloc(sizeof(int32_t) * (size_t)(T * k + 1));
    float *w = (float *)malloc(sizeof(float) * (size_t)(T * k + 1));
    if (oracle_route(L->router_w, L->router_b, x, T, H, E, k, L->n_group, L->topk_group,
                     L->route_scale, idx, w, NULL) != 0) {
        free(idx); free(w);
        return -1;
    }
    int8_t *xq = (int8_t *)malloc((size_t)H);
    float *xs = (float *)malloc(sizeof(float) * (size_t)(H / 32));
    float *yr = (float *)malloc(sizeof(float) * (size_t)k * H);
    float *ysh = (float *)malloc(sizeof(float) * (size_t)H);
    const int wb = L->weight_bits == 0 ? 4 : L->weight_bits;
    /* bytes per expert matrix: a byte holds one 8-bit, two 4-bit or four 2-bit codes */
    const size_t gq = (size_t)I * H * wb / 8;
    const size_t dq = (size_t)H * I * wb / 8;
    /* scales per expert matrix: one per row, or one per group of G columns */
    const size_t gs = G > 0 ? (size_t)I * (H / G) : (size_t)I;
    const size_t ds = G > 0 ? (size_t)H * (I / G) : (size_t)H;
    for (int t = 0; t < T; ++t) {
        oracle_quant_q8(x + (size_t)t * H, H, xq, xs);
        for (int j = 0; j < k; ++j) {
            int e = idx[t * k + j];
            expert_impl(wb, G, L->gate_q + e * gq, L->gate_s + e * gs, L->up_q + e * gq, L->up_s + e * gs,
                        L->down_q + e * dq, L->down_s + e * ds, H, I, xq, xs, yr + (size_t)j * H,
                        NULL, NULL, NULL, NULL, NULL);
        }
        if (L->has_shared) {
            int e = E;
            expert_impl(wb, G, L->gate_q + e * gq, L->gate_s + e * gs, L->up_q + e * gq, L->up_s + e * gs,
                        L->down_q + e * dq, L->down_s + e * ds, H, I, xq, xs, ysh, NULL, NULL, NULL, NULL, NULL);
        }
        oracle_combine(yr, w + (size_t)t * k, k, L->has_shared ? ysh : NULL, H, y + (size_t)t * H);
    }
    if (idx_out) memcpy(idx_out, idx, sizeof(int32_t) * (size_t)T * k);
    if (w_out) memcpy(w_out, w, sizeof(float) * (size_t)T * k);
    free(idx); free(w); free(xq); free(xs); free(yr); free(ysh);
    return 0;
}
