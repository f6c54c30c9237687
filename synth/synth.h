/*
 * synth.h — seeded, counter-addressed synthetic inputs for the MoE expert-FFN
 * layer (expert weights, router, bias, tokens, RMSNorm gains).
 *
 * This module is input generation only. It holds none of the method's
 * arithmetic (no quantisation, no dot products, no routing): it turns a
 * (seed, stream, element index) triple into a float. Both the oracle side
 * and the GPU side draw their inputs from here; the GPU twin of the weight
 * generator (synth_dev.hip) implements the same published generator and must
 * agree with this file bit for bit.
 *
 * Generator: Philox4x32-10, as defined by Salmon, Moraes, Dror and Shaw,
 * "Parallel random numbers: as easy as 1, 2, 3" (SC'11): multipliers
 * 0xD2511F53 / 0xCD9E8D57, Weyl key increments 0x9E3779B9 / 0xBB67AE85,
 * ten rounds, key bumped before every round after the first.
 *
 * Normal deviates: one Philox block (4 x 32 bits) is cut into eight 16-bit
 * uniforms h_i; z = sum_i (2*h_i - 65535) is an exact even integer with
 * |z| <= 524280 and variance 8*(65536^2-1)/3 (Irwin-Hall with n = 8, tails
 * bounded at about 4.9 sigma). The value is (float)z * c with
 * c = (float)(sigma / (65536*sqrt(8/3))), a single correctly rounded f32
 * product, so host and device produce identical bits.
 */
#ifndef SYNTH_H
#define SYNTH_H
#include <stdint.h>
#include <stddef.h>
#ifdef __cplusplus
extern "C" {
#endif

/* Philox4x32-10: out[0..3] = bijection of ctr[0..3] under key[0..1]. */
void synth_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]);

/* f32 multiplier c that turns the integer Irwin-Hall sum into N(0, sigma). */
float synth_normal_scale(double sigma);

/* Stream identifiers. The top two bits give the kind. */
uint32_t synth_stream_expert(int layer, int expert, int matrix); /* matrix: 0 gate, 1 up, 2 down */
uint32_t synth_stream_layer(int layer, int what);                /* what: 0 router W, 1 bias, 2 gamma, 3 zipf ranks */
uint32_t synth_stream_tokens(int set, int what);                 /* what: 0 iid x, 1 common part, 2 channel pick */

/* The integer Irwin-Hall sum for element n of stream (seed, stream). */
int32_t synth_normal_int(uint32_t seed, uint32_t stream, uint64_t n);

/* Fill out[rows*cols] with N(0, sigma) draws, element (r, c) at index r*cols + c.
 * If outlier_rate > 0, row r is an outlier row when its Philox word 0 on
 * counter (r, 0, 1, 0) is below outlier_rate * 2^32 (floored); that row's
 * element at column (word1 * cols) >> 32 is multiplied by outlier_mult (f32).
 * Rows are independent: fill a row range with row0/nrows. Uses OpenMP. */
void synth_fill_matrix(uint32_t seed, uint32_t stream, int64_t row0, int64_t nrows, int64_t cols,
                       double sigma, double outlier_rate, float outlier_mult, float *out);

/* floor(outlier_rate * 2^32): the row-outlier threshold on Philox word 0 (0 = none). */
uint32_t synth_outlier_threshold(double outlier_rate);

/* Outlier decision for one row (same rule as above): returns the column, or -1. */
int64_t synth_outlier_col(uint32_t seed, uint32_t stream, int64_t row, int64_t cols, double outlier_rate);

/* Uniform double in [0, 1) from words (w0, w1) of counter (n, 0, 2, 0): 53 bits. */
double synth_uniform(uint32_t seed, uint32_t stream, uint64_t n);

/* Deterministic permutation of 0..n-1 (Fisher-Yates driven by synth_uniform). */
void synth_permutation(uint32_t seed, uint32_t stream, int n, int32_t *perm);

#ifdef __cplusplus
}
#endif
#endif
