/*
 * oracle.h — plain, slow CPU reference of one MoE layer's
 * routed-expert FFN with int4 experts and Q8_0-style int8 activations.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load or call this library (either
 * build: liboracle.so, or liboracle_omp.so with the independent row loops
 * spread over OpenMP threads, bit for bit the same results). The GPU
 * library never calls it, includes it or shares code with it.
 *
 * Sources (the pages on the colibri engine):
 *   [P1 s3.1]  colibri architecture overview, section 3.1 "extreme quantisation":
 *              int4 packed = two 4-bit values per byte, one f32 scale per row;
 *              dequantise on use; the IDOT path quantises activations to int8
 *              and takes integer dot products (dot_i4i8).
 *   [P1 s4]    same page, section 4 layer figure: moe = sigmoid routing + expert
 *              compute + shared expert; kernel layer matmul_i4, dot_i4i8, rmsnorm.
 *   [P1 s5]    same page, section 5 token lifecycle: sigmoid route top-8,
 *              gate/up/SiLU/down expert matmuls on the IDOT path, shared expert.
 *   [P2 how]   README (zh-TW), "how it works": a batch reads each distinct expert
 *              once (batch union); placement never changes routing or precision.
 *   [P2 results] same README, "actual results": quality is measured, including
 *              the int4 container's cost and scale-granularity ablations.
 *   [P3 impl]  ai4coding.ru summary, "what is implemented": DeepSeek-V3-style
 *              sigmoid router, shared expert, Q8_0-style int8 activations.
 * Where the pages leave a step open, the reading taken is stated at the
 * function. Summations run in double, in index order.
 *
 * Parity pins (tests/test_oracle_*.py) tie every function here to something
 * other than itself: exact round trips, exactly representable special cases
 * that reduce to an integer matmul, brute force over all expert subsets,
 * closed forms and the statistical rounding-error law.
 */
#ifndef COLI_ORACLE_H
#define COLI_ORACLE_H
#include <stdint.h>
#ifdef __cplusplus
extern "C" {
#endif

/* O1 [P1 s3.1] int4 pack, per row: d = absmax/7 (f32), id = 1/d (0 if d == 0),
 * code = clamp(rint(w*id), -8, 7), w*id a single f32 product and rint
 * rounding half to even (an infinite product clamps; a NaN product, only
 * possible for w == 0 with id == inf, gives 0). Byte j of a row holds element 2j
 * in bits 0-3 and element 2j+1 in bits 4-7, as 4-bit two's complement.
 * q: [rows][cols/2], s: [rows]. cols must be even. */
void oracle_pack_int4_rows(const float *w, int rows, int cols, uint8_t *q, float *s);

/* O2 [P1 s3.1] decode one nibble: hi = 0 -> bits 0-3, hi = 1 -> bits 4-7. */
int oracle_nibble(uint8_t byte, int hi);

/* O2 [P1 s3.1] dequantise on use: w~[r][c] = s[r] * code[r][c] (double). */
void oracle_unpack_int4_rows(const uint8_t *q, const float *s, int rows, int cols, double *w);

/* O3 [P3 impl] Q8_0-style activation quantisation in 32-wide blocks:
 * d_b = absmax_b/127 (f32), id = 1/d_b (0 if d_b == 0),
 * code = clamp(rint(x*id), -127, 127) (same rounding and NaN rule as O1).
 * q: [n], d: [n/32]. n must be a multiple of 32. */
void oracle_quant_q8(const float *x, int n, int8_t *q, float *d);

/* O4 [P1 s3.1, dot_i4i8] exact int32 block dots S[r][b] = sum_{k in block b}
 * code4[r][k] * q8[k]. S: [rows][cols/32]. */
void oracle_block_dots(const uint8_t *q4, const int8_t *q8, int rows, int cols, int32_t *S);

/* O5 [P1 s3.1] IDOT row product: out[r] = (float)(s4[r] * sum_b d8[b]*S[r][b]),
 * the block sum taken in double in block order. */
void oracle_rowdot(const uint8_t *q4, const float *s4, const int8_t *q8, const float *d8,
                   int rows, int cols, float *out);

/* O16 [P1 s3.1 int4 format; P2 results: the quality measurements include
 * scale-granularity ablations] int4 with one scale per group of `group`
 * consecutive columns of a row instead of one per row. The pages name the
 * ablation but not the group format; the reading taken is O1 applied to
 * every group as if it were a row: d_g = absmax_g/7 (f32), the same codes,
 * rounding, clamp and nibble order. q: [rows][cols/2] as O1,
 * s: [rows][cols/group]. group must be even and divide cols. */
void oracle_pack_int4_groups(const float *w, int rows, int cols, int group, uint8_t *q, float *s);

/* O16 dequantise on use: w~[r][c] = s[r][c/group] * code[r][c] (double). */
void oracle_unpack_int4_groups(const uint8_t *q, const float *s, int rows, int cols, int group, double *w);

/* O17 [P1 s3.1, dot_i4i8 with O16 scales] IDOT row product with group scales
 * (group a multiple of 32, so a group is whole activation blocks):
 * out[r] = (float)(sum_b s[r][g(b)] * (d8[b] * S[r][b])), g(b) = 32b/group,
 * every term in double, summed in block order. With group = cols it is O5. */
void oracle_rowdot_groups(const uint8_t *q4, const float *s4, int group, const int8_t *q8, const float *d8,
                          int rows, int cols, float *out);

/* O18 [P1 s3.1: int2 packed, experimental, four 2-bit values per byte; the
 * kernel layer's matmul_i2] int2 pack, per row. The pages give no scale
 * rule; the reading taken is O1's with the 2-bit range: d = absmax/1 (the
 * largest positive code is 1, as 7 is for int4), id = 1/d (0 if d == 0),
 * code = clamp(rint(w*id), -2, 1) with O1's rounding and NaN rule, so the
 * codes in use are -1, 0, 1. Byte j of a row holds elements 4j..4j+3 in bits
 * 0-1, 2-3, 4-5, 6-7, as 2-bit two's complement. q: [rows][cols/4], s: [rows].
 * cols a multiple of 4. */
void oracle_pack_int2_rows(const float *w, int rows, int cols, uint8_t *q, float *s);

/* O18 decode one 2-bit field i (0..3) of a byte. */
int oracle_crumb(uint8_t byte, int i);

/* O18 dequantise on use: w~[r][c] = s[r] * code[r][c] (double). */
void oracle_unpack_int2_rows(const uint8_t *q, const float *s, int rows, int cols, double *w);

/* O19 [P1 s3.1, the IDOT path with int2 rows] exact int32 block dots
 * S[r][b] = sum_{k in block b} code2[r][k] * q8[k]. */
void oracle_block_dots_i2(const uint8_t *q2, const int8_t *q8, int rows, int cols, int32_t *S);

/* O19 row product: out[r] = (float)(s2[r] * sum_b d8[b]*S[r][b]), the block
 * sum in double in block order (O5 with O19's block dots). */
void oracle_rowdot_i2(const uint8_t *q2, const float *s2, const int8_t *q8, const float *d8,
                      int rows, int cols, float *out);

/* O11 [P1 s3.1, quantize_rows] int8 weights, one byte per value. The pages
 * give no scale rule for them; the reading taken is the symmetric one of
 * the Q8 activations, per row: d = absmax/127 (f32), id = 1/d (0 if d == 0),
 * code = clamp(rint(w*id), -127, 127), same rounding and NaN rule as O1.
 * Natural element order. q: [rows][cols], s: [rows]. */
void oracle_pack_int8_rows(const float *w, int rows, int cols, int8_t *q, float *s);

/* O12 [P1 s3.1, dot_i8i8] exact int32 block dots of int8 weight rows with
 * Q8 activations: S[r][b] = sum_{k in block b} qw[r][k] * q8[k]. */
void oracle_block_dots_i8(const int8_t *qw, const int8_t *q8, int rows, int cols, int32_t *S);

/* O13 [P1 s3.1] IDOT row product of int8 rows: out[r] = (float)(sw[r] * sum_b d8[b]*S[r][b]),
 * the block sum in double in block order (O5 with O12's block dots). */
void oracle_rowdot_i8(const int8_t *qw, const float *sw, const int8_t *q8, const float *d8,
                      int rows, int cols, float *out);

/* O6 [P3 impl, P1 s5] DeepSeek-V3-style sigmoid router for T tokens:
 * z = W x (double), s = 1/(1+exp(-z)), key = s + b (bias used for selection
 * only). With n_group > 1, E is split into n_group equal groups, a group's
 * score is the sum of its two largest keys, the topk_group best groups are
 * kept and experts of the others are not eligible. The top_k eligible keys
 * are taken, largest first, equal keys to the lower expert index. Weights:
 * w_j = route_scale * s_{e_j} / sum_j s_{e_j} (double, then f32).
 * W: [E][H], b: [E], x: [T][H]; idx, w: [T][top_k]; keys (optional): [T][E]. */
int oracle_route(const float *W, const float *b, const float *x, int T, int H, int E, int top_k,
                 int n_group, int topk_group, float route_scale, int32_t *idx, float *w,
                 double *keys);

/* O7 [P1 s5] one expert on one token, IDOT path: g = O5(gate, Q8(x)),
 * u = O5(up, Q8(x)), h = (float)(silu(g)*u) with silu(g) = g/(1+exp(-g)) in
 * double, hq = O3(h), y = O5(down, hq). xq/xs are the token's Q8(x).
 * gate/up: [I][H/2] + [I] scales; down: [H][I/2] + [H] scales.
 * g, u, h, hq, hs may be NULL; otherwise g,u,h: [I], hq: [I], hs: [I/32]. */
void oracle_expert(const uint8_t *gate_q, const float *gate_s, const uint8_t *up_q, const float *up_s,
                   const uint8_t *down_q, const float *down_s, int H, int I,
                   const int8_t *xq, const float *xs, float *y,
                   float *g, float *u, float *h, int8_t *hq, float *hs);

/* O7 for any weight format: wbits = 4 (O5 row products on int4 rows), 8
 * (O13 on int8 rows: gate/up [I][H] int8, down [H][I] int8) or 2 (O19 on
 * int2 rows: gate/up [I][H/4], down [H][I/4]). */
void oracle_expert_w(int wbits, const void *gate_q, const float *gate_s, const void *up_q, const float *up_s,
                     const void *down_q, const float *down_s, int H, int I,
                     const int8_t *xq, const float *xs, float *y,
                     float *g, float *u, float *h, int8_t *hq, float *hs);

/* O7 with O16 weights: every row product is O17 with the given group.
 * gate/up scales [I][H/group], down scales [H][I/group]. */
void oracle_expert_groups(int group, const uint8_t *gate_q, const float *gate_s, const uint8_t *up_q,
                          const float *up_s, const uint8_t *down_q, const float *down_s, int H, int I,
                          const int8_t *xq, const float *xs, float *y,
                          float *g_out, float *u_out, float *h_out, int8_t *hq_out, float *hs_out);

/* O7 for n tokens of one expert: token t is oracle_expert_w (wbits, or
 * oracle_expert_groups when group > 0) on row t of xq [n][H] / xs [n][H/32],
 * its outputs in row t of y [n][H], g/u/h [n][I], hq [n][I], hs [n][I/32]
 * (g..hs may be NULL). The OpenMP build takes the tokens in parallel. */
void oracle_expert_tokens(int wbits, int group, const void *gate_q, const float *gate_s, const void *up_q,
                          const float *up_s, const void *down_q, const float *down_s, int H, int I, int n,
                          const int8_t *xq, const float *xs, float *y,
                          float *g, float *u, float *h, int8_t *hq, float *hs);

/* O8 [P1 s5, P3 impl] combine for one token: y = (float)(sum_j w_j*y_j + y_shared),
 * summed in double in j order, the shared expert (weight 1) last; y_shared may
 * be NULL (no shared expert). y_routed: [k][H]. */
void oracle_combine(const float *y_routed, const float *w, int k, const float *y_shared, int H,
                    float *y);

/* O9 [P1 s4, rmsnorm] out = (float)(x * gamma / sqrt(mean(x^2) + eps)) per token,
 * mean in double. */
void oracle_rmsnorm(const float *x, const float *gamma, int T, int H, float eps, float *out);

/* O10 [P1 s3.1] fp reference without activation quantisation: dequantised
 * weights (double), unquantised x and h, all in double. Measures the IDOT
 * error; not a parity target. y: [H] double. */
void oracle_expert_dense(const uint8_t *gate_q, const float *gate_s, const uint8_t *up_q,
                         const float *up_s, const uint8_t *down_q, const float *down_s, int H, int I,
                         const float *x, double *y);

/* O14 [P1 s3.1] O10 for int8 weight rows (dequantised in double). */
void oracle_expert_dense_i8(const int8_t *gate_q, const float *gate_s, const int8_t *up_q,
                            const float *up_s, const int8_t *down_q, const float *down_s, int H, int I,
                            const float *x, double *y);

/* Threads the row loops use: the OpenMP build's thread count, 1 in the
 * plain build. */
int oracle_threads(void);

/* A whole layer, every expert in host memory. Expert e's matrices start at
 * gate_q + e*I*H/2 (int4) or gate_q + e*I*H (int8), etc.; the shared expert
 * is index E when has_shared. */
typedef struct oracle_layer {
    int H, I, E, top_k, n_group, topk_group, has_shared;
    float route_scale;
    const float *router_w, *router_b;
    const uint8_t *gate_q, *up_q, *down_q;   /* int8 rows when weight_bits == 8, int2 when 2 */
    const float *gate_s, *up_s, *down_s;
    int weight_bits;                         /* 4 (or 0), 8 or 2 */
    int group_size;                          /* 0: one scale per row; else int4 with O16 group scales,
                                                gate_s/up_s [E'][I][H/G], down_s [E'][H][I/G] */
} oracle_layer;

/* O6 -> O3 -> O7 per selected expert (+ shared) -> O8, for T tokens.
 * idx/w (optional) receive the routing. Returns 0, or -1 on bad arguments. */
int oracle_moe_forward(const oracle_layer *L, const float *x, int T, float *y, int32_t *idx, float *w);

#ifdef __cplusplus
}
#endif
#endif
