/*
 * oracle.h -- plain CPU oracle for the tiled-matmul hot path.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg may load this library. The product library never links,
 * includes or calls it, and it includes nothing from the product.
 *
 * Every routine is the plain definition: one double accumulator per output,
 * summed in ascending contraction order, rounded once to fp32 (the softmax
 * keeps double outputs).
 *
 * Element codes (dtype): 0 = fp32, 1 = bfloat16 (raw 16-bit patterns),
 * 2 = IEEE binary16 (raw 16-bit patterns). Outputs are always fp32.
 * Return value: 0 on success, -1 on a rejected argument.
 */
#ifndef CAS_ORACLE_H
#define CAS_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

int oracle_num_threads(void);
void oracle_set_threads(int n);

/* Decode n elements of the given dtype to double (exact for all three). */
int oracle_decode(const void *src, int dtype, int64_t n, double *dst);

/* Y[m*ldy+n] = sum_k X[m*ldx+k] * W[n*ldw+k];  bound (nullable) gets
 * sum_k |X*W|, the error scale used by the tolerance. */
int oracle_gemm_nt(const void *X, const void *W, float *Y, double *bound,
                   int64_t M, int64_t N, int64_t K,
                   int64_t ldx, int64_t ldw, int64_t ldy, int dtype);

/* qkv is (B,T,3,NH,HS), C = NH*HS; out is (B,NH,T,T).
 * out = scale * Q.K for t2 <= t, quiet NaN 0x7FC00000 for t2 > t. */
int oracle_trimul_causal(const void *qkv, float *out, double *bound,
                         int64_t B, int64_t T, int64_t C, int64_t NH, int dtype);

/* Storage rounding of a 16-bit score output: n binary32 values to
 * bfloat16 (dtype 1) or IEEE binary16 (dtype 2) bit patterns, to nearest
 * with ties to even, overflow to infinity, subnormals kept; every NaN
 * becomes the quiet NaN 0x7FC0 (bfloat16) or 0x7E00 (binary16). */
int oracle_round16(const float *in, uint16_t *out, int64_t n, int dtype);

/* Rows t in [t0, t1) of plane (b, nh) only; out/bound are (t1-t0) x T. */
int oracle_trimul_causal_rows(const void *qkv, float *out, double *bound,
                              int64_t B, int64_t T, int64_t C, int64_t NH,
                              int64_t b, int64_t nh, int64_t t0, int64_t t1,
                              int dtype);

/* Causal softmax of the scores, in double throughout (scores not rounded
 * to fp32). For each row t of plane (b, nh), over t2 <= t:
 *   row_max[t] = max s[t][t2],  row_logsum[t] = ln sum exp(s[t][t2] - row_max[t]),
 *   mode 0: out = (s - row_max) - row_logsum   (log-probabilities)
 *   mode 1: out = exp of that                   (probabilities)
 * and for t2 > t out = -inf (mode 0) or 0 (mode 1). out (nullable) and bound
 * (nullable, the scores' error scale as in trimul) are (t1-t0) x T; row_max
 * and row_logsum (nullable) hold t1-t0 values. */
int oracle_causal_softmax_rows(const void *qkv, double *out, double *row_max, double *row_logsum,
                               double *bound, int64_t B, int64_t T, int64_t C, int64_t NH,
                               int64_t b, int64_t nh, int64_t t0, int64_t t1, int dtype, int mode);

/* The same over every plane: out is (B,NH,T,T), row_max/row_logsum (B,NH,T). */
int oracle_causal_softmax(const void *qkv, double *out, double *row_max, double *row_logsum,
                          double *bound, int64_t B, int64_t T, int64_t C, int64_t NH, int dtype, int mode);

/* Attention output of rows t in [t0, t1) of batch b, every head:
 * y[t][nh*HS + i] = sum_{t2 <= t} p[t][t2] V[b][nh][t2][i] with p the causal
 * softmax (double throughout); y and absw (nullable: sum p |V|) are
 * (t1-t0) x C doubles. */
int oracle_causal_attention_rows(const void *qkv, double *y, double *absw, int64_t B, int64_t T, int64_t C,
                                 int64_t NH, int64_t b, int64_t t0, int64_t t1, int dtype);

/* The scale factor applied to every score: fp32 nearest to 1/sqrt(HS). */
float oracle_trimul_scale(int64_t HS);

/* Tiled product out = A.B (A [M,K], B [K,N], fp32, row-major) taken tile by
 * tile, with the global-memory element counts of that loop:
 *   counts[0] = loads of in-bounds tile elements, counts[1] = in-bounds writes,
 *   counts[2] = loads if every tile were full size (padded),
 *   counts[3] = writes if every tile were full size. */
int oracle_tiled_matmul_count(const float *A, const float *Bm, float *out,
                              int64_t M, int64_t N, int64_t K,
                              int64_t bm, int64_t bn, int64_t bk,
                              int64_t *counts);

#ifdef __cplusplus
}
#endif
#endif
