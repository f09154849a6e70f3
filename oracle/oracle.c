/*
 * oracle.c -- plain, slow, obviously correct CPU oracle for the tiled-matmul
 * hot path (dense NT product, causal triangular attention scores, their
 * causal softmax and the attention output).
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this file's library. It shares no
 * code, header, table or helper with the HIP path and imports nothing of it.
 *
 * Arithmetic: every input element is widened exactly to double, each product
 * of two widened elements is exact in double (at most 2 x 24 significant
 * bits), the products are summed in ascending contraction order in one double
 * accumulator, and the sum is rounded once to fp32 (round to nearest even).
 * Parallelism is OpenMP over independent output rows only, so the result is
 * bit-identical at any thread count.
 *
 * Parity pins (all in the CPU test suite): exact-rational brute force on tiny
 * shapes, the ramp closed form, identity and zero products, the worked tiling
 * example (864 loads, 135 writes), the triangle-versus-dense invariant, the
 * NaN count, and thread-count independence. The softmax is pinned by the
 * closed form of geometric score rows, a max-free formula on exact scores,
 * rows summing to one, and saturated rows.
 */
#include "oracle.h"

#include <math.h>
#include <omp.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------- threads */

int oracle_num_threads(void) { return omp_get_max_threads(); }

void oracle_set_threads(int n)
{
    if (n > 0) omp_set_num_threads(n);
}

/* --------------------------------------------------------------- decoding */

/* bfloat16 is the upper half of an IEEE binary32 pattern. */
static double bf16_to_double(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
static double f16_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int expo = (h >> 10) & 0x1f;
    int frac = h & 0x3ff;
    double v;
    if (expo == 0)
        v = ldexp((double)frac, -24);                /* zero or subnormal */
    else if (expo == 31)
        v = frac ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + frac), expo - 25); /* (1 + frac/2^10) 2^(e-15) */
    return sign ? -v : v;
}

/* Every bfloat16 and binary16 pattern decoded once, by bf16_to_double and
 * f16_to_double above, into a table, so the inner loops read one double
 * instead of decoding each element again (the values are the same; only the
 * time changes). Filled before any parallel region by dtype_ok(), which every
 * entry point calls first. */
static double decode_table[2][65536];
static pthread_once_t decode_once = PTHREAD_ONCE_INIT;

static void decode_table_fill(void)
{
    for (uint32_t h = 0; h < 65536u; h++) {
        decode_table[0][h] = bf16_to_double((uint16_t)h);
        decode_table[1][h] = f16_to_double((uint16_t)h);
    }
}

static double elem(const void *p, int dtype, int64_t i)
{
    switch (dtype) {
    case 0: return (double)((const float *)p)[i];
    case 1: return decode_table[0][((const uint16_t *)p)[i]];
    default: return decode_table[1][((const uint16_t *)p)[i]];
    }
}

static int dtype_ok(int dtype)
{
    pthread_once(&decode_once, decode_table_fill);
    return dtype == 0 || dtype == 1 || dtype == 2;
}

int oracle_decode(const void *src, int dtype, int64_t n, double *dst)
{
    if (!dtype_ok(dtype) || n < 0 || (n > 0 && (!src || !dst))) return -1;
    for (int64_t i = 0; i < n; i++) dst[i] = elem(src, dtype, i);
    return 0;
}

/* --------------------------------------------------------------- gemm_nt */

/* The dense layer of DietCode's test_1_local_padding.py (test_local_padding
 * docstring): Y = X W^T with X [B*T, I], W [H, I], written as the loop
 * Y[i,j] += X[i,k] * W[j,k]. Here M = B*T, N = H, K = I, with row pitches. */
int oracle_gemm_nt(const void *X, const void *W, float *Y, double *bound,
                   int64_t M, int64_t N, int64_t K,
                   int64_t ldx, int64_t ldw, int64_t ldy, int dtype)
{
    if (!dtype_ok(dtype) || M < 0 || N < 0 || K < 0) return -1;
    if (ldx < K || ldw < K || ldy < N) return -1;
    if (M == 0 || N == 0) return 0;
    if (!Y || (K > 0 && (!X || !W))) return -1;

#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; m++) {
        for (int64_t n = 0; n < N; n++) {
            double acc = 0.0, asum = 0.0;
            for (int64_t k = 0; k < K; k++) {
                double p = elem(X, dtype, m * ldx + k) * elem(W, dtype, n * ldw + k);
                acc += p;
                asum += fabs(p);
            }
            Y[m * ldy + n] = (float)acc;
            if (bound) bound[m * ldy + n] = asum;
        }
    }
    return 0;
}

/* -------------------------------------------------------- trimul_causal */

float oracle_trimul_scale(int64_t HS)
{
    /* llm.c trimat_forward.cu, trimul_cpu: the scale is 1/sqrt(HS) kept in a
     * float and applied to the finished dot product. */
    return (float)(1.0 / sqrt((double)HS));
}

static const uint32_t QNAN_BITS = 0x7FC00000u;

/* A 16-bit score output is the binary32 score rounded once more, to the
 * nearest representable value of the 16-bit format (ties to even).
 *
 * bfloat16 keeps binary32's sign and 8-bit exponent and the top 7 fraction
 * bits, so rounding works on the bit pattern: add half a unit of the 16th
 * bit (minus one when the kept last bit is even, so ties go to even) and
 * truncate. This carries into the exponent exactly when the value rounds up
 * across a binade, and into infinity above the largest finite bfloat16.
 *
 * binary16 has a 5-bit exponent (bias 15, normals from 2^-14) and 10
 * fraction bits. Every binary32 value is exact in double, and so is its
 * quotient by a power of two, so the rounding is one rint() (the default
 * round-to-nearest-even mode) of the value measured in units of the last
 * place: 2^-24 for subnormals, 2^(e-10) in binade [2^e, 2^(e+1)). */
static uint16_t round_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return 0x7FC0u; /* NaN */
    const uint32_t even = (u >> 16) & 1u;
    return (uint16_t)((u + 0x7FFFu + even) >> 16);
}

static uint16_t round_f16(float f)
{
    const double x = (double)f;
    if (isnan(x)) return 0x7E00u;
    const uint16_t sign = signbit(x) ? 0x8000u : 0;
    const double a = fabs(x);
    if (a >= 65520.0) return sign | 0x7C00u; /* at or past the midpoint above 65504: infinity */
    if (a < ldexp(1.0, -14)) {               /* subnormal range: units of 2^-24 */
        const double q = rint(ldexp(a, 24)); /* may reach 1024 = the smallest normal */
        return sign | (uint16_t)q;
    }
    int e;
    (void)frexp(a, &e);                      /* a = m * 2^e, m in [0.5, 1): binade [2^(e-1), 2^e) */
    e -= 1;
    double q = rint(ldexp(a, 10 - e));       /* significand in units of the last place: [1024, 2048] */
    if (q >= 2048.0) {
        q = 1024.0;
        e += 1;
    }
    if (e > 15) return sign | 0x7C00u;
    return sign | (uint16_t)((e + 15) << 10) | (uint16_t)(q - 1024.0);
}

int oracle_round16(const float *in, uint16_t *out, int64_t n, int dtype)
{
    if (!in || !out || n < 0 || (dtype != 1 && dtype != 2)) return -1;
    for (int64_t i = 0; i < n; ++i) out[i] = dtype == 1 ? round_bf16(in[i]) : round_f16(in[i]);
    return 0;
}

/* llm.c trimat_forward.cu, trimul_cpu (the "Referee" of Chapter I):
 * inp is (B, T, 3, NH, HS); query row t of head nh starts at
 * b*T*3C + t*3C + nh*HS, the key row t2 at the same place plus C; for
 * t2 <= t the output is the dot product times the scale, and every t2 > t
 * holds NaN (the causal mask). out is (B, NH, T, T). */
int oracle_trimul_causal_rows(const void *qkv, float *out, double *bound,
                              int64_t B, int64_t T, int64_t C, int64_t NH,
                              int64_t b, int64_t nh, int64_t t0, int64_t t1,
                              int dtype)
{
    if (!dtype_ok(dtype) || B < 0 || T < 0 || NH <= 0 || C <= 0 || C % NH != 0) return -1;
    if (b < 0 || b >= B || nh < 0 || nh >= NH || t0 < 0 || t1 > T || t0 > t1) return -1;
    if (t1 == t0) return 0;
    if (!qkv || !out) return -1;

    const int64_t HS = C / NH;
    const int64_t C3 = 3 * C;
    const float scale = oracle_trimul_scale(HS);
    float nanv;
    memcpy(&nanv, &QNAN_BITS, sizeof nanv);

#pragma omp parallel for schedule(static)
    for (int64_t t = t0; t < t1; t++) {
        const int64_t q0 = b * T * C3 + t * C3 + nh * HS;   /* Q[b][nh][t][:] */
        float *orow = out + (t - t0) * T;
        double *brow = bound ? bound + (t - t0) * T : 0;
        for (int64_t t2 = 0; t2 < T; t2++) {
            if (t2 <= t) {
                const int64_t k0 = b * T * C3 + t2 * C3 + nh * HS + C; /* K[b][nh][t2][:] */
                double acc = 0.0, asum = 0.0;
                for (int64_t i = 0; i < HS; i++) {
                    double p = elem(qkv, dtype, q0 + i) * elem(qkv, dtype, k0 + i);
                    acc += p;
                    asum += fabs(p);
                }
                orow[t2] = (float)(acc * (double)scale);
                if (brow) brow[t2] = fabs((double)scale) * asum;
            } else {
                orow[t2] = nanv;
                if (brow) brow[t2] = 0.0;
            }
        }
    }
    return 0;
}

int oracle_trimul_causal(const void *qkv, float *out, double *bound,
                         int64_t B, int64_t T, int64_t C, int64_t NH, int dtype)
{
    if (!dtype_ok(dtype) || B < 0 || T < 0 || NH < 0) return -1;
    if (B == 0 || T == 0 || NH == 0) return 0;
    if (C <= 0 || C % NH != 0) return -1;
    for (int64_t b = 0; b < B; b++) {
        for (int64_t nh = 0; nh < NH; nh++) {
            const int64_t plane = (b * NH + nh) * T * T;   /* out[b][nh][:][:] */
            int rc = oracle_trimul_causal_rows(qkv, out + plane, bound ? bound + plane : 0,
                                               B, T, C, NH, b, nh, 0, T, dtype);
            if (rc) return rc;
        }
    }
    return 0;
}

/* ------------------------------------------------------ causal softmax */

/* smallem "Kernels GPU" page, section on the softmax in two launches: a
 * first launch (row_stats) reduces every row to two numbers, its maximum and
 * ln(sum exp(x - max)); a second (softmax_rows) gives each element
 * (x - max) - logsum, or the exponential of that for probabilities. The two
 * reductions stay separate numbers, as the page recommends. Here the rows are
 * the causal score rows of trimul_cpu (llm.c trimat_forward.cu, the Referee
 * of Chapter I, whose first pass also notes the row maximum): entries
 * t2 <= t take part, and t2 > t is the causal mask, which that file says could
 * as well be -inf: log-probability -inf, probability 0. Everything is double;
 * the scores are the exact products times the fp32 scale, not rounded. */
int oracle_causal_softmax_rows(const void *qkv, double *out, double *row_max, double *row_logsum,
                               double *bound, int64_t B, int64_t T, int64_t C, int64_t NH,
                               int64_t b, int64_t nh, int64_t t0, int64_t t1, int dtype, int mode)
{
    if (!dtype_ok(dtype) || (mode != 0 && mode != 1)) return -1;
    if (B < 0 || T < 0 || NH <= 0 || C <= 0 || C % NH != 0) return -1;
    if (b < 0 || b >= B || nh < 0 || nh >= NH || t0 < 0 || t1 > T || t0 > t1) return -1;
    if (t1 == t0) return 0;
    if (!qkv) return -1;

    const int64_t HS = C / NH;
    const int64_t C3 = 3 * C;
    const double scale = (double)oracle_trimul_scale(HS);
    int failed = 0;

#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t t = t0; t < t1; t++) {
        double *s = (double *)malloc((size_t)(t + 1) * sizeof(double));
        if (!s) {
#pragma omp atomic write
            failed = 1;
            continue;
        }
        const int64_t q0 = b * T * C3 + t * C3 + nh * HS;              /* Q[b][nh][t][:] */
        for (int64_t t2 = 0; t2 <= t; t2++) {
            const int64_t k0 = b * T * C3 + t2 * C3 + nh * HS + C;     /* K[b][nh][t2][:] */
            double acc = 0.0, asum = 0.0;
            for (int64_t i = 0; i < HS; i++) {
                double p = elem(qkv, dtype, q0 + i) * elem(qkv, dtype, k0 + i);
                acc += p;
                asum += fabs(p);
            }
            s[t2] = acc * scale;
            if (bound) bound[(t - t0) * T + t2] = scale * asum;
        }
        /* row_stats: the maximum, then the log of the shifted sum */
        double mx = s[0];
        for (int64_t t2 = 1; t2 <= t; t2++)
            if (s[t2] > mx) mx = s[t2];
        double sum = 0.0;
        for (int64_t t2 = 0; t2 <= t; t2++) sum += exp(s[t2] - mx);
        const double lse = log(sum);
        if (row_max) row_max[t - t0] = mx;
        if (row_logsum) row_logsum[t - t0] = lse;
        /* softmax_rows */
        if (out) {
            double *orow = out + (t - t0) * T;
            for (int64_t t2 = 0; t2 <= t; t2++) {
                const double lp = (s[t2] - mx) - lse;
                orow[t2] = mode == 0 ? lp : exp(lp);
            }
            for (int64_t t2 = t + 1; t2 < T; t2++) orow[t2] = mode == 0 ? -INFINITY : 0.0;
        }
        if (bound)
            for (int64_t t2 = t + 1; t2 < T; t2++) bound[(t - t0) * T + t2] = 0.0;
        free(s);
    }
    return failed ? -1 : 0;
}

int oracle_causal_softmax(const void *qkv, double *out, double *row_max, double *row_logsum,
                          double *bound, int64_t B, int64_t T, int64_t C, int64_t NH, int dtype, int mode)
{
    if (!dtype_ok(dtype) || (mode != 0 && mode != 1) || B < 0 || T < 0 || NH < 0) return -1;
    if (B == 0 || T == 0 || NH == 0) return 0;
    if (C <= 0 || C % NH != 0) return -1;
    for (int64_t b = 0; b < B; b++) {
        for (int64_t nh = 0; nh < NH; nh++) {
            const int64_t row = (b * NH + nh) * T;                 /* row (b, nh, 0) */
            int rc = oracle_causal_softmax_rows(qkv, out ? out + row * T : 0, row_max ? row_max + row : 0,
                                                row_logsum ? row_logsum + row : 0, bound ? bound + row * T : 0,
                                                B, T, C, NH, b, nh, 0, T, dtype, mode);
            if (rc) return rc;
        }
    }
    return 0;
}

/* -------------------------------------------------- attention output */

/* The step after the softmax (the page's row_stats / softmax_rows feed it):
 * the attention output of query row t of head nh is the probability-weighted
 * sum of the value rows, y[b][t][nh][:] = sum_{t2 <= t} p[t][t2] V[b][nh][t2][:],
 * V[b][nh][t2][:] = inp[b][t2][2][nh][:] (the third slot of the packed row,
 * after Q and K). p is the causal softmax above, recomputed here in double.
 * y is (rows t0..t1-1 of batch b) x C, head nh at columns nh*HS..; absw
 * (nullable, same shape) gets sum_t2 p |V|, the error scale of each output. */
int oracle_causal_attention_rows(const void *qkv, double *y, double *absw, int64_t B, int64_t T, int64_t C,
                                 int64_t NH, int64_t b, int64_t t0, int64_t t1, int dtype)
{
    if (!dtype_ok(dtype) || B < 0 || T < 0 || NH <= 0 || C <= 0 || C % NH != 0) return -1;
    if (b < 0 || b >= B || t0 < 0 || t1 > T || t0 > t1) return -1;
    if (t1 == t0) return 0;
    if (!qkv || !y) return -1;

    const int64_t HS = C / NH;
    const int64_t C3 = 3 * C;
    const double scale = (double)oracle_trimul_scale(HS);
    int failed = 0;

#pragma omp parallel for collapse(2) schedule(dynamic, 4)
    for (int64_t t = t0; t < t1; t++) {
        for (int64_t nh = 0; nh < NH; nh++) {
            double *s = (double *)malloc((size_t)(t + 1) * sizeof(double));
            if (!s) {
#pragma omp atomic write
                failed = 1;
                continue;
            }
            const int64_t q0 = b * T * C3 + t * C3 + nh * HS;           /* Q[b][nh][t][:] */
            for (int64_t t2 = 0; t2 <= t; t2++) {
                const int64_t k0 = b * T * C3 + t2 * C3 + C + nh * HS;  /* K[b][nh][t2][:] */
                double acc = 0.0;
                for (int64_t i = 0; i < HS; i++) acc += elem(qkv, dtype, q0 + i) * elem(qkv, dtype, k0 + i);
                s[t2] = scale * acc;                                     /* the score of (t, t2) */
            }
            /* the softmax of row t: its maximum, then its log-sum */
            double rmax = s[0];
            for (int64_t t2 = 1; t2 <= t; t2++) rmax = s[t2] > rmax ? s[t2] : rmax;
            double rsum = 0.0;
            for (int64_t t2 = 0; t2 <= t; t2++) rsum += exp(s[t2] - rmax);
            const double rlog = log(rsum);
            double *yrow = y + (t - t0) * C + nh * HS;
            double *arow = absw ? absw + (t - t0) * C + nh * HS : 0;
            for (int64_t i = 0; i < HS; i++) {
                double acc = 0.0, aacc = 0.0;
                for (int64_t t2 = 0; t2 <= t; t2++) {
                    const double p = exp((s[t2] - rmax) - rlog);
                    const double v = elem(qkv, dtype, b * T * C3 + t2 * C3 + 2 * C + nh * HS + i); /* V[b][nh][t2][i] */
                    acc += p * v;
                    aacc += p * fabs(v);
                }
                yrow[i] = acc;
                if (arow) arow[i] = aacc;
            }
            free(s);
        }
    }
    return failed ? -1 : 0;
}

/* ------------------------------------------- tiled count (kernl tutorial) */

static int64_t min64(int64_t a, int64_t b) { return a < b ? a : b; }

/* kernl tutorial "1 - tiled matmul", section "Simple matmul with tiling":
 * loop over output tiles (M, then N), and for each over K tiles; every tile
 * of A and of B that is fetched counts its elements as global loads, the
 * tile's partial product is added into an accumulator, and the finished
 * accumulator counts its elements as global writes. Tiles are clipped at the
 * matrix edges; the padded counts are what full-size tiles would move. */
int oracle_tiled_matmul_count(const float *A, const float *Bm, float *out,
                              int64_t M, int64_t N, int64_t K,
                              int64_t bm, int64_t bn, int64_t bk,
                              int64_t *counts)
{
    if (M < 0 || N < 0 || K < 0 || bm <= 0 || bn <= 0 || bk <= 0 || !counts) return -1;
    if ((M * N > 0 && !out) || (M * N * K > 0 && (!A || !Bm))) return -1;
    int64_t loads = 0, writes = 0, ploads = 0, pwrites = 0;

    for (int64_t sm = 0; sm < M; sm += bm) {
        const int64_t em = min64(sm + bm, M);
        for (int64_t sn = 0; sn < N; sn += bn) {
            const int64_t en = min64(sn + bn, N);
            const int64_t tw = en - sn;
            /* accumulator for this output tile, in double */
            double *acc = (double *)calloc((size_t)((em - sm) * tw), sizeof(double));
            if (!acc) return -1;
            for (int64_t sk = 0; sk < K; sk += bk) {
                const int64_t ek = min64(sk + bk, K);
                loads += (em - sm) * (ek - sk);   /* tile of A */
                loads += (ek - sk) * (en - sn);   /* tile of B */
                ploads += bm * bk + bk * bn;
                for (int64_t i = sm; i < em; i++)
                    for (int64_t j = sn; j < en; j++) {
                        double part = 0.0;        /* tile_A @ tile_B, one entry */
                        for (int64_t k = sk; k < ek; k++)
                            part += (double)A[i * K + k] * (double)Bm[k * N + j];
                        acc[(i - sm) * tw + (j - sn)] += part;
                    }
            }
            for (int64_t i = sm; i < em; i++)
                for (int64_t j = sn; j < en; j++) out[i * N + j] = (float)acc[(i - sm) * tw + (j - sn)];
            free(acc);
            writes += (em - sm) * (en - sn);
            pwrites += bm * bn;
        }
    }
    counts[0] = loads;
    counts[1] = writes;
    counts[2] = ploads;
    counts[3] = pwrites;
    return 0;
}
