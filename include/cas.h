/*
 * cas.h -- C ABI of the MI355X (gfx950) tiled-matmul hot path.
 *
 * Hand-written CDNA4 kernels with fp32 accumulation:
 *
 *   cas_gemm_nt          dense Y = X W^T over ragged shapes
 *   cas_batch_matmul_nt  the same over a batch of independent products
 *   cas_trimul_causal    causal attention scores read straight from packed QKV
 *   cas_causal_row_stats per-row max and log-sum of the causal scores
 *   cas_causal_softmax   causal softmax (log-probabilities or probabilities)
 *   cas_causal_softmax_fused  both softmax launches in one
 *   cas_causal_attention the attention output: softmax probabilities times V
 *   cas_causal_attention_fused  the attention output and the row statistics in one pass
 *
 * Conventions shared by every entry point
 *   - Pointers X, W, Y, qkv, out, row_max, row_logsum are DEVICE pointers
 *     (hipMalloc or any allocator of device memory). The caller owns every buffer; the library
 *     allocates nothing, keeps no pointer after returning and never
 *     synchronises. Buffers must stay alive until the stream reaches the
 *     kernel.
 *   - stream is a hipStream_t passed as void*; NULL selects the default
 *     (null) stream. The kernel is enqueued and the call returns at once.
 *   - Shapes and pitches are int64 counts of ELEMENTS.
 *   - Arguments are validated before any HIP call; a rejected call returns a
 *     negative cas_status and writes nothing. A failed launch returns
 *     CAS_ERR_HIP and cas_last_hip_error() gives the hipError_t (per thread).
 *     Faults inside a kernel surface at the caller's next synchronisation.
 *   - Accepted (in_dtype, out_dtype) pairs: (F32, F32), (BF16, F32),
 *     (F16, F32); cas_trimul_causal and cas_causal_softmax also take out_dtype
 *     BF16 or F16 with any input type. 16-bit inputs are raw bfloat16 / IEEE
 *     binary16 patterns.
 *   - The output byte range may not overlap an input byte range.
 *   - Any alignment is accepted (the softmax and attention: elements at their
 *     natural alignment); 16-byte aligned bases and pitches select wider loads
 *     and stores, with the same results. For the packed QKV rows only the
 *     head and row lengths decide: a qkv base at its element alignment but
 *     not on a 16-byte boundary still takes 16-byte pieces.
 *   - Kernel variants are chosen by shape, dtype and alignment. Environment
 *     variables read at each call override the choice for tests and tuning:
 *     CAS_GEMM_TILE, CAS_GEMM_F32, CAS_GEMM_WIDE, CAS_VARIANT (gemm_nt and
 *     batch_matmul_nt), CAS_TRIMUL_KERNEL, CAS_TRIMUL_PASS (trimul_causal and
 *     the softmax rows), CAS_SOFTMAX_FUSED (cas_causal_softmax_fused) and
 *     CAS_SOFTMAX_KERNEL=general (the general-shape softmax and attention
 *     kernels).
 *     Every variant meets the same accuracy bounds; those with another
 *     accumulation order may differ from the default in the last bits.
 */
#ifndef CAS_H
#define CAS_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { CAS_F32 = 0, CAS_BF16 = 1, CAS_F16 = 2 } cas_dtype;

typedef enum {
    CAS_OK = 0,
    CAS_ERR_NULL = -1,   /* a required pointer is NULL                       */
    CAS_ERR_SHAPE = -2,  /* negative dim, pitch too small, C % NH != 0, overflow */
    CAS_ERR_DTYPE = -3,  /* unsupported (in_dtype, out_dtype) pair           */
    CAS_ERR_ALIAS = -4,  /* output bytes overlap input bytes                 */
    CAS_ERR_DEVICE = -5, /* current device is not gfx950, or no device       */
    CAS_ERR_HIP = -6,    /* the HIP launch failed; see cas_last_hip_error()  */
    CAS_ERR_UNSUPPORTED = -7, /* valid, but outside the kernels' domain       */
    CAS_ERR_MODE = -8    /* unknown softmax mode                             */
} cas_status;

/* Output of cas_causal_softmax. */
enum { CAS_SOFTMAX_LOG = 0, CAS_SOFTMAX_PROB = 1 };

/*
 * Dense NT product (DietCode tests/codegen/test_1_local_padding.py,
 * test_local_padding docstring: the dense layer Y = X W^T with X [B*T, I],
 * W [H, I], Y [B*T, H], i.e. Y[i,j] += X[i,k] * W[j,k]):
 *
 *   Y[m*ldy + n] = sum_{k<K} X[m*ldx + k] * W[n*ldw + k],   m < M, n < N
 *
 * X: M rows of pitch ldx (>= K), W: N rows of pitch ldw (>= K), both of
 * in_dtype; Y: M rows of pitch ldy (>= N), fp32, written only at n < N.
 * Shapes need not be tile multiples: out-of-range rows and columns are
 * zero-filled when fetched and masked when written back.
 * M == 0 or N == 0: nothing is written (OK). K == 0: Y = 0 (the empty sum).
 */
int cas_gemm_nt(const void *X, const void *W, void *Y,
                int64_t M, int64_t N, int64_t K,
                int64_t ldx, int64_t ldw, int64_t ldy,
                cas_dtype in_dtype, cas_dtype out_dtype, void *stream);

/*
 * Batched NT product (DietCode tests/codegen/test_1_local_padding.py,
 * test_local_padding_ii docstring: BatchMatmulNT over B*NH independent heads,
 * Y[i,j,k] += X[i,j,l] * W[i,k,l]):
 *
 *   Y[b*bsy + m*ldy + n] = sum_{k<K} X[b*bsx + m*ldx + k] * W[b*bsw + n*ldw + k]
 *                                       for b < batch, m < M, n < N
 *
 * Each block b is the dense product of cas_gemm_nt, with the same pitches,
 * dtypes, ragged-shape handling and K == 0 behaviour. Batch strides bsx, bsw,
 * bsy are in elements, >= 0; an input stride of 0 repeats one block for every
 * b. Output blocks may not overlap (bsy must cover one block:
 * bsy >= (M-1)*ldy + N when batch > 1), else CAS_ERR_SHAPE.
 * batch == 0, M == 0 or N == 0: nothing is written (OK).
 */
int cas_batch_matmul_nt(const void *X, const void *W, void *Y, int64_t batch,
                        int64_t M, int64_t N, int64_t K,
                        int64_t ldx, int64_t ldw, int64_t ldy,
                        int64_t bsx, int64_t bsw, int64_t bsy,
                        cas_dtype in_dtype, cas_dtype out_dtype, void *stream);

/*
 * Causal attention scores (llm.c dev/cuda/trimat_forward.cu, trimul_cpu, the
 * "Referee" of Chapter I; launched per (batch, head) as in trimul_global of
 * Chapter II):
 *
 *   qkv  (B, T, 3, NH, HS) contiguous, C = NH*HS; Q row t of head nh starts at
 *        element b*T*3C + t*3C + nh*HS, K row t2 at the same place + C; the V
 *        third is never read.
 *   out  (B, NH, T, T) contiguous, of out_dtype:
 *        out[b,nh,t,t2] = fp32(Q.K) * s  for t2 <= t, s = fp32 nearest 1/sqrt(HS)
 *        out[b,nh,t,t2] = quiet NaN, bits 0x7FC00000, for t2 > t
 *        With out_dtype CAS_BF16 / CAS_F16 each score is that fp32 value
 *        rounded to bfloat16 / binary16 (to nearest, ties to even; past the
 *        range: infinity), and the mask is 0x7FC0 / 0x7E00. Half the bytes of
 *        the fp32 output, which bounds this operation's time.
 *
 * Only tiles on or below the diagonal are computed; the tiles above it are
 * filled with the NaN pattern by the same launch. Any T >= 1 is accepted.
 * Requires C > 0, C % NH == 0, a QKV row of 3*C elements under 2^24 bytes and
 * T < 2^24 (both far beyond what fits in memory as (T, T) planes). B == 0, T == 0 or NH == 0: nothing is
 * written (OK). Offsets are 64-bit: outputs above 2^32 bytes are fine.
 */
int cas_trimul_causal(const void *qkv, void *out,
                      int64_t B, int64_t T, int64_t C, int64_t NH,
                      cas_dtype in_dtype, cas_dtype out_dtype, void *stream);

/*
 * Causal softmax of the scores, in the two launches of the smallem page
 * "Kernels GPU" (its softmax section: row_stats computes each row's maximum
 * and ln(sum exp(x - max)), kept as two numbers; softmax_rows then forms
 * (x - max) - logsum per element, or the exponential of that), applied to
 * the causal score rows of cas_trimul_causal. Neither call reads or writes
 * the (T, T) scores: both recompute them from qkv, so the scores never
 * travel to HBM.
 *
 * cas_causal_row_stats
 *   qkv         as for cas_trimul_causal, of in_dtype.
 *   row_max     (B, NH, T) fp32, written: max over t2 <= t of the fp32
 *               score x[b,nh,t,t2] of cas_trimul_causal.
 *   row_logsum  (B, NH, T) fp32, written: ln sum_{t2 <= t} exp(x - row_max).
 *
 * cas_causal_softmax
 *   row_max, row_logsum   read: the statistics of cas_causal_row_stats on the
 *               same qkv (the caller may pass others; they are used as given).
 *   out         (B, NH, T, T) of out_dtype (fp32, bfloat16 or binary16):
 *               mode CAS_SOFTMAX_LOG:  (x - row_max) - row_logsum for t2 <= t,
 *                                      -inf for t2 > t;
 *               mode CAS_SOFTMAX_PROB: exp of that for t2 <= t, 0 for t2 > t
 *               (the softmax of the scores masked to -inf above the
 *               diagonal, the mask llm.c's trimul_cpu names as an
 *               alternative to its NaN), formed in base 2 from the
 *               accumulated product a as 2^((a scale - row_max) log2 e -
 *               row_logsum log2 e) with two fused multiply-adds. 16-bit
 *               outputs are the fp32 value rounded once more (to nearest
 *               even).
 *
 * Both: fp32 arithmetic. Two sets of kernels serve the calls:
 *   - fast kernels where the QKV rows split into 16-byte pieces (qkv at its
 *     element alignment, HS and C times the element size multiples of 16), HS times the
 *     element size is at most 512 bytes, T < 2^22 and B * NH < 2^23; there
 *     the scores are bit-identical to cas_trimul_causal's (same products in
 *     the same order);
 *   - general-shape kernels elsewhere (any HS, any base aligned to the
 *     element size), with the same formulas and the same tolerance, for
 *     any head size (rows staged in chunks of at most 640 bytes).
 * With elements off their natural alignment, or with statistics not 4-byte
 * aligned: CAS_ERR_UNSUPPORTED,
 * with nothing written. Other limits,
 * empty shapes and the no-overlap rule as for cas_trimul_causal: the
 * statistics written by cas_causal_row_stats may overlap neither qkv nor each
 * other, and out may overlap neither qkv nor the statistics it reads.
 * Unknown mode: CAS_ERR_MODE.
 */
int cas_causal_row_stats(const void *qkv, float *row_max, float *row_logsum,
                         int64_t B, int64_t T, int64_t C, int64_t NH,
                         cas_dtype in_dtype, void *stream);

int cas_causal_softmax(const void *qkv, const float *row_max, const float *row_logsum, void *out,
                       int64_t B, int64_t T, int64_t C, int64_t NH, int mode,
                       cas_dtype in_dtype, cas_dtype out_dtype, void *stream);

/*
 * Both softmax launches in one (the same outputs, statistics included):
 * each 128-row block of queries has its statistics computed and then its
 * rows written by the same workgroup, so the statistics work overlaps other
 * blocks' output stores instead of taking a launch of its own. (On general
 * shapes, and for heads of 257 .. 512 bytes, the call enqueues the
 * statistics and rows kernels back to back on the stream.) Arguments,
 * modes, output types, domain and errors as for cas_causal_softmax, with
 * row_max / row_logsum written (as by cas_causal_row_stats) instead of read;
 * out, row_max and row_logsum may overlap neither qkv nor one another.
 * row_max equals cas_causal_row_stats' bit for bit; row_logsum may differ from
 * it in the last bits (another summation order), and out uses this call's
 * own row_logsum.
 */
int cas_causal_softmax_fused(const void *qkv, void *out, float *row_max, float *row_logsum,
                             int64_t B, int64_t T, int64_t C, int64_t NH, int mode,
                             cas_dtype in_dtype, cas_dtype out_dtype, void *stream);

/*
 * Attention output, the step after the softmax:
 *   y[b, t, nh*HS + i] = sum_{t2 <= t} p[b,nh,t,t2] * V[b,t2,nh,i]
 * with V the third slot of the packed rows (element b*T*3C + t2*3C + 2C +
 * nh*HS + i) and p the probabilities cas_causal_softmax (CAS_SOFTMAX_PROB)
 * forms from the given row statistics (those of cas_causal_row_stats on the
 * same qkv), bit for bit; for 16-bit inputs p is then rounded to the input
 * format (nearest even) and multiplied by V in that format, with fp32
 * accumulation. Neither the scores nor p reach HBM: both are recomputed per
 * key tile and multiplied into y on the MFMAs.
 *   y   (B, T, C) fp32 (out_dtype must be CAS_F32), written whole.
 * Domain, limits and empty shapes as for cas_causal_softmax; y (and the 4-byte aligned
 * statistics) may not overlap qkv, and y may not overlap the statistics.
 */
int cas_causal_attention(const void *qkv, const float *row_max, const float *row_logsum, void *y,
                         int64_t B, int64_t T, int64_t C, int64_t NH,
                         cas_dtype in_dtype, cas_dtype out_dtype, void *stream);

/*
 * The attention output and the row statistics in one pass:
 *   y, row_max, row_logsum   written, as cas_causal_attention's y and
 *                            cas_causal_row_stats' statistics on the same qkv.
 * Each score and its exponential are computed once. The row max is kept as it
 * goes, the exponentials are taken against a running offset (a base-2 multiple
 * of an earlier maximum, moved only when a key tile's largest score exceeds it
 * by more than 2^8), and y and the sum are rescaled whenever the offset moves,
 * so y = sum_j p_j V_j is formed as (sum_j w_j V_j) / (sum_j w_j). This is the
 * softmax of the "Kernels GPU" section (row max, then ln sum exp(x - max),
 * then the probabilities), taken over a row in one sweep instead of two.
 * row_max equals cas_causal_row_stats' bit for bit; row_logsum and y agree
 * with the two-pass results up to rounding (another summation order). For
 * 16-bit inputs the weights w_j are rounded to the input format for the
 * products with V; the sum uses them unrounded. On general shapes (see
 * cas_causal_softmax) the launch computes the statistics first, in two sweeps
 * over the keys, writes them, and forms y from them as cas_causal_attention
 * does.
 *   y   (B, T, C) fp32 (out_dtype must be CAS_F32), written whole, 16-byte
 *       stores when y is 16-byte aligned.
 * Domain, limits and empty shapes as for cas_causal_softmax; y and the 4-byte
 * aligned statistics may overlap neither qkv nor one another.
 */
int cas_causal_attention_fused(const void *qkv, void *y, float *row_max, float *row_logsum,
                               int64_t B, int64_t T, int64_t C, int64_t NH,
                               cas_dtype in_dtype, cas_dtype out_dtype, void *stream);

/* Static description of a status code; never NULL. */
const char *cas_status_string(int status);

/* hipError_t of this thread's last CAS_ERR_HIP / CAS_ERR_DEVICE, else 0. */
int cas_last_hip_error(void);

/* Library version, major*10000 + minor*100 + patch. */
int cas_version(void);

#ifdef __cplusplus
}
#endif
#endif /* CAS_H */
