// cas_api.hip -- the C ABI (include/cas.h): argument validation, variant
// choice and launch on the caller's stream.
//
// Every check that can be made without the GPU happens before the first HIP
// call, so a rejected call returns its status on any machine. No exception
// crosses the ABI and the library keeps no state besides a per-device
// "is this gfx950" answer and the per-thread last HIP error.
#include "cas.h"
#include "launch.hpp"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdlib>
#include <cstring>
#include <mutex>

#define CAS_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

thread_local int g_last_hip = 0;

constexpr int MAX_DEVICES = 64;

bool mul_ok(int64_t a, int64_t b, int64_t *r) { return !__builtin_mul_overflow(a, b, r); }
bool add_ok(int64_t a, int64_t b, int64_t *r) { return !__builtin_add_overflow(a, b, r); }

int elem_size(cas_dtype d) { return d == CAS_F32 ? 4 : 2; }

bool dtype_in_ok(cas_dtype in) { return in == CAS_F32 || in == CAS_BF16 || in == CAS_F16; }

// Dense products: fp32 output.
bool dtype_pair_ok(cas_dtype in, cas_dtype out) { return dtype_in_ok(in) && out == CAS_F32; }

// Causal scores: fp32, bfloat16 or binary16 output.
bool score_dtype_pair_ok(cas_dtype in, cas_dtype out)
{
    return dtype_in_ok(in) && (out == CAS_F32 || out == CAS_BF16 || out == CAS_F16);
}

// Byte extent of `rows` rows of `cols` elements at pitch `ld`: ((rows-1)*ld + cols)*es.
bool extent(int64_t rows, int64_t cols, int64_t ld, int es, int64_t *bytes)
{
    if (rows == 0 || cols == 0) {
        *bytes = 0;
        return true;
    }
    int64_t t;
    return mul_ok(rows - 1, ld, &t) && add_ok(t, cols, &t) && mul_ok(t, es, bytes) && *bytes < (INT64_C(1) << 62);
}

// Byte extent of `batch` such blocks, block b starting bs elements after
// block b-1: (batch-1)*bs*es + the extent of one block.
bool batch_extent(int64_t batch, int64_t bs, int64_t block_bytes, int es, int64_t *bytes)
{
    if (batch == 0 || block_bytes == 0) {
        *bytes = 0;
        return true;
    }
    int64_t t;
    return mul_ok(batch - 1, bs, &t) && mul_ok(t, es, &t) && add_ok(t, block_bytes, bytes) &&
           *bytes < (INT64_C(1) << 62);
}

bool overlap(const void *a, int64_t na, const void *b, int64_t nb)
{
    if (na == 0 || nb == 0) return false;
    const uintptr_t a0 = (uintptr_t)a, a1 = a0 + (uintptr_t)na;
    const uintptr_t b0 = (uintptr_t)b, b1 = b0 + (uintptr_t)nb;
    return a0 < b1 && b0 < a1;
}

int device_check()
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        g_last_hip = (int)e;
        return CAS_ERR_DEVICE;
    }
    if (dev < 0 || dev >= MAX_DEVICES) return CAS_ERR_DEVICE;
    static std::once_flag once[MAX_DEVICES];
    static bool is_gfx950[MAX_DEVICES];
    std::call_once(once[dev], [dev] {
        hipDeviceProp_t p;
        if (hipGetDeviceProperties(&p, dev) == hipSuccess)
            is_gfx950[dev] = std::strncmp(p.gcnArchName, "gfx950", 6) == 0;
    });
    return is_gfx950[dev] ? CAS_OK : CAS_ERR_DEVICE;
}

// Widest load (in elements, at most 16 bytes) that divides every length and
// pitch and the alignment of every base address.
int pick_vec(int es, const int64_t *lens, int nlens, const void *const *ptrs, int nptrs)
{
    for (int v = 16 / es; v > 1; v /= 2) {
        bool ok = true;
        for (int i = 0; i < nlens; ++i) ok = ok && (lens[i] % v == 0);
        for (int i = 0; i < nptrs; ++i) ok = ok && ((uintptr_t)ptrs[i] % (uintptr_t)(v * es) == 0);
        if (ok) return v;
    }
    return 1;
}

// Widest 16-byte-or-narrower piece of the packed QKV rows for the score,
// softmax and attention kernels: from the head and row lengths alone when
// the base sits at its element alignment. Their buffer loads of 16 bytes
// take any base alignment (every row then shares the base's offset within a
// 16-byte line); a base off its element alignment gets single elements.
int pick_vec_qkv(int es, int64_t HS, int64_t C, const void *qkv)
{
    if ((uintptr_t)qkv % (uintptr_t)es != 0) return 1;
    const int64_t lens[2] = {HS, C};
    return pick_vec(es, lens, 2, nullptr, 0);
}

// CAS_SOFTMAX_KERNEL=general puts the causal softmax and attention on the
// general-shape kernels (tests and tuning).
bool force_general_softmax()
{
    const char *v = std::getenv("CAS_SOFTMAX_KERNEL");
    return v && std::strcmp(v, "general") == 0;
}

// CAS_GEMM_TILE=64|128|256 forces the dense tile shape (tests and tuning;
// 256 applies where its kernel does, see gemm_wide_fits); anything else leaves
// the automatic choice.
int gemm_tile_override()
{
    const char *v = std::getenv("CAS_GEMM_TILE");
    if (!v) return cas::GEMM_TILE_AUTO;
    if (std::strcmp(v, "64") == 0) return cas::GEMM_TILE_64;
    if (std::strcmp(v, "128") == 0) return cas::GEMM_TILE_128;
    if (std::strcmp(v, "256") == 0) return cas::GEMM_TILE_256;
    return cas::GEMM_TILE_AUTO;
}

// CAS_VARIANT=predicated keeps the bounds checks inside the dense product's
// MFMA loop (on the general tile kernel): the baseline of the local-padding
// A/B measurement. Anything else is the local-padding path.
bool gemm_predicated()
{
    const char *v = std::getenv("CAS_VARIANT");
    return v && std::strcmp(v, "predicated") == 0;
}

int launch_status(hipError_t e)
{
    if (e == hipSuccess) return CAS_OK;
    g_last_hip = (int)e;
    return CAS_ERR_HIP;
}

} // namespace

CAS_EXPORT int cas_gemm_nt(const void *X, const void *W, void *Y, int64_t M, int64_t N, int64_t K, int64_t ldx,
                           int64_t ldw, int64_t ldy, cas_dtype in_dtype, cas_dtype out_dtype, void *stream)
{
    if (!dtype_pair_ok(in_dtype, out_dtype)) return CAS_ERR_DTYPE;
    if (M < 0 || N < 0 || K < 0 || ldx < K || ldw < K || ldy < N) return CAS_ERR_SHAPE;
    if (M == 0 || N == 0) return CAS_OK;
    if (!Y || (K > 0 && (!X || !W))) return CAS_ERR_NULL;
    const int es = elem_size(in_dtype);
    int64_t xb, wb, yb;
    if (!extent(M, K, ldx, es, &xb) || !extent(N, K, ldw, es, &wb) || !extent(M, N, ldy, 4, &yb))
        return CAS_ERR_SHAPE;
    if (overlap(Y, yb, X, xb) || overlap(Y, yb, W, wb)) return CAS_ERR_ALIAS;

    cas::GemmArgs a{X, W, (float *)Y, M, N, K, ldx, ldw, ldy, gemm_predicated()};
    const int tile = gemm_tile_override();
    if (cas::gemm_nt_workgroups(a, in_dtype, tile) > INT32_MAX) return CAS_ERR_SHAPE;
    const int dc = device_check();
    if (dc != CAS_OK) return dc;

    const int64_t lens[3] = {K, ldx, ldw};
    const void *ptrs[2] = {X, W};
    const int vec = K > 0 ? pick_vec(es, lens, 3, ptrs, 2) : 1;
    return launch_status(cas::launch_gemm_nt(a, in_dtype, vec, tile, (hipStream_t)stream));
}

CAS_EXPORT int cas_batch_matmul_nt(const void *X, const void *W, void *Y, int64_t batch, int64_t M, int64_t N,
                                   int64_t K, int64_t ldx, int64_t ldw, int64_t ldy, int64_t bsx, int64_t bsw,
                                   int64_t bsy, cas_dtype in_dtype, cas_dtype out_dtype, void *stream)
{
    if (!dtype_pair_ok(in_dtype, out_dtype)) return CAS_ERR_DTYPE;
    if (batch < 0 || M < 0 || N < 0 || K < 0 || ldx < K || ldw < K || ldy < N || bsx < 0 || bsw < 0 || bsy < 0)
        return CAS_ERR_SHAPE;
    if (batch == 0 || M == 0 || N == 0) return CAS_OK;
    if (!Y || (K > 0 && (!X || !W))) return CAS_ERR_NULL;
    const int es = elem_size(in_dtype);
    int64_t xb, wb, yb, xt, wt, yt;
    if (!extent(M, K, ldx, es, &xb) || !extent(N, K, ldw, es, &wb) || !extent(M, N, ldy, 4, &yb))
        return CAS_ERR_SHAPE;
    // Output blocks may not overlap one another (inputs may: bs = 0 repeats one).
    if (batch > 1 && bsy * 4 < yb) return CAS_ERR_SHAPE;
    if (!batch_extent(batch, bsx, xb, es, &xt) || !batch_extent(batch, bsw, wb, es, &wt) ||
        !batch_extent(batch, bsy, yb, 4, &yt))
        return CAS_ERR_SHAPE;
    if (overlap(Y, yt, X, xt) || overlap(Y, yt, W, wt)) return CAS_ERR_ALIAS;

    cas::GemmArgs a{X, W, (float *)Y, M, N, K, ldx, ldw, ldy, gemm_predicated(), batch, bsx, bsw, bsy};
    const int tile = gemm_tile_override();
    if (cas::gemm_nt_workgroups(a, in_dtype, tile) > INT32_MAX) return CAS_ERR_SHAPE;
    const int dc = device_check();
    if (dc != CAS_OK) return dc;

    // Vector loads must stay aligned in every block: the batch strides count too.
    const int64_t lens[5] = {K, ldx, ldw, bsx, bsw};
    const void *ptrs[2] = {X, W};
    const int vec = K > 0 ? pick_vec(es, lens, 5, ptrs, 2) : 1;
    return launch_status(cas::launch_gemm_nt(a, in_dtype, vec, tile, (hipStream_t)stream));
}

CAS_EXPORT int cas_trimul_causal(const void *qkv, void *out, int64_t B, int64_t T, int64_t C, int64_t NH,
                                 cas_dtype in_dtype, cas_dtype out_dtype, void *stream)
{
    if (!score_dtype_pair_ok(in_dtype, out_dtype)) return CAS_ERR_DTYPE;
    if (B < 0 || T < 0 || C < 0 || NH < 0) return CAS_ERR_SHAPE;
    if (B == 0 || T == 0 || NH == 0) return CAS_OK;
    if (C == 0 || C % NH != 0) return CAS_ERR_SHAPE;
    if (!qkv || !out) return CAS_ERR_NULL;
    const int es = elem_size(in_dtype), ob = elem_size(out_dtype);
    int64_t in_elems, out_elems, t, c3, inb, outb;
    if (!mul_ok(3, C, &c3) || !mul_ok(B, T, &t) || !mul_ok(t, c3, &in_elems) || !mul_ok(in_elems, es, &inb))
        return CAS_ERR_SHAPE;
    if (!mul_ok(B, NH, &t) || !mul_ok(t, T, &t) || !mul_ok(t, T, &out_elems) || !mul_ok(out_elems, ob, &outb))
        return CAS_ERR_SHAPE;
    if (inb >= (INT64_C(1) << 62) || outb >= (INT64_C(1) << 62)) return CAS_ERR_SHAPE;
    // The kernels address a 64-row tile with 31-bit buffer offsets.
    if (c3 * es >= (INT64_C(1) << 24) || T >= (INT64_C(1) << 24)) return CAS_ERR_SHAPE;
    if (overlap(out, outb, qkv, inb)) return CAS_ERR_ALIAS;
    if (cas::trimul_workgroups(B, T, NH) > INT32_MAX) return CAS_ERR_SHAPE;
    const int dc = device_check();
    if (dc != CAS_OK) return dc;

    const int64_t HS = C / NH;
    cas::TrimulArgs a{};
    a.qkv = qkv;
    a.out = out;
    a.B = B;
    a.T = T;
    a.C = C;
    a.NH = NH;
    a.HS = HS;
    a.scale = (float)(1.0 / std::sqrt((double)HS)); // nearest fp32 to 1/sqrt(HS)
    a.vec_store = ((T * ob) % 16 == 0) && ((uintptr_t)out % 16 == 0);
    a.out_kind = (int)out_dtype;
    const int vec = pick_vec_qkv(es, HS, C, qkv);
    return launch_status(cas::launch_trimul(a, in_dtype, vec, (hipStream_t)stream));
}

namespace {

// Shared checks of the causal-softmax and attention entry points: shapes,
// byte extents of qkv (inb), of one statistics array (stb) and of the output
// (outb, for out_bytes per element), the 16-byte piece width of the QKV rows
// (vec), and which kernels serve the shape: the fast ones, or (*general) the
// general-shape ones; outside both domains CAS_ERR_UNSUPPORTED. The fast
// kernels take heads of up to 512 bytes in 16-byte pieces.
int softmax_checks(const void *qkv, int64_t B, int64_t T, int64_t C, int64_t NH, cas_dtype in_dtype, int out_bytes,
                   int64_t *inb, int64_t *stb, int64_t *outb, int *vec, bool *general)
{
    if (B < 0 || T < 0 || C < 0 || NH < 0) return CAS_ERR_SHAPE;
    if (B == 0 || T == 0 || NH == 0) return 1; // nothing to do
    if (C == 0 || C % NH != 0) return CAS_ERR_SHAPE;
    const int es = elem_size(in_dtype);
    int64_t in_elems, rows, t, c3;
    if (!mul_ok(3, C, &c3) || !mul_ok(B, T, &t) || !mul_ok(t, c3, &in_elems) || !mul_ok(in_elems, es, inb))
        return CAS_ERR_SHAPE;
    if (!mul_ok(B, NH, &t) || !mul_ok(t, T, &rows) || !mul_ok(rows, 4, stb) || !mul_ok(rows, T, &t) ||
        !mul_ok(t, out_bytes, outb))
        return CAS_ERR_SHAPE;
    if (*inb >= (INT64_C(1) << 62) || *outb >= (INT64_C(1) << 62)) return CAS_ERR_SHAPE;
    if (c3 * es >= (INT64_C(1) << 24) || T >= (INT64_C(1) << 24)) return CAS_ERR_SHAPE;
    const int64_t HS = C / NH;
    *vec = qkv ? pick_vec_qkv(es, HS, C, qkv) : 1;
    const int64_t nts = (T + 127) / 128;
    if (B * NH * (nts * (nts + 1) / 2) > INT32_MAX || cas::row_stats_workgroups(B, T, NH) > INT32_MAX)
        return CAS_ERR_SHAPE;
    // the fast launches, split by query block, keep a grid below 2^32
    // work-items (256 per workgroup) while the B * NH planes of one block fit
    // in one grid
    const bool fast = cas::softmax_fits(T, HS, es, *vec);
    *general = !fast || B * NH >= (INT64_C(1) << 23) || force_general_softmax();
    if (*general && !cas::general_softmax_fits(B, T, NH, es, qkv)) return CAS_ERR_UNSUPPORTED;
    return CAS_OK;
}

cas::TrimulArgs softmax_args(const void *qkv, void *out, const float *row_max, const float *row_logsum, int64_t B,
                             int64_t T, int64_t C, int64_t NH, int out_bytes, int out_kind)
{
    cas::TrimulArgs a{};
    a.qkv = qkv;
    a.out = out;
    a.B = B;
    a.T = T;
    a.C = C;
    a.NH = NH;
    a.HS = C / NH;
    a.scale = (float)(1.0 / std::sqrt((double)a.HS)); // nearest fp32 to 1/sqrt(HS)
    a.vec_store = out && ((T * out_bytes) % 16 == 0) && ((uintptr_t)out % 16 == 0);
    a.out_kind = out_kind;
    a.row_max = row_max;
    a.row_logsum = row_logsum;
    return a;
}

} // namespace

CAS_EXPORT int cas_causal_row_stats(const void *qkv, float *row_max, float *row_logsum, int64_t B, int64_t T,
                                    int64_t C, int64_t NH, cas_dtype in_dtype, void *stream)
{
    if (!dtype_in_ok(in_dtype)) return CAS_ERR_DTYPE;
    int64_t inb, stb, outb;
    int vec = 1;
    bool general = false;
    const int rc = softmax_checks(qkv, B, T, C, NH, in_dtype, 0, &inb, &stb, &outb, &vec, &general);
    if (rc == 1) return CAS_OK;
    if (rc == CAS_ERR_SHAPE) return rc;
    if (!qkv || !row_max || !row_logsum) return CAS_ERR_NULL;
    if (rc != CAS_OK) return rc;
    if ((uintptr_t)row_max % 4 != 0 || (uintptr_t)row_logsum % 4 != 0) return CAS_ERR_UNSUPPORTED;
    if (overlap(row_max, stb, qkv, inb) || overlap(row_logsum, stb, qkv, inb) || overlap(row_max, stb, row_logsum, stb))
        return CAS_ERR_ALIAS;
    const int dc = device_check();
    if (dc != CAS_OK) return dc;
    const cas::TrimulArgs a = softmax_args(qkv, nullptr, row_max, row_logsum, B, T, C, NH, 4, 0);
    if (general) return launch_status(cas::launch_gen_row_stats(a, in_dtype, (hipStream_t)stream));
    return launch_status(cas::launch_row_stats(a, in_dtype, (hipStream_t)stream));
}

CAS_EXPORT int cas_causal_softmax(const void *qkv, const float *row_max, const float *row_logsum, void *out,
                                  int64_t B, int64_t T, int64_t C, int64_t NH, int mode, cas_dtype in_dtype,
                                  cas_dtype out_dtype, void *stream)
{
    if (!score_dtype_pair_ok(in_dtype, out_dtype)) return CAS_ERR_DTYPE;
    if (mode != CAS_SOFTMAX_LOG && mode != CAS_SOFTMAX_PROB) return CAS_ERR_MODE;
    const int ob = elem_size(out_dtype);
    int64_t inb, stb, outb;
    int vec = 1;
    bool general = false;
    const int rc = softmax_checks(qkv, B, T, C, NH, in_dtype, ob, &inb, &stb, &outb, &vec, &general);
    if (rc == 1) return CAS_OK;
    if (rc == CAS_ERR_SHAPE) return rc;
    if (!qkv || !row_max || !row_logsum || !out) return CAS_ERR_NULL;
    if (rc != CAS_OK) return rc;
    if ((uintptr_t)row_max % 4 != 0 || (uintptr_t)row_logsum % 4 != 0) return CAS_ERR_UNSUPPORTED;
    if (overlap(out, outb, qkv, inb) || overlap(out, outb, row_max, stb) || overlap(out, outb, row_logsum, stb))
        return CAS_ERR_ALIAS;
    const int dc = device_check();
    if (dc != CAS_OK) return dc;
    const cas::TrimulArgs a = softmax_args(qkv, out, row_max, row_logsum, B, T, C, NH, ob, (int)out_dtype);
    if (general) return launch_status(cas::launch_gen_softmax(a, in_dtype, mode, (hipStream_t)stream));
    return launch_status(cas::launch_softmax(a, in_dtype, mode, (hipStream_t)stream));
}

CAS_EXPORT int cas_causal_softmax_fused(const void *qkv, void *out, float *row_max, float *row_logsum, int64_t B,
                                        int64_t T, int64_t C, int64_t NH, int mode, cas_dtype in_dtype,
                                        cas_dtype out_dtype, void *stream)
{
    if (!score_dtype_pair_ok(in_dtype, out_dtype)) return CAS_ERR_DTYPE;
    if (mode != CAS_SOFTMAX_LOG && mode != CAS_SOFTMAX_PROB) return CAS_ERR_MODE;
    const int ob = elem_size(out_dtype);
    int64_t inb, stb, outb;
    int vec = 1;
    bool general = false;
    const int rc = softmax_checks(qkv, B, T, C, NH, in_dtype, ob, &inb, &stb, &outb, &vec, &general);
    if (rc == 1) return CAS_OK;
    if (rc == CAS_ERR_SHAPE) return rc;
    if (!qkv || !out || !row_max || !row_logsum) return CAS_ERR_NULL;
    if (rc != CAS_OK) return rc;
    if ((uintptr_t)row_max % 4 != 0 || (uintptr_t)row_logsum % 4 != 0) return CAS_ERR_UNSUPPORTED;
    // Three outputs: none may overlap qkv or another output.
    if (overlap(out, outb, qkv, inb) || overlap(row_max, stb, qkv, inb) || overlap(row_logsum, stb, qkv, inb) ||
        overlap(out, outb, row_max, stb) || overlap(out, outb, row_logsum, stb) ||
        overlap(row_max, stb, row_logsum, stb))
        return CAS_ERR_ALIAS;
    const int dc = device_check();
    if (dc != CAS_OK) return dc;
    const cas::TrimulArgs a = softmax_args(qkv, out, row_max, row_logsum, B, T, C, NH, ob, (int)out_dtype);
    if (general) { // the statistics launch, then the rows launch, on the caller's stream
        const hipError_t e = cas::launch_gen_row_stats(a, in_dtype, (hipStream_t)stream);
        if (e != hipSuccess) return launch_status(e);
        return launch_status(cas::launch_gen_softmax(a, in_dtype, mode, (hipStream_t)stream));
    }
    return launch_status(cas::launch_softmax_fused(a, in_dtype, mode, (hipStream_t)stream));
}

CAS_EXPORT int cas_causal_attention(const void *qkv, const float *row_max, const float *row_logsum, void *y,
                                    int64_t B, int64_t T, int64_t C, int64_t NH, cas_dtype in_dtype,
                                    cas_dtype out_dtype, void *stream)
{
    if (!dtype_in_ok(in_dtype) || out_dtype != CAS_F32) return CAS_ERR_DTYPE;
    int64_t inb, stb, outb;
    int vec = 1;
    bool general = false;
    const int rc = softmax_checks(qkv, B, T, C, NH, in_dtype, 0, &inb, &stb, &outb, &vec, &general);
    if (rc == 1) return CAS_OK;
    if (rc == CAS_ERR_SHAPE) return rc;
    if (!qkv || !row_max || !row_logsum || !y) return CAS_ERR_NULL;
    if (rc != CAS_OK) return rc;
    if ((uintptr_t)row_max % 4 != 0 || (uintptr_t)row_logsum % 4 != 0 || (uintptr_t)y % 4 != 0)
        return CAS_ERR_UNSUPPORTED;
    const int64_t yb = inb / 3 / elem_size(in_dtype) * 4; // (B, T, C) fp32
    if (overlap(y, yb, qkv, inb) || overlap(y, yb, row_max, stb) || overlap(y, yb, row_logsum, stb))
        return CAS_ERR_ALIAS;
    const int dc = device_check();
    if (dc != CAS_OK) return dc;
    cas::TrimulArgs a = softmax_args(qkv, y, row_max, row_logsum, B, T, C, NH, 4, 0);
    const hipStream_t st = (hipStream_t)stream;
    if (general) return launch_status(cas::launch_gen_attention(a, in_dtype, false, st));
    switch (in_dtype) {
    case CAS_F32: return launch_status(cas::launch_attention_f32(a, st));
    case CAS_BF16: return launch_status(cas::launch_attention_bf16(a, st));
    default: return launch_status(cas::launch_attention_f16(a, st));
    }
}

CAS_EXPORT int cas_causal_attention_fused(const void *qkv, void *y, float *row_max, float *row_logsum, int64_t B,
                                          int64_t T, int64_t C, int64_t NH, cas_dtype in_dtype, cas_dtype out_dtype,
                                          void *stream)
{
    if (!dtype_in_ok(in_dtype) || out_dtype != CAS_F32) return CAS_ERR_DTYPE;
    int64_t inb, stb, outb;
    int vec = 1;
    bool general = false;
    const int rc = softmax_checks(qkv, B, T, C, NH, in_dtype, 0, &inb, &stb, &outb, &vec, &general);
    if (rc == 1) return CAS_OK;
    if (rc == CAS_ERR_SHAPE) return rc;
    if (!qkv || !y || !row_max || !row_logsum) return CAS_ERR_NULL;
    if (rc != CAS_OK) return rc;
    if ((uintptr_t)row_max % 4 != 0 || (uintptr_t)row_logsum % 4 != 0 || (uintptr_t)y % 4 != 0)
        return CAS_ERR_UNSUPPORTED;
    const int64_t yb = inb / 3 / elem_size(in_dtype) * 4; // (B, T, C) fp32
    // Three outputs: none may overlap qkv or another output.
    if (overlap(y, yb, qkv, inb) || overlap(row_max, stb, qkv, inb) || overlap(row_logsum, stb, qkv, inb) ||
        overlap(y, yb, row_max, stb) || overlap(y, yb, row_logsum, stb) || overlap(row_max, stb, row_logsum, stb))
        return CAS_ERR_ALIAS;
    const int dc = device_check();
    if (dc != CAS_OK) return dc;
    cas::TrimulArgs a = softmax_args(qkv, y, row_max, row_logsum, B, T, C, NH, 4, 0);
    a.vec_store = (uintptr_t)y % 16 == 0; // rows and head offsets are whole 16-byte pieces (C, HS multiples of 4)
    const hipStream_t st = (hipStream_t)stream;
    if (general) return launch_status(cas::launch_gen_attention(a, in_dtype, true, st));
    switch (in_dtype) {
    case CAS_F32: return launch_status(cas::launch_attention_online_f32(a, st));
    case CAS_BF16: return launch_status(cas::launch_attention_online_bf16(a, st));
    default: return launch_status(cas::launch_attention_online_f16(a, st));
    }
}

CAS_EXPORT const char *cas_status_string(int status)
{
    switch (status) {
    case CAS_OK: return "ok";
    case CAS_ERR_NULL: return "a required pointer is NULL";
    case CAS_ERR_SHAPE: return "invalid shape: negative size, pitch smaller than the row, C % NH != 0, or overflow";
    case CAS_ERR_DTYPE: return "unsupported (in_dtype, out_dtype) pair";
    case CAS_ERR_ALIAS: return "output bytes overlap input bytes";
    case CAS_ERR_DEVICE: return "the current HIP device is not a gfx950 (MI355X) GPU or is unavailable";
    case CAS_ERR_HIP: return "HIP launch failed (see cas_last_hip_error)";
    case CAS_ERR_UNSUPPORTED:
        return "valid arguments outside the kernels' domain (softmax and attention: qkv off the element "
               "alignment, or statistics not 4-byte aligned)";
    case CAS_ERR_MODE: return "unknown softmax mode";
    default: return "unknown status";
    }
}

CAS_EXPORT int cas_last_hip_error(void) { return g_last_hip; }

CAS_EXPORT int cas_version(void) { return 210; }
