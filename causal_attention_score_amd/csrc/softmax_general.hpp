// softmax_general.hpp -- the causal softmax (row statistics, softmax rows) and
// the attention output for QKV rows outside the fast kernels' domain: heads
// whose rows do not split into 16-byte pieces (HS = 3 in fp32, misaligned
// bases) and heads over 512 bytes, of any size: a head row is staged in
// chunks of at most 640 bytes (fp32 160, 16-bit 320 elements), so three
// staged tiles stay within 64 KB of LDS.
//
// Semantics are those of the fast path (smallem "Kernels GPU", its softmax
// section: row_stats reduces a row to its maximum and ln sum exp(x - max),
// kept as two numbers; softmax_rows forms (x - max) - logsum or its
// exponential; the rows are the causal score rows of llm.c trimat_forward.cu,
// trimul_cpu), and so are the formulas: the same exact-residual base-2
// statistics, the same probability epilogue (tri::epilogue), p rounded to the
// input format before the products with V for 16-bit inputs.
//
// Layout. A workgroup is one wave and owns one 32-row query block of one
// (b, nh) plane. The block's Q rows, and per step one 32-row key tile (and
// value tile), are staged into LDS element by element -- any alignment, any
// head size -- as rows zero-padded to a whole number of 32 elements, which
// is a whole number of 32-byte MFMA steps and of 32-column output blocks
// (local padding: the contraction runs over full steps, the zeros add
// nothing). Scores come from MFMAs as D = K Q^T, so lane l holds query
// l % 32 and keys 8g + 4(l / 32) + e of the tile in register 4g + e. A head
// longer than one chunk is taken chunk after chunk, the Q and K chunks
// staged together, the products accumulating in the same registers: the
// same sums in the same order as one whole-row pass.
//
// Statistics take two sweeps over the key tiles: the row maximum of the raw
// dot products mt, then l = sum exp2(a c - ms) against ms = fl(mt c),
// c = scale log2 e, with logsum = (log2 l - (mt c - ms)) ln 2 and the
// residual mt c - ms exact in one fused multiply-add. row_max = fl(mt scale)
// is the largest fp32 score of the row.
//
// The attention output accumulates Y^T = V^T P^T per 32 head columns: the
// P^T operand of an MFMA is the probabilities the lane already holds (the
// keys of its registers are the MFMA's k-slots), the V^T operand is read
// from the staged value rows. Head columns are taken 128 at a time; wider
// heads recompute the scores per group of columns.
#pragma once

#include <type_traits>

#include "launch.hpp"
#include "tile_engine.hpp"
#include "trimul_kernel.hpp"

namespace cas {
namespace gen {

constexpr int GB = 32;          // query rows per workgroup, keys per step
constexpr int GMAX_HEAD = 640;  // bytes of one staged head chunk
constexpr int NDB = 4;          // 32-column blocks of the attention output per pass
constexpr float GLOG2E = 1.44269504088896340736f;
constexpr float GLN2 = 0.693147180559945309417f;

struct GenArgs {
    const char *qkv;
    int64_t B, T, C, NH;
    int HS;
    int hch;       // elements of one staged head chunk: HS rounded up to 32, at most GMAX_HEAD bytes
    int nch;       // chunks per head row
    int hsb;       // bytes of a staged row chunk (hch elements, zero-padded past the head)
    int pitch;     // LDS row pitch: hsb + 16
    uint32_t nqb;  // 32-row query blocks per plane
    float scale;
};

__device__ __forceinline__ float pin(float v)
{
    asm volatile("" : "+v"(v));
    return v;
}

// Elements [e0, e0 + hch) of rows [0, 32) of a head at `base` (row pitch
// ldb bytes; rows at or past `rows` and elements at or past HS become zero)
// -> LDS rows of `pitch` bytes, hsb bytes each.
template <class E>
__device__ __forceinline__ void stage_rows(char *lds, const char *__restrict__ base, int64_t ldb, int rows,
                                           const GenArgs &g, int lane, int e0 = 0)
{
    // Lane l takes elements l, l + 64, .. (M per row at most) of RG rows at a
    // time: all their loads in flight, then the LDS writes (one load, wait
    // and write per element left each load's latency exposed).
    constexpr int ES = E::ES, M = (GMAX_HEAD / ES + 63) / 64, RG = ES == 4 ? 8 : 4;
    using U = typename std::conditional<ES == 4, uint32_t, uint16_t>::type;
    const int nel = g.hsb / ES;
    for (int r0 = 0; r0 < GB; r0 += RG) {
        U v[RG][M];
#pragma unroll
        for (int rr = 0; rr < RG; ++rr)
#pragma unroll
            for (int m = 0; m < M; ++m) {
                const int r = r0 + rr, e = lane + 64 * m;
                const bool ok = r < rows && e < nel && e0 + e < g.HS;
                v[rr][m] = ok ? *reinterpret_cast<const U *>(base + (int64_t)r * ldb + (int64_t)(e0 + e) * ES) : (U)0;
            }
#pragma unroll
        for (int rr = 0; rr < RG; ++rr)
#pragma unroll
            for (int m = 0; m < M; ++m) {
                const int e = lane + 64 * m;
                if (e < nel) *reinterpret_cast<U *>(lds + (r0 + rr) * g.pitch + e * ES) = v[rr][m];
            }
    }
}

// Raw dot products of the staged key tile with the staged query block,
// added to acc: register 4g + e of lane l is key 8g + 4(l / 32) + e against
// query l % 32. Step c takes chunk 2c + h of both rows (h = l / 32, the
// MFMA k-slot).
template <class E>
__device__ __forceinline__ void score_acc(f32x16 &acc, const char *ldk, const char *ldq, const GenArgs &g, int lane)
{
    const int r = lane & 31, h = lane >> 5;
    for (int c = 0; c < g.hsb / 32; ++c) {
        const u32x4 a = *reinterpret_cast<const u32x4 *>(ldk + r * g.pitch + (2 * c + h) * 16);
        const u32x4 b = *reinterpret_cast<const u32x4 *>(ldq + r * g.pitch + (2 * c + h) * 16);
        mfma_chunk<E>(acc, a, b);
    }
}

__device__ __forceinline__ int key_of(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

struct Block {
    int64_t plane, b, nh, t0;
    int qrows;
    const char *q;  // Q row t0 of (b, nh)
    const char *k;  // K row 0 of (b, nh)
    const char *v;  // V row 0 of (b, nh)
    int64_t ldb;    // packed row pitch in bytes
};

template <class E>
__device__ __forceinline__ Block block_of(const GenArgs &g)
{
    constexpr int ES = E::ES;
    Block k;
    k.plane = blockIdx.x / g.nqb;
    const int64_t qb = blockIdx.x - k.plane * g.nqb;
    k.b = k.plane / g.NH;
    k.nh = k.plane - k.b * g.NH;
    k.t0 = qb * GB;
    k.qrows = (int)(g.T - k.t0 < GB ? g.T - k.t0 : GB);
    const int64_t C3 = 3 * g.C;
    k.ldb = C3 * ES;
    const char *row0 = g.qkv + (k.b * g.T * C3 + k.nh * g.HS) * ES; // Q row 0 of (b, nh)
    k.q = row0 + k.t0 * k.ldb;
    k.k = row0 + g.C * ES;
    k.v = row0 + 2 * g.C * ES;
    return k;
}

// Q rows of the block at ldq for the whole launch when the head is one
// chunk; longer heads stage them chunk by chunk with the keys (tile_scores).
template <class E>
__device__ __forceinline__ void stage_queries(char *ldq, const Block &bk, const GenArgs &g, int lane)
{
    if (g.nch == 1) stage_rows<E>(ldq, bk.q, bk.ldb, bk.qrows, g, lane);
}

// Raw dot products of key tile s0 with the block's queries: the K rows (and
// for a head of several chunks the Q rows) staged chunk by chunk, the
// products of every chunk accumulating in the same registers.
template <class E>
__device__ __forceinline__ f32x16 tile_scores(const GenArgs &g, const Block &bk, int64_t s0, char *ldq, char *ldk,
                                              int lane)
{
    const int krows = (int)(g.T - s0 < GB ? g.T - s0 : GB);
    f32x16 acc = {};
    for (int ch = 0; ch < g.nch; ++ch) {
        const int e0 = ch * g.hch;
        __syncthreads();
        if (g.nch > 1) stage_rows<E>(ldq, bk.q, bk.ldb, bk.qrows, g, lane, e0);
        stage_rows<E>(ldk, bk.k + s0 * bk.ldb, bk.ldb, krows, g, lane, e0);
        __syncthreads();
        score_acc<E>(acc, ldk, ldq, g, lane);
    }
    return acc;
}

// The statistics of the lane's query row (two sweeps over key tiles
// 0 .. the block's own): the raw maximum mt, the offset ms = fl(mt c) and
// l = sum exp2(a c - ms), both lane halves combined. Q staged at ldq.
template <class E>
__device__ __forceinline__ void row_stats(const GenArgs &g, const Block &bk, char *ldq, char *ldk, int lane, float &mt,
                                          float &ms, float &l)
{
    const int h = lane >> 5;
    const int64_t t = bk.t0 + (lane & 31);
    const int ntk = (int)(bk.t0 / GB) + 1;
    const float c = g.scale * GLOG2E;
    mt = -__builtin_inff();
    for (int j = 0; j < ntk; ++j) {
        const int64_t s0 = (int64_t)j * GB;
        const f32x16 acc = tile_scores<E>(g, bk, s0, ldq, ldk, lane);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int64_t key = s0 + key_of(r, h);
            if (key <= t && key < g.T) mt = fmaxf(mt, acc[r]);
        }
    }
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    ms = pin(mt * c);
    l = 0.f;
    for (int j = 0; j < ntk; ++j) {
        const int64_t s0 = (int64_t)j * GB;
        const f32x16 acc = tile_scores<E>(g, bk, s0, ldq, ldk, lane);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int64_t key = s0 + key_of(r, h);
            if (key <= t && key < g.T) l += __builtin_amdgcn_exp2f(__builtin_fmaf(acc[r], c, -ms));
        }
    }
    l += __shfl_xor(l, 32);
}

template <class E>
__global__ void __launch_bounds__(64) gen_stats_kernel(GenArgs g, float *__restrict__ row_max,
                                                       float *__restrict__ row_logsum)
{
    extern __shared__ __attribute__((aligned(16))) char glds[];
    const int lane = threadIdx.x;
    const Block bk = block_of<E>(g);
    char *ldq = glds, *ldk = glds + GB * g.pitch;
    stage_queries<E>(ldq, bk, g, lane);
    float mt, ms, l;
    row_stats<E>(g, bk, ldq, ldk, lane, mt, ms, l);
    const int q = lane & 31;
    if (lane < 32 && q < bk.qrows) {
        const float c = g.scale * GLOG2E;
        const int64_t o = bk.plane * g.T + bk.t0 + q;
        row_max[o] = mt * g.scale;
        row_logsum[o] = (__builtin_amdgcn_logf(l) - __builtin_fmaf(mt, c, -ms)) * GLN2;
    }
}

// One element of the output: the value of the epilogue, or the fill.
template <class O, class EP>
__device__ __forceinline__ void put(char *out, int64_t i, float v, bool fill)
{
    if constexpr (O::OB == 4) {
        *reinterpret_cast<uint32_t *>(out + i * 4) = fill ? tri::fill32<EP>() : __float_as_uint(v);
    } else {
        *reinterpret_cast<uint16_t *>(out + i * 2) = (uint16_t)(fill ? tri::fill16<O, EP>() : tri::round16(O{}, v));
    }
}

// Softmax rows of the block: for every key tile, the epilogue on and below
// the diagonal and the fill above it, over the whole (T, T) rows.
template <class E, class O, class EP>
__global__ void __launch_bounds__(64) gen_rows_kernel(GenArgs g, const float *__restrict__ row_max,
                                                      const float *__restrict__ row_logsum, char *__restrict__ out)
{
    extern __shared__ __attribute__((aligned(16))) char glds[];
    const int lane = threadIdx.x, h = lane >> 5;
    const Block bk = block_of<E>(g);
    char *ldq = glds, *ldk = glds + GB * g.pitch;
    stage_queries<E>(ldq, bk, g, lane);
    const int q = lane & 31;
    const int64_t t = bk.t0 + q;
    const bool row_ok = q < bk.qrows;
    const float mx = row_ok ? row_max[bk.plane * g.T + t] : 0.f;
    const float ls = row_ok ? row_logsum[bk.plane * g.T + t] : 0.f;
    const int ntk = (int)((g.T + GB - 1) / GB), own = (int)(bk.t0 / GB);
    const int64_t orow = (bk.plane * g.T + t) * g.T;
    for (int j = 0; j < ntk; ++j) {
        const int64_t s0 = (int64_t)j * GB;
        if (j <= own) {
            const f32x16 acc = tile_scores<E>(g, bk, s0, ldq, ldk, lane);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t key = s0 + key_of(r, h);
                if (row_ok && key < g.T)
                    put<O, EP>(out, orow + key, tri::epilogue<EP>(acc[r], g.scale, mx, ls), key > t);
            }
        } else {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t key = s0 + key_of(r, h);
                if (row_ok && key < g.T) put<O, EP>(out, orow + key, 0.f, true);
            }
        }
    }
}

// 16-bit probability for the MFMA with V (nearest even), and one pair packed.
template <class E> __device__ __forceinline__ uint32_t pack2(float a, float b);
template <> __device__ __forceinline__ uint32_t pack2<KBF16>(float a, float b)
{
    return (uint32_t)__builtin_bit_cast(unsigned short, (__bf16)a) |
           ((uint32_t)__builtin_bit_cast(unsigned short, (__bf16)b) << 16);
}
template <> __device__ __forceinline__ uint32_t pack2<KF16>(float a, float b)
{
    return (uint32_t)__builtin_bit_cast(unsigned short, (_Float16)a) |
           ((uint32_t)__builtin_bit_cast(unsigned short, (_Float16)b) << 16);
}

// Y^T[d][q] += sum over the tile's keys of V[key][d] p[q][key], for the
// nb <= NDB column blocks staged at ldv (the value rows from the pass's
// first column on).
template <class E>
__device__ __forceinline__ void pv_tile(f32x16 (&yt)[NDB], const float (&p)[16], const char *ldv, int nb,
                                        const GenArgs &g, int lane)
{
    const int d = lane & 31, h = lane >> 5;
    if constexpr (E::ES == 4) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const char *vrow = ldv + key_of(r, h) * g.pitch;
#pragma unroll
            for (int i = 0; i < NDB; ++i) {
                if (i >= nb) break; // past the head's last 32-column block
                const float v = *reinterpret_cast<const float *>(vrow + (i * 32 + d) * 4);
                yt[i] = __builtin_amdgcn_mfma_f32_32x32x2f32(v, p[r], yt[i], 0, 0, 0);
            }
        }
    } else {
        // MFMA j takes, in k-slots 8h .. 8h + 7, keys 8(2j + i/4) + 4h + i%4:
        // registers 8j .. 8j + 7 of the scores.
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const u32x4 pb = {pack2<E>(p[8 * j + 0], p[8 * j + 1]), pack2<E>(p[8 * j + 2], p[8 * j + 3]),
                              pack2<E>(p[8 * j + 4], p[8 * j + 5]), pack2<E>(p[8 * j + 6], p[8 * j + 7])};
#pragma unroll
            for (int i = 0; i < NDB; ++i) {
                if (i >= nb) break;
                const int col = (i * 32 + d) * 2;
                uint32_t w[4];
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    const uint32_t lo = *reinterpret_cast<const uint16_t *>(ldv + key_of(8 * j + 2 * x, h) * g.pitch + col);
                    const uint32_t hi =
                        *reinterpret_cast<const uint16_t *>(ldv + key_of(8 * j + 2 * x + 1, h) * g.pitch + col);
                    w[x] = lo | (hi << 16);
                }
                mfma_chunk<E>(yt[i], u32x4{w[0], w[1], w[2], w[3]}, pb);
            }
        }
    }
}

// The attention output of the block, y[b, t, nh HS + d] = sum_{t2 <= t}
// p[t][t2] V[t2][d]; with STATS the row statistics are computed here first
// (and written), else read.
template <class E, bool STATS>
__global__ void __launch_bounds__(64) gen_attention_kernel(GenArgs g, float *__restrict__ row_max,
                                                           float *__restrict__ row_logsum, float *__restrict__ y)
{
    extern __shared__ __attribute__((aligned(16))) char glds[];
    const int lane = threadIdx.x, h = lane >> 5;
    const Block bk = block_of<E>(g);
    char *ldq = glds, *ldk = glds + GB * g.pitch, *ldv = glds + 2 * GB * g.pitch;
    stage_queries<E>(ldq, bk, g, lane);
    const int q = lane & 31;
    const int64_t t = bk.t0 + q;
    const bool row_ok = q < bk.qrows;
    float mx, ls;
    if constexpr (STATS) {
        float mt, ms, l;
        row_stats<E>(g, bk, ldq, ldk, lane, mt, ms, l);
        const float c = g.scale * GLOG2E;
        mx = mt * g.scale;
        ls = (__builtin_amdgcn_logf(l) - __builtin_fmaf(mt, c, -ms)) * GLN2;
        if (lane < 32 && row_ok) {
            row_max[bk.plane * g.T + t] = mx;
            row_logsum[bk.plane * g.T + t] = ls;
        }
    } else {
        mx = row_ok ? row_max[bk.plane * g.T + t] : 0.f;
        ls = row_ok ? row_logsum[bk.plane * g.T + t] : 0.f;
    }
    const int ntk = (int)(bk.t0 / GB) + 1;
    const int ndb = (g.HS + 31) / 32;
    for (int db0 = 0; db0 < ndb; db0 += NDB) {
        f32x16 yt[NDB];
#pragma unroll
        for (int i = 0; i < NDB; ++i) yt[i] = f32x16{};
        for (int j = 0; j < ntk; ++j) {
            const int64_t s0 = (int64_t)j * GB;
            const int krows = (int)(g.T - s0 < GB ? g.T - s0 : GB);
            // the value rows' columns of this pass (hch >= NDB * 32 whenever
            // the head needs more than one pass), then the scores, whose
            // first barrier also orders these writes after the last pass's reads
            __syncthreads();
            stage_rows<E>(ldv, bk.v + s0 * bk.ldb, bk.ldb, krows, g, lane, db0 * 32);
            const f32x16 acc = tile_scores<E>(g, bk, s0, ldq, ldk, lane);
            float p[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t key = s0 + key_of(r, h);
                p[r] = (key <= t && key < g.T) ? tri::epilogue<tri::EpProb>(acc[r], g.scale, mx, ls) : 0.f;
            }
            pv_tile<E>(yt, p, ldv, ndb - db0 < NDB ? ndb - db0 : NDB, g, lane);
        }
        // lane: query q, head columns 32 (db0 + i) + 8(r/4) + 4h + r%4
        if (row_ok) {
            float *yrow = y + (bk.b * g.T + t) * g.C + bk.nh * g.HS;
#pragma unroll
            for (int i = 0; i < NDB; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int d = (db0 + i) * 32 + key_of(r, h);
                    if (d < g.HS) yrow[d] = yt[i][r]; // blocks past the head hold zeros, never written
                }
        }
    }
}

} // namespace gen
} // namespace cas
