// softmax_kernel.hpp -- causal softmax straight from packed QKV on gfx950.
//
// Semantics: the softmax in two launches of the smallem page "Kernels GPU"
// (row_stats, then softmax_rows), over the causal score rows of llm.c
// trimat_forward.cu's trimul_cpu (the Referee of Chapter I):
//   row_stats    row_max[t]    = max_{t2 <= t} x[t][t2]
//                row_logsum[t] = ln sum_{t2 <= t} exp(x[t][t2] - row_max[t])
//   softmax_rows log-probability (x - row_max) - row_logsum, or its exponential
// with x the fp32 score of the score kernel. The two reductions stay two
// numbers, as the page recommends: folding the small log-sum into a large
// maximum loses its digits.
//
// Neither launch reads or writes the (T, T) scores: both recompute Q K^T from
// the packed rows. The row-stats kernel below writes 8 bytes per row; the
// softmax rows are the three-role score kernel (trimul_kernel.hpp) with the
// EpLog / EpProb epilogue, whose loader waves stage the statistics of the
// rows they fetch.
//
// Row-stats kernel design:
//  * A workgroup owns one 128-row query block I of one (b, nh) plane (key
//    tiles 0..I). Workgroups are numbered longest block first, and the
//    dispatcher hands them out in index order, so the short blocks fill the
//    last round (longest_first below).
//  * Four waves, wave w owns query rows 32w..32w+31 of the block. Its Q
//    fragments stay in registers for the whole block; the 128 K rows of each
//    step are fetched by all four waves (coalesced 16-byte loads, issued a
//    step ahead) into a double-buffered LDS tile.
//  * D = K Q^T per 32-row key block, so a lane holds 16 scores of ONE query
//    row (column lane%32) and the two lane halves split the keys. Each lane
//    keeps a running maximum and a running sum for its row; the halves merge
//    once at the end.
//  * The running sum is kept in base 2 against the rounded offset
//    ms = fl(m * c), c = scale * log2(e): terms are exp2(fma(a, c, -ms)) from
//    the raw dot product a, earlier sums are rescaled by exp2(ms_old - ms),
//    and the final log-sum subtracts the exact residual m * c - ms (one fma).
//    The log-sum then carries no error of order ulp(m * c), which for
//    saturated rows (|m| in the hundreds) would otherwise dominate.
#pragma once

#include "trimul_kernel.hpp"

namespace cas {
namespace sm {

using tri::OOB;
using tri::rsrc_at;
using tri::ST;

constexpr int SW = 4; // waves per row-stats workgroup
constexpr int STATS_THREADS = SW * 64;
constexpr float LOG2E = 1.44269504088896340736f;
constexpr float LN2 = 0.693147180559945309417f;

// Position (bytes) of 16-byte chunk c of row r inside its LDS row of NCH
// chunks. ds_read_b128 serves 16 lanes at a time from 256 bytes of banks;
// the MFMA operand read takes one chunk of 16 consecutive rows, and the
// staging write takes whole rows. XOR-ing the chunk with (row / rows per 256
// bytes) makes both touch 16 distinct 16-byte bank groups.
template <int NCH> __device__ __forceinline__ uint32_t kswz(uint32_t r, uint32_t c)
{
    constexpr uint32_t SH = NCH == 8 ? 1 : 0;
    return (c ^ ((r >> SH) & (NCH - 1))) << 4;
}

typedef __attribute__((address_space(3))) void lds_void;

// A buffer resource over `rows` rows of pitch ldb from base: loads past them read zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_rows(const char *base, uint32_t rows, uint32_t ldb)
{
    // Uniform, and visibly so (a saturating subtract for rows would otherwise
    // put the size in a vector register and each load in a waterfall loop).
    const uint64_t n = (uint64_t)rows * ldb;
    const int size = __builtin_amdgcn_readfirstlane(n < 0x7FFFFFFFu ? (int)n : 0x7FFFFFFF);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(base), (short)0, size, 0x00020000);
}

// The 128 K rows of key tile J (rows J*128.. of the plane) go from HBM
// straight into LDS: buffer loads with an LDS destination, one kilobyte per
// wave instruction (lane i fills bytes 16i .. 16i + 15 of it), so each lane
// fetches the global chunk that belongs at its LDS position (chunk c of row r
// at kswz(r, c); the XOR is an involution). Wave w fills kilobytes
// w NCH/2 .. of the tile. Rows past T read zero through the size of the
// tile's buffer resource, chunks past the head through an out-of-range offset.
template <int NCH> struct KDirect {
    uint32_t vo[NCH / 2]; // per lane: offset within the tile's rows of each of its loads
};

template <int NCH>
__device__ __forceinline__ void kd_init(KDirect<NCH> &st, int w, int lane, uint32_t ldb, uint32_t head_bytes)
{
    constexpr uint32_t RB = NCH * 16, PER = NCH / 2, SH = NCH == 8 ? 1 : 0;
#pragma unroll
    for (int q = 0; q < (int)PER; ++q) {
        const uint32_t o = ((uint32_t)w * PER + (uint32_t)q) * 1024u + 16u * (uint32_t)lane;
        const uint32_t r = o / RB, p = (o % RB) / 16u;
        const uint32_t c = p ^ ((r >> SH) & (NCH - 1));
        st.vo[q] = c * 16u < head_bytes ? r * ldb + c * 16u : OOB;
    }
}

template <int NCH>
__device__ __forceinline__ void kd_fetch(const KDirect<NCH> &st, char *dst, const char *kb0, uint32_t J, uint32_t T,
                                         uint32_t ldb, int w)
{
    constexpr uint32_t PER = NCH / 2;
    const uint32_t k0 = J * ST, rows = k0 < T ? T - k0 : 0u;
    const __amdgpu_buffer_rsrc_t rk = rsrc_rows(kb0 + (uint64_t)k0 * ldb, rows, ldb);
#pragma unroll
    for (int q = 0; q < (int)PER; ++q)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void *)(dst + ((uint32_t)w * PER + (uint32_t)q) * 1024u), 16,
                                                 (int)st.vo[q], 0, 0, 0);
}

// acc[kb] += K rows 32kb.. of the LDS tile times this wave's Q rows: lane
// (r32, h) supplies chunk 2u + h of K row 32kb + r32 and of its Q row (the
// same chunk permutation on both operands, so each product appears once).
// NQ: the chunk pairs multiplied (fewer than NCH / 2 when the rest of the
// head row is zero: heads of 257 .. 384 bytes on 32-chunk rows take 12).
template <class E, int NCH, int NQ = NCH / 2>
__device__ __forceinline__ void k_mma(f32x16 (&acc)[4], const char *kb, const u32x4 (&qf)[NCH / 2], int lane)
{
    constexpr int RB = NCH * 16;
    const uint32_t r32 = (uint32_t)(lane & 31), h = (uint32_t)(lane >> 5);
#pragma unroll
    for (int u = 0; u < NQ; ++u) {
        u32x4 kf[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const uint32_t row = 32u * b + r32;
            kf[b] = *reinterpret_cast<const u32x4 *>(kb + row * RB + kswz<NCH>(row, 2u * u + h));
        }
#pragma unroll
        for (int b = 0; b < 4; ++b) mfma_chunk<E>(acc[b], kf[b], qf[u]);
    }
}

// A rounded fp32 value the compiler may not look through: the offsets
// ms = fl(m * c) must stay the rounded products the terms were built
// against, not be fused (fp-contract) into a later subtraction.
__device__ __forceinline__ float pinned(float v)
{
    asm volatile("" : "+v"(v));
    return v;
}

// Running statistics of one lane's query row over the keys it has seen:
// m the largest raw dot product (-inf before any), ms = fl(m * c) (0 while
// m = -inf), l = sum exp2(a * c - ms).
struct RowRun {
    float m, ms, l;
};

// Fold a step's accumulators into the lane's running statistics. Blocks
// b < NB take part whole; block NB (if NB < 4) with the keys after the lane's
// row masked: accumulator (b, r) is key 32b + 8(r/4) + 4h + r%4 of the step,
// against query row 32w + lane%32. NB = 4: an off-diagonal step, nothing
// masked. The diagonal step of wave w is NB = w: its blocks after w hold only
// later keys and are skipped. Two passes over the accumulators (maximum,
// then the sum), so no copy of them is kept.
template <int NB>
__device__ __forceinline__ void stats_update(const f32x16 (&acc)[4], RowRun &rr, float c, int lane)
{
    const int r32 = lane & 31, h4 = 4 * (lane >> 5);
    float v[16]; // block NB, masked
    if constexpr (NB < 4) {
#pragma unroll
        for (int r = 0; r < 16; ++r) v[r] = 8 * (r >> 2) + h4 + (r & 3) > r32 ? -__builtin_inff() : acc[NB][r];
    }
    float mx = -__builtin_inff();
#pragma unroll
    for (int b = 0; b < NB && b < 4; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, acc[b][r]);
    if constexpr (NB < 4) {
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, v[r]);
    }
    const float mn = fmaxf(rr.m, mx);
    const float msn = mn == -__builtin_inff() ? 0.f : pinned(mn * c);
    float s = 0.f;
#pragma unroll
    for (int b = 0; b < NB && b < 4; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) s += __builtin_amdgcn_exp2f(fmaf(acc[b][r], c, -msn));
    if constexpr (NB < 4) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s += __builtin_amdgcn_exp2f(fmaf(v[r], c, -msn)); // exp2(-inf) = 0
    }
    const float alpha = rr.m == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(rr.ms - msn);
    rr.l = rr.l * alpha + s;
    rr.m = mn;
    rr.ms = msn;
}

// Query blocks in decreasing length: block I of a plane has I + 1 (or
// 2I + 2) key tiles, and workgroups are dispatched in index order, so
// giving the low indices the long blocks lets the short ones fill in behind
// them (no pairing needed). Workgroup index (rank - rank0) * planes + plane
// takes block I = nt - 1 - rank of that plane.
struct BlockIdx { uint32_t plane, I; };
__device__ __forceinline__ BlockIdx longest_first(uint32_t planes, uint32_t rank0, uint32_t nt)
{
    const uint32_t q = blockIdx.x / planes;
    return BlockIdx{blockIdx.x - q * planes, nt - 1 - (rank0 + q)};
}

// Launches of planes x ranks workgroups, ranks split so that a grid stays
// below 2^32 work-items (STATS_THREADS per workgroup; planes < 2^23).
template <class F> hipError_t launch_longest_first(const TrimulArgs &a, hipStream_t s, F &&launch)
{
    const int64_t nt = (a.T + ST - 1) / ST;
    const int64_t planes = a.B * a.NH;
    const int64_t per = std::max<int64_t>(1, ((int64_t)1 << 23) / planes);
    for (int64_t r0 = 0; r0 < nt; r0 += per) {
        const int64_t n = std::min(per, nt - r0);
        launch(dim3((unsigned)(planes * n)), (uint32_t)nt, (uint32_t)planes, (uint32_t)r0);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

template <class E, int NCH, int NQ = NCH / 2>
__global__ void __launch_bounds__(STATS_THREADS)
row_stats_kernel(const char *__restrict__ qkv, float *__restrict__ row_max, float *__restrict__ row_logsum,
                 uint32_t T, uint32_t C, uint32_t NH, uint32_t HS, uint32_t nt, uint32_t planes, uint32_t rank0,
                 float scale)
{
    constexpr int RB = NCH * 16, NU = NCH / 2;
    // Two named buffers (and the loop unrolled by two) so that every LDS read
    // names its buffer: the compiler then knows the loads in flight write the
    // other one and does not wait for them before the reads.
    __shared__ __attribute__((aligned(16))) char k0s[ST * RB];
    __shared__ __attribute__((aligned(16))) char k1s[ST * RB];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const uint32_t r32 = (uint32_t)(lane & 31), h = (uint32_t)(lane >> 5);

    const BlockIdx bi = longest_first(planes, rank0, nt);
    const uint32_t plane = bi.plane, I = bi.I;
    const uint32_t b = plane / NH, nh = plane - b * NH;
    const uint32_t ldb = 3u * C * (uint32_t)E::ES;
    const uint32_t head_bytes = HS * (uint32_t)E::ES;
    const char *qb0 = qkv + ((uint64_t)b * T * (3u * C) + (uint64_t)nh * HS) * E::ES; // Q row 0 of the plane
    const char *kb0 = qb0 + (uint64_t)C * E::ES;                                     // K row 0
    const float c = scale * LOG2E;

    {
        const uint32_t t0 = I * ST;

        // Q fragments of rows t0 + 32w + r32: chunk 2u + h.
        u32x4 qf[NU];
        {
            const __amdgpu_buffer_rsrc_t rq = rsrc_at(qb0 + (uint64_t)t0 * ldb);
            const uint32_t row = 32u * w + r32;
            const bool row_ok = t0 + row < T;
#pragma unroll
            for (int u = 0; u < NQ; ++u) {
                const uint32_t ch = 2u * u + h;
                const uint32_t vo = (row_ok && ch * 16 < head_bytes) ? row * ldb + ch * 16 : OOB;
                qf[u] = __builtin_amdgcn_raw_buffer_load_b128(rq, (int)vo, 0, 0);
            }
        }

        RowRun rr{-__builtin_inff(), 0.f, 0.f};
        KDirect<NCH> kd;
        kd_init<NCH>(kd, w, lane, ldb, head_bytes);
        kd_fetch<NCH>(kd, k0s, kb0, 0, T, ldb, w);
        // Every load so far (Q fragments included) has landed: the loop's
        // waits then only ever concern the key tile fetched a step ahead.
        __builtin_amdgcn_s_waitcnt(0x70); // vmcnt(0) lgkmcnt(0)
        tri::lds_barrier();
        // Key tiles left of the diagonal (nothing masked): tile J in k<J % 2>,
        // tile J + 1 loading into the other buffer meanwhile.
        auto step = [&](const char *cur, char *next, uint32_t J) {
            kd_fetch<NCH>(kd, next, kb0, J + 1, T, ldb, w);
            f32x16 acc[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) acc[k] = f32x16{};
            k_mma<E, NCH, NQ>(acc, cur, qf, lane);
            stats_update<4>(acc, rr, c, lane);
            __builtin_amdgcn_s_waitcnt(0x70); // this wave's part of tile J + 1 in LDS
            tri::lds_barrier();                 // every wave's part; tile J's reads done before it is rewritten
        };
        uint32_t J = 0;
        for (;;) {
            if (J >= I) break;
            step(k0s, k1s, J++);
            if (J >= I) break;
            step(k1s, k0s, J++);
        }
        {   // the diagonal tile J = I (no loads in flight: the buffer may be chosen at run time)
            f32x16 acc[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) acc[k] = f32x16{};
            k_mma<E, NCH, NQ>(acc, (I & 1) ? k1s : k0s, qf, lane);
            switch (w) {
            case 0: stats_update<0>(acc, rr, c, lane); break;
            case 1: stats_update<1>(acc, rr, c, lane); break;
            case 2: stats_update<2>(acc, rr, c, lane); break;
            default: stats_update<3>(acc, rr, c, lane); break;
            }
        }

        // Merge the two lane halves (the same row, disjoint keys) and write.
        const float m2 = __shfl_xor(rr.m, 32), ms2 = __shfl_xor(rr.ms, 32), l2 = __shfl_xor(rr.l, 32);
        const float mm = fmaxf(rr.m, m2);
        const float msm = pinned(mm * c); // row 0 always holds key 0, so mm is finite
        const float la = rr.m == -__builtin_inff() ? 0.f : rr.l * __builtin_amdgcn_exp2f(rr.ms - msm);
        const float lb = m2 == -__builtin_inff() ? 0.f : l2 * __builtin_amdgcn_exp2f(ms2 - msm);
        const float resid = fmaf(mm, c, -msm); // m * c - fl(m * c), exact
        const uint32_t t = t0 + 32u * w + r32;
        if (h == 0 && t < T) {
            const uint64_t o = (uint64_t)plane * T + t;
            row_max[o] = mm * scale;
            row_logsum[o] = (__builtin_amdgcn_logf(la + lb) - resid) * LN2;
        }
    }
}

// ---------------------------------------------------------------------------
// Fused kernel: both launches in one. The three roles of the score kernel
// (loader, compute, store waves; trimul_kernel.hpp) walk whole 128-row query
// blocks. A block I takes 2 (I + 1) steps over key tiles 0..I: first the
// statistics phase, where the compute waves fold their sub-tile's scores into
// running statistics and nothing is stored, then the output phase, where they
// write (x - max) - logsum (or its exponential) and the store waves stream it
// with the mirror tiles, as for the scores. The statistics phase is vector-ALU
// work with no HBM traffic of its own, so it runs while other workgroups'
// store streams keep HBM busy, instead of being a launch of its own.
//
// Compute wave (sa, sb) holds query rows 64sa + 32qb + lane%32 (qb = 0, 1)
// against keys 64sb.. of each super-tile. Per row, its two lane halves, then
// the two waves sb = 0, 1 (through LDS), merge at the end of the statistics
// phase; both waves of a pair then hold the final statistics in registers.
// The store waves write them to row_max / row_logsum.
//
// Row blocks are dealt per XCD: XCD x owns planes [P x / 8, P (x+1) / 8) and
// its nw workgroups take that range's blocks sorted longest first (position k
// is block nt - 1 - k / P_x of plane base + k % P_x), in snake order: round r
// gives workgroup w position r nw + w (r even) or r nw + nw - 1 - w (r odd).
// Blocks differ in length (I + 1 tiles), and the snake keeps every
// workgroup's total close to the mean. Each workgroup walks its rounds
// starting from a different one (see FWalk::decode).
// ---------------------------------------------------------------------------
struct FWalk {
    uint32_t nw, w, px, pbase, nt, nblk, rounds; // fixed per workgroup
    uint32_t i, plane, I, J;
    bool out_phase, valid;

    // Round i of this workgroup's walk is round (i + w) % rounds of the deal:
    // the workgroup still takes the same blocks, but neighbours start on
    // blocks of different lengths, so their statistics phases (no stores)
    // drift apart instead of all workgroups pausing their stores together.
    __device__ __forceinline__ void decode()
    {
        valid = i < rounds;
        const uint32_t r = valid ? (i + w) % rounds : 0;
        const uint32_t k = r * nw + ((r & 1) ? nw - 1 - w : w);
        if (valid) {
            const uint32_t rank = k / px;
            I = nt - 1 - rank;
            plane = pbase + (k - rank * px);
        }
        J = 0;
        out_phase = false;
    }
    __device__ __forceinline__ void init(uint32_t P, uint32_t nt_)
    {
        const uint32_t nwg = gridDim.x, x = blockIdx.x % 8, q8 = nwg / 8, r8 = nwg % 8;
        nw = q8 + (x < r8 ? 1u : 0u);
        w = blockIdx.x / 8;
        pbase = (uint32_t)((uint64_t)P * x / 8);
        px = (uint32_t)((uint64_t)P * (x + 1) / 8) - pbase;
        nt = nt_;
        nblk = px * nt;
        // rounds whose position exists for this workgroup: the full ones, and
        // the last partial one if its position falls inside
        const uint32_t full = nblk / nw, rem = nblk - full * nw;
        rounds = full + (((full & 1) ? nw - 1 - w : w) < rem ? 1u : 0u);
        i = 0;
        decode();
    }
    __device__ __forceinline__ void advance()
    {
        if (J < I) {
            ++J;
        } else if (!out_phase) {
            out_phase = true;
            J = 0;
        } else {
            ++i;
            decode();
        }
    }
    __device__ __forceinline__ tri::Super item() const
    {
        tri::Super sp;
        sp.plane = plane;
        sp.T0 = I * ST;
        sp.S0 = J * ST;
        sp.diag = J == I;
        return sp;
    }
};

// Running statistics of a compute lane's two query rows (qb = 0, 1).
struct Run2 {
    float m[2], ms[2], l[2];
};

// Fold sub-tile scores acc[kb][qb] (keys 32kb + 8(r/4) + 4h + r%4, query
// 32qb + lane%32, both within the sub-tile) into the running statistics.
// DIAG: a sub-tile on the diagonal, whose keys after the query are left out.
template <bool DIAG>
__device__ __forceinline__ void sub_stats_update(const f32x16 (&acc)[2][2], Run2 &rn, float c, int lane)
{
    const int r32 = lane & 31, h4 = 4 * (lane >> 5);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        auto masked = [&](int kb, int r) { return DIAG && 32 * kb + 8 * (r >> 2) + h4 + (r & 3) > 32 * qb + r32; };
        float mx = -__builtin_inff();
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = masked(kb, r) ? mx : fmaxf(mx, acc[kb][qb][r]);
        const float mn = fmaxf(rn.m[qb], mx);
        const float msn = mn == -__builtin_inff() ? 0.f : pinned(mn * c);
        float s = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float e = __builtin_amdgcn_exp2f(fmaf(acc[kb][qb][r], c, -msn));
                s += masked(kb, r) ? 0.f : e;
            }
        const float alpha = rn.m[qb] == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(rn.ms[qb] - msn);
        rn.l[qb] = rn.l[qb] * alpha + s;
        rn.m[qb] = mn;
        rn.ms[qb] = msn;
    }
}

// Merge statistics (m2, ms2, l2) into (m, ms, l): the larger maximum wins and
// both sums are rescaled to its rounded offset.
__device__ __forceinline__ void stats_merge(float &m, float &ms, float &l, float m2, float ms2, float l2, float c)
{
    const float mm = fmaxf(m, m2);
    const float msm = mm == -__builtin_inff() ? 0.f : pinned(mm * c);
    const float la = m == -__builtin_inff() ? 0.f : l * __builtin_amdgcn_exp2f(ms - msm);
    const float lb = m2 == -__builtin_inff() ? 0.f : l2 * __builtin_amdgcn_exp2f(ms2 - msm);
    m = mm;
    ms = msm;
    l = la + lb;
}

template <class E, int NCH, class O, class EP>
__global__ void __launch_bounds__(tri::SUPER_THREADS)
softmax_fused_kernel(const char *__restrict__ qkv, char *__restrict__ out, float *__restrict__ row_max,
                     float *__restrict__ row_logsum, uint32_t T, uint32_t C, uint32_t NH, uint32_t HS, uint32_t P,
                     uint32_t nt, float scale, int vec_store)
{
    using namespace tri;
    constexpr int RB = NCH * 16;
    constexpr int PITCH = out_pitch<O>(), OUT_BYTES = TB * PITCH;
    __shared__ __attribute__((aligned(16))) char opb[OP_ROWS * RB];
    __shared__ __attribute__((aligned(16))) char outb[NCOMP * OUT_BYTES];
    __shared__ float part[NCOMP][3][64]; // per compute wave: m, ms, l of its 64 rows (lane-merged)
    __shared__ float stb[2 * ST];        // final statistics of the block: [0, 128) max, [128, 256) logsum

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int role = wave / NCOMP; // 0 compute, 1 store, 2 loader
    const int slot = wave % NCOMP;
    const int sa = slot >> 1, sb = slot & 1;
    char *my_out = outb + slot * OUT_BYTES;
    const uint32_t TBY = T * (uint32_t)O::OB;
    const uint32_t ldb = 3u * C * (uint32_t)E::ES;
    const bool vec = vec_store != 0;
    const float c = scale * LOG2E;

    FWalk cur;
    cur.init(P, nt);

    // Every wave passes the same barriers: one after the prologue, then X and
    // Y once per step, for as many steps as the walk has.
    if (role == 2) {
        const int cl = slot * 64 + lane;
        Staged<NCH> st;
        if (cur.valid) {
            stage_fetch<E, NCH>(st, qkv, cur.item(), T, C, NH, HS, ldb, cl);
            stage_store<NCH>(st, opb, cl);
        }
        lds_barrier();
        while (cur.valid) {
            // Every step of a block has the block's 128 Q rows: they stay in
            // LDS, and only a new block's are fetched.
            const Super was = cur.item();
            cur.advance();
            const bool more = cur.valid;
            bool with_q = true;
            if (more) {
                const Super nx = cur.item();
                with_q = !(nx.plane == was.plane && nx.T0 == was.T0);
                stage_fetch<E, NCH>(st, qkv, nx, T, C, NH, HS, ldb, cl, with_q);
            }
            lds_barrier(); // X: operand rows of this step consumed
            if (more) stage_store<NCH>(st, opb, cl, with_q);
            lds_barrier(); // Y: operand rows of the next step in LDS
        }
    } else if (role == 0) {
        const int r32 = lane & 31;
        Run2 rn;
        float mx[2] = {0.f, 0.f}, ls[2] = {0.f, 0.f};
        lds_barrier();
        while (cur.valid) {
            const Super sp = cur.item();
            const bool out_phase = cur.out_phase, first_out = out_phase && cur.J == 0;
            const bool last_stats = !out_phase && cur.J == cur.I;
            cur.advance();
            if (!out_phase && sp.S0 == 0) { // a new block: statistics start empty
#pragma unroll
                for (int qb = 0; qb < 2; ++qb) {
                    rn.m[qb] = -__builtin_inff();
                    rn.ms[qb] = 0.f;
                    rn.l[qb] = 0.f;
                }
            }
            if (first_out) { // the partner wave's statistics (written before the last Y) complete the rows
                const int ps = sa * 2 + (1 - sb);
#pragma unroll
                for (int qb = 0; qb < 2; ++qb) {
                    const int row = 32 * qb + r32;
                    stats_merge(rn.m[qb], rn.ms[qb], rn.l[qb], part[ps][0][row], part[ps][1][row], part[ps][2][row], c);
                    mx[qb] = rn.m[qb] * scale;
                    ls[qb] = (__builtin_amdgcn_logf(rn.l[qb]) - fmaf(rn.m[qb], c, -rn.ms[qb])) * LN2;
                    if (sb == 0 && lane < 32) {
                        stb[64 * sa + row] = mx[qb];
                        stb[ST + 64 * sa + row] = ls[qb];
                    }
                }
            }
            // Diagonal sub-tile (0, 1) lies wholly above the diagonal: no work.
            const bool live = !(sp.diag && sa == 0 && sb == 1);
            f32x16 acc[2][2];
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int b = 0; b < 2; ++b) acc[a][b] = f32x16{};
            if (live) sub_mma<E, NCH>(acc, opb, sa, sb, lane);
            lds_barrier(); // X: operand rows consumed, previous tile read back
            if (out_phase) {
                if (live) {
                    if (sp.diag && sa == sb) subtile_to_lds<true, O, EP>(acc, my_out, scale, lane, mx, ls);
                    else subtile_to_lds<false, O, EP>(acc, my_out, scale, lane, mx, ls);
                }
            } else {
                if (live) {
                    if (sp.diag && sa == sb) sub_stats_update<true>(acc, rn, c, lane);
                    else sub_stats_update<false>(acc, rn, c, lane);
                }
                if (last_stats) { // merge the lane halves, publish for the partner wave
#pragma unroll
                    for (int qb = 0; qb < 2; ++qb) {
                        stats_merge(rn.m[qb], rn.ms[qb], rn.l[qb], __shfl_xor(rn.m[qb], 32),
                                    __shfl_xor(rn.ms[qb], 32), __shfl_xor(rn.l[qb], 32), c);
                        if (lane < 32) {
                            part[slot][0][32 * qb + r32] = rn.m[qb];
                            part[slot][1][32 * qb + r32] = rn.ms[qb];
                            part[slot][2][32 * qb + r32] = rn.l[qb];
                        }
                    }
                }
            }
            lds_barrier(); // Y: tile in LDS / partial statistics in LDS
        }
    } else {
        lds_barrier();
        Tile pm; // mirror of the previous output step, second half pending
        bool pm_live = false, pm_full = false;
        while (cur.valid) {
            const Super sp = cur.item();
            const bool out_phase = cur.out_phase, first_out = out_phase && cur.J == 0;
            cur.advance();
            const Tile tl = sub_tile<O>(sp, sa, sb, out, T);
            const bool inside = tl.rl > 0 && tl.cl > 0;
            const uint32_t tby = opaque_s(TBY);
            const bool full = tl.rl == TB && tl.cl == TB;
            lds_barrier(); // X
            if (pm_live) {
                if (pm_full) nan_mirror_o<1, O, true, EP>(pm, T, tby, lane, vec);
                else nan_mirror_o<1, O, false, EP>(pm, T, tby, lane, vec);
            }
            pm_live = false;
            if (first_out) { // the block's statistics, written by the compute waves before X
                const int cl = slot * 64 + lane;
                const uint32_t row = sp.T0 + (uint32_t)(cl & (ST - 1));
                if (row < T) (cl < ST ? row_max : row_logsum)[(uint64_t)sp.plane * T + row] = stb[cl];
            }
            lds_barrier(); // Y: tile in LDS
            if (!out_phase || !inside) continue;
            stream_subtile<O, EP>(tl, sp.diag && sa == 0 && sb == 1, full, vec, my_out, T, tby, lane);
            if (!tl.diag) { // first half of the mirror now, the second after the next X
                pm = tl;
                pm_live = true;
                pm_full = full && vec;
                if (pm_full) nan_mirror_o<0, O, true, EP>(tl, T, tby, lane, vec);
                else nan_mirror_o<0, O, false, EP>(tl, T, tby, lane, vec);
            }
        }
        if (pm_live) {
            const uint32_t tby = opaque_s(TBY);
            if (pm_full) nan_mirror_o<1, O, true, EP>(pm, T, tby, lane, vec);
            else nan_mirror_o<1, O, false, EP>(pm, T, tby, lane, vec);
        }
    }
}

// ---------------------------------------------------------------------------
// Pipelined fused launch (16-bit inputs, heads of at most 128 bytes). The
// walk of softmax_fused_kernel runs each block's statistics steps and then its
// output steps; in the statistics steps nothing is stored. Here a step carries
// up to two items: an output tile of block k and a statistics tile of block
// k + 1, so the statistics of the next block are folded while the store
// waves stream the current one's rows. Both items' Q and K rows sit in LDS
// (two operand buffers: 2 x 32 KB at 128-byte heads). The statistics cursor
// runs at most one block ahead of the output cursor, and a block's output
// starts only after its statistics are complete (PWalk).
// ---------------------------------------------------------------------------
struct PWalk {
    uint32_t nw, w, px, pbase, nt, rounds; // the deal, as in FWalk
    uint32_t si, sJ, sPlane, sI;           // statistics cursor: block si, step sJ
    uint32_t oi, oJ, oPlane, oI;           // output cursor
    bool has_st, has_out;                  // this step's items

    __device__ __forceinline__ void block(uint32_t i, uint32_t &plane, uint32_t &I) const
    {
        const uint32_t r = i < rounds ? (i + w) % rounds : 0;
        const uint32_t k = r * nw + ((r & 1) ? nw - 1 - w : w);
        const uint32_t rank = k / px;
        I = nt - 1 - rank;
        plane = pbase + (k - rank * px);
    }
    __device__ __forceinline__ void flags()
    {
        has_out = oi < rounds && si > oi;           // statistics of block oi complete
        has_st = si < rounds && si <= oi + 1;       // at most one block ahead
    }
    __device__ __forceinline__ void init(uint32_t P, uint32_t nt_)
    {
        const uint32_t nwg = gridDim.x, x = blockIdx.x % 8, q8 = nwg / 8, r8 = nwg % 8;
        nw = q8 + (x < r8 ? 1u : 0u);
        w = blockIdx.x / 8;
        pbase = (uint32_t)((uint64_t)P * x / 8);
        px = (uint32_t)((uint64_t)P * (x + 1) / 8) - pbase;
        nt = nt_;
        const uint32_t nblk = px * nt, full = nblk / nw, rem = nblk - full * nw;
        rounds = full + (((full & 1) ? nw - 1 - w : w) < rem ? 1u : 0u);
        si = sJ = oi = oJ = 0;
        sPlane = sI = 0;
        if (rounds > 0) block(0, sPlane, sI); // px = 0 (an XCD without planes) gives no rounds
        oPlane = sPlane;
        oI = sI;
        flags();
    }
    __device__ __forceinline__ bool valid() const { return oi < rounds; }
    __device__ __forceinline__ void advance()
    {
        if (has_st && ++sJ > sI) {
            ++si;
            sJ = 0;
            if (si < rounds) block(si, sPlane, sI);
        }
        if (has_out && ++oJ > oI) {
            ++oi;
            oJ = 0;
            if (oi < rounds) block(oi, oPlane, oI);
        }
        flags();
    }
    __device__ __forceinline__ tri::Super st_item() const
    {
        tri::Super sp;
        sp.plane = sPlane;
        sp.T0 = sI * ST;
        sp.S0 = sJ * ST;
        sp.diag = sJ == sI;
        return sp;
    }
    __device__ __forceinline__ tri::Super out_item() const
    {
        tri::Super sp;
        sp.plane = oPlane;
        sp.T0 = oI * ST;
        sp.S0 = oJ * ST;
        sp.diag = oJ == oI;
        return sp;
    }
};

// SPLIT: four more waves (1024 threads). The statistics items go to waves
// 12 .. 15 and the compute waves keep the output items, so the two run side
// by side on each SIMD instead of one after the other in one wave; the
// arithmetic and its order are unchanged.
template <class E, class O, class EP, bool SPLIT>
__global__ void __launch_bounds__(SPLIT ? tri::SUPER_THREADS + tri::NCOMP_THREADS : tri::SUPER_THREADS)
softmax_pipe_kernel(const char *__restrict__ qkv, char *__restrict__ out, float *__restrict__ row_max,
                    float *__restrict__ row_logsum, uint32_t T, uint32_t C, uint32_t NH, uint32_t HS, uint32_t P,
                    uint32_t nt, float scale, int vec_store)
{
    using namespace tri;
    constexpr int NCH = 8, RB = NCH * 16;
    constexpr int PITCH = out_pitch<O>(), OUT_BYTES = TB * PITCH;
    __shared__ __attribute__((aligned(16))) char opb_st[OP_ROWS * RB];  // operand rows of the statistics item
    __shared__ __attribute__((aligned(16))) char opb_out[OP_ROWS * RB]; // operand rows of the output item
    __shared__ __attribute__((aligned(16))) char outb[NCOMP * OUT_BYTES];
    __shared__ float part[2][NCOMP][3][64]; // per block parity and compute wave: m, ms, l of its 64 rows
    __shared__ float stb[2 * ST];           // final statistics of the output block: [0, 128) max, [128, 256) logsum

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int role = wave / NCOMP; // 0 compute, 1 store, 2 loader, 3 statistics (SPLIT)
    const int slot = wave % NCOMP;
    const int sa = slot >> 1, sb = slot & 1;
    char *my_out = outb + slot * OUT_BYTES;
    const uint32_t TBY = T * (uint32_t)O::OB;
    const uint32_t ldb = 3u * C * (uint32_t)E::ES;
    const bool vec = vec_store != 0;
    const float c = scale * LOG2E;

    PWalk cur;
    cur.init(P, nt);

    // Every wave passes the same barriers: one after the prologue, then X and
    // Y once per step, for as many steps as the walk has.
    if (role == 2) {
        const int cl = slot * 64 + lane;
        Staged<NCH> ss, so;
        // The item last staged in each buffer: a next item with the same
        // plane and query block finds its Q rows already there.
        uint32_t st_plane = ~0u, st_T0 = ~0u, out_plane = ~0u, out_T0 = ~0u;
        if (cur.valid()) {
            if (cur.has_st) {
                const Super sp = cur.st_item();
                stage_fetch<E, NCH>(ss, qkv, sp, T, C, NH, HS, ldb, cl);
                stage_store<NCH>(ss, opb_st, cl);
                st_plane = sp.plane;
                st_T0 = sp.T0;
            }
            if (cur.has_out) {
                const Super sp = cur.out_item();
                stage_fetch<E, NCH>(so, qkv, sp, T, C, NH, HS, ldb, cl);
                stage_store<NCH>(so, opb_out, cl);
                out_plane = sp.plane;
                out_T0 = sp.T0;
            }
        }
        lds_barrier();
        while (cur.valid()) {
            cur.advance();
            const bool more = cur.valid();
            const bool nst = more && cur.has_st, nout = more && cur.has_out;
            bool q_st = true, q_out = true;
            if (nst) {
                const Super sp = cur.st_item();
                q_st = !(sp.plane == st_plane && sp.T0 == st_T0);
                stage_fetch<E, NCH>(ss, qkv, sp, T, C, NH, HS, ldb, cl, q_st);
                st_plane = sp.plane;
                st_T0 = sp.T0;
            }
            if (nout) {
                const Super sp = cur.out_item();
                q_out = !(sp.plane == out_plane && sp.T0 == out_T0);
                stage_fetch<E, NCH>(so, qkv, sp, T, C, NH, HS, ldb, cl, q_out);
                out_plane = sp.plane;
                out_T0 = sp.T0;
            }
            lds_barrier(); // X: operand rows of this step consumed
            if (nst) stage_store<NCH>(ss, opb_st, cl, q_st);
            if (nout) stage_store<NCH>(so, opb_out, cl, q_out);
            lds_barrier(); // Y: operand rows of the next step in LDS
        }
    } else if (role == 0 || role == 3) {
        // Without SPLIT the compute waves take both items of a step; with it
        // role 0 takes the output item and role 3 the statistics item, each
        // in a loop of its own (so neither holds the other's invariants).
        auto compute_loop = [&](auto with_st, auto with_out) {
        constexpr bool DO_ST = decltype(with_st)::value, DO_OUT = decltype(with_out)::value;
        const int r32 = lane & 31;
        Run2 rn;
        float mx[2] = {0.f, 0.f}, ls[2] = {0.f, 0.f};
        lds_barrier();
        while (cur.valid()) {
            const bool has_st = DO_ST && cur.has_st, has_out = DO_OUT && cur.has_out;
            const Super ss = cur.st_item(), so = cur.out_item();
            const bool first_out = has_out && cur.oJ == 0, last_stats = has_st && cur.sJ == cur.sI;
            const uint32_t opar = cur.oi & 1, spar = cur.si & 1;
            cur.advance();
            if (first_out) {
                // The four waves' statistics of the output block, published at
                // its last statistics step; both waves of a pair merge them in
                // the same order, so they agree exactly.
#pragma unroll
                for (int qb = 0; qb < 2; ++qb) {
                    const int row = 32 * qb + r32;
                    const int p0 = 2 * sa, p1 = 2 * sa + 1;
                    float m = part[opar][p0][0][row], ms = part[opar][p0][1][row], l = part[opar][p0][2][row];
                    stats_merge(m, ms, l, part[opar][p1][0][row], part[opar][p1][1][row], part[opar][p1][2][row], c);
                    mx[qb] = m * scale;
                    ls[qb] = (__builtin_amdgcn_logf(l) - fmaf(m, c, -ms)) * LN2;
                    if (sb == 0 && lane < 32) {
                        stb[64 * sa + row] = mx[qb];
                        stb[ST + 64 * sa + row] = ls[qb];
                    }
                }
            }
            f32x16 acc[2][2];
            if (has_st) {
                if (ss.S0 == 0) { // a new block: statistics start empty
#pragma unroll
                    for (int qb = 0; qb < 2; ++qb) {
                        rn.m[qb] = -__builtin_inff();
                        rn.ms[qb] = 0.f;
                        rn.l[qb] = 0.f;
                    }
                }
                const bool live = !(ss.diag && sa == 0 && sb == 1);
#pragma unroll
                for (int a = 0; a < 2; ++a)
#pragma unroll
                    for (int b = 0; b < 2; ++b) acc[a][b] = f32x16{};
                if (live) {
                    sub_mma<E, NCH>(acc, opb_st, sa, sb, lane);
                    if (ss.diag && sa == sb) sub_stats_update<true>(acc, rn, c, lane);
                    else sub_stats_update<false>(acc, rn, c, lane);
                }
                if (last_stats) { // merge the lane halves, publish for the block's first output step
#pragma unroll
                    for (int qb = 0; qb < 2; ++qb) {
                        stats_merge(rn.m[qb], rn.ms[qb], rn.l[qb], __shfl_xor(rn.m[qb], 32),
                                    __shfl_xor(rn.ms[qb], 32), __shfl_xor(rn.l[qb], 32), c);
                        if (lane < 32) {
                            part[spar][slot][0][32 * qb + r32] = rn.m[qb];
                            part[spar][slot][1][32 * qb + r32] = rn.ms[qb];
                            part[spar][slot][2][32 * qb + r32] = rn.l[qb];
                        }
                    }
                }
            }
            const bool live_out = has_out && !(so.diag && sa == 0 && sb == 1);
            if (has_out) {
#pragma unroll
                for (int a = 0; a < 2; ++a)
#pragma unroll
                    for (int b = 0; b < 2; ++b) acc[a][b] = f32x16{};
                if (live_out) sub_mma<E, NCH>(acc, opb_out, sa, sb, lane);
            }
            lds_barrier(); // X: operand rows consumed, previous tile read back
            if (live_out) {
                if (so.diag && sa == sb) subtile_to_lds<true, O, EP>(acc, my_out, scale, lane, mx, ls);
                else subtile_to_lds<false, O, EP>(acc, my_out, scale, lane, mx, ls);
            }
            lds_barrier(); // Y: tile in LDS / partial statistics in LDS
        }
        };
        using yes = std::true_type;
        using no = std::false_type;
        if constexpr (SPLIT) {
            if (role == 3) compute_loop(yes{}, no{});
            else compute_loop(no{}, yes{});
        } else {
            compute_loop(yes{}, yes{});
        }
    } else {
        lds_barrier();
        Tile pm; // mirror of the previous output step, second half pending
        bool pm_live = false, pm_full = false;
        while (cur.valid()) {
            const bool has_out = cur.has_out;
            const Super sp = cur.out_item();
            const bool first_out = has_out && cur.oJ == 0;
            cur.advance();
            const Tile tl = sub_tile<O>(sp, sa, sb, out, T);
            const bool inside = tl.rl > 0 && tl.cl > 0;
            const uint32_t tby = opaque_s(TBY);
            const bool full = tl.rl == TB && tl.cl == TB;
            lds_barrier(); // X
            if (pm_live) {
                if (pm_full) nan_mirror_o<1, O, true, EP>(pm, T, tby, lane, vec);
                else nan_mirror_o<1, O, false, EP>(pm, T, tby, lane, vec);
            }
            pm_live = false;
            if (first_out) { // the block's statistics, written by the compute waves before X
                const int cl = slot * 64 + lane;
                const uint32_t row = sp.T0 + (uint32_t)(cl & (ST - 1));
                if (row < T) (cl < ST ? row_max : row_logsum)[(uint64_t)sp.plane * T + row] = stb[cl];
            }
            lds_barrier(); // Y: tile in LDS
            if (!has_out || !inside) continue;
            stream_subtile<O, EP>(tl, sp.diag && sa == 0 && sb == 1, full, vec, my_out, T, tby, lane);
            if (!tl.diag) { // first half of the mirror now, the second after the next X
                pm = tl;
                pm_live = true;
                pm_full = full && vec;
                if (pm_full) nan_mirror_o<0, O, true, EP>(tl, T, tby, lane, vec);
                else nan_mirror_o<0, O, false, EP>(tl, T, tby, lane, vec);
            }
        }
        if (pm_live) {
            const uint32_t tby = opaque_s(TBY);
            if (pm_full) nan_mirror_o<1, O, true, EP>(pm, T, tby, lane, vec);
            else nan_mirror_o<1, O, false, EP>(pm, T, tby, lane, vec);
        }
    }
}

template <class E, int NCH, class O, class EP> hipError_t launch_fused(const TrimulArgs &a, hipStream_t s)
{
    auto kern = softmax_fused_kernel<E, NCH, O, EP>;
    static ResidentSlots resident, resident_pipe, resident_split;
    ResidentSlots *rs = &resident;
    int threads = tri::SUPER_THREADS;
    const int64_t nt = (a.T + ST - 1) / ST;
    if constexpr (E::ES == 2 && NCH == 8) {
        // The pipelined walk from 16 query blocks per plane on (measured,
        // outputs bit-identical: bf16 B4 T4096 probabilities to bf16 727 ->
        // 715 us, log-probabilities 737 -> 696 us, to fp32 1195 -> 1176 us;
        // at B8 T1024, 8 blocks, 54.7 -> 57.0 us, so the plain walk there).
        // With fp32 output the walk's statistics items go to waves of their
        // own (SPLIT: 1192.7 -> 1149.8 us, bit-identical); with 16-bit output
        // the two time alike (712.6 / 716.5 us), so the 768-thread kernel.
        // CAS_SOFTMAX_FUSED=plain|pipe|split overrides the choice (tuning).
        const char *env = std::getenv("CAS_SOFTMAX_FUSED");
        const bool pipe = env && !std::strcmp(env, "pipe") ? true : env && !std::strcmp(env, "plain") ? false : nt >= 16;
        const bool split = env ? !std::strcmp(env, "split") : pipe && std::is_same<O, tri::OF32>::value;
        if (split) {
            kern = softmax_pipe_kernel<E, O, EP, true>;
            rs = &resident_split;
            threads = tri::SUPER_THREADS + tri::NCOMP_THREADS;
        } else if (pipe) {
            kern = softmax_pipe_kernel<E, O, EP, false>;
            rs = &resident_pipe;
        }
    }
    const int64_t P = a.B * a.NH;
    // Persistent grid; no more workgroups than row blocks (each XCD's share).
    int64_t grid = resident_slots(*rs, kern, threads);
    const int64_t blocks = P * nt;
    if (grid > 8 * ((blocks + 7) / 8)) grid = 8 * ((blocks + 7) / 8);
    if (grid < 8) grid = 8;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(threads), 0, s, (const char *)a.qkv, (char *)a.out,
                       const_cast<float *>(a.row_max), const_cast<float *>(a.row_logsum), (uint32_t)a.T,
                       (uint32_t)a.C, (uint32_t)a.NH, (uint32_t)a.HS, (uint32_t)P, (uint32_t)nt, a.scale,
                       (int)a.vec_store);
    return hipGetLastError();
}

template <class E, class EP> hipError_t launch_fused_ep(const TrimulArgs &a, hipStream_t s)
{
    const bool narrow = a.HS * E::ES <= 128;
    if (a.out_kind == 1)
        return narrow ? launch_fused<E, 8, tri::OBF16, EP>(a, s) : launch_fused<E, 16, tri::OBF16, EP>(a, s);
    if (a.out_kind == 2)
        return narrow ? launch_fused<E, 8, tri::OF16, EP>(a, s) : launch_fused<E, 16, tri::OF16, EP>(a, s);
    return narrow ? launch_fused<E, 8, tri::OF32, EP>(a, s) : launch_fused<E, 16, tri::OF32, EP>(a, s);
}

// Both launches in one (softmax_fused_kernel); statistics written through
// a.row_max / a.row_logsum, the rows through a.out.
template <class E> hipError_t launch_row_stats_impl(const TrimulArgs &a, hipStream_t s);
template <class E> hipError_t launch_softmax_impl(const TrimulArgs &a, int mode, hipStream_t s);

template <class E> hipError_t launch_softmax_fused_impl(const TrimulArgs &a, int mode, hipStream_t s)
{
    if (a.HS * E::ES > 256) { // heads of 257 .. 512 bytes: the statistics launch, then the rows launch
        const hipError_t e = launch_row_stats_impl<E>(a, s);
        if (e != hipSuccess) return e;
        return launch_softmax_impl<E>(a, mode, s);
    }
    if (mode == 0) return launch_fused_ep<E, tri::EpLog>(a, s);
    return launch_fused_ep<E, tri::EpProb>(a, s);
}

template <class E, int NCH, int NQ = NCH / 2> hipError_t launch_row_stats_nch(const TrimulArgs &a, hipStream_t s)
{
    return launch_longest_first(a, s, [&](dim3 grid, uint32_t nt, uint32_t planes, uint32_t rank0) {
        hipLaunchKernelGGL((row_stats_kernel<E, NCH, NQ>), grid, dim3(STATS_THREADS), 0, s, (const char *)a.qkv,
                           const_cast<float *>(a.row_max), const_cast<float *>(a.row_logsum), (uint32_t)a.T,
                           (uint32_t)a.C, (uint32_t)a.NH, (uint32_t)a.HS, nt, planes, rank0, a.scale);
    });
}

// Row statistics (row_max and row_logsum written through a.row_max /
// a.row_logsum). The caller has checked that the fused path applies.
template <class E> hipError_t launch_row_stats_impl(const TrimulArgs &a, hipStream_t s)
{
    if (a.HS * E::ES <= 128) return launch_row_stats_nch<E, 8>(a, s);
    if (a.HS * E::ES > 256) { // heads of 257 .. 512 bytes
        if constexpr (std::is_same<E, KF32>::value)
            return a.HS * E::ES <= 384 ? launch_row_stats_nch<E, 32, 12>(a, s) : launch_row_stats_nch<E, 32>(a, s);
        else return launch_row_stats_wide16(a, std::is_same<E, KBF16>::value ? E_BF16 : E_F16, s);
    }
    return launch_row_stats_nch<E, 16>(a, s);
}

// Softmax rows: the three-role score kernel with the softmax epilogue; heads
// of 257 .. 512 bytes in two halves (CAS_TRIMUL_KERNEL=tile: on the per-wave
// tile kernel with the same epilogue). mode 0: log-probabilities, 1:
// probabilities.
template <class E, class EP> hipError_t launch_softmax_ep(const TrimulArgs &a, hipStream_t s)
{
    if (a.HS * E::ES > 256) {
        const char *kv = std::getenv("CAS_TRIMUL_KERNEL");
        if (kv && std::strcmp(kv, "tile") == 0) return tri::launch_tile_ep<E, EP>(a, s);
        if (a.out_kind == 1) return tri::launch_two_halves<E, tri::OBF16, EP>(a, s);
        if (a.out_kind == 2) return tri::launch_two_halves<E, tri::OF16, EP>(a, s);
        return tri::launch_two_halves<E, tri::OF32, EP>(a, s);
    }
    const bool narrow = a.HS * E::ES <= 128;
    if (a.out_kind == 1)
        return narrow ? tri::launch_super<E, 8, tri::OBF16, EP>(a, s) : tri::launch_super<E, 16, tri::OBF16, EP>(a, s);
    if (a.out_kind == 2)
        return narrow ? tri::launch_super<E, 8, tri::OF16, EP>(a, s) : tri::launch_super<E, 16, tri::OF16, EP>(a, s);
    return narrow ? tri::launch_super<E, 8, tri::OF32, EP>(a, s) : tri::launch_super<E, 16, tri::OF32, EP>(a, s);
}

template <class E> hipError_t launch_softmax_impl(const TrimulArgs &a, int mode, hipStream_t s)
{
    if (mode == 0) return launch_softmax_ep<E, tri::EpLog>(a, s);
    return launch_softmax_ep<E, tri::EpProb>(a, s);
}

// ---------------------------------------------------------------------------
// Attention output (the step after the softmax): y[b, t, nh, :] =
// sum_{t2 <= t} p[t][t2] V[b, t2, nh, :], with p the probabilities of the
// softmax-rows kernel, formed from the row statistics exactly as that kernel
// forms them, and V the third slot of the packed rows. Neither the scores nor
// the probabilities reach HBM: per key tile the scores are recomputed, turned
// into p in registers and multiplied into the output on the MFMAs.
//
// A workgroup owns one 128-row query block (longest first, as the
// row-statistics kernel), four waves of 32 query rows, each wave's Q
// fragments in registers; per step 64 keys: their K rows (for D = K Q^T) and
// V rows are fetched a step ahead into double-buffered LDS.
//  * Lane (r32, h) of the score MFMAs holds p for query r32 and keys
//    8g + 4h + e of each 32-key block (accumulator r = 4g + e).
//  * fp32 inputs (v_mfma_f32_32x32x2_f32): the product P V contracts over
//    keys, and its MFMA j takes key 8(j/4) + 4h + j%4 in k-slot h: exactly
//    accumulator j, so P feeds the A operand from the registers it was
//    computed in; the B operand is V[that key][d] from LDS. V rows sit 288
//    bytes apart, so the two keys an MFMA reads (4 apart) fall in different
//    bank halves.
//  * 16-bit inputs (v_mfma_f32_32x32x16): see the 16-bit section below (P
//    rounded to the format; K and V loaded straight into LDS, the V operand
//    read back through the LDS transpose read).
// ---------------------------------------------------------------------------
constexpr int AKT = 64;            // keys per attention step
// LDS bytes per fp32 V row: the head row (at least 256 bytes) plus 32, so
// that rows 4 apart (the two lane halves of a P V operand read) start 32
// banks apart.
template <int NCH> constexpr int av_pitch() { return (NCH * 16 > 256 ? NCH * 16 : 256) + 32; }

template <int NCH> struct AStage {
    u32x4 k[NCH / 4], v[NCH / 4];
};

// The 64 K rows and 64 V rows of key tile J (rows J*64.. of the plane), NCH
// 16-byte chunks per row; lane tid takes chunk tid % NCH of rows
// q * (256 / NCH) + tid / NCH. Rows past T and chunks past the head read zero.
template <int NCH>
__device__ __forceinline__ void a_fetch(AStage<NCH> &st, const char *kb0, const char *vb0, uint32_t J, uint32_t T,
                                        uint32_t ldb, uint32_t head_bytes, int tid)
{
    constexpr int RPJ = STATS_THREADS / NCH;
    const __amdgpu_buffer_rsrc_t rk = rsrc_at(kb0 + (uint64_t)J * AKT * ldb);
    const __amdgpu_buffer_rsrc_t rv = rsrc_at(vb0 + (uint64_t)J * AKT * ldb);
    const uint32_t c = (uint32_t)(tid % NCH), r0 = (uint32_t)(tid / NCH);
    const uint32_t lim = c * 16 < head_bytes ? T : 0u;
#pragma unroll
    for (int q = 0; q < NCH / 4; ++q) {
        const uint32_t r = (uint32_t)(q * RPJ) + r0;
        const uint32_t ok = 0u - (uint32_t)(J * AKT + r < lim);
        const uint32_t vo = ((r * ldb + c * 16) & ok) | (OOB & ~ok);
        st.k[q] = __builtin_amdgcn_raw_buffer_load_b128(rk, (int)vo, 0, 0);
        st.v[q] = __builtin_amdgcn_raw_buffer_load_b128(rv, (int)vo, 0, 0);
    }
}

template <int NCH> __device__ __forceinline__ void a_store(const AStage<NCH> &st, char *kbuf, char *vbuf, int tid)
{
    constexpr int RPJ = STATS_THREADS / NCH;
    const uint32_t c = (uint32_t)(tid % NCH), r0 = (uint32_t)(tid / NCH);
#pragma unroll
    for (int q = 0; q < NCH / 4; ++q) {
        const uint32_t r = (uint32_t)(q * RPJ) + r0;
        *reinterpret_cast<u32x4 *>(kbuf + r * (NCH * 16) + kswz<NCH>(r, c)) = st.k[q];
        *reinterpret_cast<u32x4 *>(vbuf + r * av_pitch<NCH>() + c * 16) = st.v[q];
    }
}

// One step: scores of this wave's 32 queries against the tile's 64 keys,
// p from the row statistics (mx: the row's max score, ls: its logsum), then
// y[nb] += P V for the NBV 32-column blocks of the head. DIAG: keys after the
// query (absolute index kabs0 + key > qabs) get p = 0.
// Scores of this wave's 32 queries against the tile's 64 keys: D = K Q^T
// per 32-key block b, so s[b][r] is the dot product of query lane%32 and key
// 32b + 8(r/4) + 4(lane/32) + r%4 (unscaled).
template <class E, int NCH, int NQ = NCH / 2>
__device__ __forceinline__ void attn_scores(f32x16 (&s)[2], const char *kbuf, const u32x4 (&qf)[NCH / 2], int lane)
{
    constexpr int RB = NCH * 16;
    const uint32_t r32 = (uint32_t)(lane & 31), h = (uint32_t)(lane >> 5);
#pragma unroll
    for (int u = 0; u < NQ; ++u) {
        u32x4 kf[2];
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const uint32_t row = 32u * b + r32;
            kf[b] = *reinterpret_cast<const u32x4 *>(kbuf + row * RB + kswz<NCH>(row, 2u * u + h));
        }
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            if (u == 0) s[b] = mfma_first<E>(kf[b], qf[u]);
            else mfma_chunk<E>(s[b], kf[b], qf[u]);
        }
    }
}

template <int NCH, int NBV, bool DIAG, int NQ = NCH / 2>
__device__ __forceinline__ void a_step(f32x16 (&yacc)[NBV], const char *kbuf, const char *vbuf,
                                       const u32x4 (&qf)[NCH / 2], float scale, float mx, float ls, int lane,
                                       uint32_t kabs0, uint32_t qabs)
{
    f32x16 s[2];
    const uint32_t r32 = (uint32_t)(lane & 31), h = (uint32_t)(lane >> 5);
    attn_scores<KF32, NCH, NQ>(s, kbuf, qf, lane);
    // p, in place, as the softmax-rows kernel forms it
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float p = tri::epilogue<tri::EpProb>(s[b][r], scale, mx, ls);
            if (DIAG && kabs0 + 32u * b + 8u * (r >> 2) + 4u * h + (uint32_t)(r & 3) > qabs) p = 0.f;
            s[b][r] = p;
        }
    // y += P V: MFMA j of key block b takes key 32b + 8(j/4) + 4h + j%4 in
    // k-slot h: A = s[b][j] (this lane's p), B = V[key][32 nb + lane%32].
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const uint32_t key = 32u * b + 8u * (j >> 2) + 4u * h + (uint32_t)(j & 3);
#pragma unroll
            for (int nb = 0; nb < NBV; ++nb) {
                const float v = *reinterpret_cast<const float *>(vbuf + key * av_pitch<NCH>() + (32u * nb + r32) * 4u);
                yacc[nb] = __builtin_amdgcn_mfma_f32_32x32x2f32(s[b][j], v, yacc[nb], 0, 0, 0);
            }
        }
}

// ---------------------------------------------------------------------------
// 16-bit inputs (v_mfma_f32_32x32x16_{bf16,f16}). The same walk and p; P is
// rounded to the input type (nearest even) for the P V MFMAs. Their lane
// half h supplies 8 consecutive k-slots: MFMA j (of two per 32-key block)
// takes, for k-slots 8h .. 8h + 7, keys 8(2j + i/4) + 4h + i%4 (i = 0..7),
// which are score accumulators 8j .. 8j + 7 of that lane, so P again stays
// in place. Those keys come in two runs of four of one head column, which
// the LDS transpose read delivers from V stored as read (below).
// ---------------------------------------------------------------------------

// Two fp32 values rounded (nearest even) to the input format, a in the low
// half: one packed conversion.
typedef float f32x2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2v __attribute__((ext_vector_type(2)));
template <class E> __device__ __forceinline__ uint32_t pack16(float a, float b);
template <> __device__ __forceinline__ uint32_t pack16<KBF16>(float a, float b)
{
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2v){a, b}, bf16x2v));
}
template <> __device__ __forceinline__ uint32_t pack16<KF16>(float a, float b)
{
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2v){a, b}, f16x2v));
}

// 16-bit staging. The K and V tiles go from HBM
// straight into LDS (buffer loads with an LDS destination: no registers and no
// VALU work on the way). One such wave load fills one kilobyte, lane i the
// bytes 16i .. 16i + 15, so each lane fetches the global chunk that belongs at
// its LDS position. K keeps the layout of the score reads (kswz). V is stored
// key-major, chunk c of row r at position c ^ vswz(r), and the P V operand,
// four consecutive keys of one head column per 8-byte register, comes out of
// LDS through the transpose read ds_read_b64_tr_b16: within each group of 16
// lanes, lane 4q + m receives element m of the 8 bytes that lanes
// 4e + q (e = 0..3) address, as its elements e = 0..3. Rows past T are cut by
// the size of the tile's buffer resource, chunks past the head by an
// out-of-range offset; both read zero.
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

template <int NCH> __device__ __forceinline__ uint32_t vswz(uint32_t r)
{
    // A transpose read covers 4 rows x 64 bytes per 32 lanes and 4 rows x 32
    // bytes per 16 lanes; with these chunk XORs the rows of either set fall in
    // distinct banks (256 bytes of banks, rows of NCH * 16 bytes).
    if constexpr (NCH == 8) return 2u * (r & 3u);
    else if constexpr (NCH == 16) return (0xCA60u >> (4u * (r & 3u))) & 15u;
    else return 4u * (r & 3u); // 512-byte rows: the four rows' 64-byte groups at 0, 64, 128, 192 bytes
}

// Per lane, the offset within the tile's rows of each of its NCH / 2 loads:
// wave w fills kilobytes w * NCH / 4 .. of the K tile, then the same of V.
template <int NCH> struct DStage16 {
    uint32_t vo[NCH / 2];
};

template <int NCH>
__device__ __forceinline__ void d16_init(DStage16<NCH> &st, int w, int lane, uint32_t ldb, uint32_t head_bytes)
{
    constexpr uint32_t RB = NCH * 16, PER = NCH / 4, SH = NCH == 8 ? 1 : 0;
#pragma unroll
    for (int q = 0; q < NCH / 2; ++q) {
        const bool kside = q < (int)PER;
        const uint32_t o = ((uint32_t)w * PER + (uint32_t)q % PER) * 1024u + 16u * (uint32_t)lane;
        const uint32_t r = o / RB, p = (o % RB) / 16u;
        const uint32_t c = kside ? p ^ ((r >> SH) & (NCH - 1)) : p ^ vswz<NCH>(r); // the XORs are involutions
        st.vo[q] = c * 16u < head_bytes ? r * ldb + c * 16u : OOB;
    }
}


template <int NCH>
__device__ __forceinline__ void d16_fetch(const DStage16<NCH> &st, char *kdst, char *vdst, const char *kb0,
                                          const char *vb0, uint32_t J, uint32_t T, uint32_t ldb, int w)
{
    constexpr uint32_t PER = NCH / 4;
    const uint32_t k0 = J * AKT, rows = k0 < T ? T - k0 : 0u;
    const __amdgpu_buffer_rsrc_t rk = rsrc_rows(kb0 + (uint64_t)k0 * ldb, rows, ldb);
    const __amdgpu_buffer_rsrc_t rv = rsrc_rows(vb0 + (uint64_t)k0 * ldb, rows, ldb);
#pragma unroll
    for (int q = 0; q < NCH / 2; ++q) {
        const bool kside = q < (int)PER;
        char *dst = (kside ? kdst : vdst) + ((uint32_t)w * PER + (uint32_t)q % PER) * 1024u;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(kside ? rk : rv, (lds_void *)dst, 16, (int)st.vo[q], 0, 0, 0);
    }
}

__device__ __forceinline__ u32x2 lds_read_tr16(const char *p)
{
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)p));
}

// The V operand addresses of this lane for key chunk 0, per head block nb:
// lane (h, g = lane / 16 % 2, i = lane % 16) points at row 4h + i/4 of the
// tile, column byte 64 nb + 32 g + 8 (i % 4). The transpose read then hands
// it keys 4h .. 4h + 3 of head column 32 nb + lane % 32, the k-slots its p
// occupies; rows 8 further give the other run of four, and chunk k0 adds
// k0 rows (row r % 4 = i / 4 throughout, so the swizzle is the lane's own).
template <int NCH, int NBV>
__device__ __forceinline__ void v16_lanes(const char *(&vl)[NBV], const char *vbuf, int lane)
{
    constexpr uint32_t RB = NCH * 16;
    const uint32_t h = (uint32_t)lane >> 5, i = (uint32_t)lane & 15u, e = i >> 2, q = i & 3u;
    const uint32_t g = ((uint32_t)lane >> 4) & 1u;
#pragma unroll
    for (int nb = 0; nb < NBV; ++nb)
        vl[nb] = vbuf + (4u * h + e) * RB + 16u * ((4u * nb + 2u * g + (q >> 1)) ^ vswz<NCH>(e)) + 8u * (q & 1u);
}

template <class E, int NCH, int NBV, bool DIAG, int NQ = NCH / 2>
__device__ __forceinline__ void a_step16(f32x16 (&yacc)[NBV], const char *kbuf, const char *vbuf,
                                         const u32x4 (&qf)[NCH / 2], float scale, float mx, float ls, int lane,
                                         uint32_t kabs0, uint32_t qabs)
{
    f32x16 s[2];
    const uint32_t h = (uint32_t)(lane >> 5);
    attn_scores<E, NCH, NQ>(s, kbuf, qf, lane);
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float p = tri::epilogue<tri::EpProb>(s[b][r], scale, mx, ls);
            if (DIAG && kabs0 + 32u * b + 8u * (r >> 2) + 4u * h + (uint32_t)(r & 3) > qabs) p = 0.f;
            s[b][r] = p;
        }
    const char *vl[NBV];
    v16_lanes<NCH, NBV>(vl, vbuf, lane);
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const u32x4 pa = {pack16<E>(s[b][8 * j + 0], s[b][8 * j + 1]), pack16<E>(s[b][8 * j + 2], s[b][8 * j + 3]),
                              pack16<E>(s[b][8 * j + 4], s[b][8 * j + 5]), pack16<E>(s[b][8 * j + 6], s[b][8 * j + 7])};
            const uint32_t k0 = 32u * b + 16u * j; // keys k0 + 4h .. k0 + 4h + 3 and 8 further
#pragma unroll
            for (int nb = 0; nb < NBV; ++nb) {
                const u32x2 lo = lds_read_tr16(vl[nb] + k0 * (NCH * 16));
                const u32x2 hi = lds_read_tr16(vl[nb] + (k0 + 8u) * (NCH * 16));
                mfma_chunk<E>(yacc[nb], pa, u32x4{lo[0], lo[1], hi[0], hi[1]});
            }
        }
}

// One kernel for the three input types: the staging and the step differ
// (fp32: staged through registers, V rows padded; 16-bit: loaded straight
// into LDS, V read back transposed, P rounded to the format).
template <class E, int NCH> struct AttnCfg {
    static constexpr bool F32 = std::is_same<E, KF32>::value;
    static constexpr int ES = F32 ? 4 : 2;
    static constexpr int NBV = NCH * 16 / ES / 32; // 32-column blocks of the head (HS * ES <= NCH * 16 bytes)
    static constexpr int VBYTES = AKT * av_pitch<NCH>(); // one fp32 V stage in LDS (16-bit: AKT * NCH * 16, as K)
    // Workgroups per CU the registers must allow (LDS allows more). 16-bit,
    // head <= 128 bytes: four, at 128 VGPRs, measured faster than three.
    static constexpr int MIN_WG = (!F32 && NCH == 8) ? 4 : 1;
};

template <class E, int NCH, int NQ = NCH / 2>
__global__ void __launch_bounds__(STATS_THREADS, (AttnCfg<E, NCH>::MIN_WG))
attention_kernel(const char *__restrict__ qkv, const float *__restrict__ row_max,
                 const float *__restrict__ row_logsum, float *__restrict__ y, uint32_t T, uint32_t C, uint32_t NH,
                 uint32_t HS, uint32_t nt, uint32_t planes, uint32_t rank0, float scale)
{
    using Cfg = AttnCfg<E, NCH>;
    constexpr int RB = NCH * 16, NU = NCH / 2, NBV = Cfg::NBV, KBYTES = AKT * RB, VBYTES = Cfg::VBYTES;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const uint32_t r32 = (uint32_t)(lane & 31), h = (uint32_t)(lane >> 5);

    const BlockIdx bi = longest_first(planes, rank0, nt);
    const uint32_t plane = bi.plane, I = bi.I;
    const uint32_t b = plane / NH, nh = plane - b * NH;
    const uint32_t ldb = 3u * C * (uint32_t)Cfg::ES;
    const uint32_t head_bytes = HS * (uint32_t)Cfg::ES;
    const char *qb0 = qkv + ((uint64_t)b * T * (3u * C) + (uint64_t)nh * HS) * Cfg::ES; // Q row 0 of the plane
    const char *kb0 = qb0 + (uint64_t)C * Cfg::ES;                                      // K row 0
    const char *vb0 = qb0 + (uint64_t)2 * C * Cfg::ES;                                  // V row 0

    {
        const uint32_t t0 = I * ST;
        const uint32_t qabs = t0 + 32u * w + r32; // this lane's query row (score side)

        u32x4 qf[NU];
        {
            const __amdgpu_buffer_rsrc_t rq = rsrc_at(qb0 + (uint64_t)t0 * ldb);
            const uint32_t row = 32u * w + r32;
            const bool row_ok = t0 + row < T;
#pragma unroll
            for (int u = 0; u < NQ; ++u) {
                const uint32_t ch = 2u * u + h;
                const uint32_t vo = (row_ok && ch * 16 < head_bytes) ? row * ldb + ch * 16 : OOB;
                qf[u] = __builtin_amdgcn_raw_buffer_load_b128(rq, (int)vo, 0, 0);
            }
        }
        // the row statistics of this lane's query row (rows past T: unused)
        const uint64_t so = (uint64_t)plane * T + (qabs < T ? qabs : T - 1);
        const float mx = row_max[so], ls = row_logsum[so];

        f32x16 yacc[NBV];
#pragma unroll
        for (int nb = 0; nb < NBV; ++nb) yacc[nb] = f32x16{};
        // 64-key tiles 0 .. 2I + 1: tiles below 2I lie wholly before the
        // block's first query; the last two hold the diagonal.
        const uint32_t nst = 2 * I + 2;
        if constexpr (Cfg::F32) {
            __shared__ __attribute__((aligned(16))) char kbuf[2 * KBYTES];
            __shared__ __attribute__((aligned(16))) char vbuf[2 * VBYTES];
            AStage<NCH> st;
            a_fetch<NCH>(st, kb0, vb0, 0, T, ldb, head_bytes, tid);
            a_store<NCH>(st, kbuf, vbuf, tid);
            __builtin_amdgcn_s_waitcnt(0x70); // vmcnt(0) lgkmcnt(0): Q, statistics and tile 0 in place
            tri::lds_barrier();
            uint32_t J = 0;
            for (; J + 2 < nst; ++J) {
                a_fetch<NCH>(st, kb0, vb0, J + 1, T, ldb, head_bytes, tid);
                a_step<NCH, NBV, false, NQ>(yacc, kbuf + (J & 1) * KBYTES, vbuf + (J & 1) * VBYTES, qf, scale, mx, ls,
                                        lane, J * AKT, qabs);
                a_store<NCH>(st, kbuf + ((J + 1) & 1) * KBYTES, vbuf + ((J + 1) & 1) * VBYTES, tid);
                tri::lds_barrier();
            }
            // the diagonal pair: J = nst - 2 (even, buffer 0), then nst - 1
            a_fetch<NCH>(st, kb0, vb0, J + 1, T, ldb, head_bytes, tid);
            a_step<NCH, NBV, true, NQ>(yacc, kbuf, vbuf, qf, scale, mx, ls, lane, J * AKT, qabs);
            a_store<NCH>(st, kbuf + KBYTES, vbuf + VBYTES, tid);
            tri::lds_barrier();
            a_step<NCH, NBV, true, NQ>(yacc, kbuf + KBYTES, vbuf + VBYTES, qf, scale, mx, ls, lane, (J + 1) * AKT,
                                       qabs);
        } else {
            // Direct staging into four named buffers, the loop unrolled by
            // two (the single-pass kernel's scheme: no wait on the loads in
            // flight before the reads of the current tile).
            __shared__ __attribute__((aligned(16))) char k0s[KBYTES];
            __shared__ __attribute__((aligned(16))) char k1s[KBYTES];
            __shared__ __attribute__((aligned(16))) char v0s[KBYTES];
            __shared__ __attribute__((aligned(16))) char v1s[KBYTES];
            DStage16<NCH> ds;
            d16_init<NCH>(ds, w, lane, ldb, head_bytes);
            d16_fetch<NCH>(ds, k0s, v0s, kb0, vb0, 0, T, ldb, w);
            __builtin_amdgcn_s_waitcnt(0x70); // vmcnt(0) lgkmcnt(0): Q, statistics and tile 0 in place
            tri::lds_barrier();
            uint32_t J = 0;
            for (; J + 2 < nst; J += 2) { // nst is even
                d16_fetch<NCH>(ds, k1s, v1s, kb0, vb0, J + 1, T, ldb, w);
                a_step16<E, NCH, NBV, false, NQ>(yacc, k0s, v0s, qf, scale, mx, ls, lane, J * AKT, qabs);
                __builtin_amdgcn_s_waitcnt(0x70); // this wave's part of tile J + 1 in LDS
                tri::lds_barrier();
                d16_fetch<NCH>(ds, k0s, v0s, kb0, vb0, J + 2, T, ldb, w);
                a_step16<E, NCH, NBV, false, NQ>(yacc, k1s, v1s, qf, scale, mx, ls, lane, (J + 1) * AKT, qabs);
                __builtin_amdgcn_s_waitcnt(0x70);
                tri::lds_barrier();
            }
            d16_fetch<NCH>(ds, k1s, v1s, kb0, vb0, J + 1, T, ldb, w);
            a_step16<E, NCH, NBV, true, NQ>(yacc, k0s, v0s, qf, scale, mx, ls, lane, J * AKT, qabs);
            __builtin_amdgcn_s_waitcnt(0x70);
            tri::lds_barrier();
            a_step16<E, NCH, NBV, true, NQ>(yacc, k1s, v1s, qf, scale, mx, ls, lane, (J + 1) * AKT, qabs);
        }
        // y rows: lane holds query 32w + 8(r/4) + 4h + r%4 and column 32nb + lane%32
#pragma unroll
        for (int nb = 0; nb < NBV; ++nb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const uint32_t t = t0 + 32u * w + 8u * (r >> 2) + 4u * h + (uint32_t)(r & 3);
                const uint32_t d = 32u * nb + r32;
                if (t < T && d < HS) y[((uint64_t)b * T + t) * C + (uint64_t)nh * HS + d] = yacc[nb][r];
            }
    }
}

template <class E, int NCH, int NQ = NCH / 2> hipError_t launch_attention_nch(const TrimulArgs &a, hipStream_t s)
{
    return launch_longest_first(a, s, [&](dim3 grid, uint32_t nt, uint32_t planes, uint32_t rank0) {
        hipLaunchKernelGGL((attention_kernel<E, NCH, NQ>), grid, dim3(STATS_THREADS), 0, s, (const char *)a.qkv,
                           a.row_max, a.row_logsum, (float *)a.out, (uint32_t)a.T, (uint32_t)a.C, (uint32_t)a.NH,
                           (uint32_t)a.HS, nt, planes, rank0, a.scale);
    });
}

// Attention output into a.out ((B, T, C) fp32) from a.row_max / a.row_logsum.
template <class E> hipError_t launch_attention_impl(const TrimulArgs &a, hipStream_t s)
{
    if (a.HS * AttnCfg<E, 8>::ES <= 128) return launch_attention_nch<E, 8>(a, s);
    if (a.HS * E::ES > 256) { // heads of 257 .. 512 bytes
        if constexpr (std::is_same<E, KF32>::value)
            return a.HS * E::ES <= 384 ? launch_attention_nch<E, 32, 12>(a, s) : launch_attention_nch<E, 32>(a, s);
        else return launch_attention_wide16(a, std::is_same<E, KBF16>::value ? E_BF16 : E_F16, s);
    }
    return launch_attention_nch<E, 16>(a, s);
}

// ---------------------------------------------------------------------------
// Single-pass attention: y and the row statistics in one launch, each score
// and its exponential computed once (the two-launch path computes both in the
// statistics launch and again in the attention launch).
//
// Per row the kernel keeps a running offset ms in base 2 and a running sum
// l = sum_j exp2(a_j c - ms) (c = scale log2 e), and y accumulates
// sum_j exp2(a_j c - ms) v_j; when the offset moves, l and y are rescaled by
// exp2(ms_old - ms_new), and y / l is written at the end. The offset follows
// the running maximum lazily: it moves only when a tile's largest score
// exceeds it by more than ONLINE_TAU (in base 2), so after the first steps of
// a row it rarely moves and the rescale is skipped for the whole wave. The
// exponentials are then at most 2^ONLINE_TAU, well inside every format used.
//
// For the rescale to be one factor per lane, the output is accumulated
// transposed, Y^T = V^T P^T: the MFMA operands of the P V product are
// swapped, so a lane's accumulators all belong to its own query row (the
// column of the score MFMAs), with head columns 32 nb + 8(r/4) + 4h + r%4.
// ---------------------------------------------------------------------------
constexpr float ONLINE_TAU = 8.f;


struct OnlineRow {
    float mt; // largest dot product of the row so far (row_max = mt * scale)
    float ms; // offset of the exponentials: fl(m c) of an earlier maximum m <= mt
    float l;  // this lane half's sum of exp2(a c - ms) (the halves see disjoint keys)
};

// x of lane l combined with x of lane l ^ 32, in every lane, from one VALU
// lane swap (v_permlane32_swap) instead of an LDS round trip: afterwards a
// holds x of lanes l % 32 and b of lanes l % 32 + 32.
__device__ __forceinline__ float halves_max(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]); // low half + high half in both: one order, one result
}

template <class E, int NCH, int NBV, bool DIAG, int NQ = NCH / 2>
__device__ __forceinline__ void online_step(f32x16 (&yacc)[NBV], OnlineRow &rw, const char *kbuf,
                                            const char *vbuf, const u32x4 (&qf)[NCH / 2], float c, int lane,
                                            uint32_t kabs0, uint32_t qabs)
{
    static_assert(std::is_same<E, KF32>::value, "fp32 step; online_step16 serves the 16-bit formats");
    const uint32_t r32 = (uint32_t)(lane & 31), h = (uint32_t)(lane >> 5);
    f32x16 s[2];
    attn_scores<E, NCH, NQ>(s, kbuf, qf, lane);
    // Keys after the query become -inf: no part in the maximum, exponential 0.
    float tmax = -__builtin_inff();
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            if (DIAG && kabs0 + 32u * b + 8u * (r >> 2) + 4u * h + (uint32_t)(r & 3) > qabs)
                s[b][r] = -__builtin_inff();
            tmax = fmaxf(tmax, s[b][r]);
        }
    tmax = halves_max(tmax); // the row's other lane half: both take the same offset
    rw.mt = fmaxf(rw.mt, tmax);
    const bool need = fmaf(tmax, c, -rw.ms) > ONLINE_TAU; // first step: ms = -inf
    if (__any(need)) {
        const float msn = need ? pinned(tmax * c) : rw.ms;
        const float alpha = __builtin_amdgcn_exp2f(rw.ms - msn); // 1 where the offset stays, 0 on the first step
        rw.ms = msn;
        rw.l *= alpha;
#pragma unroll
        for (int nb = 0; nb < NBV; ++nb)
#pragma unroll
            for (int r = 0; r < 16; ++r) yacc[nb][r] *= alpha;
    }
    float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float p = __builtin_amdgcn_exp2f(fmaf(s[b][r], c, -rw.ms));
            s[b][r] = p;
            part[r & 3] += p;
        }
    rw.l += (part[0] + part[1]) + (part[2] + part[3]);
    // Y^T += V^T P^T: the A operand is V (as the B operand of the P V form),
    // the B operand this lane's p, in the same k-slots.
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const uint32_t key = 32u * b + 8u * (j >> 2) + 4u * h + (uint32_t)(j & 3);
#pragma unroll
            for (int nb = 0; nb < NBV; ++nb) {
                const float v = *reinterpret_cast<const float *>(vbuf + key * av_pitch<NCH>() + (32u * nb + r32) * 4u);
                yacc[nb] = __builtin_amdgcn_mfma_f32_32x32x2f32(v, s[b][j], yacc[nb], 0, 0, 0);
            }
        }
}

// The 16-bit step: the scores and exponentials as in the fp32 step, then
// P rounded to the input format and Y^T += V^T P^T with the V operand from
// the transpose read.
template <class E, int NCH, int NBV, bool DIAG, int NQ = NCH / 2>
__device__ __forceinline__ void online_step16(f32x16 (&yacc)[NBV], OnlineRow &rw, const char *kbuf,
                                              const char *vbuf, const u32x4 (&qf)[NCH / 2], float c, int lane,
                                              uint32_t kabs0, uint32_t qabs)
{
    constexpr uint32_t RB = NCH * 16;
    const uint32_t h = (uint32_t)(lane >> 5);
    f32x16 s[2];
    attn_scores<E, NCH, NQ>(s, kbuf, qf, lane);
    // Keys after the query become -inf: no part in the maximum, exponential 0.
    float tmax = -__builtin_inff();
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            if (DIAG && kabs0 + 32u * b + 8u * (r >> 2) + 4u * h + (uint32_t)(r & 3) > qabs)
                s[b][r] = -__builtin_inff();
            tmax = fmaxf(tmax, s[b][r]);
        }
    tmax = halves_max(tmax); // the row's other lane half: both take the same offset
    rw.mt = fmaxf(rw.mt, tmax);
    const bool need = fmaf(tmax, c, -rw.ms) > ONLINE_TAU; // first step: ms = -inf
    if (__any(need)) {
        const float msn = need ? pinned(tmax * c) : rw.ms;
        const float alpha = __builtin_amdgcn_exp2f(rw.ms - msn); // 1 where the offset stays, 0 on the first step
        rw.ms = msn;
        rw.l *= alpha;
#pragma unroll
        for (int nb = 0; nb < NBV; ++nb)
#pragma unroll
            for (int r = 0; r < 16; ++r) yacc[nb][r] *= alpha;
    }
    float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float p = __builtin_amdgcn_exp2f(fmaf(s[b][r], c, -rw.ms));
            s[b][r] = p;
            part[r & 3] += p;
        }
    rw.l += (part[0] + part[1]) + (part[2] + part[3]);
    const char *vl[NBV];
    v16_lanes<NCH, NBV>(vl, vbuf, lane);
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const u32x4 pb = {pack16<E>(s[b][8 * j + 0], s[b][8 * j + 1]), pack16<E>(s[b][8 * j + 2], s[b][8 * j + 3]),
                              pack16<E>(s[b][8 * j + 4], s[b][8 * j + 5]), pack16<E>(s[b][8 * j + 6], s[b][8 * j + 7])};
            const uint32_t k0 = 32u * b + 16u * j; // keys k0 + 4h .. k0 + 4h + 3 and 8 further
#pragma unroll
            for (int nb = 0; nb < NBV; ++nb) {
                const u32x2 lo = lds_read_tr16(vl[nb] + k0 * RB);
                const u32x2 hi = lds_read_tr16(vl[nb] + (k0 + 8u) * RB);
                mfma_chunk<E>(yacc[nb], u32x4{lo[0], lo[1], hi[0], hi[1]}, pb);
            }
        }
}

template <class E, int NCH, int NQ = NCH / 2>
__global__ void __launch_bounds__(STATS_THREADS, (AttnCfg<E, NCH>::MIN_WG))
attention_online_kernel(const char *__restrict__ qkv, float *__restrict__ row_max, float *__restrict__ row_logsum,
                        float *__restrict__ y, uint32_t T, uint32_t C, uint32_t NH, uint32_t HS, uint32_t nt,
                        uint32_t planes, uint32_t rank0, float scale, int vec_y)
{
    using Cfg = AttnCfg<E, NCH>;
    constexpr int RB = NCH * 16, NU = NCH / 2, NBV = Cfg::NBV, KBYTES = AKT * RB;
    constexpr int VBYTES = Cfg::VBYTES;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const uint32_t r32 = (uint32_t)(lane & 31), h = (uint32_t)(lane >> 5);

    const BlockIdx bi = longest_first(planes, rank0, nt);
    const uint32_t plane = bi.plane, I = bi.I;
    const uint32_t b = plane / NH, nh = plane - b * NH;
    const uint32_t ldb = 3u * C * (uint32_t)Cfg::ES;
    const uint32_t head_bytes = HS * (uint32_t)Cfg::ES;
    const char *qb0 = qkv + ((uint64_t)b * T * (3u * C) + (uint64_t)nh * HS) * Cfg::ES; // Q row 0 of the plane
    const char *kb0 = qb0 + (uint64_t)C * Cfg::ES;                                      // K row 0
    const char *vb0 = qb0 + (uint64_t)2 * C * Cfg::ES;                                  // V row 0
    const float c = scale * LOG2E;

    const uint32_t t0 = I * ST;
    const uint32_t qabs = t0 + 32u * w + r32; // this lane's query row
    u32x4 qf[NU];
    {
        const __amdgpu_buffer_rsrc_t rq = rsrc_at(qb0 + (uint64_t)t0 * ldb);
        const uint32_t row = 32u * w + r32;
        const bool row_ok = t0 + row < T;
#pragma unroll
        for (int u = 0; u < NQ; ++u) {
            const uint32_t ch = 2u * u + h;
            const uint32_t vo = (row_ok && ch * 16 < head_bytes) ? row * ldb + ch * 16 : OOB;
            qf[u] = __builtin_amdgcn_raw_buffer_load_b128(rq, (int)vo, 0, 0);
        }
    }
    OnlineRow rw{-__builtin_inff(), -__builtin_inff(), 0.f};
    f32x16 yacc[NBV];
#pragma unroll
    for (int nb = 0; nb < NBV; ++nb) yacc[nb] = f32x16{};
    const uint32_t nst = 2 * I + 2; // 64-key tiles 0 .. 2I + 1; the last two hold the diagonal
    if constexpr (Cfg::F32) {
        __shared__ __attribute__((aligned(16))) char kbuf[2 * KBYTES];
        __shared__ __attribute__((aligned(16))) char vbuf[2 * VBYTES];
        AStage<NCH> st;
        a_fetch<NCH>(st, kb0, vb0, 0, T, ldb, head_bytes, tid);
        a_store<NCH>(st, kbuf, vbuf, tid);
        __builtin_amdgcn_s_waitcnt(0x70); // vmcnt(0) lgkmcnt(0): Q and tile 0 in place
        tri::lds_barrier();
        uint32_t J = 0;
        for (; J + 2 < nst; ++J) {
            a_fetch<NCH>(st, kb0, vb0, J + 1, T, ldb, head_bytes, tid);
            online_step<E, NCH, NBV, false, NQ>(yacc, rw, kbuf + (J & 1) * KBYTES, vbuf + (J & 1) * VBYTES, qf, c,
                                            lane, J * AKT, qabs);
            a_store<NCH>(st, kbuf + ((J + 1) & 1) * KBYTES, vbuf + ((J + 1) & 1) * VBYTES, tid);
            tri::lds_barrier();
        }
        a_fetch<NCH>(st, kb0, vb0, J + 1, T, ldb, head_bytes, tid);
        online_step<E, NCH, NBV, true, NQ>(yacc, rw, kbuf, vbuf, qf, c, lane, J * AKT, qabs);
        a_store<NCH>(st, kbuf + KBYTES, vbuf + VBYTES, tid);
        tri::lds_barrier();
        online_step<E, NCH, NBV, true, NQ>(yacc, rw, kbuf + KBYTES, vbuf + VBYTES, qf, c, lane, (J + 1) * AKT, qabs);
    } else {
        // Tile J + 1 streams into the other buffer while step J runs; that
        // buffer's last readers (step J - 1) passed the barrier before. The
        // buffers are four separate arrays and the loop is unrolled by two,
        // so that every LDS read names its buffer: the compiler then knows
        // the loads in flight write elsewhere and does not wait for them.
        __shared__ __attribute__((aligned(16))) char k0s[KBYTES];
        __shared__ __attribute__((aligned(16))) char k1s[KBYTES];
        __shared__ __attribute__((aligned(16))) char v0s[KBYTES];
        __shared__ __attribute__((aligned(16))) char v1s[KBYTES];
        DStage16<NCH> ds;
        d16_init<NCH>(ds, w, lane, ldb, head_bytes);
        d16_fetch<NCH>(ds, k0s, v0s, kb0, vb0, 0, T, ldb, w);
        __builtin_amdgcn_s_waitcnt(0x70); // vmcnt(0) lgkmcnt(0): Q and tile 0 in place
        tri::lds_barrier();
        uint32_t J = 0;
        for (; J + 2 < nst; J += 2) { // nst is even
            d16_fetch<NCH>(ds, k1s, v1s, kb0, vb0, J + 1, T, ldb, w);
            online_step16<E, NCH, NBV, false, NQ>(yacc, rw, k0s, v0s, qf, c, lane, J * AKT, qabs);
            __builtin_amdgcn_s_waitcnt(0x70); // this wave's part of tile J + 1 in LDS
            tri::lds_barrier();
            d16_fetch<NCH>(ds, k0s, v0s, kb0, vb0, J + 2, T, ldb, w);
            online_step16<E, NCH, NBV, false, NQ>(yacc, rw, k1s, v1s, qf, c, lane, (J + 1) * AKT, qabs);
            __builtin_amdgcn_s_waitcnt(0x70);
            tri::lds_barrier();
        }
        d16_fetch<NCH>(ds, k1s, v1s, kb0, vb0, J + 1, T, ldb, w);
        online_step16<E, NCH, NBV, true, NQ>(yacc, rw, k0s, v0s, qf, c, lane, J * AKT, qabs);
        __builtin_amdgcn_s_waitcnt(0x70);
        tri::lds_barrier();
        online_step16<E, NCH, NBV, true, NQ>(yacc, rw, k1s, v1s, qf, c, lane, (J + 1) * AKT, qabs);
    }

    // y = Y / l and the statistics; the lane halves hold disjoint keys of one row.
    const float lt = halves_sum(rw.l);
    const float inv = 1.f / lt;
    if (qabs < T) {
        float *yr = y + ((uint64_t)b * T + qabs) * C + (uint64_t)nh * HS;
#pragma unroll
        for (int nb = 0; nb < NBV; ++nb)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const uint32_t d0 = 32u * nb + 8u * g + 4u * h; // head columns d0 .. d0 + 3
                if (d0 < HS) {
                    const tri::f32x4v v = {yacc[nb][4 * g] * inv, yacc[nb][4 * g + 1] * inv, yacc[nb][4 * g + 2] * inv,
                                      yacc[nb][4 * g + 3] * inv};
                    if (vec_y) {
                        *reinterpret_cast<tri::f32x4v *>(yr + d0) = v;
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e) yr[d0 + e] = v[e];
                    }
                }
            }
        if (h == 0) {
            const uint64_t o = (uint64_t)plane * T + qabs;
            row_max[o] = rw.mt * scale;
            // ln sum exp(x - max) = (log2 l + ms - mt c) ln 2; mt c - ms in [0, ONLINE_TAU], one rounding
            row_logsum[o] = (__builtin_amdgcn_logf(lt) - fmaf(rw.mt, c, -rw.ms)) * LN2;
        }
    }
}

// Single-pass attention: y into a.out ((B, T, C) fp32, 16-byte stores when
// a.vec_store), the statistics into a.row_max / a.row_logsum.
template <class E> hipError_t launch_attention_online_impl(const TrimulArgs &a, hipStream_t s)
{
    if constexpr (!std::is_same<E, KF32>::value) { // 16-bit heads of 257 .. 512 bytes
        if (a.HS * E::ES > 256)
            return launch_attention_online_wide16(a, std::is_same<E, KBF16>::value ? E_BF16 : E_F16, s);
    }
    return launch_longest_first(a, s, [&](dim3 grid, uint32_t nt, uint32_t planes, uint32_t rank0) {
        if (a.HS * AttnCfg<E, 8>::ES <= 128)
            hipLaunchKernelGGL((attention_online_kernel<E, 8>), grid, dim3(STATS_THREADS), 0, s, (const char *)a.qkv,
                               const_cast<float *>(a.row_max), const_cast<float *>(a.row_logsum), (float *)a.out,
                               (uint32_t)a.T, (uint32_t)a.C, (uint32_t)a.NH, (uint32_t)a.HS, nt, planes, rank0,
                               a.scale, (int)a.vec_store);
        else if (a.HS * AttnCfg<E, 8>::ES <= 256)
            hipLaunchKernelGGL((attention_online_kernel<E, 16>), grid, dim3(STATS_THREADS), 0, s,
                               (const char *)a.qkv, const_cast<float *>(a.row_max),
                               const_cast<float *>(a.row_logsum), (float *)a.out, (uint32_t)a.T, (uint32_t)a.C,
                               (uint32_t)a.NH, (uint32_t)a.HS, nt, planes, rank0, a.scale, (int)a.vec_store);
        else if constexpr (std::is_same<E, KF32>::value) { // fp32 heads of 257 .. 512 bytes
            if (a.HS * E::ES <= 384)
                hipLaunchKernelGGL((attention_online_kernel<E, 32, 12>), grid, dim3(STATS_THREADS), 0, s,
                                   (const char *)a.qkv, const_cast<float *>(a.row_max),
                                   const_cast<float *>(a.row_logsum), (float *)a.out, (uint32_t)a.T, (uint32_t)a.C,
                                   (uint32_t)a.NH, (uint32_t)a.HS, nt, planes, rank0, a.scale, (int)a.vec_store);
            else
                hipLaunchKernelGGL((attention_online_kernel<E, 32>), grid, dim3(STATS_THREADS), 0, s,
                                   (const char *)a.qkv, const_cast<float *>(a.row_max),
                                   const_cast<float *>(a.row_logsum), (float *)a.out, (uint32_t)a.T, (uint32_t)a.C,
                                   (uint32_t)a.NH, (uint32_t)a.HS, nt, planes, rank0, a.scale, (int)a.vec_store);
        }
    });
}

// 16-bit heads of 257 .. 512 bytes (32 pieces per row): the kernels of the
// launchers above, compiled in their own translation unit
// (softmax_wide16.hip) without the VGPR-only MFMA form, so that their 8 x 16
// output accumulators can live in the accumulation registers.
// Heads of at most 384 bytes multiply 12 of the row's 16 chunk pairs.
template <class E> hipError_t launch_row_stats_wide16_impl(const TrimulArgs &a, hipStream_t s)
{
    return a.HS * E::ES <= 384 ? launch_row_stats_nch<E, 32, 12>(a, s) : launch_row_stats_nch<E, 32>(a, s);
}
template <class E> hipError_t launch_attention_wide16_impl(const TrimulArgs &a, hipStream_t s)
{
    return a.HS * E::ES <= 384 ? launch_attention_nch<E, 32, 12>(a, s) : launch_attention_nch<E, 32>(a, s);
}
template <class E, int NQ> hipError_t launch_attention_online_wide16_nq(const TrimulArgs &a, hipStream_t s)
{
    return launch_longest_first(a, s, [&](dim3 grid, uint32_t nt, uint32_t planes, uint32_t rank0) {
        hipLaunchKernelGGL((attention_online_kernel<E, 32, NQ>), grid, dim3(STATS_THREADS), 0, s, (const char *)a.qkv,
                           const_cast<float *>(a.row_max), const_cast<float *>(a.row_logsum), (float *)a.out,
                           (uint32_t)a.T, (uint32_t)a.C, (uint32_t)a.NH, (uint32_t)a.HS, nt, planes, rank0, a.scale,
                           (int)a.vec_store);
    });
}
template <class E> hipError_t launch_attention_online_wide16_impl(const TrimulArgs &a, hipStream_t s)
{
    return a.HS * E::ES <= 384 ? launch_attention_online_wide16_nq<E, 12>(a, s)
                               : launch_attention_online_wide16_nq<E, 16>(a, s);
}

} // namespace sm
} // namespace cas
