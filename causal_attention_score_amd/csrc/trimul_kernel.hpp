// trimul_kernel.hpp -- causal attention scores straight from packed QKV on gfx950.
//
// Semantics: llm.c dev/cuda/trimat_forward.cu, trimul_cpu ("the Referee",
// Chapter I): out[b,nh,t,t2] = (Q[b,t,nh,:] . K[b,t2,nh,:]) * s for t2 <= t
// and NaN above the diagonal, with s = fp32 nearest 1/sqrt(HS).
//
// Design (MI355X-first; differs from that file's GPU kernels on purpose):
//  * Work item = one 64x64 score tile. Only on- and below-diagonal tiles are
//    items: item -> (plane, i, j <= i) by inverting the triangular numbers. A
//    diagonal tile masks its upper part to NaN; an off-diagonal tile (i, j)
//    also writes its mirror tile (j, i) as NaN, so one launch writes the
//    whole (T, T) plane.
//  * Wave specialisation. A workgroup holds four compute waves and four store
//    waves (one of each per SIMD). A compute wave fetches its tile's Q and K
//    rows straight from the packed (B, T, 3, NH, HS) rows (pitch 3C: no
//    permute pass, V never read) into registers, prefetching the next pass
//    while the MFMAs of the current one run, then writes the scaled, masked
//    tile to LDS. A store wave streams the previous tile from LDS to HBM with
//    16-byte non-temporal stores, plus the NaN mirror tile. Compute waves issue
//    no global stores and store waves no global loads, so neither ever waits
//    on the other's memory latency (one vmcnt counts both on CDNA); the two
//    sides meet at one LDS-only barrier per step, double-buffered.
//  * Persistent grid sized to residency; the item list is split into eight
//    contiguous ranges, one per XCD (workgroups are dispatched to XCDs round
//    robin), so the Q and K rows of a plane stay within one XCD's L2.
//  * Any T >= 1, any HS >= 1: rows past T and head entries past HS are zero
//    at fetch (local padding), writes are masked; offsets are 64-bit.
//
// Contraction-order permutation: in each 16-byte chunk pair of a row, lane
// half h = lane/32 (the MFMA k-slot) takes chunk 2u + h, for A (Q) and B (K)
// alike, so each product q_k * k_k is formed exactly once.
#pragma once

#include "launch.hpp"
#include "tile_engine.hpp"

#include <cstdlib>
#include <cstring>
#include <type_traits>

namespace cas {
namespace tri {

constexpr int TB = 64;         // score tile edge
constexpr int NCOMP = 4;       // compute waves per workgroup (one per SIMD)
constexpr int NTHREADS = 2 * NCOMP * 64;
constexpr int TILE_BYTES = TB * TB * 4;
constexpr unsigned QNAN_BITS = 0x7FC00000u;

// Output element kinds of the scores: fp32, or the fp32 score rounded once
// more to bfloat16 / binary16 (nearest even). The mask above the diagonal is
// that format's quiet NaN. NAN_DW: the mask pattern filling one dword.
struct OF32 {
    static constexpr int OB = 4;
    static constexpr uint32_t NAN_DW = QNAN_BITS;
};
struct OBF16 {
    static constexpr int OB = 2;
    static constexpr uint32_t NAN16 = 0x7FC0u, NAN_DW = 0x7FC07FC0u;
};
struct OF16 {
    static constexpr int OB = 2;
    static constexpr uint32_t NAN16 = 0x7E00u, NAN_DW = 0x7E007E00u;
};
__device__ __forceinline__ uint32_t round16(OBF16, float y) { return __builtin_bit_cast(unsigned short, (__bf16)y); }
__device__ __forceinline__ uint32_t round16(OF16, float y) { return __builtin_bit_cast(unsigned short, (_Float16)y); }
__device__ __forceinline__ void st_nt16(char *p, uint32_t v)
{
    __builtin_nontemporal_store((unsigned short)v, reinterpret_cast<unsigned short *>(p));
}

// What the score kernel writes per element (the epilogue):
//   EpScore  the scaled score, NaN above the diagonal (llm.c trimul_cpu);
//   EpLog    the log-probability (x - max) - logsum of the causal softmax,
//            -inf above the diagonal;
//   EpProb   its exponential, the probability, 0 above the diagonal.
// The softmax takes each row's max and logsum from the row-stats kernel
// (smallem "Kernels GPU", the softmax in two launches: row_stats, then
// softmax_rows), recomputing the scores instead of reading them back.
struct EpScore { static constexpr int KIND = 0; };
struct EpLog { static constexpr int KIND = 1; };
struct EpProb { static constexpr int KIND = 2; };

// Fill of the masked entries, as one element's bits (fill32 for fp32 output,
// fill16 for the 16-bit types) and as a dword of them.
template <class EP> constexpr uint32_t fill32() { return EP::KIND == 0 ? QNAN_BITS : EP::KIND == 1 ? 0xFF800000u : 0u; }
template <class O, class EP> constexpr uint32_t fill16()
{
    if constexpr (EP::KIND == 0) return O::NAN16;
    else if constexpr (EP::KIND == 1) return std::is_same<O, OBF16>::value ? 0xFF80u : 0xFC00u; // -inf
    else return 0u;
}
template <class O, class EP> constexpr uint32_t fill_dw()
{
    if constexpr (O::OB == 4) return fill32<EP>();
    else return fill16<O, EP>() | (fill16<O, EP>() << 16);
}

typedef float f32x4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void st_nt(float *p, float v) { __builtin_nontemporal_store(v, p); }
__device__ __forceinline__ void st_nt4(float *p, f32x4v v) { __builtin_nontemporal_store(v, reinterpret_cast<f32x4v *>(p)); }

// Keep a value opaque to the optimiser inside the loop, so address arithmetic
// built on it is recomputed cheaply instead of hoisted into a register per use.
__device__ __forceinline__ uint32_t opaque(uint32_t v)
{
    asm volatile("" : "+v"(v));
    return v;
}
__device__ __forceinline__ uint32_t opaque_s(uint32_t v)
{
    asm volatile("" : "+s"(v));
    return v;
}

// LDS-only workgroup barrier: outstanding global stores are not waited for.
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// One 64-row operand block of a wave in MFMA layout: block mb (rows
// mb*32 + lane%32), chunk pair u (chunk 2u + lane/32 of the row's pass).
template <int U> struct Operand {
    u32x4 c[2][U];
};

// A work item, all fields wave-uniform.
struct Tile {
    const char *q; // Q row t0 of (b, nh)
    const char *k; // K row s0 of (b, nh)
    char *o;       // out plane (b, nh)
    int64_t t0, s0;
    int64_t sr;    // index of row t0 in the (B, NH, T) row statistics
    int rl, cl;    // rows / columns of the tile inside the plane (<= 64)
    bool diag;
};

__device__ __forceinline__ Tile make_tile(const char *qkv, float *out, int64_t id, int64_t L, int64_t T, int64_t C,
                                          int64_t NH, int64_t HS, int es, int ob = 4)
{
    Tile tl;
    const int64_t plane = id / L;
    const int64_t r = id - plane * L;
    // r = i(i+1)/2 + j, 0 <= j <= i
    int64_t i = (int64_t)((sqrtf(8.0f * (float)r + 1.0f) - 1.0f) * 0.5f);
    while (i * (i + 1) / 2 > r) --i;
    while ((i + 1) * (i + 2) / 2 <= r) ++i;
    const int64_t j = r - i * (i + 1) / 2;
    const int64_t b = plane / NH, nh = plane - b * NH;
    const int64_t C3 = 3 * C;
    tl.t0 = i * TB;
    tl.s0 = j * TB;
    tl.sr = plane * T + tl.t0;
    tl.q = qkv + ((b * T + tl.t0) * C3 + nh * HS) * es;
    tl.k = qkv + ((b * T + tl.s0) * C3 + C + nh * HS) * es;
    tl.o = reinterpret_cast<char *>(out) + plane * T * T * ob;
    tl.rl = (int)((T - tl.t0) < TB ? (T - tl.t0) : TB);
    tl.cl = (int)((T - tl.s0) < TB ? (T - tl.s0) : TB);
    tl.diag = i == j;
    return tl;
}

// Buffer resource over `base` (wave-uniform). Offsets at or above OOB read
// as zero: the hardware range check does the zero-fill of local padding.
constexpr uint32_t OOB = 0x80000000u;
constexpr int ST_NT = 2; // cache-policy operand of buffer stores: non-temporal
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_at(const char *base)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(base), (short)0, 0x7FFFFFFF, 0x00020000);
}

// Fetch head entries [e0, e0 + U*32/ES) of 64 rows starting at `base`
// (uniform), row pitch ldb bytes; rows at or past `rows` and entries at or
// past HS are zero.
//   VEC16 (16-byte aligned rows, HS*ES % 16 == 0): one unconditional 16-byte
//   buffer load per chunk, out-of-range lanes pointed past the record count.
//   Otherwise (unaligned or ragged head) elements are fetched one by one.
template <class E, int U, bool VEC16>
__device__ __forceinline__ void fetch_rows(Operand<U> &op, const char *__restrict__ base, uint32_t ldb, int rows,
                                           int64_t HS, int64_t e0, int lane)
{
    constexpr int ES = E::ES;
    constexpr int EPC = 16 / ES; // elements per chunk
    const int h = lane >> 5;
    if constexpr (VEC16) {
        const __amdgpu_buffer_rsrc_t rs = rsrc_at(base);
        const bool full = e0 + (int64_t)U * 2 * EPC <= HS; // uniform
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
            const int r = mb * 32 + (lane & 31);
            const uint32_t ro = (uint32_t)r * ldb + (uint32_t)(e0 * ES) + (uint32_t)h * 16;
            const uint32_t rv = r < rows ? ro : OOB;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                uint32_t vo = rv + u * 32;
                if (!full) vo = (e0 + (int64_t)(2 * u + h) * EPC < HS) ? vo : OOB;
                op.c[mb][u] = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)vo, 0, 0);
            }
        }
    } else {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
            const int r = mb * 32 + (lane & 31);
            const bool row_ok = r < rows;
            const char *rp0 = base + (uint64_t)r * ldb + e0 * ES;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t e = e0 + (int64_t)(2 * u + h) * EPC; // first head entry of the chunk
                unsigned w[4] = {0u, 0u, 0u, 0u};
                if (row_ok) {
                    const char *rp = rp0 + (2 * u + h) * 16;
#pragma unroll
                    for (int x = 0; x < EPC; ++x) {
                        if (e + x < HS) {
                            unsigned bitsv;
                            if constexpr (ES == 4) bitsv = *reinterpret_cast<const unsigned *>(rp + x * 4);
                            else bitsv = *reinterpret_cast<const unsigned short *>(rp + x * 2);
                            w[(x * ES) / 4] |= bitsv << (((x * ES) % 4) * 8);
                        }
                    }
                }
                op.c[mb][u] = u32x4{w[0], w[1], w[2], w[3]};
            }
        }
    }
}

// All four 32x32 blocks, also on diagonal tiles: there block (0, 1) lies
// above the diagonal and is masked to NaN on the way out; a branch around its
// MFMAs would make the compiler copy the accumulators, waiting on the matrix
// pipe.
template <class E, int U>
__device__ __forceinline__ void mma_pass(f32x16 (&acc)[2][2], const Operand<U> &q, const Operand<U> &k)
{
#pragma unroll
    for (int u = 0; u < U; ++u) {
        mfma_chunk<E>(acc[0][0], q.c[0][u], k.c[0][u]);
        mfma_chunk<E>(acc[0][1], q.c[0][u], k.c[1][u]);
        mfma_chunk<E>(acc[1][0], q.c[1][u], k.c[0][u]);
        mfma_chunk<E>(acc[1][1], q.c[1][u], k.c[1][u]);
    }
}

template <class EP> __device__ __forceinline__ float epilogue(float a, float scale, float mx, float ls);

// Scaled, masked tile -> LDS, row-major 64 x 64 fp32. EP other than the
// scores: the softmax epilogue of each element, st holding the tile rows'
// statistics (st[row] the row maximum, st[TB + row] the logsum), and that
// epilogue's fill right of the diagonal.
template <class EP = EpScore>
__device__ __forceinline__ void tile_to_lds(const f32x16 (&acc)[2][2], char *lds, float scale, bool diag, int lane,
                                            const float *st = nullptr)
{
    const float fill = __uint_as_float(fill32<EP>());
    const int c0 = lane & 31, h4 = 4 * (lane >> 5);
    const uint32_t lo = opaque((uint32_t)(h4 * TB + c0) * 4);
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            f32x4v mx4 = {}, ls4 = {}; // rows mb*32 + 8q + h4 .. + 3
            if constexpr (EP::KIND != 0) {
                mx4 = *reinterpret_cast<const f32x4v *>(st + mb * 32 + 8 * q + h4);
                ls4 = *reinterpret_cast<const f32x4v *>(st + TB + mb * 32 + 8 * q + h4);
            }
#pragma unroll
            for (int nb = 0; nb < 2; ++nb)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 4 * q + e;
                    const int rr = mb * 32 + 8 * q + e; // uniform part of the row
                    const int row = rr + h4, col = nb * 32 + c0;
                    float v;
                    if constexpr (EP::KIND == 0) v = acc[mb][nb][r] * scale;
                    else v = epilogue<EP>(acc[mb][nb][r], scale, mx4[e], ls4[e]);
                    if (diag && col > row) v = fill;
                    *reinterpret_cast<float *>(lds + lo + (uint32_t)(rr * TB + nb * 32) * 4) = v;
                }
        }
}

// LDS tile -> rows [t0, t0+rl) x columns [s0, s0+cl) of the plane. FULL:
// a whole 64x64 tile with 16-byte stores and no masks.
template <bool FULL>
__device__ __forceinline__ void lds_to_out(const char *lds, const Tile &tl, uint32_t T4, int lane, bool vec4)
{
    char *dst = tl.o + ((uint64_t)tl.t0 * (T4 / 4) + (uint64_t)tl.s0) * 4;
    if (FULL || vec4) { // T % 4 == 0 and 16-byte aligned: columns come in fours
        const int r4 = lane >> 4, c = (lane & 15) * 4;
        const uint32_t go = opaque((uint32_t)r4 * T4 + (uint32_t)c * 4);
        f32x4v v[TB / 4];
#pragma unroll
        for (int s = 0; s < TB / 4; ++s) v[s] = *reinterpret_cast<const f32x4v *>(lds + lane * 16 + s * 1024);
#pragma unroll
        for (int s = 0; s < TB / 4; ++s) {
            if (FULL || (c < tl.cl && s * 4 + r4 < tl.rl))
                st_nt4(reinterpret_cast<float *>(dst + ((uint32_t)(s * 4) * T4 + go)), v[s]);
        }
    } else {
        for (int s = 0; s < TB; ++s) {
            const float v = *reinterpret_cast<const float *>(lds + (s * TB + lane) * 4);
            if (s < tl.rl && lane < tl.cl) st_nt(reinterpret_cast<float *>(dst + ((uint32_t)s * T4 + (uint32_t)lane * 4)), v);
        }
    }
}

// NaN over the mirror tile (j, i): rows [s0, s0+cl) x columns [t0, t0+rl).
// H = 0 or 1 writes only the first or the second half of the mirror's rows,
// H = -1 all of them.
template <bool FULL, int H = -1, class EP = EpScore>
__device__ __forceinline__ void nan_mirror(const Tile &tl, uint32_t T4, int lane, bool vec4)
{
    constexpr int R0 = H == 1 ? TB / 2 : 0, R1 = H == 0 ? TB / 2 : TB; // mirror rows [R0, R1)
    const float qnan = __uint_as_float(fill32<EP>()); // the scores' NaN, or the softmax fill
    char *dst = tl.o + ((uint64_t)tl.s0 * (T4 / 4) + (uint64_t)tl.t0) * 4;
    if (FULL || vec4) {
        const f32x4v n4 = {qnan, qnan, qnan, qnan};
        const int r4 = lane >> 4, c = (lane & 15) * 4;
        const uint32_t go = opaque((uint32_t)r4 * T4 + (uint32_t)c * 4);
#pragma unroll
        for (int s = R0 / 4; s < R1 / 4; ++s)
            if (FULL || (c < tl.rl && s * 4 + r4 < tl.cl))
                st_nt4(reinterpret_cast<float *>(dst + ((uint32_t)(s * 4) * T4 + go)), n4);
    } else {
        for (int s = R0; s < R1; ++s)
            if (s < tl.cl && lane < tl.rl) st_nt(reinterpret_cast<float *>(dst + ((uint32_t)s * T4 + (uint32_t)lane * 4)), qnan);
    }
}

// 16-bit output from the tile kernel's fp32 LDS tile (row-major, TB floats
// per row), for output rows not in 16-byte pieces: one element per lane and
// row, rounded on the way out, the fp32 mask pattern turned into the
// format's quiet NaN. (This kernel serves the unaligned and wide-head
// shapes; the super-tile kernel has the fast path.)
template <class O>
__device__ __forceinline__ void lds_to_out16(const char *lds, const Tile &tl, int64_t T, int lane)
{
    for (int s = 0; s < TB; ++s) {
        const float v = *reinterpret_cast<const float *>(lds + (s * TB + lane) * 4);
        const uint32_t h = __float_as_uint(v) == QNAN_BITS ? O::NAN16 : round16(O{}, v);
        if (s < tl.rl && lane < tl.cl) st_nt16(tl.o + ((tl.t0 + s) * T + tl.s0 + lane) * 2, h);
    }
}

template <class O, class EP = EpScore>
__device__ __forceinline__ void nan_mirror16(const Tile &tl, int64_t T, int lane)
{
    for (int s = 0; s < TB; ++s)
        if (s < tl.cl && lane < tl.rl) st_nt16(tl.o + ((tl.s0 + s) * T + tl.t0 + lane) * 2, fill16<O, EP>());
}

// The same with 16-byte stores, for output rows in 16-byte pieces (T a
// multiple of 8, base 16-byte aligned; the tile's row and column counts are
// then multiples of 8 too): lane l covers columns 8(l%8) .. +7 of rows
// l/8 + 8s, eight rows of the tile per store instruction.
__device__ __forceinline__ uint32_t pack16(OBF16, float a, float b)
{
    const uint32_t lo = __float_as_uint(a) == QNAN_BITS ? OBF16::NAN16 : round16(OBF16{}, a);
    const uint32_t hi = __float_as_uint(b) == QNAN_BITS ? OBF16::NAN16 : round16(OBF16{}, b);
    return lo | (hi << 16);
}
__device__ __forceinline__ uint32_t pack16(OF16, float a, float b)
{
    const uint32_t lo = __float_as_uint(a) == QNAN_BITS ? OF16::NAN16 : round16(OF16{}, a);
    const uint32_t hi = __float_as_uint(b) == QNAN_BITS ? OF16::NAN16 : round16(OF16{}, b);
    return lo | (hi << 16);
}

template <class O>
__device__ __forceinline__ void lds_to_out16v(const char *lds, const Tile &tl, int64_t T, int lane)
{
    const int c = (lane & 7) * 8, r8 = lane >> 3;
    char *dst = tl.o + ((tl.t0 + r8) * T + tl.s0 + c) * 2;
#pragma unroll
    for (int s = 0; s < TB / 8; ++s) {
        const int row = r8 + 8 * s;
        const f32x4v a = *reinterpret_cast<const f32x4v *>(lds + (row * TB + c) * 4);
        const f32x4v b = *reinterpret_cast<const f32x4v *>(lds + (row * TB + c + 4) * 4);
        const u32x4 v = {pack16(O{}, a[0], a[1]), pack16(O{}, a[2], a[3]), pack16(O{}, b[0], b[1]),
                         pack16(O{}, b[2], b[3])};
        if (row < tl.rl && c < tl.cl)
            __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(dst + (int64_t)(8 * s) * T * 2));
    }
}

template <class O, class EP = EpScore>
__device__ __forceinline__ void nan_mirror16v(const Tile &tl, int64_t T, int lane)
{
    const int c = (lane & 7) * 8, r8 = lane >> 3;
    constexpr uint32_t F = fill_dw<O, EP>();
    const u32x4 v = {F, F, F, F};
    char *dst = tl.o + ((tl.s0 + r8) * T + tl.t0 + c) * 2;
#pragma unroll
    for (int s = 0; s < TB / 8; ++s)
        if (r8 + 8 * s < tl.cl && c < tl.rl)
            __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(dst + (int64_t)(8 * s) * T * 2));
}

// One step of a compute wave: the P register passes of tile `tl` (operands of
// pass 0 already in ops[SB]), prefetching each next pass -- and after the last
// pass the first pass of `nx` when has_next -- into the other buffer, then the
// scaled, masked tile to LDS. Afterwards nx's first pass sits in ops[(SB+P)%2].
// P == 0: any number of passes, each fetched and then multiplied (no prefetch).
//
// Softmax epilogue (EP other than EpScore): mxv / lsv are the statistics of
// row t0 + lane, loaded before the passes so their latency hides behind the
// MFMAs; the wave puts them in its slot st (64 maxima, then 64 logsums) for
// the cross-lane reads of tile_to_lds.
template <class E, int U, bool VEC16, int P, int SB, class EP = EpScore>
__device__ __forceinline__ void compute_tile(Operand<U> (&ops)[2][2], const Tile &tl, const Tile &nx, bool has_next,
                                             char *lds, uint32_t ldb, int64_t HS, float scale, int lane,
                                             float *st = nullptr, float mxv = 0.f, float lsv = 0.f)
{
    constexpr int64_t PASS = (int64_t)U * 32 / E::ES;
    f32x16 acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int c = 0; c < 2; ++c) acc[a][c] = f32x16{};
    if constexpr (P == 0) {
        for (int64_t e0 = 0; e0 < HS; e0 += PASS) {
            fetch_rows<E, U, VEC16>(ops[0][0], tl.q, ldb, tl.rl, HS, e0, lane);
            fetch_rows<E, U, VEC16>(ops[0][1], tl.k, ldb, tl.cl, HS, e0, lane);
            mma_pass<E, U>(acc, ops[0][0], ops[0][1]);
        }
    } else {
#pragma unroll
        for (int p = 0; p < P; ++p) {
            const int cur = (SB + p) & 1, nxt = cur ^ 1;
            if (p + 1 < P) {
                fetch_rows<E, U, VEC16>(ops[nxt][0], tl.q, ldb, tl.rl, HS, (p + 1) * PASS, lane);
                fetch_rows<E, U, VEC16>(ops[nxt][1], tl.k, ldb, tl.cl, HS, (p + 1) * PASS, lane);
            } else if (has_next) {
                fetch_rows<E, U, VEC16>(ops[nxt][0], nx.q, ldb, nx.rl, HS, 0, lane);
                fetch_rows<E, U, VEC16>(ops[nxt][1], nx.k, ldb, nx.cl, HS, 0, lane);
            }
            mma_pass<E, U>(acc, ops[cur][0], ops[cur][1]);
        }
    }
    if constexpr (EP::KIND != 0) {
        // One wave writes and reads its slot: LDS keeps a wave's accesses in
        // order, the fences keep the compiler from moving them.
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
        st[lane] = mxv;
        st[TB + lane] = lsv;
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront", "local");
    }
    tile_to_lds<EP>(acc, lds, scale, tl.diag, lane, st);
}

// EP other than EpScore: the causal softmax rows (log-probabilities or
// probabilities) from the per-row statistics row_max / row_logsum (B, NH, T).
template <class E, int U, bool VEC16, int P, class EP = EpScore>
__global__ void __launch_bounds__(NTHREADS)
trimul_kernel(const char *__restrict__ qkv, float *__restrict__ out, int64_t T, int64_t C, int64_t NH, int64_t HS,
              int64_t L, int64_t items, float scale, int vec_store, int out_kind, const float *__restrict__ row_max,
              const float *__restrict__ row_logsum)
{
    constexpr int ES = E::ES;
    constexpr bool SM = EP::KIND != 0;
    __shared__ __attribute__((aligned(16))) char lds[NCOMP * 2 * TILE_BYTES];
    __shared__ __attribute__((aligned(16))) float stl[SM ? NCOMP * 2 * TB : 4]; // per compute wave: 64 max, 64 logsum

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const bool compute = wave < NCOMP;
    const int slot = wave % NCOMP;
    char *my_lds = lds + slot * 2 * TILE_BYTES;

    // XCD-local contiguous item range (proportional to the workgroups on each
    // XCD); the workgroups of an XCD take NCOMP consecutive items per step.
    const int64_t nwg = gridDim.x;
    const int64_t x = blockIdx.x % 8, q8 = nwg / 8, r8 = nwg % 8;
    const int64_t wg_before = x * q8 + (x < r8 ? x : r8);
    const int64_t wg_on_x = q8 + (x < r8 ? 1 : 0);
    const int64_t lo = items * wg_before / nwg, hi = items * (wg_before + wg_on_x) / nwg;
    const int64_t first = lo + (blockIdx.x / 8) * NCOMP;
    const int64_t stride = wg_on_x * NCOMP;
    const int64_t steps = first < hi ? (hi - first + stride - 1) / stride : 0;

    const uint32_t T4 = (uint32_t)T * 4u;
    const uint32_t ldb = (uint32_t)(3 * C * ES);
    const bool vec4 = vec_store != 0;

    if (compute) {
        // Items of this wave: first + n*stride + slot for n < steps (while < hi).
        Operand<U> ops[2][2];
        int64_t id = first + slot;
        Tile tl = make_tile(qkv, out, id < hi ? id : lo, L, T, C, NH, HS, ES);
        if (P > 0 && id < hi) {
            fetch_rows<E, U, VEC16>(ops[0][0], tl.q, ldb, tl.rl, HS, 0, lane);
            fetch_rows<E, U, VEC16>(ops[0][1], tl.k, ldb, tl.cl, HS, 0, lane);
        }
        // Two steps per iteration so the operand buffers alternate statically.
        for (int64_t n = 0; n <= steps; n += 2) {
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const int64_t m = n + half;
                if (m <= steps) {
                    if (m < steps && id < hi) {
                        const int64_t nid = id + stride;
                        const bool has_next = m + 1 < steps && nid < hi;
                        const Tile nx = make_tile(qkv, out, has_next ? nid : id, L, T, C, NH, HS, ES);
                        char *buf = my_lds + (m & 1) * TILE_BYTES;
                        float mxv = 0.f, lsv = 0.f; // statistics of row t0 + lane (softmax)
                        if constexpr (SM) {
                            if (lane < tl.rl) {
                                mxv = row_max[tl.sr + lane];
                                lsv = row_logsum[tl.sr + lane];
                            }
                        }
                        float *st = stl + (SM ? slot * 2 * TB : 0);
                        if (half == 0 || (P & 1) == 0)
                            compute_tile<E, U, VEC16, P, 0, EP>(ops, tl, nx, has_next, buf, ldb, HS, scale, lane, st,
                                                                mxv, lsv);
                        else
                            compute_tile<E, U, VEC16, P, 1, EP>(ops, tl, nx, has_next, buf, ldb, HS, scale, lane, st,
                                                                mxv, lsv);
                        tl = nx;
                        id = nid;
                    }
                    lds_barrier();
                }
            }
        }
    } else {
        for (int64_t n = 0; n <= steps; ++n) {
            if (n >= 1) {
                const int64_t pid = first + (n - 1) * stride + slot;
                if (pid < hi && out_kind != 0) { // 16-bit output (out_kind is uniform)
                    const Tile tl = make_tile(qkv, out, pid, L, T, C, NH, HS, ES, 2);
                    const char *buf = my_lds + ((n - 1) & 1) * TILE_BYTES;
                    if (vec4) { // rows in 16-byte pieces
                        if (out_kind == 1) {
                            lds_to_out16v<OBF16>(buf, tl, T, lane);
                            if (!tl.diag) nan_mirror16v<OBF16, EP>(tl, T, lane);
                        } else {
                            lds_to_out16v<OF16>(buf, tl, T, lane);
                            if (!tl.diag) nan_mirror16v<OF16, EP>(tl, T, lane);
                        }
                    } else if (out_kind == 1) {
                        lds_to_out16<OBF16>(buf, tl, T, lane);
                        if (!tl.diag) nan_mirror16<OBF16, EP>(tl, T, lane);
                    } else {
                        lds_to_out16<OF16>(buf, tl, T, lane);
                        if (!tl.diag) nan_mirror16<OF16, EP>(tl, T, lane);
                    }
                } else if (pid < hi) {
                    const Tile tl = make_tile(qkv, out, pid, L, T, C, NH, HS, ES);
                    const uint32_t t4 = opaque_s(T4);
                    const char *buf = my_lds + ((n - 1) & 1) * TILE_BYTES;
                    if (tl.rl == TB && tl.cl == TB && vec4) {
                        lds_to_out<true>(buf, tl, t4, lane, vec4);
                        if (!tl.diag) nan_mirror<true, -1, EP>(tl, t4, lane, vec4);
                    } else {
                        lds_to_out<false>(buf, tl, t4, lane, vec4);
                        if (!tl.diag) nan_mirror<false, -1, EP>(tl, t4, lane, vec4);
                    }
                }
            }
            lds_barrier();
        }
    }
}

// ---------------------------------------------------------------------------
// Super-tile kernel (rows 16-byte aligned, HS*ES <= 256 bytes, or up to 512
// in two halves, HV below): a workgroup step is one 128x128 super-tile
// (I, J <= I). Its 128 Q rows and 128 K rows
// are fetched once, with coalesced 16-byte loads (8 or 16 lanes per row), into
// an XOR-swizzled LDS operand buffer: chunk c of row r sits at position
// c ^ (r % 8), so the MFMA operand reads (32 rows, one chunk) and the row
// writes are both free of bank conflicts. Three roles of four waves each, one
// wave of every role per SIMD:
//  * compute wave w multiplies sub-tile (w/2, w%2) as D = K Q^T (K rows are
//    the MFMA A operand), so a lane's four consecutive accumulators are four
//    consecutive output columns, and writes the raw tile to LDS with 16-byte
//    writes. It issues no global memory instruction at all.
//  * store wave w reads the tile back, applies the scale and the causal mask
//    and streams it to HBM with its NaN mirror (non-temporal 16-byte stores).
//  * loader wave w requests its quarter of the next step's operand rows into
//    registers and writes them to the operand buffer once it is free.
// On CDNA the loads and stores of a CU share one vector-memory queue, which
// the store stream keeps full: a load waits behind the stores ahead of it.
// Only the loader waves ever wait there, and they have a whole MFMA phase to
// do so, so the waves that gate the barriers never stall on memory.
// Two LDS-only barriers per step:
//   compute: MFMA(n)                        | X | acc(n) -> out LDS       | Y
//   loader:  fetch rows(n+1) -> registers   | X | rows(n+1) -> opnd LDS  | Y
//   store:   tile(n-1), 1st half mirror(n-1)| X | 2nd half mirror(n-1)   | Y
// A step lasts the longer side of each segment, added up. The store waves
// keep the write stream busy through both: the NaN mirror needs nothing from
// LDS, so half of it fills the short LDS segment and half follows tile n-1
// through the long MFMA segment. The output buffer is rewritten only after
// X, which a store wave reaches once its reads of the previous tile are done.
// On a diagonal super-tile, sub-tile (0, 1) lies wholly above the diagonal
// and is written as NaN; (0, 0) and (1, 1) are masked diagonal tiles.
// ---------------------------------------------------------------------------
constexpr int ST = 2 * TB;                    // super-tile edge
constexpr int OP_ROWS = 2 * ST;               // 128 Q rows + 128 K rows
constexpr int NCOMP_THREADS = NCOMP * 64;   // lanes of one role
constexpr int SUPER_THREADS = 3 * NCOMP_THREADS;
// LDS output rows: TB elements of the output type plus 16 bytes of bank skew.
template <class O> constexpr int out_pitch() { return TB * O::OB + 16; }

struct Super {
    uint32_t plane, T0, S0;
    bool diag;
};

// Walks the items first, first + step, ... of the per-plane triangles (row i
// holds the i + 1 super-tiles j = 0..i) as (plane, i, j). The set-up decodes
// `first` once; each advance moves whole planes, then row by row, with
// scalar integer arithmetic only: the waves that share a SIMD with the fp32
// MFMAs get few vector issue slots.
struct Walker {
    uint32_t plane, i, j, dp, dr, nt;
    __device__ __forceinline__ void init(uint32_t first, uint32_t step, uint32_t L, uint32_t nt_)
    {
        nt = nt_;
        plane = first / L;
        const uint32_t r = first - plane * L;
        dp = step / L;
        dr = step - dp * L;
        // r = i(i+1)/2 + j, 0 <= j <= i
        uint32_t q = (uint32_t)((sqrtf(8.0f * (float)r + 1.0f) - 1.0f) * 0.5f);
        while (q * (q + 1) / 2 > r) --q;
        while ((q + 1) * (q + 2) / 2 <= r) ++q;
        i = __builtin_amdgcn_readfirstlane(q);
        j = __builtin_amdgcn_readfirstlane(r - q * (q + 1) / 2);
    }
    __device__ __forceinline__ void advance()
    {
        plane += dp;
        j += dr;
        while (j > i) {
            j -= i + 1;
            if (++i == nt) {
                i = 0;
                ++plane;
            }
        }
    }
    __device__ __forceinline__ Super item() const
    {
        Super sp;
        sp.plane = plane;
        sp.T0 = i * ST;
        sp.S0 = j * ST;
        sp.diag = i == j;
        return sp;
    }
};

// Rows of the next super-tile, NCH 16-byte chunks per row, in registers.
template <int NCH> struct Staged {
    u32x4 v[NCH];
};

// Coalesced fetch of the 256 operand rows of super-tile `sp` (loader lane
// cl = wave*64 + lane of 256): chunk j*256 + cl is row (j*256 + cl) / NCH,
// chunk (cl % NCH). Rows past T and chunks past the head read zero. hoff:
// the first head byte fetched (the second half of a wide head). PART: a head
// row that ends inside a 16-byte piece; that piece's bytes past the head
// (the next head's, or the next slot's: never past the packed row) are
// zeroed in registers.
template <class E, int NCH, bool PART = false>
__device__ __forceinline__ void stage_fetch(Staged<NCH> &st, const char *qkv, const Super &sp, uint32_t T, uint32_t C,
                                            uint32_t NH, uint32_t HS, uint32_t ldb, int cl, bool with_q = true,
                                            uint32_t hoff = 0)
{
    constexpr int ES = E::ES;
    constexpr int RPJ = NCOMP_THREADS / NCH; // rows per j
    const uint32_t b = sp.plane / NH, nh = sp.plane - b * NH;
    const uint64_t rowq = (uint64_t)b * T + sp.T0, rowk = (uint64_t)b * T + sp.S0;
    const char *qb = qkv + (rowq * (3u * C) + (uint64_t)nh * HS) * ES + hoff;
    const char *kb = qkv + (rowk * (3u * C) + C + (uint64_t)nh * HS) * ES + hoff;
    const __amdgpu_buffer_rsrc_t rq = rsrc_at(qb), rk = rsrc_at(kb);
    const uint32_t c = (uint32_t)(cl % NCH), r0 = (uint32_t)(cl / NCH);
    const uint32_t lim = hoff + c * 16 < HS * ES ? T : 0u; // a chunk past the head reads zero
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
        const bool isq = j < NCH / 2; // uniform: rows 0..127 are Q, 128..255 K
        if (isq && !with_q) continue;   // Q rows already in LDS
        const uint32_t rin = (uint32_t)((isq ? j : j - NCH / 2) * RPJ) + r0;
        const uint32_t ok = 0u - (uint32_t)((isq ? sp.T0 : sp.S0) + rin < lim); // all ones in range
        const uint32_t vo = ((rin * ldb + c * 16) & ok) | (OOB & ~ok);
        st.v[j] = __builtin_amdgcn_raw_buffer_load_b128(isq ? rq : rk, (int)vo, 0, 0);
    }
    if constexpr (PART) {
        const uint32_t cb = hoff + c * 16, hb = HS * ES; // the lane's piece, the head's bytes
        if (cb < hb && hb < cb + 16) {
            u32x4 keep;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const uint32_t b0 = cb + 4u * w; // bytes b0 .. b0 + 3 of the row
                keep[w] = b0 + 4 <= hb ? 0xFFFFFFFFu : b0 >= hb ? 0u : (1u << (8u * (hb - b0))) - 1u;
            }
#pragma unroll
            for (int j = 0; j < NCH; ++j) st.v[j] &= keep;
        }
    }
}

template <int NCH>
__device__ __forceinline__ void stage_store(const Staged<NCH> &st, char *opb, int cl, bool with_q = true)
{
    constexpr int RPJ = NCOMP_THREADS / NCH;
    const int c = cl % NCH;
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
        if (j < NCH / 2 && !with_q) continue; // Q rows already in LDS
        const int row = j * RPJ + cl / NCH;
        *reinterpret_cast<u32x4 *>(opb + row * (NCH * 16) + ((c ^ (row & 7)) << 4)) = st.v[j];
    }
}

// Operand fragments of one chunk pair: K rows (A operand) and Q rows (B).
struct Frag {
    u32x4 k0, k1, q0, q1;
};

template <int NCH>
__device__ __forceinline__ Frag read_frag(const char *krow, const char *qrow, int u, int h, int xr)
{
    constexpr int RB = NCH * 16;
    const int pos = ((2 * u + h) ^ xr) << 4;
    Frag f;
    f.k0 = *reinterpret_cast<const u32x4 *>(krow + pos);
    f.k1 = *reinterpret_cast<const u32x4 *>(krow + 32 * RB + pos);
    f.q0 = *reinterpret_cast<const u32x4 *>(qrow + pos);
    f.q1 = *reinterpret_cast<const u32x4 *>(qrow + 32 * RB + pos);
    return f;
}

// Sub-tile (a, b) of the super-tile: acc[kb][qb] covers output columns
// 32kb.. (K rows 128 + 64b + 32kb..) and output rows 32qb.. (Q rows
// 64a + 32qb..). The LDS reads run two chunk pairs ahead of the MFMAs. On a
// diagonal sub-tile the block (kb=1, qb=0) lies above the diagonal; it is
// computed anyway and masked to NaN on the way out: a branch around its MFMAs
// would make the compiler copy the accumulators, waiting on the matrix pipe.
// NU: the chunk pairs multiplied (fewer than NCH / 2 when the rest of the
// staged rows is known to be zero).
template <class E, int NCH, int NU = NCH / 2>
__device__ __forceinline__ void sub_mma(f32x16 (&acc)[2][2], const char *opb, int a, int b, int lane)
{
    constexpr int RB = NCH * 16;
    static_assert(NU >= 1 && NU <= NCH / 2, "chunk pairs of the staged rows");
    const int r32 = lane & 31, h = lane >> 5, xr = r32 & 7;
    const char *qrow = opb + (a * TB + r32) * RB;
    const char *krow = opb + (ST + b * TB + r32) * RB;
    Frag f[3];
    f[0] = read_frag<NCH>(krow, qrow, 0, h, xr);
    if (NU > 1) f[1] = read_frag<NCH>(krow, qrow, 1, h, xr);
#pragma unroll
    for (int u = 0; u < NU; ++u) {
        __builtin_amdgcn_sched_barrier(0);
        if (u + 2 < NU) f[(u + 2) % 3] = read_frag<NCH>(krow, qrow, u + 2, h, xr);
        __builtin_amdgcn_sched_barrier(0);
        const Frag &g = f[u % 3];
        mfma_chunk<E>(acc[0][0], g.k0, g.q0);
        mfma_chunk<E>(acc[0][1], g.k0, g.q1);
        mfma_chunk<E>(acc[1][0], g.k1, g.q0);
        mfma_chunk<E>(acc[1][1], g.k1, g.q1);
    }
}

// The element written for accumulator value a: the fp32 score a * scale;
// for log-probabilities (x - max) - logsum of its row, where the empty asm
// keeps the score a separate fp32 value (the compiler may not fuse its
// rounding into the subtraction); for probabilities the exponential of the
// log-probability, formed in base 2 (v_exp_f32).
template <class EP>
__device__ __forceinline__ float epilogue(float a, float scale, float mx, float ls)
{
    constexpr float LOG2E = 1.44269504088896340736f;
    if constexpr (EP::KIND == 2) {
        // p = 2^((a scale - mx) log2 e - ls log2 e): two fused multiply-adds,
        // each one rounding, and ls log2 e once per row. Every rounding is
        // relative to lp or to ls <= |lp| (x <= mx and ls >= 0), never to
        // the size of the scores themselves.
        const float t = __builtin_fmaf(a, scale, -mx);
        return __builtin_amdgcn_exp2f(__builtin_fmaf(t, LOG2E, -(ls * LOG2E)));
    }
    float y = a * scale;
    if constexpr (EP::KIND == 1) {
        asm volatile("" : "+v"(y));
        y = (y - mx) - ls;
    }
    return y;
}

// Sub-tile -> LDS rows of out_pitch<O>() bytes, already in the output type.
// Lane l holds output row 32qb + l%32 and columns 32kb + 8g + 4(l/32) + 0..3
// of acc[kb][qb][4g..]: one 16-byte (fp32) or 8-byte (16-bit) write.
// DIAG: a sub-tile on the diagonal, whose entries right of it are masked.
// mx / ls: the softmax statistics of the lane's two rows (qb = 0, 1).
template <bool DIAG, class O, class EP = EpScore>
__device__ __forceinline__ void subtile_to_lds(const f32x16 (&acc)[2][2], char *lds, float scale, int lane,
                                               const float (&mx)[2], const float (&ls)[2])
{
    constexpr int PITCH = out_pitch<O>();
    const int r32 = lane & 31, h4 = 4 * (lane >> 5);
    const uint32_t lo = opaque((uint32_t)(r32 * PITCH + h4 * O::OB));
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                char *dst = lds + lo + (uint32_t)(32 * qb * PITCH + (32 * kb + 8 * g) * O::OB);
                if constexpr (O::OB == 4) {
                    const float fill = __uint_as_float(fill32<EP>());
                    f32x4v v;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float y = epilogue<EP>(acc[kb][qb][4 * g + e], scale, mx[qb], ls[qb]);
                        v[e] = (DIAG && 32 * kb + 8 * g + h4 + e > 32 * qb + r32) ? fill : y;
                    }
                    *reinterpret_cast<f32x4v *>(dst) = v;
                } else {
                    uint32_t hv[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        // The fp32 value first, then the 16-bit rounding: kept
                        // apart so the arithmetic and the conversion do not
                        // fuse into one rounding (a mixed-precision FMA would).
                        float y32 = epilogue<EP>(acc[kb][qb][4 * g + e], scale, mx[qb], ls[qb]);
                        asm volatile("" : "+v"(y32));
                        const uint32_t y = round16(O{}, y32);
                        hv[e] = (DIAG && 32 * kb + 8 * g + h4 + e > 32 * qb + r32) ? fill16<O, EP>() : y;
                    }
                    *reinterpret_cast<u32x2 *>(dst) = u32x2{hv[0] | (hv[1] << 16), hv[2] | (hv[3] << 16)};
                }
            }
}

// Store geometry of a 64 x 64 output tile in 16-byte pieces: LPR lanes per
// row, RPI rows per store instruction, NI instructions per tile, EPC
// elements per piece.
template <class O> struct Pieces {
    static constexpr int LPR = TB * O::OB / 16, RPI = 64 / LPR, NI = TB / RPI, EPC = 16 / O::OB;
};

// Store one element (index e of a 16-byte piece) of the output type.
template <class O> __device__ __forceinline__ void st_elem(char *p, const u32x4 &v, int e)
{
    if constexpr (O::OB == 4) st_nt(reinterpret_cast<float *>(p), __uint_as_float(v[e]));
    else st_nt16(p, v[e >> 1] >> (16 * (e & 1)));
}

// Rows [32H, 32H + 32) of the mirror of tile `tl` (rows s0.. of the plane,
// columns t0..), all masked (NaN for scores, EP's fill for the softmax): whole tiles with buffer stores whose row offset is a
// scalar (no vector ALU work per store); else masked to the plane, 16 bytes
// at a time when rows are 16-byte aligned (vec), one element otherwise.
template <int H, class O, bool FULL, class EP = EpScore>
__device__ __forceinline__ void nan_mirror_o(const Tile &tl, uint32_t T, uint32_t tby, int lane, bool vec)
{
    using PC = Pieces<O>;
    char *base = tl.o + ((uint64_t)tl.s0 * T + (uint64_t)tl.t0) * O::OB;
    constexpr uint32_t F = fill_dw<O, EP>();
    const u32x4 n4 = {F, F, F, F};
    const int rr = lane / PC::LPR, cc = (lane % PC::LPR) * PC::EPC;
    constexpr int S0 = H * PC::NI / 2, S1 = S0 + PC::NI / 2;
    if (FULL) {
        const __amdgpu_buffer_rsrc_t rs = rsrc_at(base);
        const uint32_t go = opaque((uint32_t)rr * tby + (uint32_t)(cc * O::OB));
#pragma unroll
        for (int s = S0; s < S1; ++s)
            __builtin_amdgcn_raw_buffer_store_b128(n4, rs, (int)go, (int)((uint32_t)(s * PC::RPI) * tby), ST_NT);
    } else if (vec) {
        const uint32_t go = opaque((uint32_t)rr * tby + (uint32_t)(cc * O::OB));
#pragma unroll
        for (int s = S0; s < S1; ++s)
            if (cc < tl.rl && s * PC::RPI + rr < tl.cl)
                *reinterpret_cast<u32x4 *>(base + ((uint32_t)(s * PC::RPI) * tby + go)) = n4;
    } else {
        for (int s = H * TB / 2; s < H * TB / 2 + TB / 2; ++s)
            if (s < tl.cl && lane < tl.rl) st_elem<O>(base + ((uint32_t)s * tby + (uint32_t)(lane * O::OB)), n4, 0);
    }
}

// Softmax statistics of the 128 query rows of super-tile `sp`, one value
// per loader lane: lanes 0..127 (loader waves 0, 1) the row maxima, lanes
// 128..255 the log-sums; rows past T read zero.
__device__ __forceinline__ float stat_fetch(const float *row_max, const float *row_logsum, const Super &sp,
                                            uint32_t T, int cl)
{
    const float *src = (cl < ST ? row_max : row_logsum) + (uint64_t)sp.plane * T; // uniform per wave
    const uint32_t r = sp.T0 + (uint32_t)(cl & (ST - 1));
    const uint32_t vo = r < T ? r * 4u : OOB;
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rsrc_at(reinterpret_cast<const char *>(src)),
                                                                (int)vo, 0, 0));
}

// Sub-tile (sa, sb) of super-tile `sp` as an output tile of the (T, T) plane.
template <class O>
__device__ __forceinline__ Tile sub_tile(const Super &sp, int sa, int sb, char *out, uint32_t T)
{
    Tile tl;
    tl.t0 = sp.T0 + sa * TB;
    tl.s0 = sp.S0 + sb * TB;
    tl.o = out + (uint64_t)sp.plane * T * T * O::OB;
    tl.rl = (int)((int64_t)T - tl.t0 < TB ? (int64_t)T - tl.t0 : TB);
    tl.cl = (int)((int64_t)T - tl.s0 < TB ? (int64_t)T - tl.s0 : TB);
    tl.diag = sp.diag;
    return tl;
}

// A store wave streams its sub-tile from LDS (rows of out_pitch<O>() bytes)
// to HBM, or the masked pattern when the sub-tile lies wholly above the
// diagonal (all_masked). Whole tiles with 16-byte aligned rows (full && vec)
// take one LDS read and one buffer store per RPI rows, the row offset a
// scalar, so no vector ALU work: the SIMD's vector issue belongs to the
// compute wave's MFMAs. Otherwise masked to the plane, 16 bytes at a time
// where rows are aligned, one element otherwise.
template <class O, class EP>
__device__ __forceinline__ void stream_subtile(const Tile &tl, bool all_masked, bool full, bool vec,
                                               const char *my_out, uint32_t T, uint32_t tby, int lane)
{
    using PC = Pieces<O>;
    constexpr int PITCH = out_pitch<O>();
    const int rr = lane / PC::LPR, cc = (lane % PC::LPR) * PC::EPC; // row in a group, first column
    const uint32_t li = (uint32_t)(rr * PITCH + cc * O::OB);
    constexpr uint32_t F = fill_dw<O, EP>();
    const u32x4 n4 = {F, F, F, F}; // the masked pattern
    char *dst = tl.o + ((uint64_t)tl.t0 * T + (uint64_t)tl.s0) * O::OB;
    const uint32_t go = opaque((uint32_t)rr * tby + (uint32_t)(cc * O::OB));
    if (full && vec) {
        const __amdgpu_buffer_rsrc_t rs = rsrc_at(dst);
        if (all_masked) {
#pragma unroll
            for (int s = 0; s < PC::NI; ++s)
                __builtin_amdgcn_raw_buffer_store_b128(n4, rs, (int)go, (int)((uint32_t)(s * PC::RPI) * tby), ST_NT);
        } else {
#pragma unroll
            for (int s = 0; s < PC::NI; ++s) {
                const u32x4 v = *reinterpret_cast<const u32x4 *>(my_out + li + s * PC::RPI * PITCH);
                __builtin_amdgcn_raw_buffer_store_b128(v, rs, (int)go, (int)((uint32_t)(s * PC::RPI) * tby), ST_NT);
            }
        }
    } else {
#pragma unroll
        for (int s = 0; s < PC::NI; ++s) {
            const u32x4 v = all_masked ? n4 : *reinterpret_cast<const u32x4 *>(my_out + li + s * PC::RPI * PITCH);
            const int row = s * PC::RPI + rr;
            if (vec) {
                if (cc < tl.cl && row < tl.rl) *reinterpret_cast<u32x4 *>(dst + ((uint32_t)(s * PC::RPI) * tby + go)) = v;
            } else {
#pragma unroll
                for (int e = 0; e < PC::EPC; ++e)
                    if (row < tl.rl && cc + e < tl.cl)
                        st_elem<O>(dst + ((uint32_t)row * tby + (uint32_t)((cc + e) * O::OB)), v, e);
            }
        }
    }
}

// HV = 2: heads of 257 .. 512 bytes in two halves of NCH * 16 = 256 bytes.
// Each super-tile then takes two steps, one per half of the head: the
// loaders stage the Q and K rows' first half, then their second half, and
// the compute waves keep accumulating into the same registers, so every
// score sums the same products in the same order as with one whole-row
// step. NU2: the chunk pairs of the second half multiplied (NCH / 4 when the
// head ends within its first 128 bytes: the rest is zero). The tile goes to
// LDS after the second step; the store waves stream it during the next
// item's first step and its mirror during the second.
template <class E, int NCH, class O, class EP = EpScore, int HV = 1, int NU2 = NCH / 2, bool PART = false>
__global__ void __launch_bounds__(SUPER_THREADS)
trimul_super_kernel(const char *__restrict__ qkv, char *__restrict__ out, uint32_t T, uint32_t C, uint32_t NH,
                    uint32_t HS, uint32_t L, uint32_t items, float scale, int vec_store,
                    const float *__restrict__ row_max, const float *__restrict__ row_logsum, int runs)
{
    static_assert(HV == 1 || HV == 2, "one or two head halves");
    constexpr int RB = NCH * 16;
    constexpr int PITCH = out_pitch<O>(), OUT_BYTES = TB * PITCH;
    constexpr bool SM = EP::KIND != 0; // softmax: per-row statistics ride along with the operand rows
    __shared__ __attribute__((aligned(16))) char opb[OP_ROWS * RB];
    __shared__ __attribute__((aligned(16))) char outb[NCOMP * OUT_BYTES];
    __shared__ float stb[SM ? 2 * ST : 1]; // [0, 128): row max, [128, 256): row logsum

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int role = wave / NCOMP; // 0 compute, 1 store, 2 loader
    const int slot = wave % NCOMP;
    const int sa = slot >> 1, sb = slot & 1; // sub-tile of this compute / store pair
    char *my_out = outb + slot * OUT_BYTES;

    // XCD-local contiguous item range; one super-tile per workgroup step.
    // runs == 0: the workgroups of an XCD take its items in turn, so at any
    // time they write neighbouring tiles. runs != 0: each takes one
    // contiguous run of the range, whose consecutive items mostly lie in one
    // row of a plane's triangle and share their Q rows, which the loaders
    // then leave in LDS (fewer reads, scattered writes; the host picks).
    const uint32_t nwg = gridDim.x;
    const uint32_t x = blockIdx.x % 8, q8 = nwg / 8, r8 = nwg % 8;
    const uint32_t wg_before = x * q8 + (x < r8 ? x : r8);
    const uint32_t wg_on_x = q8 + (x < r8 ? 1 : 0);
    const uint32_t lo = (uint32_t)((uint64_t)items * wg_before / nwg);
    const uint32_t hi = (uint32_t)((uint64_t)items * (wg_before + wg_on_x) / nwg);
    const uint32_t k = blockIdx.x / 8; // this workgroup's index on its XCD, < wg_on_x
    uint32_t first, steps, stride;
    if (runs) {
        first = lo + (uint32_t)((uint64_t)(hi - lo) * k / wg_on_x);
        steps = lo + (uint32_t)((uint64_t)(hi - lo) * (k + 1) / wg_on_x) - first;
        stride = 1;
    } else {
        first = lo + k;
        steps = first < hi ? (hi - first + wg_on_x - 1) / wg_on_x : 0;
        stride = wg_on_x;
    }

    const uint32_t TBY = T * (uint32_t)O::OB; // bytes per output row
    const uint32_t ldb = 3u * C * (uint32_t)E::ES;
    const bool vec = vec_store != 0;          // rows 16-byte aligned
    Walker cur;
    cur.init(steps > 0 ? first : 0, stride, L, (T + ST - 1) / ST);

    // Every wave passes the same barriers: one after the prologue, then X and
    // Y once per step.
    if (role == 2) {
        const int cl = slot * 64 + lane;
        Staged<NCH> st;
        float sv = 0.f;
        if (steps > 0) {
            stage_fetch<E, NCH, PART>(st, qkv, cur.item(), T, C, NH, HS, ldb, cl);
            if constexpr (SM) sv = stat_fetch(row_max, row_logsum, cur.item(), T, cl);
            stage_store<NCH>(st, opb, cl);
            if constexpr (SM) stb[cl] = sv;
        }
        lds_barrier(); // operand rows of step 0 in LDS
        for (uint32_t n = 0; n < steps; ++n) {
            if constexpr (HV == 2) { // item n's second half, then the next item's first
                stage_fetch<E, NCH, PART>(st, qkv, cur.item(), T, C, NH, HS, ldb, cl, true, RB);
                lds_barrier(); // X: first half consumed
                stage_store<NCH>(st, opb, cl);
                lds_barrier(); // Y: second half in LDS
            }
            const bool more = n + 1 < steps;
            bool with_q = true; // the next item's Q rows differ from this one's
            if (more) {
                const Super was = cur.item();
                cur.advance();
                const Super nx = cur.item();
                if constexpr (HV == 1) with_q = !(nx.plane == was.plane && nx.T0 == was.T0);
                stage_fetch<E, NCH, PART>(st, qkv, nx, T, C, NH, HS, ldb, cl, with_q);
                if constexpr (SM) sv = stat_fetch(row_max, row_logsum, nx, T, cl);
            }
            lds_barrier(); // X: operand rows of step n consumed
            if (more) {
                stage_store<NCH>(st, opb, cl, with_q);
                if constexpr (SM) stb[cl] = sv;
            }
            lds_barrier(); // Y: operand rows of step n + 1 in LDS
        }
    } else if (role == 0) {
        lds_barrier();
        for (uint32_t n = 0; n < steps; ++n) {
            const Super sp = cur.item();
            cur.advance();
            // Diagonal sub-tile (0, 1) is all NaN: its store wave writes it directly.
            const bool live = !(sp.diag && sa == 0 && sb == 1);
            float mx[2] = {0.f, 0.f}, ls[2] = {0.f, 0.f}; // statistics of rows 64sa + 32qb + lane%32
            if constexpr (SM) {
#pragma unroll
                for (int qb = 0; qb < 2; ++qb) {
                    mx[qb] = stb[64 * sa + 32 * qb + (lane & 31)];
                    ls[qb] = stb[ST + 64 * sa + 32 * qb + (lane & 31)];
                }
            }
            f32x16 acc[2][2];
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int c = 0; c < 2; ++c) acc[a][c] = f32x16{};
            if constexpr (HV == 2) { // the head's first half
                if (live) sub_mma<E, NCH>(acc, opb, sa, sb, lane);
                lds_barrier(); // X: first half consumed
                lds_barrier(); // Y: second half in LDS
            }
            if (live) sub_mma<E, NCH, HV == 2 ? NU2 : NCH / 2>(acc, opb, sa, sb, lane);
            lds_barrier(); // X: operand rows consumed, previous tile read back
            if (live) {
                if (sp.diag && sa == sb) subtile_to_lds<true, O, EP>(acc, my_out, scale, lane, mx, ls);
                else subtile_to_lds<false, O, EP>(acc, my_out, scale, lane, mx, ls);
            }
            lds_barrier(); // Y: tile n in LDS
        }
    } else {
        lds_barrier();
        Tile pm;              // mirror of the previous step, second half pending
        bool pm_live = false, pm_full = false;
        for (uint32_t n = 0; n < steps; ++n) {
            const Super sp = cur.item();
            cur.advance();
            const Tile tl = sub_tile<O>(sp, sa, sb, out, T);
            const bool inside = tl.rl > 0 && tl.cl > 0; // else the sub-tile lies past the plane edge
            const uint32_t tby = opaque_s(TBY);
            const bool full = tl.rl == TB && tl.cl == TB;
            if constexpr (HV == 2) { // the whole mirror of the previous item during this item's first step
                lds_barrier(); // X: first half consumed
                lds_barrier(); // Y: second half in LDS
                if (pm_live) {
                    if (pm_full) {
                        nan_mirror_o<0, O, true, EP>(pm, T, tby, lane, vec);
                        nan_mirror_o<1, O, true, EP>(pm, T, tby, lane, vec);
                    } else {
                        nan_mirror_o<0, O, false, EP>(pm, T, tby, lane, vec);
                        nan_mirror_o<1, O, false, EP>(pm, T, tby, lane, vec);
                    }
                }
                pm_live = false;
            }
            lds_barrier(); // X
            if (pm_live) { // second half of the previous step's mirror: needs nothing from LDS
                if (pm_full) nan_mirror_o<1, O, true, EP>(pm, T, tby, lane, vec);
                else nan_mirror_o<1, O, false, EP>(pm, T, tby, lane, vec);
            }
            pm_live = false;
            lds_barrier(); // Y: tile n in LDS
            if (!inside) continue;
            // Sub-tile (0, 1) of a diagonal super-tile lies wholly above the diagonal.
            stream_subtile<O, EP>(tl, sp.diag && sa == 0 && sb == 1, full, vec, my_out, T, tby, lane);
            if (!tl.diag) { // HV = 1: first half of the mirror now, the second after the next X
                pm = tl;
                pm_live = true;
                pm_full = full && vec;
                if constexpr (HV == 1) {
                    if (pm_full) nan_mirror_o<0, O, true, EP>(tl, T, tby, lane, vec);
                    else nan_mirror_o<0, O, false, EP>(tl, T, tby, lane, vec);
                }
            }
        }
        if (pm_live) {
            const uint32_t tby = opaque_s(TBY);
            if constexpr (HV == 2) {
                if (pm_full) nan_mirror_o<0, O, true, EP>(pm, T, tby, lane, vec);
                else nan_mirror_o<0, O, false, EP>(pm, T, tby, lane, vec);
            }
            if (pm_full) nan_mirror_o<1, O, true, EP>(pm, T, tby, lane, vec);
            else nan_mirror_o<1, O, false, EP>(pm, T, tby, lane, vec);
        }
    }
}

template <class E, int NCH, class O, class EP = EpScore, int HV = 1, int NU2 = NCH / 2, bool PART = false>
hipError_t launch_super(const TrimulArgs &a, hipStream_t s)
{
    auto kern = trimul_super_kernel<E, NCH, O, EP, HV, NU2, PART>;
    const int64_t nt = (a.T + ST - 1) / ST;
    const int64_t L = nt * (nt + 1) / 2;
    const int64_t items = a.B * a.NH * L;
    static ResidentSlots resident;
    int64_t grid = resident_slots(resident, kern, SUPER_THREADS);
    if (grid > items) grid = items;
    if (grid < 1) grid = 1;
    // Contiguous runs per workgroup for fp32 inputs with at least eight
    // super-tile rows: there the saved Q-row reloads outweigh the scattered
    // writes (fp32 B8 T1024: 85.8 -> 82.8 us; B8 T2048: 321 -> 309 us; B32
    // T512: 88.6 -> 89.9 us). The store-bound 16-bit inputs lose with them
    // (bf16 B4 T4096 to bf16: 577 -> 659 us). Two head halves (HV = 2)
    // reload the Q rows anyway.
    const int runs = HV == 1 && std::is_same<E, KF32>::value && nt >= 8;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(SUPER_THREADS), 0, s, (const char *)a.qkv, (char *)a.out,
                       (uint32_t)a.T,
                       (uint32_t)a.C, (uint32_t)a.NH, (uint32_t)a.HS, (uint32_t)L, (uint32_t)items, a.scale,
                       (int)a.vec_store, a.row_max, a.row_logsum, runs);
    return hipGetLastError();
}

// Register pass width: chunk pairs per pass (U * 32 bytes of each row); the
// two operand blocks take 16*U registers each, twice over with the prefetch.
// CAS_TRIMUL_PASS=1|2|4 overrides the choice (tuning).
inline int pick_u(int64_t HS, int es)
{
    if (const char *v = std::getenv("CAS_TRIMUL_PASS")) {
        const int u = std::atoi(v);
        if (u == 1 || u == 2 || u == 4) return u;
    }
    const int64_t row_bytes = HS * es;
    if (row_bytes > 64) return 4;
    if (row_bytes > 32) return 2;
    return 1;
}

template <class E, int U, bool VEC16, int P, class EP = EpScore>
hipError_t launch_cfg(const TrimulArgs &a, hipStream_t s)
{
    auto kern = trimul_kernel<E, U, VEC16, P, EP>;
    const int64_t nt = (a.T + TB - 1) / TB;
    const int64_t L = nt * (nt + 1) / 2;
    const int64_t items = a.B * a.NH * L;

    // Persistent grid: as many workgroups as stay resident on the device.
    static ResidentSlots resident;
    const int64_t want = (items + NCOMP - 1) / NCOMP;
    int64_t grid = resident_slots(resident, kern, NTHREADS);
    if (grid > want) grid = want;
    if (grid < 1) grid = 1;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(NTHREADS), 0, s, (const char *)a.qkv, (float *)a.out, a.T, a.C,
                       a.NH, a.HS, L, items, a.scale, (int)a.vec_store, a.out_kind, a.row_max, a.row_logsum);
    return hipGetLastError();
}

// Softmax rows (EP = EpLog or EpProb) on the tile kernel, for heads of 257 ..
// 512 bytes in 16-byte pieces: three or four 128-byte register passes.
template <class E, class EP> hipError_t launch_tile_ep(const TrimulArgs &a, hipStream_t s)
{
    const int64_t P = (a.HS * E::ES + 127) / 128;
    if (P == 3) return launch_cfg<E, 4, true, 3, EP>(a, s);
    if (P == 4) return launch_cfg<E, 4, true, 4, EP>(a, s);
    return hipErrorInvalidValue;
}

// Passes per head: P = ceil(HS*ES / (32*U)). Prefetching variants exist for
// P <= 4 at the full pass width (heads up to 512 bytes) and P == 1 at the
// narrow widths chosen for short heads; anything else takes the P == 0 path.
template <class E, int U, bool VEC16>
hipError_t launch_p(const TrimulArgs &a, hipStream_t s)
{
    const int64_t pb = 32 * U;
    const int64_t P = (a.HS * E::ES + pb - 1) / pb;
    if constexpr (U == 4) {
        switch (P) {
        case 1: return launch_cfg<E, U, VEC16, 1>(a, s);
        case 2: return launch_cfg<E, U, VEC16, 2>(a, s);
        case 3: return launch_cfg<E, U, VEC16, 3>(a, s);
        case 4: return launch_cfg<E, U, VEC16, 4>(a, s);
        default: return launch_cfg<E, U, VEC16, 0>(a, s);
        }
    } else {
        if (P == 1) return launch_cfg<E, U, VEC16, 1>(a, s);
        return launch_cfg<E, U, VEC16, 0>(a, s);
    }
}

template <class E, bool VEC16>
hipError_t launch_u(const TrimulArgs &a, hipStream_t s)
{
    switch (pick_u(a.HS, E::ES)) {
    case 4: return launch_p<E, 4, VEC16>(a, s);
    case 2: return launch_p<E, 2, VEC16>(a, s);
    default: return launch_p<E, 1, VEC16>(a, s);
    }
}

// Heads of 257 .. 512 bytes: the super-tile kernel in two 256-byte halves,
// the second multiplied over 128 bytes when the head ends there (as many
// chunks as the tile kernel's 128-byte passes take), else whole.
template <class E, class O, class EP> hipError_t launch_two_halves(const TrimulArgs &a, hipStream_t s)
{
    if (a.HS * E::ES <= 384) return launch_super<E, 16, O, EP, 2, 4>(a, s);
    return launch_super<E, 16, O, EP, 2, 8>(a, s);
}

// A head that ends inside a 16-byte piece (qkv at its element alignment,
// HS * ES not a multiple of 16): the same kernels, that piece's bytes past
// the head zeroed in the loader waves' registers (PART).
template <class E, class O> hipError_t launch_part(const TrimulArgs &a, hipStream_t s)
{
    const int64_t hb = a.HS * E::ES;
    if (hb > 384) return launch_super<E, 16, O, EpScore, 2, 8, true>(a, s);
    if (hb > 256) return launch_super<E, 16, O, EpScore, 2, 4, true>(a, s);
    if (hb > 128) return launch_super<E, 16, O, EpScore, 1, 8, true>(a, s);
    return launch_super<E, 8, O, EpScore, 1, 4, true>(a, s);
}

template <class E>
hipError_t launch_elem_impl(const TrimulArgs &a, int vec, hipStream_t s)
{
    // Super-tile kernel wherever it applies (16-byte aligned rows, heads of
    // at most 256 bytes, or up to 512 in two halves where that pays):
    // measured ahead of the per-wave tile kernel for every input type.
    // CAS_TRIMUL_KERNEL=tile forces the tile kernel (tests and tuning).
    const char *kv = std::getenv("CAS_TRIMUL_KERNEL");
    const bool force_tile = kv && std::strcmp(kv, "tile") == 0;
    const int64_t nts = (a.T + ST - 1) / ST;
    const bool ids_fit = a.B * a.NH * (nts * (nts + 1) / 2) <= INT32_MAX;
    // The super-tile kernel's buffer offsets within a 64-row tile reach 256 T
    // bytes, under the 2^31 range of its buffer resources for T < 2^22.
    // Heads of 257 .. 512 bytes take it in two halves of 256.
    const bool super_ok = ids_fit && vec * E::ES >= 16 && a.HS * E::ES <= 512 && a.T < (int64_t(1) << 22);
    if (super_ok && !force_tile) {
        if (a.HS * E::ES > 256) {
            if (a.out_kind == 1) return launch_two_halves<E, OBF16, EpScore>(a, s);
            if (a.out_kind == 2) return launch_two_halves<E, OF16, EpScore>(a, s);
            return launch_two_halves<E, OF32, EpScore>(a, s);
        }
        const bool narrow = a.HS * E::ES <= 128;
        if (a.out_kind == 1) return narrow ? launch_super<E, 8, OBF16>(a, s) : launch_super<E, 16, OBF16>(a, s);
        if (a.out_kind == 2) return narrow ? launch_super<E, 8, OF16>(a, s) : launch_super<E, 16, OF16>(a, s);
        return narrow ? launch_super<E, 8, OF32>(a, s) : launch_super<E, 16, OF32>(a, s);
    }
    const bool part_ok = ids_fit && vec * E::ES < 16 && (uintptr_t)a.qkv % E::ES == 0 && a.HS * E::ES <= 512 &&
                         a.T < (int64_t(1) << 22);
    if (part_ok && !force_tile) {
        if (a.out_kind == 1) return launch_part<E, OBF16>(a, s);
        if (a.out_kind == 2) return launch_part<E, OF16>(a, s);
        return launch_part<E, OF32>(a, s);
    }
    // 16-byte chunks need base, pitch and head offsets 16-byte aligned and
    // HS*ES a multiple of 16 (vec = elements that divide all of them).
    if (vec * E::ES >= 16) return launch_u<E, true>(a, s);
    return launch_u<E, false>(a, s);
}

} // namespace tri
} // namespace cas
