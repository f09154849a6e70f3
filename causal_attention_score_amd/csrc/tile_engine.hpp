// tile_engine.hpp -- the fetch -> LDS -> MFMA pipeline shared by the dense NT
// product and the causal score kernels (gfx950, wave64).
//
// Stage model (DietCode test_1_local_padding.py, test_local_padding
// docstring: Fetch, Compute, Writeback): every bounds predicate lives in the
// Fetch stage, which zero-fills rows past the matrix and contraction indices
// past K, and in the Writeback stage of each kernel. The Compute stage below
// runs over full tiles with no predicates ("local padding"); it never shrinks
// the LDS workspace for edge tiles (test_local_padding_ii docstring).
//
// Both operands arrive as rows that are contiguous along the contraction
// index ("NT": X rows and W rows, or Q rows and K rows), so one 16-byte LDS
// read per lane feeds an MFMA operand directly with no transposition.
//
// MFMA shapes: fp32 inputs use v_mfma_f32_32x32x2_f32 (4 per 16-byte chunk),
// bf16 / f16 inputs use v_mfma_f32_32x32x16_{bf16,f16} (1 per chunk). The
// accumulators are fp32 in every case.
//
// Contraction-order permutation: lane half h = lane/32 is the MFMA's k-slot.
// Within one BK chunk, half h feeds the contraction indices
// [h*BK/2, (h+1)*BK/2) in ascending order, so a lane reads contiguous bytes.
// A and B use the same permutation, so every product a_k*b_k is formed
// exactly once; only the fp32 summation order differs from the plain loop.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cas {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// Element kinds of the inputs (outputs are always fp32).
struct KF32 { static constexpr int ES = 4; };
struct KBF16 { static constexpr int ES = 2; };
struct KF16 { static constexpr int ES = 2; };

// One 16-byte chunk of A and of B per lane -> accumulate into a 32x32 tile.
template <class E> __device__ __forceinline__ void mfma_chunk(f32x16 &acc, u32x4 a, u32x4 b);

template <> __device__ __forceinline__ void mfma_chunk<KF32>(f32x16 &acc, u32x4 a, u32x4 b)
{
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.x), __uint_as_float(b.x), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.y), __uint_as_float(b.y), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.z), __uint_as_float(b.z), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.w), __uint_as_float(b.w), acc, 0, 0, 0);
}

template <> __device__ __forceinline__ void mfma_chunk<KBF16>(f32x16 &acc, u32x4 a, u32x4 b)
{
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
}

template <> __device__ __forceinline__ void mfma_chunk<KF16>(f32x16 &acc, u32x4 a, u32x4 b)
{
    acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                 __builtin_bit_cast(f16x8, b), acc, 0, 0, 0);
}

// The first chunk of a tile: the product alone, with a zero accumulator
// the MFMA takes as an inline constant (no register clearing).
template <class E> __device__ __forceinline__ f32x16 mfma_first(u32x4 a, u32x4 b);
template <> __device__ __forceinline__ f32x16 mfma_first<KF32>(u32x4 a, u32x4 b)
{
    f32x16 acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.x), __uint_as_float(b.x), f32x16{}, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.y), __uint_as_float(b.y), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.z), __uint_as_float(b.z), acc, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.w), __uint_as_float(b.w), acc, 0, 0, 0);
}
template <> __device__ __forceinline__ f32x16 mfma_first<KBF16>(u32x4 a, u32x4 b)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                   f32x16{}, 0, 0, 0);
}
template <> __device__ __forceinline__ f32x16 mfma_first<KF16>(u32x4 a, u32x4 b)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b),
                                                  f32x16{}, 0, 0, 0);
}

// Global-load vector types by byte width.
template <int BYTES> struct VecT;
template <> struct VecT<16> { using T = u32x4; };
template <> struct VecT<8> { using T = u32x2; };
template <> struct VecT<4> { using T = unsigned int; };
template <> struct VecT<2> { using T = unsigned short; };

// Accumulator layout of a 32x32 MFMA tile: lane l, register r holds
// row 8*(r/4) + 4*(l/32) + r%4 (an A row) and column l%32 (a B row).
__device__ __forceinline__ int acc_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

// Bounds of one output tile's operands, seen by a predicated compute stage.
struct TileBounds {
    int64_t ra0, rowsA, rb0, rowsB, K;
};

// Raw buffer loads by width. With num_records 2^31 - 1, an offset of 2^31
// lies outside the buffer and reads as zero (no access is made).
constexpr uint32_t BUF_OOB = 0x80000000u;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const char *base)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(base), (short)0, 0x7FFFFFFF, 0x00020000);
}
template <int VB> struct BufLoad;
template <> struct BufLoad<16> {
    __device__ static __forceinline__ u32x4 ld(__amdgpu_buffer_rsrc_t r, uint32_t o)
    {
        return __builtin_amdgcn_raw_buffer_load_b128(r, (int)o, 0, 0);
    }
};
template <> struct BufLoad<8> {
    __device__ static __forceinline__ u32x2 ld(__amdgpu_buffer_rsrc_t r, uint32_t o)
    {
        return __builtin_amdgcn_raw_buffer_load_b64(r, (int)o, 0, 0);
    }
};
template <> struct BufLoad<4> {
    __device__ static __forceinline__ unsigned int ld(__amdgpu_buffer_rsrc_t r, uint32_t o)
    {
        return __builtin_amdgcn_raw_buffer_load_b32(r, (int)o, 0, 0);
    }
};
template <> struct BufLoad<2> {
    __device__ static __forceinline__ unsigned short ld(__amdgpu_buffer_rsrc_t r, uint32_t o)
    {
        return __builtin_amdgcn_raw_buffer_load_b16(r, (int)o, 0, 0);
    }
};

// A workgroup barrier that orders LDS accesses only: unlike __syncthreads it
// does not wait for the wave's global loads, which may stay in flight.
__device__ __forceinline__ void lds_only_barrier()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// E: element kind. BM x BN output tile, BK contraction chunk, WGM x WGN waves,
// VEC elements per global load. PRED: the compute stage re-checks every
// operand element against the matrix bounds, zeroing those outside -- the
// predicates that local padding removes, kept for the A/B measurement.
template <class E, int BM, int BN, int BK, int WGM, int WGN, int VEC, bool PRED = false>
struct Engine {
    static constexpr int ES = E::ES;
    static constexpr int NT = WGM * WGN * 64;          // threads per workgroup
    static constexpr int WM = BM / WGM, WN = BN / WGN; // wave tile
    static constexpr int MB = WM / 32, NB = WN / 32;   // 32x32 MFMA tiles per wave
    static constexpr int ROWB = BK * ES + 16;          // LDS row pitch: +16 B skews banks
    static constexpr int A_BYTES = BM * ROWB;
    static constexpr int B_BYTES = BN * ROWB;
    static constexpr int STAGE = A_BYTES + B_BYTES;
    static constexpr int VB = VEC * ES;                // bytes per global load
    static constexpr int VPR = BK / VEC;               // loads per tile row
    static constexpr int A_IT = BM * VPR / NT;
    static constexpr int B_IT = BN * VPR / NT;
    static constexpr int HALF_B = BK * ES / 2;         // bytes of one k-slot half row
    static constexpr int CHUNKS = HALF_B / 16;
    using V = typename VecT<VB>::T;

    static_assert(WM % 32 == 0 && WN % 32 == 0, "wave tile must be whole 32x32 MFMA tiles");
    static_assert(HALF_B % 16 == 0, "half row must be whole 16-byte chunks");
    static_assert((BM * VPR) % NT == 0 && (BN * VPR) % NT == 0, "fetch must divide evenly");
    static_assert(ROWB % 16 == 0 && ((ROWB / 16) & 1) == 1, "odd 16-byte pitch keeps 8 lanes on distinct banks");

    struct Regs {
        V a[A_IT];
        V b[B_IT];
    };

    // Fetch stage: rows [ra0, ra0+BM) of A and [rb0, rb0+BN) of B, contraction
    // indices [k0, k0+BK); anything outside (rows >= rows*, k >= K) is zero.
    // Host guarantees K % VEC == 0, pitches % VEC == 0 and VB-aligned bases, so
    // a vector is either wholly inside or wholly outside.
    __device__ static __forceinline__ void fetch(Regs &R, const char *A, int64_t lda, int64_t rowsA, int64_t ra0,
                                                 const char *B, int64_t ldb, int64_t rowsB, int64_t rb0,
                                                 int64_t K, int64_t k0, int tid)
    {
#pragma unroll
        for (int it = 0; it < A_IT; ++it) {
            const int v = it * NT + tid;
            const int r = v / VPR, c = v % VPR;
            const int64_t gr = ra0 + r, gk = k0 + (int64_t)c * VEC;
            V val = {};
            if (gr < rowsA && gk < K) val = *reinterpret_cast<const V *>(A + (gr * lda + gk) * ES);
            R.a[it] = val;
        }
#pragma unroll
        for (int it = 0; it < B_IT; ++it) {
            const int v = it * NT + tid;
            const int r = v / VPR, c = v % VPR;
            const int64_t gr = rb0 + r, gk = k0 + (int64_t)c * VEC;
            V val = {};
            if (gr < rowsB && gk < K) val = *reinterpret_cast<const V *>(B + (gr * ldb + gk) * ES);
            R.b[it] = val;
        }
    }

    // The same fetch with buffer loads and no branch: an element outside the
    // matrix gets the out-of-range offset and reads zero. Loads under
    // per-lane branches make the compiler's wait at the stash cover every
    // load in flight, which a fetch several chunks ahead cannot afford. The
    // host guarantees BM * lda * ES and BN * ldb * ES below 2^31, so every
    // in-range offset from the tile's first row fits.
    __device__ static __forceinline__ void fetch_buf(Regs &R, const char *A, int64_t lda, int64_t rowsA, int64_t ra0,
                                                     const char *B, int64_t ldb, int64_t rowsB, int64_t rb0,
                                                     int64_t K, int64_t k0, int tid)
    {
        const __amdgpu_buffer_rsrc_t ra = buf_rsrc(A + (ra0 * lda + k0) * ES);
        const __amdgpu_buffer_rsrc_t rb = buf_rsrc(B + (rb0 * ldb + k0) * ES);
#pragma unroll
        for (int it = 0; it < A_IT; ++it) {
            const int v = it * NT + tid;
            const int r = v / VPR, c = v % VPR;
            const bool ok = ra0 + r < rowsA && k0 + (int64_t)c * VEC < K;
            const uint32_t o = ok ? (uint32_t)(r * lda * ES) + (uint32_t)(c * VB) : BUF_OOB;
            R.a[it] = BufLoad<VB>::ld(ra, o);
        }
#pragma unroll
        for (int it = 0; it < B_IT; ++it) {
            const int v = it * NT + tid;
            const int r = v / VPR, c = v % VPR;
            const bool ok = rb0 + r < rowsB && k0 + (int64_t)c * VEC < K;
            const uint32_t o = ok ? (uint32_t)(r * ldb * ES) + (uint32_t)(c * VB) : BUF_OOB;
            R.b[it] = BufLoad<VB>::ld(rb, o);
        }
    }

    __device__ static __forceinline__ void stash(const Regs &R, char *lds, int tid)
    {
#pragma unroll
        for (int it = 0; it < A_IT; ++it) {
            const int v = it * NT + tid;
            *reinterpret_cast<V *>(lds + (v / VPR) * ROWB + (v % VPR) * VB) = R.a[it];
        }
#pragma unroll
        for (int it = 0; it < B_IT; ++it) {
            const int v = it * NT + tid;
            *reinterpret_cast<V *>(lds + A_BYTES + (v / VPR) * ROWB + (v % VPR) * VB) = R.b[it];
        }
    }

    // Zero the elements of one 16-byte operand chunk (contraction indices
    // kidx .. kidx + 16/ES - 1 of row `row`) that lie outside the matrix.
    __device__ static __forceinline__ u32x4 mask_chunk(u32x4 v, bool row_ok, int64_t kidx, int64_t K)
    {
        constexpr int EPD = 4 / ES; // elements per dword
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            unsigned m = 0;
#pragma unroll
            for (int e = 0; e < EPD; ++e)
                if (row_ok && kidx + d * EPD + e < K) m |= (ES == 4 ? 0xFFFFFFFFu : 0xFFFFu << (16 * e));
            v[d] &= m;
        }
        return v;
    }

    // Operand fragments of one k-step u of a chunk: 16 bytes of each of the
    // wave's MFMA rows, lane half h taking the k-slot half h of the chunk.
    struct Frags {
        u32x4 a[MB];
        u32x4 b[NB];
    };

    // Read step u's fragments from the LDS stage `stage`. PRED = true: every
    // operand chunk read is masked against the bounds first (tb, contraction
    // offset k0 of this chunk).
    __device__ static __forceinline__ void read_frags(Frags &f, const char *stage, int wave_m, int wave_n, int lane,
                                                      int u, const TileBounds &tb, int64_t k0)
    {
        const int r32 = lane & 31, h = lane >> 5;
        const char *a0 = stage + (wave_m * WM + r32) * ROWB + h * HALF_B + u * 16;
        const char *b0 = stage + A_BYTES + (wave_n * WN + r32) * ROWB + h * HALF_B + u * 16;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) f.a[mb] = *reinterpret_cast<const u32x4 *>(a0 + mb * 32 * ROWB);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) f.b[nb] = *reinterpret_cast<const u32x4 *>(b0 + nb * 32 * ROWB);
        if constexpr (PRED) {
            const int64_t kidx = k0 + h * (BK / 2) + u * (16 / ES);
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
                f.a[mb] = mask_chunk(f.a[mb], tb.ra0 + wave_m * WM + mb * 32 + r32 < tb.rowsA, kidx, tb.K);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
                f.b[nb] = mask_chunk(f.b[nb], tb.rb0 + wave_n * WN + nb * 32 + r32 < tb.rowsB, kidx, tb.K);
        }
    }

    __device__ static __forceinline__ void mma(f32x16 (&acc)[MB][NB], const Frags &f)
    {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) mfma_chunk<E>(acc[mb][nb], f.a[mb], f.b[nb]);
    }

    // Compute stage: every wave multiplies its WM x WN slice of one chunk.
    __device__ static __forceinline__ void compute(f32x16 (&acc)[MB][NB], const char *lds, int wave_m, int wave_n,
                                                   int lane, const TileBounds &tb = {}, int64_t k0 = 0)
    {
#pragma unroll
        for (int u = 0; u < CHUNKS; ++u) {
            Frags f;
            read_frags(f, lds, wave_m, wave_n, lane, u, tb, k0);
            mma(acc, f);
        }
    }

    // Full contraction over K with a ring of D register sets: chunk kc + D is
    // fetched while chunk kc is multiplied, so a fetch has D - 1 chunks of
    // MFMA work to land before it is stashed (first touches of a panel come
    // from beyond the L2 and take longer than one chunk). Two LDS stages; the
    // barriers order LDS only, so the ring's loads stay in flight across them.
    template <int D>
    __device__ static __forceinline__ void mainloop_ring(f32x16 (&acc)[MB][NB], char *lds,
                                                         const char *A, int64_t lda, int64_t rowsA, int64_t ra0,
                                                         const char *B, int64_t ldb, int64_t rowsB, int64_t rb0,
                                                         int64_t K, int tid)
    {
        const int lane = tid & 63, wave = tid >> 6;
        const int wave_m = wave / WGN, wave_n = wave % WGN;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = f32x16{};

        const int64_t nk = (K + BK - 1) / BK;
        if (nk == 0) return;
        const TileBounds tb{ra0, rowsA, rb0, rowsB, K};
        // Every fetch is issued, also for chunks past the end (their offsets
        // are out of range: zeros, no memory traffic), and the loop has one
        // exit, at a whole group of D chunks. So each stash finds the same
        // loads in flight on every path, and the compiler's wait there covers
        // only the chunk it stores, not the chunks fetched after it. (With
        // the fetches under branches it waited for every load in flight, once
        // per chunk: 0.77 against 0.62 us per fp32 k-chunk at 960 x 1024.)
        Regs R[D]; // chunk c lives in R[c % D] from its fetch to its stash
#pragma unroll
        for (int d = 0; d < D; ++d) fetch_buf(R[d], A, lda, rowsA, ra0, B, ldb, rowsB, rb0, K, (int64_t)d * BK, tid);
        stash(R[0], lds, tid);
        lds_only_barrier();
        int64_t kc = 0;
        for (; kc + D < nk; kc += D) {
#pragma unroll
            for (int d = 0; d < D; ++d) {
                const int64_t c = kc + d;
                // R[d] held chunk c, stored during chunk c - 1: refill it
                fetch_buf(R[d], A, lda, rowsA, ra0, B, ldb, rowsB, rb0, K, (c + D) * BK, tid);
                compute(acc, lds + (c & 1) * STAGE, wave_m, wave_n, lane, tb, c * BK);
                stash(R[(d + 1) % D], lds + ((c + 1) & 1) * STAGE, tid);
                lds_only_barrier(); // stage of chunk c + 1 written, stage of chunk c read by every wave
            }
        }
        // The last 1 .. D chunks, already in flight in R[0 .. D - 1]; no loads.
        const int64_t rem = nk - kc;
#pragma unroll
        for (int d = 0; d < D; ++d) {
            const int64_t c = kc + d;
            if (d < rem) {
                compute(acc, lds + (c & 1) * STAGE, wave_m, wave_n, lane, tb, c * BK);
                if (d + 1 < rem) {
                    stash(R[(d + 1) % D], lds + ((c + 1) & 1) * STAGE, tid);
                    lds_only_barrier();
                }
            }
        }
    }

    // Full contraction over K for one output tile, STAGES = 1 or 2 LDS buffers.
    template <int STAGES>
    __device__ static __forceinline__ void mainloop(f32x16 (&acc)[MB][NB], char *lds,
                                                    const char *A, int64_t lda, int64_t rowsA, int64_t ra0,
                                                    const char *B, int64_t ldb, int64_t rowsB, int64_t rb0,
                                                    int64_t K, int tid)
    {
        const int lane = tid & 63, wave = tid >> 6;
        const int wave_m = wave / WGN, wave_n = wave % WGN;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = f32x16{};

        const int64_t nk = (K + BK - 1) / BK;
        Regs R;
        if constexpr (STAGES == 2) {
            if (nk > 0) {
                fetch(R, A, lda, rowsA, ra0, B, ldb, rowsB, rb0, K, 0, tid);
                stash(R, lds, tid);
            }
            __syncthreads();
            for (int64_t kc = 0; kc < nk; ++kc) {
                const char *cur = lds + (kc & 1) * STAGE;
                if (kc + 1 < nk) fetch(R, A, lda, rowsA, ra0, B, ldb, rowsB, rb0, K, (kc + 1) * BK, tid);
                compute(acc, cur, wave_m, wave_n, lane, TileBounds{ra0, rowsA, rb0, rowsB, K}, kc * BK);
                if (kc + 1 < nk) stash(R, lds + ((kc + 1) & 1) * STAGE, tid);
                __syncthreads();
            }
        } else {
            for (int64_t kc = 0; kc < nk; ++kc) {
                fetch(R, A, lda, rowsA, ra0, B, ldb, rowsB, rb0, K, kc * BK, tid);
                if (kc > 0) __syncthreads(); // every wave is done reading the previous chunk
                stash(R, lds, tid);
                __syncthreads();
                compute(acc, lds, wave_m, wave_n, lane, TileBounds{ra0, rowsA, rb0, rowsB, K}, kc * BK);
            }
        }
    }
};

// Map the hardware workgroup id so that the ids dispatched to one XCD
// (round-robin: id % 8) become one contiguous range of logical ids; the
// logical order then keeps tiles that share operand panels on one L2.
__device__ __forceinline__ int64_t xcd_remap(int64_t w, int64_t n)
{
    const int64_t q = n / 8, rem = n % 8, x = w % 8;
    return x * q + (x < rem ? x : rem) + w / 8;
}

} // namespace cas
