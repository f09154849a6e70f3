// gemm_nt_wide.hip -- dense Y = X W^T for 16-bit inputs on large shapes:
// 256 x 256 output tiles, operands streamed global -> LDS by the load unit
// itself (gfx950 buffer loads with the LDS destination), fp32 accumulation.
//
// Workload: the dense layer of DietCode's test_1_local_padding.py
// (test_local_padding docstring), Y[i,j] += X[i,k] * W[j,k], on shapes large
// enough that every CU owns at least one 256 x 256 tile (M = N = K = 4096
// gives exactly one per CU).
//
// Stage model (same docstring: Fetch, Compute, Writeback), with local padding:
//  * Fetch: each 16-byte piece of a row is requested with a buffer offset;
//    rows past M (or N) and pieces past K get an offset beyond the buffer
//    range, which the load unit turns into zeros. No other predicate exists.
//  * Compute: the MFMA loop runs over whole tiles with no predicates.
//  * Writeback: the only other place that looks at M and N.
//
// Data path. By default a workgroup holds eight waves, two per SIMD, in a
// 2 x 4 grid; each wave accumulates a 128 x 64 block as 4 x 2 MFMA tiles of
// 32 x 32 (v_mfma_f32_32x32x16_{bf16,f16}, 128 fp32 accumulators per lane; a
// four-wave layout with 128 x 128 blocks exists for tuning). Each k-chunk
// (BKB bytes of a row: 32 or 64 elements) of the 256 X rows and 256 W rows
// lands in LDS straight from the
// load unit: one load instruction fills 1 KB of LDS, lane i writing bytes
// [16i, 16i + 16). A row's 16-byte pieces are stored XOR-swizzled, the loads
// picking their source addresses to match, so the MFMA operand reads are free
// of bank conflicts. S LDS stages form a ring: the loads of chunk k + S are
// issued as soon as every wave is done with chunk k, so they have S - 1
// chunks of MFMAs to arrive.
//
// Contraction-order permutation: in a chunk, lane half h (the MFMA k-slot)
// takes the 16-byte pieces of its half of the chunk, for X and W alike, so
// every product x_k * w_k is formed exactly once.
#include "launch.hpp"
#include "tile_engine.hpp"

#include <cstdlib>
#include <cstring>
#include <string>
#include <type_traits>

namespace cas {

namespace {

constexpr int WB = 256;        // output tile edge
constexpr int WGROUP_M = 4;
constexpr uint32_t WOOB = 0x80000000u; // buffer offset the load unit reads as zero

typedef __attribute__((address_space(3))) void lds_void;
typedef float f32x4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t wide_rsrc(const char *base)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(base), (short)0, 0x7FFFFFFF, 0x00020000);
}

// s_waitcnt immediate for "at most N vector memory operations in flight and
// no LDS operation" (vmcnt is split over bits 3:0 and 15:14).
template <int N> constexpr int wait_vm_lgkm0 = (N & 15) | (7 << 4) | (0 << 8) | ((N >> 4) << 14);

// Barrier that orders this wave's LDS accesses (already waited for) against
// the other waves' without waiting for its loads still in flight.
__device__ __forceinline__ void plain_barrier() { asm volatile("s_barrier" ::: "memory"); }

// BKB: bytes of a row per k-chunk (64 or 128); S: LDS stages; NW: waves.
template <int BKB, int S, int NW> struct Wide {
    static constexpr int SPR = BKB / 16;              // 16-byte pieces per row
    static constexpr int OPB = WB * BKB;              // one operand tile per stage
    static constexpr int STAGE = 2 * OPB;
    static constexpr int ROWS_PER_LOAD = 1024 / BKB;  // rows one load instruction fills
    static constexpr int LOADS = OPB / 1024 / NW;     // per wave and operand
    static constexpr int PC = 2 * LOADS;              // per wave and chunk
    static constexpr int NU = BKB / 32;               // k16 steps per chunk
    static constexpr int SH = BKB == 128 ? 1 : 2;     // log2(256 / BKB)
    static_assert(S * STAGE <= 160 * 1024, "LDS");

    // Piece c of tile row r sits at slot c ^ f(r). The LDS serves 16-byte
    // reads 16 lanes (256 bytes) at a time, so rows whose addresses share a
    // 256-byte bank offset are 256 / BKB apart, and f steps once per such
    // stride: 16 consecutive rows read at one piece hit 16 distinct 16-byte
    // bank groups (the bank-conflict counter reads zero; with f stepping
    // every row it does not). Rows 32i + r32 share f(r32).
    __device__ static __forceinline__ int f(int r) { return (r >> SH) & (SPR - 1); }

    // Load j (< LOADS) of one operand tile at `rs`, k-chunk at byte k0b: it
    // fills the 1 KB of LDS of tile rows ROWS_PER_LOAD * (LOADS * wave + j)
    // .. + ROWS_PER_LOAD.
    __device__ static __forceinline__ void fetch(__amdgpu_buffer_rsrc_t rs, char *tile, uint32_t ldb, int rows,
                                                 uint32_t k0b, uint32_t kb, int wave, int lane, int j)
    {
        const int rsub = lane / SPR, slot = lane % SPR;
        const int blk = wave * LOADS + j;
        const int r = blk * ROWS_PER_LOAD + rsub;
        const uint32_t cb = k0b + (uint32_t)((slot ^ f(r)) * 16);
        const uint32_t vo = (r < rows && cb < kb) ? (uint32_t)r * ldb + cb : WOOB;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)(tile + blk * 1024), 16, (int)vo, 0, 0, 0);
    }
};

// Writeback of one wave's 128 x WN block: lane l, registers 4g .. 4g+3 of
// block (a, b) hold row 32a + l % 32 and columns 32b + 8g + 4(l / 32) + 0..3
// (row0 / col0: this lane's first row and column; r0 / c0: the block's): one
// 16-byte store each where the rows are 16-byte aligned and the block lies
// inside the matrix, else element by element, masked on the true M and N.
template <int NB, int WN>
__device__ __forceinline__ void write_tile(const f32x16 (&acc)[4][NB], float *Y, int64_t M, int64_t N, int64_t ldy,
                                           int64_t row0, int64_t col0, int64_t r0, int64_t c0)
{
    float *yw = Y + row0 * ldy + col0;
    const bool vec_ok = ((uintptr_t)Y % 16 == 0) && (ldy % 4 == 0);
    if (vec_ok && r0 + 128 <= M && c0 + WN <= N) {
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const f32x4v v = {acc[a][b][4 * g], acc[a][b][4 * g + 1], acc[a][b][4 * g + 2], acc[a][b][4 * g + 3]};
                    *reinterpret_cast<f32x4v *>(yw + 32 * a * ldy + 32 * b + 8 * g) = v;
                }
    } else {
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            const bool row_ok = row0 + 32 * a < M;
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int cc = 32 * b + 8 * (r >> 2) + (r & 3);
                    if (row_ok && col0 + cc < N) yw[32 * a * ldy + cc] = acc[a][b][r];
                }
        }
    }
}

// NWN: waves along N (2: four waves with 128 x 128 blocks; 4: eight waves,
// two per SIMD, with 128 x 64 blocks).
template <class E, int BKB, int S, int NWN>
__global__ void __launch_bounds__(2 * NWN * 64)
gemm_nt_wide_kernel(const char *__restrict__ X, const char *__restrict__ W, float *__restrict__ Y,
                    int64_t M, int64_t N, int64_t K, int64_t ldx, int64_t ldw, int64_t ldy,
                    int64_t tiles_m, int64_t tiles_n)
{
    constexpr int NW = 2 * NWN, WN = 256 / NWN, NB = WN / 32; // waves; wave block 128 x WN
    using G = Wide<BKB, S, NW>;
    constexpr int ES = E::ES;
    __shared__ __attribute__((aligned(1024))) char lds[S * G::STAGE];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave / NWN, wn = wave % NWN;

    // XCD-aware raster: the workgroups of one XCD take a contiguous range of
    // logical ids, walked in groups of WGROUP_M tile rows, so the X and W
    // panels of one k-chunk are shared through that XCD's L2.
    // (32-bit scalar arithmetic: the host keeps the tile count under 2^31.)
    const uint32_t ntm = (uint32_t)tiles_m, ntn = (uint32_t)tiles_n, nwg = ntm * ntn;
    const uint32_t x = blockIdx.x % 8, q8 = nwg / 8, r8 = nwg % 8;
    const uint32_t pid = x * q8 + (x < r8 ? x : r8) + blockIdx.x / 8;
    const uint32_t group = WGROUP_M * ntn;
    const uint32_t first_m = (pid / group) * WGROUP_M;
    const uint32_t gm = (ntm - first_m) < WGROUP_M ? (ntm - first_m) : WGROUP_M;
    const uint32_t tm = __builtin_amdgcn_readfirstlane(first_m + (pid % group) % gm);
    const uint32_t tn = __builtin_amdgcn_readfirstlane((pid % group) / gm);

    const int64_t m0 = (int64_t)tm * WB, n0 = (int64_t)tn * WB;
    const int rows_x = (int)(M - m0 < WB ? M - m0 : WB);
    const int rows_w = (int)(N - n0 < WB ? N - n0 : WB);
    const __amdgpu_buffer_rsrc_t rx = wide_rsrc(X + m0 * ldx * ES);
    const __amdgpu_buffer_rsrc_t rw = wide_rsrc(W + n0 * ldw * ES);
    const uint32_t ldxb = (uint32_t)(ldx * ES), ldwb = (uint32_t)(ldw * ES), kb = (uint32_t)(K * ES);
    const int nk = (int)((K * ES + BKB - 1) / BKB);

    f32x16 acc[4][NB];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[a][b] = f32x16{};

    // Load q (< PC) of this wave for chunk c: the X tile's, then the W tile's.
    // A chunk past the end reads as zeros (every piece out of range).
    auto fetch_one = [&](int c, int q) {
        char *stg = lds + (c % S) * G::STAGE;
        const uint32_t kbv = c < nk ? kb : 0u;
        if (q < G::LOADS) G::fetch(rx, stg, ldxb, rows_x, (uint32_t)c * BKB, kbv, wave, lane, q);
        else G::fetch(rw, stg + G::OPB, ldwb, rows_w, (uint32_t)c * BKB, kbv, wave, lane, q - G::LOADS);
    };
    const int r32 = lane & 31, h = lane >> 5, fr = G::f(r32);
    // Fragments of k16 step u: piece h * NU + u (lane half h is the MFMA
    // k-slot) of rows 32i + r32.
    auto read_frags = [&](const char *stage, int u, u32x4 (&af)[4], u32x4 (&bfr)[NB]) {
        const int pos = ((h * G::NU + u) ^ fr) * 16;
        const char *xa = stage + (wm * 128 + r32) * BKB + pos;
        const char *wa = stage + G::OPB + (wn * WN + r32) * BKB + pos;
#pragma unroll
        for (int i = 0; i < 4; ++i) af[i] = *reinterpret_cast<const u32x4 *>(xa + i * 32 * BKB);
#pragma unroll
        for (int i = 0; i < NB; ++i) bfr[i] = *reinterpret_cast<const u32x4 *>(wa + i * 32 * BKB);
    };

    // Pipeline: chunk c lives in stage c % S. One barrier per chunk, before
    // its last k16 step's MFMAs: by then every wave holds that step's
    // fragments in registers, so from the barrier inside chunk c on, the
    // stage of chunk c is free for chunk c + S, and the next chunk's first
    // fragments are read behind the MFMAs. Each step's reads of the next
    // step's fragments go one after each MFMA, in the order that step takes
    // them (bf16 4096^3: 115.7 against 117.7 us with all six reads issued
    // ahead of the MFMAs).
    // Chunk c's loads: one step's worth (LPS) right after the barrier inside
    // chunk c - S, the rest during steps 0 .. NU - 2 of chunk c - S + 1, one
    // load after every P MFMAs. Chunks past the end are loaded too (as zeros,
    // into stages nothing reads any more), so every step issues the same
    // loads at the same places -- no branch among the MFMAs, where a taken
    // branch stalls the matrix pipe -- and every barrier waits for the same
    // count: this wave's loads of chunk kc + 1 are done once at most those of
    // chunks kc + 2 .. kc + S - 1, (S - 2) PC loads, are in flight.
    constexpr int MPS = 4 * NB;        // MFMAs per step
    constexpr int LPS = G::PC / G::NU; // loads per step
    constexpr int P = MPS / LPS;
    static_assert(LPS * G::NU == G::PC && LPS <= MPS && MPS % LPS == 0, "load spread");
    static_assert((S - 2) * G::PC + LPS <= 63, "vmcnt range");
    u32x4 fa[2][4], fb[2][NB];
    // One k16 step: MPS MFMAs; with c >= 0 (compile-time shape: c is only
    // ever a chunk number or -1 for none), loads [q0, q0 + LPS) of chunk c.
    auto mma_step = [&](int fi, int c, int q0, auto with_loads) {
#pragma unroll
        for (int i = 0; i < MPS; ++i) {
            __builtin_amdgcn_sched_barrier(0);
            // D = W X^T: W rows are the MFMA A operand, so a lane's four
            // consecutive accumulators are four consecutive output columns.
            mfma_chunk<E>(acc[i / NB][i % NB], fb[fi][i % NB], fa[fi][i / NB]);
            if constexpr (decltype(with_loads)::value) {
                if ((i + 1) % P == 0) {
                    __builtin_amdgcn_sched_barrier(0);
                    fetch_one(c, q0 + (i + 1) / P - 1);
                }
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    // The same step with the fragment reads of the next step (stage `nst`,
    // k16 step `nu`) issued one after each of the first 4 + NB MFMAs instead
    // of all before them.
    auto mma_step_rd = [&](int fi, int c, int q0, auto with_loads, const char *nst, int nu) {
        const int pos = ((h * G::NU + nu) ^ fr) * 16;
        const char *xa = nst + (wm * 128 + r32) * BKB + pos;
        const char *wa = nst + G::OPB + (wn * WN + r32) * BKB + pos;
#pragma unroll
        for (int i = 0; i < MPS; ++i) {
            __builtin_amdgcn_sched_barrier(0);
            mfma_chunk<E>(acc[i / NB][i % NB], fb[fi][i % NB], fa[fi][i / NB]);
            // In the order the next step takes them (its MFMA j reads A
            // fragment j / NB and B fragment j % NB): a0, b0 .. b(NB-1), a1 .. a3.
            if (i == 0) fa[fi ^ 1][0] = *reinterpret_cast<const u32x4 *>(xa);
            else if (i <= NB) fb[fi ^ 1][i - 1] = *reinterpret_cast<const u32x4 *>(wa + (i - 1) * 32 * BKB);
            else if (i < 4 + NB) fa[fi ^ 1][i - NB] = *reinterpret_cast<const u32x4 *>(xa + (i - NB) * 32 * BKB);
            if constexpr (decltype(with_loads)::value) {
                if ((i + 1) % P == 0) {
                    __builtin_amdgcn_sched_barrier(0);
                    fetch_one(c, q0 + (i + 1) / P - 1);
                }
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    using loads = std::true_type;
    using no_loads = std::false_type;
    // The writeback's arguments, read from the kernel arguments now: a
    // scalar load still in flight in the main loop would make every wait for
    // the fragment reads a wait for all of them (scalar loads return out of
    // order, in the same counter).
    asm volatile("" ::"s"(Y), "s"(ldy));
    if (nk > 0) {
        for (int c = 0; c + 1 < S; ++c)
            for (int q = 0; q < G::PC; ++q) fetch_one(c, q);
        for (int q = 0; q < LPS; ++q) fetch_one(S - 1, q);
        __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0<(S - 2) * G::PC + LPS>); // chunk 0 landed
        plain_barrier();
        read_frags(lds, 0, fa[0], fb[0]);
    }
    for (int kc = 0; kc + 1 < nk; ++kc) {
        const char *cur = lds + (kc % S) * G::STAGE;
#pragma unroll
        for (int u = 0; u < G::NU; ++u) {
            const int fi = u & 1;
            if (u + 1 < G::NU) {
                mma_step_rd(fi, kc - 1 + S, (u + 1) * LPS, loads{}, cur, u + 1);
            } else {
                __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0<(S - 2) * G::PC>); // chunk kc + 1 landed
                plain_barrier(); // ... for every wave; every wave done reading chunk kc
                mma_step_rd(fi, kc + S, 0, loads{}, lds + ((kc + 1) % S) * G::STAGE, 0);
            }
        }
    }
    // The last chunk: no barrier, no loads (out of the loop, which keeps the
    // LDS waits of the loop body exact).
    if (nk > 0) {
        const char *cur = lds + ((nk - 1) % S) * G::STAGE;
#pragma unroll
        for (int u = 0; u < G::NU; ++u) {
            const int fi = u & 1;
            if (u + 1 < G::NU) read_frags(cur, u + 1, fa[fi ^ 1], fb[fi ^ 1]);
            mma_step(fi, -1, 0, no_loads{});
        }
    }
    // Loads of chunks past the end may still be writing LDS.
    __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0<0>);

    write_tile<NB, WN>(acc, Y, M, N, ldy, m0 + wm * 128 + r32, n0 + wn * WN + 4 * h, m0 + wm * 128, n0 + wn * WN);
}

// The same product for shapes whose K is a whole number of ring turns
// (K * ES a multiple of S * BKB bytes): the contraction needs no zero-fill, so
// the fetch side has no per-chunk predicate at all. Each lane's load offsets
// are computed once (rows past M or N get the out-of-range offset, as above)
// and a chunk is selected by the load's scalar offset c * BKB; the loop is
// unrolled over the S stages, so every LDS address is an immediate offset
// from a base computed once, and the last S chunks are peeled so that no load
// is issued past the end. The main loop then holds MFMAs, LDS reads, loads and
// one barrier per chunk, with no vector-ALU instruction. The MFMA sequence
// and the contraction order are the ring kernel's, so the results are the
// same bit for bit.
template <int V> using IC = std::integral_constant<int, V>;

template <class E, int BKB, int S, int NWN>
__global__ void __launch_bounds__(2 * NWN * 64)
gemm_nt_wide_full_kernel(const char *__restrict__ X, const char *__restrict__ W, float *__restrict__ Y,
                         int64_t M, int64_t N, int64_t K, int64_t ldx, int64_t ldw, int64_t ldy,
                         int64_t tiles_m, int64_t tiles_n)
{
    constexpr int NW = 2 * NWN, WN = 256 / NWN, NB = WN / 32;
    using G = Wide<BKB, S, NW>;
    constexpr int ES = E::ES;
    constexpr int MPS = 4 * NB, LPS = G::PC / G::NU, P = MPS / LPS;
    static_assert(S == 4, "the loop body is unrolled for four stages");
    static_assert(G::NU % 2 == 0 && LPS * G::NU == G::PC && MPS % LPS == 0, "load spread");
    static_assert((S - 2) * G::PC + LPS <= 63, "vmcnt range");
    __shared__ __attribute__((aligned(1024))) char lds[S * G::STAGE];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave / NWN, wn = wave % NWN;

    // XCD-aware raster, as in gemm_nt_wide_kernel.
    const uint32_t ntm = (uint32_t)tiles_m, ntn = (uint32_t)tiles_n, nwg = ntm * ntn;
    const uint32_t x = blockIdx.x % 8, q8 = nwg / 8, r8 = nwg % 8;
    const uint32_t pid = x * q8 + (x < r8 ? x : r8) + blockIdx.x / 8;
    const uint32_t group = WGROUP_M * ntn;
    const uint32_t first_m = (pid / group) * WGROUP_M;
    const uint32_t gm = (ntm - first_m) < WGROUP_M ? (ntm - first_m) : WGROUP_M;
    const uint32_t tm = __builtin_amdgcn_readfirstlane(first_m + (pid % group) % gm);
    const uint32_t tn = __builtin_amdgcn_readfirstlane((pid % group) / gm);

    const int64_t m0 = (int64_t)tm * WB, n0 = (int64_t)tn * WB;
    const int rows_x = (int)(M - m0 < WB ? M - m0 : WB);
    const int rows_w = (int)(N - n0 < WB ? N - n0 : WB);
    const __amdgpu_buffer_rsrc_t rx = wide_rsrc(X + m0 * ldx * ES);
    const __amdgpu_buffer_rsrc_t rw = wide_rsrc(W + n0 * ldw * ES);
    const uint32_t ldxb = (uint32_t)(ldx * ES), ldwb = (uint32_t)(ldw * ES);
    const int nk = (int)(K * ES / BKB); // a multiple of S, at least S (host)

    // Load q of this wave (X tile's loads first, then W's): its lane offset
    // within chunk 0; chunk c adds c * BKB through the scalar offset.
    uint32_t vo[G::PC];
    {
        const int rsub = lane / G::SPR, slot = lane % G::SPR;
#pragma unroll
        for (int q = 0; q < G::PC; ++q) {
            const int op = q / G::LOADS;
            const int r = (wave * G::LOADS + q % G::LOADS) * G::ROWS_PER_LOAD + rsub;
            vo[q] = r < (op ? rows_w : rows_x) ? (uint32_t)r * (op ? ldwb : ldxb) + (uint32_t)((slot ^ G::f(r)) * 16)
                                               : WOOB;
        }
    }
    auto load = [&](int c, int st, int q) {
        const int op = q / G::LOADS;
        char *dst = lds + st * G::STAGE + op * G::OPB + (wave * G::LOADS + q % G::LOADS) * 1024;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(op ? rw : rx, (lds_void *)dst, 16, (int)vo[q], c * BKB, 0, 0);
    };

    // Fragment bases of k16 step u (piece h * NU + u of rows 32i + r32).
    const int r32 = lane & 31, h = lane >> 5, fr = G::f(r32);
    const char *xb[G::NU], *wb[G::NU];
#pragma unroll
    for (int u = 0; u < G::NU; ++u) {
        const int pos = ((h * G::NU + u) ^ fr) * 16;
        xb[u] = lds + (wm * 128 + r32) * BKB + pos;
        wb[u] = lds + G::OPB + (wn * WN + r32) * BKB + pos;
    }

    f32x16 acc[4][NB];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[a][b] = f32x16{};
    u32x4 fa[2][4], fb[2][NB];

    // One k16 step: MPS MFMAs on fragment set fi; with rd, the fragments of
    // step nu of stage nst read into set fi ^ 1 one after each of the first
    // 4 + NB MFMAs (in the order that step takes them); nl loads (q0 on) of
    // chunk lc into stage lst, one after every P MFMAs.
    auto step = [&](int fi, int nst, int nu, bool rd, int lc, int lst, int q0, int nl) {
        const char *xa = xb[nu] + nst * G::STAGE;
        const char *wa = wb[nu] + nst * G::STAGE;
#pragma unroll
        for (int i = 0; i < MPS; ++i) {
            __builtin_amdgcn_sched_barrier(0);
            mfma_chunk<E>(acc[i / NB][i % NB], fb[fi][i % NB], fa[fi][i / NB]);
            if (rd) {
                if (i == 0) fa[fi ^ 1][0] = *reinterpret_cast<const u32x4 *>(xa);
                else if (i <= NB) fb[fi ^ 1][i - 1] = *reinterpret_cast<const u32x4 *>(wa + (i - 1) * 32 * BKB);
                else if (i < 4 + NB) fa[fi ^ 1][i - NB] = *reinterpret_cast<const u32x4 *>(xa + (i - NB) * 32 * BKB);
            }
            if (nl > 0 && (i + 1) % P == 0 && (i + 1) / P <= nl) {
                __builtin_amdgcn_sched_barrier(0);
                load(lc, lst, q0 + (i + 1) / P - 1);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    };

    asm volatile("" ::"s"(Y), "s"(ldy)); // writeback arguments read before the loop (see above)
    // Prologue: chunks 0 .. S-2 whole and the first LPS loads of chunk S-1.
    for (int c = 0; c + 1 < S; ++c)
        for (int q = 0; q < G::PC; ++q) load(c, c, q);
    for (int q = 0; q < LPS; ++q) load(S - 1, S - 1, q);
    __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0<(S - 2) * G::PC + LPS>); // chunk 0 landed
    plain_barrier();
    {
#pragma unroll
        for (int i = 0; i < 4; ++i) fa[0][i] = *reinterpret_cast<const u32x4 *>(xb[0] + i * 32 * BKB);
#pragma unroll
        for (int i = 0; i < NB; ++i) fb[0][i] = *reinterpret_cast<const u32x4 *>(wb[0] + i * 32 * BKB);
    }
    // Chunk j in stage ST. During its steps 0 .. NU-2 the rest of chunk
    // j + S - 1 is loaded (REST); its barrier waits until chunk j + 1 has
    // landed, VM loads of later chunks may stay in flight; right after it the
    // first LPS loads of chunk j + S go into stage ST, which no wave reads any
    // more (NEXT). The last chunk has no barrier.
    auto chunk = [&](int j, auto st_c, auto rest_c, auto next_c, auto vm_c, auto last_c) {
        constexpr int ST = decltype(st_c)::value, VM = decltype(vm_c)::value;
        constexpr bool REST = decltype(rest_c)::value, NEXT = decltype(next_c)::value;
        constexpr bool LAST = decltype(last_c)::value;
#pragma unroll
        for (int u = 0; u < G::NU; ++u) {
            const int fi = u & 1;
            if (u + 1 < G::NU) {
                step(fi, ST, u + 1, true, j + S - 1, (ST + S - 1) % S, LPS * (u + 1), REST ? LPS : 0);
            } else if (!LAST) {
                __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0<VM>);
                plain_barrier();
                step(fi, (ST + 1) % S, 0, true, j + S, ST, 0, NEXT ? LPS : 0);
            } else {
                step(fi, 0, 0, false, 0, 0, 0, 0);
            }
        }
    };
    using yes = std::true_type;
    using no = std::false_type;
    constexpr int VMS = (S - 2) * G::PC;
    int j = 0;
    for (; j + S < nk; j += S) {
        chunk(j + 0, IC<0>{}, yes{}, yes{}, IC<VMS>{}, no{});
        chunk(j + 1, IC<1>{}, yes{}, yes{}, IC<VMS>{}, no{});
        chunk(j + 2, IC<2>{}, yes{}, yes{}, IC<VMS>{}, no{});
        chunk(j + 3, IC<3>{}, yes{}, yes{}, IC<VMS>{}, no{});
    }
    // The last S chunks: only chunk nk - S still loads (the rest of chunk
    // nk - 1); the barriers wait for what is left.
    chunk(j + 0, IC<0>{}, yes{}, no{}, IC<VMS>{}, no{});
    chunk(j + 1, IC<1>{}, no{}, no{}, IC<(S - 3) * G::PC>{}, no{});
    chunk(j + 2, IC<2>{}, no{}, no{}, IC<0>{}, no{});
    chunk(j + 3, IC<3>{}, no{}, no{}, IC<0>{}, yes{});

    write_tile<NB, WN>(acc, Y, M, N, ldy, m0 + wm * 128 + r32, n0 + wn * WN + 4 * h, m0 + wm * 128, n0 + wn * WN);
}

} // namespace

bool gemm_wide_fits(const GemmArgs &a, int es, int vec)
{
    // 16-byte pieces (vec * es == 16), 256-row tile offsets under 2^31 bytes.
    return es == 2 && vec * es == 16 && a.ldx * es * WB + a.K * es < (int64_t(1) << 31) &&
           a.ldw * es * WB + a.K * es < (int64_t(1) << 31);
}

int64_t gemm_wide_workgroups(const GemmArgs &a) { return ((a.M + WB - 1) / WB) * ((a.N + WB - 1) / WB); }

namespace {
template <class E, int BKB, int S, int NWN>
hipError_t launch_wide_cfg(const GemmArgs &a, hipStream_t s)
{
    const int64_t tm = (a.M + WB - 1) / WB, tn = (a.N + WB - 1) / WB;
    hipLaunchKernelGGL((gemm_nt_wide_kernel<E, BKB, S, NWN>), dim3((unsigned)(tm * tn)), dim3(2 * NWN * 64), 0, s,
                       (const char *)a.X, (const char *)a.W, a.Y, a.M, a.N, a.K, a.ldx, a.ldw, a.ldy, tm, tn);
    return hipGetLastError();
}

template <class E>
hipError_t launch_wide_full(const GemmArgs &a, hipStream_t s)
{
    const int64_t tm = (a.M + WB - 1) / WB, tn = (a.N + WB - 1) / WB;
    hipLaunchKernelGGL((gemm_nt_wide_full_kernel<E, 64, 4, 4>), dim3((unsigned)(tm * tn)), dim3(512), 0, s,
                       (const char *)a.X, (const char *)a.W, a.Y, a.M, a.N, a.K, a.ldx, a.ldw, a.ldy, tm, tn);
    return hipGetLastError();
}

// Default: eight waves, 64-byte k-chunks, four stages; the full-turn kernel
// where K * 2 bytes is a multiple of the 256 bytes of one turn of the ring
// (K % 128 == 0), else the ring kernel. CAS_GEMM_WIDE=<chunk bytes>x<stages>[w8]
// picks another chunk width, stage count and four or eight waves of the ring
// kernel (tuning); CAS_GEMM_WIDE=ring forces the ring kernel's default layout.
template <class E>
hipError_t launch_wide_elem(const GemmArgs &a, hipStream_t s)
{
    const char *v = std::getenv("CAS_GEMM_WIDE");
    const std::string c = v ? v : "";
    if (c == "128x2") return launch_wide_cfg<E, 128, 2, 2>(a, s);
    if (c == "64x3") return launch_wide_cfg<E, 64, 3, 2>(a, s);
    if (c == "64x4") return launch_wide_cfg<E, 64, 4, 2>(a, s);
    if (c == "128x2w8") return launch_wide_cfg<E, 128, 2, 4>(a, s);
    if (c == "64x3w8") return launch_wide_cfg<E, 64, 3, 4>(a, s);
    if (c.empty() && a.K > 0 && (a.K * E::ES) % (4 * 64) == 0) return launch_wide_full<E>(a, s);
    return launch_wide_cfg<E, 64, 4, 4>(a, s);
}
} // namespace

hipError_t launch_gemm_wide(const GemmArgs &a, int elem, hipStream_t s)
{
    return elem == E_BF16 ? launch_wide_elem<KBF16>(a, s) : launch_wide_elem<KF16>(a, s);
}

// ---------------------------------------------------------------------------
// Rows not in 16-byte pieces (an odd pitch, a base off a 16-byte boundary, K
// not a multiple of 8). The load unit's 16-byte buffer loads take any element
// alignment, so the wide kernel runs over the first K8 = K - K % 8 columns,
// whose pieces all lie inside their rows; the last r = K % 8 columns are then
// added by a tail kernel, y += sum_{j < r} x[m][K8 + j] w[n][K8 + j], one
// fused multiply-add per column in column order (the same products; the
// tolerance of fp32 accumulation covers the order). The fp32 register ring
// on 128 x 128 tiles uses the same tail kernel for K % 4 (gemm_nt.hip).
// ---------------------------------------------------------------------------
namespace {

constexpr int KT_B = 64; // output block edge of the tail kernel

// An element's value in fp32 (exact for every input format).
template <class E> __device__ __forceinline__ float elem_f32(const char *p);
template <> __device__ __forceinline__ float elem_f32<KF32>(const char *p) { return *reinterpret_cast<const float *>(p); }
template <> __device__ __forceinline__ float elem_f32<KBF16>(const char *p)
{
    return __uint_as_float((uint32_t)*reinterpret_cast<const uint16_t *>(p) << 16);
}
template <> __device__ __forceinline__ float elem_f32<KF16>(const char *p)
{
    return (float)__builtin_bit_cast(_Float16, *reinterpret_cast<const uint16_t *>(p));
}

template <class E>
__global__ void __launch_bounds__(256) gemm_ktail_kernel(const char *__restrict__ X, const char *__restrict__ W,
                                                          float *__restrict__ Y, int64_t M, int64_t N, int64_t K8,
                                                          int r, int64_t ldx, int64_t ldw, int64_t ldy, int64_t tn)
{
    constexpr int ES = E::ES;
    __shared__ float xs[KT_B][8];
    __shared__ float ws[KT_B][8];
    const int tid = threadIdx.x;
    const int64_t bm = blockIdx.x / tn, bn = blockIdx.x - bm * tn;
    const int64_t m0 = bm * KT_B, n0 = bn * KT_B;
    // the tail columns of the block's 64 X rows and 64 W rows, as fp32 (zero past M / N)
    for (int i = tid; i < 2 * KT_B * 8; i += 256) {
        const int side = i / (KT_B * 8), row = (i / 8) % KT_B, j = i % 8;
        float v = 0.f;
        if (j < r) {
            if (side == 0 && m0 + row < M)
                v = elem_f32<E>(X + ((m0 + row) * ldx + K8 + j) * ES);
            else if (side == 1 && n0 + row < N)
                v = elem_f32<E>(W + ((n0 + row) * ldw + K8 + j) * ES);
        }
        (side == 0 ? xs : ws)[row][j] = v;
    }
    __syncthreads();
    const int c = tid % KT_B, rq = tid / KT_B; // column c; rows rq, rq + 4, ..
    const int64_t n = n0 + c;
    if (n >= N) return;
    float w[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) w[j] = ws[c][j];
    for (int i = rq; i < KT_B; i += 4) {
        const int64_t m = m0 + i;
        if (m >= M) break;
        float *y = Y + m * ldy + n;
        float v = *y;
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (j < r) v = __builtin_fmaf(xs[i][j], w[j], v);
        *y = v;
    }
}

template <class E> hipError_t launch_ktail(const GemmArgs &a, int64_t K8, hipStream_t s)
{
    const int64_t tm = (a.M + KT_B - 1) / KT_B, tn = (a.N + KT_B - 1) / KT_B;
    hipLaunchKernelGGL((gemm_ktail_kernel<E>), dim3((unsigned)(tm * tn)), dim3(256), 0, s, (const char *)a.X,
                       (const char *)a.W, a.Y, a.M, a.N, K8, (int)(a.K - K8), a.ldx, a.ldw, a.ldy, tn);
    return hipGetLastError();
}

} // namespace

bool gemm_wide_fits_unaligned(const GemmArgs &a, int es)
{
    // 16-bit elements at their alignment, at least one 8-column piece, and
    // the same 31-bit tile offsets as gemm_wide_fits; the tail grid in 2^32.
    const int64_t kt = ((a.M + KT_B - 1) / KT_B) * ((a.N + KT_B - 1) / KT_B);
    return es == 2 && (uintptr_t)a.X % 2 == 0 && (uintptr_t)a.W % 2 == 0 && a.K >= 8 &&
           a.ldx * es * WB + a.K * es < (int64_t(1) << 31) && a.ldw * es * WB + a.K * es < (int64_t(1) << 31) &&
           kt <= UINT32_MAX;
}

hipError_t launch_gemm_wide_unaligned(const GemmArgs &a, int elem, hipStream_t s)
{
    GemmArgs b = a;
    b.K = a.K - a.K % 8;
    const hipError_t e = launch_gemm_wide(b, elem, s);
    if (e != hipSuccess || b.K == a.K) return e;
    return launch_gemm_ktail(a, elem, b.K, s);
}

bool gemm_ktail_fits(const GemmArgs &a)
{
    return ((a.M + KT_B - 1) / KT_B) * ((a.N + KT_B - 1) / KT_B) <= UINT32_MAX;
}

hipError_t launch_gemm_ktail(const GemmArgs &a, int elem, int64_t K0, hipStream_t s)
{
    switch (elem) {
    case E_F32: return launch_ktail<KF32>(a, K0, s);
    case E_BF16: return launch_ktail<KBF16>(a, K0, s);
    default: return launch_ktail<KF16>(a, K0, s);
    }
}

} // namespace cas
