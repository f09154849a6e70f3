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
// Data path. A workgroup holds four waves, one per SIMD, in a 2 x 2 grid;
// each wave accumulates a 128 x 128 block as 4 x 4 MFMA tiles of 32 x 32
// (v_mfma_f32_32x32x16_{bf16,f16}, 256 fp32 accumulators per lane). Each
// k-chunk of BK = 64 elements (128-byte rows) of the 256 X rows and 256 W rows
// lands in LDS straight from the load unit: one load instruction fills 1 KB
// of LDS (8 rows), lane i writing bytes [16i, 16i + 16). Chunk c of row r is
// stored at 16-byte slot c ^ (r % 8) of its row: the loads pick their source
// addresses accordingly, and the MFMA operand reads (32 rows, one chunk per
// lane half) then hit 8 distinct bank groups per 8 lanes. Two LDS stages: the
// load of chunk k+2 is issued right after the barrier inside chunk k, so it
// has about a chunk of MFMAs (64 per wave) to arrive.
//
// Contraction-order permutation: in a chunk, lane half h (the MFMA k-slot)
// takes 16-byte pieces 4h..4h+3, for X and W alike, so every product
// x_k * w_k is formed exactly once.
#include "launch.hpp"
#include "tile_engine.hpp"

namespace cas {

namespace {

constexpr int WB = 256;              // output tile edge
constexpr int WBK_BYTES = 128;       // bytes of a row per k-chunk (64 16-bit elements)
constexpr int WSLOTS = WBK_BYTES / 16;
constexpr int WOP_BYTES = WB * WBK_BYTES;   // one operand tile per stage (32 KB)
constexpr int WSTAGE = 2 * WOP_BYTES;       // X tile + W tile
constexpr int WTHREADS = 256;
constexpr int WGROUP_M = 4;
constexpr uint32_t WOOB = 0x80000000u;      // buffer offset the load unit reads as zero

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t wide_rsrc(const char *base)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(base), (short)0, 0x7FFFFFFF, 0x00020000);
}

// Fetch stage of one operand: rows [0, 256) of the tile whose first row is at
// `rs`, k-chunk k0 (elements). Wave w issues loads j = 0..7, each filling the
// 1 KB of LDS that holds tile rows 8(8w + j) .. +8.
__device__ __forceinline__ void fetch_operand(__amdgpu_buffer_rsrc_t rs, char *lds_tile, uint32_t ldb, int rows,
                                              uint32_t k0b, uint32_t kb, int wave, int lane)
{
    const int rsub = lane >> 3, slot = lane & 7;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int r = (wave * 8 + j) * 8 + rsub;                 // tile row written by this lane
        const uint32_t cb = k0b + (uint32_t)((slot ^ (r & 7)) * 16); // its source piece (bytes)
        const uint32_t vo = (r < rows && cb < kb) ? (uint32_t)r * ldb + cb : WOOB;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)(lds_tile + (wave * 8 + j) * 1024), 16, (int)vo,
                                                 0, 0, 0);
    }
}

template <class E>
__global__ void __launch_bounds__(WTHREADS)
gemm_nt_wide_kernel(const char *__restrict__ X, const char *__restrict__ W, float *__restrict__ Y,
                    int64_t M, int64_t N, int64_t K, int64_t ldx, int64_t ldw, int64_t ldy,
                    int64_t tiles_m, int64_t tiles_n)
{
    constexpr int ES = E::ES;
    __shared__ __attribute__((aligned(1024))) char lds[2 * WSTAGE];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave >> 1, wn = wave & 1;

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
    const int64_t nk = (K * ES + WBK_BYTES - 1) / WBK_BYTES;

    f32x16 acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = f32x16{};

    const int r32 = lane & 31, h = lane >> 5;
    // Fragments of k16 step u of a chunk: 16-byte piece 4h + u of rows
    // 32i + r32 (which all share r32 % 8, hence one swizzled position).
    auto read_frags = [&](const char *stage, int u, u32x4 (&af)[4], u32x4 (&bfr)[4]) {
        const int pos = ((4 * h + u) ^ (r32 & 7)) * 16;
        const char *xa = stage + (wm * 128 + r32) * WBK_BYTES + pos;
        const char *wa = stage + WOP_BYTES + (wn * 128 + r32) * WBK_BYTES + pos;
#pragma unroll
        for (int i = 0; i < 4; ++i) af[i] = *reinterpret_cast<const u32x4 *>(xa + i * 32 * WBK_BYTES);
#pragma unroll
        for (int i = 0; i < 4; ++i) bfr[i] = *reinterpret_cast<const u32x4 *>(wa + i * 32 * WBK_BYTES);
    };
    // Stage s of LDS holds chunks s, s + 2, ... Per chunk one barrier, before
    // its last step's MFMAs: by then every wave holds that step's fragments in
    // registers, so after the barrier the chunk's stage takes the load of
    // chunk + 2 while the next chunk's first fragments are read behind the
    // MFMAs. The barrier's fence also waits for this wave's loads of
    // chunk + 1 (the only ones in flight).
    u32x4 fa[2][4], fb[2][4];
    if (nk > 0) {
        fetch_operand(rx, lds, ldxb, rows_x, 0, kb, wave, lane);
        fetch_operand(rw, lds + WOP_BYTES, ldwb, rows_w, 0, kb, wave, lane);
        __syncthreads(); // chunk 0 in LDS
        if (nk > 1) {
            fetch_operand(rx, lds + WSTAGE, ldxb, rows_x, WBK_BYTES, kb, wave, lane);
            fetch_operand(rw, lds + WSTAGE + WOP_BYTES, ldwb, rows_w, WBK_BYTES, kb, wave, lane);
        }
        read_frags(lds, 0, fa[0], fb[0]);
    }
    for (int64_t kc = 0; kc < nk; ++kc) {
        const char *cur = lds + (kc & 1) * WSTAGE;
#pragma unroll
        for (int u = 0; u < WSLOTS / 2; ++u) {
            const int f = u & 1;
            if (u + 1 < WSLOTS / 2) {
                read_frags(cur, u + 1, fa[f ^ 1], fb[f ^ 1]);
            } else if (kc + 1 < nk) {
                __syncthreads(); // chunk kc + 1 in LDS; every wave done reading chunk kc
                if (kc + 2 < nk) {
                    char *stg = lds + (kc & 1) * WSTAGE;
                    const uint32_t k0b = (uint32_t)(kc + 2) * WBK_BYTES;
                    fetch_operand(rx, stg, ldxb, rows_x, k0b, kb, wave, lane);
                    fetch_operand(rw, stg + WOP_BYTES, ldwb, rows_w, k0b, kb, wave, lane);
                }
                read_frags(lds + ((kc + 1) & 1) * WSTAGE, 0, fa[f ^ 1], fb[f ^ 1]);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
                for (int b = 0; b < 4; ++b) mfma_chunk<E>(acc[a][b], fa[f][a], fb[f][b]);
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // Writeback: lane l, register r of block (a, b) holds row
    // 32a + acc_row(r, l) and column 32b + l % 32 of this wave's block, so one
    // store instruction writes two whole 128-byte row pieces.
    const int64_t row0 = m0 + wm * 128, col0 = n0 + wn * 128;
    float *yw = Y + row0 * ldy + col0 + r32;
    if (row0 + 128 <= M && col0 + 128 <= N) {
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int b = 0; b < 4; ++b)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    __builtin_nontemporal_store(acc[a][b][r], yw + (32 * a + acc_row(r, lane)) * ldy + 32 * b);
    } else {
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const bool col_ok = col0 + 32 * b + r32 < N;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int rr = 32 * a + acc_row(r, lane);
                    if (col_ok && row0 + rr < M) __builtin_nontemporal_store(acc[a][b][r], yw + rr * ldy + 32 * b);
                }
            }
    }
}

} // namespace

bool gemm_wide_fits(const GemmArgs &a, int es, int vec)
{
    // 16-byte pieces (vec * es == 16), 256-row tile offsets under 2^31 bytes.
    return es == 2 && vec * es == 16 && a.ldx * es * WB + a.K * es < (int64_t(1) << 31) &&
           a.ldw * es * WB + a.K * es < (int64_t(1) << 31);
}

int64_t gemm_wide_workgroups(const GemmArgs &a) { return ((a.M + WB - 1) / WB) * ((a.N + WB - 1) / WB); }

hipError_t launch_gemm_wide(const GemmArgs &a, int elem, hipStream_t s)
{
    const int64_t tm = (a.M + WB - 1) / WB, tn = (a.N + WB - 1) / WB;
    if (elem == E_BF16)
        hipLaunchKernelGGL(gemm_nt_wide_kernel<KBF16>, dim3((unsigned)(tm * tn)), dim3(WTHREADS), 0, s,
                           (const char *)a.X, (const char *)a.W, a.Y, a.M, a.N, a.K, a.ldx, a.ldw, a.ldy, tm, tn);
    else
        hipLaunchKernelGGL(gemm_nt_wide_kernel<KF16>, dim3((unsigned)(tm * tn)), dim3(WTHREADS), 0, s,
                           (const char *)a.X, (const char *)a.W, a.Y, a.M, a.N, a.K, a.ldx, a.ldw, a.ldy, tm, tn);
    return hipGetLastError();
}

} // namespace cas
