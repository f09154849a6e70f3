// gemm_nt.hip -- dense Y = X W^T on gfx950 MFMA, ragged shapes by local padding.
//
// Workload: the dense layer of DietCode's test_1_local_padding.py
// (test_local_padding docstring), Y[i,j] += X[i,k] * W[j,k]. Each workgroup
// owns one BM x BN output tile and runs the shared fetch -> LDS -> MFMA
// pipeline over K; edge tiles are zero-filled at fetch and masked at
// writeback, so the MFMA loop itself has no predicates.
//
// Tile order (the blog "Tensor Core学习", GEMM optimisation notes on L2
// locality and grid raster): workgroup ids are first regrouped per XCD, then
// walked in groups of GROUP_M tile rows so that neighbouring workgroups share
// X and W panels in L2.
#include "launch.hpp"

#include <cstdlib>
#include <cstring>
#include "tile_engine.hpp"

namespace cas {

namespace {

constexpr int GROUP_M = 4;

template <class E> struct GemmBK;
template <> struct GemmBK<KF32> { static constexpr int v = 32; };
template <> struct GemmBK<KBF16> { static constexpr int v = 64; };
template <> struct GemmBK<KF16> { static constexpr int v = 64; };

// Depth of the register ring that fetches ahead (RING > 0), by tile edge and
// bytes per global load. A ring lets a fetch have three chunks of MFMA work to
// land, which the single wave per SIMD of a one-tile-per-CU launch needs. On
// 128 x 128 tiles it pays only with 16-byte loads: narrower ones take more
// registers per chunk, the kernel passes 256 VGPRs, and two workgroups per CU
// no longer fit (bf16 4096 x 4096 x 4098: 237 us without, 252 with; bf16
// 2048^3: 34.3 us without, 26.6 with). RING = 0 fetches one chunk ahead (two
// LDS stages, no ring).
template <int BM, int VB> constexpr int gemm_ring = (BM == 64 || VB == 16) ? 4 : 0;

template <class E, int BM, int BN, int WGM, int WGN, int VEC, bool PRED, int RING>
__global__ void __launch_bounds__(WGM *WGN * 64)
gemm_nt_kernel(const char *__restrict__ X, const char *__restrict__ W, float *__restrict__ Y,
               int64_t M, int64_t N, int64_t K, int64_t ldx, int64_t ldw, int64_t ldy,
               int64_t tiles_m, int64_t tiles_n, int64_t batch, int64_t bsx, int64_t bsw, int64_t bsy)
{
    using G = Engine<E, BM, BN, GemmBK<E>::v, WGM, WGN, VEC, PRED>;
    __shared__ __attribute__((aligned(16))) char lds[2 * G::STAGE];

    const int tid = threadIdx.x;
    // Logical id = batch * tiles + tile; each XCD takes a contiguous range of
    // them, so the products of one batch share that XCD's L2.
    const int64_t tiles = tiles_m * tiles_n;
    const int64_t lid = xcd_remap(blockIdx.x, tiles * batch);
    const int64_t b = lid / tiles, pid = lid - b * tiles;
    X += b * bsx * G::ES;
    W += b * bsw * G::ES;
    Y += b * bsy;
    const int64_t group = GROUP_M * tiles_n;
    const int64_t first_m = (pid / group) * GROUP_M;
    const int64_t gm = (tiles_m - first_m) < GROUP_M ? (tiles_m - first_m) : GROUP_M;
    const int64_t tm = first_m + (pid % group) % gm;
    const int64_t tn = (pid % group) / gm;

    f32x16 acc[G::MB][G::NB];
    if constexpr (RING > 0)
        G::template mainloop_ring<RING>(acc, lds, X, ldx, M, tm * BM, W, ldw, N, tn * BN, K, tid);
    else
        G::template mainloop<2>(acc, lds, X, ldx, M, tm * BM, W, ldw, N, tn * BN, K, tid);

    // Writeback stage: predicated on the true M and N.
    const int lane = tid & 63, wave = tid >> 6;
    const int wave_m = wave / WGN, wave_n = wave % WGN;
#pragma unroll
    for (int mb = 0; mb < G::MB; ++mb) {
#pragma unroll
        for (int nb = 0; nb < G::NB; ++nb) {
            const int64_t col = tn * BN + wave_n * G::WN + nb * 32 + (lane & 31);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t row = tm * BM + wave_m * G::WM + mb * 32 + acc_row(r, lane);
                if (row < M && col < N) Y[row * ldy + col] = acc[mb][nb][r];
            }
        }
    }
}

template <int BM, int BN> struct TileCfg;
template <> struct TileCfg<64, 64> { static constexpr int WGM = 2, WGN = 2; };
template <> struct TileCfg<128, 128> { static constexpr int WGM = 2, WGN = 2; };

template <class E, int BM, int BN, int VEC>
hipError_t launch_tile(const GemmArgs &a, hipStream_t s)
{
    using C = TileCfg<BM, BN>;
    const int64_t tm = (a.M + BM - 1) / BM, tn = (a.N + BN - 1) / BN;
    const dim3 grid((unsigned)(tm * tn * a.batch));
    const dim3 block(C::WGM * C::WGN * 64);
    // The ring's buffer loads address a tile's rows from its first row with
    // 32-bit offsets below 2^31 - 1.
    constexpr int64_t BKB = GemmBK<E>::v * E::ES;
    const int64_t lim = INT64_C(0x7FFFFFFF);
    const bool ring = (BM * a.ldx * E::ES + BKB) <= lim && (BN * a.ldw * E::ES + BKB) <= lim;
#define CAS_GEMM_LAUNCH(PRED, RING)                                                                                    \
    hipLaunchKernelGGL((gemm_nt_kernel<E, BM, BN, C::WGM, C::WGN, VEC, PRED, RING>), grid, block, 0, s,               \
                       (const char *)a.X, (const char *)a.W, a.Y, a.M, a.N, a.K, a.ldx, a.ldw, a.ldy, tm, tn, a.batch, \
                       a.bsx, a.bsw, a.bsy)
    constexpr int RING = gemm_ring<BM, VEC * E::ES>;
    if constexpr (RING > 0) {
        if (ring) {
            if (a.predicated) CAS_GEMM_LAUNCH(true, RING);
            else CAS_GEMM_LAUNCH(false, RING);
            return hipGetLastError();
        }
    }
    if (a.predicated) CAS_GEMM_LAUNCH(true, 0);
    else CAS_GEMM_LAUNCH(false, 0);
#undef CAS_GEMM_LAUNCH
    return hipGetLastError();
}

template <class E, int BM, int BN>
hipError_t launch_vec(const GemmArgs &a, int vec, hipStream_t s)
{
    constexpr int VMAX = 16 / E::ES;
    if (vec >= VMAX) return launch_tile<E, BM, BN, VMAX>(a, s);
    if (vec >= VMAX / 2) return launch_tile<E, BM, BN, VMAX / 2>(a, s);
    if constexpr (VMAX / 4 >= 1) {
        if (vec >= VMAX / 4) return launch_tile<E, BM, BN, VMAX / 4>(a, s);
    }
    if constexpr (VMAX / 8 >= 1) {
        if (vec >= VMAX / 8) return launch_tile<E, BM, BN, VMAX / 8>(a, s);
    }
    return launch_tile<E, BM, BN, 1>(a, s);
}

int pick_tile(const GemmArgs &a, int tile)
{
    if (tile == GEMM_TILE_64 || tile == GEMM_TILE_128) return tile;
    // Largest tile that still gives every CU (256) about one workgroup.
    const int64_t t128 = ((a.M + 127) / 128) * ((a.N + 127) / 128) * a.batch;
    return t128 >= 256 ? GEMM_TILE_128 : GEMM_TILE_64;
}

// The register ring fetches through buffer loads, which take pieces at any
// element alignment (the base's and pitches' own alignment then does not
// matter): where the ring applies, the piece width comes from K alone.
template <class E, int BM>
int ring_vec(const GemmArgs &a, int vec)
{
    constexpr int ES = E::ES;
    if ((uintptr_t)a.X % ES != 0 || (uintptr_t)a.W % ES != 0) return vec;
    constexpr int64_t BKB = GemmBK<E>::v * ES;
    const int64_t lim = INT64_C(0x7FFFFFFF);
    if (BM * a.ldx * ES + BKB > lim || BM * a.ldw * ES + BKB > lim) return vec; // no ring: pointer loads
    for (int v = 16 / ES; v > vec; v /= 2)
        if (a.K % v == 0 && (BM == 64 || v * ES == 16)) return v;
    return vec;
}

template <class E>
hipError_t launch_elem(const GemmArgs &a, int vec, int tile, hipStream_t s)
{
    if (pick_tile(a, tile) == GEMM_TILE_128) {
        // The 128 x 128 ring needs 16-byte pieces; for K not a multiple of
        // them it runs over the first K0 = K - K % VMAX columns and the tail
        // kernel adds the rest (fp32 4096^2 x 4095: the two-stage loop with
        // 4-byte loads before).
        constexpr int VMAX = 16 / E::ES;
        GemmArgs b = a;
        b.K = a.K - a.K % VMAX;
        if (a.K % VMAX != 0 && b.K > 0 && !a.predicated && a.batch == 1 && gemm_ktail_fits(a) &&
            ring_vec<E, 128>(b, 1) == VMAX) {
            const hipError_t e = launch_vec<E, 128, 128>(b, VMAX, s);
            if (e != hipSuccess) return e;
            return launch_gemm_ktail(a, std::is_same<E, KF32>::value ? E_F32
                                        : std::is_same<E, KBF16>::value ? E_BF16 : E_F16, b.K, s);
        }
        return launch_vec<E, 128, 128>(a, ring_vec<E, 128>(a, vec), s);
    }
    return launch_vec<E, 64, 64>(a, ring_vec<E, 64>(a, vec), s);
}

} // namespace

int64_t gemm_nt_workgroups(const GemmArgs &a, int /*elem*/, int tile)
{
    const int bm = pick_tile(a, tile) == GEMM_TILE_128 ? 128 : 64;
    return ((a.M + bm - 1) / bm) * ((a.N + bm - 1) / bm) * a.batch;
}

hipError_t launch_gemm_nt(const GemmArgs &a, int elem, int vec, int tile, hipStream_t s)
{
    // 256 x 256 tiles where every CU gets one (M = N = 4096 and up); rows
    // not in 16-byte pieces take them too, with a tail kernel for K % 8.
    if (elem != E_F32 && !a.predicated && a.batch == 1 &&
        (tile == GEMM_TILE_256 || (tile == GEMM_TILE_AUTO && gemm_wide_workgroups(a) >= 256))) {
        if (gemm_wide_fits(a, 2, vec)) return launch_gemm_wide(a, elem, s);
        if (gemm_wide_fits_unaligned(a, 2)) return launch_gemm_wide_unaligned(a, elem, s);
    }
    // fp32 on 64 x 64 tiles: loads straight into LDS where the rows allow
    // (CAS_GEMM_F32=ring keeps the register-ring engine, e.g. to compare).
    if (elem == E_F32 && pick_tile(a, tile) == GEMM_TILE_64 && gemm_direct_fits(a, elem, vec)) {
        const char *v = std::getenv("CAS_GEMM_F32");
        if (!v || std::strcmp(v, "ring") != 0) return launch_gemm_direct(a, s);
    }
    switch (elem) {
    case E_F32: return launch_elem<KF32>(a, vec, tile, s);
    case E_BF16: return launch_elem<KBF16>(a, vec, tile, s);
    default: return launch_elem<KF16>(a, vec, tile, s);
    }
}

} // namespace cas
