// gemm_nt_direct.hip -- dense Y = X W^T for fp32 inputs on shapes of about one
// 64 x 64 output tile per CU (the 960 x 1024 x 770 dense layer), with the
// operands streamed global -> LDS by the load unit itself.
//
// Workload: the dense layer of DietCode's test_1_local_padding.py
// (test_local_padding docstring), Y[i,j] += X[i,k] * W[j,k], in fp32.
//
// Why a kernel of its own. On a SIMD running fp32 MFMAs (v_mfma_f32_32x32x2f32)
// every other instruction that reads vector registers waits for the matrix
// pipe, so the register-staged fetch of the general engine (a global load and
// an LDS write per 8 bytes for rows of 770 floats, which are only 8-byte
// aligned, plus the out-of-range selects) costs MFMA time. Here each 16-byte
// piece of a row goes from HBM straight into LDS with one buffer load per
// kilobyte per wave (the load unit accepts 16-byte pieces at any 4-byte
// aligned address), and the main loop holds MFMAs, LDS reads, these loads, one
// barrier per chunk and scalar arithmetic only.
//
// Stage model (same docstring: Fetch, Compute, Writeback), with local padding:
//  * Fetch: each lane's piece offsets within the tile are fixed; a chunk is
//    chosen by moving the buffer resource's base, and the resource's size
//    ends at the tile's last row's last element. Rows past M (or N) get an
//    out-of-range offset; both read zero. The one piece per row that straddles
//    K (when K is not a multiple of 4) reads past the row's end, so the last
//    chunk zeroes those contraction indices in its fragments -- the only
//    predicate, outside the main loop.
//  * Compute: the MFMA loop over whole chunks has no predicate.
//  * Writeback: the only other place that looks at M and N.
//
// Layout: four waves in a 2 x 2 grid, each accumulating a 32 x 32 block
// (one f32x16 per lane) as D = W X^T, so a lane's four consecutive
// accumulators are four consecutive output columns. A chunk is 32 floats
// (128 bytes) of each of the 64 X rows and 64 W rows: 16 KB, 16 load
// instructions, four per wave. Piece c of tile row r sits at slot
// c ^ ((r / 2) % 8): the LDS serves 16-byte reads 16 lanes at a time, and
// 16 consecutive rows read at one piece then hit 16 distinct bank groups.
// S stages (four, or three where more than two workgroups per CU are needed)
// form a ring: the loads of chunk k + S are issued once every wave is done
// with chunk k. Lane half h (the MFMA k-slot) takes pieces 4h .. 4h + 3
// of a chunk for X and W alike, so every product x_k w_k is formed once.
#include "launch.hpp"
#include "tile_engine.hpp"

#include <type_traits>

namespace cas {

namespace {

constexpr int DT = 64;                     // output tile edge
constexpr int DBKB = 128;                  // bytes of a row per chunk (32 floats)
constexpr int DSPR = DBKB / 16;            // 16-byte pieces per row
constexpr int DOPB = DT * DBKB;            // one operand tile of one stage
constexpr int DSTAGE = 2 * DOPB;
constexpr int DLOADS = DOPB / 1024 / 4;    // loads per wave and operand per chunk
constexpr int DPC = 2 * DLOADS;            // loads per wave per chunk
constexpr int DNU = DSPR / 2;              // k-steps per chunk (one piece per lane half each)
constexpr int DGROUP_M = 4;                // tile rows walked together (operand panels shared in L2)
constexpr uint32_t DOOB = 0x80000000u;     // buffer offset the load unit reads as zero

static_assert(DPC == DNU, "one load per k-step");

typedef __attribute__((address_space(3))) void lds_void;
typedef float f32x4v __attribute__((ext_vector_type(4)));

// s_waitcnt immediate: at most N vector memory operations in flight, no LDS operation.
template <int N> constexpr int dwait_vm = (N & 15) | (7 << 4) | (0 << 8) | ((N >> 4) << 14);

__device__ __forceinline__ int dswz(int r) { return (r >> 1) & (DSPR - 1); }

// Buffer resource of chunk c of one operand tile: base moved c chunks along
// the rows, size ending at the tile's last element (extent bytes from the
// tile's first row). Scalar arithmetic only.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t dchunk_rsrc(const char *tile, int extent, int c)
{
    const int off = c * DBKB;
    const int n = extent - off > 0 ? extent - off : 0;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(tile + off), (short)0, n, 0x00020000);
}

template <int V> using DIC = std::integral_constant<int, V>;

template <int S>
__global__ void __launch_bounds__(256)
gemm_nt_direct_kernel(const char *__restrict__ X, const char *__restrict__ W, float *__restrict__ Y,
                      int64_t M, int64_t N, int64_t K, int64_t ldx, int64_t ldw, int64_t ldy,
                      int64_t tiles_m, int64_t tiles_n, int64_t batch, int64_t bsx, int64_t bsw, int64_t bsy)
{
    // S stages of 16 KB: S <= 4 keeps every LDS offset within the 16-bit
    // immediate of the LDS instructions.
    static_assert(S >= 3 && S * DSTAGE <= 64 * 1024 && (S - 2) * DPC + 1 <= 63, "stages");
    __shared__ __attribute__((aligned(1024))) char lds[S * DSTAGE];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave >> 1, wn = wave & 1;

    // Logical id = batch * tiles + tile; each XCD takes a contiguous range of
    // them, walked in groups of DGROUP_M tile rows.
    const int64_t tiles = tiles_m * tiles_n;
    const int64_t lid = xcd_remap(blockIdx.x, tiles * batch);
    const int64_t bt = lid / tiles, pid = lid - bt * tiles;
    const int64_t group = DGROUP_M * tiles_n;
    const int64_t first_m = (pid / group) * DGROUP_M;
    const int64_t gm = (tiles_m - first_m) < DGROUP_M ? (tiles_m - first_m) : DGROUP_M;
    const int64_t tm = first_m + (pid % group) % gm;
    const int64_t tn = (pid % group) / gm;
    const int64_t m0 = tm * DT, n0 = tn * DT;
    const int rows_x = (int)(M - m0 < DT ? M - m0 : DT);
    const int rows_w = (int)(N - n0 < DT ? N - n0 : DT);
    const uint32_t ldxb = (uint32_t)(ldx * 4), ldwb = (uint32_t)(ldw * 4);
    const char *xt = X + (bt * bsx + m0 * ldx) * 4;
    const char *wt = W + (bt * bsw + n0 * ldw) * 4;
    // The host keeps 64 rows of either pitch plus K below 2^31 bytes.
    const int ext_x = (int)((rows_x - 1) * ldx * 4 + K * 4), ext_w = (int)((rows_w - 1) * ldw * 4 + K * 4);
    Y += bt * bsy;
    const int nk = (int)((K + 31) / 32);

    // This lane's piece offsets within the tile, one per load of a chunk:
    // loads 0 .. DLOADS-1 fill X rows 8(DLOADS wave + q) .., the rest W rows.
    uint32_t vo[DPC];
    const int rsub = lane / DSPR, slot = lane % DSPR;
#pragma unroll
    for (int q = 0; q < DPC; ++q) {
        const bool isx = q < DLOADS;
        const int r = (wave * DLOADS + (isx ? q : q - DLOADS)) * 8 + rsub;
        const int c = slot ^ dswz(r);
        vo[q] = r < (isx ? rows_x : rows_w) ? (uint32_t)r * (isx ? ldxb : ldwb) + (uint32_t)c * 16 : DOOB;
    }
    // Load q of chunk c into stage st (= c % S).
    auto fetch_one = [&](int st, int c, int q) {
        const bool isx = q < DLOADS;
        char *dst = lds + st * DSTAGE + (isx ? 0 : DOPB) + (wave * DLOADS + (isx ? q : q - DLOADS)) * 1024;
        const __amdgpu_buffer_rsrc_t rs = isx ? dchunk_rsrc(xt, ext_x, c) : dchunk_rsrc(wt, ext_w, c);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)dst, 16, (int)vo[q], 0, 0, 0);
    };

    const int r32 = lane & 31, h = lane >> 5, fr = dswz(r32); // rows 32 wm + r32 share dswz(r32)
    const char *xa0 = lds + (wm * 32 + r32) * DBKB, *wa0 = lds + DOPB + (wn * 32 + r32) * DBKB;
    auto read_frags = [&](int st, int u, u32x4 &fa, u32x4 &fb) {
        const int pos = st * DSTAGE + ((h * DNU + u) ^ fr) * 16;
        fa = *reinterpret_cast<const u32x4 *>(xa0 + pos);
        fb = *reinterpret_cast<const u32x4 *>(wa0 + pos);
    };

    f32x16 acc = {};
    u32x4 fa[2], fb[2];
    // One k-step: load q of chunk c (into stage lst), the next step's
    // fragments (stage nst, step nu), then the step's four MFMAs.
    auto step = [&](int fi, int lst, int c, int q, int nst, int nu) {
        __builtin_amdgcn_sched_barrier(0);
        fetch_one(lst, c, q);
        read_frags(nst, nu, fa[fi ^ 1], fb[fi ^ 1]);
        __builtin_amdgcn_sched_barrier(0);
        mfma_chunk<KF32>(acc, fb[fi], fa[fi]);
        __builtin_amdgcn_sched_barrier(0);
    };
    // Chunk kc (not the last) in stage s: loads 1 .. DPC - 1 of chunk
    // kc - 1 + S during its first steps, then, once every wave has read the
    // chunk, load 0 of chunk kc + S; both go to the stages of chunks already
    // consumed. The barrier waits for this wave's loads of chunk kc + 1.
    auto chunk = [&](auto sc, int kc) {
        constexpr int st = decltype(sc)::value;
#pragma unroll
        for (int u = 0; u < DNU; ++u) {
            const int fi = u & 1;
            if (u + 1 < DNU) {
                step(fi, (st + S - 1) % S, kc - 1 + S, u + 1, st, u + 1);
            } else {
                __builtin_amdgcn_s_waitcnt(dwait_vm<(S - 2) * DPC>); // chunk kc + 1 landed
                __builtin_amdgcn_s_barrier(); // ... for every wave; every wave done reading chunk kc
                step(fi, st, kc + S, 0, (st + 1) % S, 0);
            }
        }
    };
    auto chunk_dyn = [&](int kc) {
        switch (kc % S) {
        case 0: chunk(DIC<0>{}, kc); break;
        case 1: chunk(DIC<1>{}, kc); break;
        case 2: chunk(DIC<2 % S>{}, kc); break;
        default: chunk(DIC<(S - 1)>{}, kc); break;
        }
    };
    static_assert(S == 3 || S == 4, "chunk_dyn covers three or four stages");

    // The writeback's arguments, read from the kernel arguments now: a scalar
    // load left in flight in the main loop would make every wait for the
    // fragment reads a wait for all of them.
    asm volatile("" ::"s"(Y), "s"(ldy));
    if (nk > 0) {
        // Chunks past the end are loaded too (in-range garbage or zeros, into
        // stages nothing reads any more), so every barrier waits for the same
        // count: this wave's loads of chunk kc + 1 are done once at most
        // those of chunks kc + 2 .. kc + S - 1 are in flight.
#pragma unroll
        for (int c = 0; c + 1 < S; ++c)
#pragma unroll
            for (int q = 0; q < DPC; ++q) fetch_one(c, c, q);
        fetch_one(S - 1, S - 1, 0);
        __builtin_amdgcn_s_waitcnt(dwait_vm<(S - 2) * DPC + 1>); // chunk 0 landed
        __builtin_amdgcn_s_barrier();
        read_frags(0, 0, fa[0], fb[0]);
    }
    int kc = 0;
    for (; kc + S < nk; kc += S) { // whole turns: each chunk has a successor
#pragma unroll
        for (int s = 0; s < S; ++s) {
            if (s == 0) chunk(DIC<0>{}, kc);
            else if (s == 1) chunk(DIC<1>{}, kc + 1);
            else if (s == 2) chunk(DIC<2 % S>{}, kc + 2);
            else chunk(DIC<(S - 1)>{}, kc + 3);
        }
    }
    for (; kc + 1 < nk; ++kc) chunk_dyn(kc);
    if (nk > 0) {
        // The last chunk: no loads, no barrier; contraction indices k >= K
        // (the straddling piece's tail, read from past the row) are zeroed.
        const int st = (nk - 1) % S;
        const int64_t kl = (int64_t)(nk - 1) * 32 + h * (4 * DNU);
#pragma unroll
        for (int u = 0; u < DNU; ++u) {
            const int fi = u & 1;
            if (u + 1 < DNU) read_frags(st, u + 1, fa[fi ^ 1], fb[fi ^ 1]);
#pragma unroll
            for (int d = 0; d < 4; ++d)
                if (kl + 4 * u + d >= K) {
                    fa[fi][d] = 0u;
                    fb[fi][d] = 0u;
                }
            mfma_chunk<KF32>(acc, fb[fi], fa[fi]);
        }
    }
    // Loads of chunks past the end may still be writing LDS.
    __builtin_amdgcn_s_waitcnt(dwait_vm<0>);

    // Writeback: lane l, registers 4g .. 4g + 3 hold row 32 wm + l % 32 and
    // columns 32 wn + 8g + 4h + 0..3, masked on the true M and N.
    const int64_t row = m0 + wm * 32 + r32, col0 = n0 + wn * 32 + 4 * h;
    if (row < M) {
        float *yr = Y + row * ldy;
        const bool vec = ((uintptr_t)Y % 16 == 0) && (ldy % 4 == 0) && n0 + wn * 32 + 32 <= N;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int64_t c = col0 + 8 * g;
            if (vec) {
                *reinterpret_cast<f32x4v *>(yr + c) = f32x4v{acc[4 * g], acc[4 * g + 1], acc[4 * g + 2], acc[4 * g + 3]};
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (c + e < N) yr[c + e] = acc[4 * g + e];
            }
        }
    }
}

} // namespace

bool gemm_direct_fits(const GemmArgs &a, int elem, int vec)
{
    // fp32 elements at their alignment (the load unit takes 16-byte pieces at
    // any element alignment), 64-row tile offsets under 2^31 bytes. Its 64 KB of LDS hold two workgroups per CU against
    // the register-ring engine's four, so with more than 512 workgroups it
    // pays only on long contractions (measured: 192 heads of 120 x 120, 768
    // workgroups, K = 64 .. 256: 10.1 .. 18.7 us on the ring against 11.2 ..
    // 20.1 us; 960 x 2304 x 770, 540 workgroups: 43.4 against 47.1 us).
    (void)vec;
    if (elem != E_F32 || a.predicated || a.K <= 0 || (uintptr_t)a.X % 4 != 0 || (uintptr_t)a.W % 4 != 0)
        return false;
    if (a.ldx * 4 * DT + a.K * 4 >= (int64_t(1) << 31) || a.ldw * 4 * DT + a.K * 4 >= (int64_t(1) << 31))
        return false;
    const int64_t wgs = ((a.M + DT - 1) / DT) * ((a.N + DT - 1) / DT) * a.batch;
    return wgs <= 512 || a.K >= 512;
}

hipError_t launch_gemm_direct(const GemmArgs &a, hipStream_t s)
{
    const int64_t tm = (a.M + DT - 1) / DT, tn = (a.N + DT - 1) / DT, wgs = tm * tn * a.batch;
    // Four stages (64 KB: two workgroups per CU) up to 512 workgroups; above
    // that three (48 KB: three per CU), so that one round holds them all
    // (960 x 2304 x 770, 540 workgroups: 39.3 against 40.8 us; 1500^2 x 3000:
    // 130.9 against 134.1 us; at 240 workgroups the two are level).
    if (wgs > 512)
        hipLaunchKernelGGL((gemm_nt_direct_kernel<3>), dim3((unsigned)wgs), dim3(256), 0, s, (const char *)a.X,
                           (const char *)a.W, a.Y, a.M, a.N, a.K, a.ldx, a.ldw, a.ldy, tm, tn, a.batch, a.bsx, a.bsw,
                           a.bsy);
    else
        hipLaunchKernelGGL((gemm_nt_direct_kernel<4>), dim3((unsigned)wgs), dim3(256), 0, s, (const char *)a.X,
                           (const char *)a.W, a.Y, a.M, a.N, a.K, a.ldx, a.ldw, a.ldy, tm, tn, a.batch, a.bsx, a.bsw,
                           a.bsy);
    return hipGetLastError();
}

} // namespace cas
