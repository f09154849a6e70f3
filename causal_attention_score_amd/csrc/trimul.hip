// trimul.hip -- causal attention scores straight from packed QKV on gfx950.
//
// Semantics: llm.c dev/cuda/trimat_forward.cu, trimul_cpu ("the Referee",
// Chapter I): out[b,nh,t,t2] = (Q[b,t,nh,:] . K[b,t2,nh,:]) * s for t2 <= t
// and NaN above the diagonal, with s = fp32 nearest 1/sqrt(HS).
//
// Differences from that file's GPU kernels (Chapters II-V), kept on purpose:
//  * Q and K tiles are fetched from the packed (B, T, 3, NH, HS) rows with
//    pitch 3C: no permute pass, and V is never read.
//  * The grid holds only the on- and below-diagonal tiles of every
//    (batch, head) plane: workgroup id -> (plane, i, j <= i) by inverting the
//    triangular numbers, instead of a square grid whose upper blocks return.
//  * The NaN mask is part of the contract: a diagonal tile writes NaN at
//    t2 > t, and every off-diagonal workgroup (i, j < i) also fills its mirror
//    tile (j, i) with NaN, so one launch writes the whole (T, T) plane.
//  * Any T >= 1 and any HS >= 1: ragged edges are zero-filled at fetch and
//    masked at writeback; offsets are 64-bit.
#include "launch.hpp"
#include "tile_engine.hpp"

#include <climits>

namespace cas {

namespace {

constexpr int BT = 128; // square score tile

template <class E> struct TriBK;
template <> struct TriBK<KF32> { static constexpr int v = 32; };
template <> struct TriBK<KBF16> { static constexpr int v = 64; };
template <> struct TriBK<KF16> { static constexpr int v = 64; };

constexpr unsigned QNAN_BITS = 0x7FC00000u;

template <class G, bool CHECK, bool DIAG>
__device__ __forceinline__ void store_scores(const f32x16 (&acc)[G::MB][G::NB], float *__restrict__ o, int64_t T,
                                             int64_t t0, int64_t s0, float scale, int wave_m, int wave_n, int lane)
{
    const float qnan = __uint_as_float(QNAN_BITS);
#pragma unroll
    for (int mb = 0; mb < G::MB; ++mb) {
#pragma unroll
        for (int nb = 0; nb < G::NB; ++nb) {
            const int64_t t2 = s0 + wave_n * G::WN + nb * 32 + (lane & 31);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t t = t0 + wave_m * G::WM + mb * 32 + acc_row(r, lane);
                float v = acc[mb][nb][r] * scale;
                if (DIAG && t2 > t) v = qnan;
                if (!CHECK || (t < T && t2 < T)) o[t * T + t2] = v;
            }
        }
    }
}

// NaN fill of rows [r0, r0+BT) x columns [c0, c0+BT) of one plane, clipped to T.
template <int NT>
__device__ __forceinline__ void fill_nan_tile(float *__restrict__ o, int64_t T, int64_t r0, int64_t c0, int tid,
                                              bool vec4)
{
    const float qnan = __uint_as_float(QNAN_BITS);
    const int64_t rows = (T - r0) < BT ? (T - r0) : BT;
    const int64_t cols = (T - c0) < BT ? (T - c0) : BT;
    if (vec4) { // T % 4 == 0 and a 16-byte aligned plane: cols is a multiple of 4
        const float4 n4 = make_float4(qnan, qnan, qnan, qnan);
#pragma unroll 4
        for (int idx = tid; idx < BT * (BT / 4); idx += NT) {
            const int r = idx / (BT / 4), c = (idx % (BT / 4)) * 4;
            if (r < rows && c < cols) *reinterpret_cast<float4 *>(o + (r0 + r) * T + c0 + c) = n4;
        }
    } else {
        for (int idx = tid; idx < BT * BT; idx += NT) {
            const int r = idx / BT, c = idx % BT;
            if (r < rows && c < cols) o[(r0 + r) * T + c0 + c] = qnan;
        }
    }
}

template <class E, int VEC>
__global__ void __launch_bounds__(256)
trimul_kernel(const char *__restrict__ qkv, float *__restrict__ out, int64_t T, int64_t C, int64_t NH, int64_t HS,
              int64_t tiles_per_plane, float scale, int vec_store)
{
    using G = Engine<E, BT, BT, TriBK<E>::v, 2, 2, VEC>;
    __shared__ __attribute__((aligned(16))) char lds[G::STAGE];

    const int tid = threadIdx.x;
    const int64_t id = blockIdx.x;
    const int64_t plane = id / tiles_per_plane;
    const int64_t r = id - plane * tiles_per_plane;
    // r = i(i+1)/2 + j with 0 <= j <= i: invert the triangular numbers.
    int64_t i = (int64_t)((sqrtf(8.0f * (float)r + 1.0f) - 1.0f) * 0.5f);
    while (i * (i + 1) / 2 > r) --i;
    while ((i + 1) * (i + 2) / 2 <= r) ++i;
    const int64_t j = r - i * (i + 1) / 2;

    const int64_t b = plane / NH, nh = plane - b * NH;
    const int64_t C3 = 3 * C;
    const char *q = qkv + (b * T * C3 + nh * HS) * G::ES; // Q[b][nh][0][:]
    const char *k = q + C * G::ES;                         // K[b][nh][0][:]
    const int64_t t0 = i * BT, s0 = j * BT;

    f32x16 acc[G::MB][G::NB];
    G::template mainloop<1>(acc, lds, q, C3, T, t0, k, C3, T, s0, HS, tid);

    float *o = out + plane * T * T;
    const int lane = tid & 63, wave = tid >> 6;
    const int wave_m = wave / 2, wave_n = wave % 2;
    const bool interior = (t0 + BT <= T); // s0 <= t0, so the columns fit too
    if (i == j) {
        if (interior) store_scores<G, false, true>(acc, o, T, t0, s0, scale, wave_m, wave_n, lane);
        else store_scores<G, true, true>(acc, o, T, t0, s0, scale, wave_m, wave_n, lane);
    } else {
        if (interior) store_scores<G, false, false>(acc, o, T, t0, s0, scale, wave_m, wave_n, lane);
        else store_scores<G, true, false>(acc, o, T, t0, s0, scale, wave_m, wave_n, lane);
        fill_nan_tile<G::NT>(o, T, s0, t0, tid, vec_store != 0); // mirror tile (j, i)
    }
}

template <class E, int VEC>
hipError_t launch_vec(const TrimulArgs &a, hipStream_t s)
{
    const int64_t nt = (a.T + BT - 1) / BT;
    const int64_t L = nt * (nt + 1) / 2;
    const int64_t nwg = a.B * a.NH * L;
    hipLaunchKernelGGL((trimul_kernel<E, VEC>), dim3((unsigned)nwg), dim3(256), 0, s, (const char *)a.qkv, a.out,
                       a.T, a.C, a.NH, a.HS, L, a.scale, (int)a.vec_store);
    return hipGetLastError();
}

template <class E>
hipError_t launch_elem(const TrimulArgs &a, int vec, hipStream_t s)
{
    constexpr int VMAX = 16 / E::ES;
    if (vec >= VMAX) return launch_vec<E, VMAX>(a, s);
    if (vec >= VMAX / 2) return launch_vec<E, VMAX / 2>(a, s);
    if constexpr (VMAX / 4 >= 1) {
        if (vec >= VMAX / 4) return launch_vec<E, VMAX / 4>(a, s);
    }
    return launch_vec<E, 1>(a, s);
}

} // namespace

int64_t trimul_workgroups(int64_t B, int64_t T, int64_t NH)
{
    const int64_t nt = (T + BT - 1) / BT;
    return B * NH * (nt * (nt + 1) / 2);
}

hipError_t launch_trimul(const TrimulArgs &a, int elem, int vec, hipStream_t s)
{
    switch (elem) {
    case E_F32: return launch_elem<KF32>(a, vec, s);
    case E_BF16: return launch_elem<KBF16>(a, vec, s);
    default: return launch_elem<KF16>(a, vec, s);
    }
}

} // namespace cas
