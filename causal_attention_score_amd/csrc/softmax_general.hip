// softmax_general.hip -- launchers of the general-shape causal softmax and
// attention kernels (softmax_general.hpp) for the three input types.
#include "softmax_general.hpp"

namespace cas {

namespace {

gen::GenArgs gen_args(const TrimulArgs &a, int es)
{
    gen::GenArgs g{};
    g.qkv = static_cast<const char *>(a.qkv);
    g.B = a.B;
    g.T = a.T;
    g.C = a.C;
    g.NH = a.NH;
    g.HS = (int)a.HS;
    // Chunks of whole 32-column blocks of the attention output, at most
    // GMAX_HEAD bytes (fp32 160, 16-bit 320 elements: at least the NDB * 32
    // columns of one attention pass).
    const int64_t hs32 = (a.HS + 31) / 32 * 32, cap = gen::GMAX_HEAD / es / 32 * 32;
    g.hch = (int)(hs32 < cap ? hs32 : cap);
    g.nch = (int)((a.HS + g.hch - 1) / g.hch);
    g.hsb = g.hch * es;
    g.pitch = g.hsb + 16;
    g.nqb = (uint32_t)((a.T + gen::GB - 1) / gen::GB);
    g.scale = a.scale;
    return g;
}

dim3 gen_grid(const gen::GenArgs &g) { return dim3((unsigned)(g.B * g.NH * (int64_t)g.nqb)); }

template <class E> hipError_t stats_e(const TrimulArgs &a, hipStream_t s)
{
    const gen::GenArgs g = gen_args(a, E::ES);
    hipLaunchKernelGGL((gen::gen_stats_kernel<E>), gen_grid(g), dim3(64), 2 * gen::GB * g.pitch, s, g,
                       const_cast<float *>(a.row_max), const_cast<float *>(a.row_logsum));
    return hipGetLastError();
}

template <class E, class O, class EP> hipError_t rows_eo(const TrimulArgs &a, hipStream_t s)
{
    const gen::GenArgs g = gen_args(a, E::ES);
    hipLaunchKernelGGL((gen::gen_rows_kernel<E, O, EP>), gen_grid(g), dim3(64), 2 * gen::GB * g.pitch, s, g,
                       a.row_max, a.row_logsum, static_cast<char *>(a.out));
    return hipGetLastError();
}

template <class E, class EP> hipError_t rows_e(const TrimulArgs &a, hipStream_t s)
{
    switch (a.out_kind) {
    case 0: return rows_eo<E, tri::OF32, EP>(a, s);
    case 1: return rows_eo<E, tri::OBF16, EP>(a, s);
    default: return rows_eo<E, tri::OF16, EP>(a, s);
    }
}

template <class E, bool STATS> hipError_t attention_e(const TrimulArgs &a, hipStream_t s)
{
    const gen::GenArgs g = gen_args(a, E::ES);
    hipLaunchKernelGGL((gen::gen_attention_kernel<E, STATS>), gen_grid(g), dim3(64), 3 * gen::GB * g.pitch, s, g,
                       const_cast<float *>(a.row_max), const_cast<float *>(a.row_logsum), static_cast<float *>(a.out));
    return hipGetLastError();
}

} // namespace

bool general_softmax_fits(int64_t B, int64_t T, int64_t NH, int es, const void *qkv)
{
    // Any head size (rows staged in chunks of at most GMAX_HEAD bytes, three
    // tiles of 32 rows within 64 KB of LDS), elements at their natural
    // alignment, one workgroup per 32-row block.
    return (uintptr_t)qkv % es == 0 && B * NH * ((T + gen::GB - 1) / gen::GB) <= INT32_MAX;
}

hipError_t launch_gen_row_stats(const TrimulArgs &a, int elem, hipStream_t s)
{
    switch (elem) {
    case E_F32: return stats_e<KF32>(a, s);
    case E_BF16: return stats_e<KBF16>(a, s);
    default: return stats_e<KF16>(a, s);
    }
}

hipError_t launch_gen_softmax(const TrimulArgs &a, int elem, int mode, hipStream_t s)
{
    const bool log = mode == 0;
    switch (elem) {
    case E_F32: return log ? rows_e<KF32, tri::EpLog>(a, s) : rows_e<KF32, tri::EpProb>(a, s);
    case E_BF16: return log ? rows_e<KBF16, tri::EpLog>(a, s) : rows_e<KBF16, tri::EpProb>(a, s);
    default: return log ? rows_e<KF16, tri::EpLog>(a, s) : rows_e<KF16, tri::EpProb>(a, s);
    }
}

hipError_t launch_gen_attention(const TrimulArgs &a, int elem, bool with_stats, hipStream_t s)
{
    switch (elem) {
    case E_F32: return with_stats ? attention_e<KF32, true>(a, s) : attention_e<KF32, false>(a, s);
    case E_BF16: return with_stats ? attention_e<KBF16, true>(a, s) : attention_e<KBF16, false>(a, s);
    default: return with_stats ? attention_e<KF16, true>(a, s) : attention_e<KF16, false>(a, s);
    }
}

} // namespace cas
