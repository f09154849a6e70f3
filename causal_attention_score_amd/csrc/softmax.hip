// softmax.hip -- dispatch of the causal softmax kernels (softmax_kernel.hpp)
// by input element type.
#include "launch.hpp"

namespace cas {

hipError_t launch_row_stats_f32(const TrimulArgs &a, hipStream_t s);
hipError_t launch_row_stats_bf16(const TrimulArgs &a, hipStream_t s);
hipError_t launch_row_stats_f16(const TrimulArgs &a, hipStream_t s);
hipError_t launch_softmax_f32(const TrimulArgs &a, int mode, hipStream_t s);
hipError_t launch_softmax_bf16(const TrimulArgs &a, int mode, hipStream_t s);
hipError_t launch_softmax_f16(const TrimulArgs &a, int mode, hipStream_t s);
hipError_t launch_softmax_fused_f32(const TrimulArgs &a, int mode, hipStream_t s);
hipError_t launch_softmax_fused_bf16(const TrimulArgs &a, int mode, hipStream_t s);
hipError_t launch_softmax_fused_f16(const TrimulArgs &a, int mode, hipStream_t s);

bool softmax_fits(int64_t T, int64_t HS, int es, int vec)
{
    // Rows in 16-byte pieces, heads of at most 512 bytes (the three-role
    // kernels up to 256, the wide variants and the per-wave tile kernel
    // above), tile offsets within 31-bit buffer ranges.
    return vec * es >= 16 && HS * es <= 512 && T < (int64_t(1) << 22);
}

int64_t row_stats_workgroups(int64_t B, int64_t T, int64_t NH)
{
    const int64_t nt = (T + 127) / 128; // 128-row query blocks, one per workgroup
    return B * NH * nt;
}

hipError_t launch_row_stats(const TrimulArgs &a, int elem, hipStream_t s)
{
    switch (elem) {
    case E_F32: return launch_row_stats_f32(a, s);
    case E_BF16: return launch_row_stats_bf16(a, s);
    default: return launch_row_stats_f16(a, s);
    }
}

hipError_t launch_softmax(const TrimulArgs &a, int elem, int mode, hipStream_t s)
{
    switch (elem) {
    case E_F32: return launch_softmax_f32(a, mode, s);
    case E_BF16: return launch_softmax_bf16(a, mode, s);
    default: return launch_softmax_f16(a, mode, s);
    }
}

hipError_t launch_softmax_fused(const TrimulArgs &a, int elem, int mode, hipStream_t s)
{
    switch (elem) {
    case E_F32: return launch_softmax_fused_f32(a, mode, s);
    case E_BF16: return launch_softmax_fused_bf16(a, mode, s);
    default: return launch_softmax_fused_f16(a, mode, s);
    }
}

} // namespace cas
