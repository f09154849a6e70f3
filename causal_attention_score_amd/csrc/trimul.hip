// trimul.hip -- dispatch of the causal score kernel (trimul_kernel.hpp) by
// input element type.
#include "launch.hpp"

namespace cas {

hipError_t launch_trimul_f32(const TrimulArgs &a, int vec, hipStream_t s);
hipError_t launch_trimul_bf16(const TrimulArgs &a, int vec, hipStream_t s);
hipError_t launch_trimul_f16(const TrimulArgs &a, int vec, hipStream_t s);

int64_t trimul_workgroups(int64_t B, int64_t T, int64_t NH)
{
    const int64_t nt = (T + 63) / 64;             // 64 x 64 score tiles
    const int64_t items = B * NH * (nt * (nt + 1) / 2);
    return (items + 3) / 4;                       // four compute waves per workgroup
}

hipError_t launch_trimul(const TrimulArgs &a, int elem, int vec, hipStream_t s)
{
    switch (elem) {
    case E_F32: return launch_trimul_f32(a, vec, s);
    case E_BF16: return launch_trimul_bf16(a, vec, s);
    default: return launch_trimul_f16(a, vec, s);
    }
}

} // namespace cas
