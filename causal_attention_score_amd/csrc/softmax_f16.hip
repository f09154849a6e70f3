// softmax_f16.hip -- f16 inputs of the causal softmax kernels (row statistics,
// softmax rows and both fused; their own translation unit so the variants compile in
// parallel).
#include "softmax_kernel.hpp"

namespace cas {

hipError_t launch_row_stats_f16(const TrimulArgs &a, hipStream_t s) { return sm::launch_row_stats_impl<KF16>(a, s); }

hipError_t launch_softmax_f16(const TrimulArgs &a, int mode, hipStream_t s)
{
    return sm::launch_softmax_impl<KF16>(a, mode, s);
}

hipError_t launch_softmax_fused_f16(const TrimulArgs &a, int mode, hipStream_t s)
{
    return sm::launch_softmax_fused_impl<KF16>(a, mode, s);
}

hipError_t launch_attention_f16(const TrimulArgs &a, hipStream_t s)
{
    return sm::launch_attention_impl<KF16>(a, s);
}

hipError_t launch_attention_online_f16(const TrimulArgs &a, hipStream_t s)
{
    return sm::launch_attention_online_impl<KF16>(a, s);
}

} // namespace cas
