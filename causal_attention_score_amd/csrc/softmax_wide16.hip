// softmax_wide16.hip -- the row statistics and the attention output (two-pass
// and single pass) for 16-bit heads of 257 .. 512 bytes (HS 129 .. 256), 32
// pieces per row. Their own translation unit, built without the VGPR-only MFMA
// form of the other softmax units: a lane holds 8 x 16 fp32 output
// accumulators, which then go to the accumulation registers.
#include "softmax_kernel.hpp"

namespace cas {

hipError_t launch_row_stats_wide16(const TrimulArgs &a, int elem, hipStream_t s)
{
    return elem == E_BF16 ? sm::launch_row_stats_wide16_impl<KBF16>(a, s) : sm::launch_row_stats_wide16_impl<KF16>(a, s);
}

hipError_t launch_attention_wide16(const TrimulArgs &a, int elem, hipStream_t s)
{
    return elem == E_BF16 ? sm::launch_attention_wide16_impl<KBF16>(a, s) : sm::launch_attention_wide16_impl<KF16>(a, s);
}

hipError_t launch_attention_online_wide16(const TrimulArgs &a, int elem, hipStream_t s)
{
    return elem == E_BF16 ? sm::launch_attention_online_wide16_impl<KBF16>(a, s)
                          : sm::launch_attention_online_wide16_impl<KF16>(a, s);
}

} // namespace cas
