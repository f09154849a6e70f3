// trimul_f16.hip -- f16 inputs of the causal score kernel (its own
// translation unit so the variants compile in parallel).
#include "trimul_kernel.hpp"

namespace cas {

hipError_t launch_trimul_f16(const TrimulArgs &a, int vec, hipStream_t s)
{
    return tri::launch_elem_impl<KF16>(a, vec, s);
}

} // namespace cas
