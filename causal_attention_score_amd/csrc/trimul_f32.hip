// trimul_f32.hip -- f32 inputs of the causal score kernel (its own
// translation unit so the variants compile in parallel).
#include "trimul_kernel.hpp"

namespace cas {

hipError_t launch_trimul_f32(const TrimulArgs &a, int vec, hipStream_t s)
{
    return tri::launch_elem_impl<KF32>(a, vec, s);
}

} // namespace cas
