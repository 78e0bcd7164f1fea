// gdn.hip -- Gated DeltaNet replay step kernels with an fp32 checkpoint.
#include "gdn_kernel.hpp"

namespace rs {

hipError_t launch_gdn_step_f32(const StepArgs& a, int io, int rc, hipStream_t s)
{
    return gdn_launch<CK_F32>(a, io, rc, s);
}

}  // namespace rs
