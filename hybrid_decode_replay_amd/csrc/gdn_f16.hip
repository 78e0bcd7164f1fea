// gdn_f16.hip -- Gated DeltaNet replay step kernels with an fp16 checkpoint.
#include "gdn_kernel.hpp"

namespace rs {

hipError_t launch_gdn_step_f16(const StepArgs& a, int io, int rc, hipStream_t s)
{
    return gdn_launch<CK_F16>(a, io, rc, s);
}

}  // namespace rs
