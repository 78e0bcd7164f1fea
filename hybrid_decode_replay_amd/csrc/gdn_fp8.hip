// gdn_fp8.hip -- Gated DeltaNet replay step kernels with an FP8 (E4M3) checkpoint.
#include "gdn_kernel.hpp"

namespace rs {

hipError_t launch_gdn_step_fp8(const StepArgs& a, int io, int rc, hipStream_t s)
{
    return gdn_launch<CK_FP8>(a, io, rc, s);
}

}  // namespace rs
