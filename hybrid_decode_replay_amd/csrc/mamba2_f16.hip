// mamba2_f16.hip -- Mamba-2 replay step kernels with an fp16 checkpoint.
#include "mamba2_kernel.hpp"

namespace rs {

hipError_t launch_mamba2_step_f16(const StepArgs& a, int io, int rc, hipStream_t s)
{
    return mamba2_launch<CK_F16>(a, io, rc, false, s);
}

}  // namespace rs
