// mamba2_fp8.hip -- Mamba-2 replay step kernels with an FP8 (E4M3) checkpoint.
#include "mamba2_kernel.hpp"

namespace rs {

hipError_t launch_mamba2_step_fp8(const StepArgs& a, int io, int rc, hipStream_t s)
{
    return mamba2_launch<CK_FP8>(a, io, rc, false, s);
}

}  // namespace rs
