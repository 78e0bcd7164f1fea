// mamba2.hip -- Mamba-2 replay step kernels with an fp32 checkpoint.
#include "mamba2_kernel.hpp"

namespace rs {

hipError_t launch_mamba2_step_f32(const StepArgs& a, int io, int rc, bool valu_fold, hipStream_t s)
{
    return mamba2_launch<CK_F32>(a, io, rc, valu_fold, s);
}

}  // namespace rs
