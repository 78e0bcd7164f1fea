// gdn.hip -- replayed Gated DeltaNet decode step for gfx950 (CDNA4).
#include "common.hpp"
#include "internal.hpp"

namespace rs {

hipError_t launch_gdn_step(const StepArgs& a, int io, int rc, hipStream_t s)
{
    (void)a; (void)io; (void)rc; (void)s;
    return hipErrorNotSupported;
}

}  // namespace rs
