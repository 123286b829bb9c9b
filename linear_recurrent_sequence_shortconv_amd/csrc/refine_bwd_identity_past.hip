// Refinement / ShortConv backward instantiated for identity steps, strictly past ShortConv taps.
#include "refine_bwd_kernel.h"

namespace prism {
template hipError_t launch_refine_bwd_main<bf16, ACT_IDENTITY, 1>(const Dims&, const RefineBwdArgs<bf16>&,
                                                         hipStream_t);
template hipError_t launch_refine_bwd_main<float, ACT_IDENTITY, 1>(const Dims&, const RefineBwdArgs<float>&,
                                                          hipStream_t);
}  // namespace prism
