// Refinement / ShortConv backward instantiated for GELU steps, ShortConv taps on the current token.
#include "refine_bwd_kernel.h"

namespace prism {
template hipError_t launch_refine_bwd_main<bf16, ACT_GELU, 0>(const Dims&, const RefineBwdArgs<bf16>&,
                                                         hipStream_t);
template hipError_t launch_refine_bwd_main<float, ACT_GELU, 0>(const Dims&, const RefineBwdArgs<float>&,
                                                          hipStream_t);
}  // namespace prism
