// Chunk-local kernel with the refinement formed inside it, instantiated for
// GELU steps (both ShortConv tap offsets).
// Multiply-adds fuse only within one expression (the C rule), never across
// statements: the refinement kernel and the chunk kernel that repeats its
// arithmetic then round identically, whatever code surrounds each.
#pragma clang fp contract(on)
#include "chunk_fwd_kernel.h"

namespace prism {
#define INST(E, OFF)                                                                          \
  template hipError_t launch_chunk_fused_var<E, ACT_GELU, OFF>(                                 \
      const Dims&, const E*, const E*, const E*, const float*, const float*, const FuseIn<E>&, \
      E*, E*, E*, E*, float*, hipStream_t);
INST(bf16, 0)
INST(bf16, 1)
INST(float, 0)
INST(float, 1)
#undef INST
}  // namespace prism
