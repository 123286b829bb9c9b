// Chunk backward: entry point over its three kernels (chunk_bwd_state.hip,
// chunk_bwd_solve.hip, chunk_bwd_pairs.hip; the adjoint they compute is
// described in chunk_bwd_common.h).
#include "chunk_bwd_common.h"

namespace prism {

template <typename E>
hipError_t launch_chunk_bwd(const Dims& d, const ChunkBwdArgs<E>& a, int stage, hipStream_t s) {
  if (stage == 0) return launch_chunk_bwd_state<E>(d, a, s);
  if (stage == 1) return launch_chunk_bwd_solve<E>(d, a, s);
  return launch_chunk_bwd_pairs<E>(d, a, s);
}

template hipError_t launch_chunk_bwd<bf16>(const Dims&, const ChunkBwdArgs<bf16>&, int, hipStream_t);
template hipError_t launch_chunk_bwd<float>(const Dims&, const ChunkBwdArgs<float>&, int, hipStream_t);

}  // namespace prism
