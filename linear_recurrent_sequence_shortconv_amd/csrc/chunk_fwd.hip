// Launchers of the chunk-local kernel (chunk_fwd_kernel.h) in its two forms
// (refinement pairs read from HBM, or formed in the kernel).
// Multiply-adds fuse only within one expression (the C rule), never across
// statements: the refinement kernel and the chunk kernel that repeats its
// arithmetic then round identically, whatever code surrounds each.
#pragma clang fp contract(on)
#include "chunk_fwd_kernel.h"

namespace prism {


template <typename E, int D, int C>
static hipError_t chunk_launch_dc(const Dims& d, const E* q, const E* k, const E* v,
                                  const float* alpha, const float* beta, const E* Kl, const E* Wl,
                                  const E* dO, E* Mt, E* HT, E* Qt, E* Oloc, float* gC,
                                  E* ET, E* UT, E* WkT, hipStream_t s) {
  const FuseIn<E> none{};
  if (dO)
    return chunk_launch_k<E, D, C, true, false, 0, 0>(d, q, k, v, alpha, beta, Kl, Wl, dO, Mt, HT,
                                                      Qt, Oloc, gC, ET, UT, WkT, none, s);
  return chunk_launch_k<E, D, C, false, false, 0, 0>(d, q, k, v, alpha, beta, Kl, Wl, dO, Mt, HT,
                                                     Qt, Oloc, gC, ET, UT, WkT, none, s);
}

template <typename E, int D>
static hipError_t chunk_launch_d(const Dims& d, const E* q, const E* k, const E* v,
                                 const float* alpha, const float* beta, const E* Kl, const E* Wl,
                                 const E* dO, E* Mt, E* HT, E* Qt, E* Oloc, float* gC,
                                 E* ET, E* UT, E* WkT, hipStream_t s) {
  switch (d.C) {
    case 16: return chunk_launch_dc<E, D, 16>(d, q, k, v, alpha, beta, Kl, Wl, dO, Mt, HT, Qt, Oloc, gC, ET, UT, WkT, s);
    case 32: return chunk_launch_dc<E, D, 32>(d, q, k, v, alpha, beta, Kl, Wl, dO, Mt, HT, Qt, Oloc, gC, ET, UT, WkT, s);
    case 64: return chunk_launch_dc<E, D, 64>(d, q, k, v, alpha, beta, Kl, Wl, dO, Mt, HT, Qt, Oloc, gC, ET, UT, WkT, s);
  }
  return hipErrorInvalidValue;
}

template <typename E>
hipError_t launch_chunk_fwd(const Dims& d, const E* q, const E* k, const E* v, const float* alpha,
                            const float* beta, const E* Kl, const E* Wl, const E* dO, E* Mt,
                            E* HT, E* Qt, E* Oloc, float* gC, E* ET, E* UT,
                            E* WkT, hipStream_t s) {
  switch (d.D) {
    case 16: return chunk_launch_d<E, 16>(d, q, k, v, alpha, beta, Kl, Wl, dO, Mt, HT, Qt, Oloc, gC, ET, UT, WkT, s);
    case 32: return chunk_launch_d<E, 32>(d, q, k, v, alpha, beta, Kl, Wl, dO, Mt, HT, Qt, Oloc, gC, ET, UT, WkT, s);
    case 64: return chunk_launch_d<E, 64>(d, q, k, v, alpha, beta, Kl, Wl, dO, Mt, HT, Qt, Oloc, gC, ET, UT, WkT, s);
    case 128:
      if constexpr (sizeof(E) == 2)
        return chunk_launch_d<E, 128>(d, q, k, v, alpha, beta, Kl, Wl, dO, Mt, HT, Qt, Oloc, gC, ET, UT, WkT, s);
      break;
  }
  return hipErrorInvalidValue;
}

template hipError_t launch_chunk_fwd<bf16>(const Dims&, const bf16*, const bf16*, const bf16*,
                                           const float*, const float*, const bf16*, const bf16*,
                                           const bf16*, bf16*, bf16*, bf16*, bf16*, float*,
                                           bf16*, bf16*, bf16*, hipStream_t);
template hipError_t launch_chunk_fwd<float>(const Dims&, const float*, const float*, const float*,
                                            const float*, const float*, const float*, const float*,
                                            const float*, float*, float*, float*, float*, float*,
                                            float*, float*, float*, hipStream_t);

template <typename E>
hipError_t launch_chunk_fwd_fused(const Dims& d, const E* q, const E* k, const E* v,
                                  const float* alpha, const float* beta, const FuseIn<E>& fz,
                                  E* Mt, E* HT, E* Qt, E* Oloc, float* gC,
                                  hipStream_t s) {
  if (d.L <= 0 || d.L > FUSE_LMAX) return hipErrorInvalidValue;
  if (d.act == ACT_IDENTITY)
    return d.off ? launch_chunk_fused_var<E, ACT_IDENTITY, 1>(d, q, k, v, alpha, beta, fz, Mt, HT, Qt, Oloc, gC, s)
                 : launch_chunk_fused_var<E, ACT_IDENTITY, 0>(d, q, k, v, alpha, beta, fz, Mt, HT, Qt, Oloc, gC, s);
  return d.off ? launch_chunk_fused_var<E, ACT_GELU, 1>(d, q, k, v, alpha, beta, fz, Mt, HT, Qt, Oloc, gC, s)
               : launch_chunk_fused_var<E, ACT_GELU, 0>(d, q, k, v, alpha, beta, fz, Mt, HT, Qt, Oloc, gC, s);
}
template hipError_t launch_chunk_fwd_fused<bf16>(const Dims&, const bf16*, const bf16*, const bf16*,
                                                 const float*, const float*, const FuseIn<bf16>&,
                                                 bf16*, bf16*, bf16*, bf16*, float*, hipStream_t);
template hipError_t launch_chunk_fwd_fused<float>(const Dims&, const float*, const float*,
                                                  const float*, const float*, const float*,
                                                  const FuseIn<float>&, float*, float*, float*,
                                                  float*, float*, hipStream_t);

}  // namespace prism
