// Host-side declarations shared by the PRISM C-ABI layer and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace prism {

typedef __bf16 bf16;

// Problem dimensions after validation.  D = d_k = d_v; C = chunk length;
// NC = ceil(T / C) chunks per sequence; Tp = NC * C padded length.
struct Dims {
  int B, T, H, D, L, C, NC, Tp;
};

// Every launcher enqueues on `stream` and returns hipGetLastError().
// Element type E is __bf16 or float.

// Stage 1 + Stage 2: ShortConv anchor and the L refinement steps.
// Writes Kl, Wl [B, H, L, Tp, D] (rows t >= T are zero).
template <typename E>
hipError_t launch_refine_fwd(const Dims& d, const E* v, const E* conv, const E* Wk, const E* Wp,
                             const E* wbeta, E* Kl, E* Wl, hipStream_t s);

// Chunk-local affine map of every chunk (parallel over B * H * NC).
// Forward mode writes Mt, HT, Qt, Oloc, gC.  Backward mode (dO != nullptr)
// writes Mt, HT, gC, M, ET (E = dO^T Qt) and nothing else.
template <typename E>
hipError_t launch_chunk_fwd(const Dims& d, const E* q, const E* k, const E* v, const float* alpha,
                            const float* beta, const E* Kl, const E* Wl, const E* dO, E* Mt,
                            float* HT, E* Qt, float* Oloc, float* gC, E* M, float* ET,
                            hipStream_t s);

// Sequential pass over chunks: S_{c+1} = exp(gC) S_c - S_c M_c + H_c.
// Stores S_c per chunk (row-major, or transposed when `transposed`).
template <typename E>
hipError_t launch_state_fwd(const Dims& d, const float* S0, const E* Mt, const float* HT,
                            const float* gC, E* Sc, float* ST, bool transposed, hipStream_t s);

// O = O_loc + Qt S_c^T, written to o [B, T, H, D].
template <typename E>
hipError_t launch_out_fwd(const Dims& d, const E* Sc, const E* Qt, const float* Oloc, E* o,
                          hipStream_t s);

}  // namespace prism
