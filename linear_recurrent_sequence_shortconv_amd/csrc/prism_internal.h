// Host-side declarations shared by the PRISM C-ABI layer and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace prism {

typedef __bf16 bf16;

// Refinement step activation: delta = GELU(p * r) or delta = p * r.
constexpr int ACT_GELU = 0, ACT_IDENTITY = 1;

// Problem dimensions after validation.  D = d_k = d_v; C = chunk length;
// NC = ceil(T / C) chunks per sequence; Tp = NC * C padded length;
// act = step activation; off = ShortConv tap offset (0: tap j reads v_{t-j},
// 1: tap j reads v_{t-1-j}).
struct Dims {
  int B, T, H, D, L, C, NC, Tp;
  int act, off;
  // packed batch: sequence b is tokens cu[b] .. cu[b+1]-1 of the [N, H, D]
  // token tensors (device array of B + 1 offsets, at most T tokens each);
  // nullptr: dense [B, T, H, D].  The kernels read the sanitised copy (every
  // offset in [0, N], non-decreasing), never the caller's array.
  const int* cu = nullptr;
  int N = 0;
};

// Sanitised copy of the packed-batch offsets: out[i] = max_{j <= i}
// clamp(d.cu[j], 0, d.N), i = 0..B.  Every sequence then lies inside the N
// rows of the packed tensors and no two overlap, whatever the caller passed.
hipError_t launch_cu_sanitize(const Dims& d, int* out, hipStream_t s);

// Every launcher enqueues on `stream` and returns hipGetLastError().
// Element type E is __bf16 or float.

// Weight matrices [H, L, D, D] in MFMA fragment order (frag_order_offset in
// prism_common.h): each non-null output receives W_p, W_k, W_p^T or W_k^T.
template <typename E>
hipError_t launch_weight_frags(const Dims& d, const E* Wk, const E* Wp, E* WpF, E* WkF, E* WpTF,
                               E* WkTF, hipStream_t s);

// Stage 1 + Stage 2: ShortConv anchor and the L refinement steps.
// Writes Kl, Wl [B, H, L, Tp, D] (rows t >= T are zero).  hist [B, 4, H, D]
// holds the four v values before the sequence (nullptr: zeros).
template <typename E>
hipError_t launch_refine_fwd(const Dims& d, const E* v, const E* hist, const E* conv, const E* Wk,
                             const E* Wp, const E* wbeta, E* Kl, E* Wl, hipStream_t s);

// Chunk-local affine map of every chunk (parallel over B * H * NC).
// Forward mode writes Mt, HT, Qt, Oloc, gC, and UT, WkT when they are not
// null (training forward).  Backward mode (dO != nullptr) writes Mt, HT, gC,
// ET (E = dO^T Qt), UT, WkT and nothing else.
template <typename E>
hipError_t launch_chunk_fwd(const Dims& d, const E* q, const E* k, const E* v, const float* alpha,
                            const float* beta, const E* Kl, const E* Wl, const E* dO, E* Mt,
                            E* HT, E* Qt, E* Oloc, float* gC, E* ET, E* UT, E* WkT,
                            hipStream_t s);

// Inputs of the refinement when the chunk kernel forms the pairs itself.
template <typename E>
struct FuseIn {
  const E* hist = nullptr;    // [B, 4, H, D] v rows before each sequence (nullptr: zeros)
  const E* conv = nullptr;    // [H, D, 4]
  const E* Wk = nullptr;      // [H, L, D, D]
  const E* Wp = nullptr;      // [H, L, D, D]
  const E* wbeta = nullptr;   // [H, L, D]
};

// Forward mode of launch_chunk_fwd with the refinement pairs formed inside
// the kernel from v (1 <= L <= 8): writes Mt, HT, Qt, Oloc, gC.  Same results
// as launch_refine_fwd followed by launch_chunk_fwd.
template <typename E>
hipError_t launch_chunk_fwd_fused(const Dims& d, const E* q, const E* k, const E* v,
                                  const float* alpha, const float* beta, const FuseIn<E>& fz,
                                  E* Mt, E* HT, E* Qt, E* Oloc, float* gC,
                                  hipStream_t s);


// Sequential pass over chunks, forward (X <- exp(gC) X - X M + H, from S0) or
// reverse (X <- exp(gC) X - X M^T + E, from dS_T).  Both read Mt = M^T; AddT
// is H^T or E^T.  Stores X per chunk before its update (row-major, or
// transposed), and the final X in `fin` when not null.
template <typename E>
hipError_t launch_state_pass(const Dims& d, const float* init, const E* Mt, const E* AddT,
                             const float* gC, E* Xc, float* fin, bool transposed, bool reverse,
                             const E* Qt, const E* Oloc, E* o, const E* dO, hipStream_t s);

// Arguments of the three chunk-parallel backward kernels (see chunk_bwd_common.h).
template <typename E>
struct ChunkBwdArgs {
  const E *q, *k, *v, *dO;
  const float *alpha, *beta;
  const E *Kl, *Wl, *UT, *WkT;
  const E* Sc;                  // chunk-entry states S_c, row-major [D][D]
  const E* dSnT;
  float *dgs, *dgp, *dbeta;
  E *dQt, *dUs, *dWks, *dKs;    // state-gradient partials (storage type)
  E *dVp, *dqp, *dkp;           // solve partials (storage type)
  // gradients of the refinement pairs: dK_l in the storage type (its users
  // round it to the MFMA operand type anyway); dW_l in fp32, since it enters
  // the difference beta^(l) dW_l - dL/dr^(l+1), which can cancel
  E* dKl;
  float* dWl;
  E *dq, *dk;
  E* dv;                        // written here only when L = 0
  float* dalpha;
};
template <typename E>
// stage 0: chunk_bwd_state, 1: chunk_bwd_solve, 2: chunk_bwd_pairs (in this order)
hipError_t launch_chunk_bwd(const Dims& d, const ChunkBwdArgs<E>& a, int stage, hipStream_t s);

// Arguments of the refinement / ShortConv backward and the weight gradients.
template <typename E>
struct RefineBwdArgs {
  const E *v, *conv, *Wk, *Wp, *wbeta;
  const E* hist;                // v before the sequence [B, 4, H, D] (nullptr: zeros)
  float* dhist;                 // its gradient (nullptr: not wanted)
  // W_p, W_p^T and W_k^T in MFMA fragment order (workspace; frag_order_offset)
  E *WpF, *WpT, *WkT;
  const E* dKl;                 // gradient of the directions k^(l) (storage type)
  const float* dWl;             // gradient of the values w^(l) (fp32)
  const E* dvdir;               // direct v-gradient of the recurrence ([bh][Tp][D])
  E* u;                         // ShortConv output rows (for the weight GEMM)
  E* dP;                        // dp rows (for the weight GEMM)
  float *dwbp, *dcp, *part;     // per-tile / per-split partial sums
  E* dv;
  float *dWk_o, *dWp_o, *dwbeta_o, *dconv_o;
};
template <typename E>
// stage 0: weights in fragment order, 1: refinement + ShortConv backward (dv, per-tile
// dw_beta and tap partials), 2: weight-gradient GEMM, 3: its reduction,
// 4: reduction of the dw_beta and tap partials
hipError_t launch_refine_bwd(const Dims& d, const RefineBwdArgs<E>& a, int stage, hipStream_t s);
int refine_bwd_splits(const Dims& d);   // split count of the weight-gradient GEMM
int refine_bwd_tiles(const Dims& d);    // token tiles per sequence (rows of the per-tile partials)

// The ShortConv history after the sequence, out[b][r] = v_{T-4+r} (from
// hist, or zero, where T-4+r < 0).  out may be hist itself.
template <typename E>
hipError_t launch_conv_state(const Dims& d, const E* v, const E* hist, E* out, hipStream_t s);

// Bytes of the fixed device array behind prism_step_noalloc (the refinement
// pairs of the recurrent step), and its device address on the device of
// `stream` (looked up once per device; see noalloc.hip).
constexpr size_t NOALLOC_SCRATCH_BYTES = size_t(16) << 20;
hipError_t noalloc_scratch(hipStream_t stream, void** ptr);

// Zero n floats (a kernel, so that the call may be captured in a graph).
hipError_t launch_zero(float* p, long n, hipStream_t s);

// Token-by-token recurrence for T tokens per sequence: S [B, H, D, D] fp32
// and the ShortConv history cstate [B, 4, H, D] (nullptr: zeros, not kept)
// are read, carried and written back in place; o [B, T, H, D].  Kl, Wl:
// room for the refinement pairs, [B, H, L, T, D] each.  stage 0 writes the
// pairs (refinement kernel, nothing when L = 0), stage 1 runs the state.
template <typename E>
hipError_t launch_step(const Dims& d, const E* q, const E* k, const E* v, const float* alpha,
                       const float* beta, const E* Wk, const E* Wp, const E* wbeta, const E* conv,
                       float* S, E* cstate, E* o, E* Kl, E* Wl, int stage, hipStream_t s);


}  // namespace prism
