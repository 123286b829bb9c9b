// Launchers of the chunk-local kernel (chunk_fwd_kernel.h) in its two forms
// (refinement pairs read from HBM, or formed in the kernel), and the ET kernel
// that the backward of a training forward runs on the kept Qt.
// Multiply-adds fuse only within one expression (the C rule), never across
// statements: the refinement kernel and the chunk kernel that repeats its
// arithmetic then round identically, whatever code surrounds each.
#pragma clang fp contract(on)
#include "chunk_fwd_kernel.h"

namespace prism {

// ET[n][r] = sum_t Qt[t][n] dO[t][r] per chunk (fp32 [D][D]), from the Qt a
// training forward kept: the reverse state pass's additive term.
template <typename E, int D, int C>
__global__ __launch_bounds__(CF_NT) void et_kernel(const E* __restrict__ Qt, const E* __restrict__ dO,
                                                   E* __restrict__ ET, int B, int T, int H, int NC,
                                                   const int* __restrict__ cu) {
  constexpr int NW = CF_NW, NT = CF_NT;
  constexpr int LR = ldpad<E>(D);
  __shared__ __attribute__((aligned(16))) E Qs[C * LR];
  __shared__ __attribute__((aligned(16))) E Os[C * LR];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nblk = B * H * NC;
  const int bid = xcd_swizzle(blockIdx.x, nblk);
  const int c = bid % NC, bh = bid / NC;
  const int h = bh % H, b = bh / H;
  const int tb = c * C;
  const int nval = min(C, seq_len(cu, b, T) - tb);
  const long ts = (long)H * D;
  const long row0 = (seq_start(cu, b, T) + tb) * H + h;
  if (nval <= 0) return;   // past the end of a packed sequence
  const long cidx = (long)bh * NC + c;
  g2s_rows<E, C, D, NT>(Qs, LR, Qt + cidx * C * D, D, C, tid);
  g2s_rows<E, C, D, NT>(Os, LR, dO + row0 * D, ts, nval, tid);
  __syncthreads();
  Acc<D, D, NW> ea;   // [n][r] = sum_t Qt[t][n] dO[t][r]: both operands k-strided in LDS
  ea.zero();
  gemm_acc<E, D, D, C, NW, false, false>(ea, Qs, LR, Os, LR, wave, lane);
  E* ETc = ET + cidx * D * D;
  for_tiles(ea, wave, lane, [&](int n0, int r, const f32x4& x) {
#pragma unroll
    for (int i = 0; i < 4; ++i) ETc[(long)(n0 + i) * D + r] = to_t<E>(x[i]);
  });
}

template <typename E, int D, int C>
static hipError_t et_launch_dc(const Dims& d, const E* Qt, const E* dO, E* ET, hipStream_t s) {
  if constexpr (sizeof(E) == 4 && D * C > 2048) return hipErrorInvalidValue;   // fp32 envelope
  hipLaunchKernelGGL((et_kernel<E, D, C>), dim3(d.B * d.H * d.NC), dim3(CF_NT), 0, s, Qt, dO, ET,
                     d.B, d.T, d.H, d.NC, d.cu);
  return hipGetLastError();
}

template <typename E, int D>
static hipError_t et_launch_d(const Dims& d, const E* Qt, const E* dO, E* ET, hipStream_t s) {
  switch (d.C) {
    case 16: return et_launch_dc<E, D, 16>(d, Qt, dO, ET, s);
    case 32: return et_launch_dc<E, D, 32>(d, Qt, dO, ET, s);
    case 64: return et_launch_dc<E, D, 64>(d, Qt, dO, ET, s);
  }
  return hipErrorInvalidValue;
}

template <typename E>
hipError_t launch_et(const Dims& d, const E* Qt, const E* dO, E* ET, hipStream_t s) {
  switch (d.D) {
    case 16: return et_launch_d<E, 16>(d, Qt, dO, ET, s);
    case 32: return et_launch_d<E, 32>(d, Qt, dO, ET, s);
    case 64: return et_launch_d<E, 64>(d, Qt, dO, ET, s);
    case 128:
      if constexpr (sizeof(E) == 2) return et_launch_d<E, 128>(d, Qt, dO, ET, s);
      break;
  }
  return hipErrorInvalidValue;
}
template hipError_t launch_et<bf16>(const Dims&, const bf16*, const bf16*, bf16*, hipStream_t);
template hipError_t launch_et<float>(const Dims&, const float*, const float*, float*, hipStream_t);

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
