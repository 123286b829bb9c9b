#pragma once
// Chunk-parallel part of the PRISM backward pass: the adjoint of the chunk
// affine map (see chunk_fwd.hip).  Shared helpers and the launch interface of
// the three kernels, each compiled on its own (chunk_bwd_{state,solve,pairs}.hip)
//
//     S_next = exp(gC) S - S M + H,    O = O_loc + Qt S^T,
//     M = Wk^T D K,  H = U^T D K + sum_l W_l^T D K_l,  Qt = e Q - R0 Wk,
//     O_loc = R0 U + sum_l R_l W_l,  U = T diag(beta) V',  Wk = T diag(beta e) K,
//     T = (I + A)^{-1},  A = diag(beta) (Gam * K K^T)_{i<t},
//     V' = V - sum_l F_l W_l,  F_l = (Gam * K K_l^T)_{i<t},  R_* = (Gam * Q K_*^T)_{i<=t},
//
// given the state S entering each chunk (stored transposed), the adjoint dS_n
// of the state leaving it (stored transposed) and dO.  Three kernels, all
// parallel over B * H * NC chunks:
//
//   chunk_bwd_state : terms through S, dS_n and dM = -S^T dS_n
//                     (dQt = dO S; D-weighted parts of dU, dWk, dK, dK_l, dW_l;
//                     the D and gC parts of dg)
//   chunk_bwd_solve : R0 terms, then the triangular solve backward
//                     (dT, dA = -T^T dT T^T, dK from the Gram matrix), dV', dbeta
//   chunk_bwd_pairs : the refinement-pair terms (R_l, F_l), final dq, dk, dK_l,
//                     dW_l, dv and dalpha (reverse cumulative sum of dg).
//
// All products are MFMA (bf16 or fp32 operands, fp32 accumulation).  The
// partials handed from one kernel to the next are stored in the element type
// E (dU, dWk, dK transposed, [D][C] per chunk), except dW_l, which stays fp32
// (the refinement backward subtracts from it).  Row and column sums needed for
// the decay gradient are reduced per wave in fixed order (no atomics), so
// results are bitwise reproducible.
#include "prism_common.h"
#include "prism_internal.h"

#include <type_traits>

namespace prism {

constexpr int CB_NW = 8;
constexpr int CB_NT = CB_NW * WAVE;

// ---------------------------------------------------------------------------
// shared helpers
// ---------------------------------------------------------------------------
// Decays of one chunk: g (cumulative log alpha), e = exp(g), Dv = exp(gC - g),
// bt = beta, be = beta e.  Padding tokens (t >= nval) have alpha = 1, beta = 0.
// chunk_decays_of takes alpha and beta already read (1 and 0 past nval).
template <int C>
__device__ __attribute__((always_inline)) inline void chunk_decays_of(float a, float bv, float* g, float* ev, float* Dv,
                                       float* bt, float* be, float* ai, int lane) {
  float s = logf(a);
  s = wave_scan(s);
  const float gC = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, s), C - 1));
  if (lane < C) {
    const float e = expf(s);
    g[lane] = s;
    ev[lane] = e;
    Dv[lane] = expf(gC - s);
    if (bt) bt[lane] = bv;
    if (be) be[lane] = bv * e;
    if (ai) ai[lane] = a;
  }
}

template <int C>
__device__ __attribute__((always_inline)) inline void chunk_decays(const float* alpha, const float* beta, long row0, int H,
                                    int nval, float* g, float* ev, float* Dv, float* bt, float* be,
                                    float* ai, int lane) {
  float lg = 0.f, bv = 0.f, a = 1.f;
  if (lane < nval) {
    a = alpha[row0 + (long)lane * H];
    lg = logf(a);
    if (beta) bv = beta[row0 + (long)lane * H];
  }
  float s = lg;
  s = wave_scan(s);
  const float gC = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, s), C - 1));
  if (lane < C) {
    const float e = expf(s);
    g[lane] = s;
    ev[lane] = e;
    Dv[lane] = expf(gC - s);
    if (bt) bt[lane] = bv;
    if (be) be[lane] = bv * e;
    if (ai) ai[lane] = a;
  }
}

// Row and column sums of products over all of a wave's accumulator tiles,
// kept in registers and reduced across lanes once (flush_*), instead of per
// tile: r[i][q] is row m0 + 16 i + 4 (lane >> 4) + q summed over this lane's
// columns, c[j] is column n0 + 16 j + (lane & 15) summed over this lane's rows.
template <int RM, int RN>
struct TileSums {
  float r[RM][4];
  float c[RN];
  __device__ inline void zero() {
#pragma unroll
    for (int i = 0; i < RM; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) r[i][q] = 0.f;
#pragma unroll
    for (int j = 0; j < RN; ++j) c[j] = 0.f;
  }
  __device__ inline void add(int i, int j, const f32x4& v, bool rows = true, bool cols = true) {
    if (rows) {
#pragma unroll
      for (int q = 0; q < 4; ++q) r[i][q] += v[q];
    }
    if (cols) c[j] += v[0] + v[1] + v[2] + v[3];
  }
  // slot[row] = row sums (one wave's private slots, each written by one
  // flush only): a row of 16 lanes summed by DPP row shifts, not by LDS
  // shuffles, and stored, not added (no read-modify-write of LDS)
  __device__ inline void flush_rows(float* slot, int m0, int lane) const {
#pragma unroll
    for (int i = 0; i < RM; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float s = row16_sum(r[i][q]);
        if ((lane & 15) == 15) slot[m0 + 16 * i + 4 * (lane >> 4) + q] = s;
      }
  }
  // slot[col] = column sums (as above)
  __device__ inline void flush_cols(float* slot, int n0, int lane) const {
#pragma unroll
    for (int j = 0; j < RN; ++j) {
      float s = c[j];
      s += __shfl_xor(s, 16);
      s += __shfl_xor(s, 32);
      if (lane < 16) slot[n0 + 16 * j + lane] = s;
    }
  }
};

// Decays Gam_ti = exp(g_t - g_i) for i <= t (else 0) at this wave's positions
// of a C x C product held as rows t, column i (Tiling<C, C, NW>): formed once
// per chunk for the products that share those positions.
template <int C, int NW, int RM, int RN>
__device__ inline void decays_ti(f32x4 (&gm)[RM][RN], const float* g, int wave, int lane) {
  typedef Tiling<C, C, NW> TL;
  static_assert(RM == TL::RM && RN == TL::RN, "tiles of a C x C product");
  if (!TL::active(wave)) return;
#pragma unroll
  for (int i = 0; i < TL::RM; ++i)
#pragma unroll
    for (int j = 0; j < TL::RN; ++j) {
      const int t0 = TL::m0(wave) + 16 * i + 4 * (lane >> 4), ii = TL::n0(wave) + 16 * j + (lane & 15);
#pragma unroll
      for (int r = 0; r < 4; ++r) gm[i][j][r] = ii <= t0 + r ? __expf(g[t0 + r] - g[ii]) : 0.f;
    }
}

// ---------------------------------------------------------------------------
// launch interface: one entry per kernel; F::run<E, D, C> launches the kernel
// for one (d, chunk) instance
// ---------------------------------------------------------------------------
template <typename E, typename F>
hipError_t cbwd_dispatch(const Dims& d, const ChunkBwdArgs<E>& a, hipStream_t s) {
  auto by_c = [&](auto dtag) -> hipError_t {
    constexpr int D = decltype(dtag)::value;
    switch (d.C) {
      case 16: return F::template run<E, D, 16>(d, a, s);
      case 32: return F::template run<E, D, 32>(d, a, s);
      case 64: return F::template run<E, D, 64>(d, a, s);
    }
    return hipErrorInvalidValue;
  };
  switch (d.D) {
    case 16: return by_c(std::integral_constant<int, 16>());
    case 32: return by_c(std::integral_constant<int, 32>());
    case 64: return by_c(std::integral_constant<int, 64>());
    case 128:
      if constexpr (sizeof(E) == 2) return by_c(std::integral_constant<int, 128>());
      break;
  }
  return hipErrorInvalidValue;
}

template <typename E>
hipError_t launch_chunk_bwd_state(const Dims& d, const ChunkBwdArgs<E>& a, hipStream_t s);
template <typename E>
hipError_t launch_chunk_bwd_solve(const Dims& d, const ChunkBwdArgs<E>& a, hipStream_t s);
template <typename E>
hipError_t launch_chunk_bwd_pairs(const Dims& d, const ChunkBwdArgs<E>& a, hipStream_t s);

}  // namespace prism
