// The only sequential part of the PRISM recurrence (summary §2.1, S_t =
// S_{t-1} A_t + B_t): chunk after chunk, S_{c+1} = exp(gC_c) S_c - S_c M_c + H_c,
// followed by the chunk-parallel readout O = O_loc + Qt S_c^T (the readout
// o_t = S_t q_t, reading R7).  The same kernel runs the adjoint pass of the
// backward in reverse chunk order: dS_c = exp(gC_c) dS_{c+1} - dS_{c+1} M_c^T + E_c.
//
// Rows of S (the value index) never mix, so the pass is split over 16-row
// tiles: one wave per (b, h, row tile) carries its 16 x D slice of the state
// in fp32 registers for the whole sequence; the product with M runs on MFMA
// with the state cast to the operand type and the matrix read straight from
// global memory (L2-resident: the D/16 row tiles of one sequence are
// scheduled on the same XCD).
#include "prism_common.h"
#include "prism_internal.h"

namespace prism {

// Forward (reverse = 0): X_0 = init (S0, or 0), per chunk c = 0..NC-1 store
//   X_c, then X <- exp(gC_c) X - X Bm_c^T + AddT_c^T, where Bm_c = M_c^T
//   (so X Bm_c^T = X M_c) and AddT_c = H_c^T.  Final X -> fin (S_T).
// Reverse (reverse = 1): X = init (dS_T, or 0), c = NC-1..0, Bm_c = M_c
//   (X Bm_c^T = X M_c^T), AddT_c = E_c^T; final X -> fin (dS_0).
// The stored per-chunk matrix is row-major, or transposed when `transposed`.
template <typename E, int D>
__global__ __launch_bounds__(64) void state_pass_kernel(const float* __restrict__ init,
                                                        const E* __restrict__ Bm,
                                                        const float* __restrict__ AddT,
                                                        const float* __restrict__ gC,
                                                        E* __restrict__ Xc, float* __restrict__ fin,
                                                        int B, int H, int NC, int transposed,
                                                        int reverse) {
  constexpr int NTL = D / 16;
  constexpr int LS = ldpad<E>(D);
  constexpr int VN = 16 / sizeof(E);
  __shared__ __attribute__((aligned(16))) E Ss[16 * LS];
  const int lane = threadIdx.x;
  const int nblk = B * H * NTL;
  const int bid = xcd_swizzle(blockIdx.x, nblk);
  const int rt = bid % NTL, bh = bid / NTL;
  const int r0 = 16 * rt;
  const int rl = 4 * (lane >> 4);    // first of this lane's 4 rows within the tile
  const int cl = lane & 15;

  Acc<16, D, 1> S;
  S.zero();
  if (init) {
#pragma unroll
    for (int j = 0; j < NTL; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) S.v[0][j][i] = init[((long)bh * D + r0 + rl + i) * D + 16 * j + cl];
  }
  for (int step = 0; step < NC; ++step) {
    const int c = reverse ? NC - 1 - step : step;
    const long cidx = (long)bh * NC + c;
#pragma unroll
    for (int j = 0; j < NTL; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) Ss[(rl + i) * LS + 16 * j + cl] = to_t<E>(S.v[0][j][i]);
    __syncthreads();
    E* Xcc = Xc + cidx * D * D;
    if (!transposed) {
      for (int e = lane; e < 16 * (D / VN); e += 64) {
        const int r = e / (D / VN), cc = (e % (D / VN)) * VN;
        st16(Xcc + (long)(r0 + r) * D + cc, ld16(Ss + r * LS + cc));
      }
    } else {
      for (int kk = lane; kk < D; kk += 64) {
#pragma unroll
        for (int p = 0; p < 16 / VN; ++p) {
          E tmp[VN];
#pragma unroll
          for (int r = 0; r < VN; ++r) tmp[r] = Ss[(p * VN + r) * LS + kk];
          uint4 pk;
          __builtin_memcpy(&pk, tmp, 16);
          st16(Xcc + (long)kk * D + r0 + p * VN, pk);
        }
      }
    }
    Acc<16, D, 1> P;
    P.zero();
    gemm_acc<E, 16, D, D, 1, true, true>(P, Ss, LS, Bm + cidx * D * D, D, 0, lane);
    const float eg = expf(gC[cidx]);
    const float* Ac = AddT + cidx * D * D;
#pragma unroll
    for (int j = 0; j < NTL; ++j) {
      const f32x4 av = *reinterpret_cast<const f32x4*>(Ac + (long)(16 * j + cl) * D + r0 + rl);
      S.v[0][j] = eg * S.v[0][j] - P.v[0][j] + av;
    }
    __syncthreads();
  }
  if (fin) {
#pragma unroll
    for (int j = 0; j < NTL; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) fin[((long)bh * D + r0 + rl + i) * D + 16 * j + cl] = S.v[0][j][i];
  }
}

template <typename E, int D>
static hipError_t state_launch_d(const Dims& d, const float* init, const E* Bm, const float* AddT,
                                 const float* gC, E* Xc, float* fin, bool tr, bool rev,
                                 hipStream_t s) {
  const int nblk = d.B * d.H * (D / 16);
  hipLaunchKernelGGL((state_pass_kernel<E, D>), dim3(nblk), dim3(64), 0, s, init, Bm, AddT, gC, Xc,
                     fin, d.B, d.H, d.NC, tr ? 1 : 0, rev ? 1 : 0);
  return hipGetLastError();
}

template <typename E>
hipError_t launch_state_pass(const Dims& d, const float* init, const E* Bm, const float* AddT,
                             const float* gC, E* Xc, float* fin, bool transposed, bool reverse,
                             hipStream_t s) {
  switch (d.D) {
    case 16: return state_launch_d<E, 16>(d, init, Bm, AddT, gC, Xc, fin, transposed, reverse, s);
    case 32: return state_launch_d<E, 32>(d, init, Bm, AddT, gC, Xc, fin, transposed, reverse, s);
    case 64: return state_launch_d<E, 64>(d, init, Bm, AddT, gC, Xc, fin, transposed, reverse, s);
    case 128:
      if constexpr (sizeof(E) == 2)
        return state_launch_d<E, 128>(d, init, Bm, AddT, gC, Xc, fin, transposed, reverse, s);
      break;
  }
  return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// readout: O[t][f] = O_loc[t][f] + sum_k Qt[t][k] S_c[f][k]
// ---------------------------------------------------------------------------
constexpr int OF_NW = 4;
constexpr int OF_NT = OF_NW * WAVE;

template <typename E, int D, int C>
__global__ __launch_bounds__(OF_NT) void out_fwd_kernel(const E* __restrict__ Sc,
                                                        const E* __restrict__ Qt,
                                                        const float* __restrict__ Oloc,
                                                        E* __restrict__ o, int B, int T, int H,
                                                        int NC) {
  constexpr int LR = ldpad<E>(D);
  __shared__ __attribute__((aligned(16))) E Ss[D * LR];
  __shared__ __attribute__((aligned(16))) E Qs[C * LR];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nblk = B * H * NC;
  const int bid = xcd_swizzle(blockIdx.x, nblk);
  const int c = bid % NC, bh = bid / NC;
  const int h = bh % H, b = bh / H;
  const long cidx = (long)bh * NC + c;
  g2s_rows<E, D, D, OF_NT>(Ss, LR, Sc + cidx * D * D, D, D, tid);
  g2s_rows<E, C, D, OF_NT>(Qs, LR, Qt + cidx * C * D, D, C, tid);
  __syncthreads();
  Acc<D, C, OF_NW> a;   // [f][t] = S[f] . Qt[t]
  a.zero();
  gemm_acc<E, D, C, D, OF_NW, true, true>(a, Ss, LR, Qs, LR, wave, lane);
  const float* Oc = Oloc + cidx * C * D;
  const int nval = min(C, T - c * C);
  E* oc = o + (((long)b * T + c * C) * H + h) * D;
  for_tiles(a, wave, lane, [&](int f0, int t, const f32x4& x) {
    if (t < nval) {
      const f32x4 ol = *reinterpret_cast<const f32x4*>(Oc + (long)t * D + f0);
#pragma unroll
      for (int r = 0; r < 4; ++r) oc[(long)t * H * D + f0 + r] = to_t<E>(ol[r] + x[r]);
    }
  });
}

template <typename E, int D, int C>
static hipError_t out_launch_dc(const Dims& d, const E* Sc, const E* Qt, const float* Oloc, E* o,
                                hipStream_t s) {
  if constexpr (sizeof(E) == 4 && D * C > 2048) return hipErrorInvalidValue;   // fp32 envelope
  hipLaunchKernelGGL((out_fwd_kernel<E, D, C>), dim3(d.B * d.H * d.NC), dim3(OF_NT), 0, s, Sc, Qt,
                     Oloc, o, d.B, d.T, d.H, d.NC);
  return hipGetLastError();
}

template <typename E, int D>
static hipError_t out_launch_d(const Dims& d, const E* Sc, const E* Qt, const float* Oloc, E* o,
                               hipStream_t s) {
  switch (d.C) {
    case 16: return out_launch_dc<E, D, 16>(d, Sc, Qt, Oloc, o, s);
    case 32: return out_launch_dc<E, D, 32>(d, Sc, Qt, Oloc, o, s);
    case 64: return out_launch_dc<E, D, 64>(d, Sc, Qt, Oloc, o, s);
  }
  return hipErrorInvalidValue;
}

template <typename E>
hipError_t launch_out_fwd(const Dims& d, const E* Sc, const E* Qt, const float* Oloc, E* o,
                          hipStream_t s) {
  switch (d.D) {
    case 16: return out_launch_d<E, 16>(d, Sc, Qt, Oloc, o, s);
    case 32: return out_launch_d<E, 32>(d, Sc, Qt, Oloc, o, s);
    case 64: return out_launch_d<E, 64>(d, Sc, Qt, Oloc, o, s);
    case 128:
      if constexpr (sizeof(E) == 2) return out_launch_d<E, 128>(d, Sc, Qt, Oloc, o, s);
      break;
  }
  return hipErrorInvalidValue;
}

template hipError_t launch_state_pass<bf16>(const Dims&, const float*, const bf16*, const float*,
                                            const float*, bf16*, float*, bool, bool, hipStream_t);
template hipError_t launch_state_pass<float>(const Dims&, const float*, const float*, const float*,
                                             const float*, float*, float*, bool, bool, hipStream_t);
template hipError_t launch_out_fwd<bf16>(const Dims&, const bf16*, const bf16*, const float*,
                                         bf16*, hipStream_t);
template hipError_t launch_out_fwd<float>(const Dims&, const float*, const float*, const float*,
                                          float*, hipStream_t);

}  // namespace prism
