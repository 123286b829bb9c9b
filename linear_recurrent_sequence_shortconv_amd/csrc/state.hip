// The only sequential part of the PRISM recurrence (summary §2.1, S_t =
// S_{t-1} A_t + B_t): chunk after chunk, S_{c+1} = exp(gC_c) S_c - S_c M_c + H_c,
// followed by the chunk-parallel readout O = O_loc + Qt S_c^T (the readout
// o_t = S_t q_t, reading R7).  The same kernel runs the adjoint pass of the
// backward in reverse chunk order: dS_c = exp(gC_c) dS_{c+1} - dS_{c+1} M_c^T + E_c.
//
// Rows of S (the value index) never mix, so the pass is split over row
// blocks, each carried in fp32 registers by one workgroup for the whole
// sequence; the product with M runs on MFMA with the state cast to the
// operand type.
#include <type_traits>

#include "prism_common.h"
#include "prism_internal.h"

namespace prism {

// Both directions take Mt_c = M_c^T (row-major in HBM and LDS):
// Forward (reverse = 0): X_0 = init (S0, or 0), per chunk c = 0..NC-1 store
//   X_c, then X <- exp(gC_c) X - X Mt_c^T + AddT_c^T (X Mt_c^T = X M_c), with
//   AddT_c = H_c^T.  Final X -> fin (S_T).
// Reverse (reverse = 1): X = init (dS_T, or 0), c = NC-1..0,
//   X <- exp(gC_c) X - X Mt_c + AddT_c^T (X Mt_c = X M_c^T; the MFMA B operand
//   is then read k-strided from LDS), with AddT_c = E_c^T; final X -> fin (dS_0).
// The stored per-chunk matrix is row-major, or transposed when `transposed`.
//
// Rows of the state never mix, so the pass splits into row blocks of RB rows:
// one workgroup of 8 waves per (b, h, row block) carries its RB x D slice of
// the state in fp32 registers (spread over the waves).  Each step needs one
// barrier: the chunk matrix Bm_c and the operand copy of the state live in
// double-buffered LDS tiles, and the next step's Bm, AddT block and decay are
// fetched from global memory (L2: the row blocks of one sequence sit on the
// same XCD) while the current step multiplies.
constexpr int SP_NW = 8;
constexpr int SP_NT = SP_NW * WAVE;
constexpr long SP_WIDE = 256;   // workgroups that fill the chip (one per CU)

template <typename E, int D, int RB, bool REV>
__global__ __launch_bounds__(SP_NT) void state_pass_kernel(const float* __restrict__ init,
                                                           const E* __restrict__ Bm,
                                                           const E* __restrict__ AddT,
                                                           const float* __restrict__ gC,
                                                           E* __restrict__ Xc, float* __restrict__ fin,
                                                           int B, int H, int NC, int transposed,
                                                           int reverse, int T, int C,
                                                           const int* __restrict__ cu) {
  constexpr int LS = ldpad<E>(D);
  constexpr int VN = 16 / sizeof(E);
  constexpr int NV = D * D / VN;                       // 16-byte vectors of Bm_c
  constexpr int PER = (NV + SP_NT - 1) / SP_NT;
  constexpr int NVR = RB * D / VN;                     // 16-byte vectors of the row block
  constexpr int NRB = D / RB;
  typedef Tiling<RB, D, SP_NW> TL;
  __shared__ __attribute__((aligned(16))) E Mb[2][D * LS];
  __shared__ __attribute__((aligned(16))) E Ss[2][RB * LS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nblk = B * H * NRB;
  const int bid = xcd_swizzle(blockIdx.x, nblk);
  const int bh = bid / NRB, rb0 = (bid % NRB) * RB;
  const bool act = TL::active(wave);
  const int m0 = TL::m0(wave), n0 = TL::n0(wave);
  const int rl = 4 * (lane >> 4), cl = lane & 15;

  Acc<RB, D, SP_NW> S;   // this wave's block of the state (rows relative to rb0)
  S.zero();
  if (init && act) {
#pragma unroll
    for (int i = 0; i < TL::RM; ++i)
#pragma unroll
      for (int j = 0; j < TL::RN; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          S.v[i][j][r] = init[((long)bh * D + rb0 + m0 + 16 * i + rl + r) * D + n0 + 16 * j + cl];
  }
  (void)reverse;   // the direction is the template parameter REV
  // chunks of this sequence (all NC in a dense batch; a packed sequence stops
  // at its own end, and the chunks after it are never read)
  const int ncb = (seq_len(cu, bh / H, T) + C - 1) / C;
  auto chunk_of = [&](int step) { return REV ? ncb - 1 - step : step; };
  // The operands of step s + 2 are requested at the start of step s (two
  // register sets, indexed by the step's parity at compile time): a step
  // then stages into LDS only data that has had a whole step to arrive.
  uint4 mst[2][PER];                    // Bm of a coming step, staged through registers
  typename Raw4Of<E>::type addn[2][TL::RM][TL::RN];   // AddT^T block of a coming step (raw)
  float egn[2] = {0.f, 0.f};            // decay of a coming step
  auto fetch = [&](int step, auto setc) {
    constexpr int Z = decltype(setc)::value;
    const long cidx = (long)bh * NC + chunk_of(step);
    const E* bm = Bm + cidx * D * D;
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int e = tid + p * SP_NT;
      if (e < NV) mst[Z][p] = ld16(bm + (long)e * VN);
    }
    if (act) {
      const E* ac = AddT + cidx * D * D + rb0;
#pragma unroll
      for (int i = 0; i < TL::RM; ++i)
#pragma unroll
        for (int j = 0; j < TL::RN; ++j)
          addn[Z][i][j] = ld_raw4(ac + (long)(n0 + 16 * j + cl) * D + m0 + 16 * i + rl);
    }
    egn[Z] = expf(gC[cidx]);
  };
  auto stage = [&](E* dst, auto setc) {
    constexpr int Z = decltype(setc)::value;
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int e = tid + p * SP_NT;
      if (e < NV) {
        const int r = e / (D / VN), c = (e % (D / VN)) * VN;
        st16(dst + r * LS + c, mst[Z][p]);
      }
    }
  };
  using Z0 = std::integral_constant<int, 0>;
  using Z1 = std::integral_constant<int, 1>;
  // one step; its operands are in set Z (Bm already staged in Mb[Z])
  auto body = [&](int step, auto setc) {
    constexpr int Z = decltype(setc)::value;
    const long cidx = (long)bh * NC + chunk_of(step);
    f32x4 addc[TL::RM][TL::RN];
#pragma unroll
    for (int i = 0; i < TL::RM; ++i)
#pragma unroll
      for (int j = 0; j < TL::RN; ++j) addc[i][j] = raw4_to_f(addn[Z][i][j]);
    const float egc = egn[Z];
    if (act) {   // state -> operand copy
#pragma unroll
      for (int i = 0; i < TL::RM; ++i)
#pragma unroll
        for (int j = 0; j < TL::RN; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            Ss[Z][(m0 + 16 * i + rl + r) * LS + n0 + 16 * j + cl] = to_t<E>(S.v[i][j][r]);
    }
    // Ss[Z] and Mb[Z] complete; every wave is past the previous step, so the
    // other buffers are free to refill
    __syncthreads();
    if (step + 2 < ncb) fetch(step + 2, setc);
    E* Xcc = Xc + cidx * D * D;
    if (!transposed) {
      for (int e = tid; e < NVR; e += SP_NT) {
        const int r = e / (D / VN), c = (e % (D / VN)) * VN;
        st16(Xcc + (long)(rb0 + r) * D + c, ld16(Ss[Z] + r * LS + c));
      }
    } else {
      for (int e = tid; e < NVR; e += SP_NT) {
        const int kk = e / (RB / VN), r0 = (e % (RB / VN)) * VN;
        E tmp[VN];
#pragma unroll
        for (int r = 0; r < VN; ++r) tmp[r] = Ss[Z][(r0 + r) * LS + kk];
        uint4 pk;
        __builtin_memcpy(&pk, tmp, 16);
        st16(Xcc + (long)kk * D + rb0 + r0, pk);
      }
    }
    Acc<RB, D, SP_NW> P;
    P.zero();
    gemm_acc<E, RB, D, D, SP_NW, true, !REV>(P, Ss[Z], LS, Mb[Z], LS, wave, lane);
    if (act) {
#pragma unroll
      for (int i = 0; i < TL::RM; ++i)
#pragma unroll
        for (int j = 0; j < TL::RN; ++j) S.v[i][j] = egc * S.v[i][j] - P.v[i][j] + addc[i][j];
    }
    if (step + 1 < ncb) stage(Mb[Z ^ 1], std::integral_constant<int, Z ^ 1>{});
  };
  if (ncb > 0) {
    fetch(0, Z0{});
    stage(Mb[0], Z0{});
    if (ncb > 1) fetch(1, Z1{});
  }
  for (int step = 0; step < ncb; step += 2) {
    body(step, Z0{});
    if (step + 1 < ncb) body(step + 1, Z1{});
  }
  if (fin && act) {
#pragma unroll
    for (int i = 0; i < TL::RM; ++i)
#pragma unroll
      for (int j = 0; j < TL::RN; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          fin[((long)bh * D + rb0 + m0 + 16 * i + rl + r) * D + n0 + 16 * j + cl] = S.v[i][j][r];
  }
}

template <typename E, int D>
static hipError_t state_launch_d(const Dims& d, const float* init, const E* Bm, const E* AddT,
                                 const float* gC, E* Xc, float* fin, bool tr, bool rev,
                                 hipStream_t s) {
  // Row blocks: the whole state below D = 128; at D = 128 blocks of 64 rows
  // (two workgroups per sequence), or of 32 or 16 rows when there are too few
  // sequence-heads to give every CU a workgroup (long sequences, small
  // batches: the pass is sequential over chunks, so its width is all the
  // parallelism it has).
  auto go = [&](auto rbc) {
    constexpr int RB = decltype(rbc)::value;
    if (rev)
      hipLaunchKernelGGL((state_pass_kernel<E, D, RB, true>), dim3(d.B * d.H * (D / RB)), dim3(SP_NT),
                         0, s, init, Bm, AddT, gC, Xc, fin, d.B, d.H, d.NC, tr ? 1 : 0, 1, d.T, d.C,
                         d.cu);
    else
      hipLaunchKernelGGL((state_pass_kernel<E, D, RB, false>), dim3(d.B * d.H * (D / RB)), dim3(SP_NT),
                         0, s, init, Bm, AddT, gC, Xc, fin, d.B, d.H, d.NC, tr ? 1 : 0, 0, d.T, d.C,
                         d.cu);
    return hipGetLastError();
  };
  if constexpr (D > 64) {
    const long nbh = (long)d.B * d.H;
    if (nbh * 2 >= SP_WIDE) return go(std::integral_constant<int, 64>{});
    if (nbh * 4 >= SP_WIDE) return go(std::integral_constant<int, 32>{});
    return go(std::integral_constant<int, 16>{});
  } else {
    return go(std::integral_constant<int, D>{});
  }
}

template <typename E>
hipError_t launch_state_pass(const Dims& d, const float* init, const E* Bm, const E* AddT,
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
                                                        const E* __restrict__ Oloc,
                                                        E* __restrict__ o, int B, int T, int H,
                                                        int NC, const int* __restrict__ cu) {
  constexpr int LR = ldpad<E>(D);
  __shared__ __attribute__((aligned(16))) E Ss[D * LR];
  __shared__ __attribute__((aligned(16))) E Qs[C * LR];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nblk = B * H * NC;
  const int bid = xcd_swizzle(blockIdx.x, nblk);
  const int c = bid % NC, bh = bid / NC;
  const int h = bh % H, b = bh / H;
  const int nval = min(C, seq_len(cu, b, T) - c * C);
  if (nval <= 0) return;   // past the end of a packed sequence: S_c was never written
  const long cidx = (long)bh * NC + c;
  g2s_rows<E, D, D, OF_NT>(Ss, LR, Sc + cidx * D * D, D, D, tid);
  g2s_rows<E, C, D, OF_NT>(Qs, LR, Qt + cidx * C * D, D, C, tid);
  // O_loc in the accumulator layout, requested before the product so that
  // its latency overlaps it: tile (i, j) holds features f0 .. f0 + 3 of token t
  typedef Tiling<D, C, OF_NW> TL;
  const E* Oc = Oloc + cidx * C * D;
  typename Raw4Of<E>::type ol[TL::RM][TL::RN];
  if (TL::active(wave)) {
#pragma unroll
    for (int i = 0; i < TL::RM; ++i)
#pragma unroll
      for (int j = 0; j < TL::RN; ++j) {
        const int f0 = TL::m0(wave) + 16 * i + 4 * (lane >> 4), t = TL::n0(wave) + 16 * j + (lane & 15);
        ol[i][j] = t < nval ? ld_raw4(Oc + (long)t * D + f0) : typename Raw4Of<E>::type{};
      }
  }
  __syncthreads();
  Acc<D, C, OF_NW> a;   // [f][t] = S[f] . Qt[t]
  a.zero();
  gemm_acc<E, D, C, D, OF_NW, true, true>(a, Ss, LR, Qs, LR, wave, lane);
  E* oc = o + ((seq_start(cu, b, T) + c * C) * H + h) * D;
  for_tiles_ij(a, wave, lane, [&](int i, int j, int f0, int t, const f32x4& x) {
    if (t < nval) {
      const f32x4 lo = raw4_to_f(ol[i][j]);
#pragma unroll
      for (int r = 0; r < 4; ++r) oc[(long)t * H * D + f0 + r] = to_t<E>(lo[r] + x[r]);
    }
  });
}

template <typename E, int D, int C>
static hipError_t out_launch_dc(const Dims& d, const E* Sc, const E* Qt, const E* Oloc, E* o,
                                hipStream_t s) {
  if constexpr (sizeof(E) == 4 && D * C > 2048) return hipErrorInvalidValue;   // fp32 envelope
  hipLaunchKernelGGL((out_fwd_kernel<E, D, C>), dim3(d.B * d.H * d.NC), dim3(OF_NT), 0, s, Sc, Qt,
                     Oloc, o, d.B, d.T, d.H, d.NC, d.cu);
  return hipGetLastError();
}

template <typename E, int D>
static hipError_t out_launch_d(const Dims& d, const E* Sc, const E* Qt, const E* Oloc, E* o,
                               hipStream_t s) {
  switch (d.C) {
    case 16: return out_launch_dc<E, D, 16>(d, Sc, Qt, Oloc, o, s);
    case 32: return out_launch_dc<E, D, 32>(d, Sc, Qt, Oloc, o, s);
    case 64: return out_launch_dc<E, D, 64>(d, Sc, Qt, Oloc, o, s);
  }
  return hipErrorInvalidValue;
}

template <typename E>
hipError_t launch_out_fwd(const Dims& d, const E* Sc, const E* Qt, const E* Oloc, E* o,
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

template hipError_t launch_state_pass<bf16>(const Dims&, const float*, const bf16*, const bf16*,
                                            const float*, bf16*, float*, bool, bool, hipStream_t);
template hipError_t launch_state_pass<float>(const Dims&, const float*, const float*, const float*,
                                             const float*, float*, float*, bool, bool, hipStream_t);
template hipError_t launch_out_fwd<bf16>(const Dims&, const bf16*, const bf16*, const bf16*,
                                         bf16*, hipStream_t);
template hipError_t launch_out_fwd<float>(const Dims&, const float*, const float*, const float*,
                                          float*, hipStream_t);

}  // namespace prism
