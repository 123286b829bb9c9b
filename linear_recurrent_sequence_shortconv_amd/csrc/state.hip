// The only sequential part of the PRISM recurrence (summary §2.1, S_t =
// S_{t-1} A_t + B_t): chunk after chunk, S_{c+1} = exp(gC_c) S_c - S_c M_c + H_c,
// and in the same step the chunk's readout O = O_loc + Qt S_c^T (the readout
// o_t = S_t q_t with the post-update state).  The same kernel runs the adjoint pass of the
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

// Both directions take Mt_c = M_c^T (in HBM in the MFMA fragment order of a
// k-contiguous B operand for bf16 at D >= 32, else row-major; row-major in LDS):
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
// same XCD) while the current step multiplies.  In the forward direction
// with Bm_c in fragment order no LDS copy of it is made: each wave loads the
// B fragments of its output columns (contiguous 1 KB pieces) into registers,
// two steps ahead, right after the step that used the previous set.
// With RO (forward only) each step also forms its row block of the chunk's
// readout, O[t][f] = O_loc[t][f] + sum_k Qt[t][k] S_c[f][k], from the operand
// copy of S_c already in LDS: the chunk's Qt rows and O_loc block are fetched
// two steps ahead with the other operands, and S_c goes to HBM only when a
// caller keeps it (Xc non-null).  The readout reads no S_c from HBM and needs
// no launch of its own.
// With FE (reverse only) each step forms its row block of the additive term
// E_c = dO_c^T Qt_c itself, from the dO rows of the block and the Qt rows a
// training forward kept (fetched two steps ahead, staged in LDS), and adds it
// to the adjoint state in fp32: no E_c round trip through HBM.
constexpr int SP_NW = 8;
constexpr int SP_NT = SP_NW * WAVE;
constexpr long SP_WIDE = 256;   // workgroups that fill the chip (one per CU)

template <typename E, int D, int RB, bool REV, int C_X>
__global__ __launch_bounds__(SP_NT) void state_pass_kernel(const float* __restrict__ init,
                                                           const E* __restrict__ Bm,
                                                           const E* __restrict__ AddT,
                                                           const float* __restrict__ gC,
                                                           E* __restrict__ Xc, float* __restrict__ fin,
                                                           int B, int H, int NC, int transposed,
                                                           int reverse, int T, int C,
                                                           const int* __restrict__ cu,
                                                           const E* __restrict__ Qt,
                                                           const E* __restrict__ Oloc,
                                                           E* __restrict__ o,
                                                           const E* __restrict__ dOg) {
  // C_X > 0: chunks of C_X tokens, with the readout fused (forward, RO) or the
  // additive term E_c formed in the pass (reverse, FE)
  constexpr bool RO = !REV && C_X > 0;
  constexpr bool FE = REV && C_X > 0;
  constexpr int CR = C_X > 0 ? C_X : 16;
  // Bm_c in fragment order (bf16, D >= 32): the forward reads each wave's B
  // fragments of the product straight into registers, and Bm needs no LDS
  // copy; the reverse pass reads Bm transposed and stages it in LDS
  constexpr bool MFO = mt_frag_order<E, D>();
  constexpr bool FO = MFO && !REV;
  typedef MfmaK<E, D> MK;
  constexpr int NKS = D / MK::KSTEP;
  // (with Bm in LDS the smallest padding: the 64-row blocks fill the LDS with
  // it already)
  constexpr int LS = FO ? ldpad<E>(D) : ldpad_min<E>(D);
  constexpr int VN = 16 / sizeof(E);
  constexpr int NV = D * D / VN;                       // 16-byte vectors of Bm_c
  constexpr int PER = (NV + SP_NT - 1) / SP_NT;
  constexpr int NVR = RB * D / VN;                     // 16-byte vectors of the row block
  constexpr int NRB = D / RB;
  typedef Tiling<RB, D, SP_NW> TL;
  __shared__ __attribute__((aligned(16))) E Mb[FO ? 1 : 2][FO ? 8 : D * LS];
  __shared__ __attribute__((aligned(16))) E Ss[2][RB * LS];
  __shared__ __attribute__((aligned(16))) E Qb[C_X > 0 ? 2 : 1][C_X > 0 ? CR * LS : 8];   // Qt rows of a step
  constexpr int LO = ldpad_min<E>(RB);
  __shared__ __attribute__((aligned(16))) E Ob[FE ? 2 : 1][FE ? CR * LO : 8];   // dO rows of the block
  constexpr int NVQ = CR * D / VN;                     // 16-byte vectors of Qt_c
  constexpr int PERQ = (NVQ + SP_NT - 1) / SP_NT;
  typedef Tiling<RB, CR, SP_NW> TLO;                   // readout tiles [f][t]
  constexpr int NVO = CR * RB / VN;                    // 16-byte vectors of the dO block
  constexpr int PERO = (NVO + SP_NT - 1) / SP_NT;
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
  // the initial state is complete before the loop: otherwise the compiler
  // keeps its loads pending at the loop head and waits there, every step,
  // for all memory operations in flight (the prefetches too)
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
  (void)reverse;   // the direction is the template parameter REV
  // chunks of this sequence (all NC in a dense batch; a packed sequence stops
  // at its own end, and the chunks after it are never read)
  // (the sequence's bounds are read once: a scalar load inside the loop
  // would hold up the LDS waits that follow it)
  const int slen = seq_len(cu, bh / H, T);
  const long sbeg = seq_start(cu, bh / H, T);
  const int ncb = (slen + C - 1) / C;
  auto chunk_of = [&](int step) { return REV ? ncb - 1 - step : step; };
  // The operands of step s + 2 are requested during step s (two register
  // sets, indexed by the step's parity at compile time), each as soon as
  // step s has used the set's previous contents: a step then stages into LDS
  // only data that has had a whole step to arrive.
  uint4 mst[2][FO ? 1 : PER];           // Bm of a coming step, staged through registers
  typename MK::frag bfr[2][FO ? TL::RN : 1][FO ? NKS : 1];   // or its B fragments (FO)
  uint4 qst[2][C_X > 0 ? PERQ : 1];     // Qt rows of a coming step (readout, E_c)
  uint4 dost[2][FE ? PERO : 1];         // dO block of a coming step (E_c)
  int nvn[2] = {0, 0};                  // its valid rows (E_c)
  typename Raw4Of<E>::type oln[2][RO ? TLO::RM : 1][RO ? TLO::RN : 1];   // its O_loc block (raw)
  typename Raw4Of<E>::type addn[2][TL::RM][TL::RN];   // AddT^T block of a coming step (raw)
  float egn[2] = {0.f, 0.f};            // log decay gC of a coming step
  auto fetch = [&](int step, auto setc) {
    constexpr int Z = decltype(setc)::value;
    const long cidx = (long)bh * NC + chunk_of(step);
    if constexpr (!FO) {
      const E* bm = Bm + cidx * D * D;
#pragma unroll
      for (int p = 0; p < PER; ++p) {
        const int e = tid + p * SP_NT;
        if (e < NV) mst[Z][p] = ld16(bm + (long)e * VN);
      }
    }
    // a vector load (its offset made opaque to the compiler): a scalar load
    // shares its wait counter with the LDS operations and may return out of
    // order, so every LDS wait after it would wait for it as well
    int zoff;
    asm volatile("v_mov_b32 %0, 0" : "=v"(zoff));
    egn[Z] = gC[cidx + zoff];
    if constexpr (C_X > 0) {
      const E* qc = Qt + cidx * CR * D;
#pragma unroll
      for (int p = 0; p < PERQ; ++p) {
        const int e = tid + p * SP_NT;
        if (e < NVQ) qst[Z][p] = ld16(qc + (long)e * VN);
      }
    }
    if constexpr (FE) {
      // rows past the sequence end read the last valid row and are zeroed
      // when staged (no load depends on a branch)
      const int h = bh % H;
      const int c0 = chunk_of(step) * CR;
      const int nval = min(CR, slen - c0);
      nvn[Z] = nval;
      const E* dc = dOg + ((sbeg + c0) * H + h) * D + rb0;
#pragma unroll
      for (int p = 0; p < PERO; ++p) {
        const int e = tid + p * SP_NT;
        if (e < NVO) {
          const int t = min(e / (RB / VN), nval - 1), c = (e % (RB / VN)) * VN;
          dost[Z][p] = ld16(dc + (long)t * H * D + c);
        }
      }
    }
  };
  // the AddT^T block of a coming step, requested once the state update has
  // used the set's previous block (a register set still in use when its
  // refill is issued costs a copy, and a wait, at the loop's end)
  auto fetch_add = [&](int step, auto setc) {
    constexpr int Z = decltype(setc)::value;
    if (act && !FE) {
      const E* ac = AddT + ((long)bh * NC + chunk_of(step)) * D * D + rb0;
#pragma unroll
      for (int i = 0; i < TL::RM; ++i)
#pragma unroll
        for (int j = 0; j < TL::RN; ++j)
          addn[Z][i][j] = ld_raw4(ac + (long)(n0 + 16 * j + cl) * D + m0 + 16 * i + rl);
    }
  };
  // the O_loc block of a coming step (RO), requested once the readout has
  // used the set's previous block
  auto fetch_ol = [&](int step, auto setc) {
    constexpr int Z = decltype(setc)::value;
    if constexpr (RO) {
      if (TLO::active(wave)) {
        const E* oc = Oloc + ((long)bh * NC + chunk_of(step)) * CR * D + rb0;
#pragma unroll
        for (int i = 0; i < TLO::RM; ++i)
#pragma unroll
          for (int j = 0; j < TLO::RN; ++j) {
            const int f0 = TLO::m0(wave) + 16 * i + 4 * (lane >> 4), t = TLO::n0(wave) + 16 * j + (lane & 15);
            oln[Z][i][j] = ld_raw4(oc + (long)t * D + f0);
          }
      }
    }
  };
  // FO: this wave's B fragments of Bm_c (output columns n0 .. n0 + 16 RN - 1)
  auto fetch_m = [&](int step, auto setc) {
    constexpr int Z = decltype(setc)::value;
    if constexpr (FO) {
      if (act) {
        const E* bm = Bm + ((long)bh * NC + chunk_of(step)) * D * D;
#pragma unroll
        for (int j = 0; j < TL::RN; ++j)
#pragma unroll
          for (int kk = 0; kk < NKS; ++kk) bfr[Z][j][kk] = load_frag_fo<E, D>(bm, (n0 >> 4) + j, kk, lane);
      }
    }
  };
  auto stage = [&](E* dst, auto setc) {
    constexpr int Z = decltype(setc)::value;
    if constexpr (!FO) {
#pragma unroll
      for (int p = 0; p < PER; ++p) {
        const int e = tid + p * SP_NT;
        if (e < NV) {
          int r, c;
          if constexpr (MFO) {
            fo_piece_rc<D>(e, r, c);
          } else {
            r = e / (D / VN);
            c = (e % (D / VN)) * VN;
          }
          st16(dst + r * LS + c, mst[Z][p]);
        }
      }
    }
    if constexpr (C_X > 0) {
#pragma unroll
      for (int p = 0; p < PERQ; ++p) {
        const int e = tid + p * SP_NT;
        if (e < NVQ) {
          const int r = e / (D / VN), c = (e % (D / VN)) * VN;
          st16(Qb[Z] + r * LS + c, qst[Z][p]);
        }
      }
    }
    if constexpr (FE) {
#pragma unroll
      for (int p = 0; p < PERO; ++p) {
        const int e = tid + p * SP_NT;
        if (e < NVO) {
          const int r = e / (RB / VN), c = (e % (RB / VN)) * VN;
          uint4 w = dost[Z][p];
          asm volatile("" : "+v"(w.x), "+v"(w.y), "+v"(w.z), "+v"(w.w));
          if (r >= nvn[Z]) w = uint4{0u, 0u, 0u, 0u};
          st16(Ob[Z] + r * LO + c, w);
        }
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
    if constexpr (!FE) {
#pragma unroll
      for (int i = 0; i < TL::RM; ++i)
#pragma unroll
        for (int j = 0; j < TL::RN; ++j) addc[i][j] = raw4_to_f(addn[Z][i][j]);
    }
    // (computed here, before the refill of set Z below, which it then
    // cannot share registers with)
    float egc = expf(egn[Z]);
    asm volatile("" : "+v"(egc));
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
    // (unconditional, the last chunk again past the end: a load under a
    // condition leaves a merge of old and new registers that the compiler
    // resolves with copies, which wait for the load at the loop's end)
    fetch(min(step + 2, ncb - 1), setc);
    if (!Xc) {
      // the chunk-entry states are not kept (readout fused, inference)
    } else if (!transposed) {
      E* Xcc = Xc + cidx * D * D;
      for (int e = tid; e < NVR; e += SP_NT) {
        const int r = e / (D / VN), c = (e % (D / VN)) * VN;
        st16(Xcc + (long)(rb0 + r) * D + c, ld16(Ss[Z] + r * LS + c));
      }
    } else {
      E* Xcc = Xc + cidx * D * D;
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
    if constexpr (FO) {
      if (act) {
#pragma unroll
        for (int kk = 0; kk < NKS; ++kk) {
          typename MK::frag a[TL::RM];
#pragma unroll
          for (int i = 0; i < TL::RM; ++i) a[i] = load_fragK<E, D>(Ss[Z], LS, m0 + 16 * i, kk * MK::KSTEP, lane);
#pragma unroll
          for (int i = 0; i < TL::RM; ++i)
#pragma unroll
            for (int j = 0; j < TL::RN; ++j) P.v[i][j] = MK::mma(a[i], bfr[Z][j][kk], P.v[i][j]);
        }
      }
      // set Z's fragments are consumed: refill it with step + 2's
      fetch_m(min(step + 2, ncb - 1), setc);
    } else {
      gemm_acc<E, RB, D, D, SP_NW, true, !REV>(P, Ss[Z], LS, Mb[Z], LS, wave, lane);
    }
    if constexpr (FE) {
      // E_c rows of the block: [r][n] = sum_t dO[t][rb0 + r] Qt[t][n] (both
      // operands k-strided in LDS), added in fp32
      Acc<RB, D, SP_NW> Ea;
      Ea.zero();
      gemm_acc<E, RB, D, CR, SP_NW, false, false>(Ea, Ob[Z], LO, Qb[Z], LS, wave, lane);
      if (act) {
#pragma unroll
        for (int i = 0; i < TL::RM; ++i)
#pragma unroll
          for (int j = 0; j < TL::RN; ++j) addc[i][j] = Ea.v[i][j];
      }
    }
    if (act) {
#pragma unroll
      for (int i = 0; i < TL::RM; ++i)
#pragma unroll
        for (int j = 0; j < TL::RN; ++j) S.v[i][j] = egc * S.v[i][j] - P.v[i][j] + addc[i][j];
    }
    // the update is done (and the AddT block it read is dead) before the
    // refill below is issued: the compiler may not move either across this
#pragma unroll
    for (int i = 0; i < TL::RM; ++i)
#pragma unroll
      for (int j = 0; j < TL::RN; ++j) asm volatile("" : "+v"(S.v[i][j])::"memory");
    fetch_add(min(step + 2, ncb - 1), setc);
    if constexpr (RO) {
      // readout rows f = rb0 .. rb0 + RB - 1 of chunk cidx: [f][t] = S_c[f] . Qt[t]
      Acc<RB, CR, SP_NW> R;
      R.zero();
      gemm_acc<E, RB, CR, D, SP_NW, true, true>(R, Ss[Z], LS, Qb[Z], LS, wave, lane);
      const int h = bh % H;
      const int c0 = chunk_of(step) * CR;
      const int nval = min(CR, slen - c0);
      E* oc = o + ((sbeg + c0) * H + h) * D + rb0;
      for_tiles_ij(R, wave, lane, [&](int i, int j, int f0, int t, const f32x4& x) {
        if (t < nval) {
          const f32x4 lo = raw4_to_f(oln[Z][i][j]);
#pragma unroll
          for (int r = 0; r < 4; ++r) oc[(long)t * H * D + f0 + r] = to_t<E>(lo[r] + x[r]);
        }
      });
      fetch_ol(min(step + 2, ncb - 1), setc);
    }
    if (step + 1 < ncb) stage(Mb[FO ? 0 : Z ^ 1], std::integral_constant<int, Z ^ 1>{});
  };
  if (ncb > 0) {
    fetch(0, Z0{});
    fetch_m(0, Z0{});
    fetch_add(0, Z0{});
    fetch_ol(0, Z0{});
    stage(Mb[0], Z0{});
    fetch(min(1, ncb - 1), Z1{});
    fetch_m(min(1, ncb - 1), Z1{});
    fetch_add(min(1, ncb - 1), Z1{});
    fetch_ol(min(1, ncb - 1), Z1{});
  }
  // two steps per iteration (register sets 0 and 1), no condition inside
  int step = 0;
  for (; step + 1 < ncb; step += 2) {
    body(step, Z0{});
    body(step + 1, Z1{});
  }
  if (step < ncb) body(step, Z0{});
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
                                 const E* Qt, const E* Oloc, E* o, const E* dO, hipStream_t s) {
  // Row blocks: the whole state below D = 128; at D = 128 blocks of 64 rows
  // (two workgroups per sequence), or of 32 or 16 rows when there are too few
  // sequence-heads to give every CU a workgroup (long sequences, small
  // batches: the pass is sequential over chunks, so its width is all the
  // parallelism it has).
  auto go = [&](auto rbc) {
    constexpr int RB = decltype(rbc)::value;
    const dim3 grid(d.B * d.H * (D / RB));
    if (rev && !dO) {
      hipLaunchKernelGGL((state_pass_kernel<E, D, RB, true, 0>), grid, dim3(SP_NT), 0, s, init, Bm,
                         AddT, gC, Xc, fin, d.B, d.H, d.NC, tr ? 1 : 0, 1, d.T, d.C, d.cu, nullptr,
                         nullptr, nullptr, nullptr);
    } else if (!rev && !o) {
      hipLaunchKernelGGL((state_pass_kernel<E, D, RB, false, 0>), grid, dim3(SP_NT), 0, s, init, Bm,
                         AddT, gC, Xc, fin, d.B, d.H, d.NC, tr ? 1 : 0, 0, d.T, d.C, d.cu, nullptr,
                         nullptr, nullptr, nullptr);
    } else {
      // forward with the readout, or reverse with E_c formed in the pass
      auto ro = [&](auto cc) -> hipError_t {
        constexpr int CC = decltype(cc)::value;
        if constexpr (sizeof(E) == 4 && D * CC > 2048) {
          return hipErrorInvalidValue;   // outside the fp32 envelope
        } else {
          if (rev)
            hipLaunchKernelGGL((state_pass_kernel<E, D, RB, true, CC>), grid, dim3(SP_NT), 0, s,
                               init, Bm, AddT, gC, Xc, fin, d.B, d.H, d.NC, tr ? 1 : 0, 1, d.T, d.C,
                               d.cu, Qt, nullptr, nullptr, dO);
          else
            hipLaunchKernelGGL((state_pass_kernel<E, D, RB, false, CC>), grid, dim3(SP_NT), 0, s,
                               init, Bm, AddT, gC, Xc, fin, d.B, d.H, d.NC, tr ? 1 : 0, 0, d.T, d.C,
                               d.cu, Qt, Oloc, o, nullptr);
          return hipSuccess;
        }
      };
      hipError_t e = hipErrorInvalidValue;
      switch (d.C) {
        case 16: e = ro(std::integral_constant<int, 16>{}); break;
        case 32: e = ro(std::integral_constant<int, 32>{}); break;
        case 64: e = ro(std::integral_constant<int, 64>{}); break;
      }
      if (e != hipSuccess) return e;
    }
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
                             const E* Qt, const E* Oloc, E* o, const E* dO,
                             hipStream_t s) {
  switch (d.D) {
    case 16: return state_launch_d<E, 16>(d, init, Bm, AddT, gC, Xc, fin, transposed, reverse, Qt, Oloc, o, dO, s);
    case 32: return state_launch_d<E, 32>(d, init, Bm, AddT, gC, Xc, fin, transposed, reverse, Qt, Oloc, o, dO, s);
    case 64: return state_launch_d<E, 64>(d, init, Bm, AddT, gC, Xc, fin, transposed, reverse, Qt, Oloc, o, dO, s);
    case 128:
      if constexpr (sizeof(E) == 2)
        return state_launch_d<E, 128>(d, init, Bm, AddT, gC, Xc, fin, transposed, reverse, Qt, Oloc,
                                      o, dO, s);
      break;
  }
  return hipErrorInvalidValue;
}

template hipError_t launch_state_pass<bf16>(const Dims&, const float*, const bf16*, const bf16*,
                                            const float*, bf16*, float*, bool, bool, const bf16*,
                                            const bf16*, bf16*, const bf16*, hipStream_t);
template hipError_t launch_state_pass<float>(const Dims&, const float*, const float*, const float*,
                                             const float*, float*, float*, bool, bool, const float*,
                                             const float*, float*, const float*, hipStream_t);
}  // namespace prism
