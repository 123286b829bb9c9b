// Chunk backward, second kernel: the R0 terms and the triangular solve backward.
#include "chunk_bwd_common.h"

namespace prism {

// ===========================================================================
// chunk_bwd_solve
// ===========================================================================
template <typename E, int D, int C>
struct CB2Lds {
  static constexpr int LR = ldpad<E>(D);
  static constexpr int LT = ldpad<E>(C);
  static constexpr int LA = C + 1;
  static constexpr int SZ_R = C * LR * (int)sizeof(E);
  static constexpr int SZ_CC = C * LT * (int)sizeof(E);
  static constexpr int SZ_F = C * LA * 4;
  // vectors: g, e, Dv, bt, be, de (6C) + slots rs, cs, bs, es, bs2 [NW][C]
  static constexpr int SZ_VEC = (6 * C + 5 * CB_NW * C) * 4;
  static constexpr int O_K = (SZ_VEC + 15) / 16 * 16;
  static constexpr int O_TB = O_K + SZ_R;
  static constexpr int O_X = O_TB + SZ_CC;
  // phase "fold": V rows (-> V' rows, live until U is formed), K_l, W_l, F
  static constexpr int F_V = O_X;
  static constexpr int F_KL = F_V + SZ_R;
  static constexpr int F_WL = F_KL + SZ_R;
  static constexpr int F_F = F_WL + SZ_R;
  static constexpr int F_END = F_F + SZ_CC;
  // phase "solve" (after V' rows): A, T fp32, scratch, T diag(beta), T diag(beta e)
  static constexpr int S_AF = F_V + SZ_R;
  static constexpr int S_TF = S_AF + SZ_F;
  static constexpr int S_XS = S_TF + SZ_F;
  static constexpr int S_TBB = S_XS + inv_scratch_floats(C) * 4;
  static constexpr int S_TBE = S_TBB + SZ_CC;
  static constexpr int S_END = S_TBE + SZ_CC;
  // phase "R0" (written after the U / Wk products have read everything above):
  // U, Wk rows (then dU, dWk rows), Q, dO, -dQt rows, R0, X0
  static constexpr int P_U = O_X;
  static constexpr int P_WK = P_U + SZ_R;
  static constexpr int P_Q = P_WK + SZ_R;
  static constexpr int P_DO = P_Q + SZ_R;
  static constexpr int P_NDQ = P_DO + SZ_R;
  static constexpr int P_R0 = P_NDQ + SZ_R;   // later dT
  static constexpr int P_XB = P_R0 + SZ_CC;   // later P1 = dT T^T (live while dG0 is formed)
  static constexpr int P_END = P_XB + SZ_CC;
  // phase "tail": dG0 fp32 and (dG0 + dG0^T) from the U slot on; they must
  // stay clear of the P1 slot, which other waves read while dG0 is written
  static constexpr int Z_F = P_U;
  static constexpr int Z_B = Z_F + SZ_F;
  static_assert(Z_F + SZ_F <= P_XB, "dG0 must not overlap P1");
  static constexpr int TOTAL = cmax(P_END, cmax(Z_B + SZ_CC, cmax(S_END, F_END)));
};

template <typename E, int D, int C>
__global__ __launch_bounds__(CB_NT) void chunk_bwd_solve_kernel(
    const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ v,
    const E* __restrict__ dO, const float* __restrict__ alpha, const float* __restrict__ beta,
    const E* __restrict__ Kl, const E* __restrict__ Wl, const E* __restrict__ dQt,
    const E* __restrict__ dUs, const E* __restrict__ dWks, const E* __restrict__ dKs,
    const float* __restrict__ dgs, E* __restrict__ dVp, E* __restrict__ dqp,
    E* __restrict__ dkp, float* __restrict__ dgp, float* __restrict__ dbeta, int B, int T,
    int H, int L, int NC, int Tp, const int* __restrict__ cu) {
  typedef CB2Lds<E, D, C> LY;
  constexpr int NW = CB_NW, NT = CB_NT;
  constexpr int LR = LY::LR, LT = LY::LT, LA = LY::LA;
  __shared__ __attribute__((aligned(16))) unsigned char smem[LY::TOTAL];
  float* g = reinterpret_cast<float*>(smem);
  float* ev = g + C;
  float* Dv = g + 2 * C;
  float* bt = g + 3 * C;
  float* be = g + 4 * C;
  float* de = g + 5 * C;
  float* rs = g + 6 * C;            // [NW][C] row sums for dg
  float* cs = rs + NW * C;          // [NW][C] column sums for dg
  float* bs = cs + NW * C;          // [NW][C] dbeta
  float* es = bs + NW * C;          // [NW][C] de
  float* bs2 = es + NW * C;         // [NW][C] dbeta, C x D products
  E* Kr = reinterpret_cast<E*>(smem + LY::O_K);
  E* Tb = reinterpret_cast<E*>(smem + LY::O_TB);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nblk = B * H * NC;
  const int bid = xcd_swizzle(blockIdx.x, nblk);
  const int c = bid % NC, bh = bid / NC;
  const int h = bh % H, b = bh / H;
  const int tb = c * C;
  const int nval = min(C, seq_len(cu, b, T) - tb);
  const long ts = (long)H * D;
  const long row0 = (seq_start(cu, b, T) + tb) * H + h;
  if (nval <= 0) return;   // past the end of a packed sequence: nothing to do
  const long cidx = (long)bh * NC + c;
  typedef Tiling<C, D, NW> TLD;
  typedef Tiling<C, C, NW> TLC;
  const bool actD = TLD::active(wave), actC = TLC::active(wave);
  // row / column sums over all products, reduced across lanes once at the end
  TileSums<TLC::RM, TLC::RN> sgc;   // rs (rows), cs (columns): decay gradient
  TileSums<TLC::RM, TLC::RN> sbc;   // bs (rows): beta gradient, C x C products
  TileSums<TLD::RM, TLD::RN> sbd;   // bs (rows): beta gradient, C x D products
  TileSums<TLD::RM, TLD::RN> sed;   // es (rows)
  sgc.zero();
  sbc.zero();
  sbd.zero();
  sed.zero();

  // K_l, W_l rows of the first fold step and the V rows are fetched early
  RegTile<E, C, D, NT> kl, wl, vn;
  if (L > 0) {
    const long lrow = (long)bh * L * Tp + tb;
    kl.load(Kl + lrow * D, D, C, tid);
    wl.load(Wl + lrow * D, D, C, tid);
  }
  vn.load(v + row0 * D, ts, nval, tid);
  for (int e = tid; e < 5 * NW * C; e += NT) rs[e] = 0.f;
  {
    // K rows requested before the decays' reads wait (one round trip)
    RegTile<E, C, D, NT> t_k;
    t_k.load(k + row0 * D, ts, nval, tid);
    if (wave == 0) chunk_decays<C>(alpha, beta, row0, H, nval, g, ev, Dv, bt, be, nullptr, lane);
    t_k.store_rows(Kr, LR, tid);
  }
  __syncthreads();
  f32x4 gamc[TLC::RM][TLC::RN];   // the decays of F_l (every fold step), R0 and dR0
  decays_ti<C, NW>(gamc, g, wave, lane);

  // ---- fold: V' = V - sum_l (Gam * K K_l^T)_{i<t} W_l  (kept in registers) ----
  Acc<C, D, NW> vp;
  vp.zero();
  {
    E* Klr = reinterpret_cast<E*>(smem + LY::F_KL);
    E* Wlr = reinterpret_cast<E*>(smem + LY::F_WL);
    E* Fb = reinterpret_cast<E*>(smem + LY::F_F);
    E* Vr = reinterpret_cast<E*>(smem + LY::F_V);
    for (int l = 0; l < L; ++l) {
      const long lrow = ((long)bh * L + l) * Tp + tb;
      kl.store_rows(Klr, LR, tid);
      wl.store_rows(Wlr, LR, tid);
      __syncthreads();
      {
        const long nrow = l + 1 < L ? lrow + Tp : lrow;   // (unconditional, as above)
        kl.load(Kl + nrow * D, D, C, tid);
        wl.load(Wl + nrow * D, D, C, tid);
      }
      Acc<C, C, NW> f;    // [t][i] = K_t . K_l,i
      f.zero();
      gemm_acc<E, C, C, D, NW, true, true>(f, Kr, LR, Klr, LR, wave, lane);
      for_tiles_ij(f, wave, lane, [&](int i, int j, int t0, int ii, const f32x4& x) {
#pragma unroll
        for (int r = 0; r < 4; ++r) Fb[(t0 + r) * LT + ii] = to_t<E>(ii < t0 + r ? gamc[i][j][r] * x[r] : 0.f);
      });
      __syncthreads();
      gemm_acc<E, C, D, C, NW, true, false>(vp, Fb, LT, Wlr, LR, wave, lane);
      __syncthreads();
    }
    vn.store_rows(Vr, LR, tid);
    __syncthreads();
    for_tiles_mut(vp, wave, lane, [&](int t0, int f, f32x4& x) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        x[r] = to_f(Vr[(t0 + r) * LR + f]) - x[r];
        Vr[(t0 + r) * LR + f] = to_t<E>(x[r]);      // V' rows, in place
      }
    });
  }

  // ---- solve: A = diag(beta)(Gam * K K^T)_{i<t}, T = (I + A)^{-1} ----
  // Q, dO rows and dQt of the next phase are fetched during the solve
  const E* dQtc = dQt + cidx * C * D;
  RegTile<E, C, D, NT> qn, on;
  RegTile<E, C, D, NT> dqn;
  qn.load(q + row0 * D, ts, nval, tid);
  on.load(dO + row0 * D, ts, nval, tid);
  dqn.load(dQtc, D, C, tid);
  E* Tbb = reinterpret_cast<E*>(smem + LY::S_TBB);
  E* Tbe = reinterpret_cast<E*>(smem + LY::S_TBE);
  {
    float* Af = reinterpret_cast<float*>(smem + LY::S_AF);
    float* Tf = reinterpret_cast<float*>(smem + LY::S_TF);
    float* Xs = reinterpret_cast<float*>(smem + LY::S_XS);
    Acc<C, C, NW> a;
    a.zero();
    gemm_acc<E, C, C, D, NW, true, true>(a, Kr, LR, Kr, LR, wave, lane);
    for_tiles(a, wave, lane, [&](int t0, int i, const f32x4& x) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = t0 + r;
        Af[t * LA + i] = i < t ? bt[t] * __expf(g[t] - g[i]) * x[r] : 0.f;
      }
    });
    __syncthreads();
    // (the wide instance reads the diagonal blocks' rows further ahead: its
    // registers peak elsewhere)
    invert_unit_lower<C, NW, false, (D >= 128 && C >= 64) ? INV_PD : 1>(Af, Tf, Xs, tid);
    // T, T diag(beta), T diag(beta e) in the operand type: column pairs, one
    // 2-element store each, all of a thread's reads issued together
    constexpr int NPR = C * C / 2, PPR = (NPR + NT - 1) / NT;
#pragma unroll
    for (int k = 0; k < PPR; ++k) {
      const int e = tid + k * NT;
      if (NPR % NT == 0 || e < NPR) {
        const int t = e / (C / 2), i = 2 * (e % (C / 2));
        const float t0 = Tf[t * LA + i], t1 = Tf[t * LA + i + 1];
        st2f(Tb + t * LT + i, t0, t1);
        st2f(Tbb + t * LT + i, t0 * bt[i], t1 * bt[i + 1]);
        st2f(Tbe + t * LT + i, t0 * be[i], t1 * be[i + 1]);
      }
    }
    __syncthreads();
  }
  E* Vpr = reinterpret_cast<E*>(smem + LY::F_V);
  E* Ur = reinterpret_cast<E*>(smem + LY::P_U);
  E* Wkr = reinterpret_cast<E*>(smem + LY::P_WK);
  {
    Acc<C, D, NW> ua, wa;   // U = T diag(beta) V', Wk = T diag(beta e) K  ([t][f])
    ua.zero();
    wa.zero();
    gemm_acc<E, C, D, C, NW, true, false>(ua, Tbb, LT, Vpr, LR, wave, lane);
    gemm_acc<E, C, D, C, NW, true, false>(wa, Tbe, LT, Kr, LR, wave, lane);
    __syncthreads();
    for_tiles(ua, wave, lane, [&](int t0, int f, const f32x4& x) {
#pragma unroll
      for (int r = 0; r < 4; ++r) Ur[(t0 + r) * LR + f] = to_t<E>(x[r]);
    });
    for_tiles(wa, wave, lane, [&](int t0, int f, const f32x4& x) {
#pragma unroll
      for (int r = 0; r < 4; ++r) Wkr[(t0 + r) * LR + f] = to_t<E>(x[r]);
    });
  }
  E* Qr = reinterpret_cast<E*>(smem + LY::P_Q);
  E* dOr = reinterpret_cast<E*>(smem + LY::P_DO);
  E* NdQ = reinterpret_cast<E*>(smem + LY::P_NDQ);
  E* R0b = reinterpret_cast<E*>(smem + LY::P_R0);
  E* Xb = reinterpret_cast<E*>(smem + LY::P_XB);
  qn.store_rows(Qr, LR, tid);
  on.store_rows(dOr, LR, tid);
  // -dQt rows (operand type)
  typedef RegTile<E, C, D, NT> DQT;
#pragma unroll
  for (int p = 0; p < DQT::PER; ++p) {
    const int u = tid + p * NT;
    const int r = u / DQT::VPR, c0 = (u % DQT::VPR) * DQT::VN;
    const E* x = reinterpret_cast<const E*>(&dqn.v[p][0]);
    if (u < DQT::NU) {
#pragma unroll
      for (int j = 0; j < DQT::VN; ++j) NdQ[r * LR + c0 + j] = to_t<E>(-to_f(x[j]));
    }
  }
  __syncthreads();
  // de_t = Q_t . dQt_t: each row is held by VPR consecutive lanes
  static_assert(DQT::VPR <= 64 && (64 % DQT::VPR) == 0, "a row within one wave");
#pragma unroll
  for (int p = 0; p < DQT::PER; ++p) {
    const int u = tid + p * NT;
    const int r = u / DQT::VPR, c0 = (u % DQT::VPR) * DQT::VN;
    const E* x = reinterpret_cast<const E*>(&dqn.v[p][0]);
    float sdq = 0.f;
    if (u < DQT::NU) {
#pragma unroll
      for (int j = 0; j < DQT::VN; ++j) sdq += to_f(Qr[r * LR + c0 + j]) * to_f(x[j]);
    }
    if constexpr (DQT::VPR == 16) {
      // a row is one 16-lane DPP row: its total in the last lane (the same
      // pairing as the xor butterfly, without LDS round trips)
      sdq = row16_sum(sdq);
      if (u < DQT::NU && (u % DQT::VPR) == DQT::VPR - 1) de[r] = sdq;
    } else {
#pragma unroll
      for (int off = 1; off < DQT::VPR; off <<= 1) sdq += __shfl_xor(sdq, off);
      if (u < DQT::NU && (u % DQT::VPR) == 0) de[r] = sdq;
    }
  }
  // dU_s, dWk_s, dK_s and dQt in the accumulator layout, for the epilogue
  // of the R0 products (fetched while they run)
  const E* dUc = dUs + cidx * C * D;
  const E* dWc = dWks + cidx * C * D;
  const E* dKc = dKs + cidx * C * D;
  // (dU_s, dWk_s, dK_s stored transposed: a lane's four tokens are contiguous,
  // kept as raw bits until used)
  typedef typename Raw4Of<E>::type R4;
  R4 pU[TLD::RM][TLD::RN], pW[TLD::RM][TLD::RN], pK[TLD::RM][TLD::RN];
  f32x4 pQ[TLD::RM][TLD::RN];
  if (actD) {
#pragma unroll
    for (int i = 0; i < TLD::RM; ++i)
#pragma unroll
      for (int j = 0; j < TLD::RN; ++j) {
        const int t0 = TLD::m0(wave) + 16 * i + 4 * (lane >> 4);
        const int f = TLD::n0(wave) + 16 * j + (lane & 15);
        const long ot = (long)f * C + t0;
        pU[i][j] = ld_raw4(dUc + ot);
        pW[i][j] = ld_raw4(dWc + ot);
        pK[i][j] = ld_raw4(dKc + ot);
#pragma unroll
        for (int r = 0; r < 4; ++r) pQ[i][j][r] = to_f(dQtc[(long)(t0 + r) * D + f]);
      }
  }

  // ---- R0 terms ----
  Acc<C, C, NW> r0;   // [t][i] = Gam * Q_t . K_i, i <= t
  r0.zero();
  gemm_acc<E, C, C, D, NW, true, true>(r0, Qr, LR, Kr, LR, wave, lane);
  if (actC) {
#pragma unroll
    for (int i = 0; i < TLC::RM; ++i)
#pragma unroll
      for (int j = 0; j < TLC::RN; ++j) {
        const int t0 = TLC::m0(wave) + 16 * i + 4 * (lane >> 4), ii = TLC::n0(wave) + 16 * j + (lane & 15);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          r0.v[i][j][r] = gamc[i][j][r] * r0.v[i][j][r];
          R0b[(t0 + r) * LT + ii] = to_t<E>(r0.v[i][j][r]);
        }
      }
  }
  {
    Acc<C, C, NW> dr;   // dR0 = dO U^T - dQt Wk^T
    dr.zero();
    gemm_acc<E, C, C, D, NW, true, true>(dr, dOr, LR, Ur, LR, wave, lane);
    gemm_acc<E, C, C, D, NW, true, true>(dr, NdQ, LR, Wkr, LR, wave, lane);
    if (actC) {
#pragma unroll
      for (int i = 0; i < TLC::RM; ++i)
#pragma unroll
        for (int j = 0; j < TLC::RN; ++j) {
          const int t0 = TLC::m0(wave) + 16 * i + 4 * (lane >> 4);
          const int ii = TLC::n0(wave) + 16 * j + (lane & 15);
          f32x4 pr;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int t = t0 + r;
            const float d_ = ii <= t ? dr.v[i][j][r] : 0.f;
            pr[r] = d_ * r0.v[i][j][r];
            Xb[t * LT + ii] = to_t<E>(gamc[i][j][r] * d_);
          }
          sgc.add(i, j, pr);
        }
    }
  }
  __syncthreads();
  Acc<C, D, NW> dq, dk;
  dq.zero();
  dk.zero();
  gemm_acc<E, C, D, C, NW, true, false>(dq, Xb, LT, Kr, LR, wave, lane);    // X0 K
  gemm_acc<E, C, D, C, NW, false, false>(dk, Xb, LT, Qr, LR, wave, lane);   // X0^T Q
  Acc<C, D, NW> du, dw;
  du.zero();
  dw.zero();
  gemm_acc<E, C, D, C, NW, false, false>(du, R0b, LT, dOr, LR, wave, lane);   // R0^T dO
  gemm_acc<E, C, D, C, NW, false, false>(dw, R0b, LT, NdQ, LR, wave, lane);   // -R0^T dQt
  __syncthreads();
  // dU = dU_s + R0^T dO, dWk = dWk_s - R0^T dQt -> rows (U, Wk slots);
  // dq += e dQt; dk += dK_s
  if (actD) {
#pragma unroll
    for (int i = 0; i < TLD::RM; ++i)
#pragma unroll
      for (int j = 0; j < TLD::RN; ++j) {
        const int t0 = TLD::m0(wave) + 16 * i + 4 * (lane >> 4);
        const int f = TLD::n0(wave) + 16 * j + (lane & 15);
        const f32x4 u4 = raw4_to_f(pU[i][j]), w4 = raw4_to_f(pW[i][j]), k4 = raw4_to_f(pK[i][j]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = t0 + r;
          Ur[t * LR + f] = to_t<E>(du.v[i][j][r] + u4[r]);
          Wkr[t * LR + f] = to_t<E>(dw.v[i][j][r] + w4[r]);
          dq.v[i][j][r] += ev[t] * pQ[i][j][r];
          dk.v[i][j][r] += k4[r];
        }
      }
  }
  E* dUr = Ur;
  E* dWkr = Wkr;
  // V' rows again (their slot was reused by Q): from the registers
  E* Vp2 = reinterpret_cast<E*>(smem + LY::P_Q);
  __syncthreads();
  for_tiles(vp, wave, lane, [&](int t0, int f, const f32x4& x) {
#pragma unroll
    for (int r = 0; r < 4; ++r) Vp2[(t0 + r) * LR + f] = to_t<E>(x[r]);
  });
  __syncthreads();

  // ---- solve backward ----
  {
    Acc<C, D, NW> x1, x2;   // T^T dU, T^T dWk  ([i][f])
    x1.zero();
    x2.zero();
    gemm_acc<E, C, D, C, NW, false, false>(x1, Tb, LT, dUr, LR, wave, lane);
    gemm_acc<E, C, D, C, NW, false, false>(x2, Tb, LT, dWkr, LR, wave, lane);
    E* dVc = dVp + cidx * C * D;
    if (actD) {
#pragma unroll
      for (int i = 0; i < TLD::RM; ++i)
#pragma unroll
        for (int j = 0; j < TLD::RN; ++j) {
          const int t0 = TLD::m0(wave) + 16 * i + 4 * (lane >> 4);
          const int f = TLD::n0(wave) + 16 * j + (lane & 15);
          f32x4 pb, pk;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int t = t0 + r;
            dVc[(long)t * D + f] = to_t<E>(bt[t] * x1.v[i][j][r]);        // dV'
            pb[r] = vp.v[i][j][r] * x1.v[i][j][r];
            pk[r] = to_f(Kr[t * LR + f]) * x2.v[i][j][r];
            dk.v[i][j][r] += be[t] * x2.v[i][j][r];
          }
          sbd.add(i, j, pb, true, false);
          sed.add(i, j, pk, true, false);
        }
    }
  }
  E* dTb = R0b;
  E* P1b = Xb;
  {
    Acc<C, C, NW> t1, t2;   // dU V'^T, dWk K^T  ([t][i])
    t1.zero();
    t2.zero();
    gemm_acc<E, C, C, D, NW, true, true>(t1, dUr, LR, Vp2, LR, wave, lane);
    gemm_acc<E, C, C, D, NW, true, true>(t2, dWkr, LR, Kr, LR, wave, lane);
    __syncthreads();
    if (actC) {
#pragma unroll
      for (int i = 0; i < TLC::RM; ++i)
#pragma unroll
        for (int j = 0; j < TLC::RN; ++j) {
          const int t0 = TLC::m0(wave) + 16 * i + 4 * (lane >> 4);
          const int ii = TLC::n0(wave) + 16 * j + (lane & 15);
#pragma unroll
          for (int r = 0; r < 4; ++r)
            dTb[(t0 + r) * LT + ii] = to_t<E>(bt[ii] * t1.v[i][j][r] + be[ii] * t2.v[i][j][r]);
        }
    }
  }
  __syncthreads();
  {
    Acc<C, C, NW> p1;   // dT T^T  ([t][i] = sum_j dT[t][j] T[i][j])
    p1.zero();
    gemm_acc<E, C, C, C, NW, true, true>(p1, dTb, LT, Tb, LT, wave, lane);
    __syncthreads();
    for_tiles(p1, wave, lane, [&](int t0, int i, const f32x4& x) {
#pragma unroll
      for (int r = 0; r < 4; ++r) P1b[(t0 + r) * LT + i] = to_t<E>(x[r]);
    });
  }
  __syncthreads();
  float* Zf = reinterpret_cast<float*>(smem + LY::Z_F);
  E* Zb = reinterpret_cast<E*>(smem + LY::Z_B);
  {
    Acc<C, C, NW> da, y;   // dA = -T^T P1 ([i][j]); Y = Gam * K K^T (recomputed)
    da.zero();
    y.zero();
    gemm_acc<E, C, C, C, NW, false, false>(da, Tb, LT, P1b, LT, wave, lane);
    gemm_acc<E, C, C, D, NW, true, true>(y, Kr, LR, Kr, LR, wave, lane);
    if (actC) {
#pragma unroll
      for (int i = 0; i < TLC::RM; ++i)
#pragma unroll
        for (int j = 0; j < TLC::RN; ++j) {
          const int t0 = TLC::m0(wave) + 16 * i + 4 * (lane >> 4);
          const int jj = TLC::n0(wave) + 16 * j + (lane & 15);
          f32x4 pb, py;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int t = t0 + r;
            const bool m = jj < t;
            const float gam = m ? __expf(g[t] - g[jj]) : 0.f;
            const float yv = gam * y.v[i][j][r];
            const float dav = m ? -da.v[i][j][r] : 0.f;
            pb[r] = dav * yv;                       // dbeta_t += dA . Y
            const float dy = bt[t] * dav;
            py[r] = dy * yv;                        // dg via Gam
            Zf[t * LA + jj] = gam * dy;             // dG0
          }
          sbc.add(i, j, pb, true, false);
          sgc.add(i, j, py);
        }
    }
  }
  __syncthreads();
  {
    // dG0 + dG0^T in the operand type: column pairs, all of a thread's reads
    // issued together, one 2-element store each
    constexpr int NPR = C * C / 2, PPR = (NPR + NT - 1) / NT;
#pragma unroll
    for (int k = 0; k < PPR; ++k) {
      const int e = tid + k * NT;
      if (NPR % NT == 0 || e < NPR) {
        const int t = e / (C / 2), i = 2 * (e % (C / 2));
        st2f(Zb + t * LT + i, Zf[t * LA + i] + Zf[i * LA + t], Zf[t * LA + i + 1] + Zf[(i + 1) * LA + t]);
      }
    }
  }
  __syncthreads();
  gemm_acc<E, C, D, C, NW, true, false>(dk, Zb, LT, Kr, LR, wave, lane);   // (dG0 + dG0^T) K

  // the state kernel's part of the decay gradient, requested ahead of the
  // output stores (loads and stores retire in issue order: requested after
  // them, its wait would cover every one of them)
  const float dgs_t = dgs[cidx * C + (tid & (C - 1))];
  // ---- outputs ----
  E* dqc = dqp + cidx * C * D;
  E* dkc = dkp + cidx * C * D;
  for_tiles(dq, wave, lane, [&](int t0, int f, const f32x4& x) {
#pragma unroll
    for (int r = 0; r < 4; ++r) dqc[(long)(t0 + r) * D + f] = to_t<E>(x[r]);
  });
  for_tiles(dk, wave, lane, [&](int t0, int f, const f32x4& x) {
#pragma unroll
    for (int r = 0; r < 4; ++r) dkc[(long)(t0 + r) * D + f] = to_t<E>(x[r]);
  });
  if (actC) {
    sgc.flush_rows(rs + wave * C, TLC::m0(wave), lane);
    sgc.flush_cols(cs + wave * C, TLC::n0(wave), lane);
    sbc.flush_rows(bs + wave * C, TLC::m0(wave), lane);
  }
  if (actD) {
    sbd.flush_rows(bs2 + wave * C, TLD::m0(wave), lane);
    sed.flush_rows(es + wave * C, TLD::m0(wave), lane);
  }
  __syncthreads();
  if (tid < C) {
    const int t = tid;
    float sr = 0.f, sb = 0.f, se = 0.f;
    for (int w = 0; w < NW; ++w) {
      sr += rs[w * C + t] - cs[w * C + t];
      sb += bs[w * C + t] + bs2[w * C + t];
      se += es[w * C + t];
    }
    // de: from Qt (Q . dQt) and from Wk (beta K . X2); e_t = exp(g_t)
    const float det = de[t] + bt[t] * se;
    dgp[cidx * C + t] = dgs_t + sr + ev[t] * det;
    if (t < nval) dbeta[row0 + (long)t * H] = sb + ev[t] * se;
  }
}

struct SolveLaunch {
  template <typename E, int D, int C>
  static hipError_t run(const Dims& d, const ChunkBwdArgs<E>& a, hipStream_t s) {
    if constexpr (sizeof(E) == 4 && D * C > 2048) {
      return hipErrorInvalidValue;   // outside the fp32 envelope (LDS)
    } else {
      const int nblk = d.B * d.H * d.NC;
      hipLaunchKernelGGL((chunk_bwd_solve_kernel<E, D, C>), dim3(nblk), dim3(CB_NT), 0, s, a.q,
                         a.k, a.v, a.dO, a.alpha, a.beta, a.Kl, a.Wl, a.dQt, a.dUs, a.dWks, a.dKs,
                         a.dgs, a.dVp, a.dqp, a.dkp, a.dgp, a.dbeta, d.B, d.T, d.H, d.L, d.NC,
                         d.Tp, d.cu);
      return hipGetLastError();
    }
  }
};

template <typename E>
hipError_t launch_chunk_bwd_solve(const Dims& d, const ChunkBwdArgs<E>& a, hipStream_t s) {
  return cbwd_dispatch<E, SolveLaunch>(d, a, s);
}

template hipError_t launch_chunk_bwd_solve<bf16>(const Dims&, const ChunkBwdArgs<bf16>&, hipStream_t);
template hipError_t launch_chunk_bwd_solve<float>(const Dims&, const ChunkBwdArgs<float>&, hipStream_t);

}  // namespace prism
