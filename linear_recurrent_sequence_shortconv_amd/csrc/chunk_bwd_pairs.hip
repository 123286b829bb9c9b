// Chunk backward, third kernel: the refinement-pair terms and the final gradients.
#include "chunk_bwd_common.h"

namespace prism {

// ===========================================================================
// chunk_bwd_pairs
// ===========================================================================
template <typename E, int D, int C>
struct CB3Lds {
  static constexpr int LR = ldpad<E>(D);
  static constexpr int LT = ldpad<E>(C);
  static constexpr int SZ_R = C * LR * (int)sizeof(E);
  static constexpr int SZ_CC = C * LT * (int)sizeof(E);
  static constexpr int SZ_VEC = (2 * C + 2 * CB_NW * C) * 4;   // g, alpha, rs, cs
  static constexpr int O_Q = (SZ_VEC + 15) / 16 * 16;
  static constexpr int O_K = O_Q + SZ_R;
  static constexpr int O_DO = O_K + SZ_R;
  static constexpr int O_DV = O_DO + SZ_R;
  static constexpr int O_KL = O_DV + SZ_R;
  static constexpr int O_WL = O_KL + SZ_R;
  static constexpr int O_RB = O_WL + SZ_R;
  static constexpr int O_XB = O_RB + SZ_CC;
  static constexpr int O_FB = O_XB + SZ_CC;
  static constexpr int O_GB = O_FB + SZ_CC;
  static constexpr int TOTAL = O_GB + SZ_CC;
};

template <typename E, int D, int C>
__global__ __launch_bounds__(CB_NT) void chunk_bwd_pairs_kernel(
    const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ dO,
    const float* __restrict__ alpha, const E* __restrict__ Kl, const E* __restrict__ Wl,
    const E* __restrict__ dVp, const E* __restrict__ dqp, const E* __restrict__ dkp,
    const float* __restrict__ dgp, E* __restrict__ dKl, float* __restrict__ dWl,
    E* __restrict__ dq, E* __restrict__ dk, E* __restrict__ dv,
    float* __restrict__ dalpha, int B, int T, int H, int L, int NC, int Tp,
    const int* __restrict__ cu) {
  typedef CB3Lds<E, D, C> LY;
  constexpr int NW = CB_NW, NT = CB_NT;
  constexpr int LR = LY::LR, LT = LY::LT;
  __shared__ __attribute__((aligned(16))) unsigned char smem[LY::TOTAL];
  float* g = reinterpret_cast<float*>(smem);
  float* al = g + C;
  float* rs = g + 2 * C;
  float* cs = rs + NW * C;
  E* Qr = reinterpret_cast<E*>(smem + LY::O_Q);
  E* Kr = reinterpret_cast<E*>(smem + LY::O_K);
  E* dOr = reinterpret_cast<E*>(smem + LY::O_DO);
  E* dVr = reinterpret_cast<E*>(smem + LY::O_DV);
  E* Klr = reinterpret_cast<E*>(smem + LY::O_KL);
  E* Wlr = reinterpret_cast<E*>(smem + LY::O_WL);
  E* Rb = reinterpret_cast<E*>(smem + LY::O_RB);
  E* Xb = reinterpret_cast<E*>(smem + LY::O_XB);
  E* NFb = reinterpret_cast<E*>(smem + LY::O_FB);
  E* Gb = reinterpret_cast<E*>(smem + LY::O_GB);

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
  typedef Tiling<C, C, NW> TLC;
  const bool actC = TLC::active(wave);

  for (int e = tid; e < 2 * NW * C; e += NT) rs[e] = 0.f;
  {
    // the four row tiles, all requested before the first is stored (one
    // memory round trip, which the decays' reads share)
    RegTile<E, C, D, NT> t_q, t_k, t_do, t_dv;
    t_q.load(q + row0 * D, ts, nval, tid);
    t_k.load(k + row0 * D, ts, nval, tid);
    t_do.load(dO + row0 * D, ts, nval, tid);
    t_dv.load(dVp + cidx * C * D, D, C, tid);
    if (wave == 0) {
      __shared__ float dummy[3 * C];
      chunk_decays<C>(alpha, nullptr, row0, H, nval, g, dummy, dummy + C, nullptr, nullptr, al, lane);
    }
    t_q.store_rows(Qr, LR, tid);
    t_k.store_rows(Kr, LR, tid);
    t_do.store_rows(dOr, LR, tid);
    t_dv.store_rows(dVr, LR, tid);
  }
  __syncthreads();

  Acc<C, D, NW> dqa, dka;
  dqa.zero();
  dka.zero();
  typedef Tiling<C, D, NW> TLD;
  TileSums<TLC::RM, TLC::RN> dgs_;   // decay-gradient row / column sums over all steps
  dgs_.zero();
  // next step's K_l, W_l rows (software prefetch); after the last step, the
  // solve kernel's parts of dq and dk (rows), which the last phase adds to
  const E* dqc = dqp + cidx * C * D;
  const E* dkc = dkp + cidx * C * D;
  RegTile<E, C, D, NT> kl, wl;
  {
    const long lrow = (long)bh * L * Tp + tb;
    kl.load(L > 0 ? Kl + lrow * D : dqc, D, C, tid);
    wl.load(L > 0 ? Wl + lrow * D : dkc, D, C, tid);
  }
  for (int l = 0; l < L; ++l) {
    const long lrow = ((long)bh * L + l) * Tp + tb;
    kl.store_rows(Klr, LR, tid);
    wl.store_rows(Wlr, LR, tid);
    __syncthreads();
    {
      // (unconditional loads into the same registers, the last step's being
      // the dq, dk parts: a load under a condition leaves a merge of old and
      // new registers that the compiler resolves with copies at the loop head,
      // which wait for every memory operation in flight, the previous step's
      // gradient stores included)
      const bool nx = l + 1 < L;
      kl.load(nx ? Kl + (lrow + Tp) * D : dqc, D, C, tid);
      wl.load(nx ? Wl + (lrow + Tp) * D : dkc, D, C, tid);
    }
    // the partial dK_l, dW_l of the state-gradient kernel (accumulator
    // layout), in flight during the products of this step; kept raw and
    // converted where they are added (a conversion next to the load would
    // make the wave wait for these scattered loads right after issuing them)
    typename Raw1Of<E>::type pkl[TLD::RM][TLD::RN][4];
    float pwl[TLD::RM][TLD::RN][4];
    if (TLD::active(wave)) {
#pragma unroll
      for (int i = 0; i < TLD::RM; ++i)
#pragma unroll
        for (int j = 0; j < TLD::RN; ++j) {
          const int t0 = TLD::m0(wave) + 16 * i + 4 * (lane >> 4);
          const int f = TLD::n0(wave) + 16 * j + (lane & 15);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            pkl[i][j][r] = ld_raw1(dKl + (lrow + t0 + r) * D + f);
            pwl[i][j][r] = dWl[(lrow + t0 + r) * D + f];
          }
        }
    }
    // the decays of R_l and F_l (formed per step: kept across the steps they
    // would push the kernel past its registers)
    f32x4 gamc[TLC::RM][TLC::RN];
    decays_ti<C, NW>(gamc, g, wave, lane);
    // R_l = (Gam * Q K_l^T)_{i<=t}, dR_l = dO W_l^T  -> Rb, Xb = Gam * dR_l
    {
      Acc<C, C, NW> r, dr;
      r.zero();
      dr.zero();
      gemm_acc<E, C, C, D, NW, true, true, true>(r, Qr, LR, Klr, LR, wave, lane);
      gemm_acc<E, C, C, D, NW, true, true, true>(dr, dOr, LR, Wlr, LR, wave, lane);
      if (actC) {
#pragma unroll
        for (int i = 0; i < TLC::RM; ++i)
#pragma unroll
          for (int j = 0; j < TLC::RN; ++j) {
            const int t0 = TLC::m0(wave) + 16 * i + 4 * (lane >> 4);
            const int ii = TLC::n0(wave) + 16 * j + (lane & 15);
            f32x4 p;
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
              const int t = t0 + rr;
              const float gam = gamc[i][j][rr];
              const float rv = gam * r.v[i][j][rr];
              const float drv = ii <= t ? dr.v[i][j][rr] : 0.f;
              p[rr] = drv * rv;
              Rb[t * LT + ii] = to_t<E>(rv);
              Xb[t * LT + ii] = to_t<E>(gam * drv);
            }
            dgs_.add(i, j, p);
          }
      }
    }
    // F_l = (Gam * K K_l^T)_{i<t}, dF_l = -(dV' W_l^T)_{i<t}  -> NFb = -F_l, Gb = Gam * dF_l
    {
      Acc<C, C, NW> f, df;
      f.zero();
      df.zero();
      gemm_acc<E, C, C, D, NW, true, true, true>(f, Kr, LR, Klr, LR, wave, lane);
      gemm_acc<E, C, C, D, NW, true, true, true>(df, dVr, LR, Wlr, LR, wave, lane);
      if (actC) {
#pragma unroll
        for (int i = 0; i < TLC::RM; ++i)
#pragma unroll
          for (int j = 0; j < TLC::RN; ++j) {
            const int t0 = TLC::m0(wave) + 16 * i + 4 * (lane >> 4);
            const int ii = TLC::n0(wave) + 16 * j + (lane & 15);
            f32x4 p;
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
              const int t = t0 + rr;
              const float gam = ii < t ? gamc[i][j][rr] : 0.f;
              const float fv = gam * f.v[i][j][rr];
              const float dfv = ii < t ? -df.v[i][j][rr] : 0.f;
              p[rr] = dfv * fv;
              NFb[t * LT + ii] = to_t<E>(-fv);
              Gb[t * LT + ii] = to_t<E>(gam * dfv);
            }
            dgs_.add(i, j, p);
          }
      }
    }
    __syncthreads();
    Acc<C, D, NW> dkl, dwl;
    dkl.zero();
    dwl.zero();
    gemm_acc<E, C, D, C, NW, false, false, true>(dkl, Xb, LT, Qr, LR, wave, lane);    // X_l^T Q
    gemm_acc<E, C, D, C, NW, false, false, true>(dkl, Gb, LT, Kr, LR, wave, lane);    // dG_l^T K
    gemm_acc<E, C, D, C, NW, false, false, true>(dwl, Rb, LT, dOr, LR, wave, lane);   // R_l^T dO
    gemm_acc<E, C, D, C, NW, false, false, true>(dwl, NFb, LT, dVr, LR, wave, lane);  // -F_l^T dV'
    gemm_acc<E, C, D, C, NW, true, false, true>(dqa, Xb, LT, Klr, LR, wave, lane);    // X_l K_l
    gemm_acc<E, C, D, C, NW, true, false, true>(dka, Gb, LT, Klr, LR, wave, lane);    // dG_l K_l
    if (TLD::active(wave)) {
#pragma unroll
      for (int i = 0; i < TLD::RM; ++i)
#pragma unroll
        for (int j = 0; j < TLD::RN; ++j) {
          const int t0 = TLD::m0(wave) + 16 * i + 4 * (lane >> 4);
          const int f = TLD::n0(wave) + 16 * j + (lane & 15);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            dKl[(lrow + t0 + r) * D + f] = to_t<E>(raw1_to_f(pkl[i][j][r]) + dkl.v[i][j][r]);
            dWl[(lrow + t0 + r) * D + f] = raw1_to_f(pwl[i][j][r]) + dwl.v[i][j][r];
          }
        }
    }
    __syncthreads();
  }

  // The lane's offsets of the last phases are formed again from an opaque copy
  // of the thread index: kept live across the refinement loop they spill.
  int tid_o = threadIdx.x;
  asm volatile("" : "+v"(tid_o));
  {
  const int tid = tid_o, lane = tid_o & 63;
  // ---- final dq, dk (and dv when L = 0) ----
  if (actC) {
    dgs_.flush_rows(rs + wave * C, TLC::m0(wave), lane);
    dgs_.flush_cols(cs + wave * C, TLC::n0(wave), lane);
  }
  // fp32 products staged in LDS (every tile buffer is free now), then added
  // to the solve kernel's parts and stored as full rows
  const E* dvc = dVp + cidx * C * D;
  const RegTile<E, C, D, NT>& rq = kl;   // the dq, dk parts, fetched during the last step
  const RegTile<E, C, D, NT>& rk = wl;
  // the decay gradient of the other kernels, requested ahead of the output
  // stores (requested after them, its wait would cover every one of them)
  const float dgp_t = dgp[cidx * C + (lane & (C - 1))];
  constexpr int LF = D + 4;
  float* Sq = reinterpret_cast<float*>(smem + LY::O_Q);
  float* Sk = Sq + C * LF;
  static_assert(LY::O_Q + 2 * C * LF * 4 <= LY::TOTAL, "staging fits");
  for_tiles(dqa, wave, lane, [&](int t0, int f, const f32x4& x) {
#pragma unroll
    for (int r = 0; r < 4; ++r) Sq[(t0 + r) * LF + f] = x[r];
  });
  for_tiles(dka, wave, lane, [&](int t0, int f, const f32x4& x) {
#pragma unroll
    for (int r = 0; r < 4; ++r) Sk[(t0 + r) * LF + f] = x[r];
  });
  __syncthreads();
  {
    typedef RegTile<E, C, D, NT> RT;
    E* dqo = dq + row0 * D;
    E* dko = dk + row0 * D;
#pragma unroll
    for (int p = 0; p < RT::PER; ++p) {
      const int u = tid + p * NT;
      const int r = u / RT::VPR, c0 = (u % RT::VPR) * RT::VN;
      if (u < RT::NU && r < nval) {
        const E* a = reinterpret_cast<const E*>(&rq.v[p][0]);
        const E* b = reinterpret_cast<const E*>(&rk.v[p][0]);
        E oq[RT::VN], ok[RT::VN];
#pragma unroll
        for (int j = 0; j < RT::VN; ++j) {
          oq[j] = to_t<E>(to_f(a[j]) + Sq[r * LF + c0 + j]);
          ok[j] = to_t<E>(to_f(b[j]) + Sk[r * LF + c0 + j]);
        }
        uint4 wq, wk;
        __builtin_memcpy(&wq, oq, 16);
        __builtin_memcpy(&wk, ok, 16);
        st16(dqo + (long)r * ts + c0, wq);
        st16(dko + (long)r * ts + c0, wk);
      }
    }
  }
  // with L > 0 the direct v-gradient dV' (chunk rows [bh][c][t] = token rows
  // [bh][c C + t]) is completed by the refinement backward; at L = 0 it is dv
  if (L == 0) {
    // (every row requested before the first is stored: one round trip)
    typedef RegTile<E, C, D, NT> VT;
    VT tv;
    tv.load(dvc, D, C, tid);
    E* dvo = dv + row0 * D;
#pragma unroll
    for (int p = 0; p < VT::PER; ++p) {
      const int u = tid + p * NT;
      int t, f;
      VT::unit(u, t, f);
      if (u < VT::NU && t < nval) st16(dvo + (long)t * ts + f, tv.v[p][0]);
    }
  }
  __syncthreads();
  // ---- dalpha: dlog(alpha)_j = sum_{t >= j} dg_t ----
  if (wave == 0) {
    float dg = 0.f;
    if (lane < C) {
      dg = dgp_t;
      for (int w = 0; w < NW; ++w) dg += rs[w * C + lane] - cs[w * C + lane];
    }
    // reverse inclusive scan over lanes 0..C-1
    float s = dg;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float y = __shfl_down(s, off);
      if (lane + off < 64) s += y;
    }
    if (lane < nval) dalpha[row0 + (long)lane * H] = s / al[lane];
  }
  }
}

struct PairsLaunch {
  template <typename E, int D, int C>
  static hipError_t run(const Dims& d, const ChunkBwdArgs<E>& a, hipStream_t s) {
    if constexpr (sizeof(E) == 4 && D * C > 2048) {
      return hipErrorInvalidValue;   // outside the fp32 envelope (LDS)
    } else {
      const int nblk = d.B * d.H * d.NC;
      hipLaunchKernelGGL((chunk_bwd_pairs_kernel<E, D, C>), dim3(nblk), dim3(CB_NT), 0, s, a.q,
                         a.k, a.dO, a.alpha, a.Kl, a.Wl, a.dVp, a.dqp, a.dkp, a.dgp, a.dKl, a.dWl,
                         a.dq, a.dk, a.dv, a.dalpha, d.B, d.T, d.H, d.L, d.NC, d.Tp, d.cu);
      return hipGetLastError();
    }
  }
};

template <typename E>
hipError_t launch_chunk_bwd_pairs(const Dims& d, const ChunkBwdArgs<E>& a, hipStream_t s) {
  return cbwd_dispatch<E, PairsLaunch>(d, a, s);
}

template hipError_t launch_chunk_bwd_pairs<bf16>(const Dims&, const ChunkBwdArgs<bf16>&, hipStream_t);
template hipError_t launch_chunk_bwd_pairs<float>(const Dims&, const ChunkBwdArgs<float>&, hipStream_t);

}  // namespace prism
