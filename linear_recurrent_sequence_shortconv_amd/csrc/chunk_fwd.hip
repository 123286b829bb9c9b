// Chunk-local part of the PRISM recurrence S_t = S_{t-1} A_t + B_t
// (PRISM technical summary §2.1, with A_t = alpha_t (I - beta_t k_t k_t^T) and
// B_t = beta_t v_t k_t^T + sum_l w_t^(l) k_t^(l)^T).  §2.2 (last paragraph)
// notes that every part of the update depends on the input only; hence a
// chunk of C tokens acts on the entering state S as one affine map
//
//     S_next = exp(gC) S - S M + H,        O = O_loc + Qt S^T,
//
// whose coefficients this kernel computes, one workgroup per (b, h, chunk):
//
//     g_t = sum_{j<=t} log alpha_j,  Gam_ti = exp(g_t - g_i),  D_t = exp(gC - g_t)
//     A   = diag(beta) (Gam * K K^T)_{i<t},   T = (I + A)^{-1}   (fp32, LDS)
//     V'  = V - sum_l (Gam * K K_l^T)_{i<t} W_l
//     U   = T diag(beta) V',   Wk = T diag(beta e^g) K
//     M   = Wk^T diag(D) K,    H  = U^T diag(D) K + sum_l W_l^T diag(D) K_l
//     R0  = (Gam * Q K^T)_{i<=t},  R_l = (Gam * Q K_l^T)_{i<=t}
//     Qt  = diag(e^g) Q - R0 Wk,   O_loc = R0 U + sum_l R_l W_l
//
// All products are bf16 (or fp32) MFMA with fp32 accumulation; T, the decays
// and the accumulators stay fp32.  Stored (global, per chunk):
//   Mt [D][D] = M^T (MFMA B operand of the state pass, both directions),
//   HT [D][D] = H^T fp32, Qt [C][D], O_loc [C][D] fp32, gC, and when asked
//   (training forward) U^T, Wk^T [D][C] for the reverse chunk kernels.
// In backward mode (dO given) the kernel instead stores Mt, HT, gC,
// ET = (dO^T Qt)^T fp32 (for the reverse state pass) and U^T, Wk^T.
// et_kernel forms ET from a saved Qt when the forward was kept.
#include "prism_common.h"
#include "prism_internal.h"

namespace prism {

constexpr int CF_NW = 8;
constexpr int CF_NT = CF_NW * WAVE;

template <typename E, int D, int C>
struct ChunkLds {
  static constexpr int LR = ldpad<E>(D);     // [C][LR]: C rows of D
  static constexpr int LT = ldpad<E>(C);     // [D][LT] transposed, and [C][LT] C x C
  static constexpr int LA = C + 1;           // fp32 C x C
  static constexpr int SZ_R = C * LR * (int)sizeof(E);
  static constexpr int SZ_T = D * LT * (int)sizeof(E);
  static constexpr int SZ_CC = C * LT * (int)sizeof(E);
  static constexpr int SZ_F = C * LA * 4;
  static constexpr int SZ_VEC = 5 * C * 4;
  // persistent
  static constexpr int O_VEC = 0;
  static constexpr int O_Q = O_VEC + SZ_VEC;
  static constexpr int O_K = O_Q + SZ_R;
  static constexpr int O_X = O_K + SZ_R;
  // phase B (per refinement step)
  static constexpr int B_KLR = O_X;
  static constexpr int B_KLTD = B_KLR + SZ_R;
  static constexpr int B_WLT = B_KLTD + SZ_T;
  static constexpr int B_F = B_WLT + SZ_T;
  static constexpr int B_RL = B_F + SZ_CC;
  static constexpr int B_END = B_RL + SZ_CC;
  // phase T (solve)
  static constexpr int C_TB = O_X;
  static constexpr int T_AF = C_TB + SZ_CC;
  static constexpr int T_TF = T_AF + SZ_F;
  static constexpr int T_XS = T_TF + SZ_F;
  static constexpr int T_END = T_XS + inv_scratch_floats(C) * 4;
  // phase C
  static constexpr int C_KTBE = C_TB + SZ_CC;   // later Wk^T
  static constexpr int C_KTD = C_KTBE + SZ_T;
  static constexpr int C_VT = C_KTD + SZ_T;     // (beta V')^T, later U^T, later Qt^T
  static constexpr int C_R0 = C_VT + SZ_T;
  static constexpr int C_V = cmax(C_R0 + SZ_CC, T_END);   // V rows, later dO^T
  static constexpr int C_END = C_V + cmax(SZ_R, SZ_T);
  static constexpr int TOTAL = cmax(B_END, C_END);
};

template <typename E, int D, int C, bool BWD>
__global__ __launch_bounds__(CF_NT) void chunk_fwd_kernel(
    const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ v,
    const float* __restrict__ alpha, const float* __restrict__ beta, const E* __restrict__ Kl,
    const E* __restrict__ Wl, const E* __restrict__ dO, E* __restrict__ Mt, float* __restrict__ HT,
    E* __restrict__ Qt, float* __restrict__ Oloc, float* __restrict__ gCo,
    float* __restrict__ ET, E* __restrict__ UTo, E* __restrict__ WkTo, int B, int T, int H, int L,
    int NC, int Tp, const int* __restrict__ cu) {
  typedef ChunkLds<E, D, C> LY;
  constexpr int NW = CF_NW, NT = CF_NT;
  constexpr int LR = LY::LR, LT = LY::LT, LA = LY::LA;
  __shared__ __attribute__((aligned(16))) unsigned char smem[LY::TOTAL];

  float* g = reinterpret_cast<float*>(smem + LY::O_VEC);
  float* ev = g + C;
  float* Dv = g + 2 * C;
  float* bt = g + 3 * C;
  float* be = g + 4 * C;
  E* Qr = reinterpret_cast<E*>(smem + LY::O_Q);
  E* Kr = reinterpret_cast<E*>(smem + LY::O_K);

  int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nblk = B * H * NC;
  const long ts = (long)H * D;
  // At d = 128 (one workgroup per CU) workgroups are persistent: they take
  // the virtual block ids blockIdx.x, + gridDim.x, ..., and a chunk's first
  // operands (Q and K rows, alpha, beta, the first K_l and W_l tiles) are
  // fetched while the previous chunk is being finished.  Smaller d launch one
  // workgroup per chunk (the loop runs once).
  constexpr bool PERSIST = D >= 128;
  const int vstride = PERSIST ? (int)gridDim.x : nblk;
  RegTile<E, C, D, NT, true> kn, wn;   // K_l, W_l tiles of the next product step
  RegTile<E, C, D, NT> qn, kr;         // Q, K rows of the next chunk
  float pa = 1.f, pb = 0.f;            // alpha, beta of the next chunk (wave 0, lane < C)
  auto prefetch = [&](int vid) {
    const int bid = xcd_swizzle(vid, nblk);
    const int c = bid % NC, bh = bid / NC;
    const int h = bh % H, b = bh / H;
    const int tb = c * C;
    const int nval = min(C, seq_len(cu, b, T) - tb);
    const long row0 = (seq_start(cu, b, T) + tb) * H + h;
    if (L > 0) {
      kn.load(Kl + (long)bh * L * Tp * D + (long)tb * D, D, C, tid);
      wn.load(Wl + (long)bh * L * Tp * D + (long)tb * D, D, C, tid);
    }
    qn.load(q + row0 * D, ts, nval, tid);
    kr.load(k + row0 * D, ts, nval, tid);
    if (wave == 0) {
      pa = lane < nval ? alpha[row0 + (long)lane * H] : 1.f;
      pb = lane < nval ? beta[row0 + (long)lane * H] : 0.f;
    }
  };
  if ((int)blockIdx.x < nblk) prefetch(blockIdx.x);
  for (int vid = blockIdx.x; vid < nblk; vid += vstride) {
  // per-lane values are redefined each iteration, so that the lane-dependent
  // address arithmetic of the body is not hoisted out of the loop and kept
  // live across it
  if constexpr (PERSIST) {
    asm volatile("" : "+v"(tid));
    lane = tid & 63;
    wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  }
  const int bid = xcd_swizzle(vid, nblk);
  const int c = bid % NC, bh = bid / NC;
  const int h = bh % H, b = bh / H;
  const int tb = c * C;
  const int nval = min(C, seq_len(cu, b, T) - tb);
  const long row0 = (seq_start(cu, b, T) + tb) * H + h;
  // past the end of a packed sequence no pass reads the chunk: a one-chunk
  // workgroup leaves; a persistent one computes its identity map (all tokens
  // padding), since a skip path here costs registers on every chunk
  if constexpr (!PERSIST) {
    if (nval <= 0) return;
  }
  const E* vc = v + row0 * D;
  const E* Klb = Kl + (long)bh * L * Tp * D + (long)tb * D;
  const E* Wlb = Wl + (long)bh * L * Tp * D + (long)tb * D;

  // ---- phase A: decays and gates; Q, K tiles ----
  if (wave == 0) {
    const float lg = logf(pa), bv = pb;   // alpha = 1, beta = 0 past the end
    float s = lg;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float y = __shfl_up(s, off);
      if (lane >= off) s += y;
    }
    const float gC = __shfl(s, C - 1);
    if (lane < C) {
      const float e = expf(s);
      g[lane] = s;
      ev[lane] = e;
      Dv[lane] = expf(gC - s);
      bt[lane] = bv;
      be[lane] = bv * e;
    }
    if (lane == 0) gCo[(long)bh * NC + c] = gC;
  }
  qn.store_rows(Qr, LR, tid);
  kr.store_rows(Kr, LR, tid);
  __syncthreads();

  // ---- phase B: refinement pairs, one step l at a time ----
  Acc<C, D, NW> vacc;    // sum_l (Gam * K K_l^T)_{i<t} W_l       [t][f]
  Acc<D, C, NW> oacc;    // O_loc^T                              [f][t]
  Acc<D, D, NW> hacc;    // H                                    [r][n]
  vacc.zero();
  oacc.zero();
  hacc.zero();
  {
    E* Klr = reinterpret_cast<E*>(smem + LY::B_KLR);
    E* KltD = reinterpret_cast<E*>(smem + LY::B_KLTD);
    E* Wlt = reinterpret_cast<E*>(smem + LY::B_WLT);
    E* F = reinterpret_cast<E*>(smem + LY::B_F);
    E* Rl = reinterpret_cast<E*>(smem + LY::B_RL);
    for (int l = 0; l < L; ++l) {
      kn.store_rows(Klr, LR, tid);
      kn.store_transposed(KltD, LT, Dv, tid);
      wn.store_transposed(Wlt, LT, nullptr, tid);
      __syncthreads();
      if (l + 1 < L) {   // next step's tiles are in flight during this step's products
        kn.load(Klb + (long)(l + 1) * Tp * D, D, C, tid);
        wn.load(Wlb + (long)(l + 1) * Tp * D, D, C, tid);
      }
      {
        Acc<C, C, NW> a;   // [i][t] = K_l,i . K_t  ->  F[t][i], i < t
        a.zero();
        gemm_acc<E, C, C, D, NW, true, true>(a, Klr, LR, Kr, LR, wave, lane);
        for_tiles(a, wave, lane, [&](int i0, int t, const f32x4& x) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int i = i0 + r;
            F[t * LT + i] = to_t<E>(i < t ? __expf(g[t] - g[i]) * x[r] : 0.f);
          }
        });
        if constexpr (!BWD) {
          Acc<C, C, NW> p;   // [i][t] = K_l,i . Q_t  ->  R_l[t][i], i <= t
          p.zero();
          gemm_acc<E, C, C, D, NW, true, true>(p, Klr, LR, Qr, LR, wave, lane);
          for_tiles(p, wave, lane, [&](int i0, int t, const f32x4& x) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int i = i0 + r;
              Rl[t * LT + i] = to_t<E>(i <= t ? __expf(g[t] - g[i]) * x[r] : 0.f);
            }
          });
        }
      }
      __syncthreads();
      gemm_acc<E, C, D, C, NW, true, true>(vacc, F, LT, Wlt, LT, wave, lane);
      if constexpr (!BWD) gemm_acc<E, D, C, C, NW, true, true>(oacc, Wlt, LT, Rl, LT, wave, lane);
      gemm_acc<E, D, D, C, NW, true, true>(hacc, Wlt, LT, KltD, LT, wave, lane);
      __syncthreads();
    }
  }

  // ---- phase T: A = diag(beta) (Gam * K K^T)_{i<t};  T = (I + A)^{-1} ----
  RegTile<E, C, D, NT> vn;   // V rows, in flight during the solve
  vn.load(vc, ts, nval, tid);
  E* Tb = reinterpret_cast<E*>(smem + LY::C_TB);
  {
    float* Af = reinterpret_cast<float*>(smem + LY::T_AF);
    float* Tf = reinterpret_cast<float*>(smem + LY::T_TF);
    float* Xs = reinterpret_cast<float*>(smem + LY::T_XS);
    Acc<C, C, NW> a;   // [t][i] = K_t . K_i
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
    invert_unit_lower<C, NW>(Af, Tf, Xs, tid);
    for (int e = tid; e < C * C; e += NT) Tb[(e / C) * LT + (e % C)] = to_t<E>(Tf[(e / C) * LA + (e % C)]);
    __syncthreads();
  }

  // ---- phase C ----
  E* Ktbe = reinterpret_cast<E*>(smem + LY::C_KTBE);   // (beta e K)^T, later Wk^T
  E* KtD = reinterpret_cast<E*>(smem + LY::C_KTD);     // (D K)^T
  E* Vt = reinterpret_cast<E*>(smem + LY::C_VT);       // (beta V')^T, later U^T / Qt^T
  E* R0 = reinterpret_cast<E*>(smem + LY::C_R0);
  E* Vr = reinterpret_cast<E*>(smem + LY::C_V);        // V rows, later dO^T
  for (int e = tid; e < C * D; e += NT) {
    const int t = e / D, f = e % D;
    const float kv = to_f(Kr[t * LR + f]);
    Ktbe[f * LT + t] = to_t<E>(be[t] * kv);
    KtD[f * LT + t] = to_t<E>(Dv[t] * kv);
  }
  vn.store_rows(Vr, LR, tid);
  RegTile<E, C, D, NT, true> on;   // dO rows (backward mode), in flight during the products below
  if constexpr (BWD) on.load(dO + row0 * D, ts, nval, tid);
  // the next chunk's first operands are fetched during the rest of this one
  // (issued after every load this chunk still waits for: loads complete in
  // order)
  if constexpr (PERSIST) {
    if (vid + vstride < nblk) prefetch(vid + vstride);
  }
  __syncthreads();
  for_tiles(vacc, wave, lane, [&](int t0, int f, const f32x4& x) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = t0 + r;
      Vt[f * LT + t] = to_t<E>(bt[t] * (to_f(Vr[t * LR + f]) - x[r]));
    }
  });
  __syncthreads();
  {
    Acc<C, D, NW> ua, wa;   // U[t][f], Wk[t][f]
    ua.zero();
    wa.zero();
    gemm_acc<E, C, D, C, NW, true, true>(ua, Tb, LT, Vt, LT, wave, lane);
    gemm_acc<E, C, D, C, NW, true, true>(wa, Tb, LT, Ktbe, LT, wave, lane);
    __syncthreads();
    for_tiles(ua, wave, lane, [&](int t0, int f, const f32x4& x) {
#pragma unroll
      for (int r = 0; r < 4; ++r) Vt[f * LT + t0 + r] = to_t<E>(x[r]);
    });
    for_tiles(wa, wave, lane, [&](int t0, int f, const f32x4& x) {
#pragma unroll
      for (int r = 0; r < 4; ++r) Ktbe[f * LT + t0 + r] = to_t<E>(x[r]);
    });
  }
  __syncthreads();
  E* Ut = Vt;
  E* Wkt = Ktbe;
  const long cidx = (long)bh * NC + c;
  if (UTo) {   // U^T, Wk^T [D][C] for the reverse chunk kernels (backward mode, training forward)
    s2g_rows<E, D, C, NT>(UTo + cidx * D * C, C, Ut, LT, D, tid);
    s2g_rows<E, D, C, NT>(WkTo + cidx * D * C, C, Wkt, LT, D, tid);
  }

  // H += U^T diag(D) K;  stored transposed (HT[n][r])
  gemm_acc<E, D, D, C, NW, true, true>(hacc, Ut, LT, KtD, LT, wave, lane);
  {
    float* HTc = HT + cidx * D * D;
    for_tiles(hacc, wave, lane, [&](int r0, int n, const f32x4& x) {
      *reinterpret_cast<f32x4*>(HTc + (long)n * D + r0) = x;
    });
  }
  {
    Acc<D, D, NW> ma;   // [k][n] = sum_t Wk[t][k] D_t K[t][n] = M[k][n]  -> stored as Mt[n][k]
    ma.zero();
    gemm_acc<E, D, D, C, NW, true, true>(ma, Wkt, LT, KtD, LT, wave, lane);
    E* Mtc = Mt + cidx * D * D;
    for_tiles(ma, wave, lane, [&](int k0, int n, const f32x4& x) {
#pragma unroll
      for (int r = 0; r < 4; ++r) Mtc[(long)n * D + k0 + r] = to_t<E>(x[r]);
    });
  }
  {
    Acc<C, C, NW> a;   // [i][t] = K_i . Q_t  ->  R0[t][i], i <= t
    a.zero();
    gemm_acc<E, C, C, D, NW, true, true>(a, Kr, LR, Qr, LR, wave, lane);
    for_tiles(a, wave, lane, [&](int i0, int t, const f32x4& x) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = i0 + r;
        R0[t * LT + i] = to_t<E>(i <= t ? __expf(g[t] - g[i]) * x[r] : 0.f);
      }
    });
  }
  __syncthreads();
  if constexpr (!BWD) {
    Acc<D, C, NW> qa;   // [f][t] = sum_i Wk[i][f] R0[t][i]
    qa.zero();
    gemm_acc<E, D, C, C, NW, true, true>(qa, Wkt, LT, R0, LT, wave, lane);
    E* Qtc = Qt + cidx * C * D;
    for_tiles(qa, wave, lane, [&](int f0, int t, const f32x4& x) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        Qtc[(long)t * D + f0 + r] = to_t<E>(ev[t] * to_f(Qr[t * LR + f0 + r]) - x[r]);
    });
    gemm_acc<E, D, C, C, NW, true, true>(oacc, Ut, LT, R0, LT, wave, lane);
    float* Oc = Oloc + cidx * C * D;
    for_tiles(oacc, wave, lane, [&](int f0, int t, const f32x4& x) {
      *reinterpret_cast<f32x4*>(Oc + (long)t * D + f0) = x;
    });
  } else {
    Acc<C, D, NW> qa;   // [t][f] = sum_i R0[t][i] Wk[i][f]  ->  Qt^T[f][t]
    qa.zero();
    gemm_acc<E, C, D, C, NW, true, true>(qa, R0, LT, Wkt, LT, wave, lane);
    E* Qtt = Vt;        // U^T is dead in backward mode once H is done
    for_tiles(qa, wave, lane, [&](int t0, int f, const f32x4& x) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = t0 + r;
        Qtt[f * LT + t] = to_t<E>(ev[t] * to_f(Qr[t * LR + f]) - x[r]);
      }
    });
    E* dOt = Vr;
    on.store_transposed(dOt, LT, nullptr, tid);
    __syncthreads();
    Acc<D, D, NW> ea;   // E[r][n] = sum_t dO[t][r] Qt[t][n]  -> stored as ET[n][r]
    ea.zero();
    gemm_acc<E, D, D, C, NW, true, true>(ea, dOt, LT, Qtt, LT, wave, lane);
    float* ETc = ET + cidx * D * D;
    for_tiles(ea, wave, lane, [&](int r0, int n, const f32x4& x) {
      *reinterpret_cast<f32x4*>(ETc + (long)n * D + r0) = x;
    });
  }
  if constexpr (!PERSIST) break;
  __syncthreads();   // LDS is reused by the next chunk
  }
}

// ET[n][r] = sum_t Qt[t][n] dO[t][r] per chunk (fp32 [D][D]), from the Qt a
// training forward kept: the reverse state pass's additive term.
template <typename E, int D, int C>
__global__ __launch_bounds__(CF_NT) void et_kernel(const E* __restrict__ Qt, const E* __restrict__ dO,
                                                   float* __restrict__ ET, int B, int T, int H, int NC,
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
  float* ETc = ET + cidx * D * D;
  for_tiles(ea, wave, lane, [&](int n0, int r, const f32x4& x) {
#pragma unroll
    for (int i = 0; i < 4; ++i) ETc[(long)(n0 + i) * D + r] = x[i];
  });
}

template <typename E, int D, int C>
static hipError_t et_launch_dc(const Dims& d, const E* Qt, const E* dO, float* ET, hipStream_t s) {
  if constexpr (sizeof(E) == 4 && D * C > 2048) return hipErrorInvalidValue;   // fp32 envelope
  hipLaunchKernelGGL((et_kernel<E, D, C>), dim3(d.B * d.H * d.NC), dim3(CF_NT), 0, s, Qt, dO, ET,
                     d.B, d.T, d.H, d.NC, d.cu);
  return hipGetLastError();
}

template <typename E, int D>
static hipError_t et_launch_d(const Dims& d, const E* Qt, const E* dO, float* ET, hipStream_t s) {
  switch (d.C) {
    case 16: return et_launch_dc<E, D, 16>(d, Qt, dO, ET, s);
    case 32: return et_launch_dc<E, D, 32>(d, Qt, dO, ET, s);
    case 64: return et_launch_dc<E, D, 64>(d, Qt, dO, ET, s);
  }
  return hipErrorInvalidValue;
}

template <typename E>
hipError_t launch_et(const Dims& d, const E* Qt, const E* dO, float* ET, hipStream_t s) {
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
template hipError_t launch_et<bf16>(const Dims&, const bf16*, const bf16*, float*, hipStream_t);
template hipError_t launch_et<float>(const Dims&, const float*, const float*, float*, hipStream_t);

template <typename E, int D, int C>
static hipError_t chunk_launch_dc(const Dims& d, const E* q, const E* k, const E* v,
                                  const float* alpha, const float* beta, const E* Kl, const E* Wl,
                                  const E* dO, E* Mt, float* HT, E* Qt, float* Oloc, float* gC,
                                  float* ET, E* UT, E* WkT, hipStream_t s) {
  if constexpr (sizeof(E) == 4 && D * C > 2048) return hipErrorInvalidValue;   // fp32 envelope
  const int nblk = d.B * d.H * d.NC;
  if (dO)
    hipLaunchKernelGGL((chunk_fwd_kernel<E, D, C, true>),
                       dim3(D >= 128 ? persistent_grid(chunk_fwd_kernel<E, D, C, true>, CF_NT, nblk) : nblk),
                       dim3(CF_NT), 0, s, q, k, v, alpha, beta, Kl, Wl, dO, Mt, HT, Qt, Oloc, gC,
                       ET, UT, WkT, d.B, d.T, d.H, d.L, d.NC, d.Tp, d.cu);
  else
    hipLaunchKernelGGL((chunk_fwd_kernel<E, D, C, false>),
                       dim3(D >= 128 ? persistent_grid(chunk_fwd_kernel<E, D, C, false>, CF_NT, nblk) : nblk),
                       dim3(CF_NT), 0, s, q, k, v, alpha, beta, Kl, Wl, dO, Mt, HT, Qt, Oloc, gC,
                       ET, UT, WkT, d.B, d.T, d.H, d.L, d.NC, d.Tp, d.cu);
  return hipGetLastError();
}

template <typename E, int D>
static hipError_t chunk_launch_d(const Dims& d, const E* q, const E* k, const E* v,
                                 const float* alpha, const float* beta, const E* Kl, const E* Wl,
                                 const E* dO, E* Mt, float* HT, E* Qt, float* Oloc, float* gC,
                                 float* ET, E* UT, E* WkT, hipStream_t s) {
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
                            float* HT, E* Qt, float* Oloc, float* gC, float* ET, E* UT,
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
                                           const bf16*, bf16*, float*, bf16*, float*, float*,
                                           float*, bf16*, bf16*, hipStream_t);
template hipError_t launch_chunk_fwd<float>(const Dims&, const float*, const float*, const float*,
                                            const float*, const float*, const float*, const float*,
                                            const float*, float*, float*, float*, float*, float*,
                                            float*, float*, float*, hipStream_t);

}  // namespace prism
