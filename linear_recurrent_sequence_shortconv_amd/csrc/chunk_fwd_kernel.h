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
// and the accumulators stay fp32.  Stored (global, per chunk, in the storage
// type E unless noted):
//   Mt [D][D] = M^T (MFMA B operand of the state pass, both directions; in
//              fragment order for bf16 at D >= 32, see mt_frag_order),
//   HT [D][D] = H^T, Qt [C][D], O_loc [C][D], gC (fp32), and when asked
//   (training forward) U^T, Wk^T [D][C] for the reverse chunk kernels.
// In backward mode (dO given) the kernel instead stores Mt, HT, gC,
// ET = (dO^T Qt)^T (for the reverse state pass) and U^T, Wk^T.
// After a training forward the reverse state pass forms E from the kept Qt.
//
// Fused form (FUSE): the refinement pairs K_l, W_l are formed inside the
// kernel from the chunk's v rows (and the 3 or 4 rows before it that the
// ShortConv taps reach) instead of being read back from HBM: the anchor,
// the two projections per step on MFMA, the activation chain and the step
// gates, in the same arithmetic and rounding as the separate refinement
// kernel, so both forms give the same bits.
#pragma once
#include <type_traits>
#include <utility>

#include "prism_common.h"
#include "prism_internal.h"

namespace prism {

constexpr int CF_NW = 8;
constexpr int CF_NT = CF_NW * WAVE;
constexpr int FUSE_LMAX = 8;   // refinement steps the fused kernel's LDS is sized for

template <typename E, int D, int C, bool FUSE = false, int HL = 3>
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
  // phase B (per refinement step); the fused form keeps K_l transposed
  static constexpr int SZ_KL = FUSE ? cmax(SZ_R, SZ_T) : SZ_R;
  static constexpr int B_KLR = O_X;
  static constexpr int B_KLTD = B_KLR + SZ_KL;
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
  // refinement formed in the kernel (phase B): anchor u (bf16: hi and lo
  // parts), step gates, w_beta rows; the v rows of the chunk and its halo
  // share the K_l^T D region, which is free until the first K_l is written
  static constexpr int SZ_U = FUSE ? SZ_R : 0;
  static constexpr int F_U = B_END;
  static constexpr int F_UL = F_U + SZ_U;
  static constexpr int F_G = F_UL + (sizeof(E) == 2 ? SZ_U : 0);
  static constexpr int F_WB = F_G + (FUSE ? FUSE_LMAX * C * 4 : 0);
  static constexpr int F_END = F_WB + (FUSE ? FUSE_LMAX * D * (int)sizeof(E) : 0);
  static constexpr int F_V = B_KLTD;
  static_assert(!FUSE || (C + HL) * D <= D * LT, "v rows and halo fit the K_l^T region");
  static constexpr int TOTAL = cmax(cmax(B_END, F_END), C_END);
};

template <typename E, int D, int C, bool BWD, bool FUSE, int ACT, int OFF>
__global__ __launch_bounds__(CF_NT) void chunk_fwd_kernel(
    const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ v,
    const float* __restrict__ alpha, const float* __restrict__ beta, const E* __restrict__ Kl,
    const E* __restrict__ Wl, const E* __restrict__ dO, E* __restrict__ Mt, E* __restrict__ HT,
    E* __restrict__ Qt, E* __restrict__ Oloc, float* __restrict__ gCo,
    E* __restrict__ ET, E* __restrict__ UTo, E* __restrict__ WkTo, int B, int T, int H, int L,
    int NC, int Tp, const int* __restrict__ cu, FuseIn<E> fz) {
  constexpr int HL = 3 + OFF;   // v rows before the chunk that the taps reach
  typedef ChunkLds<E, D, C, FUSE, HL> LY;
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
  // fused: v rows tb - HL .. tb + C - 1 of the next chunk (zeros past the
  // end; before 0 the history rows, or zeros without a history)
  constexpr int VN = 16 / (int)sizeof(E);
  constexpr int VPRW = D / VN;
  constexpr int VUN = FUSE ? (C + HL) * VPRW : 0;
  constexpr int VPER = FUSE ? (VUN + NT - 1) / NT : 1;
  uint4 vh[VPER];
  auto prefetch = [&](int vid) {
    const int bid = xcd_swizzle(vid, nblk);
    const int c = bid % NC, bh = bid / NC;
    const int h = bh % H, b = bh / H;
    const int tb = c * C;
    const int nval = min(C, seq_len(cu, b, T) - tb);
    const long row0 = (seq_start(cu, b, T) + tb) * H + h;
    if (!FUSE && wave == 0) {
      // separate-pair kernel: requested first (a wait for them then leaves
      // the tiles below in flight: vmcnt retires in issue order) and not under
      // a per-lane condition (lanes past the chunk's tokens read its last row
      // and take alpha = 1, beta = 0 at the use).  Requested last, and per
      // lane, their join waited for the whole prefetch; in the fused kernel
      // this order measured slower.
      if (nval > 0) {
        const long ab = row0 + (long)min(lane, nval - 1) * H;
        pa = alpha[ab];
        pb = beta[ab];
      }
    }
    if constexpr (FUSE) {
      const int Tb = seq_len(cu, b, T);
      const E* vs = v + (seq_start(cu, b, T) * H + h) * D;
      // (no load under a per-lane condition, whose merge made the wave wait
      // for it right after issue: rows outside the sequence and its history
      // read the chunk's own H^T block, and the store writes zeros for them)
      const E* fb = HT + ((long)bh * NC + c) * D * D;
#pragma unroll
      for (int p = 0; p < VPER; ++p) {
        const int u = min(tid + p * NT, VUN - 1);
        const int r = u / VPRW, cc = (u % VPRW) * VN;
        const int t = tb - HL + r;
        const bool in_seq = t >= 0 && t < Tb, in_hist = t < 0 && fz.hist;
        const E* src = in_seq ? vs + t * ts + cc
                     : in_hist ? fz.hist + (((long)b * 4 + 4 + t) * H + h) * D + cc : fb + cc;
        vh[p] = ld16(src);
      }
    } else if (L > 0) {
      kn.load(Kl + (long)bh * L * Tp * D + (long)tb * D, D, C, tid);
      wn.load(Wl + (long)bh * L * Tp * D + (long)tb * D, D, C, tid);
    }
    if constexpr (FUSE) {
      // (branch-free, as the v rows above; a chunk past a sequence's end
      // reads its H^T block, zeroed at the store)
      const E* fb = HT + ((long)bh * NC + c) * D * D;
      qn.load_nb(q + row0 * D, ts, nval, fb, tid);
      kr.load_nb(k + row0 * D, ts, nval, fb, tid);
    } else {
      qn.load(q + row0 * D, ts, nval, tid);
      kr.load(k + row0 * D, ts, nval, tid);
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

  // fused refinement: wave w owns feature tile fn = w mod NFT for the token
  // tiles mb, mb + WPF, ...; its weight fragments come straight from global
  // memory (L2), the anchor u is the shared MFMA A operand in LDS, and the
  // residual chain stays in registers in the accumulator layout:
  // element (j, i) is token 16 (mb + WPF j) + 4 (lane >> 4) + i, feature f
  typedef MfmaK<E, D> MK;
  typedef typename MK::frag Frag;
  constexpr int KS = MK::KSTEP;
  constexpr int NK = D / KS;
  constexpr int NFT = D / 16;
  static_assert(NW % NFT == 0, "feature tiles divide the waves");
  constexpr int WPF = NW / NFT;
  constexpr int MT = C / 16;
  constexpr int MPW = (MT + WPF - 1) / WPF;
  const int fn = wave % NFT, mb = wave / NFT;
  const int f = 16 * fn + (lane & 15);
  auto tile_ok = [&](int j) { return MT % WPF == 0 || mb + WPF * j < MT; };
  Frag bw[FUSE ? NK : 1];   // weight fragments of the next projection
  float tp[4];              // ShortConv taps of feature f
  uint4 wbn;                // w_beta rows (a vector per thread below L D / VN)
  auto load_w = [&](const E* W) {
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) bw[kk] = load_fragK<E, D>(W, D, 16 * fn, kk * KS, lane);
  };
  if constexpr (FUSE) {
    // Requested in the order they are waited for (vmcnt retires in issue
    // order): alpha and beta (wave 0; not prefetched with the next chunk's
    // tiles, where they made the wave wait for that whole prefetch, and not
    // under a per-lane condition: lanes past the chunk's tokens read its last
    // row) and the taps (before phase A's barrier), the w_beta rows (one
    // vector per thread, clamped rather than conditional; stored after the
    // anchor pass), then the W_p^(1) fragments (first used after the gates)
    if (wave == 0 && nval > 0) {
      const long ab = row0 + (long)min(lane, nval - 1) * H;
      pa = alpha[ab];
      pb = beta[ab];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) tp[j] = to_f(fz.conv[((long)h * D + f) * 4 + j]);
    static_assert(FUSE_LMAX * (D / VN) <= NT, "w_beta rows: one vector per thread");
    wbn = ld16(fz.wbeta + (long)h * L * D + (long)min(tid, L * VPRW - 1) * VN);
    load_w(fz.Wp + (long)h * L * D * D);   // W_p^(1)
    E* vb = reinterpret_cast<E*>(smem + LY::F_V);
    const int Tb = seq_len(cu, b, T);
#pragma unroll
    for (int p = 0; p < VPER; ++p) {
      const int u = tid + p * NT;
      if (u < VUN) {
        // zeros for the rows outside the sequence and its history (the empty
        // asm keeps the select here, not next to the load)
        const int t = tb - HL + u / VPRW;
        uint4 x = vh[p];
        asm volatile("" : "+v"(x.x), "+v"(x.y), "+v"(x.z), "+v"(x.w));
        if (!((t >= 0 && t < Tb) || (t < 0 && fz.hist))) x = uint4{0u, 0u, 0u, 0u};
        st16(vb + (u / VPRW) * D + (u % VPRW) * VN, x);
      }
    }
  }

  // ---- phase A: decays and gates; Q, K tiles ----
  if (wave == 0) {
    // alpha = 1, beta = 0 past the end
    const float lg = lane < nval ? logf(pa) : 0.f;
    const float bv = lane < nval ? pb : 0.f;
    const float s = wave_scan(lg);
    const float gC = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, s), C - 1));
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

  // ---- fused: anchor u_t = sum_j c_j v_{t-o-j} (to LDS, bf16 as hi + lo so
  //      that p^(l) = W_p^(l) u is fp32-accurate), residual r^(1) = v - u in
  //      registers, then the step gates sigmoid(w_beta^(l) . u_hi) ----
  float r[FUSE ? MPW : 1][4];
  if constexpr (FUSE) {
    const E* vb = reinterpret_cast<const E*>(smem + LY::F_V);   // row q: token tb - HL + q
    E* Ub = reinterpret_cast<E*>(smem + LY::F_U);
    E* Ul = reinterpret_cast<E*>(smem + LY::F_UL);
#pragma unroll
    for (int j = 0; j < MPW; ++j) {
      const int t0m = 16 * (mb + WPF * j) + 4 * (lane >> 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) r[j][i] = 0.f;
      if (tile_ok(j)) {
        // tap j of token t is buffer row t + 3 - j; the token itself row t + 3 + o
        float w[7 + OFF];
#pragma unroll
        for (int q = 0; q < 7 + OFF; ++q) w[q] = to_f(vb[(t0m + q) * D + f]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = t0m + i;
          float u = 0.f;
          if (t < nval) {
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) u += tp[jj] * w[i + 3 - jj];
            r[j][i] = w[i + 3 + OFF] - u;
          }
          const E uh = to_t<E>(u);
          Ub[t * LR + f] = uh;
          if constexpr (sizeof(E) == 2) Ul[t * LR + f] = to_t<E>(u - to_f(uh));
        }
      }
    }
    if (tid < L * VPRW) st16(reinterpret_cast<E*>(smem + LY::F_WB) + tid * VN, wbn);
    __syncthreads();
    // four threads per token (16-byte reads of u and w_beta, each thread a
    // fixed set of feature blocks in order); NT / 4C groups take the steps
    // round robin
    const E* wbs = reinterpret_cast<const E*>(smem + LY::F_WB);
    float* Gt = reinterpret_cast<float*>(smem + LY::F_G);
    constexpr int GG = NT / (4 * C);
    constexpr int KQ = (VPRW + 3) / 4;
    const int grp = tid / (4 * C), t = (tid % (4 * C)) >> 2, part = tid & 3;
    for (int l = grp; l < L; l += GG) {
      float s = 0.f;
#pragma unroll
      for (int kq = 0; kq < KQ; ++kq) {
        const int cc = (part + 4 * kq) * VN;
        if (VPRW % 4 == 0 || cc < D) {
          const uint4 ua = ld16(Ub + t * LR + cc), wa = ld16(wbs + l * D + cc);
          const E* ue = reinterpret_cast<const E*>(&ua);
          const E* we = reinterpret_cast<const E*>(&wa);
#pragma unroll
          for (int jj = 0; jj < VN; ++jj) s += to_f(we[jj]) * to_f(ue[jj]);
        }
      }
      s = quad_sum(s);
      if (part == 0) Gt[l * C + t] = sigmoidf(s);
    }
  }
  // p^(l) = W_p (u_hi + u_lo) or k^(l) = W_k u_hi for the wave's tiles
  auto fgemm = [&](bool with_lo, f32x4 (&acc)[FUSE ? MPW : 1]) {
    const E* Ub = reinterpret_cast<const E*>(smem + LY::F_U);
    const E* Ul = reinterpret_cast<const E*>(smem + LY::F_UL);
#pragma unroll
    for (int j = 0; j < MPW; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
      Frag a[MPW];
#pragma unroll
      for (int j = 0; j < MPW; ++j)
        if (tile_ok(j)) a[j] = load_fragK<E, D>(Ub, LR, 16 * (mb + WPF * j), kk * KS, lane);
#pragma unroll
      for (int j = 0; j < MPW; ++j)
        if (tile_ok(j)) acc[j] = MK::mma(a[j], bw[kk], acc[j]);
      if constexpr (sizeof(E) == 2) {
        if (with_lo) {
#pragma unroll
          for (int j = 0; j < MPW; ++j)
            if (tile_ok(j)) a[j] = load_fragK<E, D>(Ul, LR, 16 * (mb + WPF * j), kk * KS, lane);
#pragma unroll
          for (int j = 0; j < MPW; ++j)
            if (tile_ok(j)) acc[j] = MK::mma(a[j], bw[kk], acc[j]);
        }
      }
    }
  };

  // Decays Gam_ti = exp(g_t - g_i) (i <= t, else 0) at this wave's positions
  // of the C x C products that are rows i, column t (F_l, R_l of every step
  // and R0): formed once per chunk and kept in registers by the separate-pair
  // kernel; the fused kernel, at its register limit, forms them per product.
  typedef Tiling<C, C, NW> TLC;
  constexpr bool GAMC = !FUSE;
  f32x4 gamc[GAMC ? TLC::RM : 1][GAMC ? TLC::RN : 1];
  if constexpr (GAMC) {
    if (TLC::active(wave)) {
#pragma unroll
      for (int i = 0; i < TLC::RM; ++i)
#pragma unroll
        for (int j = 0; j < TLC::RN; ++j) {
          const int i0 = TLC::m0(wave) + 16 * i + 4 * (lane >> 4), t = TLC::n0(wave) + 16 * j + (lane & 15);
#pragma unroll
          for (int r = 0; r < 4; ++r) gamc[i][j][r] = i0 + r <= t ? __expf(g[t] - g[i0 + r]) : 0.f;
        }
    }
  }
  auto gam_at = [&](int i, int j, int i0, int t, int r) -> float {
    if constexpr (GAMC) return gamc[i][j][r];
    else return i0 + r <= t ? __expf(g[t] - g[i0 + r]) : 0.f;
  };
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
      if constexpr (FUSE) {
        // delta = act(p * r), r -= delta, w = beta^(l) delta  -> W_l^T;
        // k^(l) -> K_l rows and (D K_l)^T.  The next projection's weight
        // fragments are requested before each pass's arithmetic.
        const float* Gt = reinterpret_cast<const float*>(smem + LY::F_G);
        f32x4 acc[MPW];
        fgemm(true, acc);                                 // p^(l)
        load_w(fz.Wk + ((long)h * L + l) * D * D);        // W_k^(l)
        if (l == 0) __syncthreads();                      // step gates visible
#pragma unroll
        for (int j = 0; j < MPW; ++j) {
          if (!tile_ok(j)) continue;
          const int t0m = 16 * (mb + WPF * j) + 4 * (lane >> 4);
          E wv[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float z = acc[j][i] * r[j][i];
            float dl;
            if constexpr (ACT == ACT_IDENTITY) dl = z;
            else dl = gelu_erf(z);
            r[j][i] -= dl;
            wv[i] = to_t<E>(Gt[l * C + t0m + i] * dl);
          }
          st4(Wlt + f * LT + t0m, wv);
        }
        fgemm(false, acc);                                // k^(l)
        if (l + 1 < L) load_w(fz.Wp + ((long)h * L + l + 1) * D * D);   // W_p^(l+1)
#pragma unroll
        for (int j = 0; j < MPW; ++j) {
          if (!tile_ok(j)) continue;
          const int t0m = 16 * (mb + WPF * j) + 4 * (lane >> 4);
          E kb[4], kd[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            kb[i] = to_t<E>(acc[j][i]);
            kd[i] = to_t<E>(to_f(kb[i]) * Dv[t0m + i]);
          }
          st4(Klr + f * LT + t0m, kb);   // K_l^T
          st4(KltD + f * LT + t0m, kd);
        }
      } else {
        kn.store_rows(Klr, LR, tid);
        kn.store_transposed(KltD, LT, Dv, tid);
        wn.store_transposed(Wlt, LT, nullptr, tid);
      }
      __syncthreads();
      if constexpr (!FUSE) {
        {   // next step's tiles are in flight during this step's products (the
            // last step reads its own again: unconditional loads leave no
            // register merge, whose copies would wait for every load in flight)
          const long nl = l + 1 < L ? l + 1 : l;
          kn.load(Klb + nl * Tp * D, D, C, tid);
          wn.load(Wlb + nl * Tp * D, D, C, tid);
        }
      }
      {
        Acc<C, C, NW> a;   // [i][t] = K_l,i . K_t  ->  F[t][i], i < t
        a.zero();
        if constexpr (FUSE) gemm_acc<E, C, C, D, NW, false, true, !FUSE>(a, Klr, LT, Kr, LR, wave, lane);
        else gemm_acc<E, C, C, D, NW, true, true, !FUSE>(a, Klr, LR, Kr, LR, wave, lane);
        for_tiles_ij(a, wave, lane, [&](int i, int j, int i0, int t, const f32x4& x) {
          E w[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) w[r] = to_t<E>(i0 + r < t ? gam_at(i, j, i0, t, r) * x[r] : 0.f);
          st4(F + t * LT + i0, w);
        });
        if constexpr (!BWD) {
          Acc<C, C, NW> p;   // [i][t] = K_l,i . Q_t  ->  R_l[t][i], i <= t
          p.zero();
          if constexpr (FUSE) gemm_acc<E, C, C, D, NW, false, true, !FUSE>(p, Klr, LT, Qr, LR, wave, lane);
          else gemm_acc<E, C, C, D, NW, true, true, !FUSE>(p, Klr, LR, Qr, LR, wave, lane);
          for_tiles_ij(p, wave, lane, [&](int i, int j, int i0, int t, const f32x4& x) {
            E w[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) w[r] = to_t<E>(gam_at(i, j, i0, t, r) * x[r]);
            st4(Rl + t * LT + i0, w);
          });
        }
      }
      __syncthreads();
      gemm_acc<E, C, D, C, NW, true, true, !FUSE>(vacc, F, LT, Wlt, LT, wave, lane);
      if constexpr (!BWD) gemm_acc<E, D, C, C, NW, true, true, !FUSE>(oacc, Wlt, LT, Rl, LT, wave, lane);
      gemm_acc<E, D, D, C, NW, true, true, !FUSE>(hacc, Wlt, LT, KltD, LT, wave, lane);
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
    gemm_acc<E, C, C, D, NW, true, true, !FUSE>(a, Kr, LR, Kr, LR, wave, lane);
    for_tiles(a, wave, lane, [&](int t0, int i, const f32x4& x) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = t0 + r;
        Af[t * LA + i] = i < t ? bt[t] * __expf(g[t] - g[i]) * x[r] : 0.f;
      }
    });
    __syncthreads();
    // (the wide instances read the diagonal blocks' rows further ahead: their
    // registers peak elsewhere)
    invert_unit_lower<C, NW, !FUSE, (D >= 128 && C >= 64) ? INV_PD : 1>(Af, Tf, Xs, tid);
    // T in the operand type: column pairs, one 2-element store each
    constexpr int NPR = C * C / 2, PPR = (NPR + NT - 1) / NT;
#pragma unroll
    for (int k = 0; k < PPR; ++k) {
      const int e = tid + k * NT;
      if (NPR % NT == 0 || e < NPR) {
        const int t = e / (C / 2), i = 2 * (e % (C / 2));
        st2f(Tb + t * LT + i, Tf[t * LA + i], Tf[t * LA + i + 1]);
      }
    }
    __syncthreads();
  }

  // ---- phase C ----
  E* Ktbe = reinterpret_cast<E*>(smem + LY::C_KTBE);   // (beta e K)^T, later Wk^T
  E* KtD = reinterpret_cast<E*>(smem + LY::C_KTD);     // (D K)^T
  E* Vt = reinterpret_cast<E*>(smem + LY::C_VT);       // (beta V')^T, later U^T / Qt^T
  E* R0 = reinterpret_cast<E*>(smem + LY::C_R0);
  E* Vr = reinterpret_cast<E*>(smem + LY::C_V);        // V rows, later dO^T
  {
    // (beta e K)^T and (D K)^T from the K rows: row pairs read as 16-byte
    // pieces, written transposed as one 32-bit word per column (no bank
    // conflicts; an element-wise transposition wrote 2 bytes at a time to
    // addresses 8 banks apart)
    RegTile<E, C, D, NT, true> kt;
    kt.load(Kr, LR, C, tid);
    kt.store_transposed(Ktbe, LT, be, tid);
    kt.store_transposed(KtD, LT, Dv, tid);
  }
  vn.store_rows(Vr, LR, tid);
  RegTile<E, C, D, NT, true> on;   // dO rows (backward mode), in flight during the products below
  if constexpr (BWD) on.load(dO + row0 * D, ts, nval, tid);
  // the next chunk's first operands are fetched during the rest of this one
  // (issued after every load this chunk still waits for: loads complete in
  // order)
  if constexpr (PERSIST) {
    // (the fused kernel prefetches unconditionally, the last chunk again past
    // the end: the join of a conditional prefetch made the wave wait for it
    // right after issue)
    if (FUSE || vid + vstride < nblk) prefetch(FUSE ? min(vid + vstride, nblk - 1) : vid + vstride);
  }
  __syncthreads();
  for_tiles(vacc, wave, lane, [&](int t0, int f, const f32x4& x) {
    E w[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = t0 + r;
      w[r] = to_t<E>(bt[t] * (to_f(Vr[t * LR + f]) - x[r]));
    }
    st4(Vt + f * LT + t0, w);   // four consecutive tokens: one 8-byte write
  });
  __syncthreads();
  {
    Acc<C, D, NW> ua, wa;   // U[t][f], Wk[t][f]
    ua.zero();
    wa.zero();
    gemm_acc<E, C, D, C, NW, true, true, !FUSE>(ua, Tb, LT, Vt, LT, wave, lane);
    gemm_acc<E, C, D, C, NW, true, true, !FUSE>(wa, Tb, LT, Ktbe, LT, wave, lane);
    __syncthreads();
    for_tiles(ua, wave, lane, [&](int t0, int f, const f32x4& x) { st4f(Vt + f * LT + t0, x); });
    for_tiles(wa, wave, lane, [&](int t0, int f, const f32x4& x) { st4f(Ktbe + f * LT + t0, x); });
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
  gemm_acc<E, D, D, C, NW, true, true, !FUSE>(hacc, Ut, LT, KtD, LT, wave, lane);
  {
    E* HTc = HT + cidx * D * D;
    for_tiles(hacc, wave, lane, [&](int r0, int n, const f32x4& x) {
      st_f4(HTc + (long)n * D + r0, x);
    });
  }
  {
    Acc<D, D, NW> ma;   // [k][n] = sum_t Wk[t][k] D_t K[t][n] = M[k][n]  -> stored as Mt[n][k]
    ma.zero();
    gemm_acc<E, D, D, C, NW, true, true, !FUSE>(ma, Wkt, LT, KtD, LT, wave, lane);
    E* Mtc = Mt + cidx * D * D;
    for_tiles(ma, wave, lane, [&](int k0, int n, const f32x4& x) {
      if constexpr (mt_frag_order<E, D>()) {
        // fragment order: k0 .. k0 + 3 are adjacent in one 16-byte piece
        E w[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) w[r] = to_t<E>(x[r]);
        st4(Mtc + frag_order_offset<E, D>(n, k0), w);
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) Mtc[(long)n * D + k0 + r] = to_t<E>(x[r]);
      }
    });
  }
  {
    Acc<C, C, NW> a;   // [i][t] = K_i . Q_t  ->  R0[t][i], i <= t
    a.zero();
    gemm_acc<E, C, C, D, NW, true, true, !FUSE>(a, Kr, LR, Qr, LR, wave, lane);
    for_tiles_ij(a, wave, lane, [&](int i, int j, int i0, int t, const f32x4& x) {
      E w[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) w[r] = to_t<E>(gam_at(i, j, i0, t, r) * x[r]);
      st4(R0 + t * LT + i0, w);
    });
  }
  __syncthreads();
  if constexpr (!BWD) {
    Acc<D, C, NW> qa;   // [f][t] = sum_i Wk[i][f] R0[t][i]
    qa.zero();
    gemm_acc<E, D, C, C, NW, true, true, !FUSE>(qa, Wkt, LT, R0, LT, wave, lane);
    E* Qtc = Qt + cidx * C * D;
    for_tiles(qa, wave, lane, [&](int f0, int t, const f32x4& x) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        Qtc[(long)t * D + f0 + r] = to_t<E>(ev[t] * to_f(Qr[t * LR + f0 + r]) - x[r]);
    });
    gemm_acc<E, D, C, C, NW, true, true, !FUSE>(oacc, Ut, LT, R0, LT, wave, lane);
    E* Oc = Oloc + cidx * C * D;
    for_tiles(oacc, wave, lane, [&](int f0, int t, const f32x4& x) {
      st_f4(Oc + (long)t * D + f0, x);
    });
  } else {
    Acc<C, D, NW> qa;   // [t][f] = sum_i R0[t][i] Wk[i][f]  ->  Qt^T[f][t]
    qa.zero();
    gemm_acc<E, C, D, C, NW, true, true, !FUSE>(qa, R0, LT, Wkt, LT, wave, lane);
    E* Qtt = Vt;        // U^T is dead in backward mode once H is done
    for_tiles(qa, wave, lane, [&](int t0, int f, const f32x4& x) {
      E w[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = t0 + r;
        w[r] = to_t<E>(ev[t] * to_f(Qr[t * LR + f]) - x[r]);
      }
      st4(Qtt + f * LT + t0, w);
    });
    E* dOt = Vr;
    on.store_transposed(dOt, LT, nullptr, tid);
    __syncthreads();
    Acc<D, D, NW> ea;   // E[r][n] = sum_t dO[t][r] Qt[t][n]  -> stored as ET[n][r]
    ea.zero();
    gemm_acc<E, D, D, C, NW, true, true, !FUSE>(ea, dOt, LT, Qtt, LT, wave, lane);
    E* ETc = ET + cidx * D * D;
    for_tiles(ea, wave, lane, [&](int r0, int n, const f32x4& x) {
      st_f4(ETc + (long)n * D + r0, x);
    });
  }
  if constexpr (!PERSIST) break;
  __syncthreads();   // LDS is reused by the next chunk
  }
}

template <typename E, int D, int C, bool BWD, bool FUSE, int ACT, int OFF>
hipError_t chunk_launch_k(const Dims& d, const E* q, const E* k, const E* v, const float* alpha,
                          const float* beta, const E* Kl, const E* Wl, const E* dO, E* Mt,
                          E* HT, E* Qt, E* Oloc, float* gC, E* ET, E* UT, E* WkT,
                          const FuseIn<E>& fz, hipStream_t s) {
  if constexpr (sizeof(E) == 4 && D * C > 2048) {   // fp32 envelope
    return hipErrorInvalidValue;
  } else {
    auto kern = chunk_fwd_kernel<E, D, C, BWD, FUSE, ACT, OFF>;
    const int nblk = d.B * d.H * d.NC;
    hipLaunchKernelGGL(kern, dim3(D >= 128 ? persistent_grid(kern, CF_NT, nblk) : nblk),
                       dim3(CF_NT), 0, s, q, k, v, alpha, beta, Kl, Wl, dO, Mt, HT, Qt, Oloc, gC,
                       ET, UT, WkT, d.B, d.T, d.H, d.L, d.NC, d.Tp, d.cu, fz);
    return hipGetLastError();
  }
}

// The fused forward for one (activation, tap offset) variant; instantiated
// in chunk_fused_<activation>.hip.
template <typename E, int ACT, int OFF>
hipError_t launch_chunk_fused_var(const Dims& d, const E* q, const E* k, const E* v,
                                  const float* alpha, const float* beta, const FuseIn<E>& fz,
                                  E* Mt, E* HT, E* Qt, E* Oloc, float* gC,
                                  hipStream_t s) {
  auto go = [&](auto dc) -> hipError_t {
    constexpr int D = decltype(dc)::first_type::value, C = decltype(dc)::second_type::value;
    if constexpr (sizeof(E) == 4 && D > 64) {
      return hipErrorInvalidValue;
    } else {
      return chunk_launch_k<E, D, C, false, true, ACT, OFF>(
          d, q, k, v, alpha, beta, nullptr, nullptr, nullptr, Mt, HT, Qt, Oloc, gC, nullptr,
          nullptr, nullptr, fz, s);
    }
  };
  auto byc = [&](auto dd) -> hipError_t {
    typedef decltype(dd) DI;
    switch (d.C) {
      case 16: return go(std::pair<DI, std::integral_constant<int, 16>>());
      case 32: return go(std::pair<DI, std::integral_constant<int, 32>>());
      case 64: return go(std::pair<DI, std::integral_constant<int, 64>>());
    }
    return hipErrorInvalidValue;
  };
  switch (d.D) {
    case 16: return byc(std::integral_constant<int, 16>());
    case 32: return byc(std::integral_constant<int, 32>());
    case 64: return byc(std::integral_constant<int, 64>());
    case 128: return byc(std::integral_constant<int, 128>());
  }
  return hipErrorInvalidValue;
}

#define PRISM_CHUNK_FUSED_VARIANT(E, ACT, OFF)                                                    \
  extern template hipError_t launch_chunk_fused_var<E, ACT, OFF>(                                \
      const Dims&, const E*, const E*, const E*, const float*, const float*, const FuseIn<E>&,  \
      E*, E*, E*, E*, float*, hipStream_t);
PRISM_CHUNK_FUSED_VARIANT(bf16, ACT_GELU, 0)
PRISM_CHUNK_FUSED_VARIANT(bf16, ACT_GELU, 1)
PRISM_CHUNK_FUSED_VARIANT(bf16, ACT_IDENTITY, 0)
PRISM_CHUNK_FUSED_VARIANT(bf16, ACT_IDENTITY, 1)
PRISM_CHUNK_FUSED_VARIANT(float, ACT_GELU, 0)
PRISM_CHUNK_FUSED_VARIANT(float, ACT_GELU, 1)
PRISM_CHUNK_FUSED_VARIANT(float, ACT_IDENTITY, 0)
PRISM_CHUNK_FUSED_VARIANT(float, ACT_IDENTITY, 1)
#undef PRISM_CHUNK_FUSED_VARIANT

}  // namespace prism
