// Chunk-parallel part of the PRISM backward pass: the adjoint of the chunk
// affine map (see chunk_fwd.hip)
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

namespace prism {

constexpr int CB_NW = 8;
constexpr int CB_NT = CB_NW * WAVE;

// ---------------------------------------------------------------------------
// shared helpers
// ---------------------------------------------------------------------------
// Decays of one chunk: g (cumulative log alpha), e = exp(g), Dv = exp(gC - g),
// bt = beta, be = beta e.  Padding tokens (t >= nval) have alpha = 1, beta = 0.
template <int C>
__device__ inline void chunk_decays(const float* alpha, const float* beta, long row0, int H,
                                    int nval, float* g, float* ev, float* Dv, float* bt, float* be,
                                    float* ai, int lane) {
  float lg = 0.f, bv = 0.f, a = 1.f;
  if (lane < nval) {
    a = alpha[row0 + (long)lane * H];
    lg = logf(a);
    if (beta) bv = beta[row0 + (long)lane * H];
  }
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
  // slot[row] += row sums (one wave's private slots)
  __device__ inline void flush_rows(float* slot, int m0, int lane) const {
#pragma unroll
    for (int i = 0; i < RM; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float s = r[i][q];
        s += __shfl_xor(s, 1);
        s += __shfl_xor(s, 2);
        s += __shfl_xor(s, 4);
        s += __shfl_xor(s, 8);
        if ((lane & 15) == 0) slot[m0 + 16 * i + 4 * (lane >> 4) + q] += s;
      }
  }
  __device__ inline void flush_cols(float* slot, int n0, int lane) const {
#pragma unroll
    for (int j = 0; j < RN; ++j) {
      float s = c[j];
      s += __shfl_xor(s, 16);
      s += __shfl_xor(s, 32);
      if (lane < 16) slot[n0 + 16 * j + lane] += s;
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

// ===========================================================================
// chunk_bwd_state
// ===========================================================================
template <typename E, int D, int C>
struct CB1Lds {
  static constexpr int LR = ldpad<E>(D);
  static constexpr int LD2 = ldpad<E>(D);
  static constexpr int SZ_R = C * LR * (int)sizeof(E);
  static constexpr int SZ_DD = D * LD2 * (int)sizeof(E);
  static constexpr int O_VEC = 0;                                  // g, e, Dv (3C) + slots
  static constexpr int SZ_VEC = (3 * C + CB_NW * C + CB_NW) * 4;
  static constexpr int O_X1 = (O_VEC + SZ_VEC + 15) / 16 * 16;     // S, then dS_n, then dM
  static constexpr int O_X2 = O_X1 + SZ_DD;                        // dS_n^T, then dM^T
  static constexpr int O_R1 = O_X2 + SZ_DD;                        // dO rows, then K rows
  static constexpr int O_R2 = O_R1 + SZ_R;                         // U rows
  static constexpr int O_R3 = O_R2 + SZ_R;                         // K_l rows, then Wk rows
  static constexpr int O_R4 = O_R3 + SZ_R;                         // W_l rows
  static constexpr int TOTAL = O_R4 + SZ_R;
};

template <typename E, int D, int C>
__global__ __launch_bounds__(CB_NT) void chunk_bwd_state_kernel(
    const E* __restrict__ k, const E* __restrict__ dO, const float* __restrict__ alpha,
    const E* __restrict__ Kl, const E* __restrict__ Wl, const E* __restrict__ UT,
    const E* __restrict__ WkT, const E* __restrict__ Sc, const E* __restrict__ dSnT,
    E* __restrict__ dQt, E* __restrict__ dUs, E* __restrict__ dWks,
    E* __restrict__ dKs, E* __restrict__ dKls, float* __restrict__ dWls,
    float* __restrict__ dgs, int B, int T, int H, int L, int NC, int Tp,
    const int* __restrict__ cu) {
  typedef CB1Lds<E, D, C> LY;
  constexpr int NW = CB_NW, NT = CB_NT;
  constexpr int LR = LY::LR, LD2 = LY::LD2;
  __shared__ __attribute__((aligned(16))) unsigned char smem[LY::TOTAL];
  float* g = reinterpret_cast<float*>(smem + LY::O_VEC);
  float* ev = g + C;
  float* Dv = g + 2 * C;
  float* ddw = g + 3 * C;            // [NW][C] per-wave row sums of dD
  float* sdw = ddw + NW * C;         // [NW] per-wave sums of S (.) dS_n
  E* X1 = reinterpret_cast<E*>(smem + LY::O_X1);
  E* X2 = reinterpret_cast<E*>(smem + LY::O_X2);
  E* R1 = reinterpret_cast<E*>(smem + LY::O_R1);
  E* R2 = reinterpret_cast<E*>(smem + LY::O_R2);
  E* R3 = reinterpret_cast<E*>(smem + LY::O_R3);
  E* R4 = reinterpret_cast<E*>(smem + LY::O_R4);

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

  for (int e = tid; e < NW * C + NW; e += NT) ddw[e] = 0.f;
  typedef Tiling<C, D, NW> TLS;
  TileSums<TLS::RM, TLS::RN> dds;   // row sums of the dD terms, over all products
  dds.zero();
  // the first phase's tiles (dO rows, S_c and dS_n^T, both row-major), all
  // requested before the first is stored (one memory round trip, which the
  // decays' reads share)
  {
    RegTile<E, C, D, NT> t_do;
    RegTile<E, D, D, NT> t_sc, t_dsnt;
    t_do.load(dO + row0 * D, ts, nval, tid);
    t_sc.load(Sc + cidx * D * D, D, D, tid);
    t_dsnt.load(dSnT + cidx * D * D, D, D, tid);
    if (wave == 0) chunk_decays<C>(alpha, nullptr, row0, H, nval, g, ev, Dv, nullptr, nullptr, nullptr, lane);
    t_do.store_rows(R1, LR, tid);
    t_sc.store_rows(X1, LD2, tid);
    t_dsnt.store_rows(X2, LD2, tid);
  }
  // tiles of the next phase, in flight during the first products: dS_n^T
  // again (stored transposed, i.e. dS_n row-major), K rows, U^T
  RegTile<E, D, D, NT, true> dsn;
  RegTile<E, C, D, NT> kr;
  RegTile<E, D, C, NT, true> ut;
  dsn.load(dSnT + cidx * D * D, D, D, tid);
  kr.load(k + row0 * D, ts, nval, tid);
  ut.load(UT + cidx * D * C, C, D, tid);
  __syncthreads();

  // ---- dQt = dO S  ([t][k] = sum_r dO[t][r] S[r][k]);  dM = -S^T dS_n ----
  // (X1 holds S row-major: both products read it k-strided)
  {
    Acc<C, D, NW> a;
    a.zero();
    gemm_acc<E, C, D, D, NW, true, false>(a, R1, LR, X1, LD2, wave, lane);
    E* out = dQt + cidx * C * D;
    for_tiles(a, wave, lane, [&](int t0, int kk, const f32x4& x) {
#pragma unroll
      for (int r = 0; r < 4; ++r) out[(long)(t0 + r) * D + kk] = to_t<E>(x[r]);
    });
  }
  Acc<D, D, NW> dm;   // [k][n] = sum_r S[r][k] dS_n^T[n][r]  (= -dM)
  dm.zero();
  gemm_acc<E, D, D, D, NW, false, true>(dm, X1, LD2, X2, LD2, wave, lane);
  {
    // sum over all entries of S (.) dS_n = sum_{r,c} S[r][c] dS_n[r][c]: the
    // trace of dm, taken from the diagonal of the accumulator tiles
    float s = 0.f;
    for_tiles(dm, wave, lane, [&](int k0, int n, const f32x4& x) {
#pragma unroll
      for (int r = 0; r < 4; ++r) s += k0 + r == n ? x[r] : 0.f;
    });
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
    if (lane == 0) sdw[wave] = s;
  }
  __syncthreads();

  // ---- dS_n (row-major) into X1; K and U rows ----
  dsn.store_transposed(X1, LD2, nullptr, tid);
  kr.store_rows(R1, LR, tid);
  ut.store_transposed(R2, LR, nullptr, tid);
  // the first refinement step's K_l, W_l rows and the Wk^T tile of the last
  // phase are fetched during the products below
  RegTile<E, C, D, NT> kl, wl;
  RegTile<E, D, C, NT, true> wkt;
  if (L > 0) {
    const long lrow = (long)bh * L * Tp + tb;
    kl.load(Kl + lrow * D, D, C, tid);
    wl.load(Wl + lrow * D, D, C, tid);
  }
  wkt.load(WkT + cidx * D * C, C, D, tid);
  __syncthreads();

  Acc<C, D, NW> dk;   // D-weighted dK:  D (U dS_n + Wk dM)
  dk.zero();
  {
    Acc<C, D, NW> a;    // U dS_n: [t][n] = sum_r U[t][r] dS_n^T[n][r]
    a.zero();
    gemm_acc<E, C, D, D, NW, true, true>(a, R2, LR, X2, LD2, wave, lane);
    for_tiles_mut(dk, wave, lane, [&](int, int, f32x4&) {});
    {
      typedef Tiling<C, D, NW> TL;
      if (TL::active(wave)) {
#pragma unroll
        for (int i = 0; i < TL::RM; ++i)
#pragma unroll
          for (int j = 0; j < TL::RN; ++j) {
            const int t0 = TL::m0(wave) + 16 * i + 4 * (lane >> 4);
#pragma unroll
            for (int r = 0; r < 4; ++r) dk.v[i][j][r] = Dv[t0 + r] * a.v[i][j][r];
          }
      }
    }
    Acc<C, D, NW> u;    // K dS_n^T: [t][r] = sum_n K[t][n] dS_n[r][n]
    u.zero();
    gemm_acc<E, C, D, D, NW, true, true>(u, R1, LR, X1, LD2, wave, lane);
    E* out = dUs + cidx * C * D;   // stored transposed, [r][t]
    for_tiles_ij(u, wave, lane, [&](int i, int j, int t0, int rr, const f32x4& x) {
      f32x4 pu, y;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        y[r] = Dv[t0 + r] * x[r];
        pu[r] = x[r] * to_f(R2[(t0 + r) * LR + rr]);
      }
      st_f4(out + (long)rr * C + t0, y);
      dds.add(i, j, pu, true, false);
    });
  }
  // ---- refinement pairs: dW_l += D (K_l dS_n^T), dK_l += D (W_l dS_n) ----
  for (int l = 0; l < L; ++l) {
    const long lrow = ((long)bh * L + l) * Tp + tb;
    kl.store_rows(R3, LR, tid);
    wl.store_rows(R4, LR, tid);
    __syncthreads();
    {
      // (the last step reads its own rows again: a load under a condition
      // leaves a merge of old and new registers that the compiler resolves
      // with copies at the loop head, which wait for every memory operation
      // in flight, the previous step's gradient stores included)
      const long nrow = l + 1 < L ? lrow + Tp : lrow;
      kl.load(Kl + nrow * D, D, C, tid);
      wl.load(Wl + nrow * D, D, C, tid);
    }
    Acc<C, D, NW> a;
    a.zero();
    gemm_acc<E, C, D, D, NW, true, true>(a, R3, LR, X1, LD2, wave, lane);
    float* ow = dWls + lrow * D;
    for_tiles_ij(a, wave, lane, [&](int i, int j, int t0, int rr, const f32x4& x) {
      f32x4 pw;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        ow[(long)(t0 + r) * D + rr] = Dv[t0 + r] * x[r];
        pw[r] = x[r] * to_f(R4[(t0 + r) * LR + rr]);
      }
      dds.add(i, j, pw, true, false);
    });
    Acc<C, D, NW> bb;
    bb.zero();
    gemm_acc<E, C, D, D, NW, true, true>(bb, R4, LR, X2, LD2, wave, lane);
    E* ok = dKls + lrow * D;
    for_tiles(bb, wave, lane, [&](int t0, int n, const f32x4& x) {
#pragma unroll
      for (int r = 0; r < 4; ++r) ok[(long)(t0 + r) * D + n] = to_t<E>(Dv[t0 + r] * x[r]);
    });
    __syncthreads();
  }

  // The lane's offsets of the last phases are formed again from an opaque copy
  // of the thread index: kept live across the refinement loop they spill.
  int tid_o = threadIdx.x;
  asm volatile("" : "+v"(tid_o));
  {
  const int tid = tid_o, lane = tid_o & 63;
  // ---- dM (row-major into X1, transposed into X2); Wk rows ----
  __syncthreads();   // every read of dS_n / dS_n^T (X1, X2) is done
  for_tiles(dm, wave, lane, [&](int k0, int n, const f32x4& x) {
#pragma unroll
    for (int r = 0; r < 4; ++r) X1[(k0 + r) * LD2 + n] = to_t<E>(-x[r]);
    st4f(X2 + n * LD2 + k0, -x);   // four consecutive k: one write
  });
  wkt.store_transposed(R3, LR, nullptr, tid);
  __syncthreads();
  {
    Acc<C, D, NW> a;    // K dM^T: [t][k] = sum_n K[t][n] dM[k][n]
    a.zero();
    gemm_acc<E, C, D, D, NW, true, true>(a, R1, LR, X1, LD2, wave, lane);
    E* out = dWks + cidx * C * D;   // stored transposed, [k][t]
    for_tiles_ij(a, wave, lane, [&](int i, int j, int t0, int kk, const f32x4& x) {
      f32x4 pw, y;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        y[r] = Dv[t0 + r] * x[r];
        pw[r] = x[r] * to_f(R3[(t0 + r) * LR + kk]);
      }
      st_f4(out + (long)kk * C + t0, y);
      dds.add(i, j, pw, true, false);
    });
    Acc<C, D, NW> bb;   // Wk dM: [t][n] = sum_k Wk[t][k] dM^T[n][k]
    bb.zero();
    gemm_acc<E, C, D, D, NW, true, true>(bb, R3, LR, X2, LD2, wave, lane);
    E* ok = dKs + cidx * C * D;   // stored transposed, [n][t]
    typedef Tiling<C, D, NW> TL;
    if (TL::active(wave)) {
#pragma unroll
      for (int i = 0; i < TL::RM; ++i)
#pragma unroll
        for (int j = 0; j < TL::RN; ++j) {
          const int t0 = TL::m0(wave) + 16 * i + 4 * (lane >> 4);
          const int n = TL::n0(wave) + 16 * j + (lane & 15);
          f32x4 y;
#pragma unroll
          for (int r = 0; r < 4; ++r) y[r] = dk.v[i][j][r] + Dv[t0 + r] * bb.v[i][j][r];
          st_f4(ok + (long)n * C + t0, y);
        }
    }
  }
  if (TLS::active(wave)) dds.flush_rows(ddw + wave * C, TLS::m0(wave), lane);
  __syncthreads();
  // ---- dg from D_t = exp(gC - g_t) and exp(gC) ----
  if (wave == 0) {
    float dd = 0.f;
    if (lane < C)
      for (int w = 0; w < NW; ++w) dd += ddw[w * C + lane];
    const float Dd = lane < C ? Dv[lane] * dd : 0.f;
    float tot = Dd;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) tot += __shfl_xor(tot, off);
    float ssum = 0.f;
    for (int w = 0; w < NW; ++w) ssum += sdw[w];
    const float dgC = expf(g[C - 1]) * ssum + tot;
    if (lane < C) dgs[cidx * C + lane] = -Dd + (lane == C - 1 ? dgC : 0.f);
  }
  }
}

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
  // vectors: g, e, Dv, bt, be, de (6C) + slots rs, cs, bs, es [NW][C]
  static constexpr int SZ_VEC = (6 * C + 4 * CB_NW * C) * 4;
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
  for (int e = tid; e < 4 * NW * C; e += NT) rs[e] = 0.f;
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
    invert_unit_lower<C, NW>(Af, Tf, Xs, tid);
    for (int e = tid; e < C * C; e += NT) {
      const int t = e / C, i = e % C;
      const float tv = Tf[t * LA + i];
      Tb[t * LT + i] = to_t<E>(tv);
      Tbb[t * LT + i] = to_t<E>(tv * bt[i]);
      Tbe[t * LT + i] = to_t<E>(tv * be[i]);
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
#pragma unroll
    for (int off = 1; off < DQT::VPR; off <<= 1) sdq += __shfl_xor(sdq, off);
    if (u < DQT::NU && (u % DQT::VPR) == 0) de[r] = sdq;
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
  for (int e = tid; e < C * C; e += NT) {
    const int t = e / C, i = e % C;
    Zb[t * LT + i] = to_t<E>(Zf[t * LA + i] + Zf[i * LA + t]);
  }
  __syncthreads();
  gemm_acc<E, C, D, C, NW, true, false>(dk, Zb, LT, Kr, LR, wave, lane);   // (dG0 + dG0^T) K

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
    sbd.flush_rows(bs + wave * C, TLD::m0(wave), lane);
    sed.flush_rows(es + wave * C, TLD::m0(wave), lane);
  }
  __syncthreads();
  if (tid < C) {
    const int t = tid;
    float sr = 0.f, sb = 0.f, se = 0.f;
    for (int w = 0; w < NW; ++w) {
      sr += rs[w * C + t] - cs[w * C + t];
      sb += bs[w * C + t];
      se += es[w * C + t];
    }
    // de: from Qt (Q . dQt) and from Wk (beta K . X2); e_t = exp(g_t)
    const float det = de[t] + bt[t] * se;
    dgp[cidx * C + t] = dgs[cidx * C + t] + sr + ev[t] * det;
    if (t < nval) dbeta[row0 + (long)t * H] = sb + ev[t] * se;
  }
}

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
  RegTile<E, C, D, NT> kl, wl;   // next step's K_l, W_l rows (software prefetch)
  if (L > 0) {
    const long lrow = (long)bh * L * Tp + tb;
    kl.load(Kl + lrow * D, D, C, tid);
    wl.load(Wl + lrow * D, D, C, tid);
  }
  for (int l = 0; l < L; ++l) {
    const long lrow = ((long)bh * L + l) * Tp + tb;
    kl.store_rows(Klr, LR, tid);
    wl.store_rows(Wlr, LR, tid);
    __syncthreads();
    {
      // (the last step reads its own rows again: a load under a condition
      // leaves a merge of old and new registers that the compiler resolves
      // with copies at the loop head, which wait for every memory operation
      // in flight, the previous step's gradient stores included)
      const long nrow = l + 1 < L ? lrow + Tp : lrow;
      kl.load(Kl + nrow * D, D, C, tid);
      wl.load(Wl + nrow * D, D, C, tid);
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
  const E* dqc = dqp + cidx * C * D;
  const E* dkc = dkp + cidx * C * D;
  const E* dvc = dVp + cidx * C * D;
  RegTile<E, C, D, NT> rq, rk;
  rq.load(dqc, D, C, tid);
  rk.load(dkc, D, C, tid);
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
    constexpr int VN = 16 / (int)sizeof(E);
    E* dvo = dv + row0 * D;
    for (int e = tid; e < C * D / VN; e += NT) {
      const int t = e / (D / VN), f = (e % (D / VN)) * VN;
      if (t < nval) st16(dvo + (long)t * ts + f, ld16(dvc + (long)t * D + f));
    }
  }
  __syncthreads();
  // ---- dalpha: dlog(alpha)_j = sum_{t >= j} dg_t ----
  if (wave == 0) {
    float dg = 0.f;
    if (lane < C) {
      dg = dgp[cidx * C + lane];
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

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
template <typename E, int D, int C>
static hipError_t cbwd_launch_dc(const Dims& d, const ChunkBwdArgs<E>& a, int stage, hipStream_t s) {
  if constexpr (sizeof(E) == 4 && D * C > 2048) {
    return hipErrorInvalidValue;   // outside the fp32 envelope (LDS)
  } else {
    const int nblk = d.B * d.H * d.NC;
    if (stage == 0)
      hipLaunchKernelGGL((chunk_bwd_state_kernel<E, D, C>), dim3(nblk), dim3(CB_NT), 0, s, a.k, a.dO,
                         a.alpha, a.Kl, a.Wl, a.UT, a.WkT, a.Sc, a.dSnT, a.dQt, a.dUs, a.dWks,
                         a.dKs, a.dKl, a.dWl, a.dgs, d.B, d.T, d.H, d.L, d.NC, d.Tp, d.cu);
    else if (stage == 1)
      hipLaunchKernelGGL((chunk_bwd_solve_kernel<E, D, C>), dim3(nblk), dim3(CB_NT), 0, s, a.q,
                         a.k, a.v, a.dO, a.alpha, a.beta, a.Kl, a.Wl, a.dQt, a.dUs, a.dWks, a.dKs,
                         a.dgs, a.dVp, a.dqp, a.dkp, a.dgp, a.dbeta, d.B, d.T, d.H, d.L, d.NC,
                         d.Tp, d.cu);
    else
      hipLaunchKernelGGL((chunk_bwd_pairs_kernel<E, D, C>), dim3(nblk), dim3(CB_NT), 0, s, a.q,
                         a.k, a.dO, a.alpha, a.Kl, a.Wl, a.dVp, a.dqp, a.dkp, a.dgp, a.dKl, a.dWl,
                         a.dq, a.dk, a.dv, a.dalpha, d.B, d.T, d.H, d.L, d.NC, d.Tp, d.cu);
    return hipGetLastError();
  }
}

template <typename E, int D>
static hipError_t cbwd_launch_d(const Dims& d, const ChunkBwdArgs<E>& a, int stage, hipStream_t s) {
  switch (d.C) {
    case 16: return cbwd_launch_dc<E, D, 16>(d, a, stage, s);
    case 32: return cbwd_launch_dc<E, D, 32>(d, a, stage, s);
    case 64: return cbwd_launch_dc<E, D, 64>(d, a, stage, s);
  }
  return hipErrorInvalidValue;
}

template <typename E>
hipError_t launch_chunk_bwd(const Dims& d, const ChunkBwdArgs<E>& a, int stage, hipStream_t s) {
  switch (d.D) {
    case 16: return cbwd_launch_d<E, 16>(d, a, stage, s);
    case 32: return cbwd_launch_d<E, 32>(d, a, stage, s);
    case 64: return cbwd_launch_d<E, 64>(d, a, stage, s);
    case 128:
      if constexpr (sizeof(E) == 2) return cbwd_launch_d<E, 128>(d, a, stage, s);
      break;
  }
  return hipErrorInvalidValue;
}

template hipError_t launch_chunk_bwd<bf16>(const Dims&, const ChunkBwdArgs<bf16>&, int, hipStream_t);
template hipError_t launch_chunk_bwd<float>(const Dims&, const ChunkBwdArgs<float>&, int, hipStream_t);

}  // namespace prism
