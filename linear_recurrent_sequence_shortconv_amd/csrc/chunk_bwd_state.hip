// Chunk backward, first kernel: the terms through S, dS_n and dM = -S^T dS_n.
#include "chunk_bwd_common.h"

namespace prism {

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
  __shared__ __attribute__((aligned(16))) unsigned char smem_[LY::TOTAL];

  int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nblk = B * H * NC;
  const long ts = (long)H * D;
  // At d = 128 (one workgroup per CU) dense batches launch persistent
  // workgroups: they take the virtual block ids blockIdx.x, + gridDim.x, ...,
  // and a chunk's first tiles (dO rows, S_c and dS_n^T, alpha) are fetched
  // while the previous chunk is being finished.  Packed batches (which have
  // chunks past a sequence's end) and smaller d launch one workgroup per
  // chunk: the loop runs once.
  constexpr bool PERSIST = D >= 128;
  const int vstride = PERSIST ? (int)gridDim.x : nblk;
  RegTile<E, C, D, NT> t_do;
  RegTile<E, D, D, NT> t_sc, t_dsnt;
  float pa = 1.f;   // alpha of the next chunk (wave 0, lane < C)
  auto prefetch = [&](int vid) {
    const int bid = xcd_swizzle(vid, nblk);
    const int c = bid % NC, bh = bid / NC;
    const int h = bh % H, b = bh / H;
    const int tb = c * C;
    const int nval = min(C, seq_len(cu, b, T) - tb);
    const long row0 = (seq_start(cu, b, T) + tb) * H + h;
    const long cidx = (long)bh * NC + c;
    t_do.load(dO + row0 * D, ts, nval, tid);
    t_sc.load(Sc + cidx * D * D, D, D, tid);
    t_dsnt.load(dSnT + cidx * D * D, D, D, tid);
    if (wave == 0) pa = lane < nval ? alpha[row0 + (long)lane * H] : 1.f;
  };
  if ((int)blockIdx.x < nblk) prefetch(blockIdx.x);
  for (int vid = blockIdx.x; vid < nblk; vid += vstride) {
  // per-lane values are redefined each iteration, so that the lane-dependent
  // address arithmetic of the body is not hoisted out of the loop and kept
  // live across it
  if constexpr (PERSIST) {
    asm volatile("" : "+v"(tid));
    tid &= NT - 1;   // (its range: tile loops over exactly NT units need no guard)
    lane = tid & 63;
    wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  }
  const int bid = xcd_swizzle(vid, nblk);
  const int c = bid % NC, bh = bid / NC;
  const int h = bh % H, b = bh / H;
  const int tb = c * C;
  const int nval = min(C, seq_len(cu, b, T) - tb);
  const long row0 = (seq_start(cu, b, T) + tb) * H + h;
  const long cidx = (long)bh * NC + c;
  const bool more = PERSIST && vid + vstride < nblk;
  // past the end of a packed sequence: nothing to do (one workgroup per chunk)
  if (nval <= 0) return;
  unsigned char* smem = PERSIST ? lds_opaque(smem_) : smem_;
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

  for (int e = tid; e < NW * C + NW; e += NT) ddw[e] = 0.f;
  typedef Tiling<C, D, NW> TLS;
  TileSums<TLS::RM, TLS::RN> dds;   // row sums of the dD terms, over all products
  dds.zero();
  // the first phase's tiles (dO rows, S_c and dS_n^T, both row-major)
  if (wave == 0) chunk_decays_of<C>(pa, 0.f, g, ev, Dv, nullptr, nullptr, nullptr, lane);
  t_do.store_rows(R1, LR, tid);
  t_sc.store_rows(X1, LD2, tid);
  t_dsnt.store_rows(X2, LD2, tid);
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
    s = wave_sum(s);
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
  // the next chunk's first tiles are fetched during the rest of this one
  // (issued after every load this chunk still waits for: loads complete in
  // order).  Everything in flight before them is a phase old; waiting for it
  // here costs little, and otherwise the compiler's bookkeeping at the
  // refinement loop's exit has a later register reuse wait for the prefetch
  // too (the last step's unconditional K_l, W_l reads are never used).
  if constexpr (PERSIST) __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
  if (more) prefetch(vid + vstride);
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
    const float tot = wave_sum(Dd);
    float ssum = 0.f;
    for (int w = 0; w < NW; ++w) ssum += sdw[w];
    const float dgC = expf(g[C - 1]) * ssum + tot;
    if (lane < C) dgs[cidx * C + lane] = -Dd + (lane == C - 1 ? dgC : 0.f);
  }
  }
  if constexpr (!PERSIST) break;
  __syncthreads();   // LDS is reused by the next chunk
  }
}

struct StateLaunch {
  template <typename E, int D, int C>
  static hipError_t run(const Dims& d, const ChunkBwdArgs<E>& a, hipStream_t s) {
    if constexpr (sizeof(E) == 4 && D * C > 2048) {
      return hipErrorInvalidValue;   // outside the fp32 envelope (LDS)
    } else {
      const int nblk = d.B * d.H * d.NC;
      auto kern = chunk_bwd_state_kernel<E, D, C>;
      hipLaunchKernelGGL(kern, dim3(D >= 128 && !d.cu ? persistent_grid(kern, CB_NT, nblk) : nblk),
                         dim3(CB_NT), 0, s, a.k, a.dO, a.alpha, a.Kl, a.Wl, a.UT, a.WkT, a.Sc,
                         a.dSnT, a.dQt, a.dUs, a.dWks, a.dKs, a.dKl, a.dWl, a.dgs, d.B, d.T, d.H,
                         d.L, d.NC, d.Tp, d.cu);
      return hipGetLastError();
    }
  }
};

template <typename E>
hipError_t launch_chunk_bwd_state(const Dims& d, const ChunkBwdArgs<E>& a, hipStream_t s) {
  return cbwd_dispatch<E, StateLaunch>(d, a, s);
}

template hipError_t launch_chunk_bwd_state<bf16>(const Dims&, const ChunkBwdArgs<bf16>&, hipStream_t);
template hipError_t launch_chunk_bwd_state<float>(const Dims&, const ChunkBwdArgs<float>&, hipStream_t);

}  // namespace prism
