// Backward of Stage 1 and Stage 2 (PRISM summary §2.2): given the gradients
// of the refinement pairs (dK_l = d k^(l), dW_l = d w^(l)) and the direct
// v-gradient of the recurrence, produce dv, dW_k, dW_p, dw_beta and the
// ShortConv tap gradients.
//
// Per token, with a = dL/dr^(l+1) (zero for the last step):
//   dbeta^(l) = delta^(l) . dw^(l);  ddelta = beta^(l) dw^(l) - a
//   dz = ddelta * GELU'(z);  dp = dz * r^(l);  a += dz * p^(l)
//   du += W_p^(l)^T dp + W_k^(l)^T dk^(l) + dlogit w_beta^(l),
//   dlogit = dbeta^(l) beta^(l) (1 - beta^(l))
// then dv = dv_direct + a + (ShortConv adjoint of du - a):
//   dv_s += sum_j conv[:, j] (du - a)_{s+o+j},  dconv[:, j] += (du - a)_t v_{t-o-j}
// (o = 0: taps on the current token; o = 1: strictly past taps).
// With the identity step (delta = p * r) GELU' is 1.
// Weight gradients are reductions over all B * T tokens:
//   dW_p^(l) = sum_t dp u^T,  dW_k^(l) = sum_t dk^(l) u^T   (split-K MFMA GEMM)
// with fixed-order partial sums (no atomics).
//
// The kernel template lives in this header; the variant files instantiate it
// once per (step activation, tap offset), so the variants compile in parallel.
#pragma once

#include <type_traits>

#include "prism_common.h"
#include "prism_internal.h"

namespace prism {

// A workgroup computes the refinement backward for RB_TT consecutive tokens
// but owns only the first RB_TT - 3 - o of them: the ShortConv adjoint of
// token s needs du at s + o .. s + o + 3, so the last 3 + o tokens are a halo
// recomputed by the next workgroup, and dv, dconv, dw_beta and the rows for
// the weight GEMM come out of the same kernel.
constexpr int RB_TT = 32;
constexpr int RB_NW = 4;                // one wave per feature group
constexpr int RB_NT = RB_NW * WAVE;
constexpr int rb_own(int off) { return RB_TT - 3 - off; }

template <typename E, int D, int LMAX, int ACT, int OFF>
__global__ __launch_bounds__(RB_NT, 2) void refine_bwd_kernel(
    const E* __restrict__ v, const E* __restrict__ hist, const E* __restrict__ conv,
    const E* __restrict__ Wp,   // W_p, W_k^T, W_p^T in fragment order (frag_order_offset)
    const E* __restrict__ WkT, const E* __restrict__ WpT, const E* __restrict__ wbeta,
    const E* __restrict__ dKl, const float* __restrict__ dWl, const E* __restrict__ dvdir,
    E* __restrict__ uo, E* __restrict__ dPo, E* __restrict__ dv, float* __restrict__ dwbp,
    float* __restrict__ dcp, float* __restrict__ dhist, int B, int T, int H, int L, int Tp,
    int ntiles, const int* __restrict__ cu) {
  constexpr int LD = ldpad<E>(D);
  constexpr int LW = D + 4;               // fp32 rows: staggers rows 4 apart across banks
  constexpr int NFT = D / 16;
  constexpr int FPW = (NFT + 3) / 4;      // feature tiles per wave
  // feature tile n exists; always true when the tiles divide evenly over the
  // feature groups (then the test folds away at compile time)
#define FT_OK(n) (NFT % 4 == 0 || (n) < NFT)
  typedef MfmaK<E, D> MK;
  constexpr int KS = MK::KSTEP;
  constexpr int VN = 16 / sizeof(E);
  constexpr int HL = 3 + OFF;             // v rows before the tile that the taps reach
  constexpr int OWN = rb_own(OFF);
  __shared__ __attribute__((aligned(16))) E vbuf[(RB_TT + HL) * D];  // v rows t0-HL .. t0+RB_TT-1
  __shared__ __attribute__((aligned(16))) E ubuf[RB_TT * LD];
  __shared__ __attribute__((aligned(16))) E ulo[sizeof(E) == 2 ? RB_TT * LD : 16];   // u - bf16(u)
  __shared__ __attribute__((aligned(16))) E dpbuf[RB_TT * LD];        // dp rows; at the end dv rows
  __shared__ __attribute__((aligned(16))) float gk[RB_TT * LW];       // dW_l rows (fp32); at the end du
  __shared__ __attribute__((aligned(16))) E gkk[RB_TT * LD];          // dK_l rows (the product's operand type)
  __shared__ float gate[LMAX][RB_TT];
  __shared__ float gsum[4][RB_TT];
  __shared__ float dlog[RB_TT];
  __shared__ __attribute__((aligned(16))) E wbl[LMAX * D];            // w_beta^(l) rows of this head
  __shared__ float ctp[D * 4];                                        // conv taps of this head
  __shared__ float red[RB_NT * 4];                                    // dconv partials per thread
  float* gw = gk;

  const int tid = threadIdx.x, lane = tid & 63;
  // wave = feature group; at D = 128 taken as wave-uniform, so that the
  // weight fragments' bases are scalar (the registers that frees hold the
  // kept residual rows below; the smaller instances use fewer registers
  // without it)
  const int fq = D >= 128 ? __builtin_amdgcn_readfirstlane(tid >> 6) : tid >> 6;
  const int nblk = ntiles * B * H;
  const int bid = xcd_swizzle(blockIdx.x, nblk);
  const int h = bid / (B * ntiles);
  const int rest = bid % (B * ntiles);
  const int b = rest / ntiles, tile = rest % ntiles;
  const int t0 = tile * OWN;
  const int Tb = seq_len(cu, b, T);        // this sequence's length
  const int own = min(OWN, Tb - t0);        // owned tokens (<= 0 past the end)
  const int nrow = min(RB_TT, Tb - t0);     // computed tokens that exist
  if (own <= 0) {
    // past the end of a packed sequence: zero partial sums (and a zero
    // history gradient for an empty sequence), nothing else
    const int tile_id_ = (int)(((long)b * H + h) * ntiles + tile);
    for (int e = tid; e < L * D; e += RB_NT) dwbp[(long)tile_id_ * L * D + e] = 0.f;
    for (int e = tid; e < 4 * D; e += RB_NT) dcp[(long)tile_id_ * D * 4 + e] = 0.f;
    if (tile == 0 && dhist)
      for (int e = tid; e < 4 * D; e += RB_NT)
        dhist[(((long)b * 4 + e / D) * H + h) * D + e % D] = 0.f;
    return;
  }
  const long tok_stride = (long)H * D;
  const E* vseq = v + (seq_start(cu, b, T) * H + h) * D;
  const long bh = (long)b * H + h;
  const E* ch = conv + (long)h * D * 4;
  const int tile_id = (int)(bh * ntiles + tile);

  // The set-up's reads (w_beta rows, taps, the v rows of the tile and its
  // halo) are all issued before the first is stored: one memory round trip,
  // where copy loops that store each value as it arrives wait once per
  // iteration.  No load sits in a per-lane branch (its merge would make the
  // wave wait for it at issue): out-of-range v rows read row 0 and are zeroed
  // at the store.
  constexpr int NWB = LMAX * (D / VN), PWB = (NWB + RB_NT - 1) / RB_NT;
  constexpr int NCT = 4 * D, PCT = (NCT + RB_NT - 1) / RB_NT;
  constexpr int NVB = (RB_TT + HL) * (D / VN), PVB = (NVB + RB_NT - 1) / RB_NT;
  const int nwb = L * (D / VN);
  uint4 wbv[PWB], vbv[PVB];
  E ctv[PCT];
  bool vz[PVB];
  if (nwb > 0) {   // (uniform: no refinement, no w_beta)
#pragma unroll
    for (int p = 0; p < PWB; ++p)
      wbv[p] = ld16(wbeta + (long)h * L * D + (long)min(tid + p * RB_NT, nwb - 1) * VN);
  }
#pragma unroll
  for (int p = 0; p < PCT; ++p) ctv[p] = ch[min(tid + p * RB_NT, NCT - 1)];
#pragma unroll
  for (int p = 0; p < PVB; ++p) {
    const int e = min(tid + p * RB_NT, NVB - 1);
    const int r = e / (D / VN), c = (e % (D / VN)) * VN;
    const int t = t0 - HL + r;
    const bool in_seq = t >= 0 && t < Tb, in_hist = t < 0 && hist;
    vz[p] = !in_seq && !in_hist;
    const E* src = in_seq ? vseq + t * tok_stride + c
                 : in_hist ? hist + (((long)b * 4 + 4 + t) * H + h) * D + c : vseq + c;
    vbv[p] = ld16(src);
  }
  // dW, dK rows of the first reverse step, in flight during the set-up
  RegTile<float, RB_TT, D, RB_NT> pw;   // dW_l rows (fp32)
  RegTile<E, RB_TT, D, RB_NT> pk;       // dK_l rows
  {
    const long lrow = (bh * L + (L - 1)) * Tp + t0;
    pw.load(dWl + lrow * D, D, nrow, tid);
    pk.load(dKl + lrow * D, D, nrow, tid);
  }
  // Weight fragments (B operands) of this wave's feature tiles.  Every
  // product takes them preloaded: a fragment load issued ahead of the work
  // that precedes its product keeps its L2 latency off the critical path, and
  // issuing it before the row prefetches and stores of a step keeps the
  // product's wait (vmcnt counts in issue order) from covering those.
  typedef typename MK::frag Frag;
  // (the weights come in fragment order: each fragment is one contiguous
  // 64-lane piece)
  auto load_w = [&](const E* W, Frag (&bw)[FPW][D / KS]) {
#pragma unroll
    for (int nn = 0; nn < FPW; ++nn)
#pragma unroll
      for (int kk = 0; kk < D / KS; ++kk)
        if (FT_OK(fq + 4 * nn)) bw[nn][kk] = load_frag_fo<E, D>(W, fq + 4 * nn, kk, lane);
  };
  // Up to three steps (EARLY_W) the first projection's fragments are
  // requested here, with the set-up's reads.
  constexpr bool EARLY_W = LMAX <= 3;
  Frag bwp[FPW][D / KS];   // W_p^(l) fragments
  if (EARLY_W && L > 0) load_w(Wp + (long)h * L * D * D, bwp);
#pragma unroll
  for (int p = 0; p < PWB; ++p)
    if (tid + p * RB_NT < nwb) st16(wbl + (tid + p * RB_NT) * VN, wbv[p]);
#pragma unroll
  for (int p = 0; p < PCT; ++p)
    if (tid + p * RB_NT < NCT) ctp[tid + p * RB_NT] = to_f(ctv[p]);
#pragma unroll
  for (int p = 0; p < PVB; ++p) {
    const int e = tid + p * RB_NT;
    if (e < NVB) {
      uint4 x = vbv[p];
      asm volatile("" : "+v"(x.x), "+v"(x.y), "+v"(x.z), "+v"(x.w));
      if (vz[p]) x = uint4{0u, 0u, 0u, 0u};
      const int r = e / (D / VN), c = (e % (D / VN)) * VN;
      st16(vbuf + r * D + c, x);
    }
  }
  __syncthreads();
  // anchor u (fp32; to LDS as the MFMA operand, hi and lo parts) and residual
  // r^(1) = v - u in the accumulator layout:
  // element (m, nn, i): token 16 m + 4 (lane >> 4) + i, feature 16 n + (lane & 15), n = fq + 4 nn
  float r[2][FPW][4];
#pragma unroll
  for (int nn = 0; nn < FPW; ++nn) {
    const int n = fq + 4 * nn;
    const int f = 16 * n + (lane & 15);
    float tp[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) tp[j] = (FT_OK(n)) ? ctp[f * 4 + j] : 0.f;
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 16 * m + 4 * (lane >> 4) + i;
        float u = 0.f, val = 0.f;
        if (FT_OK(n) && t < nrow) {
#pragma unroll
          for (int j = 0; j < 4; ++j) u += tp[j] * to_f(vbuf[(t + HL - OFF - j) * D + f]);
          val = to_f(vbuf[(t + HL) * D + f]) - u;
        }
        r[m][nn][i] = val;
        if (FT_OK(n)) {
          const E uh = to_t<E>(u);
          ubuf[t * LD + f] = uh;
          if constexpr (sizeof(E) == 2) ulo[t * LD + f] = to_t<E>(u - to_f(uh));
        }
      }
  }
  __syncthreads();
  // owned u rows for the weight-gradient GEMM; gates (4 threads per token,
  // 16-byte reads of u and w_beta; the RB_NT / 4 RB_TT thread groups take
  // the steps round robin)
  s2g_rows<E, RB_TT, D, RB_NT>(uo + (bh * Tp + t0) * D, D, ubuf, LD, own, tid);
  {
    constexpr int GG = RB_NT / (4 * RB_TT);
    static_assert(GG >= 1, "a thread group per step");
    const int grp = tid / (4 * RB_TT), t = (tid % (4 * RB_TT)) >> 2, part = tid & 3;
    for (int l = grp; l < L; l += GG) {
      float s = 0.f;
      for (int c = part * VN; c < D; c += 4 * VN) {
        const uint4 ua = ld16(ubuf + t * LD + c), wa = ld16(wbl + l * D + c);
        const E* ue = reinterpret_cast<const E*>(&ua);
        const E* we = reinterpret_cast<const E*>(&wa);
#pragma unroll
        for (int j = 0; j < VN; ++j) s += to_f(we[j]) * to_f(ue[j]);
      }
      s = quad_sum(s);
      if (part == 0) gate[l][t] = sigmoidf(s);
    }
  }
  pw.store_rows_f32(gw, LW, tid);
  pk.store_rows(gkk, LD, tid);
  __syncthreads();

  // p^(l) = W_p^(l) (u_hi + u_lo) for this wave's tiles (same as the forward)
  auto project = [&](const Frag (&bws)[FPW][D / KS], f32x4 (&acc)[2][FPW]) {
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int nn = 0; nn < FPW; ++nn) acc[m][nn] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k0 = 0; k0 < D; k0 += KS) {
      typename MK::frag a[2], al[2];
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        a[m] = load_fragK<E, D>(ubuf, LD, 16 * m, k0, lane);
        if constexpr (sizeof(E) == 2) al[m] = load_fragK<E, D>(ulo, LD, 16 * m, k0, lane);
      }
#pragma unroll
      for (int nn = 0; nn < FPW; ++nn) {
        const int n = fq + 4 * nn;
        if (FT_OK(n)) {
          const typename MK::frag bw = bws[nn][k0 / KS];
#pragma unroll
          for (int m = 0; m < 2; ++m) {
            acc[m][nn] = MK::mma(a[m], bw, acc[m][nn]);
            if constexpr (sizeof(E) == 2) acc[m][nn] = MK::mma(al[m], bw, acc[m][nn]);
          }
        }
      }
    }
  };
  // acc += X W  where X holds rows [t][i] in LDS (operand type) and bws holds
  // the fragments of WT[j][i] = W[i][j]
  auto project_t = [&](const E* X, int ldx, const Frag (&bws)[FPW][D / KS], f32x4 (&acc)[2][FPW]) {
#pragma unroll
    for (int k0 = 0; k0 < D; k0 += KS) {
      typename MK::frag a[2];
#pragma unroll
      for (int m = 0; m < 2; ++m) a[m] = load_fragK<E, D>(X, ldx, 16 * m, k0, lane);
#pragma unroll
      for (int nn = 0; nn < FPW; ++nn) {
        const int n = fq + 4 * nn;
        if (FT_OK(n)) {
          const typename MK::frag bw = bws[nn][k0 / KS];
#pragma unroll
          for (int m = 0; m < 2; ++m) acc[m][nn] = MK::mma(a[m], bw, acc[m][nn]);
        }
      }
    }
  };

  // ---- forward quantities of every step.  Up to four steps: the gains
  // p^(l) (they depend on u only; r stays r^(1) and the reverse replays the
  // chain, VALU work instead of a second projection).  More steps: the
  // residuals r^(l) (registers for L gains would spill), p^(l) projected again
  // in the reverse. ----
  constexpr bool REPLAY = LMAX <= 4;
  f32x4 ps[REPLAY ? LMAX : 1][2][FPW];
  float rs[REPLAY ? 1 : LMAX][2][FPW][4];
  // Up to three steps the registers hold a second fragment set: the next
  // step's fragments are requested before this step's product, and each
  // reverse step requests its first product's fragments before the chain
  // replay.  More steps keep one set, requested just before its product.
#pragma unroll
  for (int l = 0; l < LMAX; ++l) {
    if (l >= L) break;
    Frag bwn[FPW][D / KS];
    if (!EARLY_W) load_w(Wp + ((long)h * L + l) * D * D, bwp);
    else if (l + 1 < L) load_w(Wp + ((long)h * L + l + 1) * D * D, bwn);
    if constexpr (REPLAY) {
      project(bwp, ps[l]);
    } else {
      f32x4 p[2][FPW];
      project(bwp, p);
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int nn = 0; nn < FPW; ++nn)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            rs[l][m][nn][i] = r[m][nn][i];
            const float z = p[m][nn][i] * r[m][nn][i];
            if constexpr (ACT == ACT_IDENTITY) r[m][nn][i] -= z;
            else r[m][nn][i] -= gelu_erf(z);
          }
    }
    if constexpr (EARLY_W) {
#pragma unroll
      for (int nn = 0; nn < FPW; ++nn)
#pragma unroll
        for (int kk = 0; kk < D / KS; ++kk) bwp[nn][kk] = bwn[nn][kk];
    }
  }

  // ---- reverse: gw / gkk hold dW_l, dK_l of the current step ----
  float a_[2][FPW][4];
  E dvd[2][FPW][4];         // direct v-gradient (fetched during the last step; converted at use)
  f32x4 du[2][FPW];
  // Three or four steps: r^(l-1), kept from the replay of reverse step l for
  // step l - 1 (four steps: steps 3 and 1 replay the chain, step 2 takes the
  // kept rows, 4 replayed GELUs instead of 6; three steps: step 2 replays,
  // step 1 takes the kept rows, 2 instead of 3).  Only when the instance's
  // step count is the runtime one (a uniform test): with fewer steps the
  // first reverse step is not the last step and the kept rows would be read
  // unwritten.  (Three fp32 steps: the kept rows would cost the D = 64
  // instance a wave per SIMD; three steps with past-only taps: they spill.)
  constexpr bool KEEP = LMAX == 4 || (LMAX == 3 && sizeof(E) == 2 && OFF == 0);
  const bool keep = KEEP && L == LMAX;
  float rkeep[KEEP ? 2 : 1][FPW][4];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int nn = 0; nn < FPW; ++nn) {
      du[m][nn] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a_[m][nn][i] = 0.f;
        dvd[m][nn][i] = to_t<E>(0.f);
      }
    }
#pragma unroll
  for (int l = LMAX - 1; l >= 0; --l) {
    if (l >= L) continue;
    // W_p^(l)^T fragments of this step's first transposed product (in flight
    // during the chain replay and the gate gradient when EARLY_W)
    Frag bpt[FPW][D / KS], bkt[FPW][D / KS];
    if constexpr (EARLY_W) load_w(WpT + ((long)h * L + l) * D * D, bpt);
    // (up to three steps) the next step's dW, dK rows right after: the
    // registers are free (this step's rows are in LDS), and the GELU and
    // gate-gradient phases hide their latency
    if (EARLY_W && l > 0) {
      const long lrow = (bh * L + (l - 1)) * Tp + t0;
      pw.load(dWl + lrow * D, D, nrow, tid);
      pk.load(dKl + lrow * D, D, nrow, tid);
    }
    // p^(l) and r^(l) of this step
    f32x4 p[2][FPW];
    float rl[2][FPW][4];
    if constexpr (REPLAY) {
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int nn = 0; nn < FPW; ++nn) p[m][nn] = ps[l][m][nn];
      if (keep && l >= 1 && ((LMAX - 1 - l) & 1)) {
        // the previous reverse step replayed through r^(l)
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
          for (int nn = 0; nn < FPW; ++nn)
#pragma unroll
            for (int i = 0; i < 4; ++i) rl[m][nn][i] = rkeep[m][nn][i];
      } else {
        // r^(l) by replaying the chain from r^(1): l steps of VALU work
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
          for (int nn = 0; nn < FPW; ++nn)
#pragma unroll
            for (int i = 0; i < 4; ++i) rl[m][nn][i] = r[m][nn][i];
#pragma unroll
        for (int j = 0; j < l; ++j) {
          if (keep && j + 1 == l) {   // rl holds r^(l-1) before this last replay step
#pragma unroll
            for (int m = 0; m < 2; ++m)
#pragma unroll
              for (int nn = 0; nn < FPW; ++nn)
#pragma unroll
                for (int i = 0; i < 4; ++i) rkeep[m][nn][i] = rl[m][nn][i];
          }
#pragma unroll
          for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int nn = 0; nn < FPW; ++nn)
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const float z = ps[j][m][nn][i] * rl[m][nn][i];
                if constexpr (ACT == ACT_IDENTITY) rl[m][nn][i] -= z;
                else rl[m][nn][i] -= gelu_erf(z);
              }
        }
      }
    } else {
      Frag bw[FPW][D / KS];
      load_w(Wp + ((long)h * L + l) * D * D, bw);
      project(bw, p);
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int nn = 0; nn < FPW; ++nn)
#pragma unroll
          for (int i = 0; i < 4; ++i) rl[m][nn][i] = rs[l][m][nn][i];
    }
    // GELU'(z) once per element; gate-gradient sum_f delta dw
    float dg_[2][FPW][4];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      f32x4 part = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int nn = 0; nn < FPW; ++nn) {
        const int n = fq + 4 * nn;
        const int f = 16 * n + (lane & 15);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = 16 * m + 4 * (lane >> 4) + i;
          float dl;
          const float z = p[m][nn][i] * rl[m][nn][i];
          if constexpr (ACT == ACT_IDENTITY) {
            dl = z;
            dg_[m][nn][i] = 1.f;
          } else {
            gelu_and_grad(z, dl, dg_[m][nn][i]);
          }
          if (FT_OK(n)) part[i] += dl * gw[t * LW + f];
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float s = row16_sum(part[i]);
        if ((lane & 15) == 15) gsum[fq][16 * m + 4 * (lane >> 4) + i] = s;
      }
    }
    __syncthreads();
    if (tid < RB_TT) {
      const float gt = gate[l][tid];
      dlog[tid] = (gsum[0][tid] + gsum[1][tid] + gsum[2][tid] + gsum[3][tid]) * gt * (1.f - gt);
    }
    // chain step; dp rows
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int nn = 0; nn < FPW; ++nn) {
        const int n = fq + 4 * nn;
        if (!FT_OK(n)) continue;
        const int f = 16 * n + (lane & 15);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = 16 * m + 4 * (lane >> 4) + i;
          const float ddl = gate[l][t] * gw[t * LW + f] - a_[m][nn][i];
          const float dzz = ddl * dg_[m][nn][i];
          a_[m][nn][i] += dzz * p[m][nn][i];
          dpbuf[t * LD + f] = to_t<E>(dzz * rl[m][nn][i]);
        }
      }
    __syncthreads();
    // weight fragments of both products first, then the next step's dW, dK
    // rows (or, in the last step, the direct v-gradient), fetched during the
    // products below
    if constexpr (!EARLY_W) load_w(WpT + ((long)h * L + l) * D * D, bpt);
    else load_w(WkT + ((long)h * L + l) * D * D, bkt);
    if (!EARLY_W && l > 0) {
      const long lrow = (bh * L + (l - 1)) * Tp + t0;
      pw.load(dWl + lrow * D, D, nrow, tid);
      pk.load(dKl + lrow * D, D, nrow, tid);
    } else if (l == 0) {
      const E* dvs = dvdir + (bh * Tp + t0) * D;
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int nn = 0; nn < FPW; ++nn) {
          const int n = fq + 4 * nn;
          const int f = 16 * n + (lane & 15);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int t = 16 * m + 4 * (lane >> 4) + i;
            dvd[m][nn][i] = (FT_OK(n) && t < own) ? dvs[(long)t * D + f] : to_t<E>(0.f);
          }
        }
    }
    const long lrow = (bh * L + l) * Tp + t0;
    s2g_rows<E, RB_TT, D, RB_NT>(dPo + lrow * D, D, dpbuf, LD, own, tid);
    project_t(dpbuf, LD, bpt, du);
    if constexpr (!EARLY_W) load_w(WkT + ((long)h * L + l) * D * D, bkt);
    project_t(gkk, LD, bkt, du);
    // du += dlogit w_beta; dw_beta partial = sum over owned t of dlogit_t u_t
    const E* wb = wbl + l * D;
#pragma unroll
    for (int nn = 0; nn < FPW; ++nn) {
      const int n = fq + 4 * nn;
      if (!FT_OK(n)) continue;
      const int f = 16 * n + (lane & 15);
      const float wbf = to_f(wb[f]);
      float cs = 0.f;
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = 16 * m + 4 * (lane >> 4) + i;
          du[m][nn][i] += dlog[t] * wbf;
          if (t < own) cs += dlog[t] * to_f(ubuf[t * LD + f]);
        }
      cs += __shfl_xor(cs, 16);
      cs += __shfl_xor(cs, 32);
      if (lane < 16) dwbp[((long)tile_id * L + l) * D + f] = cs;
    }
    __syncthreads();   // every read of gw, gkk, dpbuf and dlog is done
    if (l > 0) {
      pw.store_rows_f32(gw, LW, tid);
      pk.store_rows(gkk, LD, tid);
      __syncthreads();
    }
  }

  // ---- ShortConv adjoint: du - a into LDS (fp32 rows) ----
  float* dub = gk;
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int nn = 0; nn < FPW; ++nn) {
      const int n = fq + 4 * nn;
      if (!FT_OK(n)) continue;
      const int f = 16 * n + (lane & 15);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 16 * m + 4 * (lane >> 4) + i;
        dub[t * LW + f] = t < nrow ? du[m][nn][i] - a_[m][nn][i] : 0.f;
      }
    }
  __syncthreads();
  // dv_s = dv_direct_s + a_s + sum_j conv[:, j] du_{s+o+j}   (owned s; s + o + j < T):
  // the lane's four tokens need seven consecutive du rows (rows >= nrow are zero)
#pragma unroll
  for (int nn = 0; nn < FPW; ++nn) {
    const int n = fq + 4 * nn;
    if (!FT_OK(n)) continue;
    const int f = 16 * n + (lane & 15);
    float tp[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) tp[j] = ctp[f * 4 + j];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int t0m = 16 * m + 4 * (lane >> 4);
      float w[7];
#pragma unroll
      for (int q = 0; q < 7; ++q) {
        const int row = t0m + OFF + q;
        w[q] = row < RB_TT ? dub[row * LW + f] : 0.f;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = t0m + i;
        if (t < own) {
          // the conversion stays here (empty asm): next to the load it
          // would make the prefetch wait for its data at issue
          E dr = dvd[m][nn][i];
          asm volatile("" : "+v"(dr));
          float val = to_f(dr) + a_[m][nn][i];
#pragma unroll
          for (int j = 0; j < 4; ++j) val += tp[j] * w[i + j];
          dpbuf[t * LD + f] = to_t<E>(val);
        }
      }
    }
  }
  // dconv partial: sum over owned t of du_t v_{t-o-j} (vbuf row t + 3 - j);
  // each token group takes a contiguous range, so the four v rows slide
  constexpr int NG = RB_NT / D;   // token groups; red is [NG][D][4]
  constexpr int TPG = (OWN + NG - 1) / NG;
  {
    const int f = tid % D, grp = tid / D;
    const int tb = grp * TPG;
    auto vrow = [&](int row) { return row < RB_TT + HL ? to_f(vbuf[row * D + f]) : 0.f; };
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    float x0 = vrow(tb), x1 = vrow(tb + 1), x2 = vrow(tb + 2);
#pragma unroll
    for (int k = 0; k < TPG; ++k) {
      const int t = tb + k;
      const float x3 = vrow(t + 3);
      if (t < own) {
        const float d_ = dub[t * LW + f];
        acc[0] += d_ * x3;
        acc[1] += d_ * x2;
        acc[2] += d_ * x1;
        acc[3] += d_ * x0;
      }
      x0 = x1;
      x1 = x2;
      x2 = x3;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) red[(grp * D + f) * 4 + j] = acc[j];
  }
  __syncthreads();
  s2g_rows<E, RB_TT, D, RB_NT>(dv + (seq_start(cu, b, T) + t0) * tok_stride + (long)h * D, tok_stride,
                               dpbuf, LD, own, tid);
  if (tid < D) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float x = 0.f;
      for (int g2 = 0; g2 < NG; ++g2) x += red[(g2 * D + tid) * 4 + j];
      dcp[((long)tile_id * D + tid) * 4 + j] = x;
    }
  }
  // gradient of the history rows v_{-4} .. v_{-1}: the adjoint at s < 0,
  // dh_s = sum_j conv[:, j] du_{s+o+j} over 0 <= s+o+j (first tile only)
  if (tile == 0 && dhist) {
    for (int e = tid; e < 4 * D; e += RB_NT) {
      const int r = e / D, f = e % D;
      float x = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int t = r - 4 + OFF + j;
        if (t >= 0 && t < nrow) x += ctp[f * 4 + j] * dub[t * LW + f];
      }
      dhist[(((long)b * 4 + r) * H + h) * D + f] = x;
    }
  }
}

// Stage 1 of the refinement backward for one (activation, tap offset)
// variant: picks the head-dimension and step-count instantiation.
template <typename E, int ACT, int OFF>
hipError_t launch_refine_bwd_main(const Dims& d, const RefineBwdArgs<E>& a, hipStream_t s) {
  const int ntiles = refine_bwd_tiles(d);
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3(ntiles * d.B * d.H), dim3(RB_NT), 0, s, a.v, a.hist, a.conv, a.WpF,
                       a.WkT, a.WpT, a.wbeta, a.dKl, a.dWl, a.dvdir, a.u, a.dP, a.dv, a.dwbp, a.dcp,
                       a.dhist, d.B, d.T, d.H, d.L, d.Tp, ntiles, d.cu);
    return hipGetLastError();
  };
  auto by_l = [&](auto dd) {
    constexpr int D = decltype(dd)::value;
    // L = 3 has its own instance; the LMAX = 4 instance keeps replayed
    // residuals only when its runtime L is 4 (it also serves no other L here)
    if (d.L <= 2) return go(refine_bwd_kernel<E, D, 2, ACT, OFF>);
    if (d.L == 3) return go(refine_bwd_kernel<E, D, 3, ACT, OFF>);
    if (d.L <= 4) return go(refine_bwd_kernel<E, D, 4, ACT, OFF>);
    return go(refine_bwd_kernel<E, D, 8, ACT, OFF>);
  };
  switch (d.D) {
    case 16: return by_l(std::integral_constant<int, 16>{});
    case 32: return by_l(std::integral_constant<int, 32>{});
    case 64: return by_l(std::integral_constant<int, 64>{});
    case 128:
      if constexpr (sizeof(E) == 2) return by_l(std::integral_constant<int, 128>{});
      break;
  }
  return hipErrorInvalidValue;
}

#define PRISM_RB_VARIANT(ACT, OFF)                                                              \
  extern template hipError_t launch_refine_bwd_main<bf16, ACT, OFF>(const Dims&,              \
                                                                     const RefineBwdArgs<bf16>&, \
                                                                     hipStream_t);              \
  extern template hipError_t launch_refine_bwd_main<float, ACT, OFF>(                          \
      const Dims&, const RefineBwdArgs<float>&, hipStream_t);
PRISM_RB_VARIANT(ACT_GELU, 0)
PRISM_RB_VARIANT(ACT_GELU, 1)
PRISM_RB_VARIANT(ACT_IDENTITY, 0)
PRISM_RB_VARIANT(ACT_IDENTITY, 1)
#undef PRISM_RB_VARIANT

#undef FT_OK
}  // namespace prism
