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
//   dv_s += sum_j conv[:, j] (du - a)_{s+j},  dconv[:, j] += (du - a)_t v_{t-j}.
// Weight gradients are reductions over all B * T tokens:
//   dW_p^(l) = sum_t dp u^T,  dW_k^(l) = sum_t dk^(l) u^T   (split-K MFMA GEMM)
// with fixed-order partial sums (no atomics).
#include <type_traits>

#include "prism_common.h"
#include "prism_internal.h"

namespace prism {

// A workgroup computes the refinement backward for RB_TT consecutive tokens
// but owns only the first RB_OWN of them: the ShortConv adjoint of token s
// needs du at s .. s+3, so the last three tokens are a halo recomputed by the
// next workgroup, and dv, dconv, dw_beta and the rows for the weight GEMM
// come out of the same kernel.
constexpr int RB_TT = 32;
constexpr int RB_OWN = RB_TT - 3;
constexpr int RB_NW = 4;                // one wave per feature group
constexpr int RB_NT = RB_NW * WAVE;

int refine_bwd_tiles(const Dims& d) { return (d.T + RB_OWN - 1) / RB_OWN; }

// WT[h][l][j][i] = W[h][l][i][j] for W in {Wk, Wp}
template <typename E>
__global__ void transpose_weights_kernel(const E* __restrict__ Wk, const E* __restrict__ Wp,
                                         E* __restrict__ WkT, E* __restrict__ WpT, int HL, int D) {
  const long n = (long)HL * D * D;
  for (long e = blockIdx.x * (long)blockDim.x + threadIdx.x; e < n; e += (long)gridDim.x * blockDim.x) {
    const long m = e / ((long)D * D);
    const int i = (int)((e / D) % D), j = (int)(e % D);
    const long dst = (m * D + j) * D + i;
    WkT[dst] = Wk[e];
    WpT[dst] = Wp[e];
  }
}

// MFMA A-operand fragment of bf16 (or fp32) values read from an fp32 LDS
// row tile X[row][k] (k contiguous), rounded to the operand type.
template <typename E>
__device__ inline typename Mfma<E>::frag frag_from_f32(const float* X, int ld, int row0, int k0, int lane) {
  if constexpr (sizeof(E) == 4) {
    return load_frag<float, true>(X, ld, row0, k0, lane);
  } else {
    const float* p = X + (row0 + (lane & 15)) * ld + k0 + 8 * (lane >> 4);
    const f32x4 x0 = *reinterpret_cast<const f32x4*>(p);
    const f32x4 x1 = *reinterpret_cast<const f32x4*>(p + 4);
    bf16x8 f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f[j] = (bf16)x0[j];
      f[4 + j] = (bf16)x1[j];
    }
    return f;
  }
}

template <typename E, int D, int LMAX>
__global__ __launch_bounds__(RB_NT, 2) void refine_bwd_kernel(
    const E* __restrict__ v, const E* __restrict__ conv, const E* __restrict__ Wp,
    const E* __restrict__ WkT, const E* __restrict__ WpT, const E* __restrict__ wbeta,
    const float* __restrict__ dKl, const float* __restrict__ dWl, const float* __restrict__ dvdir,
    E* __restrict__ uo, E* __restrict__ dPo, E* __restrict__ dv, float* __restrict__ dwbp,
    float* __restrict__ dcp, int B, int T, int H, int L, int Tp, int ntiles) {
  constexpr int LD = ldpad<E>(D);
  constexpr int LW = D + 4;               // fp32 rows: staggers rows 4 apart across banks
  constexpr int NFT = D / 16;
  constexpr int FPW = (NFT + 3) / 4;      // feature tiles per wave
  // feature tile n exists; always true when the tiles divide evenly over the
  // feature groups (then the test folds away at compile time)
#define FT_OK(n) (NFT % 4 == 0 || (n) < NFT)
  constexpr int KS = Mfma<E>::KSTEP;
  constexpr int VN = 16 / sizeof(E);
  __shared__ __attribute__((aligned(16))) E vbuf[(RB_TT + 3) * D];   // v rows t0-3 .. t0+RB_TT-1
  __shared__ __attribute__((aligned(16))) E ubuf[RB_TT * LD];
  __shared__ __attribute__((aligned(16))) E ulo[sizeof(E) == 2 ? RB_TT * LD : 16];   // u - bf16(u)
  __shared__ __attribute__((aligned(16))) E dpbuf[RB_TT * LD];        // dp rows; at the end dv rows
  __shared__ __attribute__((aligned(16))) float gk[2 * RB_TT * LW];   // dW_l, dK_l rows; at the end du
  __shared__ float gate[LMAX][RB_TT];
  __shared__ float gsum[4][RB_TT];
  __shared__ float dlog[RB_TT];
  __shared__ __attribute__((aligned(16))) E wbl[LMAX * D];            // w_beta^(l) rows of this head
  __shared__ float ctp[D * 4];                                        // conv taps of this head
  __shared__ float red[RB_NT * 4];                                    // dconv partials per thread
  float* gw = gk;
  float* gkk = gk + RB_TT * LW;

  const int tid = threadIdx.x, lane = tid & 63, fq = tid >> 6;   // wave = feature group
  const int nblk = ntiles * B * H;
  const int bid = xcd_swizzle(blockIdx.x, nblk);
  const int h = bid / (B * ntiles);
  const int rest = bid % (B * ntiles);
  const int b = rest / ntiles, tile = rest % ntiles;
  const int t0 = tile * RB_OWN;
  const int own = min(RB_OWN, T - t0);      // owned tokens (>= 1)
  const int nrow = min(RB_TT, T - t0);      // computed tokens that exist
  const long tok_stride = (long)H * D;
  const E* vseq = v + ((long)b * T * H + h) * D;
  const long bh = (long)b * H + h;
  const E* ch = conv + (long)h * D * 4;
  const int tile_id = (int)(bh * ntiles + tile);

  for (int e = tid; e < L * (D / VN); e += RB_NT)
    st16(wbl + e * VN, ld16(wbeta + (long)h * L * D + e * VN));
  for (int e = tid; e < D * 4; e += RB_NT) ctp[e] = to_f(ch[e]);
  for (int e = tid; e < (RB_TT + 3) * (D / VN); e += RB_NT) {
    const int r = e / (D / VN), c = (e % (D / VN)) * VN;
    const int t = t0 - 3 + r;
    uint4 x = {0u, 0u, 0u, 0u};
    if (t >= 0 && t < T) x = ld16(vseq + t * tok_stride + c);
    st16(vbuf + r * D + c, x);
  }
  // dW, dK rows of the first reverse step, in flight during the set-up
  RegTile<float, RB_TT, D, RB_NT> pw, pk;
  {
    const long lrow = (bh * L + (L - 1)) * Tp + t0;
    pw.load(dWl + lrow * D, D, nrow, tid);
    pk.load(dKl + lrow * D, D, nrow, tid);
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
          for (int j = 0; j < 4; ++j) u += tp[j] * to_f(vbuf[(t + 3 - j) * D + f]);
          val = to_f(vbuf[(t + 3) * D + f]) - u;
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
  // 16-byte reads of u and w_beta)
  s2g_rows<E, RB_TT, D, RB_NT>(uo + (bh * Tp + t0) * D, D, ubuf, LD, own, tid);
  if (tid < RB_TT * 4) {
    const int t = tid >> 2, part = tid & 3;
    for (int l = 0; l < L; ++l) {
      float s = 0.f;
      for (int c = part * VN; c < D; c += 4 * VN) {
        const uint4 ua = ld16(ubuf + t * LD + c), wa = ld16(wbl + l * D + c);
        const E* ue = reinterpret_cast<const E*>(&ua);
        const E* we = reinterpret_cast<const E*>(&wa);
#pragma unroll
        for (int j = 0; j < VN; ++j) s += to_f(we[j]) * to_f(ue[j]);
      }
      s += __shfl_xor(s, 1);
      s += __shfl_xor(s, 2);
      if (part == 0) gate[l][t] = sigmoidf(s);
    }
  }
  pw.store_rows(gw, LW, tid);
  pk.store_rows(gkk, LW, tid);
  __syncthreads();

  // p^(l) = W_p^(l) (u_hi + u_lo) for this wave's tiles (same as the forward)
  auto project = [&](const E* W, f32x4 (&acc)[2][FPW]) {
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int nn = 0; nn < FPW; ++nn) acc[m][nn] = f32x4{0.f, 0.f, 0.f, 0.f};
    typename Mfma<E>::frag bws[FPW][D / KS];
#pragma unroll
    for (int nn = 0; nn < FPW; ++nn)
#pragma unroll
      for (int kk = 0; kk < D / KS; ++kk)
        if (FT_OK(fq + 4 * nn)) bws[nn][kk] = load_frag<E, true>(W, D, 16 * (fq + 4 * nn), kk * KS, lane);
#pragma unroll
    for (int k0 = 0; k0 < D; k0 += KS) {
      typename Mfma<E>::frag a[2], al[2];
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        a[m] = load_frag<E, true>(ubuf, LD, 16 * m, k0, lane);
        if constexpr (sizeof(E) == 2) al[m] = load_frag<E, true>(ulo, LD, 16 * m, k0, lane);
      }
#pragma unroll
      for (int nn = 0; nn < FPW; ++nn) {
        const int n = fq + 4 * nn;
        if (FT_OK(n)) {
          const typename Mfma<E>::frag bw = bws[nn][k0 / KS];
#pragma unroll
          for (int m = 0; m < 2; ++m) {
            acc[m][nn] = Mfma<E>::mma(a[m], bw, acc[m][nn]);
            if constexpr (sizeof(E) == 2) acc[m][nn] = Mfma<E>::mma(al[m], bw, acc[m][nn]);
          }
        }
      }
    }
  };
  // acc += X W  where X holds rows [t][i] (operand type in LDS, or fp32 in
  // LDS when XF) and WT[j][i] = W[i][j]
  auto project_t = [&](auto xf, const void* X, int ldx, const E* WT, f32x4 (&acc)[2][FPW]) {
    constexpr bool XF = decltype(xf)::value;
    typename Mfma<E>::frag bws[FPW][D / KS];
#pragma unroll
    for (int nn = 0; nn < FPW; ++nn)
#pragma unroll
      for (int kk = 0; kk < D / KS; ++kk)
        if (FT_OK(fq + 4 * nn)) bws[nn][kk] = load_frag<E, true>(WT, D, 16 * (fq + 4 * nn), kk * KS, lane);
#pragma unroll
    for (int k0 = 0; k0 < D; k0 += KS) {
      typename Mfma<E>::frag a[2];
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        if constexpr (XF) a[m] = frag_from_f32<E>(static_cast<const float*>(X), ldx, 16 * m, k0, lane);
        else a[m] = load_frag<E, true>(static_cast<const E*>(X), ldx, 16 * m, k0, lane);
      }
#pragma unroll
      for (int nn = 0; nn < FPW; ++nn) {
        const int n = fq + 4 * nn;
        if (FT_OK(n)) {
          const typename Mfma<E>::frag bw = bws[nn][k0 / KS];
#pragma unroll
          for (int m = 0; m < 2; ++m) acc[m][nn] = Mfma<E>::mma(a[m], bw, acc[m][nn]);
        }
      }
    }
  };

  // ---- forward chain: keep r^(l) for every step ----
  float rs[LMAX][2][FPW][4];
#pragma unroll
  for (int l = 0; l < LMAX; ++l) {
    if (l >= L) break;
    f32x4 p[2][FPW];
    project(Wp + ((long)h * L + l) * D * D, p);
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int nn = 0; nn < FPW; ++nn)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          rs[l][m][nn][i] = r[m][nn][i];
          r[m][nn][i] -= gelu_erf(p[m][nn][i] * r[m][nn][i]);
        }
  }

  // ---- reverse: gw / gkk hold dW_l, dK_l of the current step ----
  float a_[2][FPW][4];
  float dvd[2][FPW][4];     // direct v-gradient (fetched during the last step)
  f32x4 du[2][FPW];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int nn = 0; nn < FPW; ++nn) {
      du[m][nn] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 4; ++i) a_[m][nn][i] = dvd[m][nn][i] = 0.f;
    }
#pragma unroll
  for (int l = LMAX - 1; l >= 0; --l) {
    if (l >= L) continue;
    f32x4 p[2][FPW];
    project(Wp + ((long)h * L + l) * D * D, p);
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
          gelu_and_grad(p[m][nn][i] * rs[l][m][nn][i], dl, dg_[m][nn][i]);
          if (FT_OK(n)) part[i] += dl * gw[t * LW + f];
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float s = part[i];
        s += __shfl_xor(s, 1);
        s += __shfl_xor(s, 2);
        s += __shfl_xor(s, 4);
        s += __shfl_xor(s, 8);
        if ((lane & 15) == 0) gsum[fq][16 * m + 4 * (lane >> 4) + i] = s;
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
          dpbuf[t * LD + f] = to_t<E>(dzz * rs[l][m][nn][i]);
        }
      }
    __syncthreads();
    // the next step's dW, dK rows (or, in the last step, the direct
    // v-gradient) are fetched during the products below
    if (l > 0) {
      const long lrow = (bh * L + (l - 1)) * Tp + t0;
      pw.load(dWl + lrow * D, D, nrow, tid);
      pk.load(dKl + lrow * D, D, nrow, tid);
    } else {
      const float* dvs = dvdir + (bh * Tp + t0) * D;
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int nn = 0; nn < FPW; ++nn) {
          const int n = fq + 4 * nn;
          const int f = 16 * n + (lane & 15);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int t = 16 * m + 4 * (lane >> 4) + i;
            dvd[m][nn][i] = (FT_OK(n) && t < own) ? dvs[(long)t * D + f] : 0.f;
          }
        }
    }
    const long lrow = (bh * L + l) * Tp + t0;
    s2g_rows<E, RB_TT, D, RB_NT>(dPo + lrow * D, D, dpbuf, LD, own, tid);
    project_t(std::false_type{}, dpbuf, LD, WpT + ((long)h * L + l) * D * D, du);
    project_t(std::true_type{}, gkk, LW, WkT + ((long)h * L + l) * D * D, du);
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
      pw.store_rows(gw, LW, tid);
      pk.store_rows(gkk, LW, tid);
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
  // dv_s = dv_direct_s + a_s + sum_j conv[:, j] du_{s+j}   (owned s; s + j < T)
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
        if (t < own) {
          float val = dvd[m][nn][i] + a_[m][nn][i];
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (t + j < nrow) val += ctp[f * 4 + j] * dub[(t + j) * LW + f];
          dpbuf[t * LD + f] = to_t<E>(val);
        }
      }
    }
  // dconv partial: sum over owned t of du_t v_{t-j}  (v_{t-j} is vbuf row t + 3 - j)
  constexpr int NG = RB_NT / D;   // token groups; red is [NG][D][4]
  {
    const int f = tid % D, grp = tid / D;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < (RB_OWN + NG - 1) / NG; ++k) {
      const int t = grp + k * NG;
      if (t < own) {
        const float d_ = dub[t * LW + f];
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] += d_ * to_f(vbuf[(t + 3 - j) * D + f]);
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) red[(grp * D + f) * 4 + j] = acc[j];
  }
  __syncthreads();
  s2g_rows<E, RB_TT, D, RB_NT>(dv + ((long)b * T + t0) * tok_stride + (long)h * D, tok_stride,
                               dpbuf, LD, own, tid);
  if (tid < D) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float x = 0.f;
      for (int g2 = 0; g2 < NG; ++g2) x += red[(g2 * D + tid) * 4 + j];
      dcp[((long)tile_id * D + tid) * 4 + j] = x;
    }
  }
}

// Split-K weight-gradient GEMM: for (h, l, which, split):
//   P[i][j] = sum_{n in split} X[n][i] u[n][j],  X = dK_l (fp32, which = 0)
//   or dp (operand type, which = 1); n runs over (b, t), t < T.
constexpr int WG_NW = 8;
constexpr int WG_NT = WG_NW * WAVE;
constexpr int WG_ROWS = 64;

// One 64-row chunk of a [B][*][Tp][D] tensor (row n -> b = n / Tp, t = n % Tp;
// rows with t >= T are zeros) read as 16-byte vectors into registers, later
// stored transposed into LDS: s[f * ld + r].  Consecutive threads take
// consecutive row groups of one column block (two rows each when E is
// 16-bit), so each transposed store writes one 32-bit word per lane to
// consecutive words: no LDS bank conflicts.
template <typename E, typename X, int D>
struct RowChunk {
  static constexpr int VN = 16 / (int)sizeof(X);
  static constexpr int VPR = D / VN;
  static constexpr int RG = sizeof(E) == 2 ? 2 : 1;
  static constexpr int NG = WG_ROWS / RG;
  static constexpr int NU = NG * VPR;
  static constexpr int PER = (NU + WG_NT - 1) / WG_NT;
  uint4 v[PER][RG];
  __device__ inline void load(const X* base, long rowstride_b, int Tp, int T, long n0, long nend, int tid) {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int u = tid + p * WG_NT;
      const int r0 = (u % NG) * RG, c = (u / NG) * VN;
#pragma unroll
      for (int q = 0; q < RG; ++q) {
        v[p][q] = uint4{0u, 0u, 0u, 0u};
        const long n = n0 + r0 + q;
        if (u < NU && n < nend) {
          const long bb = n / Tp, t = n % Tp;
          if (t < T) v[p][q] = ld16(base + bb * rowstride_b + t * D + c);
        }
      }
    }
  }
  __device__ inline void store_t(E* s, int ld, int tid) const {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int u = tid + p * WG_NT;
      if (u >= NU) continue;
      const int r0 = (u % NG) * RG, c = (u / NG) * VN;
      if constexpr (RG == 2) {
        const X* x0 = reinterpret_cast<const X*>(&v[p][0]);
        const X* x1 = reinterpret_cast<const X*>(&v[p][1]);
#pragma unroll
        for (int j = 0; j < VN; ++j) {
          E pr[2] = {to_t<E>(to_f(x0[j])), to_t<E>(to_f(x1[j]))};
          uint32_t w;
          __builtin_memcpy(&w, pr, 4);
          *reinterpret_cast<uint32_t*>(s + (c + j) * ld + r0) = w;
        }
      } else {
        const X* x = reinterpret_cast<const X*>(&v[p][0]);
#pragma unroll
        for (int j = 0; j < VN; ++j) s[(c + j) * ld + r0] = to_t<E>(to_f(x[j]));
      }
    }
  }
};

template <typename E, int D>
__global__ __launch_bounds__(WG_NT) void wgrad_gemm_kernel(const float* __restrict__ dKl,
                                                           const E* __restrict__ dP,
                                                           const E* __restrict__ u,
                                                           float* __restrict__ part, int B, int H,
                                                           int L, int T, int Tp, int NS) {
  constexpr int LTT = ldpad<E>(WG_ROWS);
  __shared__ __attribute__((aligned(16))) E Xt[D * LTT];
  __shared__ __attribute__((aligned(16))) E Ut[D * LTT];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int s = blockIdx.x % NS;
  const int which = (blockIdx.x / NS) % 2;
  const int hl = blockIdx.x / (2 * NS);
  const int h = hl / L, l = hl % L;
  const long N = (long)B * Tp;
  const long per = ((N + NS - 1) / NS + WG_ROWS - 1) / WG_ROWS * WG_ROWS;
  const long n_begin = s * per, n_end = min(N, n_begin + per);
  Acc<D, D, WG_NW> acc;
  acc.zero();
  const long xs_b = (long)H * L * Tp * D;      // X row stride between batches
  const long us_b = (long)H * Tp * D;
  const float* xk = dKl + (((long)h * L + l) * Tp) * D;
  const E* xp = dP + (((long)h * L + l) * Tp) * D;
  const E* ub = u + ((long)h * Tp) * D;
  RowChunk<E, float, D> xf;
  RowChunk<E, E, D> xe, uu;
  // software pipeline: chunk n0 + 64 is fetched while chunk n0 is multiplied
  if (n_begin < n_end) {
    if (which == 0) xf.load(xk, xs_b, Tp, T, n_begin, n_end, tid);
    else xe.load(xp, xs_b, Tp, T, n_begin, n_end, tid);
    uu.load(ub, us_b, Tp, T, n_begin, n_end, tid);
  }
  for (long n0 = n_begin; n0 < n_end; n0 += WG_ROWS) {
    if (which == 0) xf.store_t(Xt, LTT, tid);
    else xe.store_t(Xt, LTT, tid);
    uu.store_t(Ut, LTT, tid);
    __syncthreads();
    const long nn = n0 + WG_ROWS;
    if (nn < n_end) {
      if (which == 0) xf.load(xk, xs_b, Tp, T, nn, n_end, tid);
      else xe.load(xp, xs_b, Tp, T, nn, n_end, tid);
      uu.load(ub, us_b, Tp, T, nn, n_end, tid);
    }
    gemm_acc<E, D, D, WG_ROWS, WG_NW, true, true>(acc, Xt, LTT, Ut, LTT, wave, lane);
    __syncthreads();
  }
  float* out = part + (long)blockIdx.x * D * D;
  for_tiles(acc, wave, lane, [&](int i0, int j, const f32x4& x) {
#pragma unroll
    for (int r = 0; r < 4; ++r) out[(long)(i0 + r) * D + j] = x[r];
  });
}

// Fixed-order reduction of the split-K partial products into dW_k, dW_p.
__global__ void wgrad_reduce_kernel(const float* __restrict__ part, float* __restrict__ dWk,
                                    float* __restrict__ dWp, int H, int L, int D, int NS) {
  const long nW = (long)H * L * D * D;
  for (long e = blockIdx.x * (long)blockDim.x + threadIdx.x; e < 2 * nW; e += (long)gridDim.x * blockDim.x) {
    const int which = e < nW ? 0 : 1;
    const long x = e - which * nW;
    const long hl = x / ((long)D * D), ij = x % ((long)D * D);
    const float* p = part + ((hl * 2 + which) * NS) * (long)D * D + ij;
    float s = 0.f;
    for (int k = 0; k < NS; ++k) s += p[(long)k * D * D];
    (which == 0 ? dWk : dWp)[x] = s;
  }
}

// Fixed-order reduction of the per-tile partial sums of dw_beta and of the
// ShortConv taps: 16 outputs per block, each summed by 16 threads over a
// strided slice of the B * ntiles partials, then the 16 slices in order.
constexpr int BR_OUT = 16, BR_SL = 16;
__global__ __launch_bounds__(BR_OUT * BR_SL) void bias_reduce_kernel(
    const float* __restrict__ dwbp, const float* __restrict__ dcp, float* __restrict__ dwbeta,
    float* __restrict__ dconv, int B, int H, int L, int D, int ntiles) {
  __shared__ float red[BR_SL][BR_OUT];
  const int oi = threadIdx.x % BR_OUT, sl = threadIdx.x / BR_OUT;
  const long o = (long)blockIdx.x * BR_OUT + oi;
  const long nB = (long)H * L * D, nC = (long)H * D * 4;
  const int P = B * ntiles;
  float s = 0.f;
  if (o < nB) {
    const long h = o / ((long)L * D), lf = o % ((long)L * D);
#pragma unroll 4
    for (int p = sl; p < P; p += BR_SL) {
      const int bb = p / ntiles, t = p % ntiles;
      s += dwbp[(((long)bb * H + h) * ntiles + t) * L * D + lf];
    }
  } else if (o < nB + nC) {
    const long x = o - nB;
    const long h = x / ((long)D * 4), fj = x % ((long)D * 4);
#pragma unroll 4
    for (int p = sl; p < P; p += BR_SL) {
      const int bb = p / ntiles, t = p % ntiles;
      s += dcp[(((long)bb * H + h) * ntiles + t) * D * 4 + fj];
    }
  }
  red[sl][oi] = s;
  __syncthreads();
  if (sl == 0 && o < nB + nC) {
    float x = 0.f;
#pragma unroll
    for (int k = 0; k < BR_SL; ++k) x += red[k][oi];
    if (o < nB) dwbeta[o] = x;
    else dconv[o - nB] = x;
  }
}

// ---------------------------------------------------------------------------
template <typename E, int D, int LMAX>
static void refine_bwd_launch(const Dims& d, const RefineBwdArgs<E>& a, int ntiles, hipStream_t s) {
  hipLaunchKernelGGL((refine_bwd_kernel<E, D, LMAX>), dim3(ntiles * d.B * d.H), dim3(RB_NT), 0, s,
                     a.v, a.conv, a.Wp, a.WkT, a.WpT, a.wbeta, a.dKl, a.dWl, a.dvdir, a.u, a.dP,
                     a.dv, a.dwbp, a.dcp, d.B, d.T, d.H, d.L, d.Tp, ntiles);
}

template <typename E, int D>
static hipError_t refine_bwd_d(const Dims& d, const RefineBwdArgs<E>& a, int NS, int stage,
                               hipStream_t s) {
  const int ntiles = refine_bwd_tiles(d);
  const long nw = (long)d.H * d.L * D * D;
  switch (stage) {
    case 0:
      hipLaunchKernelGGL((transpose_weights_kernel<E>),
                         dim3((unsigned)((nw + 255) / 256 < 4096 ? (nw + 255) / 256 : 4096)), dim3(256),
                         0, s, a.Wk, a.Wp, a.WkT, a.WpT, d.H * d.L, D);
      break;
    case 1:
      if (d.L <= 2)
        refine_bwd_launch<E, D, 2>(d, a, ntiles, s);
      else if (d.L <= 4)
        refine_bwd_launch<E, D, 4>(d, a, ntiles, s);
      else
        refine_bwd_launch<E, D, 8>(d, a, ntiles, s);
      break;
    case 2:
      hipLaunchKernelGGL((wgrad_gemm_kernel<E, D>), dim3(d.H * d.L * 2 * NS), dim3(WG_NT), 0, s,
                         a.dKl, a.dP, a.u, a.part, d.B, d.H, d.L, d.T, d.Tp, NS);
      break;
    case 3: {
      const unsigned grid = (unsigned)((2 * nw + 255) / 256 < 8192 ? (2 * nw + 255) / 256 : 8192);
      hipLaunchKernelGGL(wgrad_reduce_kernel, dim3(grid), dim3(256), 0, s, a.part, a.dWk_o, a.dWp_o,
                         d.H, d.L, D, NS);
      break;
    }
    default: {
      const long nout = (long)d.H * d.L * D + (long)d.H * D * 4;
      hipLaunchKernelGGL(bias_reduce_kernel, dim3((unsigned)((nout + BR_OUT - 1) / BR_OUT)),
                         dim3(BR_OUT * BR_SL), 0, s, a.dwbp, a.dcp, a.dwbeta_o, a.dconv_o, d.B, d.H,
                         d.L, D, ntiles);
    }
  }
  return hipGetLastError();
}

int refine_bwd_splits(const Dims& d) {
  const long N = (long)d.B * d.Tp;
  int ns = (int)(1024 / (2L * d.H * (d.L > 0 ? d.L : 1)));
  if (ns < 1) ns = 1;
  const long maxs = (N + WG_ROWS - 1) / WG_ROWS;
  if (ns > maxs) ns = (int)maxs;
  return ns;
}

template <typename E>
hipError_t launch_refine_bwd(const Dims& d, const RefineBwdArgs<E>& a, int stage, hipStream_t s) {
  if (d.L == 0) return hipSuccess;
  const int NS = refine_bwd_splits(d);
  switch (d.D) {
    case 16: return refine_bwd_d<E, 16>(d, a, NS, stage, s);
    case 32: return refine_bwd_d<E, 32>(d, a, NS, stage, s);
    case 64: return refine_bwd_d<E, 64>(d, a, NS, stage, s);
    case 128:
      if constexpr (sizeof(E) == 2) return refine_bwd_d<E, 128>(d, a, NS, stage, s);
      break;
  }
  return hipErrorInvalidValue;
}

template hipError_t launch_refine_bwd<bf16>(const Dims&, const RefineBwdArgs<bf16>&, int, hipStream_t);
template hipError_t launch_refine_bwd<float>(const Dims&, const RefineBwdArgs<float>&, int, hipStream_t);

#undef FT_OK
}  // namespace prism
