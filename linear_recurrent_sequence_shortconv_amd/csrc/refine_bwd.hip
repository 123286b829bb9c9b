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
// then dv += a, du -= a, and the ShortConv adjoint
//   dv_{t-j} += conv[:, j] * du_t,  dconv[:, j] += du_t * v_{t-j}.
// Weight gradients are reductions over all B * T tokens:
//   dW_p^(l) = sum_t dp u^T,  dW_k^(l) = sum_t dk^(l) u^T   (split-K MFMA GEMM)
// with fixed-order partial sums (no atomics).
#include "prism_common.h"
#include "prism_internal.h"

namespace prism {

constexpr int RB_TT = kRefineTile;      // tokens per workgroup
constexpr int RB_TH = RB_TT / 32;       // token groups of 32 (one per 4 waves)
constexpr int RB_NW = 4 * RB_TH;
constexpr int RB_NT = RB_NW * WAVE;

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

template <typename E, int D, int LMAX>
__global__ __launch_bounds__(RB_NT, 2) void refine_bwd_kernel(
    const E* __restrict__ v, const E* __restrict__ conv, const E* __restrict__ Wp,
    const E* __restrict__ WkT, const E* __restrict__ WpT, const E* __restrict__ wbeta,
    const float* __restrict__ dKl, const float* __restrict__ dWl, float* __restrict__ dvdir,
    E* __restrict__ uo, float* __restrict__ duo, E* __restrict__ dPo, float* __restrict__ dwbp,
    int B, int T, int H, int L, int Tp) {
  constexpr int LD = ldpad<E>(D);
  constexpr int NFT = D / 16;
  constexpr int FPW = (NFT + 3) / 4;     // feature tiles per wave (4 feature groups)
  constexpr int KS = Mfma<E>::KSTEP;
  constexpr int VN = 16 / sizeof(E);
  __shared__ E vbuf[(RB_TT + 3) * D];
  __shared__ __attribute__((aligned(16))) E ubuf[RB_TT * LD];
  __shared__ __attribute__((aligned(16))) E ulo[sizeof(E) == 2 ? RB_TT * LD : 16];   // u - bf16(u)
  __shared__ __attribute__((aligned(16))) E dpbuf[RB_TT * LD];
  __shared__ __attribute__((aligned(16))) E dkbuf[RB_TT * LD];
  __shared__ float gate[8][RB_TT];
  __shared__ float gsum[4][RB_TT];
  __shared__ float dlog[RB_TT];
  __shared__ float wbs[RB_TH][D];
  __shared__ __attribute__((aligned(16))) E wbl[8 * D];      // w_beta^(l) rows of this head
  __shared__ float ctp[D * 4];                               // conv taps of this head

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int th = wave >> 2, fq = wave & 3;     // token group, feature group
  const int ntiles = (Tp + RB_TT - 1) / RB_TT;
  const int nblk = ntiles * B * H;
  const int bid = xcd_swizzle(blockIdx.x, nblk);
  const int h = bid / (B * ntiles);
  const int rest = bid % (B * ntiles);
  const int b = rest / ntiles, tile = rest % ntiles;
  const int t0 = tile * RB_TT;
  const long tok_stride = (long)H * D;
  const E* vseq = v + ((long)b * T * H + h) * D;
  const long bh = (long)b * H + h;
  const E* ch = conv + (long)h * D * 4;

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
  __syncthreads();
  for (int e = tid; e < RB_TT * D; e += RB_NT) {
    const int t = e / D, f = e % D;
    float u = 0.f;
    if (t0 + t < T) {
#pragma unroll
      for (int j = 0; j < 4; ++j) u += ctp[f * 4 + j] * to_f(vbuf[(t + 3 - j) * D + f]);
    }
    const E uh = to_t<E>(u);
    ubuf[t * LD + f] = uh;
    if constexpr (sizeof(E) == 2) ulo[t * LD + f] = to_t<E>(u - to_f(uh));
  }
  __syncthreads();
  // u rows for the weight-gradient GEMM; gates
  {
    const int nval = min(RB_TT, Tp - t0);
    s2g_rows<E, RB_TT, D, RB_NT>(uo + (bh * Tp + t0) * D, D, ubuf, LD, nval, tid);
  }
  if (tid < RB_TT * 4) {
    const int t = tid >> 2, part = tid & 3;
    for (int l = 0; l < L; ++l) {
      const E* wb = wbl + l * D;
      float s = 0.f;
      for (int f = part * (D / 4); f < (part + 1) * (D / 4); ++f) s += to_f(wb[f]) * to_f(ubuf[t * LD + f]);
      s += __shfl_xor(s, 1);
      s += __shfl_xor(s, 2);
      if (part == 0) gate[l][t] = sigmoidf(s);
    }
  }
  // residual r^(1) = v - u in the accumulator layout:
  // element (m, nn, i): token 32 th + 16 m + 4 (lane >> 4) + i, feature 16 n + (lane & 15), n = fq + 4 nn
  float r[2][FPW][4];
#pragma unroll
  for (int nn = 0; nn < FPW; ++nn) {
    const int n = fq + 4 * nn;
    const int f = 16 * n + (lane & 15);
    float tp[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) tp[j] = (n < NFT) ? ctp[f * 4 + j] : 0.f;
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 32 * th + 16 * m + 4 * (lane >> 4) + i;
        float val = 0.f;
        if (n < NFT && t0 + t < T) {
          float u = 0.f;
#pragma unroll
          for (int j = 0; j < 4; ++j) u += tp[j] * to_f(vbuf[(t + 3 - j) * D + f]);
          val = to_f(vbuf[(t + 3) * D + f]) - u;
        }
        r[m][nn][i] = val;
      }
  }
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
        if (fq + 4 * nn < NFT) bws[nn][kk] = load_frag<E, true>(W, D, 16 * (fq + 4 * nn), kk * KS, lane);
#pragma unroll
    for (int k0 = 0; k0 < D; k0 += KS) {
      typename Mfma<E>::frag a[2], al[2];
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        a[m] = load_frag<E, true>(ubuf, LD, 32 * th + 16 * m, k0, lane);
        if constexpr (sizeof(E) == 2) al[m] = load_frag<E, true>(ulo, LD, 32 * th + 16 * m, k0, lane);
      }
#pragma unroll
      for (int nn = 0; nn < FPW; ++nn) {
        const int n = fq + 4 * nn;
        if (n < NFT) {
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
  // acc += X W  where X is an LDS row tile [t][i] and WT[j][i] = W[i][j]
  auto project_t = [&](const E* X, const E* WT, f32x4 (&acc)[2][FPW]) {
    typename Mfma<E>::frag bws[FPW][D / KS];
#pragma unroll
    for (int nn = 0; nn < FPW; ++nn)
#pragma unroll
      for (int kk = 0; kk < D / KS; ++kk)
        if (fq + 4 * nn < NFT) bws[nn][kk] = load_frag<E, true>(WT, D, 16 * (fq + 4 * nn), kk * KS, lane);
#pragma unroll
    for (int k0 = 0; k0 < D; k0 += KS) {
      typename Mfma<E>::frag a[2];
#pragma unroll
      for (int m = 0; m < 2; ++m) a[m] = load_frag<E, true>(X, LD, 32 * th + 16 * m, k0, lane);
#pragma unroll
      for (int nn = 0; nn < FPW; ++nn) {
        const int n = fq + 4 * nn;
        if (n < NFT) {
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

  // ---- reverse ----
  float a_[2][FPW][4];
  f32x4 du[2][FPW];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int nn = 0; nn < FPW; ++nn) {
      du[m][nn] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 4; ++i) a_[m][nn][i] = 0.f;
    }
  const int tile_id = (int)(bh * ntiles + tile);
#pragma unroll
  for (int l = LMAX - 1; l >= 0; --l) {
    if (l >= L) continue;
    const long lrow = (bh * L + l) * Tp + t0;
    const float* dkl = dKl + lrow * D;
    const float* dwl = dWl + lrow * D;
    // this step's incoming gradients, issued before the projection so that
    // their latency overlaps it
    float dw_[2][FPW][4], dk_[2][FPW][4];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int nn = 0; nn < FPW; ++nn) {
        const int n = fq + 4 * nn;
        const int f = 16 * n + (lane & 15);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = 32 * th + 16 * m + 4 * (lane >> 4) + i;
          const bool ok = n < NFT && t0 + t < Tp;    // rows past Tp do not exist
          dw_[m][nn][i] = ok ? dwl[(long)t * D + f] : 0.f;
          dk_[m][nn][i] = ok ? dkl[(long)t * D + f] : 0.f;
        }
      }
    f32x4 p[2][FPW];
    project(Wp + ((long)h * L + l) * D * D, p);
    // GELU'(z) once per element (GELU(z) only enters the gate-gradient sum
    // sum_f delta dw)
    float dg_[2][FPW][4];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      f32x4 part = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int nn = 0; nn < FPW; ++nn) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float dl;
          gelu_and_grad(p[m][nn][i] * rs[l][m][nn][i], dl, dg_[m][nn][i]);
          part[i] += dl * dw_[m][nn][i];
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float s = part[i];
        s += __shfl_xor(s, 1);
        s += __shfl_xor(s, 2);
        s += __shfl_xor(s, 4);
        s += __shfl_xor(s, 8);
        if ((lane & 15) == 0) gsum[fq][32 * th + 16 * m + 4 * (lane >> 4) + i] = s;
      }
    }
    __syncthreads();
    if (tid < RB_TT) {
      const float gt = gate[l][tid];
      dlog[tid] = (gsum[0][tid] + gsum[1][tid] + gsum[2][tid] + gsum[3][tid]) * gt * (1.f - gt);
    }
    // chain step, dp and dk rows
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int nn = 0; nn < FPW; ++nn) {
        const int n = fq + 4 * nn;
        if (n >= NFT) continue;
        const int f = 16 * n + (lane & 15);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = 32 * th + 16 * m + 4 * (lane >> 4) + i;
          const float rr = rs[l][m][nn][i];
          const float ddl = gate[l][t] * dw_[m][nn][i] - a_[m][nn][i];
          const float dzz = ddl * dg_[m][nn][i];
          a_[m][nn][i] += dzz * p[m][nn][i];
          const float dp = dzz * rr;
          dpbuf[t * LD + f] = to_t<E>(dp);
          dkbuf[t * LD + f] = to_t<E>(dk_[m][nn][i]);
        }
      }
    __syncthreads();
    {
      const int nval = min(RB_TT, Tp - t0);
      s2g_rows<E, RB_TT, D, RB_NT>(dPo + lrow * D, D, dpbuf, LD, nval, tid);
    }
    project_t(dpbuf, WpT + ((long)h * L + l) * D * D, du);
    project_t(dkbuf, WkT + ((long)h * L + l) * D * D, du);
    const E* wb = wbl + l * D;
    // du += dlogit w_beta; dw_beta partial = sum_t dlogit_t u_t
#pragma unroll
    for (int nn = 0; nn < FPW; ++nn) {
      const int n = fq + 4 * nn;
      if (n >= NFT) continue;
      const int f = 16 * n + (lane & 15);
      const float wbf = to_f(wb[f]);
      float cs = 0.f;
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = 32 * th + 16 * m + 4 * (lane >> 4) + i;
          du[m][nn][i] += dlog[t] * wbf;
          cs += dlog[t] * to_f(ubuf[t * LD + f]);
        }
      cs += __shfl_xor(cs, 16);
      cs += __shfl_xor(cs, 32);
      if (lane < 16) wbs[th][f] = cs;
    }
    __syncthreads();
    for (int f = tid; f < D; f += RB_NT) {
      float x = 0.f;
#pragma unroll
      for (int g = 0; g < RB_TH; ++g) x += wbs[g][f];
      dwbp[((long)tile_id * L + l) * D + f] = x;
    }
    __syncthreads();
  }
  // ---- dv += a, du -= a ----
  float* dvd = dvdir + (bh * Tp + t0) * D;
  float* duc = duo + (bh * Tp + t0) * D;
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int nn = 0; nn < FPW; ++nn) {
      const int n = fq + 4 * nn;
      if (n >= NFT) continue;
      const int f = 16 * n + (lane & 15);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 32 * th + 16 * m + 4 * (lane >> 4) + i;
        if (t0 + t < Tp) {
          dvd[(long)t * D + f] += a_[m][nn][i];
          duc[(long)t * D + f] = du[m][nn][i] - a_[m][nn][i];
        }
      }
    }
}

// dv_s = dvdir_s + sum_j conv[:, j] du_{s+j}  (s + j < T), written in the
// input layout; per-tile partial dconv[:, j] = sum_t du_t v_{t-j}.
template <typename E, int D>
__global__ __launch_bounds__(256) void conv_bwd_kernel(const E* __restrict__ v,
                                                       const E* __restrict__ conv,
                                                       const float* __restrict__ du,
                                                       const float* __restrict__ dvdir,
                                                       E* __restrict__ dv, float* __restrict__ dcp,
                                                       int B, int T, int H, int Tp) {
  constexpr int NG = 256 / D;             // token groups
  constexpr int TPG = RB_TT / NG;         // tokens per group
  __shared__ float red[NG][D][4];
  const int tid = threadIdx.x;
  const int f = tid % D, grp = tid / D;
  const int ntiles = (Tp + RB_TT - 1) / RB_TT;
  const int nblk = ntiles * B * H;
  const int bid = blockIdx.x;
  const int h = bid / (B * ntiles);
  const int rest = bid % (B * ntiles);
  const int b = rest / ntiles, tile = rest % ntiles;
  const int t0 = tile * RB_TT;
  const long bh = (long)b * H + h;
  const long tok_stride = (long)H * D;
  const E* vseq = v + ((long)b * T * H + h) * D + f;
  E* dvseq = dv + ((long)b * T * H + h) * D + f;
  const float* dus = du + bh * Tp * D + f;
  const float* dvd = dvdir + bh * Tp * D + f;
  float c[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) c[j] = to_f(conv[((long)h * D + f) * 4 + j]);
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int s = t0 + grp * TPG; s < t0 + (grp + 1) * TPG; ++s) {
    if (s >= T) break;
    float val = dvd[(long)s * D];
    const float dus_s = dus[(long)s * D];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (s + j < T) val += c[j] * dus[(long)(s + j) * D];
      if (s - j >= 0) acc[j] += dus_s * to_f(vseq[(long)(s - j) * tok_stride]);
    }
    dvseq[(long)s * tok_stride] = to_t<E>(val);
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) red[grp][f][j] = acc[j];
  __syncthreads();
  if (tid < D) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float s = 0.f;
      for (int g2 = 0; g2 < NG; ++g2) s += red[g2][tid][j];
      dcp[((long)(bh * ntiles + tile) * D + tid) * 4 + j] = s;
    }
  }
  (void)nblk;
}

// Split-K weight-gradient GEMM: for (h, l, which, split):
//   P[i][j] = sum_{n in split} X[n][i] u[n][j],  X = dK_l (fp32, which = 0)
//   or dp (operand type, which = 1); n runs over (b, t), t < Tp.
constexpr int WG_NW = 8;
constexpr int WG_NT = WG_NW * WAVE;
constexpr int WG_ROWS = 64;

// One 64-row chunk of a [B][*][Tp][D] tensor (row n -> b = n / Tp, t = n % Tp)
// read as 16-byte vectors into registers (coalesced), later stored
// transposed into LDS: s[f * ld + r].
template <typename E, typename X, int D>
struct RowChunk {
  static constexpr int VN = 16 / (int)sizeof(X);
  static constexpr int NV = WG_ROWS * D / VN;               // vectors per chunk
  static constexpr int PER = (NV + WG_NT - 1) / WG_NT;      // vectors per thread
  uint4 v[PER];
  __device__ inline void load(const X* base, long rowstride_b, int Tp, long n0, long nend, int tid) {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int e = tid + p * WG_NT;
      v[p] = uint4{0u, 0u, 0u, 0u};
      if (e < NV) {
        const int r = e / (D / VN), c = (e % (D / VN)) * VN;
        const long n = n0 + r;
        if (n < nend) {
          const long bb = n / Tp, t = n % Tp;
          v[p] = ld16(base + bb * rowstride_b + t * D + c);
        }
      }
    }
  }
  __device__ inline void store_t(E* s, int ld, int tid) const {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int e = tid + p * WG_NT;
      if (e < NV) {
        const int r = e / (D / VN), c = (e % (D / VN)) * VN;
        const X* x = reinterpret_cast<const X*>(&v[p]);
#pragma unroll
        for (int j = 0; j < VN; ++j) s[(c + j) * ld + r] = to_t<E>(to_f(x[j]));
      }
    }
  }
};

template <typename E, int D>
__global__ __launch_bounds__(WG_NT) void wgrad_gemm_kernel(const float* __restrict__ dKl,
                                                           const E* __restrict__ dP,
                                                           const E* __restrict__ u,
                                                           float* __restrict__ part, int B, int H,
                                                           int L, int Tp, int NS) {
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
    if (which == 0) xf.load(xk, xs_b, Tp, n_begin, n_end, tid);
    else xe.load(xp, xs_b, Tp, n_begin, n_end, tid);
    uu.load(ub, us_b, Tp, n_begin, n_end, tid);
  }
  for (long n0 = n_begin; n0 < n_end; n0 += WG_ROWS) {
    if (which == 0) xf.store_t(Xt, LTT, tid);
    else xe.store_t(Xt, LTT, tid);
    uu.store_t(Ut, LTT, tid);
    __syncthreads();
    const long nn = n0 + WG_ROWS;
    if (nn < n_end) {
      if (which == 0) xf.load(xk, xs_b, Tp, nn, n_end, tid);
      else xe.load(xp, xs_b, Tp, nn, n_end, tid);
      uu.load(ub, us_b, Tp, nn, n_end, tid);
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

// Fixed-order reduction of all partial sums into the weight gradients.
__global__ void wgrad_reduce_kernel(const float* __restrict__ part, const float* __restrict__ dwbp,
                                    const float* __restrict__ dcp, float* __restrict__ dWk,
                                    float* __restrict__ dWp, float* __restrict__ dwbeta,
                                    float* __restrict__ dconv, int B, int H, int L, int D, int NS,
                                    int ntiles) {
  const long nW = (long)H * L * D * D;
  const long nB = (long)H * L * D;
  const long nC = (long)H * D * 4;
  const long total = 2 * nW + nB + nC;
  for (long e = blockIdx.x * (long)blockDim.x + threadIdx.x; e < total; e += (long)gridDim.x * blockDim.x) {
    if (e < 2 * nW) {
      const int which = e < nW ? 0 : 1;
      const long x = e - which * nW;
      const long hl = x / ((long)D * D), ij = x % ((long)D * D);
      const float* p = part + ((hl * 2 + which) * NS) * (long)D * D + ij;
      float s = 0.f;
      for (int k = 0; k < NS; ++k) s += p[(long)k * D * D];
      (which == 0 ? dWk : dWp)[x] = s;
    } else if (e < 2 * nW + nB) {
      const long x = e - 2 * nW;               // (h, l, f)
      const long h = x / ((long)L * D), lf = x % ((long)L * D);
      float s = 0.f;
      for (int b = 0; b < B; ++b)
        for (int t = 0; t < ntiles; ++t) s += dwbp[(((long)b * H + h) * ntiles + t) * L * D + lf];
      dwbeta[x] = s;
    } else {
      const long x = e - 2 * nW - nB;          // (h, f, j)
      const long h = x / ((long)D * 4), fj = x % ((long)D * 4);
      float s = 0.f;
      for (int b = 0; b < B; ++b)
        for (int t = 0; t < ntiles; ++t) s += dcp[(((long)b * H + h) * ntiles + t) * D * 4 + fj];
      dconv[x] = s;
    }
  }
}

// ---------------------------------------------------------------------------
template <typename E, int D, int LMAX>
static void refine_bwd_launch(const Dims& d, const RefineBwdArgs<E>& a, hipStream_t s) {
  const int ntiles = (d.Tp + RB_TT - 1) / RB_TT;
  hipLaunchKernelGGL((refine_bwd_kernel<E, D, LMAX>), dim3(ntiles * d.B * d.H), dim3(RB_NT), 0, s,
                     a.v, a.conv, a.Wp, a.WkT, a.WpT, a.wbeta, a.dKl, a.dWl, a.dvdir, a.u, a.du,
                     a.dP, a.dwbp, d.B, d.T, d.H, d.L, d.Tp);
}

template <typename E, int D>
static hipError_t refine_bwd_d(const Dims& d, const RefineBwdArgs<E>& a, int NS, int stage,
                               hipStream_t s) {
  const int ntiles = (d.Tp + RB_TT - 1) / RB_TT;
  const long nw = (long)d.H * d.L * D * D;
  switch (stage) {
    case 0:
      hipLaunchKernelGGL((transpose_weights_kernel<E>),
                         dim3((unsigned)((nw + 255) / 256 < 4096 ? (nw + 255) / 256 : 4096)), dim3(256),
                         0, s, a.Wk, a.Wp, a.WkT, a.WpT, d.H * d.L, D);
      break;
    case 1:
      if (d.L <= 2)
        refine_bwd_launch<E, D, 2>(d, a, s);
      else if (d.L <= 4)
        refine_bwd_launch<E, D, 4>(d, a, s);
      else
        refine_bwd_launch<E, D, 8>(d, a, s);
      break;
    case 2:
      hipLaunchKernelGGL((conv_bwd_kernel<E, D>), dim3(ntiles * d.B * d.H), dim3(256), 0, s, a.v,
                         a.conv, a.du, a.dvdir, a.dv, a.dcp, d.B, d.T, d.H, d.Tp);
      break;
    case 3:
      hipLaunchKernelGGL((wgrad_gemm_kernel<E, D>), dim3(d.H * d.L * 2 * NS), dim3(WG_NT), 0, s,
                         a.dKl, a.dP, a.u, a.part, d.B, d.H, d.L, d.Tp, NS);
      break;
    default: {
      const long total = 2 * nw + (long)d.H * d.L * D + (long)d.H * D * 4;
      const unsigned grid = (unsigned)((total + 255) / 256 < 8192 ? (total + 255) / 256 : 8192);
      hipLaunchKernelGGL(wgrad_reduce_kernel, dim3(grid), dim3(256), 0, s, a.part, a.dwbp, a.dcp,
                         a.dWk_o, a.dWp_o, a.dwbeta_o, a.dconv_o, d.B, d.H, d.L, D, NS, ntiles);
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

}  // namespace prism
