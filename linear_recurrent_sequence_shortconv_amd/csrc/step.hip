// Token-by-token form of the PRISM layer (summary §2.1 "Write-Forget
// Decoupling" and §2.2 "Input-Anchored Loop Unrolling"): the decode step of
// serving, and the exact hand-over of a sequence from one call to the next.
//
// The refinement pairs (k^(l), w^(l)) depend on v and the ShortConv history
// only, never on S, so a step is two kernels: the refinement kernel (with
// one token per sequence it tiles 64 sequences of a head on MFMA, reading
// the head's weights once per tile) writes the pairs, then the state kernel
// here applies, per token of one (b, h),
//   S <- alpha (S - beta (S k) k^T) + beta v k^T + sum_l w^(l) k^(l)^T,
//   o  = S q.
// One workgroup owns one (b, h) for all T tokens: the fp32 state stays in
// registers between tokens, so it crosses HBM once per call (8 D^2 bytes
// read and written), which is what bounds a decode step.  The workgroup
// also rolls the ShortConv history forward.
#include <type_traits>

#include "prism_common.h"
#include "prism_internal.h"

namespace prism {

constexpr int ST_LMAX = 8;

// Threads of the state kernel: four waves, or one for d = 16 (each lane
// holds four consecutive columns of one or more rows).
constexpr int st_waves(int D) { return D * D / 256 < 4 ? D * D / 256 : 4; }

template <typename E, int D>
__global__ __launch_bounds__(64 * st_waves(D)) void step_state_kernel(
    const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ v,
    const float* __restrict__ alpha, const float* __restrict__ beta, const E* __restrict__ Kl,
    const E* __restrict__ Wl, float* __restrict__ S, E* __restrict__ cstate, E* __restrict__ o,
    int B, int T, int H, int L) {
  constexpr int NW = st_waves(D);
  constexpr int NT = 64 * NW;
  constexpr int CPR = D / 4;                // lanes per state row (four columns each)
  constexpr int RPI = WAVE / CPR;           // rows per wave per load: one contiguous block
  constexpr int RPW = D / NW;               // rows per wave
  constexpr int NR = RPW / RPI;             // rows per lane
  __shared__ __attribute__((aligned(16))) float kv[D];
  __shared__ __attribute__((aligned(16))) float qv[D];
  __shared__ __attribute__((aligned(16))) float vv[D];
  __shared__ __attribute__((aligned(16))) float kl[ST_LMAX * D];
  __shared__ __attribute__((aligned(16))) float wl[ST_LMAX * D];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nblk = B * H;
  const int bid = xcd_swizzle(blockIdx.x, nblk);
  const int h = bid / B, b = bid % B;
  const long bh = (long)b * H + h;
  const long tok = (long)H * D;
  const long base = ((long)b * T * H + h) * D;   // token t of this (b, h) at base + t * tok

  // lane (wave w, lane l): columns 4 cc .. 4 cc + 3 of rows w RPW + j RPI + l / CPR,
  // so each load instruction of a wave reads RPI whole consecutive rows
  const int cc = lane % CPR;
  const int row0 = wave * RPW + lane / CPR;
  float* Sp = S + (bh * D + row0) * D + 4 * cc;
  f32x4 s[NR];
#pragma unroll
  for (int j = 0; j < NR; ++j) s[j] = *reinterpret_cast<const f32x4*>(Sp + (long)j * RPI * D);

  // sum over the CPR lanes of a row, left in every one of them
  auto row_sum = [](float x) {
#pragma unroll
    for (int off = CPR / 2; off > 0; off >>= 1) x += __shfl_xor(x, off);
    return x;
  };

  for (int t = 0; t < T; ++t) {
    const long at = base + t * tok;
    for (int e = tid; e < D; e += NT) {
      kv[e] = to_f(k[at + e]);
      qv[e] = to_f(q[at + e]);
      vv[e] = to_f(v[at + e]);
    }
    for (int e = tid; e < L * D; e += NT) {
      const int l = e / D, f = e % D;
      const long src = ((bh * L + l) * T + t) * D + f;
      kl[e] = to_f(Kl[src]);
      wl[e] = to_f(Wl[src]);
    }
    const long ab = ((long)b * T + t) * H + h;
    const float a = alpha[ab], bt = beta[ab];
    __syncthreads();

    const f32x4 k4 = *reinterpret_cast<const f32x4*>(kv + 4 * cc);
    // S <- a (S - bt (S k) k^T) + bt v k^T + sum_l w^(l) k^(l)^T, row by row
#pragma unroll
    for (int j = 0; j < NR; ++j) {
      const int row = row0 + j * RPI;
      const float y = row_sum(s[j][0] * k4[0] + s[j][1] * k4[1] + s[j][2] * k4[2] + s[j][3] * k4[3]);
      const float coef = bt * (vv[row] - a * y);
#pragma unroll
      for (int c = 0; c < 4; ++c) s[j][c] = a * s[j][c] + coef * k4[c];
    }
    for (int l = 0; l < L; ++l) {
      const f32x4 kr = *reinterpret_cast<const f32x4*>(kl + l * D + 4 * cc);
#pragma unroll
      for (int j = 0; j < NR; ++j) {
        const float wi = wl[l * D + row0 + j * RPI];
#pragma unroll
        for (int c = 0; c < 4; ++c) s[j][c] += wi * kr[c];
      }
    }
    // o = S q
    const f32x4 q4 = *reinterpret_cast<const f32x4*>(qv + 4 * cc);
#pragma unroll
    for (int j = 0; j < NR; ++j) {
      const float ot = row_sum(s[j][0] * q4[0] + s[j][1] * q4[1] + s[j][2] * q4[2] + s[j][3] * q4[3]);
      if (cc == 0) o[at + row0 + j * RPI] = to_t<E>(ot);
    }
    __syncthreads();   // the next token rewrites kv, qv, vv, kl, wl
  }

#pragma unroll
  for (int j = 0; j < NR; ++j) *reinterpret_cast<f32x4*>(Sp + (long)j * RPI * D) = s[j];
  // ShortConv history after the tokens: row r holds v_{T-4+r}; each thread
  // reads its feature's four values before writing any
  for (int f = tid; cstate && f < D; f += NT) {
    E x[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = T - 4 + r;
      x[r] = t >= 0 ? v[base + t * tok + f] : cstate[(((long)b * 4 + T + r) * H + h) * D + f];
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) cstate[(((long)b * 4 + r) * H + h) * D + f] = x[r];
  }
}

// Refinement pairs of a decode step (one token per sequence), summary §2.2
// Stages 1-2: a workgroup owns 32 sequences of one head and 64 of its output
// features; wave w takes the 16-feature MFMA tile w mod 4 for 16 of the
// sequences (two waves per SIMD hide each other's latency).  The pairs of
// all sequences of a head thus come from MFMA products with the head's
// weights, read once per 32 sequences.  All loads of the set-up (weights of
// two steps, taps, w_beta, tokens and histories) are issued before the first
// barrier; the chain runs in registers and the pairs are stored from the
// accumulators, so the L steps need no barrier.
constexpr int DR_NW = 8;
constexpr int DR_NT = DR_NW * WAVE;
constexpr int DR_ROWS = 32;   // sequences per workgroup
constexpr int DR_MPW = DR_ROWS / 32;   // 16-sequence MFMA tiles per wave
constexpr int DR_FG = 64;     // output features per workgroup (4 tiles of 16)

template <typename E, int D, int ACT, int OFF>
__global__ __launch_bounds__(DR_NT) void decode_refine_kernel(
    const E* __restrict__ v, const E* __restrict__ hist, const E* __restrict__ conv,
    const E* __restrict__ Wk, const E* __restrict__ Wp, const E* __restrict__ wbeta,
    E* __restrict__ Kl, E* __restrict__ Wl, int B, int H, int L) {
  constexpr int LD = ldpad<E>(D);
  typedef MfmaK<E, D> MK;
  constexpr int KS = MK::KSTEP;
  constexpr int NK = D / KS;
  constexpr int VN = 16 / (int)sizeof(E);
  constexpr int FG = D < DR_FG ? D : DR_FG;   // features of this workgroup
  constexpr int NFG = D / FG;
  constexpr int RW = FG + 4;                  // fp32 residual rows
  constexpr int GT = DR_NT / DR_ROWS;         // threads per gate dot product
  typedef typename MK::frag Frag;
  __shared__ __attribute__((aligned(16))) E ubuf[DR_ROWS * LD];
  __shared__ __attribute__((aligned(16))) E ulo[sizeof(E) == 2 ? DR_ROWS * LD : 16];
  __shared__ __attribute__((aligned(16))) float rbuf[DR_ROWS * RW];
  __shared__ float gate[ST_LMAX][DR_ROWS];
  __shared__ __attribute__((aligned(16))) E wbs[ST_LMAX * D];
  __shared__ float ctp[D * 4];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nbt = (B + DR_ROWS - 1) / DR_ROWS;
  const int bid = blockIdx.x;
  const int h = bid / (nbt * NFG);
  const int rest = bid % (nbt * NFG);
  const int b0 = (rest / NFG) * DR_ROWS, f0 = (rest % NFG) * FG;
  const int ft = wave & 3, half = wave >> 2;  // feature tile, half of the sequences
  const bool has = ft < FG / 16;              // this wave owns a feature tile
  const int n = f0 / 16 + ft;

  Frag wp[2][NK], wk[2][NK];
  auto load_w = [&](int l, Frag (&p)[NK], Frag (&k)[NK]) {
    const E* P = Wp + ((long)h * L + l) * D * D;
    const E* K = Wk + ((long)h * L + l) * D * D;
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
      p[kk] = load_fragK<E, D>(P, D, 16 * n, kk * KS, lane);
      k[kk] = load_fragK<E, D>(K, D, 16 * n, kk * KS, lane);
    }
  };
  if (has) {
    load_w(0, wp[0], wk[0]);
    if (L > 1) load_w(1, wp[1], wk[1]);
  }
  for (int e = tid; e < L * (D / VN); e += DR_NT)
    st16(wbs + e * VN, ld16(wbeta + (long)h * L * D + e * VN));
  for (int e = tid; e < D * 4; e += DR_NT) ctp[e] = to_f(conv[(long)h * D * 4 + e]);
  // tokens and histories of the thread's 16-byte chunks, x_s = v_{-s}:
  // x_0 is the token, x_s (s >= 1) history row 4 - s
  constexpr int NCHUNK = DR_ROWS * (D / VN);
  constexpr int NCH = (NCHUNK + DR_NT - 1) / DR_NT;
  uint4 xv[NCH][4 + OFF];
#pragma unroll
  for (int ci = 0; ci < NCH; ++ci) {
    const int e = tid + ci * DR_NT;
    const int r = e / (D / VN), c = (e % (D / VN)) * VN;
    const int bs = b0 + r;
#pragma unroll
    for (int s = 0; s < 4 + OFF; ++s) xv[ci][s] = uint4{0u, 0u, 0u, 0u};
    if (e < NCHUNK && bs < B) {
      xv[ci][0] = ld16(v + ((long)bs * H + h) * D + c);
      if (hist) {
#pragma unroll
        for (int s = 1; s < 4 + OFF; ++s) xv[ci][s] = ld16(hist + (((long)bs * 4 + 4 - s) * H + h) * D + c);
      }
    }
  }
  __syncthreads();   // taps and w_beta in LDS

  // anchor u of every feature (hi and lo parts, the MFMA operand) and the
  // residual r = v - u of this workgroup's features
#pragma unroll
  for (int ci = 0; ci < NCH; ++ci) {
    const int e = tid + ci * DR_NT;
    if (e >= NCHUNK) break;
    const int r = e / (D / VN), c = (e % (D / VN)) * VN;
#pragma unroll
    for (int j = 0; j < VN; ++j) {
      float x[4 + OFF];
#pragma unroll
      for (int s = 0; s < 4 + OFF; ++s) x[s] = to_f(reinterpret_cast<const E*>(&xv[ci][s])[j]);
      const float* tp = ctp + (c + j) * 4;
      const float u = tp[0] * x[OFF] + tp[1] * x[OFF + 1] + tp[2] * x[OFF + 2] + tp[3] * x[OFF + 3];
      const E uh = to_t<E>(u);
      ubuf[r * LD + c + j] = uh;
      if constexpr (sizeof(E) == 2) ulo[r * LD + c + j] = to_t<E>(u - to_f(uh));
      if (c + j >= f0 && c + j < f0 + FG) rbuf[r * RW + c + j - f0] = x[0] - u;
    }
  }
  __syncthreads();
  // step gates sigmoid(w_beta^(l) . u): GT threads per sequence
  {
    const int t = tid / GT, part = tid % GT;
    for (int l = 0; l < L; ++l) {
      float s = 0.f;
      for (int c = part * VN; c < D; c += GT * VN) {
        const uint4 ua = ld16(ubuf + t * LD + c), wa = ld16(wbs + l * D + c);
        const E* ue = reinterpret_cast<const E*>(&ua);
        const E* we = reinterpret_cast<const E*>(&wa);
#pragma unroll
        for (int j = 0; j < VN; ++j) s += to_f(we[j]) * to_f(ue[j]);
      }
#pragma unroll
      for (int off = GT / 2; off > 0; off >>= 1) s += __shfl_xor(s, off);
      if (part == 0) gate[l][t] = sigmoidf(s);
    }
  }
  __syncthreads();
  if (!has) return;   // no barrier follows

  // residual in the accumulator layout: (m, i) is sequence
  // rb + 16 m + 4 (lane >> 4) + i of the tile
  const int fl = 16 * ft + (lane & 15);
  const int rb = 16 * DR_MPW * half;
  float r[DR_MPW][4];
#pragma unroll
  for (int m = 0; m < DR_MPW; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i) r[m][i] = rbuf[(rb + 16 * m + 4 * (lane >> 4) + i) * RW + fl];

#pragma unroll
  for (int l = 0; l < ST_LMAX; ++l) {
    if (l >= L) break;
    const int sl = l & 1;
    f32x4 ap[DR_MPW], ak[DR_MPW];
#pragma unroll
    for (int m = 0; m < DR_MPW; ++m) ap[m] = ak[m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
#pragma unroll
      for (int m = 0; m < DR_MPW; ++m) {
        const Frag a = load_fragK<E, D>(ubuf, LD, rb + 16 * m, kk * KS, lane);
        ap[m] = MK::mma(a, wp[sl][kk], ap[m]);
        ak[m] = MK::mma(a, wk[sl][kk], ak[m]);
        if constexpr (sizeof(E) == 2) {
          const Frag al = load_fragK<E, D>(ulo, LD, rb + 16 * m, kk * KS, lane);
          ap[m] = MK::mma(al, wp[sl][kk], ap[m]);
        }
      }
    }
    if (l + 2 < L) load_w(l + 2, wp[sl], wk[sl]);
#pragma unroll
    for (int m = 0; m < DR_MPW; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = rb + 16 * m + 4 * (lane >> 4) + i;
        const float z = ap[m][i] * r[m][i];
        float dl;
        if constexpr (ACT == ACT_IDENTITY) dl = z;
        else dl = gelu_erf(z);
        r[m][i] -= dl;
        const int bs = b0 + row;
        if (bs < B) {
          const long o = (((long)bs * H + h) * L + l) * D + f0 + fl;
          Kl[o] = to_t<E>(ak[m][i]);
          Wl[o] = to_t<E>(gate[l][row] * dl);
        }
      }
  }
}

// out[b][r] = v_{T-4+r}, from hist (or zero) where T-4+r < 0.  One thread
// per (b, h, feature) reads its four values before writing any, so out may
// be hist itself.
template <typename E>
__global__ void conv_state_kernel(const E* __restrict__ v, const E* hist, E* out, int B, int T,
                                  int HD, const int* __restrict__ cu) {
  const long n = (long)B * HD;
  for (long e = blockIdx.x * (long)blockDim.x + threadIdx.x; e < n; e += (long)gridDim.x * blockDim.x) {
    const long b = e / HD, hf = e % HD;
    const long s0 = seq_start(cu, (int)b, T);
    const int Tb = seq_len(cu, (int)b, T);
    E x[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = Tb - 4 + r;
      x[r] = t >= 0 ? v[(s0 + t) * HD + hf] : hist ? hist[(b * 4 + 4 + t) * HD + hf] : to_t<E>(0.f);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) out[(b * 4 + r) * HD + hf] = x[r];
  }
}

__global__ void zero_kernel(float* p, long n) {
  for (long e = blockIdx.x * (long)blockDim.x + threadIdx.x; e < n; e += (long)gridDim.x * blockDim.x)
    p[e] = 0.f;
}

// One workgroup walks the B + 1 offsets in tiles of 256: clamp into [0, N],
// then a running maximum (inclusive max-scan in LDS, carried across tiles).
__global__ __launch_bounds__(256) void cu_sanitize_kernel(const int* __restrict__ cu,
                                                          int* __restrict__ out, int n, int N) {
  __shared__ int sm[256];
  const int tid = threadIdx.x;
  int carry = 0;
  for (int base = 0; base < n; base += 256) {
    const int i = base + tid;
    int x = i < n ? min(max(cu[i], 0), N) : 0;
    sm[tid] = x;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
      const int y = tid >= off ? sm[tid - off] : 0;
      __syncthreads();
      x = max(x, y);
      sm[tid] = x;
      __syncthreads();
    }
    if (i < n) out[i] = max(x, carry);
    carry = max(carry, sm[255]);
    __syncthreads();
  }
}

hipError_t launch_cu_sanitize(const Dims& d, int* out, hipStream_t s) {
  hipLaunchKernelGGL(cu_sanitize_kernel, dim3(1), dim3(256), 0, s, d.cu, out, d.B + 1, d.N);
  return hipGetLastError();
}

static unsigned grid_for(long n) {
  const long g = (n + 255) / 256;
  return (unsigned)(g < 4096 ? (g > 0 ? g : 1) : 4096);
}

template <typename E>
hipError_t launch_conv_state(const Dims& d, const E* v, const E* hist, E* out, hipStream_t s) {
  const long n = (long)d.B * d.H * d.D;
  hipLaunchKernelGGL((conv_state_kernel<E>), dim3(grid_for(n)), dim3(256), 0, s, v, hist, out, d.B,
                     d.T, d.H * d.D, d.cu);
  return hipGetLastError();
}

hipError_t launch_zero(float* p, long n, hipStream_t s) {
  hipLaunchKernelGGL(zero_kernel, dim3(grid_for(n)), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

template <typename E>
hipError_t launch_step(const Dims& d, const E* q, const E* k, const E* v, const float* alpha,
                       const float* beta, const E* Wk, const E* Wp, const E* wbeta, const E* conv,
                       float* S, E* cs, E* o, E* Kl, E* Wl, int stage, hipStream_t s) {
  if (d.L > ST_LMAX) return hipErrorInvalidValue;
  if (stage == 0) {
    if (d.L == 0) return hipSuccess;
    if (d.T > 1) {
      Dims r = d;
      r.Tp = d.T;   // pairs stored unpadded: [B, H, L, T, D]
      return launch_refine_fwd<E>(r, v, cs, conv, Wk, Wp, wbeta, Kl, Wl, s);
    }
    auto go = [&](auto kern, int nfg) {
      const int nblk = d.H * ((d.B + DR_ROWS - 1) / DR_ROWS) * nfg;
      hipLaunchKernelGGL(kern, dim3(nblk), dim3(DR_NT), 0, s, v, cs, conv, Wk, Wp, wbeta, Kl, Wl,
                         d.B, d.H, d.L);
      return hipGetLastError();
    };
    auto by_d = [&](auto dd) {
      constexpr int D = decltype(dd)::value;
      constexpr int nfg = D < DR_FG ? 1 : D / DR_FG;
      if (d.act == ACT_IDENTITY)
        return d.off ? go(decode_refine_kernel<E, D, ACT_IDENTITY, 1>, nfg)
                     : go(decode_refine_kernel<E, D, ACT_IDENTITY, 0>, nfg);
      return d.off ? go(decode_refine_kernel<E, D, ACT_GELU, 1>, nfg)
                   : go(decode_refine_kernel<E, D, ACT_GELU, 0>, nfg);
    };
    switch (d.D) {
      case 16: return by_d(std::integral_constant<int, 16>{});
      case 32: return by_d(std::integral_constant<int, 32>{});
      case 64: return by_d(std::integral_constant<int, 64>{});
      case 128: return by_d(std::integral_constant<int, 128>{});
    }
    return hipErrorInvalidValue;
  }
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3(d.B * d.H), dim3(64 * st_waves(d.D)), 0, s, q, k, v, alpha, beta,
                       Kl, Wl, S, cs, o, d.B, d.T, d.H, d.L);
    return hipGetLastError();
  };
  switch (d.D) {
    case 16: return go(step_state_kernel<E, 16>);
    case 32: return go(step_state_kernel<E, 32>);
    case 64: return go(step_state_kernel<E, 64>);
    case 128: return go(step_state_kernel<E, 128>);
  }
  return hipErrorInvalidValue;
}

template hipError_t launch_conv_state<bf16>(const Dims&, const bf16*, const bf16*, bf16*, hipStream_t);
template hipError_t launch_conv_state<float>(const Dims&, const float*, const float*, float*,
                                             hipStream_t);
template hipError_t launch_step<bf16>(const Dims&, const bf16*, const bf16*, const bf16*,
                                      const float*, const float*, const bf16*, const bf16*,
                                      const bf16*, const bf16*, float*, bf16*, bf16*, bf16*, bf16*,
                                      int, hipStream_t);
template hipError_t launch_step<float>(const Dims&, const float*, const float*, const float*,
                                       const float*, const float*, const float*, const float*,
                                       const float*, const float*, float*, float*, float*, float*,
                                       float*, int, hipStream_t);

}  // namespace prism
