// Token-by-token form of the PRISM layer (summary §2.1 "Write-Forget
// Decoupling" and §2.2 "Input-Anchored Loop Unrolling"): the decode step of
// serving, and the exact hand-over of a sequence from one call to the next.
//
// For each token of one (b, h):
//   u   = sum_j c[:, j] v_{t-o-j}        (ShortConv over the carried history)
//   r   = v - u;  for l: p = W_p^(l) u, k^(l) = W_k^(l) u,
//         g = sigmoid(w_beta^(l) . u), delta = act(p * r), r -= delta,
//         w^(l) = g delta
//   S  <- alpha (S - beta (S k) k^T) + beta v k^T + sum_l w^(l) k^(l)^T
//   o   = S q
// One workgroup owns one (b, h) for all T tokens: the fp32 state stays in
// registers between tokens, so it crosses HBM once per call (read and
// write, 8 D^2 bytes), which is what bounds a decode step.  Workgroups are
// ordered head-major so that the sequences of one head share an XCD and its
// L2 holds that head's weights.
#include "prism_common.h"
#include "prism_internal.h"

namespace prism {

constexpr int ST_NT = 256;
constexpr int ST_NW = ST_NT / WAVE;
constexpr int ST_LMAX = 8;

template <typename E, int D, int ACT, int OFF>
__global__ __launch_bounds__(ST_NT) void step_kernel(
    const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ v,
    const float* __restrict__ alpha, const float* __restrict__ beta, const E* __restrict__ Wk,
    const E* __restrict__ Wp, const E* __restrict__ wbeta, const E* __restrict__ conv,
    float* __restrict__ S, E* __restrict__ cstate, E* __restrict__ o, int B, int T, int H, int L) {
  constexpr int TPR = ST_NT / D;            // threads per state row
  constexpr int NCOL = D / TPR;             // state columns per thread
  constexpr int VN = 16 / (int)sizeof(E);   // weight elements per 16-byte load
  constexpr int LPR = D / VN;               // lanes per weight row
  constexpr int RPW = WAVE / LPR;           // weight rows per wave and pass
  constexpr int PS = 2 * D + 4;             // projections of one step: p, k^(l), gate logit
  __shared__ __attribute__((aligned(16))) float kv[D];
  __shared__ __attribute__((aligned(16))) float qv[D];
  __shared__ __attribute__((aligned(16))) float vv[D];
  __shared__ __attribute__((aligned(16))) float uv[D];
  __shared__ __attribute__((aligned(16))) float proj[ST_LMAX * PS];
  __shared__ __attribute__((aligned(16))) float wl[ST_LMAX * D];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nblk = B * H;
  const int bid = xcd_swizzle(blockIdx.x, nblk);
  const int h = bid / B, b = bid % B;
  const long bh = (long)b * H + h;
  const long tok = (long)H * D;
  const long base = ((long)b * T * H + h) * D;   // token t of this (b, h) at base + t * tok

  // state row `row`, columns c0 .. c0 + NCOL - 1
  const int row = tid / TPR, c0 = (tid % TPR) * NCOL;
  float* Sp = S + (bh * D + row) * D + c0;
  float s[NCOL];
  if constexpr (NCOL % 4 == 0) {
#pragma unroll
    for (int c = 0; c < NCOL; c += 4) *reinterpret_cast<f32x4*>(s + c) = *reinterpret_cast<const f32x4*>(Sp + c);
  } else {
#pragma unroll
    for (int c = 0; c < NCOL; ++c) s[c] = Sp[c];
  }
  // feature f = tid (< D): its taps and the four values before the sequence
  float tp[4] = {0.f, 0.f, 0.f, 0.f}, hv[4] = {0.f, 0.f, 0.f, 0.f};
  if (tid < D) {
    if (L > 0) {
#pragma unroll
      for (int j = 0; j < 4; ++j) tp[j] = to_f(conv[((long)h * D + tid) * 4 + j]);
    }
    if (cstate) {
#pragma unroll
      for (int r = 0; r < 4; ++r) hv[r] = to_f(cstate[(((long)b * 4 + r) * H + h) * D + tid]);
    }
  }
  const int nproj = L * PS;

  for (int t = 0; t < T; ++t) {
    const long at = base + t * tok;
    float vt = 0.f;
    if (tid < D) {
      vt = to_f(v[at + tid]);
      kv[tid] = to_f(k[at + tid]);
      qv[tid] = to_f(q[at + tid]);
      vv[tid] = vt;
    }
    const long ab = ((long)b * T + t) * H + h;
    const float a = alpha[ab], bt = beta[ab];
    float r = 0.f;
    if (L > 0 && tid < D) {
      float u;
      if constexpr (OFF == 0) u = tp[0] * vt + tp[1] * hv[3] + tp[2] * hv[2] + tp[3] * hv[1];
      else u = tp[0] * hv[3] + tp[1] * hv[2] + tp[2] * hv[1] + tp[3] * hv[0];
      uv[tid] = u;
      r = vt - u;
    }
    hv[0] = hv[1];
    hv[1] = hv[2];
    hv[2] = hv[3];
    hv[3] = vt;
    __syncthreads();

    if (L > 0) {
      // every projection of every step at once (none depends on the chain):
      // row n of step l = n / PS is W_p^(l) row m (m < D), W_k^(l) row m - D
      // (m < 2D) or w_beta^(l) (m = 2D); LPR lanes share one row
      const int sub = lane / LPR, part = lane % LPR;
      float ue[VN];
#pragma unroll
      for (int j = 0; j < VN; ++j) ue[j] = uv[part * VN + j];
      for (int n0 = wave * RPW; n0 < nproj; n0 += ST_NW * RPW) {
        const int n = n0 + sub;
        const int l = n / PS, m = n % PS;
        float acc = 0.f;
        if (n < nproj && m <= 2 * D) {
          const E* wr = m < D ? Wp + (((long)h * L + l) * D + m) * D
                       : m < 2 * D ? Wk + (((long)h * L + l) * D + (m - D)) * D
                                   : wbeta + ((long)h * L + l) * D;
          const uint4 x = ld16(wr + part * VN);
          const E* xe = reinterpret_cast<const E*>(&x);
#pragma unroll
          for (int j = 0; j < VN; ++j) acc += to_f(xe[j]) * ue[j];
        }
#pragma unroll
        for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
        if (part == 0 && n < nproj) proj[n] = acc;
      }
      __syncthreads();
      // the residual chain of feature tid
      if (tid < D) {
        for (int l = 0; l < L; ++l) {
          const float z = proj[l * PS + tid] * r;
          float dl;
          if constexpr (ACT == ACT_IDENTITY) dl = z;
          else dl = gelu_erf(z);
          r -= dl;
          wl[l * D + tid] = sigmoidf(proj[l * PS + 2 * D]) * dl;
        }
      }
      __syncthreads();
    }

    // S k for this row (TPR consecutive lanes share the row)
    float y = 0.f;
#pragma unroll
    for (int c = 0; c < NCOL; ++c) y += s[c] * kv[c0 + c];
#pragma unroll
    for (int off = TPR / 2; off > 0; off >>= 1) y += __shfl_xor(y, off);
    const float coef = bt * (vv[row] - a * y);
#pragma unroll
    for (int c = 0; c < NCOL; ++c) s[c] = a * s[c] + coef * kv[c0 + c];
    for (int l = 0; l < L; ++l) {
      const float wi = wl[l * D + row];
      const float* kl = proj + l * PS + D + c0;
#pragma unroll
      for (int c = 0; c < NCOL; ++c) s[c] += wi * kl[c];
    }
    float ot = 0.f;
#pragma unroll
    for (int c = 0; c < NCOL; ++c) ot += s[c] * qv[c0 + c];
#pragma unroll
    for (int off = TPR / 2; off > 0; off >>= 1) ot += __shfl_xor(ot, off);
    if (tid % TPR == 0) o[at + row] = to_t<E>(ot);
    __syncthreads();   // the next token rewrites kv, qv, vv, uv, proj, wl
  }

  if constexpr (NCOL % 4 == 0) {
#pragma unroll
    for (int c = 0; c < NCOL; c += 4) *reinterpret_cast<f32x4*>(Sp + c) = *reinterpret_cast<const f32x4*>(s + c);
  } else {
#pragma unroll
    for (int c = 0; c < NCOL; ++c) Sp[c] = s[c];
  }
  if (cstate && tid < D) {
#pragma unroll
    for (int r = 0; r < 4; ++r) cstate[(((long)b * 4 + r) * H + h) * D + tid] = to_t<E>(hv[r]);
  }
}

// out[b][r] = v_{T-4+r}, from hist (or zero) where T-4+r < 0.  One thread
// per (b, h, feature) reads its four values before writing any, so out may
// be hist itself.
template <typename E>
__global__ void conv_state_kernel(const E* __restrict__ v, const E* hist, E* out, int B, int T,
                                  int HD) {
  const long n = (long)B * HD;
  for (long e = blockIdx.x * (long)blockDim.x + threadIdx.x; e < n; e += (long)gridDim.x * blockDim.x) {
    const long b = e / HD, hf = e % HD;
    E x[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = T - 4 + r;
      x[r] = t >= 0 ? v[(b * T + t) * HD + hf] : hist ? hist[(b * 4 + 4 + t) * HD + hf] : to_t<E>(0.f);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) out[(b * 4 + r) * HD + hf] = x[r];
  }
}

__global__ void zero_kernel(float* p, long n) {
  for (long e = blockIdx.x * (long)blockDim.x + threadIdx.x; e < n; e += (long)gridDim.x * blockDim.x)
    p[e] = 0.f;
}

static unsigned grid_for(long n) {
  const long g = (n + 255) / 256;
  return (unsigned)(g < 4096 ? (g > 0 ? g : 1) : 4096);
}

template <typename E>
hipError_t launch_conv_state(const Dims& d, const E* v, const E* hist, E* out, hipStream_t s) {
  const long n = (long)d.B * d.H * d.D;
  hipLaunchKernelGGL((conv_state_kernel<E>), dim3(grid_for(n)), dim3(256), 0, s, v, hist, out, d.B,
                     d.T, d.H * d.D);
  return hipGetLastError();
}

hipError_t launch_zero(float* p, long n, hipStream_t s) {
  hipLaunchKernelGGL(zero_kernel, dim3(grid_for(n)), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

template <typename E, int D>
static hipError_t step_d(const Dims& d, const E* q, const E* k, const E* v, const float* alpha,
                         const float* beta, const E* Wk, const E* Wp, const E* wbeta,
                         const E* conv, float* S, E* cs, E* o, hipStream_t s) {
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3(d.B * d.H), dim3(ST_NT), 0, s, q, k, v, alpha, beta, Wk, Wp,
                       wbeta, conv, S, cs, o, d.B, d.T, d.H, d.L);
  };
  if (d.act == ACT_IDENTITY)
    d.off ? go(step_kernel<E, D, ACT_IDENTITY, 1>) : go(step_kernel<E, D, ACT_IDENTITY, 0>);
  else
    d.off ? go(step_kernel<E, D, ACT_GELU, 1>) : go(step_kernel<E, D, ACT_GELU, 0>);
  return hipGetLastError();
}

template <typename E>
hipError_t launch_step(const Dims& d, const E* q, const E* k, const E* v, const float* alpha,
                       const float* beta, const E* Wk, const E* Wp, const E* wbeta, const E* conv,
                       float* S, E* cs, E* o, hipStream_t s) {
  if (d.L > ST_LMAX) return hipErrorInvalidValue;
  switch (d.D) {
    case 16: return step_d<E, 16>(d, q, k, v, alpha, beta, Wk, Wp, wbeta, conv, S, cs, o, s);
    case 32: return step_d<E, 32>(d, q, k, v, alpha, beta, Wk, Wp, wbeta, conv, S, cs, o, s);
    case 64: return step_d<E, 64>(d, q, k, v, alpha, beta, Wk, Wp, wbeta, conv, S, cs, o, s);
    case 128: return step_d<E, 128>(d, q, k, v, alpha, beta, Wk, Wp, wbeta, conv, S, cs, o, s);
  }
  return hipErrorInvalidValue;
}

template hipError_t launch_conv_state<bf16>(const Dims&, const bf16*, const bf16*, bf16*, hipStream_t);
template hipError_t launch_conv_state<float>(const Dims&, const float*, const float*, float*,
                                             hipStream_t);
template hipError_t launch_step<bf16>(const Dims&, const bf16*, const bf16*, const bf16*,
                                      const float*, const float*, const bf16*, const bf16*,
                                      const bf16*, const bf16*, float*, bf16*, bf16*, hipStream_t);
template hipError_t launch_step<float>(const Dims&, const float*, const float*, const float*,
                                       const float*, const float*, const float*, const float*,
                                       const float*, const float*, float*, float*, float*,
                                       hipStream_t);

}  // namespace prism
