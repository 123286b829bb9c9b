// Weight gradients of the refinement backward and the dispatcher of its
// stages (PRISM summary §2.2): the transposed weights, the split-K MFMA GEMM
// dW_p^(l) = sum_t dp u^T, dW_k^(l) = sum_t dk^(l) u^T with its fixed-order
// reduction, and the reduction of the per-tile dw_beta and tap partials.  The
// per-token kernel itself is in refine_bwd_kernel.h.
#include "refine_bwd_kernel.h"

namespace prism {

int refine_bwd_tiles(const Dims& d) { return (d.T + rb_own(d.off) - 1) / rb_own(d.off); }

// Weight matrices in fragment order (frag_order_offset) for the projection
// kernels: up to four outputs, each a copy of W_p or W_k, or of a transpose.
// The forward takes W_p, W_k (p = W_p u, k = W_k u); the refinement backward
// W_p, W_p^T, W_k^T (du = W_p^T dp + W_k^T dk).  One thread per KPL-element
// piece of a fragment: it gathers the piece's KPL values (one 16-byte read
// from a row, or KPL strided reads for a transpose, where consecutive threads
// read consecutive columns) and writes them as one piece.
constexpr int TW_NT = 256;
template <typename E>
struct FragJobs {
  const E* src[4];
  E* dst[4];
  int trans[4];
};
template <typename E, int D>
__global__ __launch_bounds__(TW_NT) void weight_frags_kernel(FragJobs<E> jobs, int nout, int nmat) {
  typedef MfmaK<E, D> MK;
  constexpr int KS = MK::KSTEP, KPL = MK::KPL, NK = D / KS;
  constexpr int PIECES = D * D / KPL;
  const long gid = (long)blockIdx.x * TW_NT + threadIdx.x;
  if (gid >= (long)nout * nmat * PIECES) return;
  const int which = (int)(gid / ((long)nmat * PIECES));
  const long rem = gid % ((long)nmat * PIECES);
  const long m = rem / PIECES;
  const int c = (int)(rem % PIECES);
  const int l = c % 64, f = c / 64;
  const int nt = f / NK, kk = f % NK;
  const int row = 16 * nt + (l & 15), k0 = kk * KS + KPL * (l >> 4);
  const E* src = jobs.src[which] + m * D * D;
  const bool tr = jobs.trans[which] != 0;
  E x[KPL];
#pragma unroll
  for (int e = 0; e < KPL; ++e) x[e] = tr ? src[(long)(k0 + e) * D + row] : src[(long)row * D + k0 + e];
  __builtin_memcpy(jobs.dst[which] + m * D * D + (long)c * KPL, x, KPL * sizeof(E));
}

template <typename E, int D>
static hipError_t weight_frags_d(const Dims& d, const FragJobs<E>& j, int nout, hipStream_t s) {
  typedef MfmaK<E, D> MK;
  const long total = (long)nout * d.H * d.L * (D * D / MK::KPL);
  hipLaunchKernelGGL((weight_frags_kernel<E, D>), dim3((unsigned)((total + TW_NT - 1) / TW_NT)),
                     dim3(TW_NT), 0, s, j, nout, d.H * d.L);
  return hipGetLastError();
}

template <typename E>
hipError_t launch_weight_frags(const Dims& d, const E* Wk, const E* Wp, E* WpF, E* WkF, E* WpTF,
                               E* WkTF, hipStream_t s) {
  if (d.L == 0) return hipSuccess;
  FragJobs<E> j{};
  int n = 0;
  auto add = [&](const E* src, E* dst, int tr) {
    if (dst) {
      j.src[n] = src;
      j.dst[n] = dst;
      j.trans[n] = tr;
      ++n;
    }
  };
  add(Wp, WpF, 0);
  add(Wk, WkF, 0);
  add(Wp, WpTF, 1);
  add(Wk, WkTF, 1);
  if (n == 0) return hipSuccess;
  if (n > 4) return hipErrorInvalidValue;
  switch (d.D) {
    case 16: return weight_frags_d<E, 16>(d, j, n, s);
    case 32: return weight_frags_d<E, 32>(d, j, n, s);
    case 64: return weight_frags_d<E, 64>(d, j, n, s);
    case 128:
      if constexpr (sizeof(E) == 2) return weight_frags_d<E, 128>(d, j, n, s);
      break;
  }
  return hipErrorInvalidValue;
}
template hipError_t launch_weight_frags<bf16>(const Dims&, const bf16*, const bf16*, bf16*, bf16*,
                                              bf16*, bf16*, hipStream_t);
template hipError_t launch_weight_frags<float>(const Dims&, const float*, const float*, float*,
                                               float*, float*, float*, hipStream_t);

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
  static_assert(PER * RG <= 32, "validity bits");
  uint4 v[PER][RG];
  unsigned ok = 0;   // bit p * RG + q: the row of v[p][q] exists (else it reads as zeros)
  // Rows past the split or the sequence end read a row inside the tensor in
  // their place and are zeroed by store_t: no load sits in a per-lane branch
  // (its merge would make the prefetch wait for its data at issue).
  __device__ inline void load(const X* base, long rowstride_b, int Tp, int T, const int* cu, long n0,
                              long nend, int tid) {
    ok = 0;
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int u = min(tid + p * WG_NT, NU - 1);   // threads past the last unit read it again
      const int r0 = (u % NG) * RG, c = (u / NG) * VN;
#pragma unroll
      for (int q = 0; q < RG; ++q) {
        const long n = n0 + r0 + q;
        const long nc = n < nend ? n : nend - 1;
        const long bb = nc / Tp, t = nc % Tp;
        if (n < nend && t < seq_len(cu, (int)bb, T)) ok |= 1u << (p * RG + q);
        v[p][q] = ld16(base + bb * rowstride_b + t * D + c);
      }
    }
  }
  __device__ inline uint4 get(int p, int q) const {
    uint4 w = v[p][q];
    asm volatile("" : "+v"(w.x), "+v"(w.y), "+v"(w.z), "+v"(w.w));
    return (ok >> (p * RG + q)) & 1u ? w : uint4{0u, 0u, 0u, 0u};
  }
  __device__ inline void store_t(E* s, int ld, int tid) const {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int u = tid + p * WG_NT;
      if (u >= NU) continue;
      const int r0 = (u % NG) * RG, c = (u / NG) * VN;
      if constexpr (RG == 2) {
        const uint4 w0 = get(p, 0), w1 = get(p, 1);
        const X* x0 = reinterpret_cast<const X*>(&w0);
        const X* x1 = reinterpret_cast<const X*>(&w1);
#pragma unroll
        for (int j = 0; j < VN; ++j) {
          E pr[2] = {to_t<E>(to_f(x0[j])), to_t<E>(to_f(x1[j]))};
          uint32_t w;
          __builtin_memcpy(&w, pr, 4);
          *reinterpret_cast<uint32_t*>(s + (c + j) * ld + r0) = w;
        }
      } else {
        const uint4 w = get(p, 0);
        const X* x = reinterpret_cast<const X*>(&w);
#pragma unroll
        for (int j = 0; j < VN; ++j) s[(c + j) * ld + r0] = to_t<E>(to_f(x[j]));
      }
    }
  }
};

template <typename E, int D>
__global__ __launch_bounds__(WG_NT) void wgrad_gemm_kernel(const E* __restrict__ dKl,
                                                           const E* __restrict__ dP,
                                                           const E* __restrict__ u,
                                                           float* __restrict__ part, int B, int H,
                                                           int L, int T, int Tp, int NS,
                                                           const int* __restrict__ cu) {
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
  // rows of dK_l (which = 0) or dp_l (which = 1), and of u
  const E* xs = (which == 0 ? dKl : dP) + (((long)h * L + l) * Tp) * D;
  const E* ub = u + ((long)h * Tp) * D;
  RowChunk<E, E, D> xe, uu;
  // software pipeline: chunk n0 + 64 is fetched while chunk n0 is multiplied
  if (n_begin < n_end) {
    xe.load(xs, xs_b, Tp, T, cu, n_begin, n_end, tid);
    uu.load(ub, us_b, Tp, T, cu, n_begin, n_end, tid);
  }
  for (long n0 = n_begin; n0 < n_end; n0 += WG_ROWS) {
    xe.store_t(Xt, LTT, tid);
    uu.store_t(Ut, LTT, tid);
    __syncthreads();
    const long nn = n0 + WG_ROWS;
    if (nn < n_end) {
      xe.load(xs, xs_b, Tp, T, cu, nn, n_end, tid);
      uu.load(ub, us_b, Tp, T, cu, nn, n_end, tid);
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

// Fixed-order reduction of the split-K partial products into dW_k, dW_p: each
// thread sums four consecutive entries over the splits in split order.
__global__ void wgrad_reduce_kernel(const float* __restrict__ part, float* __restrict__ dWk,
                                    float* __restrict__ dWp, int H, int L, int D, int NS) {
  const long nW4 = (long)H * L * D * D / 4;
  for (long e = blockIdx.x * (long)blockDim.x + threadIdx.x; e < 2 * nW4; e += (long)gridDim.x * blockDim.x) {
    const int which = e < nW4 ? 0 : 1;
    const long x = (e - which * nW4) * 4;
    const long hl = x / ((long)D * D), ij = x % ((long)D * D);
    const float* p = part + ((hl * 2 + which) * NS) * (long)D * D + ij;
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
    for (int k = 0; k < NS; ++k) {
      const f32x4 y = *reinterpret_cast<const f32x4*>(p + (long)k * D * D);
#pragma unroll
      for (int c = 0; c < 4; ++c) s[c] += y[c];
    }
    *reinterpret_cast<f32x4*>((which == 0 ? dWk : dWp) + x) = s;
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
template <typename E, int D>
static hipError_t refine_bwd_d(const Dims& d, const RefineBwdArgs<E>& a, int NS, int stage,
                               hipStream_t s) {
  const int ntiles = refine_bwd_tiles(d);
  const long nw = (long)d.H * d.L * D * D;
  switch (stage) {
    case 0:   // (the caller may instead have formed them with launch_weight_frags)
      return launch_weight_frags<E>(d, a.Wk, a.Wp, a.WpF, nullptr, a.WpT, a.WkT, s);
    case 1:
      if (d.act == ACT_IDENTITY)
        return d.off ? launch_refine_bwd_main<E, ACT_IDENTITY, 1>(d, a, s)
                     : launch_refine_bwd_main<E, ACT_IDENTITY, 0>(d, a, s);
      return d.off ? launch_refine_bwd_main<E, ACT_GELU, 1>(d, a, s)
                   : launch_refine_bwd_main<E, ACT_GELU, 0>(d, a, s);
    case 2:
      hipLaunchKernelGGL((wgrad_gemm_kernel<E, D>), dim3(d.H * d.L * 2 * NS), dim3(WG_NT), 0, s,
                         a.dKl, a.dP, a.u, a.part, d.B, d.H, d.L, d.T, d.Tp, NS, d.cu);
      break;
    case 3: {
      const long n4 = 2 * nw / 4;
      const unsigned grid = (unsigned)((n4 + 255) / 256 < 8192 ? (n4 + 255) / 256 : 8192);
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

}  // namespace prism
