// Stage 1 (ShortConv anchor) and Stage 2 (L unrolled refinement steps) of the
// PRISM layer, one kernel.  PRISM technical summary §2.2 "Input-Anchored Loop
// Unrolling":
//   u_t      = sum_{j=0..3} c[:, j] * v_{t-o-j}    (depthwise causal conv over v;
//              o = 0 taps the current token, o = 1 strictly past tokens)
//   r^(1)    = v_t - u_t
//   k^(l)    = W_k^(l) u_t,  p^(l) = W_p^(l) u_t,  beta^(l) = sigmoid(w_beta^(l) . u_t)
//   delta^(l)= GELU(p^(l) * r^(l)) (or p^(l) * r^(l)),  r^(l+1) = r^(l) - delta^(l)
//   output pairs (k^(l), w^(l) = beta^(l) delta^(l)), whose outer products form
//   the rank-L injection B_t of §2.2.
//
// The step is elementwise per token apart from the two projections, so it is
// HBM-bound: read v once, write 2 L rows per token.  One workgroup owns 64
// tokens of one (b, h); wave w owns output features {16 n : n = w mod 4} for
// all 64 tokens.  Its weight fragments come straight from global memory (each
// weight row is read by exactly one wave per workgroup), the anchor u is the
// shared MFMA A operand in LDS, and the residual chain stays in registers in
// the accumulator layout.  Outputs are staged in LDS and stored as full
// 16-byte rows.
// Multiply-adds fuse only within one expression (the C rule), never across
// statements: the refinement kernel and the chunk kernel that repeats its
// arithmetic then round identically, whatever code surrounds each.
#pragma clang fp contract(on)
#include "prism_common.h"
#include "prism_internal.h"

namespace prism {

constexpr int RF_TT = 64;    // tokens per workgroup
constexpr int RF_NT = 256;   // threads per workgroup
constexpr int RF_NW = 4;

template <typename E, int D, int ACT, int OFF>
__global__ __launch_bounds__(RF_NT) void refine_fwd_kernel(
    const E* __restrict__ v, const E* __restrict__ hist, const E* __restrict__ conv,
    const E* __restrict__ Wk, const E* __restrict__ Wp, const E* __restrict__ wbeta,
    E* __restrict__ Kl, E* __restrict__ Wl, int B, int T, int H, int L, int Tp,
    const int* __restrict__ cu) {
  constexpr int LD = ldpad<E>(D);
  constexpr int NFT = D / 16;                          // feature tiles
  constexpr int FPW = (NFT + RF_NW - 1) / RF_NW;       // feature tiles per wave
  // feature tile n exists; always true when the tiles divide evenly over the
  // feature groups (then the test folds away at compile time)
#define FT_OK(n) (NFT % RF_NW == 0 || (n) < NFT)
  typedef MfmaK<E, D> MK;
  constexpr int KS = MK::KSTEP;
  constexpr int NK = D / KS;
  constexpr int VN = 16 / sizeof(E);
  constexpr int HL = 3 + OFF;   // v rows before the tile that the taps reach

  // v rows (t0-HL .. t0+63) until the residual is formed, then the k^(l) staging tile
  constexpr int VB = cmax((RF_TT + HL) * D, RF_TT * LD);
  __shared__ __attribute__((aligned(16))) E vbuf[VB];
  E* obk = vbuf;
  __shared__ __attribute__((aligned(16))) E ubuf[RF_TT * LD];
  // bf16 only: u - bf16(u), so that p^(l) = W_p^(l) (u_hi + u_lo) is fp32-accurate
  // (the GELU chain amplifies errors in p; k^(l) uses u_hi alone)
  __shared__ __attribute__((aligned(16))) E ulo[sizeof(E) == 2 ? RF_TT * LD : 16];
  __shared__ __attribute__((aligned(16))) E obw[RF_TT * LD];
  __shared__ float gate[8][RF_TT];
  __shared__ __attribute__((aligned(16))) E wbs[8 * D];   // w_beta^(l) rows of this head

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ntiles = Tp / RF_TT + ((Tp % RF_TT) ? 1 : 0);
  const int nblk = ntiles * B * H;
  const int bid = xcd_swizzle(blockIdx.x, nblk);
  // head-major logical order: one XCD sees a contiguous range of heads
  const int h = bid / (B * ntiles);
  const int rest = bid % (B * ntiles);
  const int b = rest / ntiles, tile = rest % ntiles;
  const int t0 = tile * RF_TT;
  const long tok_stride = (long)H * D;
  const E* vseq = v + (seq_start(cu, b, T) * H + h) * D;   // row t at vseq + t * tok_stride
  const int Tb = seq_len(cu, b, T);
  // a tile past the end of a packed sequence lies past its last chunk (tiles
  // are multiples of the chunk length): nothing reads it.  Never in a dense
  // batch, whose tiles all start before T.
  if (t0 >= Tb) return;

  // ---- w_beta rows of this head (L x D) and the v rows t0-HL .. t0+63
  //      (zeros past T; before 0 the history rows [B, 4, H, D], or zeros
  //      without a history): every read issued before the first store (one
  //      memory round trip, where a copy loop that stores each vector as it
  //      arrives waits once per iteration), none in a per-lane branch
  //      (out-of-range rows read row 0 and are zeroed at the store) ----
  {
    constexpr int NWB = 8 * (D / VN), PWB = (NWB + RF_NT - 1) / RF_NT;
    constexpr int NVB = (RF_TT + HL) * (D / VN), PVB = (NVB + RF_NT - 1) / RF_NT;
    const int nwb = L * (D / VN);
    uint4 wbv[PWB], vbv[PVB];
    bool vz[PVB];
#pragma unroll
    for (int p = 0; p < PWB; ++p)   // (L >= 1: nwb > 0)
      wbv[p] = ld16(wbeta + (long)h * L * D + (long)min(tid + p * RF_NT, nwb - 1) * VN);
#pragma unroll
    for (int p = 0; p < PVB; ++p) {
      const int e = min(tid + p * RF_NT, NVB - 1);
      const int r = e / (D / VN), c = (e % (D / VN)) * VN;
      const int t = t0 - HL + r;
      const bool in_seq = t >= 0 && t < Tb, in_hist = t < 0 && hist;
      vz[p] = !in_seq && !in_hist;
      const E* src = in_seq ? vseq + t * tok_stride + c
                   : in_hist ? hist + (((long)b * 4 + 4 + t) * H + h) * D + c : vseq + c;
      vbv[p] = ld16(src);
    }
#pragma unroll
    for (int p = 0; p < PWB; ++p)
      if (tid + p * RF_NT < nwb) st16(wbs + (tid + p * RF_NT) * VN, wbv[p]);
#pragma unroll
    for (int p = 0; p < PVB; ++p) {
      const int e = tid + p * RF_NT;
      if (e < NVB) {
        uint4 x = vbv[p];
        asm volatile("" : "+v"(x.x), "+v"(x.y), "+v"(x.z), "+v"(x.w));
        if (vz[p]) x = uint4{0u, 0u, 0u, 0u};
        const int r = e / (D / VN), c = (e % (D / VN)) * VN;
        st16(vbuf + r * D + c, x);
      }
    }
  }
  typedef typename MK::frag Frag;
  auto load_w = [&](const E* W, Frag (&bw)[FPW][NK]) {
#pragma unroll
    for (int nn = 0; nn < FPW; ++nn) {
      const int n = wave + RF_NW * nn;
#pragma unroll
      for (int kk = 0; kk < NK; ++kk)
        if (FT_OK(n)) bw[nn][kk] = load_fragK<E, D>(W, D, 16 * n, kk * KS, lane);
    }
  };
  // taps of the lane's features, requested with the v rows (one round trip)
  // and before the W_p^(1) fragments: their wait (at the set-up's barrier)
  // then leaves the fragments, first used after the gates, in flight
  const E* ch = conv + (long)h * D * 4;
  float taps[FPW][4];
#pragma unroll
  for (int nn = 0; nn < FPW; ++nn) {
    const int n = wave + RF_NW * nn;
    const int f = 16 * n + (lane & 15);
#pragma unroll
    for (int j = 0; j < 4; ++j) taps[nn][j] = (FT_OK(n)) ? to_f(ch[f * 4 + j]) : 0.f;
  }
  Frag bw[FPW][NK];   // weight fragments of the next projection (W_p^(1) now)
  // (unconditional: the kernel runs only with L >= 1, and a branch here made
  // the taps' wait cover these fragments at its join)
  load_w(Wp + (long)h * L * D * D, bw);
  __syncthreads();

  // ---- anchor u (fp32; to LDS as the MFMA operand, hi and lo parts) and
  //      residual r^(1) = v - u, both in the accumulator layout:
  //      element (m, n, i): token 16 m + 4 (lane >> 4) + i, feature 16 n + (lane & 15)
  float r[4][FPW][4];
#pragma unroll
  for (int nn = 0; nn < FPW; ++nn) {
    const int n = wave + RF_NW * nn;
    const int f = 16 * n + (lane & 15);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      // the lane's four tokens t0m .. t0m + 3 read v rows t0m .. t0m + 6 + o
      // of the tile (tap j of token t is row t + 3 - j, the token itself row
      // t + 3 + o): each row once
      const int t0m = 16 * m + 4 * (lane >> 4);
      float w[7 + OFF];
#pragma unroll
      for (int q = 0; q < 7 + OFF; ++q) w[q] = FT_OK(n) ? to_f(vbuf[(t0m + q) * D + f]) : 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = t0m + i;
        float u = 0.f, val = 0.f;
        if (FT_OK(n) && t0 + t < Tb) {
#pragma unroll
          for (int j = 0; j < 4; ++j) u += taps[nn][j] * w[i + 3 - j];
          val = w[i + 3 + OFF] - u;
        }
        r[m][nn][i] = val;
        if (FT_OK(n)) {
          const E uh = to_t<E>(u);
          ubuf[t * LD + f] = uh;
          if constexpr (sizeof(E) == 2) ulo[t * LD + f] = to_t<E>(u - to_f(uh));
        }
      }
    }
  }
  __syncthreads();

  // ---- step gates beta^(l) = sigmoid(w_beta^(l) . u): 4 threads per token,
  //      16-byte reads of u and w_beta ----
  {
    const int t = tid >> 2, part = tid & 3;
    for (int l = 0; l < L; ++l) {
      float s = 0.f;
      for (int c = part * VN; c < D; c += 4 * VN) {
        const uint4 ua = ld16(ubuf + t * LD + c), wa = ld16(wbs + l * D + c);
        const E* ue = reinterpret_cast<const E*>(&ua);
        const E* we = reinterpret_cast<const E*>(&wa);
#pragma unroll
        for (int j = 0; j < VN; ++j) s += to_f(we[j]) * to_f(ue[j]);
      }
      s = quad_sum(s);
      if (part == 0) gate[l][t] = sigmoidf(s);
    }
  }
  __syncthreads();   // gates visible

  E* Klseq = Kl + (((long)b * H + h) * L) * Tp * D;
  E* Wlseq = Wl + (((long)b * H + h) * L) * Tp * D;
  const int nvalid = min(RF_TT, Tp - t0);

  // Per step l: gain pass p = W_p (u_hi + u_lo) -> chain -> w; direction pass
  // k = W_k u_hi.  Weight fragments of the next pass are requested before the
  // current pass's arithmetic so their latency overlaps it.
  auto gemm = [&](const Frag (&bw)[FPW][NK], bool with_lo, f32x4 (&acc)[4][FPW]) {
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int nn = 0; nn < FPW; ++nn) acc[m][nn] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
      Frag a[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) a[m] = load_fragK<E, D>(ubuf, LD, 16 * m, kk * KS, lane);
#pragma unroll
      for (int nn = 0; nn < FPW; ++nn)
        if (FT_OK(wave + RF_NW * nn)) {
#pragma unroll
          for (int m = 0; m < 4; ++m) acc[m][nn] = MK::mma(a[m], bw[nn][kk], acc[m][nn]);
        }
      if constexpr (sizeof(E) == 2) {
        if (with_lo) {
#pragma unroll
          for (int m = 0; m < 4; ++m) a[m] = load_fragK<E, D>(ulo, LD, 16 * m, kk * KS, lane);
#pragma unroll
          for (int nn = 0; nn < FPW; ++nn)
            if (FT_OK(wave + RF_NW * nn)) {
#pragma unroll
              for (int m = 0; m < 4; ++m) acc[m][nn] = MK::mma(a[m], bw[nn][kk], acc[m][nn]);
            }
        }
      }
    }
  };

  for (int l = 0; l < L; ++l) {
    const E* wk = Wk + ((long)h * L + l) * D * D;
    f32x4 acc[4][FPW];
    gemm(bw, true, acc);                       // p^(l)
    load_w(wk, bw);                            // prefetch W_k^(l)
    // residual chain, one step
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int nn = 0; nn < FPW; ++nn) {
        const int n = wave + RF_NW * nn;
        if (FT_OK(n)) {
          const int f = 16 * n + (lane & 15);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int t = 16 * m + 4 * (lane >> 4) + i;
            const float z = acc[m][nn][i] * r[m][nn][i];
            float dl;
            if constexpr (ACT == ACT_IDENTITY) dl = z;
            else dl = gelu_erf(z);
            r[m][nn][i] -= dl;
            obw[t * LD + f] = to_t<E>(gate[l][t] * dl);
          }
        }
      }
    gemm(bw, false, acc);                      // k^(l)
    if (l + 1 < L) load_w(Wp + ((long)h * L + l + 1) * D * D, bw);   // prefetch W_p^(l+1)
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int nn = 0; nn < FPW; ++nn) {
        const int n = wave + RF_NW * nn;
        if (FT_OK(n)) {
          const int f = 16 * n + (lane & 15);
#pragma unroll
          for (int i = 0; i < 4; ++i) obk[(16 * m + 4 * (lane >> 4) + i) * LD + f] = to_t<E>(acc[m][nn][i]);
        }
      }
    __syncthreads();
    s2g_rows<E, RF_TT, D, RF_NT>(Klseq + ((long)l * Tp + t0) * D, D, obk, LD, nvalid, tid);
    s2g_rows<E, RF_TT, D, RF_NT>(Wlseq + ((long)l * Tp + t0) * D, D, obw, LD, nvalid, tid);
    __syncthreads();
  }
}

template <typename E, int D>
static hipError_t refine_launch_d(const Dims& d, const E* v, const E* hist, const E* conv,
                                  const E* Wk, const E* Wp, const E* wbeta, E* Kl, E* Wl,
                                  hipStream_t s) {
  const int ntiles = (d.Tp + RF_TT - 1) / RF_TT;
  const int nblk = ntiles * d.B * d.H;
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3(nblk), dim3(RF_NT), 0, s, v, hist, conv, Wk, Wp, wbeta, Kl, Wl,
                       d.B, d.T, d.H, d.L, d.Tp, d.cu);
  };
  if (d.act == ACT_IDENTITY)
    d.off ? go(refine_fwd_kernel<E, D, ACT_IDENTITY, 1>) : go(refine_fwd_kernel<E, D, ACT_IDENTITY, 0>);
  else
    d.off ? go(refine_fwd_kernel<E, D, ACT_GELU, 1>) : go(refine_fwd_kernel<E, D, ACT_GELU, 0>);
  return hipGetLastError();
}

template <typename E>
hipError_t launch_refine_fwd(const Dims& d, const E* v, const E* hist, const E* conv, const E* Wk,
                             const E* Wp, const E* wbeta, E* Kl, E* Wl, hipStream_t s) {
  if (d.L == 0) return hipSuccess;
  switch (d.D) {
    case 16: return refine_launch_d<E, 16>(d, v, hist, conv, Wk, Wp, wbeta, Kl, Wl, s);
    case 32: return refine_launch_d<E, 32>(d, v, hist, conv, Wk, Wp, wbeta, Kl, Wl, s);
    case 64: return refine_launch_d<E, 64>(d, v, hist, conv, Wk, Wp, wbeta, Kl, Wl, s);
    case 128:
      if constexpr (sizeof(E) == 2)
        return refine_launch_d<E, 128>(d, v, hist, conv, Wk, Wp, wbeta, Kl, Wl, s);
      break;
  }
  return hipErrorInvalidValue;
}

template hipError_t launch_refine_fwd<bf16>(const Dims&, const bf16*, const bf16*, const bf16*,
                                            const bf16*, const bf16*, const bf16*, bf16*, bf16*,
                                            hipStream_t);
template hipError_t launch_refine_fwd<float>(const Dims&, const float*, const float*, const float*,
                                             const float*, const float*, const float*, float*,
                                             float*, hipStream_t);

#undef FT_OK
}  // namespace prism
