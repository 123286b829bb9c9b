// C ABI of the PRISM layer: argument validation, workspace carving and the
// launch sequence.  The launch sequence of the forward pass is
//   refine_fwd  (ShortConv anchor + L refinement steps, summary §2.2)
//   chunk_fwd   (chunk-local affine maps of S_t = S_{t-1} A_t + B_t, §2.1)
//   state_fwd   (sequential pass over chunks, fp32 state, with the readout
//                o_t = S_t q_t of each chunk formed in the same step)
// The training pair keeps the forward's refinement pairs, chunk maps, chunk
// states and solve results in a caller buffer, so that its backward starts at
// the reverse state pass instead of recomputing them.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/prism.h"
#include "prism_internal.h"

namespace {

thread_local std::string g_err;

prism_status fail(prism_status st, const std::string& msg) {
  g_err = msg;
  return st;
}

// ---------------------------------------------------------------- timing
struct TimedLaunch {
  const char* name;
  hipEvent_t a, b;
};
bool g_timing = false;
std::vector<TimedLaunch> g_launches;
std::vector<hipEvent_t> g_pool;

hipEvent_t pool_event() {
  if (!g_pool.empty()) {
    hipEvent_t e = g_pool.back();
    g_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

template <typename F>
hipError_t timed(const char* name, hipStream_t s, F&& f) {
  if (!g_timing) return f();
  hipEvent_t a = pool_event(), b = pool_event();
  if (a) (void)hipEventRecord(a, s);
  hipError_t err = f();
  if (b) (void)hipEventRecord(b, s);
  if (a && b) g_launches.push_back({name, a, b});
  return err;
}

// ---------------------------------------------------------------- layout
size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct Carve {
  size_t off = 0;
  char* base = nullptr;
  template <typename P>
  P* take(size_t bytes) {
    P* p = base ? reinterpret_cast<P*>(base + off) : nullptr;
    off += align256(bytes);
    return p;
  }
};

template <typename E>
struct FwdWs {
  E *Kl, *Wl, *Mt, *Qt, *Sc, *UT, *WkT;
  E *HT, *Oloc;   // H^T and O_loc per chunk (storage type)
  float* gC;
  int* cu;        // sanitised packed-batch offsets (packed batches only)
};

// What a training forward keeps for its backward (caller-owned buffer).
template <typename E>
struct Kept {
  E *Kl, *Wl, *Mt, *Qt, *Sc, *UT, *WkT;
  float* gC;
};

template <typename E>
Kept<E> carve_kept(const prism::Dims& d, Carve& cv) {
  const size_t bh = (size_t)d.B * d.H;
  const size_t es = sizeof(E);
  const size_t DD = (size_t)d.D * d.D, CD = (size_t)d.C * d.D;
  Kept<E> k;
  k.Kl = cv.take<E>(bh * d.L * d.Tp * d.D * es);
  k.Wl = cv.take<E>(bh * d.L * d.Tp * d.D * es);
  k.Mt = cv.take<E>(bh * d.NC * DD * es);
  k.Qt = cv.take<E>(bh * d.NC * CD * es);
  k.Sc = cv.take<E>(bh * d.NC * DD * es);
  k.UT = cv.take<E>(bh * d.NC * CD * es);
  k.WkT = cv.take<E>(bh * d.NC * CD * es);
  k.gC = cv.take<float>(bh * d.NC * 4);
  return k;
}

template <typename E>
FwdWs<E> carve_fwd(const prism::Dims& d, Carve& cv, bool train) {
  const size_t bh = (size_t)d.B * d.H;
  const size_t es = sizeof(E);
  FwdWs<E> w;
  // No room for the refinement pairs: the inference forward forms them inside
  // the chunk kernel, the training forward keeps them in its buffer.  The
  // training forward also keeps M^T, Qt, gC, S_c, U^T, W_k^T there; the
  // inference forward stores no S_c at all.
  w.Kl = w.Wl = nullptr;
  w.Sc = w.UT = w.WkT = nullptr;
  w.Mt = train ? nullptr : cv.take<E>(bh * d.NC * d.D * d.D * es);
  w.HT = cv.take<E>(bh * d.NC * d.D * d.D * sizeof(E));
  w.Qt = train ? nullptr : cv.take<E>(bh * d.NC * d.C * d.D * es);
  w.Oloc = cv.take<E>(bh * d.NC * d.C * d.D * sizeof(E));
  w.gC = train ? nullptr : cv.take<float>(bh * d.NC * 4);
  w.cu = cv.take<int>(((size_t)d.B + 1) * 4);
  return w;
}

// ---------------------------------------------------------------- checks
prism_status check_desc(const prism_desc* desc, prism::Dims* out) {
  if (!desc) return fail(PRISM_ERR_NULL, "desc is NULL");
  const prism_desc& d = *desc;
  if (d.B < 1 || d.T < 1 || d.H < 1)
    return fail(PRISM_ERR_SHAPE, "B, T and H must be >= 1 (got B=" + std::to_string(d.B) +
                                     " T=" + std::to_string(d.T) + " H=" + std::to_string(d.H) + ")");
  if (d.dk < 1 || d.dv < 1 || d.L < 0 || d.chunk < 1 || d.conv_width < 1)
    return fail(PRISM_ERR_SHAPE, "dk, dv, chunk, conv_width must be >= 1 and L >= 0");
  if (d.dtype != PRISM_F32 && d.dtype != PRISM_BF16)
    return fail(PRISM_ERR_UNSUPPORTED, "dtype must be PRISM_F32 or PRISM_BF16");
  if (d.dk != d.dv) return fail(PRISM_ERR_UNSUPPORTED, "dk must equal dv");
  const bool dok = d.dk == 16 || d.dk == 32 || d.dk == 64 || (d.dk == 128 && d.dtype == PRISM_BF16);
  if (!dok)
    return fail(PRISM_ERR_UNSUPPORTED, "head dimension " + std::to_string(d.dk) +
                                           " not supported (bf16: 16/32/64/128, f32: 16/32/64)");
  if (d.L > 8) return fail(PRISM_ERR_UNSUPPORTED, "L must be <= 8");
  if (d.dtype == PRISM_F32 && d.dk * d.chunk > 2048)
    return fail(PRISM_ERR_UNSUPPORTED, "PRISM_F32 needs dk * chunk <= 2048 (d=64: chunk <= 32)");
  if (d.chunk != 16 && d.chunk != 32 && d.chunk != 64)
    return fail(PRISM_ERR_UNSUPPORTED, "chunk must be 16, 32 or 64");
  if (d.conv_width != 4) return fail(PRISM_ERR_UNSUPPORTED, "conv_width must be 4");
  if (d.activation != PRISM_ACT_GELU && d.activation != PRISM_ACT_IDENTITY)
    return fail(PRISM_ERR_UNSUPPORTED, "activation must be PRISM_ACT_GELU or PRISM_ACT_IDENTITY");
  if (d.conv_offset != 0 && d.conv_offset != 1)
    return fail(PRISM_ERR_UNSUPPORTED, "conv_offset must be 0 or 1");
  // a token row is H * dk elements apart: the kernels address a tile of up to
  // 64 rows by 32-bit byte offsets from its base
  if ((long long)d.H * d.dk > (1LL << 22))
    return fail(PRISM_ERR_SHAPE, "H * dk must be <= 4194304 (got " + std::to_string((long long)d.H * d.dk) + ")");
  const double elems = (double)d.B * d.T * d.H * d.dk * (d.L + 1);
  if (elems > 4.0e12) return fail(PRISM_ERR_SHAPE, "problem too large");
  if ((long long)d.B * d.H * ((d.T + d.chunk - 1) / d.chunk) > 0x7fffffffLL)
    return fail(PRISM_ERR_SHAPE, "too many chunks for one launch");
  prism::Dims x;
  x.B = d.B;
  x.T = d.T;
  x.H = d.H;
  x.D = d.dk;
  x.L = d.L;
  x.C = d.chunk;
  x.NC = (d.T + d.chunk - 1) / d.chunk;
  x.Tp = x.NC * x.C;
  x.act = d.activation == PRISM_ACT_IDENTITY ? prism::ACT_IDENTITY : prism::ACT_GELU;
  x.off = d.conv_offset;
  *out = x;
  return PRISM_OK;
}

prism_status check_ptr(const void* p, const char* name, bool required) {
  if (!p) return required ? fail(PRISM_ERR_NULL, std::string(name) + " is NULL") : PRISM_OK;
  if (reinterpret_cast<uintptr_t>(p) & 15u)
    return fail(PRISM_ERR_ALIGN, std::string(name) + " is not 16-byte aligned");
  return PRISM_OK;
}

// Packed batches: the offsets must be a 4-byte aligned device array and the
// packed tensors' row count N must be given; the offsets themselves are read
// on the device only, where a sanitising pass clamps them into [0, N] before
// any kernel uses them (prism::launch_cu_sanitize).
prism_status check_cu(const int* cu, const prism_desc* desc, prism::Dims* d) {
  if (cu && (reinterpret_cast<uintptr_t>(cu) & 3u))
    return fail(PRISM_ERR_ALIGN, "cu_seqlens is not 4-byte aligned");
  if (cu && desc->packed_tokens < 0)
    return fail(PRISM_ERR_SHAPE, "packed_tokens must be >= 0 with cu_seqlens");
  d->cu = cu;
  d->N = cu ? desc->packed_tokens : 0;
  return PRISM_OK;
}

#define CHECK_PTR(p, req)                              \
  do {                                                 \
    prism_status st_ = check_ptr((p), #p, (req));      \
    if (st_ != PRISM_OK) return st_;                   \
  } while (0)

#define HIP_TRY(name, stream, expr)                                                   \
  do {                                                                               \
    hipError_t e_ = timed((name), (stream), [&]() { return (expr); });               \
    if (e_ != hipSuccess)                                                            \
      return fail(PRISM_ERR_HIP, std::string(name) + ": " + hipGetErrorString(e_));   \
  } while (0)

template <typename E>
struct BwdWs {
  E *Kl, *Wl, *Mt, *UT, *WkT, *Sc, *dSnT, *u, *dP, *WkW, *WpW, *WpF, *dKl;
  float* dWl;
  E *dQt, *dUs, *dWks, *dKs, *dVp, *dqp, *dkp;
  E *HT, *ET;     // H^T, E^T per chunk (storage type)
  float *gC, *dgs, *dgp;
  float *dwbp, *dcp, *part;
  int* cu;        // sanitised packed-batch offsets (packed batches only)
};

template <typename E>
BwdWs<E> carve_bwd(const prism::Dims& d, Carve& cv, bool train) {
  const size_t bh = (size_t)d.B * d.H;
  const size_t es = sizeof(E);
  const size_t DD = (size_t)d.D * d.D, CD = (size_t)d.C * d.D;
  const size_t ntiles = (size_t)prism::refine_bwd_tiles(d);
  const size_t L1 = d.L > 0 ? d.L : 1;
  BwdWs<E> w;
  // the forward intermediates: recomputed by the stateless backward, read
  // from the saved buffer by the training backward (which forms E itself and
  // needs no H^T)
  w.Kl = w.Wl = w.Mt = w.HT = w.ET = w.UT = w.WkT = w.Sc = nullptr;
  w.gC = nullptr;
  if (!train) {
    w.Kl = cv.take<E>(bh * d.L * d.Tp * d.D * es);
    w.Wl = cv.take<E>(bh * d.L * d.Tp * d.D * es);
    w.Mt = cv.take<E>(bh * d.NC * DD * es);
    w.HT = cv.take<E>(bh * d.NC * DD * es);
    w.ET = cv.take<E>(bh * d.NC * DD * es);
    w.gC = cv.take<float>(bh * d.NC * 4);
    w.UT = cv.take<E>(bh * d.NC * CD * es);
    w.WkT = cv.take<E>(bh * d.NC * CD * es);
    w.Sc = cv.take<E>(bh * d.NC * DD * es);
  }
  w.dSnT = cv.take<E>(bh * d.NC * DD * es);
  w.dQt = cv.take<E>(bh * d.NC * CD * es);
  w.dUs = cv.take<E>(bh * d.NC * CD * es);
  w.dWks = cv.take<E>(bh * d.NC * CD * es);
  w.dKs = cv.take<E>(bh * d.NC * CD * es);
  w.dVp = cv.take<E>(bh * d.NC * CD * es);
  w.dqp = cv.take<E>(bh * d.NC * CD * es);
  w.dkp = cv.take<E>(bh * d.NC * CD * es);
  w.dKl = cv.take<E>(bh * d.L * d.Tp * d.D * es);
  w.dWl = cv.take<float>(bh * d.L * d.Tp * d.D * 4);
  w.dgs = cv.take<float>(bh * d.NC * d.C * 4);
  w.dgp = cv.take<float>(bh * d.NC * d.C * 4);
  w.u = cv.take<E>(bh * d.Tp * d.D * es);
  w.dP = cv.take<E>(bh * d.L * d.Tp * d.D * es);
  w.dwbp = cv.take<float>(bh * ntiles * L1 * d.D * 4);
  w.dcp = cv.take<float>(bh * ntiles * d.D * 4 * 4);
  w.part = cv.take<float>((size_t)d.H * L1 * 2 * prism::refine_bwd_splits(d) * DD * 4);
  w.WkW = cv.take<E>((size_t)d.H * d.L * DD * es);
  w.WpW = cv.take<E>((size_t)d.H * d.L * DD * es);
  w.WpF = cv.take<E>((size_t)d.H * d.L * DD * es);
  w.cu = cv.take<int>(((size_t)d.B + 1) * 4);
  return w;
}

size_t bwd_ws_bytes(const prism::Dims& d, prism_dtype dt, bool train) {
  Carve cv;
  if (dt == PRISM_BF16)
    carve_bwd<prism::bf16>(d, cv, train);
  else
    carve_bwd<float>(d, cv, train);
  return cv.off;
}

size_t kept_bytes(const prism::Dims& d, prism_dtype dt) {
  Carve cv;
  if (dt == PRISM_BF16)
    carve_kept<prism::bf16>(d, cv);
  else
    carve_kept<float>(d, cv);
  return cv.off;
}

// prism_step: the refinement pairs of every token, two arrays of
// B * H * L * T * D elements, each rounded up to 256 bytes
size_t step_ws_bytes(const prism::Dims& d, prism_dtype dt) {
  const size_t es = dt == PRISM_BF16 ? 2 : 4;
  const size_t one = ((size_t)d.B * d.H * d.L * d.T * d.D * es + 255) / 256 * 256;
  return 2 * one;
}

size_t fwd_ws_bytes(const prism::Dims& d, prism_dtype dt, bool train) {
  Carve cv;
  if (dt == PRISM_BF16)
    carve_fwd<prism::bf16>(d, cv, train);
  else
    carve_fwd<float>(d, cv, train);
  return cv.off;
}

template <typename E>
prism_status run_forward(const prism::Dims& d0, const void* q, const void* k, const void* v,
                         const float* alpha, const float* beta, const void* Wk, const void* Wp,
                         const void* wbeta, const void* conv, const float* S0, const void* hist,
                         void* o, float* ST, void* hist_out, void* ws, void* keep, hipStream_t s) {
  Carve cv;
  cv.base = static_cast<char*>(ws);
  FwdWs<E> w = carve_fwd<E>(d0, cv, keep != nullptr);
  // packed batch: every kernel reads the sanitised copy of the offsets
  prism::Dims d = d0;
  if (d0.cu) {
    HIP_TRY("cu_sanitize", s, prism::launch_cu_sanitize(d0, w.cu, s));
    d.cu = w.cu;
  }
  if (keep) {   // training forward: what the backward reads lives in the kept buffer
    Carve ck;
    ck.base = static_cast<char*>(keep);
    const Kept<E> kp = carve_kept<E>(d, ck);
    w.Kl = kp.Kl;
    w.Wl = kp.Wl;
    w.Mt = kp.Mt;
    w.Qt = kp.Qt;
    w.Sc = kp.Sc;
    w.UT = kp.UT;
    w.WkT = kp.WkT;
    w.gC = kp.gC;
  }
  const E* q_ = static_cast<const E*>(q);
  const E* k_ = static_cast<const E*>(k);
  const E* v_ = static_cast<const E*>(v);
  const E* hist_ = static_cast<const E*>(hist);
  if (d.L > 0 && !keep) {
    // inference: the chunk kernel forms the refinement pairs itself, so they
    // never go to HBM
    prism::FuseIn<E> fz;
    fz.hist = hist_;
    fz.conv = static_cast<const E*>(conv);
    fz.Wk = static_cast<const E*>(Wk);
    fz.Wp = static_cast<const E*>(Wp);
    fz.wbeta = static_cast<const E*>(wbeta);
    HIP_TRY("chunk_fwd_fused", s,
            prism::launch_chunk_fwd_fused<E>(d, q_, k_, v_, alpha, beta, fz, w.Mt, w.HT, w.Qt,
                                             w.Oloc, w.gC, s));
  } else {
    // training forward (the backward reads the pairs), or no refinement
    if (d.L > 0)
      HIP_TRY("refine_fwd", s,
              prism::launch_refine_fwd<E>(d, v_, hist_, static_cast<const E*>(conv),
                                          static_cast<const E*>(Wk), static_cast<const E*>(Wp),
                                          static_cast<const E*>(wbeta), w.Kl, w.Wl, s));
    HIP_TRY("chunk_fwd", s,
            prism::launch_chunk_fwd<E>(d, q_, k_, v_, alpha, beta, w.Kl, w.Wl, nullptr, w.Mt,
                                       w.HT, w.Qt, w.Oloc, w.gC, nullptr, w.UT, w.WkT, s));
  }
  // state pass with the readout fused; the chunk-entry states go to HBM only
  // when the training forward keeps them
  HIP_TRY("state_fwd", s,
          prism::launch_state_pass<E>(d, S0, w.Mt, w.HT, w.gC, keep ? w.Sc : nullptr, ST, false,
                                      false, w.Qt, w.Oloc, static_cast<E*>(o), nullptr, s));
  // after every read of hist, which hist_out may overwrite
  if (hist_out)
    HIP_TRY("conv_state", s, prism::launch_conv_state<E>(d, v_, hist_, static_cast<E*>(hist_out), s));
  return PRISM_OK;
}

template <typename E>
prism_status run_backward(const prism::Dims& d0, const void* q, const void* k, const void* v,
                          const float* alpha, const float* beta, const void* Wk, const void* Wp,
                          const void* wbeta, const void* conv, const float* S0, const void* hist,
                          const void* dO, const float* dST, void* dq, void* dk, void* dv,
                          float* dalpha, float* dbeta, float* dWk, float* dWp, float* dwbeta,
                          float* dconv, float* dS0, float* dhist, void* ws, const void* kept,
                          hipStream_t s) {
  Carve cv;
  cv.base = static_cast<char*>(ws);
  BwdWs<E> w = carve_bwd<E>(d0, cv, kept != nullptr);
  prism::Dims d = d0;
  if (d0.cu) {
    HIP_TRY("cu_sanitize", s, prism::launch_cu_sanitize(d0, w.cu, s));
    d.cu = w.cu;
  }
  const E* q_ = static_cast<const E*>(q);
  const E* k_ = static_cast<const E*>(k);
  const E* v_ = static_cast<const E*>(v);
  const E* dO_ = static_cast<const E*>(dO);
  const E* hist_ = static_cast<const E*>(hist);
  if (kept) {
    // the forward's intermediates: only E = dO^T Qt per chunk is new
    Carve ck;
    ck.base = static_cast<char*>(const_cast<void*>(kept));
    const Kept<E> kp = carve_kept<E>(d, ck);
    w.Kl = kp.Kl;
    w.Wl = kp.Wl;
    w.Mt = kp.Mt;
    w.Sc = kp.Sc;
    w.UT = kp.UT;
    w.WkT = kp.WkT;
    w.gC = kp.gC;
  } else {
    if (d.L > 0)
      HIP_TRY("refine_fwd_recompute", s,
              prism::launch_refine_fwd<E>(d, v_, hist_, static_cast<const E*>(conv),
                                          static_cast<const E*>(Wk), static_cast<const E*>(Wp),
                                          static_cast<const E*>(wbeta), w.Kl, w.Wl, s));
    HIP_TRY("chunk_fwd_bwdmode", s,
            prism::launch_chunk_fwd<E>(d, q_, k_, v_, alpha, beta, w.Kl, w.Wl, dO_, w.Mt, w.HT,
                                       nullptr, nullptr, w.gC, w.ET, w.UT, w.WkT, s));
    HIP_TRY("state_fwd_recompute", s,
            prism::launch_state_pass<E>(d, S0, w.Mt, w.HT, w.gC, w.Sc, nullptr, false, false,
                                        nullptr, nullptr, nullptr, nullptr, s));
  }
  // reverse state pass; after a training forward it forms E_c = dO^T Qt from
  // the kept Qt itself, otherwise it adds the E^T of the backward-mode chunk kernel
  const E* Qk = nullptr;
  if (kept) {
    Carve ck;
    ck.base = static_cast<char*>(const_cast<void*>(kept));
    Qk = carve_kept<E>(d, ck).Qt;
  }
  if (kept)
    HIP_TRY("state_bwd", s,
            prism::launch_state_pass<E>(d, dST, w.Mt, nullptr, w.gC, w.dSnT, dS0, true, true, Qk,
                                        nullptr, nullptr, dO_, s));
  else
    HIP_TRY("state_bwd_stateless", s,
            prism::launch_state_pass<E>(d, dST, w.Mt, w.ET, w.gC, w.dSnT, dS0, true, true, nullptr,
                                        nullptr, nullptr, nullptr, s));
  prism::ChunkBwdArgs<E> a;
  a.q = q_; a.k = k_; a.v = v_; a.dO = dO_; a.alpha = alpha; a.beta = beta;
  a.Kl = w.Kl; a.Wl = w.Wl; a.UT = w.UT; a.WkT = w.WkT; a.Sc = w.Sc; a.dSnT = w.dSnT;
  a.dQt = w.dQt; a.dUs = w.dUs; a.dWks = w.dWks; a.dKs = w.dKs; a.dKl = w.dKl; a.dWl = w.dWl;
  a.dgs = w.dgs; a.dVp = w.dVp; a.dqp = w.dqp; a.dkp = w.dkp; a.dgp = w.dgp; a.dbeta = dbeta;
  a.dq = static_cast<E*>(dq); a.dk = static_cast<E*>(dk);
  a.dv = static_cast<E*>(dv); a.dalpha = dalpha;
  HIP_TRY("chunk_bwd_state", s, prism::launch_chunk_bwd<E>(d, a, 0, s));
  HIP_TRY("chunk_bwd_solve", s, prism::launch_chunk_bwd<E>(d, a, 1, s));
  HIP_TRY("chunk_bwd_pairs", s, prism::launch_chunk_bwd<E>(d, a, 2, s));
  if (d.L > 0) {
    prism::RefineBwdArgs<E> r;
    r.v = v_; r.conv = static_cast<const E*>(conv); r.Wk = static_cast<const E*>(Wk);
    r.Wp = static_cast<const E*>(Wp); r.wbeta = static_cast<const E*>(wbeta);
    r.WkT = w.WkW; r.WpT = w.WpW; r.WpF = w.WpF; r.dKl = w.dKl; r.dWl = w.dWl; r.dvdir = w.dVp; r.u = w.u;
    r.dP = w.dP; r.dwbp = w.dwbp; r.dcp = w.dcp; r.part = w.part;
    r.dv = static_cast<E*>(dv); r.dWk_o = dWk; r.dWp_o = dWp; r.dwbeta_o = dwbeta;
    r.dconv_o = dconv;
    r.hist = hist_;
    r.dhist = dhist;
    HIP_TRY("weight_frags", s, prism::launch_refine_bwd<E>(d, r, 0, s));
    HIP_TRY("refine_bwd", s, prism::launch_refine_bwd<E>(d, r, 1, s));
    HIP_TRY("wgrad_gemm", s, prism::launch_refine_bwd<E>(d, r, 2, s));
    HIP_TRY("wgrad_reduce", s, prism::launch_refine_bwd<E>(d, r, 3, s));
    HIP_TRY("bias_reduce", s, prism::launch_refine_bwd<E>(d, r, 4, s));
  } else if (dhist) {   // without refinement the history does not reach the outputs
    HIP_TRY("zero_hist_grad", s, prism::launch_zero(dhist, (long)d.B * 4 * d.H * d.D, s));
  }
  return PRISM_OK;
}

template <typename E>
prism_status run_step(const prism::Dims& d, const void* q, const void* k, const void* v,
                      const float* alpha, const float* beta, const void* Wk, const void* Wp,
                      const void* wbeta, const void* conv, float* S, void* cs, void* o, char* Kl,
                      char* Wl, hipStream_t s) {
  auto go = [&](int stage) {
    return prism::launch_step<E>(d, static_cast<const E*>(q), static_cast<const E*>(k),
                                 static_cast<const E*>(v), alpha, beta, static_cast<const E*>(Wk),
                                 static_cast<const E*>(Wp), static_cast<const E*>(wbeta),
                                 static_cast<const E*>(conv), S, static_cast<E*>(cs),
                                 static_cast<E*>(o), reinterpret_cast<E*>(Kl),
                                 reinterpret_cast<E*>(Wl), stage, s);
  };
  if (d.L > 0) HIP_TRY("step_refine", s, go(0));
  HIP_TRY("step_state", s, go(1));
  return PRISM_OK;
}

}  // namespace

extern "C" {

const char* prism_status_string(prism_status st) {
  switch (st) {
    case PRISM_OK: return "PRISM_OK";
    case PRISM_ERR_NULL: return "PRISM_ERR_NULL";
    case PRISM_ERR_SHAPE: return "PRISM_ERR_SHAPE";
    case PRISM_ERR_UNSUPPORTED: return "PRISM_ERR_UNSUPPORTED";
    case PRISM_ERR_ALIGN: return "PRISM_ERR_ALIGN";
    case PRISM_ERR_WORKSPACE: return "PRISM_ERR_WORKSPACE";
    case PRISM_ERR_HIP: return "PRISM_ERR_HIP";
  }
  return "PRISM_ERR_UNKNOWN";
}

const char* prism_last_error(void) { return g_err.c_str(); }

prism_status prism_forward_workspace(const prism_desc* desc, size_t* bytes) {
  if (bytes) *bytes = 0;
  if (!bytes) return fail(PRISM_ERR_NULL, "bytes is NULL");
  prism::Dims d;
  prism_status st = check_desc(desc, &d);
  if (st != PRISM_OK) return st;
  *bytes = fwd_ws_bytes(d, desc->dtype, false);
  return PRISM_OK;
}

prism_status prism_backward_workspace(const prism_desc* desc, size_t* bytes) {
  if (bytes) *bytes = 0;
  if (!bytes) return fail(PRISM_ERR_NULL, "bytes is NULL");
  prism::Dims d;
  prism_status st = check_desc(desc, &d);
  if (st != PRISM_OK) return st;
  *bytes = bwd_ws_bytes(d, desc->dtype, false);
  return PRISM_OK;
}

prism_status prism_forward_train_workspace(const prism_desc* desc, size_t* bytes) {
  if (bytes) *bytes = 0;
  if (!bytes) return fail(PRISM_ERR_NULL, "bytes is NULL");
  prism::Dims d;
  prism_status st = check_desc(desc, &d);
  if (st != PRISM_OK) return st;
  *bytes = fwd_ws_bytes(d, desc->dtype, true);
  return PRISM_OK;
}

prism_status prism_backward_train_workspace(const prism_desc* desc, size_t* bytes) {
  if (bytes) *bytes = 0;
  if (!bytes) return fail(PRISM_ERR_NULL, "bytes is NULL");
  prism::Dims d;
  prism_status st = check_desc(desc, &d);
  if (st != PRISM_OK) return st;
  *bytes = bwd_ws_bytes(d, desc->dtype, true);
  return PRISM_OK;
}

prism_status prism_saved_bytes(const prism_desc* desc, size_t* bytes) {
  if (bytes) *bytes = 0;
  if (!bytes) return fail(PRISM_ERR_NULL, "bytes is NULL");
  prism::Dims d;
  prism_status st = check_desc(desc, &d);
  if (st != PRISM_OK) return st;
  *bytes = kept_bytes(d, desc->dtype);
  return PRISM_OK;
}

}  // extern "C"

namespace {

prism_status check_buffer(const void* p, size_t have, size_t need, const char* what) {
  if (!p) return fail(PRISM_ERR_WORKSPACE, std::string(what) + " is NULL");
  if (reinterpret_cast<uintptr_t>(p) & 255u)
    return fail(PRISM_ERR_ALIGN, std::string(what) + " is not 256-byte aligned");
  if (have < need)
    return fail(PRISM_ERR_WORKSPACE, std::string(what) + " has " + std::to_string(have) +
                                         " bytes, needs " + std::to_string(need));
  return PRISM_OK;
}

prism_status forward_entry(const prism_desc* desc, const void* q, const void* k, const void* v,
                           const float* alpha, const float* beta, const void* Wk, const void* Wp,
                           const void* wbeta, const void* conv, const float* S0,
                           const void* conv_hist, const int* cu_seqlens, void* o, float* ST,
                           void* conv_hist_out, void* saved, size_t saved_bytes, bool train,
                           void* workspace, size_t workspace_bytes, hipStream_t stream) {
  try {
    g_err.clear();
    prism::Dims d;
    prism_status st = check_desc(desc, &d);
    if (st != PRISM_OK) return st;
    st = check_cu(cu_seqlens, desc, &d);
    if (st != PRISM_OK) return st;
    const bool refine = d.L > 0;
    CHECK_PTR(q, true);
    CHECK_PTR(k, true);
    CHECK_PTR(v, true);
    CHECK_PTR(alpha, true);
    CHECK_PTR(beta, true);
    CHECK_PTR(Wk, refine);
    CHECK_PTR(Wp, refine);
    CHECK_PTR(wbeta, refine);
    CHECK_PTR(conv, refine);
    CHECK_PTR(S0, false);
    CHECK_PTR(conv_hist, false);
    CHECK_PTR(o, true);
    CHECK_PTR(ST, false);
    CHECK_PTR(conv_hist_out, false);
    if (train) {
      st = check_buffer(saved, saved_bytes, kept_bytes(d, desc->dtype), "saved");
      if (st != PRISM_OK) return st;
    }
    st = check_buffer(workspace, workspace_bytes, fwd_ws_bytes(d, desc->dtype, train), "workspace");
    if (st != PRISM_OK) return st;
    void* keep = train ? saved : nullptr;
    if (desc->dtype == PRISM_BF16)
      return run_forward<prism::bf16>(d, q, k, v, alpha, beta, Wk, Wp, wbeta, conv, S0, conv_hist,
                                      o, ST, conv_hist_out, workspace, keep, stream);
    return run_forward<float>(d, q, k, v, alpha, beta, Wk, Wp, wbeta, conv, S0, conv_hist, o, ST,
                              conv_hist_out, workspace, keep, stream);
  } catch (...) {
    return fail(PRISM_ERR_HIP, "unexpected host exception");
  }
}

prism_status backward_entry(const prism_desc* desc, const void* q, const void* k, const void* v,
                            const float* alpha, const float* beta, const void* Wk, const void* Wp,
                            const void* wbeta, const void* conv, const float* S0,
                            const void* conv_hist, const int* cu_seqlens, const void* saved,
                            size_t saved_bytes, bool train, const void* dO, const float* dST,
                            void* dq, void* dk, void* dv, float* dalpha, float* dbeta, float* dWk,
                            float* dWp, float* dwbeta, float* dconv, float* dS0,
                            float* dconv_hist, void* workspace, size_t workspace_bytes,
                            hipStream_t stream) {
  try {
    g_err.clear();
    prism::Dims d;
    prism_status st = check_desc(desc, &d);
    if (st != PRISM_OK) return st;
    st = check_cu(cu_seqlens, desc, &d);
    if (st != PRISM_OK) return st;
    const bool refine = d.L > 0;
    CHECK_PTR(q, true);
    CHECK_PTR(k, true);
    CHECK_PTR(v, true);
    CHECK_PTR(alpha, true);
    CHECK_PTR(beta, true);
    CHECK_PTR(Wk, refine);
    CHECK_PTR(Wp, refine);
    CHECK_PTR(wbeta, refine);
    CHECK_PTR(conv, refine);
    CHECK_PTR(S0, false);
    CHECK_PTR(conv_hist, false);
    CHECK_PTR(dO, true);
    CHECK_PTR(dST, false);
    CHECK_PTR(dq, true);
    CHECK_PTR(dk, true);
    CHECK_PTR(dv, true);
    CHECK_PTR(dalpha, true);
    CHECK_PTR(dbeta, true);
    CHECK_PTR(dWk, refine);
    CHECK_PTR(dWp, refine);
    CHECK_PTR(dwbeta, refine);
    CHECK_PTR(dconv, refine);
    CHECK_PTR(dS0, false);
    CHECK_PTR(dconv_hist, false);
    if (train) {
      st = check_buffer(saved, saved_bytes, kept_bytes(d, desc->dtype), "saved");
      if (st != PRISM_OK) return st;
    }
    st = check_buffer(workspace, workspace_bytes, bwd_ws_bytes(d, desc->dtype, train), "workspace");
    if (st != PRISM_OK) return st;
    const void* kept = train ? saved : nullptr;
    if (desc->dtype == PRISM_BF16)
      return run_backward<prism::bf16>(d, q, k, v, alpha, beta, Wk, Wp, wbeta, conv, S0, conv_hist,
                                       dO, dST, dq, dk, dv, dalpha, dbeta, dWk, dWp, dwbeta,
                                       dconv, dS0, dconv_hist, workspace, kept, stream);
    return run_backward<float>(d, q, k, v, alpha, beta, Wk, Wp, wbeta, conv, S0, conv_hist, dO,
                               dST, dq, dk, dv, dalpha, dbeta, dWk, dWp, dwbeta, dconv, dS0,
                               dconv_hist, workspace, kept, stream);
  } catch (...) {
    return fail(PRISM_ERR_HIP, "unexpected host exception");
  }
}

}  // namespace

extern "C" {

prism_status prism_forward(const prism_desc* desc, const void* q, const void* k, const void* v,
                           const float* alpha, const float* beta, const void* Wk, const void* Wp,
                           const void* wbeta, const void* conv, const float* S0,
                           const void* conv_hist, const int* cu_seqlens, void* o, float* ST,
                           void* conv_hist_out, void* workspace, size_t workspace_bytes,
                           hipStream_t stream) {
  return forward_entry(desc, q, k, v, alpha, beta, Wk, Wp, wbeta, conv, S0, conv_hist, cu_seqlens,
                       o, ST, conv_hist_out, nullptr, 0, false, workspace, workspace_bytes, stream);
}

prism_status prism_forward_train(const prism_desc* desc, const void* q, const void* k,
                                 const void* v, const float* alpha, const float* beta,
                                 const void* Wk, const void* Wp, const void* wbeta,
                                 const void* conv, const float* S0, const void* conv_hist,
                                 const int* cu_seqlens, void* o, float* ST, void* conv_hist_out,
                                 void* saved, size_t saved_bytes, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream) {
  return forward_entry(desc, q, k, v, alpha, beta, Wk, Wp, wbeta, conv, S0, conv_hist, cu_seqlens,
                       o, ST, conv_hist_out, saved, saved_bytes, true, workspace, workspace_bytes,
                       stream);
}

prism_status prism_backward(const prism_desc* desc, const void* q, const void* k, const void* v,
                            const float* alpha, const float* beta, const void* Wk, const void* Wp,
                            const void* wbeta, const void* conv, const float* S0,
                            const void* conv_hist, const int* cu_seqlens, const void* dO,
                            const float* dST, void* dq, void* dk, void* dv, float* dalpha,
                            float* dbeta, float* dWk, float* dWp, float* dwbeta, float* dconv,
                            float* dS0, float* dconv_hist, void* workspace,
                            size_t workspace_bytes, hipStream_t stream) {
  return backward_entry(desc, q, k, v, alpha, beta, Wk, Wp, wbeta, conv, S0, conv_hist,
                        cu_seqlens, nullptr, 0, false, dO, dST, dq, dk, dv, dalpha, dbeta, dWk,
                        dWp, dwbeta, dconv, dS0, dconv_hist, workspace, workspace_bytes, stream);
}

prism_status prism_backward_train(const prism_desc* desc, const void* q, const void* k,
                                  const void* v, const float* alpha, const float* beta,
                                  const void* Wk, const void* Wp, const void* wbeta,
                                  const void* conv, const float* S0, const void* conv_hist,
                                  const int* cu_seqlens, const void* saved, size_t saved_bytes,
                                  const void* dO, const float* dST, void* dq, void* dk, void* dv,
                                  float* dalpha, float* dbeta, float* dWk, float* dWp,
                                  float* dwbeta, float* dconv, float* dS0, float* dconv_hist,
                                  void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return backward_entry(desc, q, k, v, alpha, beta, Wk, Wp, wbeta, conv, S0, conv_hist,
                        cu_seqlens, saved, saved_bytes, true, dO, dST, dq, dk, dv, dalpha, dbeta,
                        dWk, dWp, dwbeta, dconv, dS0, dconv_hist, workspace, workspace_bytes,
                        stream);
}

prism_status prism_step_workspace(const prism_desc* desc, size_t* bytes) {
  if (bytes) *bytes = 0;
  if (!bytes) return fail(PRISM_ERR_NULL, "bytes is NULL");
  prism::Dims d;
  prism_status st = check_desc(desc, &d);
  if (st != PRISM_OK) return st;
  *bytes = step_ws_bytes(d, desc->dtype);
  return PRISM_OK;
}

}  // extern "C"

namespace {

// prism_step and prism_step_noalloc: the same checks and kernels; the
// refinement pairs go to the caller's workspace or (noalloc) to the fixed
// device array of noalloc.hip.
prism_status step_entry(const prism_desc* desc, const void* q, const void* k, const void* v,
                        const float* alpha, const float* beta, const void* Wk, const void* Wp,
                        const void* wbeta, const void* conv, float* S, void* conv_state, void* o,
                        void* workspace, size_t workspace_bytes, bool noalloc,
                        hipStream_t stream) {
  try {
    g_err.clear();
    prism::Dims d;
    prism_status st = check_desc(desc, &d);
    if (st != PRISM_OK) return st;
    const bool refine = d.L > 0;
    CHECK_PTR(q, true);
    CHECK_PTR(k, true);
    CHECK_PTR(v, true);
    CHECK_PTR(alpha, true);
    CHECK_PTR(beta, true);
    CHECK_PTR(Wk, refine);
    CHECK_PTR(Wp, refine);
    CHECK_PTR(wbeta, refine);
    CHECK_PTR(conv, refine);
    CHECK_PTR(S, true);
    CHECK_PTR(conv_state, false);
    CHECK_PTR(o, true);
    const size_t need = step_ws_bytes(d, desc->dtype);
    if (noalloc) {
      if (need > prism::NOALLOC_SCRATCH_BYTES)
        return fail(PRISM_ERR_WORKSPACE,
                    "prism_step_noalloc: the refinement pairs of B * H * L * T * D elements need " +
                        std::to_string(need) + " bytes; its fixed device array holds " +
                        std::to_string(prism::NOALLOC_SCRATCH_BYTES) + " (use prism_step)");
      if (need > 0) {
        const hipError_t e = prism::noalloc_scratch(stream, &workspace);
        if (e != hipSuccess)
          return fail(PRISM_ERR_HIP, std::string("prism_step_noalloc: device array address: ") +
                                         hipGetErrorString(e));
      }
    } else if (need > 0) {
      st = check_buffer(workspace, workspace_bytes, need, "workspace");
      if (st != PRISM_OK) return st;
    }
    // the refinement pairs, [B, H, L, T, D] each
    const size_t half = need / 2;
    char* ws = static_cast<char*>(workspace);
    if (desc->dtype == PRISM_BF16)
      return run_step<prism::bf16>(d, q, k, v, alpha, beta, Wk, Wp, wbeta, conv, S, conv_state, o,
                                   need ? ws : nullptr, need ? ws + half : nullptr, stream);
    return run_step<float>(d, q, k, v, alpha, beta, Wk, Wp, wbeta, conv, S, conv_state, o,
                           need ? ws : nullptr, need ? ws + half : nullptr, stream);
  } catch (...) {
    return fail(PRISM_ERR_HIP, "unexpected host exception");
  }
}

}  // namespace

extern "C" {

prism_status prism_step(const prism_desc* desc, const void* q, const void* k, const void* v,
                        const float* alpha, const float* beta, const void* Wk, const void* Wp,
                        const void* wbeta, const void* conv, float* S, void* conv_state, void* o,
                        void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return step_entry(desc, q, k, v, alpha, beta, Wk, Wp, wbeta, conv, S, conv_state, o, workspace,
                    workspace_bytes, false, stream);
}

prism_status prism_step_noalloc(const prism_desc* desc, const void* q, const void* k,
                                const void* v, const float* alpha, const float* beta,
                                const void* Wk, const void* Wp, const void* wbeta,
                                const void* conv, float* S, void* conv_state, void* o,
                                hipStream_t stream) {
  return step_entry(desc, q, k, v, alpha, beta, Wk, Wp, wbeta, conv, S, conv_state, o, nullptr, 0,
                    true, stream);
}

void prism_timing_begin(void) {
  g_timing = true;
  g_launches.clear();
}

int prism_timing_end(const char** names, double* total_ms, int* launches, int capacity) {
  g_timing = false;
  std::vector<const char*> nm;
  std::vector<double> ms;
  std::vector<int> cnt;
  for (auto& l : g_launches) {
    float t = 0.f;
    (void)hipEventSynchronize(l.b);
    (void)hipEventElapsedTime(&t, l.a, l.b);
    size_t i = 0;
    for (; i < nm.size(); ++i)
      if (std::strcmp(nm[i], l.name) == 0) break;
    if (i == nm.size()) {
      nm.push_back(l.name);
      ms.push_back(0.0);
      cnt.push_back(0);
    }
    ms[i] += t;
    cnt[i] += 1;
    g_pool.push_back(l.a);
    g_pool.push_back(l.b);
  }
  g_launches.clear();
  const int n = (int)nm.size();
  for (int i = 0; i < n && i < capacity; ++i) {
    if (names) names[i] = nm[i];
    if (total_ms) total_ms[i] = ms[i];
    if (launches) launches[i] = cnt[i];
  }
  return n;
}

}  // extern "C"
