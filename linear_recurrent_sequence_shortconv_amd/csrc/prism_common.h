// Device-side building blocks shared by the PRISM kernels (gfx950 / CDNA4).
//
// * Element type T is either __bf16 (bf16 storage, bf16 MFMA operands,
//   fp32 accumulation) or float (fp32 storage, fp32 MFMA).
// * All matrix products go through 16x16 output tiles of one MFMA family:
//     bf16: v_mfma_f32_16x16x32_bf16 (k = 32 per instruction, 8 per lane)
//     fp32: v_mfma_f32_16x16x4_f32   (k = 4 per instruction, 1 per lane)
//   Operand fragments: lane l holds row (l & 15) of its 16-row slab and the
//   KPL consecutive k values starting at KPL * (l >> 4).
//   Accumulator: lane l holds column (l & 15) and rows 4 * (l >> 4) + i,
//   i = 0..3 (four consecutive rows of one column).
// * A workgroup of NW waves computes an M x N product by splitting the
//   (M/16) x (N/16) tile grid into a WM x WN grid of per-wave blocks; each
//   wave keeps its block's accumulators in registers (register blocking).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <map>
#include <mutex>
#include <utility>

namespace prism {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int WAVE = 64;

constexpr int cmax(int a, int b) { return a > b ? a : b; }

template <typename T> struct Mfma;

template <> struct Mfma<bf16> {
  static constexpr int KSTEP = 32;
  static constexpr int KPL = 8;
  typedef bf16x8 frag;
  __device__ static inline f32x4 mma(const frag& a, const frag& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};

template <> struct Mfma<float> {
  static constexpr int KSTEP = 4;
  static constexpr int KPL = 1;
  typedef float frag;
  __device__ static inline f32x4 mma(const frag& a, const frag& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
};

// --------------------------------------------------------------------------
// scalar conversions (round to nearest even for bf16)
// --------------------------------------------------------------------------
template <typename T> __device__ inline T to_t(float x);
template <> __device__ inline float to_t<float>(float x) { return x; }
template <> __device__ inline bf16 to_t<bf16>(float x) { return (bf16)x; }
__device__ inline float to_f(float x) { return x; }
__device__ inline float to_f(bf16 x) { return (float)x; }

// 16-byte vector of T (8 bf16 or 4 float) for coalesced global <-> LDS copies
template <typename T> struct Vec16 {
  static constexpr int N = 16 / sizeof(T);
  typedef uint4 raw;
};

__device__ inline uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

// The LDS array's address as a value the compiler cannot see through.  Taken
// at the head of a persistent workgroup's loop, the LDS addresses formed from
// it are computed in the loop body; formed from the array itself they are
// constants, which the compiler materializes once before the loop and keeps in
// registers across all of it.
__device__ inline unsigned char* lds_opaque(unsigned char* p) {
  typedef __attribute__((address_space(3))) unsigned char L;
  L* q = (L*)p;
  asm volatile("" : "+s"(q));
  return (unsigned char*)__builtin_assume_aligned((unsigned char*)q, 16);
}
__device__ inline void st16(void* p, const uint4& v) { *reinterpret_cast<uint4*>(p) = v; }

// --------------------------------------------------------------------------
// MFMA fragment loads from LDS
//   KC = true : element (row, k) at p[row * ld + k]   (k contiguous)
//   KC = false: element (row, k) at p[k * ld + row]   (k strided)
// For 16-bit elements the strided case uses the gfx950 LDS transpose read
// (ds_read_b64_tr_b16).  Its lane mapping, measured on the device: within
// each group of 16 lanes, lane j supplies the address of 4 consecutive
// elements M[j][0..3], and lane i receives M[4e + i/4][i % 4], e = 0..3.
// Pointing lane j = 4e + q at p[(k + e) * ld + row + 4q] therefore hands lane
// i the four values p[(k + e) * ld + row + i], e = 0..3, i.e. four
// consecutive k of row (row + i): one 8-byte read replaces four 2-byte ones.
// Needs ld and row multiples of 4 (8-byte aligned reads).
// --------------------------------------------------------------------------
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// four consecutive k (k0 + 4 * (lane >> 4) .. + 3) of row row0 + (lane & 15)
__device__ inline s16x4 lds_read_tr4(const bf16* p, int ld, int row0, int k0, int lane) {
  const int j = lane & 15;
  const bf16* a = p + (k0 + 4 * (lane >> 4) + (j >> 2)) * ld + row0 + 4 * (j & 3);
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(a));
}

template <typename T, bool KC>
__device__ inline typename Mfma<T>::frag load_frag(const T* p, int ld, int row0, int k0, int lane) {
  constexpr int KPL = Mfma<T>::KPL;
  const int r = row0 + (lane & 15);
  const int k = k0 + KPL * (lane >> 4);
  typename Mfma<T>::frag f;
  if constexpr (KC) {
    f = *reinterpret_cast<const typename Mfma<T>::frag*>(p + r * ld + k);
  } else if constexpr (KPL == 1) {
    f = p[k * ld + r];
  } else {
    // 8 consecutive k starting at k0 + 8 (lane >> 4): two transpose reads
    // (k .. k+3 and k+4 .. k+7); each lane group g reads rows k0 + 8g + e
    const int j = lane & 15;
    const T* a = p + (k0 + 8 * (lane >> 4) + (j >> 2)) * ld + row0 + 4 * (j & 3);
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(a));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(a + 4 * ld));
    const short __attribute__((ext_vector_type(8))) w = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    __builtin_memcpy(&f, &w, 16);
  }
  return f;
}

// MFMA of the projection kernels for an inner size K: bf16 takes
// v_mfma_f32_16x16x32_bf16 (8 k per lane) unless K = 16, where it takes
// v_mfma_f32_16x16x16_bf16 (4 k per lane); fp32 takes 16x16x4 in both cases.
template <typename T, int K> struct MfmaK : Mfma<T> {};
template <> struct MfmaK<bf16, 16> {
  static constexpr int KSTEP = 16;
  static constexpr int KPL = 4;
  typedef s16x4 frag;
  __device__ static inline f32x4 mma(const frag& a, const frag& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
  }
};

// k-contiguous MfmaK fragment: KPL consecutive k (from k0 + KPL (lane >> 4))
// of row row0 + (lane & 15), from LDS or global memory
template <typename T, int K>
__device__ inline typename MfmaK<T, K>::frag load_fragK(const T* p, int ld, int row0, int k0, int lane) {
  typedef MfmaK<T, K> MK;
  const int r = row0 + (lane & 15);
  const int k = k0 + MK::KPL * (lane >> 4);
  return *reinterpret_cast<const typename MK::frag*>(p + r * ld + k);
}

// Fragment order of a D x D matrix W that serves as a k-contiguous MfmaK<T, D>
// operand (rows in 16-row tiles): fragment (tile nt, k step kk) holds, for lane
// l, row 16 nt + (l & 15) and k = kk KSTEP + KPL (l >> 4) .. + KPL - 1, and is
// stored contiguously at ((nt NK + kk) 64 + l) KPL.  A wave then reads a whole
// fragment as one contiguous piece (1 KB for bf16), where the row-major layout
// spreads it over 16 rows in 64-byte pieces.
template <typename T, int D>
__device__ inline long frag_order_offset(int row, int k) {
  typedef MfmaK<T, D> MK;
  constexpr int NK = D / MK::KSTEP;
  const int nt = row >> 4, kk = k / MK::KSTEP, q = (k % MK::KSTEP) / MK::KPL, e = k % MK::KPL;
  return ((long)(nt * NK + kk) * 64 + (row & 15) + 16 * q) * MK::KPL + e;
}
template <typename T, int D>
__device__ inline typename MfmaK<T, D>::frag load_frag_fo(const T* W, int nt, int kk, int lane) {
  typedef MfmaK<T, D> MK;
  constexpr int NK = D / MK::KSTEP;
  // (the fragment's base, then the lane's 32-bit unsigned byte offset: with a
  // wave-uniform matrix and tile the load takes the scalar-base form, no 64-bit
  // address arithmetic per fragment)
  const char* b = reinterpret_cast<const char*>(W) + (long)(nt * NK + kk) * (64 * MK::KPL * (int)sizeof(T));
  return *reinterpret_cast<const typename MK::frag*>(b + (unsigned)lane * (unsigned)(MK::KPL * sizeof(T)));
}

// The chunk kernels store the per-chunk matrix M^T ([D][D], rows = the column
// of the state product) in fragment order where one lane's fragment is a
// whole 16-byte piece (bf16, D >= 32: 8 consecutive k); elsewhere row-major.
template <typename T, int D> constexpr bool mt_frag_order() {
  return sizeof(T) == 2 && D >= 32;
}
// Row and first k of the 16-byte piece e of a matrix in that fragment order
// (8 consecutive k of one row).
template <int D>
__device__ inline void fo_piece_rc(int e, int& row, int& k) {
  constexpr int NK = D / 32;
  const int ln = e & 63, f = e >> 6;
  row = 16 * (f / NK) + (ln & 15);
  k = 32 * (f % NK) + 8 * (ln >> 4);
}

// --------------------------------------------------------------------------
// wave-grid tiling of an M x N output over NW waves
// --------------------------------------------------------------------------
// Choose WN (waves along N): among splits WM x WN = NW that divide the tile
// grid evenly, the one with the fewest fragment loads per k step (RM + RN);
// if the grid has fewer tiles than waves, some waves stay idle.
constexpr int tiling_wn(int TM, int TN, int NW) {
  int best = -1, cost = 1 << 30;
  for (int wn = 1; wn <= NW; wn *= 2) {
    const int wm = NW / wn;
    if (wn > TN || wm > TM || TN % wn || TM % wm) continue;
    const int c = TM / wm + TN / wn;
    if (c < cost) { cost = c; best = wn; }
  }
  if (best > 0) return best;
  return TN < NW ? TN : NW;
}

template <int M, int N, int NW> struct Tiling {
  static constexpr int TM = M / 16;
  static constexpr int TN = N / 16;
  static constexpr int WN = tiling_wn(TM, TN, NW);
  static constexpr int WM0 = NW / WN;
  static constexpr int WM = TM < WM0 ? TM : WM0;
  static constexpr int RM = (TM + WM - 1) / WM;   // tiles per wave along M
  static constexpr int RN = (TN + WN - 1) / WN;   // tiles per wave along N
  static_assert(M % 16 == 0 && N % 16 == 0, "tile multiple");
  static_assert(TM % WM == 0 && TN % WN == 0, "even split");
  // every wave of the workgroup is active when the grid uses all NW (folds at
  // compile time)
  __device__ static inline bool active(int wave) { return WM * WN >= NW || wave < WM * WN; }
  // first tile row / col of this wave's block
  __device__ static inline int m0(int wave) { return (wave / WN) * RM * 16; }
  __device__ static inline int n0(int wave) { return (wave % WN) * RN * 16; }
};

template <int M, int N, int NW> struct Acc {
  typedef Tiling<M, N, NW> TL;
  f32x4 v[TL::RM][TL::RN];
  __device__ inline void zero() {
#pragma unroll
    for (int i = 0; i < TL::RM; ++i)
#pragma unroll
      for (int j = 0; j < TL::RN; ++j) v[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
};

// bf16 fragments of 4 k values for v_mfma_f32_16x16x16_bf16 (inner sizes of 16)
template <bool KC>
__device__ inline s16x4 load_frag4(const bf16* p, int ld, int row0, int k0, int lane) {
  const int r = row0 + (lane & 15);
  const int k = k0 + 4 * (lane >> 4);
  s16x4 f;
  if constexpr (KC) {
    f = *reinterpret_cast<const s16x4*>(p + r * ld + k);
  } else {
    f = lds_read_tr4(p, ld, row0, k0, lane);
  }
  return f;
}

// acc += A * B^T over k in [0, K): A is M x K, B is N x K (both as LDS views).
// The k steps are unrolled fully (every fragment read of the product is issued
// before the products that wait for it) unless KU2 asks for pairs of steps, for
// a kernel at its register limit.
template <typename T, int M, int N, int K, int NW, bool AKC, bool BKC, bool KU2 = false>
__device__ inline void gemm_acc(Acc<M, N, NW>& acc, const T* A, int lda, const T* B, int ldb,
                                int wave, int lane) {
  typedef Tiling<M, N, NW> TL;
  if (!TL::active(wave)) return;
  const int m0 = TL::m0(wave), n0 = TL::n0(wave);
  constexpr int KS = Mfma<T>::KSTEP;
  if constexpr (sizeof(T) == 2 && K % KS != 0) {
    static_assert(K % 16 == 0, "k multiple of 16");
#pragma unroll
    for (int k0 = 0; k0 < K; k0 += 16) {
      s16x4 a[TL::RM], b[TL::RN];
#pragma unroll
      for (int i = 0; i < TL::RM; ++i) a[i] = load_frag4<AKC>(A, lda, m0 + 16 * i, k0, lane);
#pragma unroll
      for (int j = 0; j < TL::RN; ++j) b[j] = load_frag4<BKC>(B, ldb, n0 + 16 * j, k0, lane);
#pragma unroll
      for (int i = 0; i < TL::RM; ++i)
#pragma unroll
        for (int j = 0; j < TL::RN; ++j)
          acc.v[i][j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a[i], b[j], acc.v[i][j], 0, 0, 0);
    }
  } else {
    static_assert(K % KS == 0, "k multiple");
    if constexpr (KU2) {
#pragma unroll 2
      for (int k0 = 0; k0 < K; k0 += KS) {
        typename Mfma<T>::frag a[TL::RM], b[TL::RN];
#pragma unroll
        for (int i = 0; i < TL::RM; ++i) a[i] = load_frag<T, AKC>(A, lda, m0 + 16 * i, k0, lane);
#pragma unroll
        for (int j = 0; j < TL::RN; ++j) b[j] = load_frag<T, BKC>(B, ldb, n0 + 16 * j, k0, lane);
#pragma unroll
        for (int i = 0; i < TL::RM; ++i)
#pragma unroll
          for (int j = 0; j < TL::RN; ++j) acc.v[i][j] = Mfma<T>::mma(a[i], b[j], acc.v[i][j]);
      }
    } else {
      auto kstep = [&](int k0) {
        typename Mfma<T>::frag a[TL::RM], b[TL::RN];
  #pragma unroll
        for (int i = 0; i < TL::RM; ++i) a[i] = load_frag<T, AKC>(A, lda, m0 + 16 * i, k0, lane);
  #pragma unroll
        for (int j = 0; j < TL::RN; ++j) b[j] = load_frag<T, BKC>(B, ldb, n0 + 16 * j, k0, lane);
  #pragma unroll
        for (int i = 0; i < TL::RM; ++i)
  #pragma unroll
          for (int j = 0; j < TL::RN; ++j) acc.v[i][j] = Mfma<T>::mma(a[i], b[j], acc.v[i][j]);
      };
#pragma unroll
      for (int k0 = 0; k0 < K; k0 += KS) kstep(k0);
    }
  }
}

// Visit this wave's accumulator tiles: f(row0, col, f32x4 vals) where
// vals[i] belongs to (row0 + i, col).
template <int M, int N, int NW, typename F>
__device__ inline void for_tiles(const Acc<M, N, NW>& acc, int wave, int lane, F&& f) {
  typedef Tiling<M, N, NW> TL;
  if (!TL::active(wave)) return;
  const int m0 = TL::m0(wave), n0 = TL::n0(wave);
#pragma unroll
  for (int i = 0; i < TL::RM; ++i)
#pragma unroll
    for (int j = 0; j < TL::RN; ++j)
      f(m0 + 16 * i + 4 * (lane >> 4), n0 + 16 * j + (lane & 15), acc.v[i][j]);
}

// Same visit, also passing the tile indices: f(i, j, row0, col, vals).
template <int M, int N, int NW, typename F>
__device__ inline void for_tiles_ij(const Acc<M, N, NW>& acc, int wave, int lane, F&& f) {
  typedef Tiling<M, N, NW> TL;
  if (!TL::active(wave)) return;
  const int m0 = TL::m0(wave), n0 = TL::n0(wave);
#pragma unroll
  for (int i = 0; i < TL::RM; ++i)
#pragma unroll
    for (int j = 0; j < TL::RN; ++j)
      f(i, j, m0 + 16 * i + 4 * (lane >> 4), n0 + 16 * j + (lane & 15), acc.v[i][j]);
}

// Same visit, with a mutable accumulator (to rescale or reset in place).
template <int M, int N, int NW, typename F>
__device__ inline void for_tiles_mut(Acc<M, N, NW>& acc, int wave, int lane, F&& f) {
  typedef Tiling<M, N, NW> TL;
  if (!TL::active(wave)) return;
  const int m0 = TL::m0(wave), n0 = TL::n0(wave);
#pragma unroll
  for (int i = 0; i < TL::RM; ++i)
#pragma unroll
    for (int j = 0; j < TL::RN; ++j)
      f(m0 + 16 * i + 4 * (lane >> 4), n0 + 16 * j + (lane & 15), acc.v[i][j]);
}

// --------------------------------------------------------------------------
// T = (I + A)^{-1} for a strictly lower triangular C x C matrix A (fp32 in
// LDS, leading dimension C + 1), written to Tm (same layout, zeros above the
// diagonal).  Xs is scratch of inv_scratch_floats(C) floats.  All NW waves of
// the workgroup take part; ends with a barrier.
//  * 16 x 16 diagonal blocks: forward substitution, one lane per column with
//    the column in registers.  Row r of a column c is
//    T[r][c] = [r == c] - sum_{m < r} A[r][m] T[m][c]; entries above the
//    diagonal come out as zero by themselves, so every lane runs the same
//    unrolled code.
//  * then block doubling, S = 16, 32, ...: for each pair of S-blocks on the
//    diagonal, T21 = -T22 (A21 T11), two fp32 MFMA products.
// --------------------------------------------------------------------------
constexpr int inv_scratch_floats(int C) { return C >= 32 ? ((C / 2) * (C / 2 + 1) + 3) / 4 * 4 : 4; }

template <int C, int S, int NW, bool KU2>
__device__ __attribute__((always_inline)) inline void invert_double_level(const float* A, float* Tm, float* Xs, int wave, int lane) {
  constexpr int LA = C + 1, P = C / (2 * S), LX = S + 1;
  static_assert(NW % P == 0, "waves per block pair");
  constexpr int NWP = NW / P;
  const int pr = wave / NWP, w = wave % NWP;
  const int o = 2 * S * pr;
  float* X = Xs + pr * S * LX;
  {
    Acc<S, S, NWP> x;   // X = A21 T11
    x.zero();
    gemm_acc<float, S, S, S, NWP, true, false, KU2>(x, A + (o + S) * LA + o, LA, Tm + o * LA + o, LA, w, lane);
    for_tiles(x, w, lane, [&](int r0, int cc, const f32x4& v) {
#pragma unroll
      for (int r = 0; r < 4; ++r) X[(r0 + r) * LX + cc] = v[r];
    });
  }
  __syncthreads();
  {
    Acc<S, S, NWP> y;   // T21 = -T22 X
    y.zero();
    gemm_acc<float, S, S, S, NWP, true, false, KU2>(y, Tm + (o + S) * LA + o + S, LA, X, LX, w, lane);
    for_tiles(y, w, lane, [&](int r0, int cc, const f32x4& v) {
#pragma unroll
      for (int r = 0; r < 4; ++r) Tm[(o + S + r0 + r) * LA + o + cc] = -v[r];
    });
  }
  __syncthreads();
}

// Always inlined: as a call it would make the caller wait for every load in
// flight (its prefetches of the next phase) and spill around the call.  KU2 as
// for gemm_acc.
// PD: rows of A read ahead of the one computed in the diagonal blocks (more
// rows hide more LDS latency and hold more registers).
#ifndef INV_PD
#define INV_PD 3
#endif
template <int C, int NW, bool KU2 = false, int PD = 1>
__device__ __attribute__((always_inline)) inline void invert_unit_lower(const float* A, float* Tm,
                                                                       float* Xs, int tid) {
  constexpr int NB = C / 16, LA = C + 1;
  static_assert(NB >= 1 && NB <= 4 && C % 16 == 0, "C in {16, 32, 48, 64}");
  // (tid >> 6 is the same in every lane of a wave: keep the wave index scalar)
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  for (int e = tid; e < C * C; e += NW * WAVE) {
    const int r = e / C, cc = e % C;
    if (cc > r) Tm[r * LA + cc] = 0.f;
  }
  if (wave == 0 && lane < NB * 16) {
    const int base = 16 * (lane >> 4), col = lane & 15;
    const float* Ab = A + base * LA + base;
    // row r + PD of A is read from LDS while row r is computed (a ring of
    // PD + 1 rows in registers: an LDS round trip is longer than the FMA chain
    // of a short row); the empty asm (which takes t[r] and clobbers memory)
    // pins that order, so the reads are not all hoisted up front with 120
    // values held in registers
    static_assert(PD >= 1 && PD < 16, "rows ahead");
    float t[16], an[PD + 1][16];
#pragma unroll
    for (int k = 1; k < PD && k < 16; ++k)
#pragma unroll
      for (int m = 0; m < k; ++m) an[k % (PD + 1)][m] = Ab[k * LA + m];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      if (r + PD < 16) {
#pragma unroll
        for (int m = 0; m < r + PD; ++m) an[(r + PD) % (PD + 1)][m] = Ab[(r + PD) * LA + m];
      }
      float s = (r == col) ? 1.f : 0.f;
#pragma unroll
      for (int m = 0; m < r; ++m) s = fmaf(-an[r % (PD + 1)][m], t[m], s);
      t[r] = s;
      asm volatile("" : "+v"(t[r]) : : "memory");
    }
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (r >= col) Tm[(base + r) * LA + base + col] = t[r];
  }
  __syncthreads();
  if constexpr (C >= 32) invert_double_level<C, 16, NW, KU2>(A, Tm, Xs, wave, lane);
  if constexpr (C >= 64) invert_double_level<C, 32, NW, KU2>(A, Tm, Xs, wave, lane);
}

// two consecutive elements from fp32 values (one 4- or 8-byte store, aligned)
template <typename E>
__device__ inline void st2f(E* p, float a, float b) {
  if constexpr (sizeof(E) == 2) {
    const E x[2] = {to_t<E>(a), to_t<E>(b)};
    uint32_t w;
    __builtin_memcpy(&w, x, 4);
    *reinterpret_cast<uint32_t*>(p) = w;
  } else {
    *reinterpret_cast<float2*>(p) = make_float2(a, b);
  }
}

// four consecutive elements (8 or 16 bytes, aligned) to LDS or global memory
template <typename E>
__device__ inline void st4(E* p, const E (&x)[4]) {
  if constexpr (sizeof(E) == 2) {
    uint2 w;
    __builtin_memcpy(&w, x, 8);
    *reinterpret_cast<uint2*>(p) = w;
  } else {
    uint4 w;
    __builtin_memcpy(&w, x, 16);
    *reinterpret_cast<uint4*>(p) = w;
  }
}

// four consecutive fp32 accumulator values, converted, as one st4
template <typename E>
__device__ inline void st4f(E* p, const f32x4& x) {
  const E w[4] = {to_t<E>(x[0]), to_t<E>(x[1]), to_t<E>(x[2]), to_t<E>(x[3])};
  st4(p, w);
}

// --------------------------------------------------------------------------
// cooperative global <-> LDS tile copies (16-byte vectors)
// --------------------------------------------------------------------------
// A ROWS x COLS tile of T held in registers as 16-byte vectors spread over
// NT threads: load() issues the global reads early (software prefetch);
// store_rows / store_transposed later write it into LDS.  Rows >= nvalid are
// zeros: load() reads the last valid row in their place (no load sits in a
// per-lane branch, whose merge would make the prefetch wait for its data at
// issue) and the stores write zeros for them.
// TR = false: consecutive threads take consecutive vectors of a row (fully
//   coalesced reads; for row stores).
// TR = true: consecutive threads take consecutive row groups of one 16-byte
//   column block, RG = 2 rows per thread for 2-byte T (1 for 4-byte T), so
//   the transposed store writes one 32-bit word per column and lane, to
//   consecutive words: free of LDS bank conflicts.
template <typename T, int ROWS, int COLS, int NT, bool TR = false>
struct RegTile {
  static constexpr int VN = 16 / (int)sizeof(T);
  static constexpr int VPR = COLS / VN;
  static constexpr int RG = (TR && sizeof(T) == 2) ? 2 : 1;
  static constexpr int NG = ROWS / RG;
  static constexpr int NU = NG * VPR;                 // units of RG vectors
  static constexpr int PER = (NU + NT - 1) / NT;
  static_assert(ROWS % RG == 0, "row pairs");
  uint4 v[PER][RG];
  int nv = ROWS;   // rows >= nv are zeros
  __device__ static inline void unit(int u, int& r0, int& c) {
    if constexpr (TR) {
      r0 = (u % NG) * RG;
      c = (u / NG) * VN;
    } else {
      r0 = u / VPR;
      c = (u % VPR) * VN;
    }
  }
  __device__ inline void load(const T* g, long gstride, int nvalid, int tid) {
    nv = nvalid;
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      // threads past the last unit read it again (the stores skip them)
      const int u = min(tid + p * NT, NU - 1);
      int r0, c;
      unit(u, r0, c);
#pragma unroll
      for (int q = 0; q < RG; ++q) {
        v[p][q] = uint4{0u, 0u, 0u, 0u};
        // (a 32-bit unsigned byte offset from the tile's base: no 64-bit
        // address arithmetic per vector)
        if (nvalid > 0)
          v[p][q] = ld16(reinterpret_cast<const char*>(g) +
                         ((unsigned)min(r0 + q, nvalid - 1) * (unsigned)gstride + (unsigned)c) * (unsigned)sizeof(T));
      }
    }
  }
  // load() without its branch on nvalid, whose join (registers zeroed on one
  // side, loaded on the other) can make the wave wait for every load in
  // flight right after issuing these: with nvalid <= 0 every lane reads the
  // first 16 bytes at fallback (any valid address) instead, and the rows are
  // zeros at the store as with load()
  __device__ inline void load_nb(const T* g, long gstride, int nvalid, const T* fallback, int tid) {
    nv = nvalid;
    const bool any = nvalid > 0;   // (uniform: scalar selects below)
    const T* base = any ? g : fallback;
    const unsigned st = any ? (unsigned)gstride : 0u;
    const int last = any ? nvalid - 1 : 0;
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int u = min(tid + p * NT, NU - 1);
      int r0, c;
      unit(u, r0, c);
      if (!any) c = 0;
#pragma unroll
      for (int q = 0; q < RG; ++q)
        v[p][q] = ld16(reinterpret_cast<const char*>(base) +
                       ((unsigned)min(r0 + q, last) * st + (unsigned)c) * (unsigned)sizeof(T));
    }
  }
  // vector (p, q) of row r: zeros past the valid rows.  The empty asm keeps
  // this select here, not next to the load.
  __device__ inline uint4 get(int p, int q, int r) const {
    uint4 w = v[p][q];
    asm volatile("" : "+v"(w.x), "+v"(w.y), "+v"(w.z), "+v"(w.w));
    return r < nv ? w : uint4{0u, 0u, 0u, 0u};
  }
  __device__ inline void store_rows(T* s, int ld, int tid) const {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int u = tid + p * NT;
      int r0, c;
      unit(u, r0, c);
      if (u < NU) {
#pragma unroll
        for (int q = 0; q < RG; ++q) st16(s + (r0 + q) * ld + c, get(p, q, r0 + q));
      }
    }
  }
  // rows into an fp32 LDS tile (values converted from T).  The empty asm
  // keeps the conversion here: hoisted into load(), it would make the
  // prefetch wait for its own data right after issuing it.
  __device__ inline void store_rows_f32(float* s, int ld, int tid) const {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int u = tid + p * NT;
      int r0, c;
      unit(u, r0, c);
      if (u < NU) {
#pragma unroll
        for (int q = 0; q < RG; ++q) {
          const uint4 w = get(p, q, r0 + q);
          const T* x = reinterpret_cast<const T*>(&w);
#pragma unroll
          for (int j = 0; j < VN; j += 4)
            *reinterpret_cast<f32x4*>(s + (r0 + q) * ld + c + j) =
                f32x4{to_f(x[j]), to_f(x[j + 1]), to_f(x[j + 2]), to_f(x[j + 3])};
        }
      }
    }
  }
  // element (r, c) -> s[c * ld + r], times scale[r] (nullptr = 1)
  __device__ inline void store_transposed(T* s, int ld, const float* scale, int tid) const {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int u = tid + p * NT;
      int r0, c;
      unit(u, r0, c);
      if (u < NU) {
        if constexpr (RG == 2) {
          const uint4 w0 = get(p, 0, r0), w1 = get(p, 1, r0 + 1);
          const T* x0 = reinterpret_cast<const T*>(&w0);
          const T* x1 = reinterpret_cast<const T*>(&w1);
          const float s0 = scale ? scale[r0] : 1.0f, s1 = scale ? scale[r0 + 1] : 1.0f;
#pragma unroll
          for (int j = 0; j < VN; ++j) {
            T pr[2] = {to_t<T>(to_f(x0[j]) * s0), to_t<T>(to_f(x1[j]) * s1)};
            uint32_t w;
            __builtin_memcpy(&w, pr, 4);
            *reinterpret_cast<uint32_t*>(s + (c + j) * ld + r0) = w;
          }
        } else {
#pragma unroll
          for (int q = 0; q < RG; ++q) {
            const uint4 w = get(p, q, r0 + q);
            const T* x = reinterpret_cast<const T*>(&w);
            const float sc = scale ? scale[r0 + q] : 1.0f;
#pragma unroll
            for (int j = 0; j < VN; ++j) s[(c + j) * ld + r0 + q] = to_t<T>(to_f(x[j]) * sc);
          }
        }
      }
    }
  }
};

// Global rows -> LDS rows (rows >= nvalid are zeros), all loads of the tile
// issued before the first store: one memory round trip, where a copy loop
// that stores each vector as it arrives waits once per iteration.
template <typename T, int ROWS, int COLS, int NT>
__device__ inline void g2s_rows(T* s, int ld, const T* g, long gstride, int nvalid, int tid) {
  RegTile<T, ROWS, COLS, NT> t;
  t.load(g, gstride, nvalid, tid);
  t.store_rows(s, ld, tid);
}

// Four consecutive values of T to global memory, converted from fp32.
__device__ inline void st_f4(float* p, const f32x4& x) { *reinterpret_cast<f32x4*>(p) = x; }
__device__ inline void st_f4(bf16* p, const f32x4& x) {
  const bf16 b[4] = {(bf16)x[0], (bf16)x[1], (bf16)x[2], (bf16)x[3]};
  uint2 w;
  __builtin_memcpy(&w, b, 8);
  *reinterpret_cast<uint2*>(p) = w;
}
// Four consecutive values of T from global memory, held as raw bits until
// raw4_to_f converts them where they are used: a conversion next to the load
// would make a prefetch wait for its data at issue (the empty asm keeps the
// conversion at the use).
template <typename T> struct Raw4Of { typedef f32x4 type; };
template <> struct Raw4Of<bf16> { typedef uint2 type; };
template <typename T> __device__ inline typename Raw4Of<T>::type ld_raw4(const T* p) {
  return *reinterpret_cast<const typename Raw4Of<T>::type*>(p);
}
__device__ inline f32x4 raw4_to_f(const f32x4& x) { return x; }
__device__ inline f32x4 raw4_to_f(uint2 w) {
  asm volatile("" : "+v"(w.x), "+v"(w.y));
  return f32x4{__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u),
               __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xffff0000u)};
}

// One storage-type value kept raw in a register until its use, the same way.
template <typename T> struct Raw1Of { typedef float type; };
template <> struct Raw1Of<bf16> { typedef unsigned int type; };
__device__ inline float ld_raw1(const float* p) { return *p; }
__device__ inline unsigned int ld_raw1(const bf16* p) { return *reinterpret_cast<const unsigned short*>(p); }
__device__ inline float raw1_to_f(float x) {
  asm volatile("" : "+v"(x));
  return x;
}
__device__ inline float raw1_to_f(unsigned int w) {
  asm volatile("" : "+v"(w));
  return __uint_as_float(w << 16);
}

// LDS tile -> global rows (first nvalid rows only)
template <typename T, int ROWS, int COLS, int NT>
__device__ inline void s2g_rows(T* g, long gstride, const T* s, int ld, int nvalid, int tid) {
  constexpr int VN = 16 / sizeof(T);
  constexpr int VPR = COLS / VN;
  for (int e = tid; e < ROWS * VPR; e += NT) {
    const int r = e / VPR, c = (e % VPR) * VN;
    if (r < nvalid)
      st16(reinterpret_cast<T*>(reinterpret_cast<char*>(g) + ((unsigned)r * (unsigned)gstride + (unsigned)c) * (unsigned)sizeof(T)),
           ld16(s + r * ld + c));
  }
}

// Padded LDS leading dimension for a row of n elements of T.  Measured on
// gfx950 with the LDS bank-conflict counters, for the access patterns of
// these kernels over 16 consecutive rows: 16-byte fragment reads are
// conflict-free when the row stride is 8 (mod 16) dwords and take twice the
// LDS cycles at 4 (mod 8) dwords (e.g. 136 bf16); the transposed 8-byte
// reads (ds_read_b64_tr_b16) cost the same at either; 4-byte reads of fp32
// rows are best at 4 (mod 8) dwords.  So 2-byte rows of 32 or more elements
// get the smallest stride >= n + 8 that is 8 (mod 16) dwords (e.g. 128 ->
// 144, 64 -> 80); shorter rows and 4-byte rows keep a 16-byte pad.
template <typename T> constexpr int ldpad(int n) {
  if (sizeof(T) != 2 || n < 32) return n + 16 / (int)sizeof(T);
  int m = n + 8;
  while ((m / 2) % 16 != 8) m += 8;
  return m;
}
// The smallest padding (16 bytes), where LDS space is tighter than bandwidth.
template <typename T> constexpr int ldpad_min(int n) { return n + 16 / (int)sizeof(T); }
static_assert(ldpad<__bf16>(128) == 144 && ldpad<__bf16>(64) == 80 && ldpad<__bf16>(32) == 48 &&
                  ldpad<__bf16>(16) == 24 && ldpad<float>(64) == 68,
              "row strides");

// --------------------------------------------------------------------------
// math
// --------------------------------------------------------------------------
// Standard normal tail q(x) = Phi(-x) = erfc(x / sqrt 2) / 2 for x >= 0, with
// erfc from Abramowitz & Stegun, Handbook of Mathematical Functions, formula
// 7.1.26:
//   erfc(y) = (a1 s + a2 s^2 + a3 s^3 + a4 s^4 + a5 s^5) exp(-y^2),
//   s = 1 / (1 + p y), y >= 0, |error| <= 1.5e-7.
// With y = x / sqrt 2 the 1 / sqrt 2 goes into p and the halving into the
// coefficients (exact: a power of two); exp(-x^2 / 2) is one v_exp_f32 of
// -x^2 log2(e) / 2 and is returned for reuse; s is one v_rcp_f32 (1 ulp, far
// below the formula's own error).
__device__ inline float normal_tail(float x, float& e) {
  const float s = __builtin_amdgcn_rcpf(fmaf(0.3275911f * 0.70710678118654752f, x, 1.0f));
  float poly = fmaf(0.5f * 1.061405429f, s, 0.5f * -1.453152027f);
  poly = fmaf(poly, s, 0.5f * 1.421413741f);
  poly = fmaf(poly, s, 0.5f * -0.284496736f);
  poly = fmaf(poly, s, 0.5f * 0.254829592f);
  e = __builtin_amdgcn_exp2f((x * -0.72134752044448170f) * x);   // 2^(-x^2 log2(e) / 2)
  return poly * s * e;
}
// GELU(z) = z Phi(z) (exact-erf form, to the accuracy above): Phi(z) = 1 - q(|z|)
// for z >= 0 and q(|z|) below, so z Phi(z) = max(z, 0) - |z| q(|z|) either way.
__device__ inline float gelu_erf(float z) {
  const float x = fabsf(z);
  float e;
  return fmaf(-x, normal_tail(x, e), fmaxf(z, 0.f));
}
// GELU and its derivative d/dz GELU = Phi(z) + z phi(z), phi(z) = exp(-z^2/2) / sqrt(2 pi)
__device__ inline void gelu_and_grad(float z, float& g, float& dg) {
  float e;
  const float q = normal_tail(fabsf(z), e);
  const float c = z >= 0.f ? 1.f - q : q;
  g = z * c;
  dg = fmaf(z * 0.39894228040143268f, e, c);
}
// --------------------------------------------------------------------------
// cross-lane sums by DPP (VALU operations with a lane-shifted source) instead
// of LDS shuffles (ds_bpermute, an LDS round trip each)
// --------------------------------------------------------------------------
#define PRISM_DPP(v, ctrl, rowm, bc) \
  __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, (v)), (ctrl), (rowm), 0xf, (bc)))
// Sum over each quad of lanes (4k .. 4k + 3), in every lane of the quad:
// quad_perm [1,0,3,2], then [2,3,0,1] (the pairing of an xor 1, 2 butterfly).
__device__ inline float quad_sum(float v) {
  v += PRISM_DPP(v, 0xB1, 0xf, false);
  v += PRISM_DPP(v, 0x4E, 0xf, false);
  return v;
}
// Sum over each row of 16 lanes (16k .. 16k + 15), left in lane 16k + 15: an
// inclusive prefix sum by row shifts 1, 2, 4, 8 with zero fill (the pairing
// tree of an xor 1, 2, 4, 8 butterfly).
__device__ inline float row16_sum(float v) {
  v += PRISM_DPP(v, 0x111, 0xf, true);
  v += PRISM_DPP(v, 0x112, 0xf, true);
  v += PRISM_DPP(v, 0x114, 0xf, true);
  v += PRISM_DPP(v, 0x118, 0xf, true);
  return v;
}
// Sum over the 64 lanes of the wave, in every lane: the row sums, then the four
// row totals read from lanes 15, 31, 47 and 63.
__device__ inline float wave_sum(float v) {
  v = row16_sum(v);
  const int b = __builtin_bit_cast(int, v);
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 15));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 31));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 47));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 63));
  return (r0 + r1) + (r2 + r3);
}
// Inclusive prefix sum over the 64 lanes of the wave: row scans by row shifts,
// then each row's carry from the rows before it by row broadcasts (lane 15 to
// rows 1 and 3, then lane 31 to rows 2 and 3).
__device__ inline float wave_scan(float v) {
  v = row16_sum(v);
  v += PRISM_DPP(v, 0x142, 0xa, false);
  v += PRISM_DPP(v, 0x143, 0xc, false);
  return v;
}
#undef PRISM_DPP

__device__ inline float sigmoidf(float x) { return __builtin_amdgcn_rcpf(1.0f + __expf(-x)); }

// Sequence b of a batch: its first token and its length.  A dense batch
// (cu == nullptr) has B sequences of T tokens; a packed one lists offsets
// cu[0..B], sequence b being tokens cu[b] .. cu[b+1] - 1 (at most T of them).
__device__ inline long seq_start(const int* cu, int b, int T) { return cu ? (long)cu[b] : (long)b * T; }
__device__ inline int seq_len(const int* cu, int b, int T) {
  return cu ? max(0, min(cu[b + 1] - cu[b], T)) : T;
}

// XCD-aware block order: consecutive hardware dispatch slots go round-robin
// over the 8 XCDs; return a logical block id such that the blocks one XCD
// receives are contiguous in logical order (neighbouring tiles share L2).
__device__ inline int xcd_swizzle(int bid, int nblocks) {
  constexpr int NXCD = 8;
  if (nblocks % NXCD != 0) return bid;
  const int per = nblocks / NXCD;
  return (bid % NXCD) * per + bid / NXCD;
}

// --------------------------------------------------------------------------
// host: grid of a persistent kernel = resident workgroups per CU x CUs on the
// current device (at most nblk), cached per kernel and device
// --------------------------------------------------------------------------
template <typename K>
inline int persistent_grid(K kernel, int threads, int nblk) {
  static std::mutex mu;
  static std::map<std::pair<const void*, int>, int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return nblk;
  const std::pair<const void*, int> key(reinterpret_cast<const void*>(kernel), dev);
  int g = 0;
  {
    std::lock_guard<std::mutex> lk(mu);
    auto it = cache.find(key);
    if (it != cache.end()) g = it->second;
  }
  if (g == 0) {
    int ncu = 0, per = 0;
    if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, kernel, threads, 0) != hipSuccess ||
        ncu <= 0 || per <= 0)
      return nblk;
    g = ncu * per;
    std::lock_guard<std::mutex> lk(mu);
    cache[key] = g;
  }
  return g < nblk ? g : nblk;
}

}  // namespace prism
