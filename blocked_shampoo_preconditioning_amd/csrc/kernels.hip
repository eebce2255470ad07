// HIP kernels of the blocked Shampoo step for CDNA4 (gfx950).
//
// Steps of one optimizer step (page "Shampoo optimizer", matrix-case loop;
// DASH page, abstract, for the stacked block batch):
//   pack      gradient blocks -> Gp [B][br][bc] and its transpose GpT
//   stats     L <- beta2 L + g Gp Gp^T,  R <- beta2 R + g Gp^T Gp  (MFMA, SYRK)
//   norms     s = ||A||_F or min(||A||_F, ||A||_inf) * 2/5 per factor
//   newton    coupled Newton for A^(-1/4): T = (5I - M)/4, X <- X T,
//             M <- T^4 M (MFMA GEMM chains, symmetric outputs)
//   apply     W -= lr * X_L Gp X_R (two MFMA products, update in the epilogue)
//
// Every dense product here has the form C = P^T Q with P (K x M) and Q
// (K x N) stored row-major, so both operands stream along K in contiguous
// rows ("k-major") and go to LDS without a transpose. The statistics read
// GpT / Gp, the Newton products read symmetric matrices (P^T = P), the
// apply reads Gp and the transposed intermediate it writes itself.
//
// MFMA: v_mfma_f32_32x32x2_f32 (fp32 in, fp32 accumulate). Operand layout
// for one 32x32x2 step: lane l supplies A[m = l % 32][k = l / 32] and
// B[k = l / 32][n = l % 32]; accumulator register r of lane l holds
// D[m = 8 (r / 4) + 4 (l / 32) + r % 4][n = l % 32].
#include "kernels.h"

#include <math.h>
#include <cstring>
#include <mutex>

#include <type_traits>

namespace shp {
namespace {

typedef float floatx16 __attribute__((ext_vector_type(16)));
// Native 4-wide vector: HIP's float4 is a union-based struct that the
// compiler has kept in scratch memory when held in register arrays.
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Tile shape: WM x WN waves, each owning FM x FN 32x32 MFMA fragments; K
// advances BK at a time.
template <int WM_, int WN_, int FM_, int FN_, int BK_ = 16>
struct Cfg {
  static constexpr int WM = WM_, WN = WN_, FM = FM_, FN = FN_;
  static constexpr int NT = 64 * WM * WN;
  static constexpr int BM = 32 * FM * WM;
  static constexpr int BN = 32 * FN * WN;
  static constexpr int BK = BK_;
  // LDS row pitch: the two half-waves of an operand read rows k and k+1;
  // a pitch of 32 (mod 64) banks keeps them on disjoint banks.
  static constexpr int LDP = BM + ((BM % 64) == 0 ? 32 : 0);
  static constexpr int LDQ = BN + ((BN % 64) == 0 ? 32 : 0);
  static constexpr int LDS_FP32 = 2 * BK * (LDP + LDQ);
  // bf16 operands: K-tiles of 32, rows of k contiguous, pitch 40 (16-byte
  // aligned rows, 32 + 8 so consecutive rows start on different banks)
  static constexpr int BKH = 32, LDKH = BKH + 8;
  static constexpr int LDS_BF16 = 2 * (BM + BN) * LDKH / 2;  // in floats
  static constexpr int LDS_FLOATS = LDS_FP32 > LDS_BF16 ? LDS_FP32 : LDS_BF16;
  // split products: K-tiles of 16, each operand row as three bf16 planes,
  // rows of 16 values padded to 24 (48 bytes: 16-byte aligned rows whose
  // 16-byte reads from eight consecutive rows fall on distinct banks)
  static constexpr int LDX = 24;
  static constexpr int LDS_SPLIT = 2 * 3 * (BM + BN) * LDX / 2;  // in floats
  static constexpr int LDS_SPLITH = 2 * 2 * (BM + BN) * LDX / 2;  // two fp16 planes
  static constexpr int PV = BM / 4, QV = BN / 4;           // float4 per operand row
  static constexpr int PPT = BK * PV / NT, QPT = BK * QV / NT;  // float4 per thread
  static_assert(PPT >= 1 && QPT >= 1, "tile too small for the thread count");
  static_assert((BK * PV) % NT == 0 && (BK * QV) % NT == 0, "uneven operand load");
};

using Cfg128 = Cfg<2, 2, 2, 2>;  // 128 x 128, 256 threads
using Cfg64 = Cfg<2, 2, 1, 1>;   //  64 x  64, 256 threads
using Cfg32 = Cfg<1, 1, 1, 1>;   //  32 x  32,  64 threads
// 256 x 256, 512 threads (8 waves of 128 x 64): split-path full products
// only; its LDS (147 KiB) allows one workgroup per CU
using Cfg256 = Cfg<2, 4, 4, 2>;

// Workgroups are dispatched round-robin over the 8 XCDs (workgroup w runs on
// XCD w % 8). xcd_remap gives every XCD a contiguous range of logical tiles so
// the tiles of one matrix share an L2.
__device__ __forceinline__ int xcd_remap(int w, int total) {
  const int per = total / 8, rem = total % 8;
  const int xcd = w % 8, idx = w / 8;
  return xcd * per + min(xcd, rem) + idx;
}

// acc[fm][fn] = sum over K of P[k][m0 + ...] * Q[k][n0 + ...]
// Double-buffered LDS: the global loads of K-tile kt+1 are issued before the
// MFMAs of tile kt and written to the other LDS buffer after them, so their
// latency hides behind the matrix work. No lambdas here: captured register
// arrays have been demoted to scratch memory by the compiler.
// MASK selects the fragments (bit i * FN + j) whose MFMAs run; the others
// only take part in the loads and barriers.
// (wm, wn) is the wave's fragment block inside the tile; every wave loads its
// share of the operand tiles whatever its block.
template <class C, int MASK = -1>
__device__ __forceinline__ void mainloop_w(const float* __restrict__ P, const float* __restrict__ Q,
                                           int M, int N, int K, int m0, int n0, int wm, int wn,
                                           floatx16 (&acc)[C::FM][C::FN], float* lds) {
  float* sP = lds;
  float* sQ = lds + 2 * C::BK * C::LDP;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int half = lane >> 5, l32 = lane & 31;
  static_assert(C::LDS_FP32 <= C::LDS_FLOATS, "LDS");

#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // this thread's float4 slots of a K-tile: global row offset and LDS offset
  const float* gp = P + m0;
  const float* gq = Q + n0;
  const int p_row0 = tid / C::PV, p_c4 = (tid % C::PV) * 4;
  const int q_row0 = tid / C::QV, q_c4 = (tid % C::QV) * 4;
  constexpr int P_ROWS = C::NT / C::PV, Q_ROWS = C::NT / C::QV;  // rows per slot step
  const size_t p_tile = (size_t)C::BK * M, q_tile = (size_t)C::BK * N;
  gp += (size_t)p_row0 * M + p_c4;
  gq += (size_t)q_row0 * N + q_c4;
  const int lp = p_row0 * C::LDP + p_c4, lq = q_row0 * C::LDQ + q_c4;

  f32x4 pr[C::PPT], qr[C::QPT];
#pragma unroll
  for (int i = 0; i < C::PPT; ++i) pr[i] = *reinterpret_cast<const f32x4*>(gp + (size_t)i * P_ROWS * M);
#pragma unroll
  for (int i = 0; i < C::QPT; ++i) qr[i] = *reinterpret_cast<const f32x4*>(gq + (size_t)i * Q_ROWS * N);
#pragma unroll
  for (int i = 0; i < C::PPT; ++i) *reinterpret_cast<f32x4*>(sP + lp + i * P_ROWS * C::LDP) = pr[i];
#pragma unroll
  for (int i = 0; i < C::QPT; ++i) *reinterpret_cast<f32x4*>(sQ + lq + i * Q_ROWS * C::LDQ) = qr[i];
  __syncthreads();

  const int nk = K / C::BK;
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) {
      gp += p_tile;
      gq += q_tile;
#pragma unroll
      for (int i = 0; i < C::PPT; ++i)
        pr[i] = *reinterpret_cast<const f32x4*>(gp + (size_t)i * P_ROWS * M);
#pragma unroll
      for (int i = 0; i < C::QPT; ++i)
        qr[i] = *reinterpret_cast<const f32x4*>(gq + (size_t)i * Q_ROWS * N);
    }
    const float* p = sP + buf * C::BK * C::LDP + wm * 32 * C::FM + l32 + half * C::LDP;
    const float* q = sQ + buf * C::BK * C::LDQ + wn * 32 * C::FN + l32 + half * C::LDQ;
#pragma unroll
    for (int kk = 0; kk < C::BK; kk += 2) {
      float a[C::FM], b[C::FN];
#pragma unroll
      for (int i = 0; i < C::FM; ++i) a[i] = p[kk * C::LDP + i * 32];
#pragma unroll
      for (int j = 0; j < C::FN; ++j) b[j] = q[kk * C::LDQ + j * 32];
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
          if (MASK & (1 << (i * C::FN + j)))
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    if (more) {
      float* dP = sP + (buf ^ 1) * C::BK * C::LDP + lp;
      float* dQ = sQ + (buf ^ 1) * C::BK * C::LDQ + lq;
#pragma unroll
      for (int i = 0; i < C::PPT; ++i) *reinterpret_cast<f32x4*>(dP + i * P_ROWS * C::LDP) = pr[i];
#pragma unroll
      for (int i = 0; i < C::QPT; ++i) *reinterpret_cast<f32x4*>(dQ + i * Q_ROWS * C::LDQ) = qr[i];
    }
    __syncthreads();
  }
}

template <class C, int MASK = -1>
__device__ __forceinline__ void mainloop(const float* __restrict__ P, const float* __restrict__ Q,
                                         int M, int N, int K, int m0, int n0,
                                         floatx16 (&acc)[C::FM][C::FN], float* lds) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  mainloop_w<C, MASK>(P, Q, M, N, K, m0, n0, wave % C::WM, wave / C::WM, acc, lds);
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// One thread's share of a bf16 K-tile (BKH wide) of both operands in
// registers: 16-byte chunks, CPR per row; chunk c = tid + i NT is row c / CPR,
// k (c % CPR) 8.
template <class C>
struct Bf16Stage {
  static constexpr int CPR = C::BKH / 8;
  static constexpr int CA = C::BM * CPR, CB = C::BN * CPR;
  static_assert(CA % C::NT == 0 && CB % C::NT == 0, "uneven operand load");
  static constexpr int PA = CA / C::NT, PB = CB / C::NT;
  u32x4 a[PA], b[PB];
};

// Row of 16-byte chunk c of a bf16 K-tile (four chunks per row, chunk c % 4
// within it): the 16 lanes of one LDS write group take rows {0, 4, 8, 12}
// (plus 0..3 by group) of a 16-row band, so at the 80-byte row pitch their
// 64-byte row segments start 0, 20, 40 and 60 banks apart (mod 64; 0, 4 mod
// 8-lane groups of 32 banks) and the group writes every bank once; four
// consecutive lanes still load one row's 64 contiguous bytes.
__device__ __forceinline__ int bf16_row(int c) {
  const int g = c >> 4, w = c & 15;
  return ((g >> 2) << 4) + (g & 3) + ((w >> 2) << 2);
}

template <class C, bool SAME = false>
__device__ __forceinline__ void bf16_load(Bf16Stage<C>& st, const uint16_t* __restrict__ X, int K,
                                          int m0, int n0, int kt) {
  using S = Bf16Stage<C>;
  static_assert(S::CPR == 4 && C::BM % 16 == 0 && C::BN % 16 == 0, "chunk layout");
  const int tid = threadIdx.x, k0 = kt * C::BKH;
#pragma unroll
  for (int i = 0; i < S::PA; ++i) {
    const int c = tid + i * C::NT;
    st.a[i] = *reinterpret_cast<const u32x4*>(X + (size_t)(m0 + bf16_row(c)) * K + k0 +
                                              (c % S::CPR) * 8);
  }
  if constexpr (!SAME) {
#pragma unroll
    for (int i = 0; i < S::PB; ++i) {
      const int c = tid + i * C::NT;
      st.b[i] = *reinterpret_cast<const u32x4*>(X + (size_t)(n0 + bf16_row(c)) * K + k0 +
                                                (c % S::CPR) * 8);
    }
  }
}

// Into LDS buffer buf: [BM][LDKH] of A then [BN][LDKH] of B per buffer.
template <class C, bool SAME = false>
__device__ __forceinline__ void bf16_store(const Bf16Stage<C>& st, uint16_t* sA, uint16_t* sB,
                                           int buf) {
  using S = Bf16Stage<C>;
  constexpr int LD = C::LDKH;
  const int tid = threadIdx.x;
  uint16_t* dA = sA + buf * C::BM * LD;
  uint16_t* dB = sB + buf * C::BN * LD;
#pragma unroll
  for (int i = 0; i < S::PA; ++i) {
    const int c = tid + i * C::NT;
    *reinterpret_cast<u32x4*>(dA + bf16_row(c) * LD + (c % S::CPR) * 8) = st.a[i];
  }
  if constexpr (!SAME) {
#pragma unroll
    for (int i = 0; i < S::PB; ++i) {
      const int c = tid + i * C::NT;
      *reinterpret_cast<u32x4*>(dB + bf16_row(c) * LD + (c % S::CPR) * 8) = st.b[i];
    }
  }
}

// The MFMAs of the K-tile in LDS buffer buf (v_mfma_f32_32x32x16_bf16): per
// 16 k, lane l supplies A[m = l % 32][k = 8 (l / 32) + 0..7] and
// B[k = 8 (l / 32) + 0..7][n = l % 32], each a 16-byte read of one LDS row.
template <class C, int MASK>
__device__ __forceinline__ void bf16_mma(floatx16 (&acc)[C::FM][C::FN], const uint16_t* sA,
                                         const uint16_t* sB, int buf, int wm, int wn) {
  constexpr int LD = C::LDKH;
  const int lane = threadIdx.x & 63;
  const int half = lane >> 5, l32 = lane & 31;
  const uint16_t* a0 = sA + buf * C::BM * LD + (wm * 32 * C::FM + l32) * LD + half * 8;
  const uint16_t* b0 = sB + buf * C::BN * LD + (wn * 32 * C::FN + l32) * LD + half * 8;
#pragma unroll
  for (int ks = 0; ks < C::BKH; ks += 16) {
    bf16x8 a[C::FM], b[C::FN];
#pragma unroll
    for (int i = 0; i < C::FM; ++i) a[i] = *reinterpret_cast<const bf16x8*>(a0 + i * 32 * LD + ks);
#pragma unroll
    for (int j = 0; j < C::FN; ++j) b[j] = *reinterpret_cast<const bf16x8*>(b0 + j * 32 * LD + ks);
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
      for (int j = 0; j < C::FN; ++j)
        if (MASK & (1 << (i * C::FN + j)))
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
  }
}

// acc = X[m0 ..] X[n0 ..]^T over K for bf16 rows with k contiguous (row
// stride K, a multiple of BKH). Two LDS buffers and two register stages:
// while the MFMAs run on K-tile kt, tile kt + 1 (loaded one phase earlier)
// goes to the other buffer and tile kt + 2 is loaded into the freed stage, so
// every load has a full phase to land; an odd last tile runs alone.
// SAME: a diagonal tile (n0 == m0): the rows are loaded once and read as
// both operands.
template <class C, int MASK = -1, bool SAME = false>
__device__ __forceinline__ void mainloop_bf16(const uint16_t* __restrict__ X, int K, int m0, int n0,
                                              int wm, int wn, floatx16 (&acc)[C::FM][C::FN],
                                              float* lds) {
  static_assert(!SAME || C::BM == C::BN, "a shared panel is square");
  uint16_t* sA = reinterpret_cast<uint16_t*>(lds);           // [2][BM][LDKH]
  uint16_t* sB = SAME ? sA : sA + 2 * C::BM * C::LDKH;      // [2][BN][LDKH]
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  const int nk = K / C::BKH;
  Bf16Stage<C> s0, s1;
  bf16_load<C, SAME>(s0, X, K, m0, n0, 0);
  if (nk > 1) bf16_load<C, SAME>(s1, X, K, m0, n0, 1);
  bf16_store<C, SAME>(s0, sA, sB, 0);
  __syncthreads();
  int kt = 0;
  for (; kt + 1 < nk; kt += 2) {
    if (kt + 2 < nk) bf16_load<C, SAME>(s0, X, K, m0, n0, kt + 2);
    bf16_mma<C, MASK>(acc, sA, sB, 0, wm, wn);
    bf16_store<C, SAME>(s1, sA, sB, 1);
    __syncthreads();
    if (kt + 3 < nk) bf16_load<C, SAME>(s1, X, K, m0, n0, kt + 3);
    bf16_mma<C, MASK>(acc, sA, sB, 1, wm, wn);
    if (kt + 2 < nk) bf16_store<C, SAME>(s0, sA, sB, 0);
    __syncthreads();
  }
  if (kt < nk) bf16_mma<C, MASK>(acc, sA, sB, 0, wm, wn);
}

// ---------------------------------------------------------------------------
// Split products: fp32 operands, bf16 matrix cores.
// x = h + m + l exactly, each term a bf16 value: h keeps the top 16 bits of
// x (sign, exponent, 7 fraction bits), m the top 16 bits of r = x - h, and
// l = r - m, which has at most 8 significant bits left (for |x| >= 2^-103;
// below that the last bits of l can be lost). Then
//   x y = hh + (hm + mh) + (hl + mm + lh) + O(2^-24 |x y|):
// six bf16 products, each exact in fp32, accumulated in fp32 by the MFMA,
// cost 6 / 16 of the fp32 MFMA time at the same accuracy as fp32 products.
// Non-finite inputs give NaN. Two values per call, packed as bf16 pairs
// (first value in the low half).
// ---------------------------------------------------------------------------
struct Split3 {
  uint32_t h, m, l;
};

__device__ __forceinline__ Split3 split3(float x0, float x1) {
  const uint32_t u0 = __float_as_uint(x0), u1 = __float_as_uint(x1);
  const float r0 = x0 - __uint_as_float(u0 & 0xffff0000u);
  const float r1 = x1 - __uint_as_float(u1 & 0xffff0000u);
  const uint32_t v0 = __float_as_uint(r0), v1 = __float_as_uint(r1);
  const float t0 = r0 - __uint_as_float(v0 & 0xffff0000u);
  const float t1 = r1 - __uint_as_float(v1 & 0xffff0000u);
  Split3 o;
  // v_perm_b32: bytes 2, 3 of the second source, then bytes 2, 3 of the first
  o.h = __builtin_amdgcn_perm(u1, u0, 0x07060302u);
  o.m = __builtin_amdgcn_perm(v1, v0, 0x07060302u);
  o.l = __builtin_amdgcn_perm(__float_as_uint(t1), __float_as_uint(t0), 0x07060302u);
  return o;
}

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// fp16 split products: each operand of a product is first scaled by a power
// of two, 2^e, that brings its largest |value| into [2^14, 2^15) (exact; the
// result is scaled back by 2^-(e_A + e_B), also exact). Then x = h + l + d
// with h = fp16(x) and l = fp16(x - h), both rounded to nearest (x - h is
// exact in fp32): |d| <= 2^-22 |x| while l is normal, and |d| <= 2^-25 below
// that, which is 2^-39 of the operand's largest value. Three fp16 products
//   x y = hh + hl + lh + O(2^-21 |x y|)
// each exact in fp32, accumulated in fp32 by the MFMA: fp32-level accuracy
// with half the products and two thirds of the planes of the bf16 split.
// A non-finite input gives a non-finite high term and a NaN low term, so the
// result is not finite either.
// ---------------------------------------------------------------------------
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

struct Split2 {
  uint32_t h, l;
};

__device__ __forceinline__ Split2 split2h(float x0, float x1, int e) {
  x0 = ldexpf(x0, e);
  x1 = ldexpf(x1, e);
  // one packed conversion for both high terms (v_cvt_pk_f16_f32)
  const f16x2 h = __builtin_convertvector((f32x2){x0, x1}, f16x2);
  const _Float16 l0 = (_Float16)(x0 - (float)h[0]), l1 = (_Float16)(x1 - (float)h[1]);
  Split2 o;
  o.h = __builtin_bit_cast(uint32_t, h);
  o.l = __builtin_bit_cast(uint32_t, (f16x2){l0, l1});
  return o;
}

// Scale exponent of an operand from its versioned maximum word: 2^e brings
// the largest |value| into [2^14, 2^15) (a zero or subnormal maximum is
// treated as 2^-126; an infinite or NaN maximum takes 0, so those values
// propagate as they are).
__device__ __forceinline__ int f16_exp(uint64_t w) {
  const int e = (int)(w & 0xffu);
  return e == 0xff ? 0 : 141 - (e > 0 ? e : 1);
}


// Row of 4-value chunk c of a split operand tile (its chunk within the row is
// c % 4). The 16 lanes of one 128-byte LDS write group take rows {0, 2, 4, 6}
// (odd groups {1, 3, 5, 7}) of an 8-row band: at the 48-byte row pitch their
// 32-byte segments start 24 banks apart (mod 32), so the group covers all 32
// banks once. Consecutive rows would put rows 0 and 3 on the same banks.
__device__ __forceinline__ int split_row(int c) {
  const int g = c >> 4, w = c & 15;
  return (g >> 1) * 8 + ((w >> 2) << 1) + (g & 1);
}

// Three planes of 4 consecutive k of one row.
__device__ __forceinline__ void store_split4(uint16_t* d, int plane, const f32x4& v) {
  const Split3 a = split3(v[0], v[1]), b = split3(v[2], v[3]);
  *reinterpret_cast<u32x2*>(d) = (u32x2){a.h, b.h};
  *reinterpret_cast<u32x2*>(d + plane) = (u32x2){a.m, b.m};
  *reinterpret_cast<u32x2*>(d + 2 * plane) = (u32x2){a.l, b.l};
}

// The two fp16 planes of 4 consecutive k of one row, scaled by 2^e.
__device__ __forceinline__ void store_split4h(uint16_t* d, int plane, const f32x4& v, int e) {
  const Split2 a = split2h(v[0], v[1], e), b = split2h(v[2], v[3], e);
  *reinterpret_cast<u32x2*>(d) = (u32x2){a.h, b.h};
  *reinterpret_cast<u32x2*>(d + plane) = (u32x2){a.l, b.l};
}

// One thread's share of one operand of a split K-tile (16 wide) in
// registers. Rows mode (the operand stored [ROWS][K], k contiguous): NR
// 4-value chunks, row split_row(c) and chunk c % 4 for c = tid + i NT.
// Columns mode (stored [K][ROWS], rows contiguous): KC consecutive k of row
// tid % ROWS, one value per load, consecutive lanes on consecutive rows.
template <class C, int ROWS, bool COLS>
struct SplitOperand {
  static constexpr int NR = ROWS * 4 / C::NT;
  static constexpr int KC = 16 * ROWS / C::NT;
  static_assert(COLS ? (C::NT % ROWS == 0 && (KC == 4 || KC == 8))
                     : (ROWS % 8 == 0 && NR >= 1 && (ROWS * 4) % C::NT == 0),
                "operand tile does not fit the thread count");
  f32x4 r[COLS ? 1 : NR];
  float c[COLS ? KC : 1];
};

template <class C, int ROWS, bool COLS>
__device__ __forceinline__ void split_load(SplitOperand<C, ROWS, COLS>& o,
                                           const float* __restrict__ X, int ld, int r0, int k0) {
  using O = SplitOperand<C, ROWS, COLS>;
  const int tid = threadIdx.x;
  if constexpr (COLS) {
    const int row = tid % ROWS, kq = (tid / ROWS) * O::KC;
#pragma unroll
    for (int q = 0; q < O::KC; ++q) o.c[q] = X[(size_t)(k0 + kq + q) * ld + r0 + row];
  } else {
#pragma unroll
    for (int i = 0; i < O::NR; ++i) {
      const int c = tid + i * C::NT;
      o.r[i] = *reinterpret_cast<const f32x4*>(X + (size_t)(r0 + split_row(c)) * ld + k0 + (c % 4) * 4);
    }
  }
}

// Splits one operand's share into the planes at d ([plane][row][k], rows of
// LDX): three bf16 planes, or with F16 two fp16 planes of the values scaled
// by 2^e.
template <class C, int ROWS, bool COLS, bool F16 = false>
__device__ __forceinline__ void split_store(const SplitOperand<C, ROWS, COLS>& o, uint16_t* d,
                                            int e = 0) {
  using O = SplitOperand<C, ROWS, COLS>;
  constexpr int LD = C::LDX, P = ROWS * LD;
  const int tid = threadIdx.x;
  if constexpr (F16 && COLS) {
    uint16_t* dr = d + (tid % ROWS) * LD + (tid / ROWS) * O::KC;
    if constexpr (O::KC == 8) {
      const Split2 s0 = split2h(o.c[0], o.c[1], e), s1 = split2h(o.c[2], o.c[3], e);
      const Split2 s2 = split2h(o.c[4], o.c[5], e), s3 = split2h(o.c[6], o.c[7], e);
      *reinterpret_cast<u32x4*>(dr) = (u32x4){s0.h, s1.h, s2.h, s3.h};
      *reinterpret_cast<u32x4*>(dr + P) = (u32x4){s0.l, s1.l, s2.l, s3.l};
    } else {
      store_split4h(dr, P, (f32x4){o.c[0], o.c[1], o.c[2], o.c[3]}, e);
    }
  } else if constexpr (F16) {
#pragma unroll
    for (int i = 0; i < O::NR; ++i) {
      const int c = tid + i * C::NT;
      store_split4h(d + split_row(c) * LD + (c % 4) * 4, P, o.r[i], e);
    }
  } else if constexpr (COLS) {
    uint16_t* dr = d + (tid % ROWS) * LD + (tid / ROWS) * O::KC;
    if constexpr (O::KC == 8) {
      // 16-byte writes: eight consecutive rows per 128-byte group, 12 banks
      // apart, cover all 32 banks once
      const Split3 s0 = split3(o.c[0], o.c[1]), s1 = split3(o.c[2], o.c[3]);
      const Split3 s2 = split3(o.c[4], o.c[5]), s3 = split3(o.c[6], o.c[7]);
      *reinterpret_cast<u32x4*>(dr) = (u32x4){s0.h, s1.h, s2.h, s3.h};
      *reinterpret_cast<u32x4*>(dr + P) = (u32x4){s0.m, s1.m, s2.m, s3.m};
      *reinterpret_cast<u32x4*>(dr + 2 * P) = (u32x4){s0.l, s1.l, s2.l, s3.l};
    } else {
      store_split4(dr, P, (f32x4){o.c[0], o.c[1], o.c[2], o.c[3]});
    }
  } else {
#pragma unroll
    for (int i = 0; i < O::NR; ++i) {
      const int c = tid + i * C::NT;
      store_split4(d + split_row(c) * LD + (c % 4) * 4, P, o.r[i]);
    }
  }
}

// The six products of one K-tile from one LDS buffer: per fragment the wave
// reads 8 consecutive k of one row from every plane (lane l: row l % 32,
// k 8 (l / 32) + 0..7, the 32x32x16 bf16 MFMA's operand layout for both A and
// B), then runs the products product-major (smallest terms first), so
// consecutive MFMAs go to different accumulators.
template <class C, int MASK, bool F16 = false>
__device__ __forceinline__ void split_mma(floatx16 (&acc)[C::FM][C::FN], const uint16_t* sA,
                                          const uint16_t* sB, int wm, int wn) {
  constexpr int LD = C::LDX, PA = C::BM * LD, PB = C::BN * LD;
  const int lane = threadIdx.x & 63;
  const int half = lane >> 5, l32 = lane & 31;
  const uint16_t* a0 = sA + (wm * 32 * C::FM + l32) * LD + half * 8;
  const uint16_t* b0 = sB + (wn * 32 * C::FN + l32) * LD + half * 8;
  if constexpr (F16) {
    // the fp16 terms: lh, hl, hh (same operand layout as the bf16 MFMA)
    f16x8 a[2][C::FM], b[2][C::FN];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
#pragma unroll
      for (int i = 0; i < C::FM; ++i) a[p][i] = *reinterpret_cast<const f16x8*>(a0 + p * PA + i * 32 * LD);
#pragma unroll
      for (int j = 0; j < C::FN; ++j) b[p][j] = *reinterpret_cast<const f16x8*>(b0 + p * PB + j * 32 * LD);
    }
    constexpr int PP[3][2] = {{1, 0}, {0, 1}, {0, 0}};
#pragma unroll
    for (int q = 0; q < 3; ++q)
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
          if (MASK & (1 << (i * C::FN + j)))
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[PP[q][0]][i], b[PP[q][1]][j],
                                                               acc[i][j], 0, 0, 0);
    return;
  }
  bf16x8 a[3][C::FM], b[3][C::FN];
#pragma unroll
  for (int p = 0; p < 3; ++p) {
#pragma unroll
    for (int i = 0; i < C::FM; ++i) a[p][i] = *reinterpret_cast<const bf16x8*>(a0 + p * PA + i * 32 * LD);
#pragma unroll
    for (int j = 0; j < C::FN; ++j) b[p][j] = *reinterpret_cast<const bf16x8*>(b0 + p * PB + j * 32 * LD);
  }
  constexpr int PP[6][2] = {{2, 0}, {1, 1}, {0, 2}, {1, 0}, {0, 1}, {0, 0}};
#pragma unroll
  for (int q = 0; q < 6; ++q)
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
      for (int j = 0; j < C::FN; ++j)
        if (MASK & (1 << (i * C::FN + j)))
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[PP[q][0]][i], b[PP[q][1]][j],
                                                              acc[i][j], 0, 0, 0);
}

// ---------------------------------------------------------------------------
// Staggered main loop of the fp16 split on 256 x 256 tiles of eight waves.
// The waves of a workgroup run on SIMD w % 4, so waves 0-3 (group 0) and 4-7
// (group 1) put one wave of each group on every SIMD. Each group loads,
// splits and stores its half of the rows of every K-tile, and the groups run
// half a K-step apart: in every slot between two barriers one group runs the
// MFMAs of a K-tile on fragments already in registers, while the other reads
// the fragments of its next K-tile from LDS, splits its share of the tile
// after next into the other LDS buffer and issues the loads of the tile after
// that. On every SIMD the matrix work of one wave then overlaps the operand
// work of the other, where the lockstep loop (all waves in the same phase)
// serialises them. Each accumulator sees the same MFMAs in the same order as
// in the lockstep loop, so the results are bit-identical.
// ---------------------------------------------------------------------------
// One group's half (128 rows) of one row operand ([rows][K], k contiguous)
// of a K-tile of 16, 256 threads: two 4-value chunks, row split_row(c) and
// chunk c % 4 for c = tg + 256 i.
struct HalfOperand {
  f32x4 r[2];
};

__device__ __forceinline__ void half_load(HalfOperand& o, const float* __restrict__ X, int ld,
                                          int r0, int k0, int tg) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int c = tg + i * 256;
    o.r[i] = *reinterpret_cast<const f32x4*>(X + (size_t)(r0 + split_row(c)) * ld + k0 + (c % 4) * 4);
  }
}

// The two fp16 planes (scaled by 2^e) of a group's half at d, the group's
// first row in plane 0; planes P 16-bit words apart, rows of LDX.
template <class C>
__device__ __forceinline__ void half_store(const HalfOperand& o, uint16_t* d, int P, int e, int tg) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int c = tg + i * 256;
    store_split4h(d + split_row(c) * C::LDX + (c % 4) * 4, P, o.r[i], e);
  }
}

// A wave's fp16 fragments of one K-tile (both planes of A and of B), in the
// operand layout of split_mma.
template <class C>
struct HalfFrags {
  f16x8 a[2][C::FM], b[2][C::FN];
};

template <class C>
__device__ __forceinline__ void half_frag_read(HalfFrags<C>& f, const uint16_t* sA,
                                               const uint16_t* sB, int wm, int wn) {
  constexpr int LD = C::LDX, PA = C::BM * LD, PB = C::BN * LD;
  const int lane = threadIdx.x & 63;
  const int half = lane >> 5, l32 = lane & 31;
  const uint16_t* a0 = sA + (wm * 32 * C::FM + l32) * LD + half * 8;
  const uint16_t* b0 = sB + (wn * 32 * C::FN + l32) * LD + half * 8;
#pragma unroll
  for (int p = 0; p < 2; ++p) {
#pragma unroll
    for (int i = 0; i < C::FM; ++i) f.a[p][i] = *reinterpret_cast<const f16x8*>(a0 + p * PA + i * 32 * LD);
#pragma unroll
    for (int j = 0; j < C::FN; ++j) f.b[p][j] = *reinterpret_cast<const f16x8*>(b0 + p * PB + j * 32 * LD);
  }
}

// The three fp16 products (lh, hl, hh) of one K-tile, product-major.
template <class C, int MASK>
__device__ __forceinline__ void half_frag_mma(floatx16 (&acc)[C::FM][C::FN], const HalfFrags<C>& f) {
  constexpr int PP[3][2] = {{1, 0}, {0, 1}, {0, 0}};
#pragma unroll
  for (int q = 0; q < 3; ++q)
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
      for (int j = 0; j < C::FN; ++j)
        if (MASK & (1 << (i * C::FN + j)))
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(f.a[PP[q][0]][i], f.b[PP[q][1]][j],
                                                             acc[i][j], 0, 0, 0);
}

// A workgroup barrier that the scheduler does not move instructions across
// (left alone, it sinks MFMAs below an s_barrier, which undoes the stagger).
__device__ __forceinline__ void slot_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  __syncthreads();
  __builtin_amdgcn_sched_barrier(0);
}

// C = A B^T with both operands by rows ([rows][K], k contiguous), K a
// multiple of 16 and at least 32. Slots: group 0 runs the MFMAs of tile q in
// slot 2q and its operand work in slot 2q + 1; group 1 one slot later. Tile
// q + 2 goes into the buffer of tile q, whose last fragment reads (group 1,
// slot 2q) precede its first store (group 0, slot 2q + 1); tile q is
// complete after slot 2q - 2 and first read in slot 2q - 1. Both groups pass
// 2 nk + 1 barriers.
template <class C, int MASK, bool SAME>
__device__ __forceinline__ void mainloop_stagger(const float* __restrict__ A, int lda,
                                                 const float* __restrict__ B, int ldb, int K,
                                                 int m0, int n0, int wm, int wn,
                                                 floatx16 (&acc)[C::FM][C::FN], float* lds,
                                                 int ea, int eb) {
  static_assert(C::NT == 512 && C::BM == 256 && C::BN == 256, "256-tiles of eight waves");
  constexpr int PA = C::BM * C::LDX, PB = C::BN * C::LDX;
  uint16_t* sA0 = reinterpret_cast<uint16_t*>(lds);  // [2][2][BM][LDX]
  uint16_t* sA1 = sA0 + 2 * PA;
  uint16_t* sB0 = SAME ? sA0 : sA0 + 4 * PA;          // [2][2][BN][LDX]
  uint16_t* sB1 = SAME ? sA1 : sB0 + 2 * PB;
  const int grp = __builtin_amdgcn_readfirstlane(threadIdx.x >> 8);
  const int tg = threadIdx.x & 255;
  const int ra = m0 + grp * 128, rb = n0 + grp * 128;
  const int oa = grp * 128 * C::LDX;  // the group's first row in a plane
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  const int nk = K / 16;  // >= 2
  HalfOperand a, b;
  HalfFrags<C> fr;
  half_load(a, A, lda, ra, 0, tg);
  if constexpr (!SAME) half_load(b, B, ldb, rb, 0, tg);
  half_store<C>(a, sA0 + oa, PA, ea, tg);
  if constexpr (!SAME) half_store<C>(b, sB0 + oa, PB, eb, tg);
  half_load(a, A, lda, ra, 16, tg);
  if constexpr (!SAME) half_load(b, B, ldb, rb, 16, tg);
  half_store<C>(a, sA1 + oa, PA, ea, tg);
  if constexpr (!SAME) half_store<C>(b, sB1 + oa, PB, eb, tg);
  __syncthreads();
  if (nk > 2) {
    half_load(a, A, lda, ra, 32, tg);
    if constexpr (!SAME) half_load(b, B, ldb, rb, 32, tg);
  }
  half_frag_read<C>(fr, sA0, sB0, wm, wn);
  if (grp == 1) slot_barrier();  // group 1 runs one slot behind
  for (int q = 0; q < nk; ++q) {
    half_frag_mma<C, MASK>(acc, fr);
    slot_barrier();
    // operand slot: the fragments of tile q + 1 first (their LDS latency
    // then overlaps the split), then tile q + 2 where tile q was, then the
    // loads of tile q + 3
    const bool odd = q & 1;
    if (q + 1 < nk) half_frag_read<C>(fr, odd ? sA0 : sA1, odd ? sB0 : sB1, wm, wn);
    if (q + 2 < nk) {
      half_store<C>(a, (odd ? sA1 : sA0) + oa, PA, ea, tg);
      if constexpr (!SAME) half_store<C>(b, (odd ? sB1 : sB0) + oa, PB, eb, tg);
      if (q + 3 < nk) {
        half_load(a, A, lda, ra, (q + 3) * 16, tg);
        if constexpr (!SAME) half_load(b, B, ldb, rb, (q + 3) * 16, tg);
      }
    }
    if (grp == 0 || q + 1 < nk) slot_barrier();
  }
}

// acc[fm][fn] = sum over K of A[m0 + ...][k] * B[n0 + ...][k]: A is [M][K]
// with row stride lda (k contiguous), or with PCOLS its transpose [K][M] (row
// stride lda, m contiguous); B likewise [N][K] or, with QCOLS, [K][N]. K is a
// multiple of 32. Two LDS buffers of split planes and two register stages:
// while the MFMAs run on K-tile kt, the stage of tile kt + 1 (loaded one
// phase earlier) is split into the other buffer and tile kt + 2 is loaded
// into the freed stage, so every load has a full phase to land. F16: two
// fp16 planes of A 2^ea and B 2^eb and three products instead (the caller
// scales the sums back by 2^-(ea + eb)). SAME: B is A (same rows, same
// scale: a diagonal tile of a matrix times itself), so its rows are loaded,
// split and stored once and read as both operands.
template <class C, bool PCOLS, bool QCOLS, int MASK = -1, bool F16 = false, bool SAME = false>
__device__ __forceinline__ void mainloop_x6(const float* __restrict__ A, int lda,
                                            const float* __restrict__ B, int ldb, int K, int m0,
                                            int n0, int wm, int wn,
                                            floatx16 (&acc)[C::FM][C::FN], float* lds,
                                            int ea = 0, int eb = 0) {
  static_assert(!SAME || (C::BM == C::BN && PCOLS == QCOLS), "a shared panel is square");
  // the staggered loop for row operands on full tiles. With a column operand
  // (one scalar load per value) it measured slower than the lockstep loop's
  // two register stages (statistics of columns 5.63 -> 5.85 ms per launch at
  // 1152 blocks of 1024^2). On a diagonal tile (every wave masked) a slot
  // lasts as long as the busiest role of its group, 4 + 7 fragments of MFMAs
  // per K-tile, where lockstep pays the busiest SIMD's pair, 3 + 7.
  if constexpr (F16 && C::NT == 512 && C::BM == 256 && C::BN == 256 && !PCOLS && !QCOLS &&
                MASK == -1) {
    mainloop_stagger<C, MASK, SAME>(A, lda, B, ldb, K, m0, n0, wm, wn, acc, lds, ea, eb);
    return;
  }
  constexpr int NPL = F16 ? 2 : 3;                          // planes per operand
  constexpr int PA = C::BM * C::LDX, PB = C::BN * C::LDX;  // one plane, in 16-bit words
  uint16_t* sA0 = reinterpret_cast<uint16_t*>(lds);  // [2][NPL][BM][LDX]
  uint16_t* sA1 = sA0 + NPL * PA;
  uint16_t* sB0 = SAME ? sA0 : sA0 + 2 * NPL * PA;    // [2][NPL][BN][LDX]
  uint16_t* sB1 = SAME ? sA1 : sB0 + NPL * PB;
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  const int nk = K / 16;  // even
  SplitOperand<C, C::BM, PCOLS> a0, a1;
  SplitOperand<C, C::BN, QCOLS> b0, b1;
  split_load<C, C::BM, PCOLS>(a0, A, lda, m0, 0);
  if constexpr (!SAME) split_load<C, C::BN, QCOLS>(b0, B, ldb, n0, 0);
  split_load<C, C::BM, PCOLS>(a1, A, lda, m0, 16);
  if constexpr (!SAME) split_load<C, C::BN, QCOLS>(b1, B, ldb, n0, 16);
  split_store<C, C::BM, PCOLS, F16>(a0, sA0, ea);
  if constexpr (!SAME) split_store<C, C::BN, QCOLS, F16>(b0, sB0, eb);
  __syncthreads();
  for (int kt = 0; kt < nk; kt += 2) {
    // tile kt from buffer 0; tile kt + 1 (stage 1) into buffer 1; tile kt + 2
    // into stage 0 (the last pair repeats tile nk - 1, in bounds and unused)
    const int k2 = min(kt + 2, nk - 1) * 16, k3 = min(kt + 3, nk - 1) * 16;
    split_load<C, C::BM, PCOLS>(a0, A, lda, m0, k2);
    if constexpr (!SAME) split_load<C, C::BN, QCOLS>(b0, B, ldb, n0, k2);
    split_mma<C, MASK, F16>(acc, sA0, sB0, wm, wn);
    split_store<C, C::BM, PCOLS, F16>(a1, sA1, ea);
    if constexpr (!SAME) split_store<C, C::BN, QCOLS, F16>(b1, sB1, eb);
    __syncthreads();
    // tile kt + 1 from buffer 1; tile kt + 2 (stage 0) into buffer 0; tile
    // kt + 3 into stage 1
    split_load<C, C::BM, PCOLS>(a1, A, lda, m0, k3);
    if constexpr (!SAME) split_load<C, C::BN, QCOLS>(b1, B, ldb, n0, k3);
    split_mma<C, MASK, F16>(acc, sA1, sB1, wm, wn);
    if (kt + 2 < nk) {
      split_store<C, C::BM, PCOLS, F16>(a0, sA0, ea);
      if constexpr (!SAME) split_store<C, C::BN, QCOLS, F16>(b0, sB0, eb);
    }
    __syncthreads();
  }
}

// Undoes the operand scaling of the fp16 split on the sums (exact unless the
// result leaves the fp32 range).
template <class C>
__device__ __forceinline__ void unscale_acc(floatx16 (&acc)[C::FM][C::FN], int e) {
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = ldexpf(acc[i][j][r], e);
}

template <int FM, int FN>
constexpr int upper_mask() {
  int m = 0;
  for (int i = 0; i < FM; ++i)
    for (int j = 0; j < FN; ++j)
      if (i <= j) m |= 1 << (i * FN + j);
  return m;
}

// Fragments of rows i < FM / 2 (top) or i >= FM / 2 (bottom).
template <int FM, int FN>
constexpr int half_mask(bool bottom) {
  int m = 0;
  for (int i = 0; i < FM; ++i)
    for (int j = 0; j < FN; ++j)
      if ((i >= FM / 2) == bottom) m |= 1 << (i * FN + j);
  return m;
}

// Which fragments a wave computes on a symmetric product's tile. Off the
// diagonal: its own block, all fragments. On a diagonal tile only the upper
// triangle is needed: a wave on the diagonal runs its upper fragments; the
// block above the diagonal is split by rows between its own wave and the
// mirror wave below the diagonal (which would otherwise idle), so the tile
// takes 3 fragment times instead of 4 with 2 x 2 fragments per wave. The
// choice is per wave (the wave index is uniform; readfirstlane tells the
// compiler so) and made outside the K loop.
template <class C, bool SQUARE = (C::FM == C::FN && C::WM == C::WN)>
struct SymWave {
  int wm, wn, mask;
  __device__ __forceinline__ SymWave(bool diag) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    wm = wave % C::WM;
    wn = wave / C::WM;
    mask = -1;
    if (!diag) return;
    if (wm == wn) {
      mask = upper_mask<C::FM, C::FN>();
    } else if (C::FM >= 2) {
      const bool below = wm > wn;
      if (below) {
        const int t = wm;
        wm = wn;
        wn = t;
      }
      mask = below ? half_mask<C::FM, C::FN>(true) : half_mask<C::FM, C::FN>(false);
    } else if (wm > wn) {
      mask = 0;
    }
  }
};

// 256 x 256 tiles of eight waves of 128 x 64 (2 x 4 waves, 4 x 2 fragments
// each). On a diagonal tile only the upper triangle of the 8 x 8 fragments
// (36) is needed: the blocks crossing the diagonal take 3 or 7 fragments, the
// two full blocks above it are split in halves of 4, the two blocks below it
// are not computed. Wave w runs on SIMD w % 4, so the roles are dealt to pair
// a 3 with a 7 and a 4 with a 4 on every SIMD: the busiest SIMD runs 10
// fragment products where a full tile runs 16.
template <class C>
struct SymWave<C, false> {
  static_assert(C::WM == 2 && C::WN == 4 && C::FM == 4 && C::FN == 2, "the 256-tile layout");
  static constexpr int kCross0 = 0x0B;   // rows 0-3 x cols 0-1 on or above the diagonal
  static constexpr int kCross1 = 0xBF;   // rows 0-3 x cols 2-3 on or above the diagonal
  static constexpr int kTop = 0x0F, kBottom = 0xF0;
  int wm, wn, mask;
  __device__ __forceinline__ SymWave(bool diag) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    wm = wave % C::WM;
    wn = wave / C::WM;
    mask = -1;
    if (!diag) return;
    // role of wave 0..7: block (wm, wn) and its fragment mask
    constexpr int kWm = 0x22;        // bits: waves 1 and 5 take blocks of row 1
    constexpr int kWn = 0xEDE8;      // two bits per wave: 0, 2, 2, 3, 1, 3, 2, 3
    wm = (kWm >> wave) & 1;
    wn = (kWn >> (2 * wave)) & 3;
    mask = (wave & 3) < 2 ? ((wave & 4) ? kCross1 : kCross0) : ((wave & 4) ? kBottom : kTop);
  }
};

// The symmetric products' main-loop dispatch by the wave's fragment mask
// (-1 off the diagonal, the roles of a diagonal tile on it).
template <class C>
__device__ __forceinline__ void mainloop_sym(const float* __restrict__ P,
                                             const float* __restrict__ Q, int M, int N, int K,
                                             int m0, int n0, floatx16 (&acc)[C::FM][C::FN],
                                             float* lds, const SymWave<C>& sw) {
  constexpr int kUpper = upper_mask<C::FM, C::FN>();
  constexpr int kTop = half_mask<C::FM, C::FN>(false), kBottom = half_mask<C::FM, C::FN>(true);
  if (sw.mask == -1)
    mainloop_w<C>(P, Q, M, N, K, m0, n0, sw.wm, sw.wn, acc, lds);
  else if (sw.mask == kUpper)
    mainloop_w<C, kUpper>(P, Q, M, N, K, m0, n0, sw.wm, sw.wn, acc, lds);
  else if (C::FM >= 2 && sw.mask == kTop)
    mainloop_w<C, kTop>(P, Q, M, N, K, m0, n0, sw.wm, sw.wn, acc, lds);
  else if (C::FM >= 2 && sw.mask == kBottom)
    mainloop_w<C, kBottom>(P, Q, M, N, K, m0, n0, sw.wm, sw.wn, acc, lds);
  else
    mainloop_w<C, 0>(P, Q, M, N, K, m0, n0, sw.wm, sw.wn, acc, lds);
}

template <class C>
__device__ __forceinline__ void mainloop_sym_bf16(const uint16_t* __restrict__ X, int K, int m0,
                                                  int n0, floatx16 (&acc)[C::FM][C::FN],
                                                  float* lds, const SymWave<C>& sw) {
  if (sw.mask == -1) {
    mainloop_bf16<C>(X, K, m0, n0, sw.wm, sw.wn, acc, lds);
  } else if constexpr (C::FM != C::FN) {
    using W = SymWave<C>;
    // a diagonal tile reads one panel
    if (sw.mask == W::kCross0)
      mainloop_bf16<C, W::kCross0, true>(X, K, m0, m0, sw.wm, sw.wn, acc, lds);
    else if (sw.mask == W::kCross1)
      mainloop_bf16<C, W::kCross1, true>(X, K, m0, m0, sw.wm, sw.wn, acc, lds);
    else if (sw.mask == W::kTop)
      mainloop_bf16<C, W::kTop, true>(X, K, m0, m0, sw.wm, sw.wn, acc, lds);
    else
      mainloop_bf16<C, W::kBottom, true>(X, K, m0, m0, sw.wm, sw.wn, acc, lds);
    return;
  } else {
  constexpr int kUpper = upper_mask<C::FM, C::FN>();
  constexpr int kTop = half_mask<C::FM, C::FN>(false), kBottom = half_mask<C::FM, C::FN>(true);
  if (sw.mask == kUpper)
    mainloop_bf16<C, kUpper>(X, K, m0, n0, sw.wm, sw.wn, acc, lds);
  else if (C::FM >= 2 && sw.mask == kTop)
    mainloop_bf16<C, kTop>(X, K, m0, n0, sw.wm, sw.wn, acc, lds);
  else if (C::FM >= 2 && sw.mask == kBottom)
    mainloop_bf16<C, kBottom>(X, K, m0, n0, sw.wm, sw.wn, acc, lds);
  else
    mainloop_bf16<C, 0>(X, K, m0, n0, sw.wm, sw.wn, acc, lds);
  }
}

// COLS: both operands stored [K][M] (m contiguous, row stride M), as the
// statistics of a matrix's columns read the packed block; otherwise rows
// with k contiguous (row stride K).
template <class C, bool COLS, bool F16 = false>
__device__ __forceinline__ void mainloop_sym_x6(const float* __restrict__ A,
                                                const float* __restrict__ B, int M, int K, int m0,
                                                int n0, floatx16 (&acc)[C::FM][C::FN],
                                                float* lds, const SymWave<C>& sw, int ea = 0,
                                                int eb = 0) {
  const int ld = COLS ? M : K;
  if (sw.mask == -1) {
    mainloop_x6<C, COLS, COLS, -1, F16>(A, ld, B, ld, K, m0, n0, sw.wm, sw.wn, acc, lds, ea, eb);
  } else if constexpr (C::FM != C::FN) {
    using W = SymWave<C>;
    // a diagonal tile of a matrix times itself: one panel serves both operands
    const bool same = A == B && ea == eb;
    if (same) {
      if (sw.mask == W::kCross0)
        mainloop_x6<C, COLS, COLS, W::kCross0, F16, true>(A, ld, A, ld, K, m0, m0, sw.wm, sw.wn, acc, lds, ea, ea);
      else if (sw.mask == W::kCross1)
        mainloop_x6<C, COLS, COLS, W::kCross1, F16, true>(A, ld, A, ld, K, m0, m0, sw.wm, sw.wn, acc, lds, ea, ea);
      else if (sw.mask == W::kTop)
        mainloop_x6<C, COLS, COLS, W::kTop, F16, true>(A, ld, A, ld, K, m0, m0, sw.wm, sw.wn, acc, lds, ea, ea);
      else
        mainloop_x6<C, COLS, COLS, W::kBottom, F16, true>(A, ld, A, ld, K, m0, m0, sw.wm, sw.wn, acc, lds, ea, ea);
    } else if (sw.mask == W::kCross0)
      mainloop_x6<C, COLS, COLS, W::kCross0, F16>(A, ld, B, ld, K, m0, n0, sw.wm, sw.wn, acc, lds, ea, eb);
    else if (sw.mask == W::kCross1)
      mainloop_x6<C, COLS, COLS, W::kCross1, F16>(A, ld, B, ld, K, m0, n0, sw.wm, sw.wn, acc, lds, ea, eb);
    else if (sw.mask == W::kTop)
      mainloop_x6<C, COLS, COLS, W::kTop, F16>(A, ld, B, ld, K, m0, n0, sw.wm, sw.wn, acc, lds, ea, eb);
    else
      mainloop_x6<C, COLS, COLS, W::kBottom, F16>(A, ld, B, ld, K, m0, n0, sw.wm, sw.wn, acc, lds, ea, eb);
    return;
  } else {
  constexpr int kUpper = upper_mask<C::FM, C::FN>();
  constexpr int kTop = half_mask<C::FM, C::FN>(false), kBottom = half_mask<C::FM, C::FN>(true);
  if (sw.mask == kUpper)
    mainloop_x6<C, COLS, COLS, kUpper, F16>(A, ld, B, ld, K, m0, n0, sw.wm, sw.wn, acc, lds, ea, eb);
  else if (C::FM >= 2 && sw.mask == kTop)
    mainloop_x6<C, COLS, COLS, kTop, F16>(A, ld, B, ld, K, m0, n0, sw.wm, sw.wn, acc, lds, ea, eb);
  else if (C::FM >= 2 && sw.mask == kBottom)
    mainloop_x6<C, COLS, COLS, kBottom, F16>(A, ld, B, ld, K, m0, n0, sw.wm, sw.wn, acc, lds, ea, eb);
  else
    mainloop_x6<C, COLS, COLS, 0, F16>(A, ld, B, ld, K, m0, n0, sw.wm, sw.wn, acc, lds, ea, eb);
  }
}

// Row / column of accumulator register r of fragment (i, j) of the wave's
// block (wm, wn).
template <class C>
__device__ __forceinline__ int frag_row_w(int m0, int wm, int i, int r) {
  const int lane = threadIdx.x & 63;
  return m0 + wm * 32 * C::FM + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
}
template <class C>
__device__ __forceinline__ int frag_col_w(int n0, int wn, int j) {
  const int lane = threadIdx.x & 63;
  return n0 + wn * 32 * C::FN + j * 32 + (lane & 31);
}
template <class C>
__device__ __forceinline__ int frag_row(int m0, int i, int r) {
  return frag_row_w<C>(m0, (threadIdx.x >> 6) % C::WM, i, r);
}
template <class C>
__device__ __forceinline__ int frag_col(int n0, int j) {
  return frag_col_w<C>(n0, (threadIdx.x >> 6) / C::WM, j);
}

// ---------------------------------------------------------------------------
// Symmetric product: only tiles on or above the diagonal are computed; each
// is written to its place and mirrored, so the stored result is exactly
// symmetric. Used by the statistics (EMA epilogue) and the Newton chain.
// ---------------------------------------------------------------------------
// Operand paths of the products: fp32 MFMA, bf16 operands (bf16
// statistics), fp32 operands split into three bf16 terms or (scaled) into two
// fp16 terms, each with operands read by rows or by columns.
enum : int {
  kPathF32 = 0,
  kPathBF16 = 1,
  kPathSplit = 2,
  kPathSplitCols = 3,
  kPathSplitH = 4,
  kPathSplitHCols = 5
};
constexpr bool path_split(int p) { return p >= kPathSplit; }
constexpr bool path_f16(int p) { return p == kPathSplitH || p == kPathSplitHCols; }
constexpr bool path_cols(int p) { return p == kPathSplitCols || p == kPathSplitHCols; }

template <class C, int PATH>
constexpr int lds_floats() {
  return path_f16(PATH) ? C::LDS_SPLITH : path_split(PATH) ? C::LDS_SPLIT : C::LDS_FLOATS;
}

// The main loop of one tile of a symmetric product on its operand path.
template <class C, int PATH>
__device__ __forceinline__ void sym_mainloop(const GemmProblem& pb, int f, int m0, int n0,
                                             floatx16 (&acc)[C::FM][C::FN], float* lds,
                                             const SymWave<C>& sw) {
  if constexpr (PATH == kPathBF16) {
    mainloop_sym_bf16<C>(pb.Xh + (size_t)f * pb.sXh, pb.K, m0, n0, acc, lds, sw);
  } else if constexpr (path_f16(PATH)) {
    const int ea = f16_exp(pb.mP[f]), eb = f16_exp(pb.mQ[f]);
    mainloop_sym_x6<C, path_cols(PATH), true>(pb.P + (size_t)f * pb.sP,
                                                    pb.Q + (size_t)f * pb.sQ, pb.M, pb.K, m0, n0,
                                                    acc, lds, sw, ea, eb);
    unscale_acc<C>(acc, -(ea + eb));
  } else if constexpr (path_split(PATH)) {
    // operands by rows, or (statistics of a matrix's columns) by columns
    mainloop_sym_x6<C, path_cols(PATH)>(pb.P + (size_t)f * pb.sP, pb.Q + (size_t)f * pb.sQ,
                                              pb.M, pb.K, m0, n0, acc, lds, sw);
  } else {
    mainloop_sym<C>(pb.P + (size_t)f * pb.sP, pb.Q + (size_t)f * pb.sQ, pb.M, pb.N, pb.K, m0,
                          n0, acc, lds, sw);
  }
}

// The affine terms D of fragments q0 .. q0 + GF - 1 of a wave's block (zero
// for masked fragments, or without D).
template <class C, int GF>
__device__ __forceinline__ void sym_load_terms(float (&d)[GF][16], int q0, const SymWave<C>& sw,
                                               int m0, int n0, int N, const float* Db) {
#pragma unroll
  for (int q = 0; q < GF; ++q) {
    const int i = (q0 + q) / C::FN, j = (q0 + q) % C::FN;
    if (!((sw.mask >> (i * C::FN + j)) & 1)) continue;  // wave-uniform
    const int col = frag_col_w<C>(n0, sw.wn, j);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const uint32_t o = (uint32_t)(frag_row_w<C>(m0, sw.wm, i, r) * N + col);
      d[q][r] = Db != nullptr ? Db[o] : 0.f;
    }
  }
}

// The symmetric epilogue over a wave's fragments (see sym_product): C =
// alpha acc + beta D + beta2 D2 (+ the Chebyshev terms) + gamma I on and
// above the diagonal and the mirror below it. diag: the tile holds the
// diagonal (elements below it are not stored, the identity term applies on
// it); off the diagonal every element lies strictly above it, and a branch
// per fragment takes stores without per-element tests (two instantiations
// of the whole epilogue, one per kind of tile, ran out of registers). Offsets
// are 32-bit (a factor has at most 4096^2 elements): one 32-bit offset per
// element instead of 64-bit index arithmetic.
// Adds this lane's share of ||C - I||_F^2 to rs and of max |C| to mx, in the
// order of the elements.
template <class C, int PATH, bool TERMS, bool AFF2 = true>
__device__ __forceinline__ void sym_epilogue(const floatx16 (&acc)[C::FM][C::FN],
                                             const SymWave<C>& sw, bool diag, float* lds, int m0,
                                             int n0, int N,
                                             float* Cb, const float* Db, const float* D2b,
                                             const float* E1b, const float* E2b, float e_alpha,
                                             float e_beta, float e_beta2, float e_gamma,
                                             float e_t1, float e_t2, float& rs, float& mx) {
  // AFF2: the second affine term may be present (the Chebyshev products'
  // Clenshaw term). The statistics (the EMA term) and the Newton products
  // have one term at most, and its registers let one whole fragment load per
  // round trip (a wait for a load also waits for every store before it, so
  // fewer round trips mean fewer waits on the stores).
  constexpr bool WIDE = PATH == kPathSplit || PATH == kPathSplitH;
  constexpr bool BATCH = WIDE || !AFF2;
  constexpr int NF = C::FM * C::FN;
  constexpr int GF = WIDE && NF >= 2 && AFF2 ? 2 : 1;  // fragments per batch
  constexpr int HOIST = BATCH ? 16 : 4;
  // PIPE (whole-fragment batches with the EMA or Newton term only): the
  // terms of the next fragment are loaded before this fragment's stores, so
  // the wait for them does not cover those stores; one fragment of terms in
  // flight while another is consumed takes the registers of the second term
  // (per launch on the 1B sets: bf16 statistics 5.75 -> 4.79 ms, statistics
  // of columns 5.25 -> 5.15, of rows 4.52 -> 4.41; two fragments per batch
  // measured slower, 5.17 for the bf16 statistics).
  constexpr bool PIPE = BATCH && !AFF2 && !TERMS;
  float nxt[GF][16];
  if constexpr (PIPE) sym_load_terms<C, GF>(nxt, 0, sw, m0, n0, N, Db);
  // Off-diagonal mirrors pass through a wave-private 32 x 32 transpose buffer
  // (rows of kTP floats: the 16-byte writes of 16 lanes cover the 64 banks
  // once) and leave as whole 128-byte row segments instead of 16 bytes in
  // each of 64 rows. Every main loop ends with a barrier after its last LDS
  // read; the buffers start after the residual partials (lds[0..7]).
  constexpr int kTP = 36;
  static_assert(64 + (C::NT / 64) * 32 * kTP <= lds_floats<C, PATH>(), "LDS of the transpose buffers");
  const int lane = threadIdx.x & 63;
  float* tw = lds + 64 + (threadIdx.x >> 6) * 32 * kTP;
  // The affine terms are loaded before their stores: the stores may alias
  // them as far as the compiler knows (the statistics update in place), which
  // would otherwise hold every load behind the store before it. No store
  // below targets an element another lane reads here. With one term at most
  // (PIPE) a whole fragment's terms load per round trip, the next fragment's
  // before this one's stores; with two, the split rows paths load two whole
  // fragments per batch and the others HOIST registers of one fragment at a
  // time.
#pragma unroll
  for (int q0 = 0; q0 < NF; q0 += GF) {
    float dv[GF][HOIST], d2v[GF][HOIST], ev[GF][TERMS ? HOIST : 1];
    if constexpr (PIPE) {
#pragma unroll
      for (int q = 0; q < GF; ++q)
#pragma unroll
        for (int r = 0; r < HOIST; ++r) {
          dv[q][r] = nxt[q][r];
          d2v[q][r] = 0.f;
        }
      if (q0 + GF < NF) sym_load_terms<C, GF>(nxt, q0 + GF, sw, m0, n0, N, Db);
    } else if constexpr (BATCH) {
#pragma unroll
      for (int q = 0; q < GF; ++q) {
        const int i = (q0 + q) / C::FN, j = (q0 + q) % C::FN;
        if (!((sw.mask >> (i * C::FN + j)) & 1)) continue;  // wave-uniform
        const int col = frag_col_w<C>(n0, sw.wn, j);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const uint32_t o = (uint32_t)(frag_row_w<C>(m0, sw.wm, i, r) * N + col);
          dv[q][r] = Db != nullptr ? Db[o] : 0.f;
          d2v[q][r] = AFF2 && D2b != nullptr ? D2b[o] : 0.f;
          if constexpr (TERMS)
            ev[q][r] = (E1b != nullptr ? e_t1 * E1b[o] : 0.f) + (E2b != nullptr ? e_t2 * E2b[o] : 0.f);
        }
      }
    }
#pragma unroll
    for (int q = 0; q < GF; ++q) {
      const int i = (q0 + q) / C::FN, j = (q0 + q) % C::FN;
      if (!((sw.mask >> (i * C::FN + j)) & 1)) continue;  // wave-uniform
      const int col = frag_col_w<C>(n0, sw.wn, j);
      // off the diagonal (a uniform test per fragment) every element is stored
      // and mirrored, the identity term never applies: the same arithmetic
      // without the per-element tests of a diagonal tile
      if (!TERMS && !diag) {  // (the Chebyshev products' registers keep them on one path)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          if constexpr (!BATCH) {
            if ((4 * g4) % HOIST == 0) {
#pragma unroll
              for (int r = 0; r < HOIST; ++r) {
                const uint32_t o = (uint32_t)(frag_row_w<C>(m0, sw.wm, i, 4 * g4 + r) * N + col);
                dv[q][r] = Db != nullptr ? Db[o] : 0.f;
                d2v[q][r] = AFF2 && D2b != nullptr ? D2b[o] : 0.f;
                if constexpr (TERMS)
                  ev[q][r] = (E1b != nullptr ? e_t1 * E1b[o] : 0.f) +
                             (E2b != nullptr ? e_t2 * E2b[o] : 0.f);
              }
            }
          }
          const int row0 = frag_row_w<C>(m0, sw.wm, i, 4 * g4);
          f32x4 v;
#pragma unroll
          for (int qq = 0; qq < 4; ++qq) {
            const int h = (4 * g4 + qq) % HOIST;
            float x = e_alpha * acc[i][j][4 * g4 + qq];
            x += e_beta * dv[q][h];
            x += e_beta2 * d2v[q][h];
            if constexpr (TERMS) x += ev[q][h];
            v[qq] = x;
            Cb[(uint32_t)((row0 + qq) * N + col)] = x;
            rs += 2.f * x * x;
            if constexpr (path_f16(PATH)) mx = fmaxf(mx, fabsf(x));
          }
          *reinterpret_cast<f32x4*>(tw + (lane & 31) * kTP + g4 * 8 + (lane >> 5) * 4) = v;
        }
        // the mirror: row cbase + rr of the result, columns rbase + cc..+3
        const int rbase = m0 + sw.wm * 32 * C::FM + i * 32, cbase = col - (lane & 31);
#pragma unroll
        for (int it = 0; it < 4; ++it) {
          const int rr = it * 8 + (lane >> 3), cc = (lane & 7) * 4;
          *reinterpret_cast<f32x4*>(Cb + (uint32_t)((cbase + rr) * N + rbase + cc)) =
              *reinterpret_cast<const f32x4*>(tw + rr * kTP + cc);
        }
        continue;
      }
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        if constexpr (!BATCH) {
          if ((4 * g4) % HOIST == 0) {
#pragma unroll
            for (int r = 0; r < HOIST; ++r) {
              const uint32_t o = (uint32_t)(frag_row_w<C>(m0, sw.wm, i, 4 * g4 + r) * N + col);
              dv[q][r] = Db != nullptr ? Db[o] : 0.f;
              d2v[q][r] = AFF2 && D2b != nullptr ? D2b[o] : 0.f;
              if constexpr (TERMS)
                ev[q][r] = (E1b != nullptr ? e_t1 * E1b[o] : 0.f) +
                           (E2b != nullptr ? e_t2 * E2b[o] : 0.f);
            }
          }
        }
        const int row0 = frag_row_w<C>(m0, sw.wm, i, 4 * g4);
        f32x4 v;
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
          const int row = row0 + qq;
          const int h = (4 * g4 + qq) % HOIST;
          float x = e_alpha * acc[i][j][4 * g4 + qq];
          x += e_beta * dv[q][h];
          x += e_beta2 * d2v[q][h];
          if constexpr (TERMS) x += ev[q][h];
          if (diag && row == col) x += e_gamma;
          v[qq] = x;
          if (!diag || row <= col) {
            Cb[(uint32_t)(row * N + col)] = x;
            const float d = x - (diag && row == col ? 1.f : 0.f);
            rs += (diag && row == col ? 1.f : 2.f) * d * d;
            if constexpr (path_f16(PATH)) mx = fmaxf(mx, fabsf(x));
          }
        }
        if (!diag || row0 + 3 < col) {
          *reinterpret_cast<f32x4*>(Cb + (uint32_t)(col * N + row0)) = v;
        } else {
#pragma unroll
          for (int qq = 0; qq < 4; ++qq)
            if (row0 + qq < col) Cb[(uint32_t)(col * N + row0 + qq)] = v[qq];
        }
      }
    }
  }
}

// One tile (ti <= tj) of a symmetric product for factor f.
template <class C, int PATH, bool TERMS, bool AFF2>
__device__ __forceinline__ void sym_tile(const GemmProblem& pb, int f, int tile, int T, float* lds,
                                         float* red) {
  int t = tile, ti = 0;
  while (t >= T - ti) {
    t -= T - ti;
    ++ti;
  }
  const int tj = ti + t;
  const int m0 = ti * C::BM, n0 = tj * C::BN;

  const bool diag = (ti == tj);
  const SymWave<C> sw(diag);
  floatx16 acc[C::FM][C::FN];
  sym_mainloop<C, PATH>(pb, f, m0, n0, acc, lds, sw);

  float* Cb = pb.C + (size_t)f * pb.sC;
  const float* Db = pb.D != nullptr ? pb.D + (size_t)f * pb.sD : nullptr;
  const float* D2b = pb.D2 != nullptr ? pb.D2 + (size_t)f * pb.sD2 : nullptr;
  float e_alpha = pb.alpha, e_beta = pb.beta, e_beta2 = pb.beta2, e_gamma = pb.gamma;
  float e_t1 = 0.f, e_t2 = 0.f;
  if (pb.coef != nullptr) {
    const float* cf = pb.coef + (size_t)(pb.f0 + f) * pb.coef_stride;
    e_alpha = cf[0];
    e_beta = cf[1];
    e_beta2 = cf[2];
    e_gamma = cf[3];
    if constexpr (TERMS) {
      e_t1 = cf[4];
      e_t2 = cf[5];
    }
  }
  const float* E1b = TERMS && pb.E1 != nullptr ? pb.E1 + (size_t)f * pb.sE : nullptr;
  const float* E2b = TERMS && pb.E2 != nullptr ? pb.E2 + (size_t)f * pb.sE : nullptr;
  const int N = pb.N;
  float rs = 0.f;
  float mx = 0.f;  // largest |value| stored (fp16 split: the result's maximum)
  sym_epilogue<C, PATH, TERMS, AFF2>(acc, sw, diag, lds, m0, n0, N, Cb, Db, D2b, E1b, E2b,
                                     e_alpha, e_beta, e_beta2, e_gamma, e_t1, e_t2, rs, mx);
  if constexpr (path_f16(PATH))
    if (pb.mC != nullptr) raise_max(pb.mC + f, mx, pb.ver);
  if (pb.resid != nullptr) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) rs += __shfl_xor(rs, o);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = rs;
    __syncthreads();
    if (threadIdx.x == 0) {
      float s = 0.f;
      for (int w = 0; w < C::NT / 64; ++w) s += red[w];
      pb.resid[(size_t)(pb.f0 + f) * pb.resid_stride + tile] = s;
    }
  }
}


// Live-factor table of a persistent symmetric launch, one byte per factor
// slot of the workgroup's XCD; problems with more slots read the status words
// per tile instead.
constexpr int kMaxSlots = 4096;

// Persistent Newton products on 256-tiles only: they hold one workgroup per
// CU and the whole register file either way, while the loop's extra live
// values would cost the smaller tiles a wave per SIMD.
template <class C>
constexpr bool kPersistSym = C::NT == 512;

// TERMS: the epilogue also adds coef[4] E1 + coef[5] E2 (the Chebyshev giant
// steps); a separate instantiation, so the other products keep their registers.
//
// Matrices are dealt to the XCDs round-robin (matrix f on XCD f % 8; the XCD
// workgroup b runs on is b % 8) and each XCD runs the units (matrix slot j,
// tile) of its matrices in order, so an L2 serves all tiles of a matrix and,
// when converged factors drop out of a Newton launch, every XCD keeps its
// share of the remaining ones. Without PERSIST a workgroup takes one unit.
// PERSIST (the Newton products, whose launches lose factors as they
// converge): the grid holds at most as
// many workgroups as the device runs at once, each taking every (gridDim.x /
// 8)-th unit of its XCD, so a launch whose factors have all stopped costs one
// status read per factor instead of the dispatch of every tile.
// AFF2 = false (the statistics): no second affine term.
template <class C, int PATH = kPathF32, bool TERMS = false, bool PERSIST = false, bool AFF2 = true>
__device__ __forceinline__ void sym_product(const GemmLaunch& g) {
  __shared__ float lds[lds_floats<C, PATH>()];
  float* red = lds;  // residual partials reuse the operand tiles after the K loop
  const GemmProblem& pb = g.p[blockIdx.y];
  const int T = pb.M / C::BM;
  const int ntile = T * (T + 1) / 2;
  const int xcd = blockIdx.x & 7;
  if constexpr (!PERSIST) {
    const int u = blockIdx.x >> 3;
    const int j = u / ntile;
    const int tile = u - j * ntile;
    const int f = j * 8 + xcd;
    if (f >= pb.batch) return;
    if (pb.status != nullptr) {
      const int st = pb.status[pb.f0 + f];
      if (st != 0 && !(pb.also_status != 0 && st == pb.also_status)) return;
    }
    sym_tile<C, PATH, TERMS, AFF2>(pb, f, tile, T, lds, red);
  } else {
    // live-factor table, one byte per slot of this XCD; problems with more
    // slots read the status words per tile instead
    __shared__ uint8_t live[kMaxSlots];
    const int nslot = (pb.batch - xcd + 7) / 8;  // slots j: factor f = 8 j + xcd < batch
    if (nslot <= 0) return;
    const bool filter = pb.status != nullptr;
    const bool table = filter && nslot <= kMaxSlots;
    if (table) {
      int n = 0;
      for (int j = threadIdx.x; j < nslot; j += C::NT) {
        const int st = pb.status[pb.f0 + j * 8 + xcd];
        const int a = st == 0 || (pb.also_status != 0 && st == pb.also_status);
        live[j] = (uint8_t)a;
        n += a;
      }
      if (!__syncthreads_or(n)) return;
    }
    const int units = nslot * ntile;
    for (int u = blockIdx.x >> 3; u < units; u += gridDim.x >> 3) {
      const int j = u / ntile;
      const int tile = u - j * ntile;
      const int f = j * 8 + xcd;
      if (table && !live[j]) continue;
      if (filter && !table) {
        const int st = pb.status[pb.f0 + f];
        if (st != 0 && !(pb.also_status != 0 && st == pb.also_status)) continue;
      }
      // the previous tile's last LDS uses (transpose buffers, partials) end here
      __syncthreads();
      sym_tile<C, PATH, TERMS, AFF2>(pb, f, tile, T, lds, red);
    }
  }
}

// Statistics: L <- beta2 L + g Gp Gp^T, R <- beta2 R + g Gp^T Gp (fp32 path:
// P = Q = GpT for L, Gp for R; split path: the row operands, Gp for L and
// GpT for R).
template <class C, int PATH>
__global__ __launch_bounds__(C::NT, path_split(PATH) ? 2 : 4) void syrk_ema_kernel(GemmLaunch g) {
  sym_product<C, PATH, false, false, false>(g);
}

// Statistics from bf16 packed gradients: L <- beta2 L + g Gp Gp^T reads GpH
// (rows of Gp), R <- beta2 R + g Gp^T Gp reads GpTH (rows of Gp^T).
template <class C>
__global__ __launch_bounds__(C::NT, C::NT == 512 ? 2 : 3) void syrk_bf16_kernel(GemmLaunch g) {
  sym_product<C, kPathBF16, false, false, false>(g);
}

// One product of the coupled Newton chain (T T, X T, T2 T2 or T4 M); every
// operand is symmetric, so P and Q serve as row operands as they are.
template <class C, int PATH>
__global__ __launch_bounds__(C::NT, path_split(PATH) ? 2 : 4) void newton_sym_kernel(GemmLaunch g) {
  sym_product<C, PATH, false, kPersistSym<C>, false>(g);
}

// The product's main loop on either path: fp32 (C = P^T Q, P [K][M] and
// Q [K][N]) or split (C = A B^T with A = P [M][K], or with PCOLS P = A^T
// [K][M]; B = Q [N][K], or with QCOLS Q = B^T [K][N]).
// Root products with a second affine term (the Chebyshev recurrence's
// B_(k+2)), one tile per workgroup.
template <class C, int PATH>
__global__ __launch_bounds__(C::NT, path_split(PATH) ? 2 : 4) void sym_d2_kernel(GemmLaunch g) {
  sym_product<C, PATH>(g);
}

template <class C, int PATH, bool PCOLS, bool QCOLS>
__device__ __forceinline__ void full_mainloop(const GemmProblem& pb, int f, int m0, int n0,
                                              floatx16 (&acc)[C::FM][C::FN], float* lds) {
  const float* P = pb.P + (size_t)f * pb.sP;
  const float* Q = pb.Q + (size_t)f * pb.sQ;
  if constexpr (PATH == kPathSplitH) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int ea = f16_exp(pb.mP[f]), eb = f16_exp(pb.mQ[f]);
    mainloop_x6<C, PCOLS, QCOLS, -1, true>(P, PCOLS ? pb.M : pb.K, Q, QCOLS ? pb.N : pb.K, pb.K,
                                           m0, n0, wave % C::WM, wave / C::WM, acc, lds, ea, eb);
    unscale_acc<C>(acc, -(ea + eb));
  } else if constexpr (PATH == kPathSplit) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    mainloop_x6<C, PCOLS, QCOLS>(P, PCOLS ? pb.M : pb.K, Q, QCOLS ? pb.N : pb.K, pb.K, m0, n0,
                                 wave % C::WM, wave / C::WM, acc, lds);
  } else {
    mainloop<C>(P, Q, pb.M, pb.N, pb.K, m0, n0, acc, lds);
  }
}

// A giant step of the Chebyshev sum: a symmetric product whose epilogue has
// the two extra terms (Ahat and T_2 with per-factor weights).
template <class C, int PATH>
__global__ __launch_bounds__(C::NT, path_split(PATH) ? 2 : 4) void cheb_sym_kernel(GemmLaunch g) {
  sym_product<C, PATH, true>(g);
}

// Plain product, every tile, C = acc (first apply product).
template <class C, int PATH, bool PCOLS, bool QCOLS>
__global__ __launch_bounds__(C::NT) void apply_left_kernel(GemmLaunch g) {
  __shared__ float lds[lds_floats<C, PATH>()];
  const GemmProblem& pb = g.p[blockIdx.y];
  const int TM = pb.M / C::BM, TN = pb.N / C::BN;
  const int ntile = TM * TN;
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  if (logical >= ntile * pb.batch) return;
  const int f = logical / ntile;
  const int tile = logical - f * ntile;
  const int m0 = (tile / TN) * C::BM, n0 = (tile % TN) * C::BN;
  floatx16 acc[C::FM][C::FN];
  full_mainloop<C, PATH, PCOLS, QCOLS>(pb, f, m0, n0, acc, lds);
  float* Cb = pb.C + (size_t)f * pb.sC;
  float mx = 0.f;
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j) {
      const int col = frag_col<C>(n0, j);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        Cb[(size_t)frag_row<C>(m0, i, r) * pb.N + col] = acc[i][j][r];
        if constexpr (path_f16(PATH)) mx = fmaxf(mx, fabsf(acc[i][j][r]));
      }
    }
  if constexpr (path_f16(PATH))
    if (pb.mC != nullptr) raise_max(pb.mC + f, mx, pb.ver);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// fp32 -> bfloat16, round to nearest, ties to even (NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// The parameter update of one tile on the split paths: the parameters of a
// batch of fragments are all loaded before any of them is updated and
// stored. A store to the parameter array holds back every later load from it
// (the compiler must assume they alias), so each batch costs one memory round
// trip, where one per fragment had stalled the workgroup eight times on the
// 256-tiles. BF16: parameters stored as bfloat16 (updated in fp32, rounded
// to nearest even).
template <class C, bool BF16>
__device__ __forceinline__ void update_batched(const floatx16 (&acc)[C::FM][C::FN],
                                               const BlockMeta& bm, const MatMeta& mm, float lr,
                                               int m0, int n0) {
  typedef typename std::conditional<BF16, uint16_t, float>::type P;
  P* w = reinterpret_cast<P*>(mm.param) + (size_t)bm.r0 * mm.ld + bm.c0;
  constexpr int NF = C::FM * C::FN;
  const int lane = threadIdx.x & 63;
  const int wm = __builtin_amdgcn_readfirstlane((threadIdx.x >> 6) % C::WM);
  const int wn = __builtin_amdgcn_readfirstlane((threadIdx.x >> 6) / C::WM);
  const int ld = (int)mm.ld;  // <= 2^26 (checked at init): 31 ld + col fits in 32 bits
  // The parameters of the next fragment are loaded before this fragment's
  // stores (the stores may alias them as far as the compiler knows, so loads
  // written after a store stay behind it, and the wait for them would cover
  // the stores before them). Each fragment's rows start at a pointer common
  // to the wave and its elements sit at 32-bit offsets under 32 rows, so the
  // two fragments in flight hold no 64-bit addresses per element.
  float wv[2][16];
#pragma unroll
  for (int q = 0; q <= NF; ++q) {
    if (q < NF) {
      const int i = q / C::FN, j = q % C::FN;
      const int r0 = m0 + wm * 32 * C::FM + i * 32;  // the fragment's first row (uniform)
      const int col = n0 + wn * 32 * C::FN + j * 32 + (lane & 31);
      const P* wf = w + (size_t)r0 * ld;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int rl = (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
        float v = 0.f;
        if (col < bm.n && r0 + rl < bm.m) {
          const P x = wf[(uint32_t)(rl * ld + col)];
          if constexpr (BF16)
            v = bf16_to_f32(x);
          else
            v = x;
        }
        wv[q & 1][r] = v;
      }
    }
    if (q > 0) {
      const int i = (q - 1) / C::FN, j = (q - 1) % C::FN;
      const int r0 = m0 + wm * 32 * C::FM + i * 32;
      const int col = n0 + wn * 32 * C::FN + j * 32 + (lane & 31);
      P* wf = w + (size_t)r0 * ld;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int rl = (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
        if (col < bm.n && r0 + rl < bm.m) {
          const float v = wv[(q - 1) & 1][r] - lr * acc[i][j][r];
          if constexpr (BF16)
            wf[(uint32_t)(rl * ld + col)] = f32_to_bf16(v);
          else
            wf[(uint32_t)(rl * ld + col)] = v;
        }
      }
    }
  }
}

// Second apply product with the parameter update in the epilogue:
// W[r0 + row][c0 + col] -= lr * U[row][col] on the block's real extent.
template <class C, int PATH>
__global__ __launch_bounds__(C::NT, path_split(PATH) ? 2 : 4) void apply_update_kernel(GemmLaunch g, UpdateArgs u) {
  __shared__ float lds[lds_floats<C, PATH>()];
  const GemmProblem& pb = g.p[0];
  const int TM = pb.M / C::BM, TN = pb.N / C::BN;
  const int ntile = TM * TN;
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  if (logical >= ntile * pb.batch) return;
  const int f = logical / ntile;
  const int tile = logical - f * ntile;
  const int m0 = (tile / TN) * C::BM, n0 = (tile % TN) * C::BN;
  floatx16 acc[C::FM][C::FN];
  full_mainloop<C, PATH, false, false>(pb, f, m0, n0, acc, lds);
  if (u.out_packed != nullptr) {
    float* Ub = u.out_packed + (size_t)f * pb.M * pb.N;
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
      for (int j = 0; j < C::FN; ++j) {
        const int col = frag_col<C>(n0, j);
#pragma unroll
        for (int r = 0; r < 16; ++r) Ub[(size_t)frag_row<C>(m0, i, r) * pb.N + col] = acc[i][j][r];
      }
    return;
  }
  const BlockMeta bm = u.blocks[f];
  const MatMeta mm = u.mats[bm.mat];
  const float lr = u.lr;
  if constexpr (path_split(PATH)) {
    if (u.param_bf16)
      update_batched<C, true>(acc, bm, mm, u.lr, m0, n0);
    else
      update_batched<C, false>(acc, bm, mm, u.lr, m0, n0);
    return;
  }
  // fp32 MFMA path (four waves per SIMD, fewer free registers): per fragment,
  // four parameters at a time are loaded, then updated and stored.
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j) {
      const int col = frag_col<C>(n0, j);
      if (col >= bm.n) continue;
      const size_t base = (size_t)bm.r0 * mm.ld + bm.c0 + col;
      constexpr int HOIST = 4;  // registers per batch
      if (u.param_bf16) {
        uint16_t* w = reinterpret_cast<uint16_t*>(mm.param) + base;
#pragma unroll
        for (int r0 = 0; r0 < 16; r0 += HOIST) {
          uint16_t wv[HOIST];
#pragma unroll
          for (int r = 0; r < HOIST; ++r) {
            const int row = frag_row<C>(m0, i, r0 + r);
            wv[r] = row < bm.m ? w[(size_t)row * mm.ld] : (uint16_t)0;
          }
#pragma unroll
          for (int r = 0; r < HOIST; ++r) {
            const int row = frag_row<C>(m0, i, r0 + r);
            if (row < bm.m)
              w[(size_t)row * mm.ld] = f32_to_bf16(bf16_to_f32(wv[r]) - lr * acc[i][j][r0 + r]);
          }
        }
      } else {
        float* w = reinterpret_cast<float*>(mm.param) + base;
#pragma unroll
        for (int r0 = 0; r0 < 16; r0 += HOIST) {
          float wv[HOIST];
#pragma unroll
          for (int r = 0; r < HOIST; ++r) {
            const int row = frag_row<C>(m0, i, r0 + r);
            wv[r] = row < bm.m ? w[(size_t)row * mm.ld] : 0.f;
          }
#pragma unroll
          for (int r = 0; r < HOIST; ++r) {
            const int row = frag_row<C>(m0, i, r0 + r);
            if (row < bm.m) w[(size_t)row * mm.ld] = wv[r] - lr * acc[i][j][r0 + r];
          }
        }
      }
    }
}

// ---------------------------------------------------------------------------
// Pack / unpack: 64 x 64 tiles of a block, 256 threads, 16-byte accesses.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float4 load4(const void* base, int64_t off, int bf16) {
  if (bf16) {
    const uint2 h = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(base) + off);
    return make_float4(__uint_as_float(h.x << 16), __uint_as_float(h.x & 0xffff0000u),
                       __uint_as_float(h.y << 16), __uint_as_float(h.y & 0xffff0000u));
  }
  return *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(base) + off);
}
__device__ __forceinline__ float load1(const void* base, int64_t off, int bf16) {
  if (bf16) return bf16_to_f32(reinterpret_cast<const uint16_t*>(base)[off]);
  return reinterpret_cast<const float*>(base)[off];
}

__device__ __forceinline__ uint2 bf16_bits4(float4 v) {
  // v holds bf16 values widened exactly: their bits are the upper halves
  return make_uint2((__float_as_uint(v.x) >> 16) | (__float_as_uint(v.y) & 0xffff0000u),
                    (__float_as_uint(v.z) >> 16) | (__float_as_uint(v.w) & 0xffff0000u));
}

__global__ __launch_bounds__(256) void pack_kernel(const BlockMeta* __restrict__ blocks,
                                                   const MatMeta* __restrict__ mats, int br, int bc,
                                                   int bf16, float* __restrict__ Gp,
                                                   float* __restrict__ GpT, float* __restrict__ Mom,
                                                   float momentum, uint16_t* __restrict__ GpH,
                                                   uint16_t* __restrict__ GpTH, MaxOut mo) {
  __shared__ float tile[64][65];
  float mg = 0.f, mmom = 0.f;  // largest |value| written to Gp and Mom
  const int b = blockIdx.y;
  const BlockMeta bm = blocks[b];
  const MatMeta mm = mats[bm.mat];
  const int tcn = (bc + 63) / 64;
  const int rr0 = (blockIdx.x / tcn) * 64, cc0 = (blockIdx.x % tcn) * 64;
  const int tid = threadIdx.x;
  // 4-element vector loads need ld % 4 == 0 and a 4-element-aligned base
  const bool vec = (mm.ld & 3) == 0 &&
                   (reinterpret_cast<uintptr_t>(mm.grad) & (bf16 ? 7u : 15u)) == 0;
  // All four rows' loads (gradient, momentum) are issued before the first
  // store: the compiler cannot tell the gradient from the outputs, so loads
  // written after a store stay behind it, and a wait for them would also wait
  // for the stores before them.
  float4 v[4], mv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = tid / 16 + 16 * i;
    const int c = (tid % 16) * 4;
    const int pr = rr0 + row, pc = cc0 + c;  // position inside the packed block
    v[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (pr < bm.m && pc < bm.n) {
      const int64_t off = (int64_t)(bm.r0 + pr) * mm.ld + bm.c0 + pc;
      if (vec && pc + 3 < bm.n) {
        v[i] = load4(mm.grad, off, bf16);
      } else {
        v[i].x = load1(mm.grad, off, bf16);
        if (pc + 1 < bm.n) v[i].y = load1(mm.grad, off + 1, bf16);
        if (pc + 2 < bm.n) v[i].z = load1(mm.grad, off + 2, bf16);
        if (pc + 3 < bm.n) v[i].w = load1(mm.grad, off + 3, bf16);
      }
    }
    if (Mom != nullptr && pr < br && pc < bc)
      mv[i] = *reinterpret_cast<const float4*>(Mom + ((size_t)b * br + pr) * bc + pc);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = tid / 16 + 16 * i;
    const int c = (tid % 16) * 4;
    const int pr = rr0 + row, pc = cc0 + c;
    if (pr < br && pc < bc) {
      const size_t o = ((size_t)b * br + pr) * bc + pc;
      *reinterpret_cast<float4*>(Gp + o) = v[i];
      mg = fmaxf(mg, fmaxf(fmaxf(fabsf(v[i].x), fabsf(v[i].y)), fmaxf(fabsf(v[i].z), fabsf(v[i].w))));
      if (GpH != nullptr) *reinterpret_cast<uint2*>(GpH + o) = bf16_bits4(v[i]);
      if (Mom != nullptr) {  // momentum folded in before preconditioning
        float4 m = mv[i];
        m.x = momentum * m.x + v[i].x;
        m.y = momentum * m.y + v[i].y;
        m.z = momentum * m.z + v[i].z;
        m.w = momentum * m.w + v[i].w;
        *reinterpret_cast<float4*>(Mom + o) = m;
        mmom = fmaxf(mmom, fmaxf(fmaxf(fabsf(m.x), fabsf(m.y)), fmaxf(fabsf(m.z), fabsf(m.w))));
      }
    }
    tile[row][c] = v[i].x;
    tile[row][c + 1] = v[i].y;
    tile[row][c + 2] = v[i].z;
    tile[row][c + 3] = v[i].w;
  }
  // one atomic per workgroup and word (a block's 64 x 64 tiles are many
  // workgroups raising the same word)
  if (mo.a != nullptr || mo.b != nullptr)
    raise_max2_wg<256>(mo.a != nullptr ? mo.a + b : nullptr, mg,
                       mo.b != nullptr ? mo.b + b : nullptr, mmom, mo.ver);
  // no transpose wanted (the split products read the packed block by rows
  // and by columns): done (uniform over the workgroup)
  if (GpT == nullptr && GpTH == nullptr) return;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int tc = tid / 16 + 16 * i;  // column of the tile = row of GpT
    const int r = (tid % 16) * 4;
    if (cc0 + tc < bc && rr0 + r < br) {
      const float4 v = make_float4(tile[r][tc], tile[r + 1][tc], tile[r + 2][tc], tile[r + 3][tc]);
      const size_t o = ((size_t)b * bc + cc0 + tc) * br + rr0 + r;
      if (GpTH != nullptr)
        *reinterpret_cast<uint2*>(GpTH + o) = bf16_bits4(v);
      else
        *reinterpret_cast<float4*>(GpT + o) = v;
    }
  }
}

__global__ __launch_bounds__(256) void unpack_kernel(const BlockMeta* __restrict__ blocks,
                                                     const MatMeta* __restrict__ dst, int br, int bc,
                                                     const float* __restrict__ Gp) {
  const int b = blockIdx.y;
  const BlockMeta bm = blocks[b];
  const MatMeta mm = dst[bm.mat];
  const int tcn = (bc + 63) / 64;
  const int rr0 = (blockIdx.x / tcn) * 64, cc0 = (blockIdx.x % tcn) * 64;
  const int tid = threadIdx.x;
  float* out = reinterpret_cast<float*>(mm.param);
  const bool vec = (mm.ld & 3) == 0 && (reinterpret_cast<uintptr_t>(out) & 15u) == 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int pr = rr0 + tid / 16 + 16 * i;
    const int pc = cc0 + (tid % 16) * 4;
    if (pr >= bm.m || pc >= bm.n) continue;
    const float4 v = *reinterpret_cast<const float4*>(Gp + ((size_t)b * br + pr) * bc + pc);
    const int64_t off = (int64_t)(bm.r0 + pr) * mm.ld + bm.c0 + pc;
    if (vec && pc + 3 < bm.n) {
      *reinterpret_cast<float4*>(out + off) = v;
    } else {
      out[off] = v.x;
      if (pc + 1 < bm.n) out[off + 1] = v.y;
      if (pc + 2 < bm.n) out[off + 2] = v.z;
      if (pc + 3 < bm.n) out[off + 3] = v.w;
    }
  }
}

// L = R = eps * I over the whole padded factor (left factors, then right).
__global__ __launch_bounds__(256) void init_state_kernel(float* LR, int64_t nelemL, int nl,
                                                         int64_t nelemR, int nr, float eps) {
  const int64_t total = nelemL + nelemR;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * blockDim.x) {
    const bool left = e < nelemL;
    const int n = left ? nl : nr;
    const int64_t w = (left ? e : e - nelemL) % ((int64_t)n * n);
    LR[e] = (w / n == w % n) ? eps : 0.f;
  }
}

__device__ __forceinline__ const float* factor_ptr(const float* base, const FactorSet& fs, int f,
                                                   int& n) {
  const int g = f / fs.B, i = f - g * fs.B;
  n = fs.side[g];
  return base + fs.off[g] + (int64_t)i * n * n;
}

// ---------------------------------------------------------------------------
// Norm scaling: one workgroup per factor, fixed-order reductions.
//   mode 0: s = ||A||_F
//   mode 1: s = min(||A||_F, ||A||_inf) * 2 / (p + 1)
//   mode 3: mode 2's s; the coupled Newton iteration then scales itself
//           every step (newton_check_kernel), starting from an estimate of the
//           spectrum's bottom made here
//   mode 2: s = lam / 2, lam the power-iteration estimate ||A v_k|| of the
//           largest eigenvalue after kPowerIters (8) products from
//           v_0 = 1 / sqrt(n). For symmetric A the ratios ||A^(j+1) v|| /
//           ||A^j v|| never decrease, so lam >= lam_max |c_1|^(1/8) with c_1
//           the component of v_0 on the top eigenvector: the spectrum of A / s
//           stays inside the iteration's convergence region (0, p + 1)
//           unless |c_1| < (2 / (p + 1))^8 (6.6e-4 for p = 4). lam = 0 falls
//           back to mode 1. The Chebyshev interval takes kPowerItersCheb (16).
// Only the real extent of a factor enters.
// ---------------------------------------------------------------------------
__device__ __forceinline__ double block_sum(double v, double* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  return red[0] + red[1] + red[2] + red[3];
}

// sym_matvec for a factor of at most 256 columns (a single column chunk,
// which would leave three waves idle): each wave runs down a quarter of the
// rows (a lane: four consecutive columns, the loads of eight rows issued
// together), and wave 0 adds the four partial columns in wave order from
// part ([2][4][64] float4 in LDS). Every thread of the workgroup calls it.
template <bool TWO>
__device__ __forceinline__ void sym_matvec_small(const float* __restrict__ Af, int n, int nr,
                                                 const float* x, const float* xu, float* y,
                                                 float* yu, float4* part) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = lane * 4;
  const int rq = (nr + 3) / 4;
  const int r0 = min(nr, wave * rq), r1 = min(nr, r0 + rq);
  float4 s = make_float4(0.f, 0.f, 0.f, 0.f), t = make_float4(0.f, 0.f, 0.f, 0.f);
  if (j + 3 < nr) {
    const float* col = Af + j;
    int r = r0;
    for (; r + 8 <= r1; r += 8) {
      float4 a[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) a[u] = *reinterpret_cast<const float4*>(col + (int64_t)(r + u) * n);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float xr = x[r + u];
        s.x += a[u].x * xr;
        s.y += a[u].y * xr;
        s.z += a[u].z * xr;
        s.w += a[u].w * xr;
        if constexpr (TWO) {
          const float ur = xu[r + u];
          t.x += a[u].x * ur;
          t.y += a[u].y * ur;
          t.z += a[u].z * ur;
          t.w += a[u].w * ur;
        }
      }
    }
    for (; r < r1; ++r) {
      const float4 a = *reinterpret_cast<const float4*>(col + (int64_t)r * n);
      const float xr = x[r];
      s.x += a.x * xr;
      s.y += a.y * xr;
      s.z += a.z * xr;
      s.w += a.w * xr;
      if constexpr (TWO) {
        const float ur = xu[r];
        t.x += a.x * ur;
        t.y += a.y * ur;
        t.z += a.z * ur;
        t.w += a.w * ur;
      }
    }
  } else if (j < nr) {
    // the ragged last columns one by one
    for (int r = r0; r < r1; ++r) {
      const float* a = Af + (int64_t)r * n + j;
      const float xr = x[r], ur = TWO ? xu[r] : 0.f;
      s.x += a[0] * xr;
      if (j + 1 < nr) s.y += a[1] * xr;
      if (j + 2 < nr) s.z += a[2] * xr;
      if constexpr (TWO) {
        t.x += a[0] * ur;
        if (j + 1 < nr) t.y += a[1] * ur;
        if (j + 2 < nr) t.z += a[2] * ur;
      }
    }
  }
  part[wave * 64 + lane] = s;
  if constexpr (TWO) part[256 + wave * 64 + lane] = t;
  __syncthreads();
  if (wave == 0 && j < nr) {
    const float4 p0 = part[lane], p1 = part[64 + lane], p2 = part[128 + lane], p3 = part[192 + lane];
    const float sv[4] = {(p0.x + p1.x) + (p2.x + p3.x), (p0.y + p1.y) + (p2.y + p3.y),
                         (p0.z + p1.z) + (p2.z + p3.z), (p0.w + p1.w) + (p2.w + p3.w)};
    float tv[4] = {0.f, 0.f, 0.f, 0.f};
    if constexpr (TWO) {
      const float4 q0 = part[256 + lane], q1 = part[320 + lane], q2 = part[384 + lane],
                   q3 = part[448 + lane];
      tv[0] = (q0.x + q1.x) + (q2.x + q3.x);
      tv[1] = (q0.y + q1.y) + (q2.y + q3.y);
      tv[2] = (q0.z + q1.z) + (q2.z + q3.z);
      tv[3] = (q0.w + q1.w) + (q2.w + q3.w);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (j + k < nr) {
        y[j + k] = sv[k];
        if (TWO) yu[j + k] = tv[k];
      }
    }
  }
}

// y = A x and, with TWO, yu = A xu for a symmetric factor A (row stride n,
// real extent nr; x, xu, y, yu in LDS). Wave w owns the 256-column chunks
// w, w + 4, ... (four consecutive columns a lane) and runs down every row, so
// y_j = sum_r A_rj x_r, which is (A x)_j since A is symmetric, needs no sum
// across lanes or waves: one 16-byte load and four FMAs per row and vector.
// Four partial sums per column (rows r mod 4) keep the fp32 chains short.
template <bool TWO>
__device__ __forceinline__ void sym_matvec(const float* __restrict__ Af, int n, int nr,
                                           const float* x, const float* xu, float* y, float* yu) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int c0 = wave * 256; c0 < nr; c0 += 1024) {
    const int j = c0 + lane * 4;
    float4 s[4], t[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      s[q] = make_float4(0.f, 0.f, 0.f, 0.f);
      t[q] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    if (j + 3 < nr) {
      const float* col = Af + j;
      const int r4 = nr & ~3;
      for (int r = 0; r < r4; r += 4) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 a = *reinterpret_cast<const float4*>(col + (int64_t)(r + q) * n);
          const float xr = x[r + q];
          s[q].x += a.x * xr;
          s[q].y += a.y * xr;
          s[q].z += a.z * xr;
          s[q].w += a.w * xr;
          if constexpr (TWO) {
            const float ur = xu[r + q];
            t[q].x += a.x * ur;
            t[q].y += a.y * ur;
            t[q].z += a.z * ur;
            t[q].w += a.w * ur;
          }
        }
      }
      for (int r = r4; r < nr; ++r) {
        const float4 a = *reinterpret_cast<const float4*>(col + (int64_t)r * n);
        const float xr = x[r];
        s[0].x += a.x * xr;
        s[0].y += a.y * xr;
        s[0].z += a.z * xr;
        s[0].w += a.w * xr;
        if constexpr (TWO) {
          const float ur = xu[r];
          t[0].x += a.x * ur;
          t[0].y += a.y * ur;
          t[0].z += a.z * ur;
          t[0].w += a.w * ur;
        }
      }
    } else if (j < nr) {
      // the ragged end of the last chunk: the columns below nr one by one
      for (int r = 0; r < nr; ++r) {
        const float* a = Af + (int64_t)r * n + j;
        const float xr = x[r], ur = TWO ? xu[r] : 0.f;
        s[0].x += a[0] * xr;
        if (j + 1 < nr) s[0].y += a[1] * xr;
        if (j + 2 < nr) s[0].z += a[2] * xr;
        if constexpr (TWO) {
          t[0].x += a[0] * ur;
          if (j + 1 < nr) t[0].y += a[1] * ur;
          if (j + 2 < nr) t[0].z += a[2] * ur;
        }
      }
    }
    if (j < nr) {
      const float4 sv = make_float4((s[0].x + s[1].x) + (s[2].x + s[3].x),
                                    (s[0].y + s[1].y) + (s[2].y + s[3].y),
                                    (s[0].z + s[1].z) + (s[2].z + s[3].z),
                                    (s[0].w + s[1].w) + (s[2].w + s[3].w));
      const float4 tv = make_float4((t[0].x + t[1].x) + (t[2].x + t[3].x),
                                    (t[0].y + t[1].y) + (t[2].y + t[3].y),
                                    (t[0].z + t[1].z) + (t[2].z + t[3].z),
                                    (t[0].w + t[1].w) + (t[2].w + t[3].w));
      y[j] = sv.x;
      if (TWO) yu[j] = tv.x;
      if (j + 1 < nr) {
        y[j + 1] = sv.y;
        if (TWO) yu[j + 1] = tv.y;
      }
      if (j + 2 < nr) {
        y[j + 2] = sv.z;
        if (TWO) yu[j + 2] = tv.z;
      }
      if (j + 3 < nr) {
        y[j + 3] = sv.w;
        if (TWO) yu[j + 3] = tv.w;
      }
    }
  }
}

// Scalar map of one coupled Newton iteration on an eigenvalue m of M scaled
// by mu: f(mu m) = mu m ((p + 1 - mu m) / p)^p.
__device__ __forceinline__ double newton_map(double m, int p, double mu) {
  if (p == 4) {
    // the same value without a division (dividing by 4 is exact): the
    // bisection of the scale runs 80 of these in a dependent chain
    const double y = mu * m, t = (5.0 - y) * 0.25;
    return y * (((t * t) * t) * t);
  }
  const double y = mu * m, t = (p + 1 - y) / p;
  double tp = 1.0;
  for (int i = 0; i < p; ++i) tp *= t;
  return y * tp;
}

// mu in [1, 0.9 (p + 1)] with f(mu a) = f(mu): bisection, kBalanceSteps steps.
__device__ double newton_balance(double a, int p) {
  double lo = 1.0, hi = 0.9 * (p + 1);
  if (newton_map(a, p, hi) < newton_map(1.0, p, hi)) return hi;
  for (int i = 0; i < kBalanceSteps; ++i) {
    const double mid = 0.5 * (lo + hi);
    if (newton_map(a, p, mid) < newton_map(1.0, p, mid))
      lo = mid;
    else
      hi = mid;
  }
  return lo;
}

// Epilogue quadruples (alpha, beta, beta2, gamma) of one iteration at scale
// mu: T = ((p + 1) I - mu M) / p,
//   T^2   = (mu^2 M M - 2 (p + 1) mu M + (p + 1)^2 I) / p^2
//   X' = mu^(1/p) X T = ((p + 1) mu^(1/p) X - mu^(1 + 1/p) X M) / p
//   M' = T^p (mu M).
__device__ void write_newton_coefs(float* rec, double mu, int p) {
  const double pp = (double)p * p, q = p + 1.0, mr = pow(mu, 1.0 / p);
  rec[kCoefT2 + 0] = (float)(mu * mu / pp);
  rec[kCoefT2 + 1] = (float)(-2.0 * q * mu / pp);
  rec[kCoefT2 + 2] = 0.f;
  rec[kCoefT2 + 3] = (float)(q * q / pp);
  rec[kCoefXT + 0] = (float)(-mu * mr / p);
  rec[kCoefXT + 1] = (float)(q * mr / p);
  rec[kCoefXT + 2] = 0.f;
  rec[kCoefXT + 3] = 0.f;
  rec[kCoefM + 0] = (float)mu;
  rec[kCoefM + 1] = 0.f;
  rec[kCoefM + 2] = 0.f;
  rec[kCoefM + 3] = 0.f;
}

__global__ __launch_bounds__(256) void norms_kernel(const float* __restrict__ A, FactorSet fs,
                                                    NewtonCtl c) {
  __shared__ double red[4];
  __shared__ double red_inf[4];
  __shared__ double red_min[4];
  __shared__ float4 part[2 * 4 * 64];  // partial products of factors of <= 256 columns
  // four vectors of the largest side (dynamic LDS, sized at launch): the top
  // power iteration's vector and product, the bottom one's (scale mode 3)
  extern __shared__ float4 vecs4[];  // float4: 16-byte aligned for the vector loads
  float* vecs = reinterpret_cast<float*>(vecs4);
  const int ms = (fs.max_side() + 3) & ~3;
  float* v = vecs;
  float* w = vecs + ms;
  float* u = vecs + 2 * ms;
  float* wu = vecs + 3 * ms;
  const int f = blockIdx.x;
  int n;
  const float* Af = factor_ptr(A, fs, f, n);
  const int nr = fs.nreal[f];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const bool db = c.solver == kNewtonDB;
  const bool cheb = c.solver == kChebyshev;
  const bool power = c.scale_mode >= 2 || cheb;
  const bool scaled = c.scale_mode == 3 && c.solver == kCoupledNewton;
  const float inv0 = (float)(1.0 / sqrt((double)nr));
  // pass 1, by columns as in sym_matvec: squares, absolute column sums (the
  // absolute row sums: A is symmetric), w = A 1 (the column sums) and, in
  // mode 3, wu = A u_0 with u_0 = (1, -1, 1, ...) / sqrt(n); then the smallest
  // diagonal entry
  double sq = 0.0, rowmax = 0.0, dmin = INFINITY;
  for (int c0 = wave * 256; c0 < nr; c0 += 1024) {
    const int j = c0 + lane * 4;
    if (j >= nr) continue;
    double as[4] = {0.0, 0.0, 0.0, 0.0}, rs[4] = {0.0, 0.0, 0.0, 0.0}, alt[4] = {0.0, 0.0, 0.0, 0.0};
    for (int r = 0; r < nr; ++r) {
      const float* a = Af + (int64_t)r * n + j;
      float xs[4];
      if (j + 3 < nr) {
        const float4 x4 = *reinterpret_cast<const float4*>(a);
        xs[0] = x4.x;
        xs[1] = x4.y;
        xs[2] = x4.z;
        xs[3] = x4.w;
      } else {
        xs[0] = a[0];
        xs[1] = j + 1 < nr ? a[1] : 0.f;
        xs[2] = j + 2 < nr ? a[2] : 0.f;
        xs[3] = 0.f;
      }
      const double sgn = (r & 1) ? -1.0 : 1.0;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const double x = xs[k];
        as[k] += fabs(x);
        rs[k] += x;
        alt[k] += sgn * x;
        sq += x * x;
      }
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (j + k >= nr) break;
      rowmax = fmax(rowmax, as[k]);
      if (power) w[j + k] = (float)rs[k];
      if (scaled) wu[j + k] = (float)(alt[k] * inv0);
    }
  }
  for (int r = threadIdx.x; r < nr; r += 256) dmin = fmin(dmin, (double)Af[(int64_t)r * n + r]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    rowmax = fmax(rowmax, __shfl_xor(rowmax, o));
    dmin = fmin(dmin, __shfl_xor(dmin, o));
  }
  if (scaled)
    for (int r = threadIdx.x; r < nr; r += 256) u[r] = (r & 1) ? -inv0 : inv0;
  if (lane == 0) {
    red_inf[wave] = rowmax;
    red_min[wave] = dmin;
  }
  const double fro = sqrt(block_sum(sq, red));
  const double inf = fmax(fmax(red_inf[0], red_inf[1]), fmax(red_inf[2], red_inf[3]));
  const double bound = fmin(fro, inf);
  // spectral target: Newton converges on (0, p + 1), the Denman-Beavers pair on (0, 2)
  const double mode1 = db ? 1.0 : 2.0 / (c.p + 1);
  double s = c.scale_mode == 0 ? fro : bound * mode1;
  double lam = 0.0, q = INFINITY;
  if (power) {
    // Top power iteration from v_0 = 1 / sqrt(n); in mode 3 the bottom one
    // runs beside it on lam_j I - A from u_0 (one pass over A per step serves
    // both): q_j = u_j^T A u_j, u_(j+1) = normalised lam_j u_j - A u_j.
    const int steps = cheb ? kPowerItersCheb : kPowerIters;
    for (int it = 0; it < steps; ++it) {
      if (it > 0) {
        if (nr <= 256) {
          if (scaled)
            sym_matvec_small<true>(Af, n, nr, v, u, w, wu, part);
          else
            sym_matvec_small<false>(Af, n, nr, v, nullptr, w, nullptr, part);
        } else if (scaled) {
          sym_matvec<true>(Af, n, nr, v, u, w, wu);
        } else {
          sym_matvec<false>(Af, n, nr, v, nullptr, w, nullptr);
        }
      }
      __syncthreads();
      double nn = 0.0;
      for (int r = threadIdx.x; r < nr; r += 256) nn += (double)w[r] * w[r];
      // v_0 = 1 / sqrt(nr) is folded in: the first product is the row sum
      nn = block_sum(nn, red) / (it == 0 ? (double)nr : 1.0);
      lam = sqrt(nn);
      if (scaled) {
        double qq = 0.0;
        for (int r = threadIdx.x; r < nr; r += 256) qq += (double)u[r] * wu[r];
        q = block_sum(qq, red);
        double nu = 0.0;
        for (int r = threadIdx.x; r < nr; r += 256) {
          const float y = (float)(lam * u[r] - wu[r]);
          wu[r] = y;
          nu += (double)y * y;
        }
        nu = block_sum(nu, red);
        const float invu = nu > 0.0 ? (float)(1.0 / sqrt(nu)) : 0.f;
        if (nu > 0.0 && lam > 0.0)
          for (int r = threadIdx.x; r < nr; r += 256) u[r] = wu[r] * invu;
      }
      const float inv = lam > 0.0 ? (float)(1.0 / (lam * (it == 0 ? sqrt((double)nr) : 1.0))) : 0.f;
      for (int r = threadIdx.x; r < nr; r += 256) v[r] = w[r] * inv;
      __syncthreads();
      if (lam == 0.0) break;
    }
    s = lam > 0.0 ? lam * (db ? 1.0 : 0.5) : bound * mode1;
    // Chebyshev needs an upper bound of the spectrum: lam >= 0.55 lam_max
    // unless v_0 is almost orthogonal to the top eigenvector; the norm bound
    // holds always
    if (cheb) s = lam > 0.0 ? fmin(lam / 0.55, bound) : bound;
  }
  // the bottom estimate: both the smallest diagonal entry and q are Rayleigh
  // quotients, never below the smallest eigenvalue
  const double est = fmin(fmin(fmin(red_min[0], red_min[1]), fmin(red_min[2], red_min[3])), q);
  if (threadIdx.x == 0) {
    const bool ok = s > 0.0 && isfinite(s) && isfinite(fro);
    c.scale[f] = (float)s;
    c.cfac[f] = ok ? (float)pow(s, -1.0 / c.p) : 0.f;
    c.status[f] = ok ? 0 : 3;
    c.final_iter[f] = 0;
    c.rprev[f] = INFINITY;
    if (scaled) {
      // the estimate for M after the first, unscaled iteration: f(a_0) for the
      // bottom, f(b_0) for the top (b_0 = lam / s = 2, or (p + 1) / 2 when the
      // norm bound was used)
      const double b0 = lam > 0.0 ? 2.0 : 0.5 * (c.p + 1);
      const double a0 = ok ? fmax(est, 0.0) / s : 0.0;
      c.lo[f] = (float)fmin(newton_map(a0, c.p, 1.0), newton_map(b0, c.p, 1.0));
      float* rec = c.coef + (size_t)f * kCoefRecord;
      write_newton_coefs(rec, 1.0, c.p);
      rec[kCoefPrevMu] = 1.f;
    }
  }
}

// Coupled Newton: M0 = A / s (identity on the padded part) and
// X1 = s^(-1/p) ((p + 1) I - M0) / p. Denman-Beavers: Y0 = A / s (into M0) and Z0 = I
// (into X1).
__global__ __launch_bounds__(256) void newton_init_kernel(const float* __restrict__ A,
                                                          float* __restrict__ M0,
                                                          float* __restrict__ X1, FactorSet fs,
                                                          NewtonCtl c, MaxOut mo) {
  const int f = blockIdx.y;
  if (c.status[f] != 0) return;
  float mm = 0.f, mx = 0.f;
  int n;
  const float* Af = factor_ptr(A, fs, f, n);
  const int64_t base = Af - A;
  const int nr = fs.nreal[f];
  const float s = c.scale[f], cf = c.cfac[f];
  const float ip = 1.f / (float)c.p, ip1 = (float)(c.p + 1) / (float)c.p;
  // four consecutive elements of one row per step (sides are multiples of
  // 32); four steps' loads are issued before their stores (a load written
  // after a store stays behind it, and the wait for it would cover the store)
  const int nn4 = n * n / 4;
  const int stride = gridDim.x * blockDim.x;
  for (int e0 = blockIdx.x * blockDim.x + threadIdx.x; e0 < nn4; e0 += 4 * stride) {
    float4 a4[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e4 = e0 + u * stride;
      if (e4 < nn4) a4[u] = *reinterpret_cast<const float4*>(Af + 4 * e4);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e4 = e0 + u * stride;
      if (e4 >= nn4) break;
      const int e = 4 * e4, r = e / n, col = e - r * n;
      const float av[4] = {a4[u].x, a4[u].y, a4[u].z, a4[u].w};
      float m[4], x[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float id = (r == col + k) ? 1.f : 0.f;
        m[k] = (r < nr && col + k < nr) ? av[k] / s : id;
        mm = fmaxf(mm, fabsf(m[k]));
        x[k] = c.solver == kNewtonDB ? id : cf * (ip1 * id - ip * m[k]);
      }
      *reinterpret_cast<float4*>(M0 + base + e) = make_float4(m[0], m[1], m[2], m[3]);
      if (c.solver != kChebyshev) {
        *reinterpret_cast<float4*>(X1 + base + e) = make_float4(x[0], x[1], x[2], x[3]);
        mx = fmaxf(mx, fmaxf(fmaxf(fabsf(x[0]), fabsf(x[1])), fmaxf(fabsf(x[2]), fabsf(x[3]))));
      }
    }
  }
  if (mo.a != nullptr || mo.b != nullptr)
    raise_max2_wg<256>(mo.a != nullptr ? mo.a + f : nullptr, mm,
                       mo.b != nullptr ? mo.b + f : nullptr, mx, mo.ver);
}

// After iteration `iter` (which produced M_{iter+1} and X_{iter+1}): residual
// and stopping rule per factor; counts the factors of each group that took
// part in the iteration and adds the algorithmic flops of its symmetric
// products (prod_before for every factor that entered, prod_after for those
// still running; n^2 (n + 1) each).
__global__ __launch_bounds__(1024) void newton_check_kernel(FactorSet fs, NewtonCtl c, int iter,
                                                            int shift, int prod_before,
                                                            int prod_after) {
  __shared__ int cnt[kMaxGroups];
  __shared__ int cnt_out[kMaxGroups];
  __shared__ int cnt_x[kMaxGroups];
  if (threadIdx.x < kMaxGroups) {
    cnt[threadIdx.x] = 0;
    cnt_out[threadIdx.x] = 0;
    cnt_x[threadIdx.x] = 0;
  }
  __syncthreads();
  const int cur = iter + shift;  // the iterate whose residual was just formed
  const int nf = fs.count();
  const bool scaled = c.scale_mode == 3 && c.solver == kCoupledNewton && c.coef != nullptr;
  for (int f = threadIdx.x; f < nf; f += blockDim.x) {
    const int g = f / fs.B;
    if (c.status[f] == kStatusFinalX) {
      // the iteration just run formed only this factor's X: it is the result
      c.status[f] = 1;
      c.final_iter[f] = cur;
      atomicAdd(&cnt_x[g], 1);
      continue;
    }
    if (c.status[f] != 0) continue;
    atomicAdd(&cnt[g], 1);
    const int nt = c.ntiles[g];
    const float* p = c.resid + (size_t)f * c.resid_stride;
    float s = 0.f;
    for (int t = 0; t < nt; ++t) s += p[t];
    const float r = sqrtf(s) / sqrtf((float)fs.nreal[f]);
    // Scale mode 3: this iterate was made with M scaled by mu (mu > 1 lifts
    // the slow small eigenvalues and may raise the residual), the previous one
    // with mu_prev; only unscaled iterates take the monotone tests, and the
    // first of them after the scaled phase is compared with nothing.
    float* rec = scaled ? c.coef + (size_t)f * kCoefRecord : nullptr;
    const float mu = scaled ? rec[kCoefM] : 1.f;
    const float mu_prev = scaled ? rec[kCoefPrevMu] : 1.f;
    const float rp = mu_prev > 1.f ? INFINITY : c.rprev[f];
    // In exact arithmetic both iterations shrink the residual every step, so a
    // growth means trouble: from a residual above kFloorGuard it is divergence,
    // below it the fp32 floor has been reached (stalled, the previous iterate
    // is kept and is as good).
    const bool monotone = c.tol > 0.f && mu == 1.f;
    int st = 0;
    if (!isfinite(r)) {
      st = 3;
    } else if (monotone && r > 1.2f * rp && rp > kFloorGuard) {
      st = 3;
    } else if (monotone && r >= rp) {
      st = 2;
    } else {
      c.rprev[f] = r;
      c.final_iter[f] = cur;
      if (c.tol > 0.f && r <= c.tol)
        st = 1;
      else if (cur >= c.max_iters)
        st = 4;
    }
    // a rejected iterate leaves final_iter at the previous (accepted) one
    c.status[f] = st;
    if (st == 0) {
      double mun = 1.0;
      if (scaled) {
        // the next scale balances the scalar map at the tracked estimate of the
        // spectrum's bottom; the estimate follows the map
        const double a = c.lo[f];
        mun = a < kScaledPhaseEnd ? newton_balance(a, c.p) : 1.0;
        c.lo[f] = (float)newton_map(a, c.p, mun);
        write_newton_coefs(rec, mun, c.p);
        rec[kCoefPrevMu] = mu;
      }
      // Coupled Newton near the fixed point: the next residual is at most
      // C sqrt(n) r^2, C = (p + 1) / (2 p). When that already meets tol, the
      // next iteration forms only X (its M would be formed only to be checked).
      if (shift == 1 && c.tol > 0.f && mu == 1.f && mun == 1.0 && cur < c.max_iters) {
        const float bound = (float)((c.p + 1) / (2.0 * c.p) * sqrt((double)fs.nreal[f]) *
                                    (double)r * r);
        if (fmaxf(bound, kRoundingFloor) <= c.tol) {
          st = kStatusFinalX;
          c.status[f] = st;
          c.rprev[f] = bound;
        }
      }
      atomicAdd(&cnt_out[g], 1);
    }
  }
  __syncthreads();
  if (threadIdx.x < fs.n_groups) c.active_count[iter * kMaxGroups + threadIdx.x] = cnt[threadIdx.x];
  if (threadIdx.x == 0) {
    double fl = 0.0;
    for (int g = 0; g < fs.n_groups; ++g) {
      const double n = fs.side[g];
      // factors that finished with an X-only iteration ran one product in it
      fl += (prod_before * (double)cnt[g] + prod_after * (double)cnt_out[g] + (double)cnt_x[g]) *
            n * n * (n + 1.0);
    }
    c.flops_acc[0] += fl;
  }
}

// Put the kept iterate into the root buffer: X_k lives in Xroot for even k
// and in Xalt for odd k; X_0 = s^(-1/p) I is never stored.
// scale = 1 (Denman-Beavers): the kept Z is multiplied by s^(-1/p), and Z_0 = I
// is stored in Xroot by the stage-2 init.
__global__ __launch_bounds__(256) void newton_final_kernel(float* __restrict__ Xroot,
                                                           const float* __restrict__ Xalt,
                                                           FactorSet fs, NewtonCtl c, int scale,
                                                           MaxOut mo) {
  const int f = blockIdx.y;
  const int k = c.final_iter[f];
  if (!scale && k > 0 && (k & 1) == 0) return;
  const bool odd = scale == 1 && (k & 1);  // scale 2: the result is in Xroot
  const bool dead = scale == 2 && c.status[f] == 3;  // no valid scale: the root is 0
  int n;
  const float* xf = factor_ptr(Xroot, fs, f, n);
  const int64_t base = xf - Xroot;
  const float cf = c.cfac[f];
  // four consecutive elements of one row per step (sides are multiples of
  // 32); four steps' loads are issued before their stores (a load written
  // after a store stays behind it, and the wait for it would cover the store)
  const int nn4 = n * n / 4;
  const int stride = gridDim.x * blockDim.x;
  const bool copy = !dead && (scale || k > 0);
  const float* src = (scale && !odd ? Xroot : Xalt) + base;
  float mx = 0.f;
  for (int e0 = blockIdx.x * blockDim.x + threadIdx.x; e0 < nn4; e0 += 4 * stride) {
    float4 x4[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e4 = e0 + u * stride;
      if (copy && e4 < nn4) x4[u] = *reinterpret_cast<const float4*>(src + 4 * e4);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e4 = e0 + u * stride;
      if (e4 >= nn4) break;
      const int e = 4 * e4, r = e / n, col = e - r * n;
      float4 x;
      if (dead) {
        x = make_float4(0.f, 0.f, 0.f, 0.f);
      } else if (copy) {
        x = x4[u];
        if (scale) {
          x.x *= cf;
          x.y *= cf;
          x.z *= cf;
          x.w *= cf;
        }
      } else {  // X_0 = s^(-1/p) I
        x = make_float4(r == col ? cf : 0.f, r == col + 1 ? cf : 0.f, r == col + 2 ? cf : 0.f,
                        r == col + 3 ? cf : 0.f);
      }
      *reinterpret_cast<float4*>(Xroot + base + e) = x;
      mx = fmaxf(mx, fmaxf(fmaxf(fabsf(x.x), fabsf(x.y)), fmaxf(fabsf(x.z), fabsf(x.w))));
    }
  }
  if (mo.a != nullptr) raise_max(mo.a + f, mx, mo.ver);
}

// ---------------------------------------------------------------------------
// Coupled Newton for factors of side <= 64 in one launch: one workgroup per
// factor runs every iteration with its iterates in LDS, the products as fp32
// FMAs (exact fp32 products, fp32 sums; no operand split). Small blocks would
// otherwise spend their step launching the per-iteration kernels, most of
// them with nothing left to do. The iteration, its scaling (mode 3), stop
// rules, final-step X-only iteration and records are those of the
// newton_sym / newton_check / newton_final chain; it starts from M_0 and X_1
// of newton_init and writes the kept iterate to Xroot (with its maximum word).
// ---------------------------------------------------------------------------
// C = alpha P Q + beta D + gamma I for n x n matrices in LDS (row stride n, n
// a multiple of 32; P symmetric, read by rows). The 4 x 4 blocks on and above
// the diagonal are computed and mirrored, so C is exactly symmetric. Returns
// this thread's share of ||C - I||_F^2 when want_resid.
__device__ __forceinline__ float small_product(float* __restrict__ C, const float* __restrict__ P,
                                               const float* __restrict__ Q,
                                               const float* __restrict__ D, float alpha,
                                               float beta, float gamma, int n, bool want_resid) {
  const int nb = n / 4;
  float rs = 0.f;
  for (int t = threadIdx.x; t < nb * nb; t += blockDim.x) {
    const int bi = t / nb, bj = t - bi * nb;
    if (bi > bj) continue;
    const int r0 = 4 * bi, c0 = 4 * bj;
    float acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;
    // the LDS loads of eight k are issued together, then their FMAs (one k
    // at a time waited on every load: 9 us per 64^3 product); n % 32 == 0
    for (int k0 = 0; k0 < n; k0 += 8) {
      f32x4 a[8], b[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        a[u] = *reinterpret_cast<const f32x4*>(P + (k0 + u) * n + r0);
        b[u] = *reinterpret_cast<const f32x4*>(Q + (k0 + u) * n + c0);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[u][i], b[u][j], acc[i][j]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row = r0 + i, col = c0 + j;
        if (row > col) continue;
        float x = alpha * acc[i][j];
        if (D != nullptr) x += beta * D[row * n + col];
        if (row == col) x += gamma;
        C[row * n + col] = x;
        C[col * n + row] = x;
        if (want_resid) {
          const float d = x - (row == col ? 1.f : 0.f);
          rs += (row == col ? 1.f : 2.f) * d * d;
        }
      }
  }
  return rs;
}

// Sum over the workgroup (256 threads), the same value in every thread.
__device__ __forceinline__ float small_sum(float v, float* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

__global__ __launch_bounds__(256) void newton_small_kernel(const float* __restrict__ Mbuf,
                                                           const float* __restrict__ Xbuf,
                                                           float* __restrict__ Xroot, FactorSet fs,
                                                           NewtonCtl c, MaxOut mo) {
  __shared__ __align__(16) float sm[6][kSmallSide * kSmallSide];
  __shared__ float red[4];
  const int f = blockIdx.x;
  int n;
  const float* mf = factor_ptr(Mbuf, fs, f, n);
  const int64_t base = mf - Mbuf;
  const int nn = n * n;
  const int p = c.p;
  const bool scaled = c.scale_mode == 3 && c.coef != nullptr;
  float* rec = scaled ? c.coef + (size_t)f * kCoefRecord : nullptr;
  // the coefficients of the next iteration (scale mode 3: the record's)
  const double pp = (double)p * p, q = p + 1.0;
  float t2a = (float)(1.0 / pp), t2b = (float)(-2.0 * q / pp), t2g = (float)(q * q / pp);
  float xa = (float)(-1.0 / p), xb = (float)(q / p), ma = 1.f, mu_prev = 1.f;
  if (scaled) {
    t2a = rec[kCoefT2 + 0];
    t2b = rec[kCoefT2 + 1];
    t2g = rec[kCoefT2 + 3];
    xa = rec[kCoefXT + 0];
    xb = rec[kCoefXT + 1];
    ma = rec[kCoefM + 0];
    mu_prev = rec[kCoefPrevMu];
  }
  int st = c.status[f], fin = c.final_iter[f];
  float rprev = c.rprev[f];
  float lo = scaled ? c.lo[f] : 0.f;
  // slots: the accepted M and X, the new ones, T^2, T^4 (for p = 6, 8, T^p
  // goes to the new-M slot and M' to T^2's)
  int iM = 0, iMn = 1, iX = 2, iXn = 3;
  float* T2 = sm[4];
  float* T4 = sm[5];
  for (int e = threadIdx.x; e < nn; e += blockDim.x) {
    sm[iM][e] = mf[e];
    sm[iXn][e] = Xbuf[base + e];  // X_1, formed by the init kernel
  }
  __syncthreads();
  const double cube = (double)n * n * (n + 1.0);
  const int per_iter = p == 4 ? 4 : 5;
  double flops = 0.0;
  for (int k = 0; k < c.max_iters && (st == 0 || st == kStatusFinalX); ++k) {
    const int cur = k + 1;
    float* M = sm[iM];
    float* X = sm[iX];
    float* Xn = sm[iXn];
    if (k > 0) small_product(Xn, X, M, X, xa, xb, 0.f, n, false);  // X' = mu^(1/p) X T
    __syncthreads();
    if (st == kStatusFinalX) {  // the iteration forms only X, which is the result
      flops += cube;
      st = 1;
      fin = cur;
      const int t = iX;
      iX = iXn;
      iXn = t;
      break;
    }
    small_product(T2, M, M, M, t2a, t2b, t2g, n, false);
    __syncthreads();
    small_product(T4, T2, T2, nullptr, 1.f, 0.f, 0.f, n, false);
    __syncthreads();
    float* Tp = T4;
    if (p == 6 || p == 8) {
      // T^6 = T^4 T^2, T^8 = T^4 T^4, into the new-M slot, then M' into T^2's
      small_product(sm[iMn], T4, p == 6 ? T2 : T4, nullptr, 1.f, 0.f, 0.f, n, false);
      __syncthreads();
      Tp = sm[iMn];
    }
    float* Mn = (p == 6 || p == 8) ? T2 : sm[iMn];
    const float part = small_product(Mn, Tp, M, nullptr, ma, 0.f, 0.f, n, true);  // T^p (mu M)
    const float s = small_sum(part, red);
    flops += (k == 0 ? per_iter - 1 : per_iter) * cube;
    const float r = sqrtf(s) / sqrtf((float)fs.nreal[f]);
    // the stopping rule of newton_check_kernel
    const float mu = ma;
    const float rp = mu_prev > 1.f ? INFINITY : rprev;
    const bool monotone = c.tol > 0.f && mu == 1.f;
    bool accept = false;
    if (!isfinite(r)) {
      st = 3;
    } else if (monotone && r > 1.2f * rp && rp > kFloorGuard) {
      st = 3;
    } else if (monotone && r >= rp) {
      st = 2;
    } else {
      accept = true;
      rprev = r;
      fin = cur;
      if (c.tol > 0.f && r <= c.tol)
        st = 1;
      else if (cur >= c.max_iters)
        st = 4;
    }
    if (accept) {
      if (p == 6 || p == 8) {
        // M' sits in T^2's slot: copy it into the new-M slot
        for (int e = threadIdx.x; e < nn; e += blockDim.x) sm[iMn][e] = T2[e];
        __syncthreads();
      }
      int t = iM;
      iM = iMn;
      iMn = t;
      t = iX;
      iX = iXn;
      iXn = t;
    }
    if (st == 0) {
      double mun = 1.0;
      if (scaled) {
        const double a = lo;
        mun = a < kScaledPhaseEnd ? newton_balance(a, p) : 1.0;
        lo = (float)newton_map(a, p, mun);
        const double mr = pow(mun, 1.0 / p);
        t2a = (float)(mun * mun / pp);
        t2b = (float)(-2.0 * q * mun / pp);
        t2g = (float)(q * q / pp);
        xa = (float)(-mun * mr / p);
        xb = (float)(q * mr / p);
        ma = (float)mun;
        mu_prev = mu;
      }
      if (c.tol > 0.f && mu == 1.f && mun == 1.0 && cur < c.max_iters) {
        const float bound = (float)((p + 1) / (2.0 * p) * sqrt((double)fs.nreal[f]) * (double)r * r);
        if (fmaxf(bound, kRoundingFloor) <= c.tol) {
          st = kStatusFinalX;
          rprev = bound;
        }
      }
    }
  }
  // the kept iterate: X_fin (X_0 = s^(-1/p) I is never stored)
  const float* X = sm[iX];
  const float cf = c.cfac[f];
  float mx = 0.f;
  for (int e = threadIdx.x; e < nn; e += blockDim.x) {
    const int row = e / n, col = e - row * n;
    const float x = fin == 0 ? (row == col ? cf : 0.f) : X[e];
    Xroot[base + e] = x;
    mx = fmaxf(mx, fabsf(x));
  }
  if (mo.a != nullptr) raise_max2_wg<256>(mo.a + f, mx, nullptr, 0.f, mo.ver);
  if (threadIdx.x == 0) {
    c.status[f] = st;
    c.final_iter[f] = fin;
    c.rprev[f] = rprev;
    if (scaled) {
      c.lo[f] = lo;
      write_newton_coefs(rec, ma, p);
      rec[kCoefPrevMu] = mu_prev;
    }
    if (flops > 0.0) atomicAdd(c.flops_acc, flops);
  }
}

// Stage 1's kept Y (index final_iter, Ybuf0 for even, Ybuf1 for odd) becomes
// stage 2's Y0 in Ybuf0, and Z0 = I goes to Z0buf. A factor whose stage 1
// diverged keeps its status and gets no stage 2 (its root becomes s^(-1/p) I).
__global__ __launch_bounds__(256) void db_stage2_init_kernel(float* __restrict__ Ybuf0,
                                                             const float* __restrict__ Ybuf1,
                                                             float* __restrict__ Z0buf,
                                                             FactorSet fs, NewtonCtl c, MaxOut mo) {
  const int f = blockIdx.y;
  const int k = c.final_iter[f];
  const bool dead = c.status[f] == 3;
  const bool copy = !dead && (k & 1);
  float my = 0.f;
  int n;
  const float* yf = factor_ptr(Ybuf0, fs, f, n);
  const int64_t base = yf - Ybuf0;
  const int64_t nn = (int64_t)n * n;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < nn;
       e += (int64_t)gridDim.x * blockDim.x) {
    if (copy) {
      const float y = Ybuf1[base + e];
      Ybuf0[base + e] = y;
      my = fmaxf(my, fabsf(y));
    }
    Z0buf[base + e] = (e / n == e % n) ? 1.f : 0.f;
  }
  // Ybuf0 keeps its word where it was not rewritten; Z0 = I has maximum 1
  if (copy && mo.a != nullptr) raise_max(mo.a + f, my, mo.ver);
  if (mo.b != nullptr) raise_max(mo.b + f, 1.f, mo.ver);
}

__global__ __launch_bounds__(256) void rebase_words_kernel(uint64_t* __restrict__ w, int64_t n,
                                                           uint64_t ver) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    w[i] = max_word(ver, (uint32_t)(w[i] & 0xffu));
}

// After the copy above has read every factor's final_iter: stage 2 starts.
__global__ __launch_bounds__(256) void db_stage2_reset_kernel(FactorSet fs, NewtonCtl c) {
  const int f = blockIdx.x * blockDim.x + threadIdx.x;
  if (f >= fs.count()) return;
  if (c.status[f] != 3) {
    c.status[f] = 0;
    c.rprev[f] = INFINITY;
  }
  c.final_iter[f] = 0;
}

// ---------------------------------------------------------------------------
// Chebyshev inverse root: X = s^(-1/p) q(A / s), q the degree-d interpolant of
// x^(-1/p) on [r, 1] at the Chebyshev points, r = floor / s; Clenshaw in
// matrices, one symmetric product per degree.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void cheb_setup_kernel(FactorSet fs, NewtonCtl c) {
  __shared__ double fx[1025];
  __shared__ double cp[1025 + kChebBaby];
  const int f = blockIdx.x;
  const int d = c.degree, N = d + 1;
  const int m = cheb_giant(d);
  float* q = c.cheb + (size_t)f * cheb_floats(d);
  const double s = c.scale[f];
  const bool ok = c.status[f] == 0 && s > 0.0;
  const double r = ok ? fmin((double)c.floor / s, 0.999) : 0.5;
  const double pi = 3.14159265358979323846;
  for (int j = threadIdx.x; j < N; j += blockDim.x) {
    const double th = pi * (j + 0.5) / N;
    const double x = ((1.0 - r) * cos(th) + 1.0 + r) * 0.5;
    fx[j] = pow(x, -1.0 / c.p);
  }
  for (int k = threadIdx.x; k < m * kChebBaby + kChebBaby; k += blockDim.x) cp[k] = 0.0;
  __syncthreads();
  // c_j of the interpolant at the Chebyshev points, c_0 halved so that
  // p(y) = sum_j cp[j] T_j(y), y = (2 x - (1 + r)) / (1 - r)
  for (int k = threadIdx.x; k < N; k += blockDim.x) {
    double ck = 0.0;
    for (int j = 0; j < N; ++j) ck += fx[j] * cos(k * pi * (j + 0.5) / N);
    cp[k] = ck * (k == 0 ? 1.0 : 2.0) / N;
  }
  __syncthreads();
  if (threadIdx.x != 0) return;
  // y = (a/2) Ahat + (b/2) I with a = 4 / (1 - r), b = -2 (1 + r) / (1 - r)
  const double a = 4.0 / (1.0 - r), b = -2.0 * (1.0 + r) / (1.0 - r);
  for (int e = 0; e < cheb_floats(d); ++e) q[e] = 0.f;
  // T_2 = 2 y^2 - I = (a^2 / 2) Ahat Ahat + a b Ahat + (b^2 / 2 - 1) I
  q[0] = (float)(0.5 * a * a);
  q[1] = (float)(a * b);
  q[3] = (float)(0.5 * b * b - 1.0);
  // z = T_3 = 2 y T_2 - T_1 = a Ahat T_2 + b T_2 - (a/2) Ahat - (b/2) I
  q[kChebRec + 0] = (float)a;
  q[kChebRec + 1] = (float)b;
  q[kChebRec + 2] = (float)(-0.5 * a);
  q[kChebRec + 3] = (float)(-0.5 * b);
  // Giant-step form, from the top: T_(3k) T_r = (T_(3k+r) + T_(3k-r)) / 2 for
  // k, r >= 1, so the weight of T_(3k) T_r is 2 cp[3k + r], which also puts
  // cp[3k + r] on T_(3k - r) (one block lower); T_(3k) T_0 = T_(3k).
  // B_k = w0 I + w1 T_1 + w2 T_2 = (w0 + w1 b/2) I + (w1 a/2) Ahat + w2 T_2.
  for (int k = m; k >= 0; --k) {
    double w[kChebBaby];
    for (int rr = kChebBaby - 1; rr >= 1; --rr) {
      const int j = k * kChebBaby + rr;
      if (k > 0) {
        w[rr] = 2.0 * cp[j];
        cp[k * kChebBaby - rr] -= cp[j];
      } else {
        w[rr] = cp[j];
      }
    }
    w[0] = cp[k * kChebBaby];
    float* rec = q + (2 + k) * kChebRec;
    // the step k < m: beta_k = B_k + 2 z beta_(k+1) - beta_(k+2); k = 0 takes
    // z beta_1 once; beta_(m+1) = 0 (no beta2 term at k = m - 1)
    rec[0] = k == 0 ? 1.f : 2.f;
    rec[1] = 0.f;
    rec[2] = k + 2 <= m ? -1.f : 0.f;
    rec[3] = (float)(w[0] + 0.5 * b * w[1]);
    rec[4] = (float)(0.5 * a * w[1]);
    rec[5] = (float)w[2];
  }
  c.status[f] = ok ? 4 : 3;
  c.final_iter[f] = 0;
  c.rprev[f] = 0.f;
}

// out = gamma I + t_A Ahat + t_2 T2 with the weights of record `rec`.
__global__ __launch_bounds__(256) void cheb_combine_kernel(const float* __restrict__ Ahat,
                                                           const float* __restrict__ T2,
                                                           float* __restrict__ out, FactorSet fs,
                                                           NewtonCtl c, int rec, MaxOut mo) {
  const int f = blockIdx.y;
  int n;
  const float* af = factor_ptr(Ahat, fs, f, n);
  const int64_t base = af - Ahat;
  const float* q = c.cheb + (size_t)f * cheb_floats(c.degree) + rec * kChebRec;
  const float g = q[3], ta = q[4], t2 = q[5];
  const int64_t nn = (int64_t)n * n;
  float mx = 0.f;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < nn;
       e += (int64_t)gridDim.x * blockDim.x) {
    const float id = (e / n == e % n) ? g : 0.f;
    const float x = id + ta * af[e] + t2 * T2[base + e];
    out[base + e] = x;
    mx = fmaxf(mx, fabsf(x));
  }
  if (mo.a != nullptr) raise_max(mo.a + f, mx, mo.ver);
}

template <class C>
int grid_sym(const GemmLaunch& g) {
  int mx = 0;
  for (int i = 0; i < g.n_problems; ++i) {
    const int T = g.p[i].M / C::BM;
    mx = max(mx, T * (T + 1) / 2 * 8 * ((g.p[i].batch + 7) / 8));
  }
  return mx;
}
// Workgroups of a kernel that the current device holds at once, rounded down
// to a multiple of the 8 XCDs (0 if the runtime cannot tell); cached per
// kernel and device.
int resident_grid(const void* kernel, int nt) {
  static std::mutex mu;
  struct Entry {
    const void* k;
    int dev, cap;
  };
  static Entry cache[256];
  static int n = 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  std::lock_guard<std::mutex> lock(mu);
  for (int i = 0; i < n; ++i)
    if (cache[i].k == kernel && cache[i].dev == dev) return cache[i].cap;
  int cus = 0, occ = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kernel, nt, 0) != hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  const int cap = occ * cus / 8 * 8;
  if (n < 256) cache[n++] = Entry{kernel, dev, cap};
  return cap;
}

// Grid of a persistent symmetric launch: one workgroup per unit (slot, tile)
// when the device holds them all, else as many as it holds.
template <class C>
int grid_persist(const GemmLaunch& g, const void* kernel) {
  const int gx = grid_sym<C>(g);
  if (!kPersistSym<C>) return gx;
  const int cap = resident_grid(kernel, C::NT);
  return cap >= 8 && cap < gx ? cap : gx;
}

template <class C>
int grid_full(const GemmLaunch& g) {
  int mx = 0;
  for (int i = 0; i < g.n_problems; ++i)
    mx = max(mx, (g.p[i].M / C::BM) * (g.p[i].N / C::BN) * g.p[i].batch);
  return mx;
}

}  // namespace

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
hipError_t launch_pack(const BlockMeta* blocks, const MatMeta* mats, int32_t B, int32_t br,
                       int32_t bc, int32_t grad_bf16, float* Gp, float* GpT, float* Mom,
                       float momentum, uint16_t* GpH, uint16_t* GpTH, hipStream_t s, MaxOut mo) {
  if (B == 0) return hipSuccess;
  dim3 grid(((br + 63) / 64) * ((bc + 63) / 64), B);
  hipLaunchKernelGGL(pack_kernel, grid, dim3(256), 0, s, blocks, mats, br, bc, grad_bf16, Gp, GpT,
                     Mom, momentum, GpH, GpTH, mo);
  return hipGetLastError();
}

hipError_t launch_unpack(const BlockMeta* blocks, const MatMeta* dst, int32_t B, int32_t br,
                         int32_t bc, const float* Gp, hipStream_t s) {
  if (B == 0) return hipSuccess;
  dim3 grid(((br + 63) / 64) * ((bc + 63) / 64), B);
  hipLaunchKernelGGL(unpack_kernel, grid, dim3(256), 0, s, blocks, dst, br, bc, Gp);
  return hipGetLastError();
}

hipError_t launch_init_state(float* LR, int64_t nelemL, int32_t nl, int64_t nelemR, int32_t nr,
                             int32_t B, float eps, hipStream_t s) {
  if (B == 0) return hipSuccess;
  const int64_t total = nelemL + nelemR;
  const int blocks = (int)std::min<int64_t>((total + 255) / 256, 65536);
  hipLaunchKernelGGL(init_state_kernel, dim3(blocks), dim3(256), 0, s, LR, nelemL, nl, nelemR, nr,
                     eps);
  return hipGetLastError();
}

// The split main loop runs K-tiles of 16 in pairs.
// Split modes: K a multiple of 32 (the main loop takes K-tiles in pairs);
// the fp16 split also needs every operand's maximum words.
bool split_ok(const GemmLaunch& g, int mode) {
  if (mode == kGemmF32) return true;
  for (int i = 0; i < g.n_problems; ++i) {
    if (g.p[i].K % 32 != 0) return false;
    if (mode == kGemmSplitF16 && (g.p[i].mP == nullptr || g.p[i].mQ == nullptr)) return false;
  }
  return true;
}
bool mode_ok(int mode) { return mode == kGemmF32 || mode == kGemmSplit || mode == kGemmSplitF16; }

hipError_t launch_gemm_sym(const GemmLaunch& g, int tile, bool newton, int mode, hipStream_t s) {
  if (g.n_problems == 0) return hipSuccess;
  if (!mode_ok(mode) || !split_ok(g, mode)) return hipErrorInvalidValue;
  int ncols = 0;
  for (int i = 0; i < g.n_problems; ++i) {
    // symmetric problems read both operands the same way; columns on the
    // split path, for the statistics only
    if ((g.p[i].p_cols != 0) != (g.p[i].q_cols != 0)) return hipErrorInvalidValue;
    if (g.p[i].M != g.p[i].N) return hipErrorInvalidValue;  // square results only
    if (g.p[i].p_cols != 0 && (mode == kGemmF32 || newton)) return hipErrorInvalidValue;
    ncols += g.p[i].p_cols != 0;
  }
  if (ncols != 0 && ncols != g.n_problems) {
    // rows and columns in one call: one launch each (each kernel keeps the
    // registers of its own operand path)
    GemmLaunch r{}, c{};
    for (int i = 0; i < g.n_problems; ++i) {
      GemmLaunch& d = g.p[i].p_cols ? c : r;
      d.p[d.n_problems++] = g.p[i];
    }
    const hipError_t e = launch_gemm_sym(r, tile, newton, mode, s);
    return e != hipSuccess ? e : launch_gemm_sym(c, tile, newton, mode, s);
  }
  const bool cols = ncols != 0;
  int nterms = 0;
  for (int i = 0; i < g.n_problems; ++i) {
    const bool t = g.p[i].E1 != nullptr || g.p[i].E2 != nullptr;
    if (t && (g.p[i].coef == nullptr || g.p[i].coef_stride < 6 || cols)) return hipErrorInvalidValue;
    nterms += t;
  }
  if (nterms != 0 && nterms != g.n_problems) return hipErrorInvalidValue;
  // a second affine term: root products only (the Newton kernel is compiled
  // without it; such launches take their own kernel)
  int nd2 = 0;
  for (int i = 0; i < g.n_problems; ++i) nd2 += g.p[i].D2 != nullptr;
  if (nd2 != 0 && !newton) return hipErrorInvalidValue;
  switch (tile) {
#define SHP_SYM_KERNEL(KERNEL, CFG)                                                            \
  hipLaunchKernelGGL(KERNEL, dim3(grid_persist<CFG>(g, reinterpret_cast<const void*>(KERNEL)),  \
                                  g.n_problems),                                               \
                     dim3(CFG::NT), 0, s, g);
#define SHP_SYM_PLAIN(KERNEL, CFG)                                                             \
  hipLaunchKernelGGL(KERNEL, dim3(gx, g.n_problems), dim3(CFG::NT), 0, s, g);
#define SHP_SYM_LAUNCH(CFG, PATH)                                                              \
  if (nterms)                                                                                  \
    SHP_SYM_PLAIN((cheb_sym_kernel<CFG, PATH>), CFG)                                           \
  else if (newton && nd2)                                                                      \
    SHP_SYM_PLAIN((sym_d2_kernel<CFG, PATH>), CFG)                                             \
  else if (newton)                                                                             \
    SHP_SYM_KERNEL((newton_sym_kernel<CFG, PATH>), CFG)                                        \
  else                                                                                         \
    SHP_SYM_PLAIN((syrk_ema_kernel<CFG, PATH>), CFG)
#define SHP_SYM_CASE(T, CFG)                                                                   \
  case T: {                                                                                    \
    const int gx = grid_sym<CFG>(g);                                                           \
    if (!gx) break;                                                                            \
    if (cols && mode == kGemmSplitF16) {                                                       \
      SHP_SYM_PLAIN((syrk_ema_kernel<CFG, kPathSplitHCols>), CFG)                              \
    } else if (cols) {                                                                         \
      SHP_SYM_PLAIN((syrk_ema_kernel<CFG, kPathSplitCols>), CFG)                               \
    } else if (mode == kGemmSplitF16) {                                                        \
      SHP_SYM_LAUNCH(CFG, kPathSplitH)                                                         \
    } else if (mode == kGemmSplit) {                                                           \
      SHP_SYM_LAUNCH(CFG, kPathSplit)                                                          \
    } else {                                                                                   \
      SHP_SYM_LAUNCH(CFG, kPathF32)                                                            \
    }                                                                                          \
    break;                                                                                     \
  }
    case 256: {
      // 256-tiles: fp16 split only
      if (mode != kGemmSplitF16) return hipErrorInvalidValue;
      const int gx = grid_sym<Cfg256>(g);
      if (!gx) break;
      if (cols) {
        SHP_SYM_PLAIN((syrk_ema_kernel<Cfg256, kPathSplitHCols>), Cfg256)
      } else {
        SHP_SYM_LAUNCH(Cfg256, kPathSplitH)
      }
      break;
    }
    SHP_SYM_CASE(128, Cfg128)
    SHP_SYM_CASE(64, Cfg64)
    SHP_SYM_CASE(32, Cfg32)
#undef SHP_SYM_CASE
#undef SHP_SYM_LAUNCH
#undef SHP_SYM_KERNEL
#undef SHP_SYM_PLAIN
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_gemm_sym_bf16(const GemmLaunch& g, int tile, hipStream_t s) {
  if (g.n_problems == 0) return hipSuccess;
  switch (tile) {
#define SHP_SYMH_CASE(T, CFG)                                                                    \
  case T: {                                                                                      \
    const int gx = grid_sym<CFG>(g);                                                             \
    if (gx)                                                                                      \
      hipLaunchKernelGGL(syrk_bf16_kernel<CFG>, dim3(gx, g.n_problems), dim3(CFG::NT), 0, s, g);  \
    break;                                                                                       \
  }
    SHP_SYMH_CASE(256, Cfg256)
    SHP_SYMH_CASE(128, Cfg128)
    SHP_SYMH_CASE(64, Cfg64)
    SHP_SYMH_CASE(32, Cfg32)
#undef SHP_SYMH_CASE
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

namespace {
template <class CFG>
void launch_full_cfg(const GemmLaunch& g, int mode, bool pcols, bool qcols, hipStream_t s) {
  const int gx = grid_full<CFG>(g);
  if (!gx) return;
  const dim3 grid(gx, g.n_problems), block(CFG::NT);
  if (mode == kGemmSplitF16 && qcols)
    hipLaunchKernelGGL((apply_left_kernel<CFG, kPathSplitH, false, true>), grid, block, 0, s, g);
  else if (mode == kGemmSplitF16 && pcols)
    hipLaunchKernelGGL((apply_left_kernel<CFG, kPathSplitH, true, false>), grid, block, 0, s, g);
  else if (mode == kGemmSplitF16)
    hipLaunchKernelGGL((apply_left_kernel<CFG, kPathSplitH, false, false>), grid, block, 0, s, g);
  else if (mode == kGemmSplit && qcols)
    hipLaunchKernelGGL((apply_left_kernel<CFG, kPathSplit, false, true>), grid, block, 0, s, g);
  else if (mode == kGemmSplit && pcols)
    hipLaunchKernelGGL((apply_left_kernel<CFG, kPathSplit, true, false>), grid, block, 0, s, g);
  else if (mode == kGemmSplit)
    hipLaunchKernelGGL((apply_left_kernel<CFG, kPathSplit, false, false>), grid, block, 0, s, g);
  else if constexpr (CFG::BM <= 128)
    hipLaunchKernelGGL((apply_left_kernel<CFG, kPathF32, false, false>), grid, block, 0, s, g);
}
template <class CFG>
void launch_update_cfg(const GemmLaunch& g, const UpdateArgs& u, int mode, hipStream_t s) {
  const int gx = grid_full<CFG>(g);
  if (!gx) return;
  if (mode == kGemmSplitF16)
    hipLaunchKernelGGL((apply_update_kernel<CFG, kPathSplitH>), dim3(gx), dim3(CFG::NT), 0, s, g, u);
  else if (mode == kGemmSplit)
    hipLaunchKernelGGL((apply_update_kernel<CFG, kPathSplit>), dim3(gx), dim3(CFG::NT), 0, s, g, u);
  else if constexpr (CFG::BM <= 128)
    hipLaunchKernelGGL((apply_update_kernel<CFG, kPathF32>), dim3(gx), dim3(CFG::NT), 0, s, g, u);
}
}  // namespace

hipError_t launch_gemm_full(const GemmLaunch& g, int tile, int mode, hipStream_t s) {
  if (g.n_problems == 0) return hipSuccess;
  if (!mode_ok(mode) || !split_ok(g, mode)) return hipErrorInvalidValue;
  const bool pcols = g.p[0].p_cols != 0, qcols = g.p[0].q_cols != 0;
  for (int i = 1; i < g.n_problems; ++i)
    if ((g.p[i].p_cols != 0) != pcols || (g.p[i].q_cols != 0) != qcols) return hipErrorInvalidValue;
  if ((pcols || qcols) && mode == kGemmF32) return hipErrorInvalidValue;
  if (pcols && qcols) return hipErrorInvalidValue;  // no kernel reads both by columns
  if (tile == 256 && mode == kGemmF32) return hipErrorInvalidValue;
  switch (tile) {
    case 256: launch_full_cfg<Cfg256>(g, mode, pcols, qcols, s); break;
    case 128: launch_full_cfg<Cfg128>(g, mode, pcols, qcols, s); break;
    case 64: launch_full_cfg<Cfg64>(g, mode, pcols, qcols, s); break;
    case 32: launch_full_cfg<Cfg32>(g, mode, pcols, qcols, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_gemm_update(const GemmLaunch& g, const UpdateArgs& u, int tile, int mode,
                              hipStream_t s) {
  if (g.n_problems != 1 || g.p[0].p_cols != 0 || g.p[0].q_cols != 0) return hipErrorInvalidValue;
  if (!mode_ok(mode) || !split_ok(g, mode)) return hipErrorInvalidValue;
  if (tile == 256 && mode == kGemmF32) return hipErrorInvalidValue;
  switch (tile) {
    case 256: launch_update_cfg<Cfg256>(g, u, mode, s); break;
    case 128: launch_update_cfg<Cfg128>(g, u, mode, s); break;
    case 64: launch_update_cfg<Cfg64>(g, u, mode, s); break;
    case 32: launch_update_cfg<Cfg32>(g, u, mode, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_norms(const float* A, FactorSet fs, NewtonCtl c, hipStream_t s) {
  if (fs.B == 0) return hipSuccess;
  // sides are multiples of 4 or small, so the vectors stay 16-byte aligned
  const int ms = (fs.max_side() + 3) & ~3;
  hipLaunchKernelGGL(norms_kernel, dim3(fs.count()), dim3(256), 4 * ms * sizeof(float), s, A, fs, c);
  return hipGetLastError();
}

hipError_t launch_newton_init(const float* A, float* M0, float* X1, FactorSet fs, NewtonCtl c,
                              hipStream_t s, MaxOut mo) {
  if (fs.B == 0) return hipSuccess;
  const int nmax = fs.max_side();
  const int chunks = std::max(1, std::min(64, (int)(((int64_t)nmax * nmax + 4095) / 4096)));
  hipLaunchKernelGGL(newton_init_kernel, dim3(chunks, fs.count()), dim3(256), 0, s, A, M0, X1, fs, c,
                     mo);
  return hipGetLastError();
}

hipError_t launch_newton_check(FactorSet fs, NewtonCtl c, int32_t iter, int32_t shift,
                               int32_t prod_before, int32_t prod_after, hipStream_t s) {
  if (fs.B == 0) return hipSuccess;
  hipLaunchKernelGGL(newton_check_kernel, dim3(1), dim3(1024), 0, s, fs, c, iter, shift,
                     prod_before, prod_after);
  return hipGetLastError();
}

hipError_t launch_newton_final(float* Xroot, const float* Xalt, FactorSet fs, NewtonCtl c,
                               int32_t scale, hipStream_t s, MaxOut mo) {
  if (fs.B == 0) return hipSuccess;
  const int nmax = fs.max_side();
  const int chunks = std::max(1, std::min(64, (int)(((int64_t)nmax * nmax + 4095) / 4096)));
  hipLaunchKernelGGL(newton_final_kernel, dim3(chunks, fs.count()), dim3(256), 0, s, Xroot, Xalt, fs,
                     c, scale, mo);
  return hipGetLastError();
}

hipError_t launch_cheb_setup(FactorSet fs, NewtonCtl c, hipStream_t s) {
  if (fs.B == 0) return hipSuccess;
  hipLaunchKernelGGL(cheb_setup_kernel, dim3(fs.count()), dim3(256), 0, s, fs, c);
  return hipGetLastError();
}

hipError_t launch_cheb_combine(const float* Ahat, const float* T2, float* out, FactorSet fs,
                               NewtonCtl c, int32_t rec, hipStream_t s, MaxOut mo) {
  if (fs.B == 0) return hipSuccess;
  if (rec < 0 || rec >= cheb_floats(c.degree) / kChebRec) return hipErrorInvalidValue;
  const int nmax = fs.max_side();
  const int chunks = std::max(1, std::min(64, (int)(((int64_t)nmax * nmax + 4095) / 4096)));
  hipLaunchKernelGGL(cheb_combine_kernel, dim3(chunks, fs.count()), dim3(256), 0, s, Ahat, T2, out,
                     fs, c, rec, mo);
  return hipGetLastError();
}

// Host tables (block map, pointer tables) travel as kernel arguments, 2 KiB
// per launch.
constexpr int kUploadWords = 256;
struct UploadChunk {
  uint64_t w[kUploadWords];
};

__global__ __launch_bounds__(kUploadWords) void upload_kernel(uint64_t* __restrict__ dst,
                                                              UploadChunk c, int n) {
  const int i = threadIdx.x;
  if (i < n) dst[i] = c.w[i];
}

// The scratch of the entry points that allocate nothing (file scope, one
// copy per GPU).
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
constexpr int kMaxDevices = 64;

hipError_t scratch_address(void** ptr) {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t launch_upload(void* dst, const void* src, int64_t bytes, hipStream_t s) {
  const int64_t words = (bytes + 7) / 8;
  for (int64_t o = 0; o < words; o += kUploadWords) {
    UploadChunk c{};
    const int n = (int)std::min<int64_t>(kUploadWords, words - o);
    std::memcpy(c.w, static_cast<const char*>(src) + 8 * o, (size_t)std::min<int64_t>(8 * n, bytes - 8 * o));
    hipLaunchKernelGGL(upload_kernel, dim3(1), dim3(kUploadWords), 0, s,
                       static_cast<uint64_t*>(dst) + o, c, n);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

__global__ __launch_bounds__(256) void zero_words_kernel(uint64_t* __restrict__ w, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    w[i] = 0;
}

hipError_t launch_zero_words(uint64_t* w, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int blocks = (int)std::min<int64_t>((n + 255) / 256, 1024);
  hipLaunchKernelGGL(zero_words_kernel, dim3(blocks), dim3(256), 0, s, w, n);
  return hipGetLastError();
}

hipError_t launch_newton_small(const float* M0, const float* X1, float* Xroot, FactorSet fs,
                               NewtonCtl c, hipStream_t s, MaxOut mo) {
  if (fs.B == 0) return hipSuccess;
  if (fs.max_side() > kSmallSide || c.solver != kCoupledNewton) return hipErrorInvalidValue;
  hipLaunchKernelGGL(newton_small_kernel, dim3(fs.count()), dim3(256), 0, s, M0, X1, Xroot, fs, c, mo);
  return hipGetLastError();
}

hipError_t launch_rebase_words(uint64_t* w, int64_t n, uint64_t ver, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int blocks = (int)std::min<int64_t>((n + 255) / 256, 1024);
  hipLaunchKernelGGL(rebase_words_kernel, dim3(blocks), dim3(256), 0, s, w, n, ver);
  return hipGetLastError();
}

hipError_t launch_db_stage2_init(float* Ybuf0, const float* Ybuf1, float* Z0buf, FactorSet fs,
                                 NewtonCtl c, hipStream_t s, MaxOut mo) {
  if (fs.B == 0) return hipSuccess;
  const int nmax = fs.max_side();
  const int chunks = std::max(1, std::min(64, (int)(((int64_t)nmax * nmax + 4095) / 4096)));
  hipLaunchKernelGGL(db_stage2_init_kernel, dim3(chunks, fs.count()), dim3(256), 0, s, Ybuf0, Ybuf1,
                     Z0buf, fs, c, mo);
  hipLaunchKernelGGL(db_stage2_reset_kernel, dim3((fs.count() + 255) / 256), dim3(256), 0, s, fs, c);
  return hipGetLastError();
}

}  // namespace shp
