// Internal interface between the runtime (runtime.cpp) and the HIP kernels
// (kernels.hip). Not part of the public C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace shp {

// One block of one registered matrix (device copy of the block map).
struct BlockMeta {
  int32_t mat;     // matrix index, registration order
  int32_t r0, c0;  // origin of the block inside the matrix
  int32_t m, n;    // real extent (block shape minus the zero-padded tail)
  int32_t pad_;
};

// Per registered matrix; the pointers are refreshed whenever a step passes
// different ones.
struct MatMeta {
  const void* grad;
  void* param;
  int64_t ld;
};

// C[m][n] = alpha * sum_k P[k][m] Q[k][n] + beta * D[m][n] + beta2 * D2[m][n]
//           + gamma * I[m][n]
// for every element of a batch of independent matrices, all stored row-major
// and contiguous: P is K x M (element stride sP between batch members), Q is
// K x N, C and D are M x N. D may be C itself (the statistics' EMA reads the
// old value). The Newton products use the affine part to form
// T = (5 I - M) / 4 without touching the operands:
//   T T = M M / 16 - 5 M / 8 + 25 I / 16,   X T = 5 X / 4 - X M / 4.
struct GemmProblem {
  const float* P;
  const float* Q;
  float* C;
  const float* D;
  const float* D2;  // second affine term (Clenshaw's B_(k+2)), weight beta2
  int64_t sP, sQ, sC, sD, sD2;
  int32_t M, N, K;
  int32_t batch;
  float alpha, beta, gamma, beta2;
  // per-factor epilogue coefficients: if set, alpha, beta, beta2, gamma are
  // coef[(f0 + i) * coef_stride + 0..3]
  const float* coef;
  int32_t coef_stride;
  // factors with status[f0 + i] != 0 are skipped (Newton early exit), except
  // those whose status equals also_status (when non-zero)
  const int32_t* status;
  int32_t f0;
  int32_t also_status;
  // residual partials: resid[(f0 + i) * resid_stride + tile] = sum (C - I)^2
  float* resid;
  int32_t resid_stride;
  // bf16 statistics (launch_gemm_sym_bf16): C = alpha X X^T + beta D with X
  // [M][K] bf16 row-major (k contiguous), element stride sXh between members
  const uint16_t* Xh;
  int64_t sXh;
  // split path: P holds A^T [K][M] (m contiguous, row stride M) instead of
  // A [M][K], Q holds B^T [K][N] instead of B [N][K]. Full products take at
  // most one of the two; symmetric products (statistics) both or neither.
  int32_t p_cols;
  int32_t q_cols;
  // symmetric products only: two more affine terms of the epilogue, laid out
  // like D (element stride sE between members), weights coef[4] and coef[5]
  // (per-factor coefficients required)
  const float* E1;
  const float* E2;
  int64_t sE;
  // fp16 split path (kGemmSplitF16): the binary exponent of the largest
  // |value| of each operand and of the result per batch member, as versioned
  // words (max_word): member i scales P by mP[i] and Q by mQ[i] and, when mC
  // is set, raises mC[i] with version ver over the values it stores
  const uint64_t* mP;
  const uint64_t* mQ;
  uint64_t* mC;
  uint64_t ver;
};

// Versioned maximum of a buffer's values: (version << 8) | biased exponent
// of the largest |value| written with that version (255 for infinity or
// NaN). Writers raise it by 64-bit atomic max, so the word describes the
// latest write (a later version wins whatever its exponent) and no word is
// ever cleared. Versions are below 2^56 and grow by one with every launch
// that writes such words (a per-handle count).
__host__ __device__ inline uint64_t max_word(uint64_t ver, uint32_t exp_bits) {
  return (ver << 8) | (exp_bits & 0xffu);
}

// Output maxima of the per-factor elementwise root kernels (init, final
// copy, Denman-Beavers restart, Chebyshev combination): a and b are indexed
// by factor and may be NULL.
struct MaxOut {
  uint64_t* a;
  uint64_t* b;
  uint64_t ver;
};

// Raises the versioned maximum word *slot over this wave's values (m: this
// lane's largest |value|, non-negative); one 64-bit atomic per wave. Every
// lane of the wave must call it. fmaxf drops NaN, which the products
// propagate anyway.
__device__ __forceinline__ void raise_max(uint64_t* slot, float m, uint64_t ver) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  if ((threadIdx.x & 63) == 0)
    atomicMax(reinterpret_cast<unsigned long long*>(slot),
              (unsigned long long)max_word(ver, __float_as_uint(m) >> 23));
}

// As raise_max for up to two words (a or b may be NULL), one atomic per word
// and workgroup of NT threads: for kernels whose many workgroups raise the
// same word (many atomics on one address serialise). Every thread of the
// workgroup must call it.
template <int NT>
__device__ __forceinline__ void raise_max2_wg(uint64_t* a, float ma, uint64_t* b, float mb,
                                              uint64_t ver) {
  __shared__ float red[2][NT / 64];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    ma = fmaxf(ma, __shfl_xor(ma, o));
    mb = fmaxf(mb, __shfl_xor(mb, o));
  }
  __syncthreads();  // the workgroup's LDS may still be read by earlier code
  if ((threadIdx.x & 63) == 0) {
    red[0][threadIdx.x >> 6] = ma;
    red[1][threadIdx.x >> 6] = mb;
  }
  __syncthreads();
  if (threadIdx.x < 2) {
    uint64_t* slot = threadIdx.x == 0 ? a : b;
    if (slot != nullptr) {
      float m = red[threadIdx.x][0];
      for (int w = 1; w < NT / 64; ++w) m = fmaxf(m, red[threadIdx.x][w]);
      atomicMax(reinterpret_cast<unsigned long long*>(slot),
                (unsigned long long)max_word(ver, __float_as_uint(m) >> 23));
    }
  }
}

// How the fp32 products run. kGemmF32: C = P^T Q on the fp32 MFMA, P [K][M]
// and Q [K][N]. kGemmSplit: C = A B^T on the bf16 MFMA, each fp32 operand
// split into three bf16 terms (six products, fp32 accuracy); P holds A [M][K]
// and Q holds B [N][K], both with k contiguous and row stride K. For the
// symmetric products (statistics, root iterations) the two readings coincide
// when the operands are symmetric; the statistics pass the transposed
// operands on the split path. kGemmSplitF16: as kGemmSplit, but each operand,
// scaled by a power of two from its recorded maximum, is split into two fp16
// terms and three fp16 MFMA products are summed; every problem needs mP and
// mQ.
enum GemmMode : int { kGemmF32 = 0, kGemmSplit = 1, kGemmSplitF16 = 2 };

constexpr int kMaxProblems = 8;

struct GemmLaunch {
  GemmProblem p[kMaxProblems];
  int32_t n_problems;
};

// Parameter update epilogue of the second apply product.
struct UpdateArgs {
  const BlockMeta* blocks;
  const MatMeta* mats;
  float lr;
  int32_t param_bf16;
  float* out_packed;  // non-null: store U packed instead of updating params
};

// Factor addressing for the per-factor kernels: factors come in groups (the
// left and right statistics of a matrix block, or one statistic per tensor
// dimension), B factors per group; factor f = g * B + i is the i-th factor
// of group g, side side[g], stored at element offset off[g] + i * side[g]^2.
constexpr int kMaxGroups = 4;

struct FactorSet {
  int32_t B;
  int32_t n_groups;
  int32_t side[kMaxGroups];
  int64_t off[kMaxGroups];
  const int32_t* nreal;  // real extent of every factor [n_groups * B]
  __host__ __device__ int32_t count() const { return n_groups * B; }
  __host__ __device__ int32_t max_side() const {
    int32_t m = 0;
    for (int g = 0; g < n_groups; ++g) m = side[g] > m ? side[g] : m;
    return m;
  }
};

// Power-iteration products of scale modes 2 and 3 (the first shares the norm
// pass); the Chebyshev interval, which must contain the whole spectrum, takes
// more.
constexpr int kPowerIters = 8;
constexpr int kPowerItersCheb = 16;
constexpr int kMaxSide = 4096;

enum RootSolver { kCoupledNewton = 0, kNewtonDB = 1, kChebyshev = 2 };

// A residual that grows from below this value is the fp32 floor, not divergence.
constexpr float kFloorGuard = 1e-3f;

// Per-factor status of the root iterations: 0 running, 1 converged, 2 stalled,
// 3 diverged, 4 capped, 5 converged once the next iteration has formed X
// (the final-step bound met tol; that iteration runs only the X T product).
constexpr int kStatusFinalX = 5;
// Residual level below which fp32 rounding, not the iteration, decides.
constexpr float kRoundingFloor = 2.f * 1.1920929e-7f;

// Chebyshev roots by baby steps and giant steps: p(y) = sum_j c_j T_j(y) =
// sum_k B_k(y) T_k(z) with z = T_3(y) (T_(3k) = T_k o T_3) and B_k in the span
// of T_0, T_1, T_2. Per factor, records of kChebRec floats: 0 forms T_2, 1
// forms z, 2 + k the giant step k (k = 0 .. cheb_giant(degree)); each record
// holds alpha, beta, beta2, gamma and the weights of Ahat and T_2.
constexpr int kChebBaby = 3;
constexpr int kChebRec = 8;
__host__ __device__ inline int cheb_giant(int degree) {
  return degree < kChebBaby ? 0 : (degree - (kChebBaby - 1) + kChebBaby - 1) / kChebBaby;
}
__host__ __device__ inline int cheb_floats(int degree) { return (cheb_giant(degree) + 3) * kChebRec; }

struct NewtonCtl {
  int32_t solver;       // RootSolver
  float floor;          // lower bound of every statistic's spectrum: beta2^t eps
  float* cheb;          // Chebyshev records [factor][cheb_floats(degree)]
  int32_t degree;
  int32_t* status;
  int32_t* final_iter;
  float* scale;
  float* rprev;
  float* cfac;          // s^(-1/p)
  float* resid;         // partials [factor][resid_stride]
  int32_t resid_stride;
  int32_t ntiles[kMaxGroups];  // tiles actually written per factor of each group
  int32_t* active_count;       // [iter][kMaxGroups] factors active during the iteration
  double* flops_acc;           // algorithmic flops of the Newton products run
  float tol;
  int32_t max_iters;
  int32_t scale_mode;
  int32_t p;            // the root is A^(-1/p)
  // scale mode 3 (coupled Newton scaling itself every iteration):
  float* lo;            // per factor: estimate of the bottom of the spectrum of the next M
  float* coef;          // per factor kCoefRecord floats: epilogue quadruples of the next
                        // iteration's T^2, X T and M' products, then the previous scale
};

// Scale mode 3 (see newton_check_kernel): record layout per factor.
constexpr int kCoefRecord = 16;
constexpr int kCoefT2 = 0, kCoefXT = 4, kCoefM = 8, kCoefPrevMu = 12;
constexpr double kScaledPhaseEnd = 0.75;
constexpr int kBalanceSteps = 40;

// ---- launchers (return hipGetLastError()) ----
// Mom (nullable): momentum buffer [B][br][bc], updated as Mom = momentum * Mom + Gp.
// GpT (fp32 transpose; nullable, then not written) or, for bf16 gradients,
// GpH / GpTH: the packed block and its transpose as bf16 (the gradient's own
// values), for the bf16 statistics. mo: maxima of Gp (a) and Mom (b) per block.
hipError_t launch_pack(const BlockMeta* blocks, const MatMeta* mats, int32_t B, int32_t br, int32_t bc,
                       int32_t grad_bf16, float* Gp, float* GpT, float* Mom, float momentum,
                       uint16_t* GpH, uint16_t* GpTH, hipStream_t s, MaxOut mo = MaxOut{});
hipError_t launch_unpack(const BlockMeta* blocks, const MatMeta* dst, int32_t B, int32_t br,
                         int32_t bc, const float* Gp, hipStream_t s);
hipError_t launch_init_state(float* LR, int64_t nelemL, int32_t nl, int64_t nelemR, int32_t nr,
                             int32_t B, float eps, hipStream_t s);
hipError_t launch_gemm_sym(const GemmLaunch& g, int tile, bool newton, int mode, hipStream_t s);
// Statistics from bf16 operands on the bf16 MFMA (exact products, fp32
// accumulation): the problems' Xh / sXh, same epilogue as the symmetric
// product. M and K multiples of the tile and of 32.
hipError_t launch_gemm_sym_bf16(const GemmLaunch& g, int tile, hipStream_t s);
hipError_t launch_gemm_full(const GemmLaunch& g, int tile, int mode, hipStream_t s);
hipError_t launch_gemm_update(const GemmLaunch& g, const UpdateArgs& u, int tile, int mode,
                              hipStream_t s);
hipError_t launch_norms(const float* A, FactorSet fs, NewtonCtl c, hipStream_t s);
// mo: maxima of M0 (a) and X1 (b) per factor.
hipError_t launch_newton_init(const float* A, float* M0, float* X1, FactorSet fs, NewtonCtl c,
                              hipStream_t s, MaxOut mo = MaxOut{});
// shift: the residual just computed belongs to iterate iter + shift (1 for
// coupled Newton, whose products first make the next iterate; 0 for the
// Denman-Beavers pair, whose residual product comes first). prod_before /
// prod_after: symmetric products per factor launched before the check (all
// factors entering it) and after it (those still running), for the flop count.
hipError_t launch_newton_check(FactorSet fs, NewtonCtl c, int32_t iter, int32_t shift,
                               int32_t prod_before, int32_t prod_after, hipStream_t s);
// scale: multiply the kept iterate by s^(-1/p) (Denman-Beavers result).
// mo.a: maxima of Xroot per factor (raised where this kernel writes).
hipError_t launch_newton_final(float* Xroot, const float* Xalt, FactorSet fs, NewtonCtl c,
                               int32_t scale, hipStream_t s, MaxOut mo = MaxOut{});
// Chebyshev: per factor, the interval [r, 1] (r = floor / s), the interpolant's
// coefficients c_j at degree + 1 Chebyshev points, their giant-step form and
// the epilogue records (kChebRec); status = capped (a fixed-degree result).
hipError_t launch_cheb_setup(FactorSet fs, NewtonCtl c, hipStream_t s);
// out = gamma I + t_A Ahat + t_2 T2 with the weights of record `rec` of each
// factor (the giant sum's leading term B_m).
hipError_t launch_cheb_combine(const float* Ahat, const float* T2, float* out, FactorSet fs,
                               NewtonCtl c, int32_t rec, hipStream_t s, MaxOut mo = MaxOut{});
// Between the two Denman-Beavers stages: Y1 (kept pair of stage 1, in Ybuf0 or
// Ybuf1 by parity) becomes stage 2's Y0 in Ybuf0, Z0 = I goes to Z0buf.
// mo: maxima of Ybuf0 (a) and Z0buf (b) per factor.
hipError_t launch_db_stage2_init(float* Ybuf0, const float* Ybuf1, float* Z0buf, FactorSet fs,
                                 NewtonCtl c, hipStream_t s, MaxOut mo = MaxOut{});
// Coupled Newton for factor sets whose sides are all <= kSmallSide: every
// iteration in one launch (one workgroup per factor, iterates in LDS, fp32
// FMA products), from M0 and X1 of launch_newton_init to the kept root in
// Xroot, with the status, iteration, residual and scaling records of the
// per-iteration kernels and the roots' maximum words (mo.a).
constexpr int kSmallSide = 64;
hipError_t launch_newton_small(const float* M0, const float* X1, float* Xroot, FactorSet fs,
                               NewtonCtl c, hipStream_t s, MaxOut mo = MaxOut{});
// Maximum words w[0 .. n) keep their exponents and take version ver (after a
// restore wrote words of another handle's versions).
hipError_t launch_rebase_words(uint64_t* w, int64_t n, uint64_t ver, hipStream_t s);
// Copies `bytes` of host memory at src to device memory at dst (8-byte
// aligned, with room for bytes rounded up to a multiple of 8) through the
// arguments of small kernels: they are copied when a launch is enqueued, so
// src may be freed or reused as soon as this returns and the host never
// waits for a copy from pageable memory.
hipError_t launch_upload(void* dst, const void* src, int64_t bytes, hipStream_t s);

// Library-held scratch for callers that cannot allocate: a static device
// array of kScratchBytes per GPU, alive until the process ends. Its device
// address on the current device (hipGetSymbolAddress, fetched once per
// device; host code must use this address, never the array's name). Every
// call that uses it on one GPU shares it: calls that overlap there race.
constexpr int64_t kScratchBytes = int64_t(64) << 20;
hipError_t scratch_address(void** ptr);
// w[0 .. n) = 0 by a kernel (no memset node, so it can be captured).
hipError_t launch_zero_words(uint64_t* w, int64_t n, hipStream_t s);

// Tiles written by a symmetric product of side n with square tile t.
inline int32_t sym_tiles(int32_t n, int32_t t) {
  int32_t T = n / t;
  return T * (T + 1) / 2;
}

}  // namespace shp

// ===========================================================================
// Order-k tensors (podcast "Preconditioned Optimization Without the Full
// Matrix Cost", cue 26): one statistic per dimension. A packed block is a
// dense row-major [b_0][b_1]...[b_(k-1)] array (E elements), zero past the
// block's real extent.
// ===========================================================================
namespace shp {

constexpr int kMaxOrder = 4;
constexpr int kMaxSmallSide = 8;  // dimensions blocked at <= 8 take the small-side kernels

struct TensorMeta {
  const void* grad;
  void* param;
  int64_t stride[kMaxOrder];  // element strides of the tensor
};

struct TBlockMeta {
  int32_t tensor;
  int32_t origin[kMaxOrder];
  int32_t extent[kMaxOrder];
  int32_t pad_;
};

struct TensorGeom {
  int32_t order;
  int32_t b[kMaxOrder];  // packed extent of every dimension
  int32_t E;             // elements of a packed block
  // division by b[d] as a multiply-high: q = umulhi64(x, magic[d]) with
  // magic = ceil(2^64 / b) (exact for 32-bit x); 0 when b = 1
  uint64_t magic[kMaxOrder];
};

// ceil(2^64 / d) for d >= 2; 0 for d = 1 (division by 1 is skipped).
inline uint64_t division_magic(uint32_t d) {
  return d <= 1 ? 0 : ~(uint64_t)0 / d + 1;
}

// Gp[blk][e] (+ Mom = momentum Mom + Gp) from the tensors; mo: maxima of
// Gp (a) and Mom (b) per block.
hipError_t launch_tensor_pack(const TBlockMeta* blocks, const TensorMeta* tensors, TensorGeom g,
                              int32_t B, int32_t grad_bf16, float* Gp, float* Mom, float momentum,
                              hipStream_t s, MaxOut mo = MaxOut{});
// mode 0: dst[...] = Src (unpack into the param pointers of `tensors`);
// mode 1: param -= lr * Src (update; bf16 parameters rounded to nearest even).
hipError_t launch_tensor_scatter(const TBlockMeta* blocks, const TensorMeta* tensors, TensorGeom g,
                                 int32_t B, const float* Src, float lr, int32_t param_bf16,
                                 int32_t update, hipStream_t s);
// Out[blk] = transpose of In[blk] viewed as R x C (Out is C x R); each Out
// block holds out_stride elements, the R * C of the transpose then zeros.
hipError_t launch_transpose(const float* In, int64_t in_stride, float* Out, int64_t out_stride,
                            int32_t R, int32_t C, int32_t B, hipStream_t s);
// Small-side statistic of dimension with extent n (<= 8) of In[blk] viewed as
// [A][n][C]: H <- beta2 H + gamma sum_(a, c) In[a][l][c] In[a][l'][c].
// partial: scratch of B * chunks * 36 floats.
hipError_t launch_small_gram(const float* In, int64_t in_stride, int32_t A, int32_t n, int32_t C,
                             int32_t B, float* partial, int32_t chunks, float* H, float beta2,
                             float gamma, hipStream_t s);
// Out[blk][r][j] = sum_l X[blk][j][l] In[blk][l][r]: the product along the
// leading dimension (extent n), which moves that dimension last. FMA kernel
// for small n or a row count R that the MFMA tiles do not divide.
// mo.a: maxima of Out per block.
hipError_t launch_mode_product(const float* In, int64_t in_stride, const float* X, int64_t x_stride,
                               float* Out, int64_t out_stride, int32_t n, int32_t R, int32_t B,
                               hipStream_t s, MaxOut mo = MaxOut{});
// The last product (leading dimension k-1, extent <= 8) with the update
// W -= lr * U written straight into the parameters (no packed U).
hipError_t launch_mode_product_update(const float* In, int64_t in_stride, const float* X,
                                      int64_t x_stride, const TBlockMeta* blocks,
                                      const TensorMeta* tensors, TensorGeom g, int32_t R, int32_t B,
                                      float lr, int32_t param_bf16, hipStream_t s);
// Largest side of the two-dimension fusions below (small statistics, last
// two mode products with the update).
constexpr int kMaxFusedSide = 5;
// Statistics of two small trailing dimensions of one side n <= kMaxFusedSide in
// one pass over the blocks ([A][n][n] each): chunk partials of both (pairs of
// dimension order - 2, then of order - 1, in one row of kMaxPairs), then the
// EMA of H2 and H3.
hipError_t launch_small_gram2(const float* In, int64_t in_stride, int32_t A, int32_t n,
                              int32_t B, float* partial, int32_t chunks, float* H2, float* H3,
                              float beta2, float gamma, hipStream_t s);
// The last two mode products fused with the update, for two small trailing
// dimensions of equal side n = g.b[order - 1] <= kMaxFusedSide: In is the
// block rotated to [n][n][R], X2 and X3 the roots of dimensions order - 2 and
// order - 1 (n x n per block, x_stride apart).
hipError_t launch_mode_product2_update(const float* In, int64_t in_stride, const float* X2,
                                       const float* X3, int64_t x_stride,
                                       const TBlockMeta* blocks, const TensorMeta* tensors,
                                       TensorGeom g, int32_t R, int32_t B, float lr,
                                       int32_t param_bf16, hipStream_t s);
// Small-side roots: per factor (count factors of side n, real extent nreal[f]),
// fp64 cyclic Jacobi of H, X = V diag(max(lam, floor)^(-1/p)) V^T on the real
// extent, zero elsewhere. status / final_iter / resid of each factor are written
// (1 / sweeps / relative off-diagonal norm left; 3 if H is not finite).
hipError_t launch_small_root(const float* H, float* X, int32_t n, int32_t count,
                             const int32_t* nreal, float floor, int32_t p, int32_t* status,
                             int32_t* final_iter, float* resid, hipStream_t s);

}  // namespace shp
