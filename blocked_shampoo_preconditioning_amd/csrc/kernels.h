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
  // factors with status[f0 + i] != 0 are skipped (Newton early exit)
  const int32_t* status;
  int32_t f0;
  // residual partials: resid[(f0 + i) * resid_stride + tile] = sum (C - I)^2
  float* resid;
  int32_t resid_stride;
};

constexpr int kMaxProblems = 4;

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

// Factor addressing for the per-factor kernels: factors [0, B) are left
// statistics of side nl, [B, 2B) right statistics of side nr; left factors
// start at baseL, right factors at baseR (element offsets into a buffer).
struct FactorSet {
  int32_t B;
  int32_t nl, nr;
  int64_t offL, offR;  // element offsets of the first left / right factor
  const int32_t* nreal;
};

// Power-iteration products of scale mode 2 (the first shares the norm pass).
constexpr int kPowerIters = 16;
constexpr int kMaxSide = 4096;

enum RootSolver { kCoupledNewton = 0, kNewtonDB = 1, kChebyshev = 2 };

// A residual that grows from below this value is the fp32 floor, not divergence.
constexpr float kFloorGuard = 1e-3f;

struct NewtonCtl {
  int32_t solver;       // RootSolver
  float floor;          // lower bound of every statistic's spectrum: beta2^t eps
  float* cheb;          // Chebyshev coefficient quadruples [2B][degree + 1][4]
  int32_t degree;
  int32_t* status;
  int32_t* final_iter;
  float* scale;
  float* rprev;
  float* cfac;          // s^(-1/4)
  float* resid;         // partials [2B][resid_stride]
  int32_t resid_stride;
  int32_t ntiles_l, ntiles_r;  // tiles actually written per left / right factor
  int32_t* active_count;       // [iter][2] factors active during the iteration
  double* flops_acc;           // algorithmic flops of the Newton products run
  float tol;
  int32_t max_iters;
  int32_t scale_mode;
};

// ---- launchers (return hipGetLastError()) ----
// Mom (nullable): momentum buffer [B][br][bc], updated as Mom = momentum * Mom + Gp.
hipError_t launch_pack(const BlockMeta* blocks, const MatMeta* mats, int32_t B, int32_t br, int32_t bc,
                       int32_t grad_bf16, float* Gp, float* GpT, float* Mom, float momentum,
                       hipStream_t s);
hipError_t launch_unpack(const BlockMeta* blocks, const MatMeta* dst, int32_t B, int32_t br,
                         int32_t bc, const float* Gp, hipStream_t s);
hipError_t launch_init_state(float* LR, int64_t nelemL, int32_t nl, int64_t nelemR, int32_t nr,
                             int32_t B, float eps, hipStream_t s);
hipError_t launch_gemm_sym(const GemmLaunch& g, int tile, bool newton, hipStream_t s);
hipError_t launch_gemm_full(const GemmLaunch& g, int tile, hipStream_t s);
hipError_t launch_gemm_update(const GemmLaunch& g, const UpdateArgs& u, int tile, hipStream_t s);
hipError_t launch_norms(const float* A, FactorSet fs, NewtonCtl c, hipStream_t s);
hipError_t launch_newton_init(const float* A, float* M0, float* X1, FactorSet fs, NewtonCtl c,
                              hipStream_t s);
// shift: the residual just computed belongs to iterate iter + shift (1 for
// coupled Newton, whose products first make the next iterate; 0 for the
// Denman-Beavers pair, whose residual product comes first). prod_before /
// prod_after: symmetric products per factor launched before the check (all
// factors entering it) and after it (those still running), for the flop count.
hipError_t launch_newton_check(FactorSet fs, NewtonCtl c, int32_t iter, int32_t shift,
                               int32_t prod_before, int32_t prod_after, hipStream_t s);
// scale: multiply the kept iterate by s^(-1/4) (Denman-Beavers result).
hipError_t launch_newton_final(float* Xroot, const float* Xalt, FactorSet fs, NewtonCtl c,
                               int32_t scale, hipStream_t s);
// Chebyshev: per factor, the interval [r, 1] (r = floor / s), the interpolant's
// coefficients and the Clenshaw epilogue quadruples; status = capped.
hipError_t launch_cheb_setup(FactorSet fs, NewtonCtl c, hipStream_t s);
// B_d = c_d I and B_(d-1) = c_(d-1) I + 2 c_d T(Ahat), T = (2 Ahat - (1 + r) I) / (1 - r).
hipError_t launch_cheb_init(const float* Ahat, float* Bd, float* Bd1, FactorSet fs, NewtonCtl c,
                            hipStream_t s);
// Between the two Denman-Beavers stages: Y1 (kept pair of stage 1, in Ybuf0 or
// Ybuf1 by parity) becomes stage 2's Y0 in Ybuf0, Z0 = I goes to Z0buf.
hipError_t launch_db_stage2_init(float* Ybuf0, const float* Ybuf1, float* Z0buf, FactorSet fs,
                                 NewtonCtl c, hipStream_t s);

// Tiles written by a symmetric product of side n with square tile t.
inline int32_t sym_tiles(int32_t n, int32_t t) {
  int32_t T = n / t;
  return T * (T + 1) / 2;
}

}  // namespace shp
