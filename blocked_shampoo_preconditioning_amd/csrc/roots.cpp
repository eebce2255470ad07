// Inverse roots A^(-1/p) of batches of symmetric statistics on the symmetric
// MFMA product core: norm scaling, then the coupled Newton iteration (any
// even p up to 8), the Denman-Beavers pair (p = 4) or the Chebyshev
// interpolant (any p). Every launch goes to the caller's stream; per-factor
// stop rules run on the device (no host synchronisation).
#include <cmath>

#include "runtime_common.h"

namespace shp_rt {
namespace {

// Symmetric-product launches of one stage, one per MFMA tile size in use.
struct SymLaunches {
  int n = 0;
  int tile[shp::kMaxGroups];
  shp::GemmLaunch g[shp::kMaxGroups];
};

shp::GemmProblem sym_problem(const float* P, const float* Q, float* C, int64_t stride, int n, int k,
                             int batch) {
  shp::GemmProblem g{};
  g.P = P;
  g.Q = Q;
  g.C = C;
  g.sP = stride;
  g.sQ = stride;
  g.sC = (int64_t)n * n;
  g.M = n;
  g.N = n;
  g.K = k;
  g.batch = batch;
  g.alpha = 1.f;
  return g;
}

// Maximum words of one of the job's buffers (fp16 split products), or NULL.
uint64_t* slot_of(const RootJob& j, const float* buf) {
  if (buf == nullptr) return nullptr;
  const float* bufs[6] = {j.xroot, j.xalt, j.s[0], j.s[1], j.s[2], j.s[3]};
  for (int i = 0; i < 6; ++i)
    if (bufs[i] == buf) return j.mx[i];
  return nullptr;
}

shp::MaxOut max_out(shampoo_ctx* h, const RootJob& j, const float* a, const float* b) {
  shp::MaxOut mo{};
  mo.a = slot_of(j, a);
  mo.b = slot_of(j, b);
  if (mo.a != nullptr || mo.b != nullptr) mo.ver = h->next_ver();
  return mo;
}

// C = alpha P Q + beta D + gamma I over every factor; groups of one side and
// tile stored back to back share a problem. coef_slot >= 0: the epilogue
// coefficients come per factor from that slot of the scale-mode-3 records.
void factor_problems(const RootJob& j, SymLaunches& L, const float* P, const float* Q, float* C,
                     const float* D, float alpha, float beta, float gamma, bool resid,
                     int coef_slot = -1, int also_status = 0) {
  const shp::FactorSet& fs = j.fs;
  for (int g = 0; g < fs.n_groups;) {
    int e = g + 1;
    while (e < fs.n_groups && fs.side[e] == fs.side[g] && j.tile[e] == j.tile[g] &&
           fs.off[e] == fs.off[e - 1] + (int64_t)fs.B * fs.side[g] * fs.side[g])
      ++e;
    const int n = fs.side[g];
    const int64_t off = fs.off[g];
    shp::GemmProblem q = sym_problem(P + off, Q + off, C + off, (int64_t)n * n, n, n,
                                     (e - g) * fs.B);
    q.alpha = alpha;
    q.beta = beta;
    q.gamma = gamma;
    if (D != nullptr) {
      q.D = D + off;
      q.sD = (int64_t)n * n;
    }
    q.status = j.c.status;
    q.f0 = g * fs.B;
    q.also_status = also_status;
    if (coef_slot >= 0 && j.c.coef != nullptr) {
      q.coef = j.c.coef + coef_slot;
      q.coef_stride = shp::kCoefRecord;
    }
    if (resid) {
      q.resid = j.c.resid;
      q.resid_stride = j.c.resid_stride;
    }
    // operand and result maxima of the fp16 split (member i is factor f0 + i)
    uint64_t* mp = slot_of(j, P);
    uint64_t* mq = slot_of(j, Q);
    uint64_t* mc = slot_of(j, C);
    q.mP = mp != nullptr ? mp + q.f0 : nullptr;
    q.mQ = mq != nullptr ? mq + q.f0 : nullptr;
    q.mC = mc != nullptr ? mc + q.f0 : nullptr;
    int li = 0;
    while (li < L.n && L.tile[li] != j.tile[g]) ++li;
    if (li == L.n) {
      L.tile[L.n] = j.tile[g];
      L.g[L.n] = shp::GemmLaunch{};
      ++L.n;
    }
    L.g[li].p[L.g[li].n_problems++] = q;
    g = e;
  }
}

int launch_all(shampoo_ctx* h, const RootJob& j, const SymLaunches& L, double flops,
               hipStream_t s) {
  for (int i = 0; i < L.n; ++i) {
    shp::GemmLaunch g = L.g[i];
    const uint64_t ver = h->next_ver();
    for (int k = 0; k < g.n_problems; ++k) g.p[k].ver = ver;
    const int rc = timed(h, kNewtonGemm, i == 0 ? flops : 0.0, 0.0, s,
                         [&] { return shp::launch_gemm_sym(g, L.tile[i], true, j.gemm_mode, s); });
    if (rc) return rc;
  }
  return SHAMPOO_OK;
}

// Bytes the norm pass reads: every factor (at its padded side) once, and again
// for each power-iteration step after the first (scale modes 2 and 3, Chebyshev).
double norm_bytes(const RootJob& j) {
  const bool power = j.c.scale_mode >= 2 || j.c.solver == shp::kChebyshev;
  const double passes =
      power ? (j.c.solver == shp::kChebyshev ? shp::kPowerItersCheb : shp::kPowerIters) : 1.0;
  double b = 0.0;
  for (int g = 0; g < j.fs.n_groups; ++g) b += 4.0 * j.fs.B * (double)j.fs.side[g] * j.fs.side[g];
  return b * passes;
}

// Coupled Newton for A^(-1/p), p in {4, 6, 8} (scale mode 3: M scaled by a
// per-factor mu each iteration, X by mu^(1/p), folded into the same
// epilogues): T = ((p + 1) I - M) / p enters through the affine epilogues
//   T T = (M M - 2 (p + 1) M + (p + 1)^2 I) / p^2,   X T = ((p + 1) X - X M) / p,
// then T^p by squaring (T^6 = T^4 T^2, T^8 = T^4 T^4) and M <- T^p M.
// Buffers: M in s[iM], T^2 in s[iT], T^4 in s[2], T^6 / T^8 in s[3]; the new M
// overwrites T^2 and the two swap roles. X ping-pongs between xroot (even
// iterates) and xalt (odd); X_1 is formed by the init kernel.
int newton(shampoo_ctx* h, const RootJob& j, hipStream_t s) {
  const shp::FactorSet& fs = j.fs;
  const shp::NewtonCtl& c = j.c;
  int rc = timed(h, kNorms, 0.0, norm_bytes(j), s, [&] { return shp::launch_norms(j.A, fs, c, s); });
  if (rc) return rc;
  rc = timed(h, kNewtonAux, 0.0, 0.0, s, [&] {
    return shp::launch_newton_init(j.A, j.s[0], j.xalt, fs, c, s, max_out(h, j, j.s[0], j.xalt));
  });
  if (rc) return rc;
  if (fs.max_side() <= shp::kSmallSide) {
    // small factors: the whole iteration in one launch (its flops are counted
    // on the device)
    return timed(h, kNewtonGemm, 0.0, 0.0, s, [&] {
      return shp::launch_newton_small(j.s[0], j.xalt, j.xroot, fs, c, s,
                                      max_out(h, j, j.xroot, nullptr));
    });
  }
  const double p = c.p;
  const float a2 = (float)(1.0 / (p * p)), b2 = (float)(-2.0 * (p + 1.0) / (p * p)),
              g2 = (float)((p + 1.0) * (p + 1.0) / (p * p));
  const float xa = (float)(-1.0 / p), xb = (float)((p + 1.0) / p);
  const int per_iter = c.p == 4 ? 4 : 5;  // symmetric products of one iteration
  int iM = 0, iT = 1;
  for (int k = 0; k < c.max_iters; ++k) {
    float* M = j.s[iM];
    float* T2 = j.s[iT];
    float* T4 = j.s[2];
    float* Xcur = (k % 2 == 0) ? j.xroot : j.xalt;
    float* Xnext = (k % 2 == 0) ? j.xalt : j.xroot;
    // scale mode 3: per-factor coefficients of the scaled iteration (the
    // check kernel writes the next iteration's)
    const bool sc = c.scale_mode == 3 && c.coef != nullptr;
    SymLaunches l1, l2, l3, l4;
    factor_problems(j, l1, M, M, T2, M, a2, b2, g2, false, sc ? shp::kCoefT2 : -1);  // T^2
    // X T runs also for the factors whose final-step bound met tol: their last
    // iteration forms only X
    if (k > 0)
      factor_problems(j, l1, Xcur, M, Xnext, Xcur, xa, xb, 0.f, false,
                      sc ? shp::kCoefXT : -1, shp::kStatusFinalX);              // X T
    factor_problems(j, l2, T2, T2, T4, nullptr, 1.f, 0.f, 0.f, false);            // T^4
    const float* Tp = T4;
    if (c.p == 6 || c.p == 8) {
      factor_problems(j, l3, T4, c.p == 6 ? T2 : T4, j.s[3], nullptr, 1.f, 0.f, 0.f, false);
      Tp = j.s[3];
    }
    factor_problems(j, l4, Tp, M, T2, nullptr, 1.f, 0.f, 0.f, true,
                    sc ? shp::kCoefM : -1);  // M <- T^p (mu M)
    if ((rc = launch_all(h, j, l1, 0.0, s))) return rc;
    if ((rc = launch_all(h, j, l2, 0.0, s))) return rc;
    if ((rc = launch_all(h, j, l3, 0.0, s))) return rc;
    if ((rc = launch_all(h, j, l4, 0.0, s))) return rc;
    const int before = k == 0 ? per_iter - 1 : per_iter;
    rc = timed(h, kNewtonAux, 0.0, 0.0, s,
               [&] { return shp::launch_newton_check(fs, c, k, 1, before, 0, s); });
    if (rc) return rc;
    std::swap(iM, iT);
  }
  return timed(h, kNewtonAux, 0.0, 0.0, s, [&] {
    return shp::launch_newton_final(j.xroot, j.xalt, fs, c, 0, s, max_out(h, j, j.xroot, nullptr));
  });
}

// Newton-DB: two Denman-Beavers square-root stages in inverse-free form on
// the symmetric GEMM core. Y ping-pongs between s[0] (even k) and s[1] (odd),
// Z between xroot and xalt, M = Z Y goes to s[2]. Per iteration: M (with the
// residual partials), the check, then Y' = 3Y/2 - Y M/2 and Z' = 3Z/2 - M Z/2
// in one launch. Stage 2 restarts from stage 1's kept Y with Z = I; the root
// is s^(-1/4) times stage 2's kept Z.
int newton_db(shampoo_ctx* h, const RootJob& j, hipStream_t s) {
  const shp::FactorSet& fs = j.fs;
  const shp::NewtonCtl& c = j.c;
  int rc = timed(h, kNorms, 0.0, norm_bytes(j), s, [&] { return shp::launch_norms(j.A, fs, c, s); });
  if (rc) return rc;
  rc = timed(h, kNewtonAux, 0.0, 0.0, s, [&] {
    return shp::launch_newton_init(j.A, j.s[0], j.xroot, fs, c, s, max_out(h, j, j.s[0], j.xroot));
  });
  if (rc) return rc;
  const int kmax = c.max_iters;
  for (int stage = 0; stage < 2; ++stage) {
    for (int k = 0; k <= kmax; ++k) {
      float* Y = j.s[k & 1];
      float* Z = (k & 1) ? j.xalt : j.xroot;
      float* Yn = j.s[(k + 1) & 1];
      float* Zn = ((k + 1) & 1) ? j.xalt : j.xroot;
      SymLaunches l1;
      factor_problems(j, l1, Z, Y, j.s[2], nullptr, 1.f, 0.f, 0.f, true);  // M = Z Y
      if ((rc = launch_all(h, j, l1, 0.0, s))) return rc;
      const int after = k < kmax ? 2 : 0;
      rc = timed(h, kNewtonAux, 0.0, 0.0, s,
                 [&] { return shp::launch_newton_check(fs, c, k, 0, 1, after, s); });
      if (rc) return rc;
      if (k == kmax) break;
      SymLaunches l2;
      factor_problems(j, l2, Y, j.s[2], Yn, Y, -0.5f, 1.5f, 0.f, false);  // Y (3I - M) / 2
      factor_problems(j, l2, j.s[2], Z, Zn, Z, -0.5f, 1.5f, 0.f, false);  // (3I - M) Z / 2
      if ((rc = launch_all(h, j, l2, 0.0, s))) return rc;
    }
    if (stage == 0) {
      rc = timed(h, kNewtonAux, 0.0, 0.0, s, [&] {
        return shp::launch_db_stage2_init(j.s[0], j.s[1], j.xroot, fs, c, s,
                                          max_out(h, j, j.s[0], j.xroot));
      });
      if (rc) return rc;
    }
  }
  return timed(h, kNewtonAux, 0.0, 0.0, s, [&] {
    return shp::launch_newton_final(j.xroot, j.xalt, fs, c, 1, s, max_out(h, j, j.xroot, nullptr));
  });
}

// Chebyshev: X = s^(-1/p) p(Ahat), Ahat = A / s, p = sum_j c_j T_j(y) with
// y = (2 Ahat - (1 + r) I) / (1 - r), evaluated by baby steps and giant steps:
// T_2 and z = T_3 (two products), then the Clenshaw recurrence in z over
// p = sum_k B_k T_k(z), B_k = w0 I + w1 T_1 + w2 T_2 (T_(3k) = T_k o T_3): one
// product per giant step with B_k added in its epilogue, cheb_giant(d) of
// them, 2 + ceil((d - 2) / 3) products in all instead of d - 1. Buffers: T_2
// in s[0], z in s[1], beta_k in xroot / s[2] / s[3] by k % 3.
int chebyshev(shampoo_ctx* h, const RootJob& j, hipStream_t s) {
  const shp::FactorSet& fs = j.fs;
  shp::NewtonCtl c = j.c;
  c.floor = (float)(std::pow(h->cfg.beta2, (double)j.t_stats) * h->cfg.eps);
  const int d = c.degree;
  const int m = shp::cheb_giant(d);
  const int rec_floats = shp::cheb_floats(d);
  if (j.s[3] == nullptr) return fail(SHAMPOO_ERR_INVALID_ARG, "Chebyshev roots need a fourth scratch buffer");
  int rc = timed(h, kNorms, 0.0, norm_bytes(j), s, [&] { return shp::launch_norms(j.A, fs, c, s); });
  if (rc) return rc;
  // Ahat in xalt (identity on tail padding); the records (which mark every
  // factor as a fixed-degree result)
  rc = timed(h, kNewtonAux, 0.0, 0.0, s, [&] {
    return shp::launch_newton_init(j.A, j.xalt, nullptr, fs, c, s, max_out(h, j, j.xalt, nullptr));
  });
  if (rc) return rc;
  rc = timed(h, kNewtonAux, 0.0, 0.0, s, [&] { return shp::launch_cheb_setup(fs, c, s); });
  if (rc) return rc;
  float* Ahat = j.xalt;
  float* T2 = j.s[0];
  float* Z = j.s[1];
  float* ring[3] = {j.xroot, j.s[2], j.s[3]};  // beta_k in ring[k % 3]; p = beta_0 in xroot
  // one symmetric product per factor group, C = P Q with the epilogue of
  // record `rec`: beta D + beta2 D2 (+ the Ahat and T_2 terms when `terms`)
  auto step = [&](const float* P, const float* Q, float* C, const float* D, const float* D2,
                  int rec, bool terms) {
    SymLaunches L;
    factor_problems(j, L, P, Q, C, D, 1.f, 0.f, 0.f, false);
    for (int li = 0; li < L.n; ++li)
      for (int i = 0; i < L.g[li].n_problems; ++i) {
        shp::GemmProblem& q = L.g[li].p[i];
        const int64_t off = q.C - C;
        q.D2 = D2 != nullptr ? D2 + off : nullptr;
        q.sD2 = q.sC;
        if (terms) {
          q.E1 = Ahat + off;
          q.E2 = T2 + off;
          q.sE = q.sC;
        }
        q.status = nullptr;  // every factor runs the whole sum
        q.coef = c.cheb + (size_t)rec * shp::kChebRec;
        q.coef_stride = rec_floats;
      }
    return launch_all(h, j, L, j.real_cube, s);
  };
  // baby steps: T_2 = (a^2/2) Ahat Ahat + a b Ahat + ..., z = a Ahat T_2 + b T_2 - (a/2) Ahat + ...
  if ((rc = step(Ahat, Ahat, T2, Ahat, nullptr, 0, false))) return rc;
  if (m > 0 && (rc = step(Ahat, T2, Z, T2, Ahat, 1, false))) return rc;
  // giant steps: beta_m = B_m, then beta_k = B_k + 2 z beta_(k+1) - beta_(k+2)
  // down to p = B_0 + z beta_1 - beta_2
  rc = timed(h, kNewtonAux, 0.0, 0.0, s, [&] {
    return shp::launch_cheb_combine(Ahat, T2, ring[m % 3], fs, c, 2 + m, s,
                                    max_out(h, j, ring[m % 3], nullptr));
  });
  if (rc) return rc;
  for (int k = m - 1; k >= 0; --k) {
    const float* D2 = k + 2 <= m ? ring[(k + 2) % 3] : nullptr;
    if ((rc = step(Z, ring[(k + 1) % 3], ring[k % 3], nullptr, D2, 2 + k, true))) return rc;
  }
  return timed(h, kNewtonAux, 0.0, 0.0, s, [&] {
    return shp::launch_newton_final(j.xroot, j.xalt, fs, c, 2, s, max_out(h, j, j.xroot, nullptr));
  });
}

}  // namespace

int run_roots(shampoo_ctx* h, const RootJob& j, hipStream_t s) {
  if (j.fs.B == 0 || j.fs.n_groups == 0) return SHAMPOO_OK;
  switch (j.c.solver) {
    case shp::kNewtonDB:
      return newton_db(h, j, s);
    case shp::kChebyshev:
      return chebyshev(h, j, s);
    default:
      return newton(h, j, s);
  }
}

}  // namespace shp_rt
