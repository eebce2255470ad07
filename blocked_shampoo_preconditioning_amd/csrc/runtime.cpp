// Host runtime behind the C ABI of include/shampoo.h: block map, workspace
// plan, refresh schedule and the launch sequence of one step, all on the
// caller's stream. The library never allocates device memory: every device
// buffer lives in the caller's workspace.
#include "../../include/shampoo.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "kernels.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const std::string& msg) {
  g_last_error = msg;
  return code;
}

int hip_fail(hipError_t e, const char* where) {
  return fail(SHAMPOO_ERR_HIP, std::string(where) + ": " + hipGetErrorString(e));
}

#define HIP_CHECK(expr)                            \
  do {                                             \
    hipError_t e_ = (expr);                        \
    if (e_ != hipSuccess) return hip_fail(e_, #expr); \
  } while (0)

constexpr int64_t kAlign = 256;
int64_t align_up(int64_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

int pick_tile(int a, int b) {
  int g = a, h = b;
  while (h) {
    int t = g % h;
    g = h;
    h = t;
  }
  if (g % 128 == 0) return 128;
  if (g % 64 == 0) return 64;
  return 32;
}

// Layout of the caller's workspace (byte offsets, 256-byte aligned).
struct Plan {
  int64_t B = 0;
  int br = 0, bc = 0, n_mats = 0, tile = 32, max_iters = 1;
  int ntiles_l = 0, ntiles_r = 0, resid_stride = 0;
  int64_t fl = 0, fr = 0;  // elements of all left / right factors
  int64_t off_blocks, off_mats, off_umats, off_nreal, off_status, off_final, off_scale, off_rprev,
      off_cfac, off_active, off_flops, off_resid, off_gp, off_mom, off_lr, off_xroot, off_xalt,
      off_s0, off_s1, off_s2, off_cheb, total;
  bool momentum = false;
};

int validate_config(const shampoo_config_t* c) {
  if (!c) return fail(SHAMPOO_ERR_INVALID_ARG, "config is NULL");
  if (c->block_rows <= 0 || c->block_cols <= 0 || c->block_rows > 4096 || c->block_cols > 4096)
    return fail(SHAMPOO_ERR_INVALID_ARG, "block shape must be in 1..4096");
  if (c->block_rows % 32 || c->block_cols % 32)
    return fail(SHAMPOO_ERR_UNSUPPORTED, "block_rows and block_cols must be multiples of 32");
  if (!std::isfinite(c->beta2) || c->beta2 < 0.0 || c->beta2 > 1.0)
    return fail(SHAMPOO_ERR_INVALID_ARG, "beta2 must be in [0, 1]");
  if (!std::isfinite(c->stat_scale))
    return fail(SHAMPOO_ERR_INVALID_ARG, "stat_scale must be finite");
  if (!(c->eps > 0.0) || !std::isfinite(c->eps) || !((float)c->eps > 0.f))
    return fail(SHAMPOO_ERR_INVALID_ARG, "eps must be finite and > 0 in fp32");
  if (!std::isfinite(c->lr)) return fail(SHAMPOO_ERR_INVALID_ARG, "lr must be finite");
  if (c->root_every < 0) return fail(SHAMPOO_ERR_INVALID_ARG, "root_every must be >= 0");
  if (c->newton_max_iters < 1 || c->newton_max_iters > 64)
    return fail(SHAMPOO_ERR_INVALID_ARG, "newton_max_iters must be in 1..64");
  if (!std::isfinite(c->newton_tol))
    return fail(SHAMPOO_ERR_INVALID_ARG, "newton_tol must be finite");
  if (c->newton_scale_mode < 0 || c->newton_scale_mode > 2)
    return fail(SHAMPOO_ERR_UNSUPPORTED, "newton_scale_mode must be 0, 1 or 2");
  if (c->root_method != shp::kCoupledNewton && c->root_method != shp::kNewtonDB &&
      c->root_method != shp::kChebyshev)
    return fail(SHAMPOO_ERR_UNSUPPORTED,
                "root_method must be 0 (coupled Newton), 1 (Newton-DB) or 2 (Chebyshev)");
  if (c->root_method == shp::kChebyshev && (c->cheb_degree < 2 || c->cheb_degree > 1024))
    return fail(SHAMPOO_ERR_INVALID_ARG, "cheb_degree must be in 2..1024");
  if (!std::isfinite(c->momentum) || c->momentum < 0.0 || c->momentum >= 1.0)
    return fail(SHAMPOO_ERR_INVALID_ARG, "momentum must be in [0, 1)");
  if ((c->param_dtype != SHAMPOO_F32 && c->param_dtype != SHAMPOO_BF16) ||
      (c->grad_dtype != SHAMPOO_F32 && c->grad_dtype != SHAMPOO_BF16))
    return fail(SHAMPOO_ERR_UNSUPPORTED, "dtypes must be SHAMPOO_F32 or SHAMPOO_BF16");
  return SHAMPOO_OK;
}

int validate_mats(const shampoo_matrix_desc_t* m, int32_t n) {
  if (n < 0) return fail(SHAMPOO_ERR_INVALID_ARG, "n_mats must be >= 0");
  if (n > 0 && !m) return fail(SHAMPOO_ERR_INVALID_ARG, "matrix descriptors are NULL");
  for (int i = 0; i < n; ++i) {
    if (m[i].rows < 0 || m[i].cols < 0 || m[i].rows > (1 << 30) || m[i].cols > (1 << 30))
      return fail(SHAMPOO_ERR_INVALID_ARG, "matrix " + std::to_string(i) + ": bad shape");
    if (m[i].ld < m[i].cols || m[i].ld <= 0)
      return fail(SHAMPOO_ERR_INVALID_ARG, "matrix " + std::to_string(i) + ": ld < cols");
  }
  return SHAMPOO_OK;
}

Plan make_plan(const shampoo_config_t* c, const shampoo_matrix_desc_t* m, int32_t n) {
  Plan p;
  p.br = c->block_rows;
  p.bc = c->block_cols;
  p.n_mats = n;
  p.max_iters = c->newton_max_iters;
  for (int i = 0; i < n; ++i)
    p.B += ((m[i].rows + p.br - 1) / p.br) * ((m[i].cols + p.bc - 1) / p.bc);
  p.tile = pick_tile(p.br, p.bc);
  p.ntiles_l = shp::sym_tiles(p.br, p.tile);
  p.ntiles_r = shp::sym_tiles(p.bc, p.tile);
  p.resid_stride = std::max(p.ntiles_l, p.ntiles_r);
  p.fl = p.B * p.br * p.br;
  p.fr = p.B * p.bc * p.bc;
  const int64_t fbytes = (p.fl + p.fr) * 4;
  int64_t o = 0;
  auto take = [&](int64_t bytes) {
    const int64_t at = o;
    o = align_up(o + std::max<int64_t>(bytes, 1));
    return at;
  };
  p.off_blocks = take(p.B * (int64_t)sizeof(shp::BlockMeta));
  p.off_mats = take(n * (int64_t)sizeof(shp::MatMeta));
  p.off_umats = take(n * (int64_t)sizeof(shp::MatMeta));
  p.off_nreal = take(2 * p.B * 4);
  p.off_status = take(2 * p.B * 4);
  p.off_final = take(2 * p.B * 4);
  p.off_scale = take(2 * p.B * 4);
  p.off_rprev = take(2 * p.B * 4);
  p.off_cfac = take(2 * p.B * 4);
  p.off_active = take((int64_t)(p.max_iters + 1) * 2 * 4);
  p.off_flops = take(8);
  p.off_cheb = c->root_method == shp::kChebyshev
                   ? take(2 * p.B * (int64_t)(c->cheb_degree + 1) * 4 * 4)
                   : -1;
  p.off_resid = take(2 * p.B * p.resid_stride * 4);
  p.off_gp = take(p.B * p.br * p.bc * 4);
  p.momentum = c->momentum > 0.0;
  p.off_mom = p.momentum ? take(p.B * p.br * p.bc * 4) : -1;
  p.off_lr = take(fbytes);
  p.off_xroot = take(fbytes);
  p.off_xalt = take(fbytes);
  p.off_s0 = take(fbytes);
  p.off_s1 = take(fbytes);
  p.off_s2 = take(fbytes);
  p.total = o;
  return p;
}

enum { kPack = 0, kStats = 1, kNorms = 2, kNewtonGemm = 3, kNewtonAux = 4, kApply = 5 };

struct TimedLaunch {
  int cls;
  hipEvent_t start, stop;
  double flops, bytes;
};

}  // namespace

struct shampoo_ctx {
  shampoo_config_t cfg;
  Plan plan;
  char* ws = nullptr;
  std::vector<shampoo_matrix_desc_t> mats;
  std::vector<shp::BlockMeta> blocks;
  std::vector<shp::MatMeta> meta_host;   // what the device table holds
  bool meta_valid = false;
  hipEvent_t meta_copied = nullptr;      // the last upload of meta_host has finished
  int64_t t = 0;
  bool roots_valid = false;
  float stat_scale = 0.f;
  // timing
  bool timing = false;
  std::vector<TimedLaunch> timed;
  std::vector<hipEvent_t> event_pool;
  double newton_flops_base = 0.0;

  template <class T>
  T* at(int64_t off) const { return reinterpret_cast<T*>(ws + off); }
  float* gp() const { return at<float>(plan.off_gp); }
  float* mom() const { return plan.momentum ? at<float>(plan.off_mom) : nullptr; }
  float* lr() const { return at<float>(plan.off_lr); }
  float* xroot() const { return at<float>(plan.off_xroot); }
  float* xalt() const { return at<float>(plan.off_xalt); }
  float* s(int i) const {
    return at<float>(i == 0 ? plan.off_s0 : i == 1 ? plan.off_s1 : plan.off_s2);
  }
  float* gpT() const { return s(2); }   // packed transpose lives in Newton scratch
  float* tmpT() const { return s(1); }  // apply intermediate likewise

  shp::FactorSet factors() const {
    shp::FactorSet fs;
    fs.B = (int32_t)plan.B;
    fs.nl = plan.br;
    fs.nr = plan.bc;
    fs.offL = 0;
    fs.offR = plan.fl;
    fs.nreal = at<int32_t>(plan.off_nreal);
    return fs;
  }
  shp::NewtonCtl newton_ctl() const {
    shp::NewtonCtl c;
    c.solver = cfg.root_method;
    c.status = at<int32_t>(plan.off_status);
    c.final_iter = at<int32_t>(plan.off_final);
    c.scale = at<float>(plan.off_scale);
    c.rprev = at<float>(plan.off_rprev);
    c.cfac = at<float>(plan.off_cfac);
    c.resid = at<float>(plan.off_resid);
    c.resid_stride = plan.resid_stride;
    c.ntiles_l = plan.ntiles_l;
    c.ntiles_r = plan.ntiles_r;
    c.active_count = at<int32_t>(plan.off_active);
    c.flops_acc = at<double>(plan.off_flops);
    c.tol = (float)cfg.newton_tol;
    c.floor = 0.f;
    c.cheb = plan.off_cheb >= 0 ? at<float>(plan.off_cheb) : nullptr;
    c.degree = cfg.cheb_degree;
    c.max_iters = cfg.newton_max_iters;
    c.scale_mode = cfg.newton_scale_mode;
    return c;
  }

  hipEvent_t get_event() {
    if (!event_pool.empty()) {
      hipEvent_t e = event_pool.back();
      event_pool.pop_back();
      return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
  }
};

namespace {

// Run `launch` with HIP events around it when timing is enabled.
template <class F>
int timed(shampoo_ctx* h, int cls, double flops, double bytes, hipStream_t s, F&& launch) {
  hipEvent_t a = nullptr, b = nullptr;
  if (h->timing) {
    a = h->get_event();
    b = h->get_event();
    if (!a || !b) return fail(SHAMPOO_ERR_HIP, "hipEventCreate failed");
    HIP_CHECK(hipEventRecord(a, s));
  }
  hipError_t e = launch();
  if (e != hipSuccess) return hip_fail(e, "kernel launch");
  if (h->timing) {
    HIP_CHECK(hipEventRecord(b, s));
    h->timed.push_back({cls, a, b, flops, bytes});
  }
  return SHAMPOO_OK;
}

int upload_meta(shampoo_ctx* h, const void* const* grads, void* const* params, hipStream_t s) {
  const int n = h->plan.n_mats;
  std::vector<shp::MatMeta> m(n);
  for (int i = 0; i < n; ++i) {
    m[i].grad = grads ? grads[i] : (h->meta_valid ? h->meta_host[i].grad : nullptr);
    m[i].param = params ? params[i] : (h->meta_valid ? h->meta_host[i].param : nullptr);
    m[i].ld = h->mats[i].ld;
  }
  bool same = h->meta_valid && n == (int)h->meta_host.size();
  for (int i = 0; same && i < n; ++i)
    same = m[i].grad == h->meta_host[i].grad && m[i].param == h->meta_host[i].param;
  if (same) return SHAMPOO_OK;
  // the previous upload reads meta_host: let it finish before overwriting
  if (h->meta_copied) HIP_CHECK(hipEventSynchronize(h->meta_copied));
  h->meta_host = m;
  h->meta_valid = true;
  if (n) {
    HIP_CHECK(hipMemcpyAsync(h->at<void>(h->plan.off_mats), h->meta_host.data(),
                             n * sizeof(shp::MatMeta), hipMemcpyHostToDevice, s));
    if (!h->meta_copied) HIP_CHECK(hipEventCreateWithFlags(&h->meta_copied, hipEventDisableTiming));
    HIP_CHECK(hipEventRecord(h->meta_copied, s));
  }
  return SHAMPOO_OK;
}

int check_ptrs(const shampoo_ctx* h, const void* const* ptrs, int dtype, const char* what) {
  if (h->plan.n_mats > 0 && !ptrs) return fail(SHAMPOO_ERR_INVALID_ARG, std::string(what) + " is NULL");
  const uintptr_t align = dtype == SHAMPOO_BF16 ? 2 : 4;
  for (int i = 0; i < h->plan.n_mats; ++i) {
    const bool empty = h->mats[i].rows == 0 || h->mats[i].cols == 0;
    if (!ptrs[i] && !empty)
      return fail(SHAMPOO_ERR_INVALID_ARG, std::string(what) + "[" + std::to_string(i) + "] is NULL");
    if (reinterpret_cast<uintptr_t>(ptrs[i]) % align)
      return fail(SHAMPOO_ERR_MISALIGNED,
                  std::string(what) + "[" + std::to_string(i) + "] is not " + std::to_string(align) +
                      "-byte aligned");
  }
  return SHAMPOO_OK;
}

double sym_flops(double n, double k) { return n * (n + 1.0) * k; }

int do_pack(shampoo_ctx* h, hipStream_t s) {
  const Plan& p = h->plan;
  double real = 0.0;
  for (const auto& b : h->blocks) real += (double)b.m * b.n;
  const double esz = h->cfg.grad_dtype == SHAMPOO_BF16 ? 2.0 : 4.0;
  const double bytes = real * esz + (p.momentum ? 4.0 : 2.0) * 4.0 * (double)p.B * p.br * p.bc;
  return timed(h, kPack, 0.0, bytes, s, [&] {
    return shp::launch_pack(h->at<shp::BlockMeta>(p.off_blocks), h->at<shp::MatMeta>(p.off_mats),
                            (int32_t)p.B, p.br, p.bc, h->cfg.grad_dtype == SHAMPOO_BF16, h->gp(),
                            h->gpT(), h->mom(), (float)h->cfg.momentum, s);
  });
}

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
  g.beta = 0.f;
  g.gamma = 0.f;
  return g;
}

int do_stats(shampoo_ctx* h, hipStream_t s) {
  const Plan& p = h->plan;
  if (p.B == 0) return SHAMPOO_OK;
  shp::GemmLaunch g{};
  // L = beta2 L + g Gp Gp^T: C[m][n] = sum_k GpT[k][m] GpT[k][n]
  g.p[0] = sym_problem(h->gpT(), h->gpT(), h->lr(), (int64_t)p.bc * p.br, p.br, p.bc, (int)p.B);
  // R = beta2 R + g Gp^T Gp: C[m][n] = sum_k Gp[k][m] Gp[k][n]
  g.p[1] = sym_problem(h->gp(), h->gp(), h->lr() + p.fl, (int64_t)p.br * p.bc, p.bc, p.br, (int)p.B);
  for (int i = 0; i < 2; ++i) {
    g.p[i].alpha = h->stat_scale;
    g.p[i].beta = (float)h->cfg.beta2;
    g.p[i].D = g.p[i].C;  // EMA: reads the old statistic in place
    g.p[i].sD = g.p[i].sC;
  }
  g.n_problems = 2;
  double flops = 0.0;
  for (const auto& b : h->blocks) flops += sym_flops(b.m, b.n) + sym_flops(b.n, b.m);
  const double bytes = 4.0 * (double)p.B * (2.0 * p.br * p.bc + 2.0 * (double)p.br * p.br +
                                            2.0 * (double)p.bc * p.bc);
  return timed(h, kStats, flops, bytes, s, [&] { return shp::launch_gemm_sym(g, p.tile, false, s); });
}

// One batched symmetric product over all factors (left and right problems):
// C = alpha P Q + beta D + gamma I.
void factor_problems(const shampoo_ctx* h, shp::GemmLaunch& g, const float* P, const float* Q,
                     float* C, const float* D, float alpha, float beta, float gamma, bool resid) {
  const Plan& p = h->plan;
  const shp::NewtonCtl c = h->newton_ctl();
  auto add = [&](int64_t off, int n, int batch, int f0) {
    shp::GemmProblem q = sym_problem(P + off, Q + off, C + off, (int64_t)n * n, n, n, batch);
    q.alpha = alpha;
    q.beta = beta;
    q.gamma = gamma;
    if (D != nullptr) {
      q.D = D + off;
      q.sD = (int64_t)n * n;
    }
    q.status = c.status;
    q.f0 = f0;
    if (resid) {
      q.resid = c.resid;
      q.resid_stride = c.resid_stride;
    }
    g.p[g.n_problems++] = q;
  };
  if (p.br == p.bc) {
    add(0, p.br, (int)(2 * p.B), 0);
  } else {
    add(0, p.br, (int)p.B, 0);
    add(p.fl, p.bc, (int)p.B, (int)p.B);
  }
}

int do_refresh_db(shampoo_ctx* h, hipStream_t s);
int do_refresh_cheb(shampoo_ctx* h, int64_t t_stats, hipStream_t s);

// t_stats: the step whose statistics the roots are taken of (for the
// Chebyshev interval's lower end beta2^t eps).
int do_refresh(shampoo_ctx* h, hipStream_t s, int64_t t_stats) {
  const Plan& p = h->plan;
  if (p.B == 0) {
    h->roots_valid = true;
    return SHAMPOO_OK;
  }
  if (h->cfg.root_method == shp::kNewtonDB) return do_refresh_db(h, s);
  if (h->cfg.root_method == shp::kChebyshev) return do_refresh_cheb(h, t_stats, s);
  const shp::FactorSet fs = h->factors();
  const shp::NewtonCtl c = h->newton_ctl();
  double nbytes = 0.0;
  for (const auto& b : h->blocks) nbytes += 4.0 * ((double)b.m * b.m + (double)b.n * b.n);
  int rc = timed(h, kNorms, 0.0, nbytes, s, [&] { return shp::launch_norms(h->lr(), fs, c, s); });
  if (rc) return rc;
  rc = timed(h, kNewtonAux, 0.0, 0.0, s,
             [&] { return shp::launch_newton_init(h->lr(), h->s(0), h->xalt(), fs, c, s); });
  if (rc) return rc;
  int mi = 0;  // M_k lives in s(mi); T2 goes to s(1 - mi), T4 to s(2)
  for (int k = 0; k < h->cfg.newton_max_iters; ++k) {
    float* Mk = h->s(mi);
    float* T2 = h->s(1 - mi);
    float* T4 = h->s(2);
    float* Xcur = (k % 2 == 0) ? h->xroot() : h->xalt();
    float* Xnext = (k % 2 == 0) ? h->xalt() : h->xroot();
    // T = (5 I - M) / 4 enters through the affine epilogue:
    shp::GemmLaunch g1{};
    factor_problems(h, g1, Mk, Mk, T2, Mk, 0.0625f, -0.625f, 1.5625f, false);  // T2 = T T
    if (k > 0) factor_problems(h, g1, Xcur, Mk, Xnext, Xcur, -0.25f, 1.25f, 0.f, false);  // X T
    shp::GemmLaunch g2{};
    factor_problems(h, g2, T2, T2, T4, nullptr, 1.f, 0.f, 0.f, false);      // T4 = T2 T2
    shp::GemmLaunch g3{};
    factor_problems(h, g3, T4, Mk, T2, nullptr, 1.f, 0.f, 0.f, true);       // M' = T4 M
    rc = timed(h, kNewtonGemm, 0.0, 0.0, s, [&] { return shp::launch_gemm_sym(g1, p.tile, true, s); });
    if (rc) return rc;
    rc = timed(h, kNewtonGemm, 0.0, 0.0, s, [&] { return shp::launch_gemm_sym(g2, p.tile, true, s); });
    if (rc) return rc;
    rc = timed(h, kNewtonGemm, 0.0, 0.0, s, [&] { return shp::launch_gemm_sym(g3, p.tile, true, s); });
    if (rc) return rc;
    const int before = k == 0 ? 3 : 4;
    rc = timed(h, kNewtonAux, 0.0, 0.0, s,
               [&] { return shp::launch_newton_check(fs, c, k, 1, before, 0, s); });
    if (rc) return rc;
    mi = 1 - mi;
  }
  rc = timed(h, kNewtonAux, 0.0, 0.0, s,
             [&] { return shp::launch_newton_final(h->xroot(), h->xalt(), fs, c, 0, s); });
  if (rc) return rc;
  h->roots_valid = true;
  return SHAMPOO_OK;
}

// Newton-DB: two Denman-Beavers square-root stages in inverse-free form on
// the symmetric GEMM core. Y ping-pongs between S0 (even k) and S1 (odd), Z
// between Xroot and Xalt, M = Z Y goes to S2. Per iteration: M (with the
// residual partials), the check, then Y' = 3Y/2 - Y M/2 and Z' = 3Z/2 - M Z/2
// in one launch. Stage 2 restarts from stage 1's kept Y with Z = I; the root
// is s^(-1/4) times stage 2's kept Z.
int do_refresh_db(shampoo_ctx* h, hipStream_t s) {
  const Plan& p = h->plan;
  const shp::FactorSet fs = h->factors();
  const shp::NewtonCtl c = h->newton_ctl();
  double nbytes = 0.0;
  for (const auto& b : h->blocks) nbytes += 4.0 * ((double)b.m * b.m + (double)b.n * b.n);
  int rc = timed(h, kNorms, 0.0, nbytes, s, [&] { return shp::launch_norms(h->lr(), fs, c, s); });
  if (rc) return rc;
  rc = timed(h, kNewtonAux, 0.0, 0.0, s,
             [&] { return shp::launch_newton_init(h->lr(), h->s(0), h->xroot(), fs, c, s); });
  if (rc) return rc;
  const int kmax = h->cfg.newton_max_iters;
  for (int stage = 0; stage < 2; ++stage) {
    for (int k = 0; k <= kmax; ++k) {
      float* Y = h->s(k & 1);
      float* Z = (k & 1) ? h->xalt() : h->xroot();
      float* Yn = h->s((k + 1) & 1);
      float* Zn = ((k + 1) & 1) ? h->xalt() : h->xroot();
      shp::GemmLaunch g1{};
      factor_problems(h, g1, Z, Y, h->s(2), nullptr, 1.f, 0.f, 0.f, true);  // M = Z Y
      rc = timed(h, kNewtonGemm, 0.0, 0.0, s, [&] { return shp::launch_gemm_sym(g1, p.tile, true, s); });
      if (rc) return rc;
      const int after = k < kmax ? 2 : 0;
      rc = timed(h, kNewtonAux, 0.0, 0.0, s,
                 [&] { return shp::launch_newton_check(fs, c, k, 0, 1, after, s); });
      if (rc) return rc;
      if (k == kmax) break;
      shp::GemmLaunch g2{};
      factor_problems(h, g2, Y, h->s(2), Yn, Y, -0.5f, 1.5f, 0.f, false);  // Y (3I - M) / 2
      factor_problems(h, g2, h->s(2), Z, Zn, Z, -0.5f, 1.5f, 0.f, false);  // (3I - M) Z / 2
      rc = timed(h, kNewtonGemm, 0.0, 0.0, s, [&] { return shp::launch_gemm_sym(g2, p.tile, true, s); });
      if (rc) return rc;
    }
    if (stage == 0) {
      rc = timed(h, kNewtonAux, 0.0, 0.0, s, [&] {
        return shp::launch_db_stage2_init(h->s(0), h->s(1), h->xroot(), fs, c, s);
      });
      if (rc) return rc;
    }
  }
  rc = timed(h, kNewtonAux, 0.0, 0.0, s,
             [&] { return shp::launch_newton_final(h->xroot(), h->xalt(), fs, c, 1, s); });
  if (rc) return rc;
  h->roots_valid = true;
  return SHAMPOO_OK;
}

int do_refresh_cheb(shampoo_ctx* h, int64_t t_stats, hipStream_t s) {
  const Plan& p = h->plan;
  const shp::FactorSet fs = h->factors();
  shp::NewtonCtl c = h->newton_ctl();
  c.floor = (float)(std::pow(h->cfg.beta2, (double)t_stats) * h->cfg.eps);
  const int d = h->cfg.cheb_degree;
  double nbytes = 0.0;
  for (const auto& b : h->blocks) nbytes += 4.0 * ((double)b.m * b.m + (double)b.n * b.n);
  int rc = timed(h, kNorms, 0.0, nbytes, s, [&] { return shp::launch_norms(h->lr(), fs, c, s); });
  if (rc) return rc;
  // Ahat = A / s in Xalt (identity on tail padding); then the coefficients
  // (which mark every factor as a fixed-degree result); B_d, B_(d-1) in S0, S1
  rc = timed(h, kNewtonAux, 0.0, 0.0, s,
             [&] { return shp::launch_newton_init(h->lr(), h->xalt(), nullptr, fs, c, s); });
  if (rc) return rc;
  rc = timed(h, kNewtonAux, 0.0, 0.0, s, [&] { return shp::launch_cheb_setup(fs, c, s); });
  if (rc) return rc;
  rc = timed(h, kNewtonAux, 0.0, 0.0, s,
             [&] { return shp::launch_cheb_init(h->xalt(), h->s(0), h->s(1), fs, c, s); });
  if (rc) return rc;
  double fprod = 0.0;
  for (const auto& b : h->blocks)
    fprod += (double)b.m * b.m * (b.m + 1.0) + (double)b.n * b.n * (b.n + 1.0);
  // B_k = a Ahat B_(k+1) + b B_(k+1) - B_(k+2) + c_k I, buffer of B_k: S[(d - k) % 3];
  // the last product (k = 0) forms p into Xroot
  for (int k = d - 2; k >= 0; --k) {
    float* Bk1 = h->s((d - k - 1) % 3);
    float* Bk2 = h->s((d - k - 2) % 3);
    float* Bk = k == 0 ? h->xroot() : h->s((d - k) % 3);
    shp::GemmLaunch g{};
    factor_problems(h, g, h->xalt(), Bk1, Bk, Bk1, 1.f, 0.f, 0.f, false);
    for (int i = 0; i < g.n_problems; ++i) {
      g.p[i].D2 = Bk2 + (g.p[i].D - Bk1);
      g.p[i].sD2 = g.p[i].sD;
      g.p[i].status = nullptr;  // every factor runs the whole recurrence
      g.p[i].coef = c.cheb + (size_t)k * 4;
      g.p[i].coef_stride = (d + 1) * 4;
    }
    rc = timed(h, kNewtonGemm, fprod, 0.0, s, [&] { return shp::launch_gemm_sym(g, p.tile, true, s); });
    if (rc) return rc;
  }
  rc = timed(h, kNewtonAux, 0.0, 0.0, s,
             [&] { return shp::launch_newton_final(h->xroot(), h->xalt(), fs, c, 2, s); });
  if (rc) return rc;
  h->roots_valid = true;
  return SHAMPOO_OK;
}

int do_apply(shampoo_ctx* h, hipStream_t s, float* out_packed) {
  const Plan& p = h->plan;
  if (p.B == 0) return SHAMPOO_OK;
  // TmpT[m][n] = sum_k Gp[k][m] X_L[k][n]   (= (X_L Gp)^T, bc x br); with
  // momentum the preconditioned matrix is the momentum buffer
  shp::GemmLaunch g1{};
  shp::GemmProblem a{};
  a.P = p.momentum ? h->mom() : h->gp();
  a.sP = (int64_t)p.br * p.bc;
  a.Q = h->xroot();
  a.sQ = (int64_t)p.br * p.br;
  a.C = h->tmpT();
  a.sC = (int64_t)p.bc * p.br;
  a.M = p.bc;
  a.N = p.br;
  a.K = p.br;
  a.batch = (int)p.B;
  a.alpha = 1.f;
  g1.p[0] = a;
  g1.n_problems = 1;
  // U[m][n] = sum_k TmpT[k][m] X_R[k][n]   (= X_L Gp X_R, br x bc)
  shp::GemmLaunch g2{};
  shp::GemmProblem b{};
  b.P = h->tmpT();
  b.sP = (int64_t)p.bc * p.br;
  b.Q = h->xroot() + p.fl;
  b.sQ = (int64_t)p.bc * p.bc;
  b.C = nullptr;
  b.M = p.br;
  b.N = p.bc;
  b.K = p.bc;
  b.batch = (int)p.B;
  b.alpha = 1.f;
  g2.p[0] = b;
  g2.n_problems = 1;
  shp::UpdateArgs u{};
  u.blocks = h->at<shp::BlockMeta>(p.off_blocks);
  u.mats = h->at<shp::MatMeta>(p.off_mats);
  u.lr = (float)h->cfg.lr;
  u.param_bf16 = h->cfg.param_dtype == SHAMPOO_BF16;
  u.out_packed = out_packed;
  double f1 = 0.0, f2 = 0.0;
  for (const auto& bl : h->blocks) {
    f1 += 2.0 * bl.m * bl.m * (double)bl.n;
    f2 += 2.0 * bl.m * (double)bl.n * bl.n;
  }
  int rc = timed(h, kApply, f1, 0.0, s, [&] { return shp::launch_gemm_full(g1, p.tile, s); });
  if (rc) return rc;
  return timed(h, kApply, f2, 0.0, s, [&] { return shp::launch_gemm_update(g2, u, p.tile, s); });
}

}  // namespace

// ===========================================================================
// C ABI
// ===========================================================================
extern "C" {

int shampoo_config_default(shampoo_config_t* cfg) {
  if (!cfg) return fail(SHAMPOO_ERR_INVALID_ARG, "config is NULL");
  cfg->block_rows = 1024;
  cfg->block_cols = 1024;
  cfg->beta2 = 0.999;
  cfg->stat_scale = -1.0;
  cfg->eps = 1e-6;
  cfg->lr = 1e-3;
  cfg->root_every = 10;
  cfg->newton_max_iters = 25;
  cfg->newton_tol = 1e-6;
  cfg->newton_scale_mode = 2;
  cfg->param_dtype = SHAMPOO_F32;
  cfg->grad_dtype = SHAMPOO_F32;
  cfg->momentum = 0.0;
  cfg->root_method = shp::kCoupledNewton;
  cfg->cheb_degree = 128;
  return SHAMPOO_OK;
}

int shampoo_workspace_size(const shampoo_config_t* cfg, const shampoo_matrix_desc_t* mats,
                           int32_t n_mats, size_t* bytes_out) {
  int rc = validate_config(cfg);
  if (rc) return rc;
  rc = validate_mats(mats, n_mats);
  if (rc) return rc;
  if (!bytes_out) return fail(SHAMPOO_ERR_INVALID_ARG, "bytes_out is NULL");
  *bytes_out = (size_t)make_plan(cfg, mats, n_mats).total;
  return SHAMPOO_OK;
}

int shampoo_init(const shampoo_config_t* cfg, const shampoo_matrix_desc_t* mats, int32_t n_mats,
                 void* workspace, size_t workspace_bytes, void* hip_stream, shampoo_t* out) {
  int rc = validate_config(cfg);
  if (rc) return rc;
  rc = validate_mats(mats, n_mats);
  if (rc) return rc;
  if (!out) return fail(SHAMPOO_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  if (!workspace) return fail(SHAMPOO_ERR_INVALID_ARG, "workspace is NULL");
  if (reinterpret_cast<uintptr_t>(workspace) % kAlign)
    return fail(SHAMPOO_ERR_MISALIGNED, "workspace is not 256-byte aligned");
  const Plan plan = make_plan(cfg, mats, n_mats);
  if ((int64_t)workspace_bytes < plan.total)
    return fail(SHAMPOO_ERR_WORKSPACE_TOO_SMALL,
                "workspace has " + std::to_string(workspace_bytes) + " bytes, needs " +
                    std::to_string(plan.total));
  if (plan.B > (int64_t)1 << 28) return fail(SHAMPOO_ERR_UNSUPPORTED, "too many blocks");
  shampoo_ctx* h = new (std::nothrow) shampoo_ctx();
  if (!h) return fail(SHAMPOO_ERR_INVALID_ARG, "out of host memory");
  h->cfg = *cfg;
  h->plan = plan;
  h->ws = static_cast<char*>(workspace);
  h->mats.assign(mats, mats + n_mats);
  h->stat_scale = (float)(cfg->stat_scale < 0.0 ? 1.0 - cfg->beta2 : cfg->stat_scale);
  // block map: matrices in registration order, row-major blocks inside each
  std::vector<int32_t> nreal;
  for (int i = 0; i < n_mats; ++i) {
    const int64_t nbr = (mats[i].rows + plan.br - 1) / plan.br;
    const int64_t nbc = (mats[i].cols + plan.bc - 1) / plan.bc;
    for (int64_t bi = 0; bi < nbr; ++bi)
      for (int64_t bj = 0; bj < nbc; ++bj) {
        shp::BlockMeta b;
        b.mat = i;
        b.r0 = (int32_t)(bi * plan.br);
        b.c0 = (int32_t)(bj * plan.bc);
        b.m = (int32_t)std::min<int64_t>(plan.br, mats[i].rows - b.r0);
        b.n = (int32_t)std::min<int64_t>(plan.bc, mats[i].cols - b.c0);
        b.pad_ = 0;
        h->blocks.push_back(b);
      }
  }
  nreal.resize(2 * plan.B);
  for (int64_t b = 0; b < plan.B; ++b) {
    nreal[b] = h->blocks[b].m;
    nreal[plan.B + b] = h->blocks[b].n;
  }
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  auto cleanup = [&](int code) {
    delete h;
    return code;
  };
  hipError_t e = hipSuccess;
  if (plan.B) {
    e = hipMemcpyAsync(h->at<void>(plan.off_blocks), h->blocks.data(),
                       plan.B * sizeof(shp::BlockMeta), hipMemcpyHostToDevice, s);
    if (e == hipSuccess)
      e = hipMemcpyAsync(h->at<void>(plan.off_nreal), nreal.data(), nreal.size() * 4,
                         hipMemcpyHostToDevice, s);
    if (e == hipSuccess) e = hipMemsetAsync(h->at<void>(plan.off_status), 0, 2 * plan.B * 4, s);
    if (e == hipSuccess) e = hipMemsetAsync(h->at<void>(plan.off_final), 0, 2 * plan.B * 4, s);
    if (e == hipSuccess) e = hipMemsetAsync(h->at<void>(plan.off_scale), 0, 2 * plan.B * 4, s);
    if (e == hipSuccess) e = hipMemsetAsync(h->at<void>(plan.off_flops), 0, 8, s);
    if (e == hipSuccess && plan.momentum)
      e = hipMemsetAsync(h->at<void>(plan.off_mom), 0, plan.B * plan.br * plan.bc * 4, s);
    if (e == hipSuccess)
      e = shp::launch_init_state(h->lr(), plan.fl, plan.br, plan.fr, plan.bc, (int32_t)plan.B,
                                 (float)cfg->eps, s);
    // the host copies above are from pageable memory; make sure they are done
    // before the temporaries go away
    if (e == hipSuccess) e = hipStreamSynchronize(s);
  }
  if (e != hipSuccess) return cleanup(hip_fail(e, "shampoo_init"));
  *out = h;
  return SHAMPOO_OK;
}

int shampoo_step(shampoo_t h, void* const* params, const void* const* grads, uint32_t flags,
                 void* hip_stream) {
  if (!h) return fail(SHAMPOO_ERR_INVALID_ARG, "handle is NULL");
  int rc = check_ptrs(h, params, h->cfg.param_dtype, "params");
  if (rc) return rc;
  rc = check_ptrs(h, grads, h->cfg.grad_dtype, "grads");
  if (rc) return rc;
  const int64_t t = h->t + 1;
  const int k = h->cfg.root_every;
  bool refresh = (flags & SHAMPOO_FORCE_REFRESH) != 0;
  if (!refresh && !(flags & SHAMPOO_NO_AUTO_REFRESH))
    refresh = (k > 0 && (t - 1) % k == 0) || (!h->roots_valid && k > 0);
  if (!refresh && !h->roots_valid)
    return fail(SHAMPOO_ERR_NO_ROOTS, "no roots yet: pass SHAMPOO_FORCE_REFRESH or call "
                                      "shampoo_refresh_roots first");
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  rc = upload_meta(h, grads, params, s);
  if (rc) return rc;
  if ((rc = do_pack(h, s))) return rc;
  if ((rc = do_stats(h, s))) return rc;
  if (refresh && (rc = do_refresh(h, s, t))) return rc;
  if ((rc = do_apply(h, s, nullptr))) return rc;
  h->t = t;
  return SHAMPOO_OK;
}

int shampoo_refresh_roots(shampoo_t h, void* hip_stream) {
  if (!h) return fail(SHAMPOO_ERR_INVALID_ARG, "handle is NULL");
  return do_refresh(h, static_cast<hipStream_t>(hip_stream), h->t);
}

int shampoo_destroy(shampoo_t h) {
  if (!h) return fail(SHAMPOO_ERR_INVALID_ARG, "handle is NULL");
  for (auto& r : h->timed) {
    (void)hipEventDestroy(r.start);
    (void)hipEventDestroy(r.stop);
  }
  for (auto e : h->event_pool) (void)hipEventDestroy(e);
  if (h->meta_copied) (void)hipEventDestroy(h->meta_copied);
  delete h;
  return SHAMPOO_OK;
}

int shampoo_state_layout(shampoo_t h, shampoo_layout_t* out) {
  if (!h || !out) return fail(SHAMPOO_ERR_INVALID_ARG, "NULL argument");
  out->n_blocks = h->plan.B;
  out->grad_packed = h->plan.off_gp;
  out->stats = h->plan.off_lr;
  out->roots = h->plan.off_xroot;
  out->newton_status = h->plan.off_status;
  out->newton_iters = h->plan.off_final;
  out->newton_scale = h->plan.off_scale;
  out->newton_residual = h->plan.off_rprev;
  out->momentum = h->plan.off_mom;
  out->workspace_bytes = h->plan.total;
  return SHAMPOO_OK;
}

int shampoo_get_step(shampoo_t h, int64_t* t_out) {
  if (!h || !t_out) return fail(SHAMPOO_ERR_INVALID_ARG, "NULL argument");
  *t_out = h->t;
  return SHAMPOO_OK;
}

int shampoo_set_step(shampoo_t h, int64_t t) {
  if (!h || t < 0) return fail(SHAMPOO_ERR_INVALID_ARG, "NULL handle or negative step");
  h->t = t;
  return SHAMPOO_OK;
}

int shampoo_pack(shampoo_t h, const void* const* grads, void* hip_stream) {
  if (!h) return fail(SHAMPOO_ERR_INVALID_ARG, "handle is NULL");
  int rc = check_ptrs(h, grads, h->cfg.grad_dtype, "grads");
  if (rc) return rc;
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  rc = upload_meta(h, grads, nullptr, s);
  if (rc) return rc;
  return do_pack(h, s);
}

int shampoo_unpack(shampoo_t h, void* const* dst, void* hip_stream) {
  if (!h) return fail(SHAMPOO_ERR_INVALID_ARG, "handle is NULL");
  int rc = check_ptrs(h, dst, SHAMPOO_F32, "dst");
  if (rc) return rc;
  const Plan& p = h->plan;
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  std::vector<shp::MatMeta> m(p.n_mats);
  for (int i = 0; i < p.n_mats; ++i) {
    m[i].grad = nullptr;
    m[i].param = dst[i];
    m[i].ld = h->mats[i].ld;
  }
  if (p.n_mats) {
    HIP_CHECK(hipMemcpyAsync(h->at<void>(p.off_umats), m.data(), m.size() * sizeof(shp::MatMeta),
                             hipMemcpyHostToDevice, s));
  }
  HIP_CHECK(shp::launch_unpack(h->at<shp::BlockMeta>(p.off_blocks), h->at<shp::MatMeta>(p.off_umats),
                               (int32_t)p.B, p.br, p.bc, h->gp(), s));
  // the descriptor copy is from pageable host memory that dies here
  HIP_CHECK(hipStreamSynchronize(s));
  return SHAMPOO_OK;
}

int shampoo_precondition(shampoo_t h, void* out, void* hip_stream) {
  if (!h) return fail(SHAMPOO_ERR_INVALID_ARG, "handle is NULL");
  if (!out && h->plan.B) return fail(SHAMPOO_ERR_INVALID_ARG, "out is NULL");
  if (reinterpret_cast<uintptr_t>(out) % 16) return fail(SHAMPOO_ERR_MISALIGNED, "out not 16-byte aligned");
  if (!h->roots_valid) return fail(SHAMPOO_ERR_NO_ROOTS, "no roots yet");
  return do_apply(h, static_cast<hipStream_t>(hip_stream), static_cast<float*>(out));
}

int shampoo_get_status(shampoo_t h, void* hip_stream, int32_t* n_diverged_out) {
  if (!h || !n_diverged_out) return fail(SHAMPOO_ERR_INVALID_ARG, "NULL argument");
  const Plan& p = h->plan;
  std::vector<int32_t> st(2 * p.B);
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  if (p.B) {
    HIP_CHECK(hipMemcpyAsync(st.data(), h->at<void>(p.off_status), st.size() * 4,
                             hipMemcpyDeviceToHost, s));
  }
  HIP_CHECK(hipStreamSynchronize(s));
  int32_t n = 0;
  for (int32_t v : st) n += v == 3;
  *n_diverged_out = n;
  return SHAMPOO_OK;
}

int shampoo_set_timing(shampoo_t h, int32_t enable, void* hip_stream) {
  if (!h) return fail(SHAMPOO_ERR_INVALID_ARG, "handle is NULL");
  for (auto& r : h->timed) {
    h->event_pool.push_back(r.start);
    h->event_pool.push_back(r.stop);
  }
  h->timed.clear();
  h->timing = enable != 0;
  if (h->timing)
    HIP_CHECK(hipMemsetAsync(h->at<void>(h->plan.off_flops), 0, 8,
                             static_cast<hipStream_t>(hip_stream)));
  return SHAMPOO_OK;
}

int shampoo_get_timing(shampoo_t h, shampoo_timing_t* out) {
  if (!h || !out) return fail(SHAMPOO_ERR_INVALID_ARG, "NULL argument");
  std::memset(out, 0, sizeof(*out));
  for (auto& r : h->timed) {
    HIP_CHECK(hipEventSynchronize(r.stop));
    float ms = 0.f;
    HIP_CHECK(hipEventElapsedTime(&ms, r.start, r.stop));
    out->ms[r.cls] += ms;
    out->flops[r.cls] += r.flops;
    out->bytes[r.cls] += r.bytes;
    out->launches[r.cls] += 1;
  }
  // Newton flops depend on how many factors were still iterating; the check
  // kernels accumulate them on the device (all of them ran before the last
  // recorded event).
  double nf = 0.0;
  HIP_CHECK(hipMemcpy(&nf, h->at<void>(h->plan.off_flops), sizeof(double), hipMemcpyDeviceToHost));
  out->flops[kNewtonGemm] += nf;  // the Chebyshev products are counted on the host
  return SHAMPOO_OK;
}

const char* shampoo_status_string(int status) {
  switch (status) {
    case SHAMPOO_OK: return "ok";
    case SHAMPOO_ERR_INVALID_ARG: return "invalid argument";
    case SHAMPOO_ERR_UNSUPPORTED: return "unsupported";
    case SHAMPOO_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case SHAMPOO_ERR_MISALIGNED: return "misaligned pointer or leading dimension";
    case SHAMPOO_ERR_NO_ROOTS: return "no roots computed yet";
    case SHAMPOO_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* shampoo_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
