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
#include "runtime_common.h"

namespace shp_rt {

thread_local std::string g_last_error;

int fail(int code, const std::string& msg) {
  g_last_error = msg;
  return code;
}

int hip_fail(hipError_t e, const char* where) {
  return fail(SHAMPOO_ERR_HIP, std::string(where) + ": " + hipGetErrorString(e));
}

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

// tensor: the block shape comes with the tensor descriptors, block_rows /
// block_cols are not read
int validate_config(const shampoo_config_t* c, bool tensor) {
  if (!c) return fail(SHAMPOO_ERR_INVALID_ARG, "config is NULL");
  if (!tensor && (c->block_rows <= 0 || c->block_cols <= 0 || c->block_rows > 4096 ||
                  c->block_cols > 4096))
    return fail(SHAMPOO_ERR_INVALID_ARG, "block shape must be in 1..4096");
  if (!tensor && (c->block_rows % 32 || c->block_cols % 32))
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
  if (c->newton_scale_mode < 0 || c->newton_scale_mode > 3)
    return fail(SHAMPOO_ERR_UNSUPPORTED, "newton_scale_mode must be 0, 1, 2 or 3");
  if (c->root_method != shp::kCoupledNewton && c->root_method != shp::kNewtonDB &&
      c->root_method != shp::kChebyshev)
    return fail(SHAMPOO_ERR_UNSUPPORTED,
                "root_method must be 0 (coupled Newton), 1 (Newton-DB) or 2 (Chebyshev)");
  if (c->root_method == shp::kChebyshev && (c->cheb_degree < 2 || c->cheb_degree > 1024))
    return fail(SHAMPOO_ERR_INVALID_ARG, "cheb_degree must be in 2..1024");
  if (c->fp32_gemm != SHAMPOO_GEMM_F32 && c->fp32_gemm != SHAMPOO_GEMM_SPLIT_BF16 &&
      c->fp32_gemm != SHAMPOO_GEMM_SPLIT_F16)
    return fail(SHAMPOO_ERR_INVALID_ARG,
                "fp32_gemm must be 0 (fp32 MFMA), 1 (split bf16) or 2 (split fp16)");
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
    // the parameter update addresses 32 rows of a block from one base with
    // 32-bit element offsets
    if (m[i].ld > (int64_t{1} << 26))
      return fail(SHAMPOO_ERR_INVALID_ARG, "matrix " + std::to_string(i) + ": ld > 2^26");
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
  // (a 256-wide block would be one diagonal tile: 128-tiles balance it better)
  p.sym_tile = c->fp32_gemm == SHAMPOO_GEMM_SPLIT_F16 && p.br % 256 == 0 && p.bc % 256 == 0 &&
                       p.br >= 512 && p.bc >= 512
                   ? 256 : p.tile;
  p.bf16_tile = p.br % 256 == 0 && p.bc % 256 == 0 && p.br >= 512 && p.bc >= 512 ? 256 : p.tile;
  p.ntiles_l = shp::sym_tiles(p.br, p.sym_tile);
  p.ntiles_r = shp::sym_tiles(p.bc, p.sym_tile);
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
  p.off_lo = take(2 * p.B * 4);
  p.off_coef = take(2 * p.B * shp::kCoefRecord * 4);
  p.off_active = take((int64_t)(p.max_iters + 1) * shp::kMaxGroups * 4);
  p.off_flops = take(8);
  p.off_cheb = c->root_method == shp::kChebyshev
                   ? take(2 * p.B * (int64_t)shp::cheb_floats(c->cheb_degree) * 4)
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
  p.off_s3 = c->root_method == shp::kChebyshev ? take(fbytes) : -1;  // the giant steps' third buffer
  p.off_mx = c->fp32_gemm == SHAMPOO_GEMM_SPLIT_F16 ? take((6 * 2 * p.B + 3 * p.B) * 8) : -1;
  p.total = o;
  return p;
}

}  // namespace shp_rt

hipEvent_t shampoo_ctx::get_event() {
  if (!event_pool.empty()) {
    hipEvent_t e = event_pool.back();
    event_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

namespace shp_rt {
namespace {

// Matrix-handle buffers inside the workspace.
float* m_gp(const shampoo_ctx* h) { return h->at<float>(h->plan.off_gp); }
float* m_mom(const shampoo_ctx* h) {
  return h->plan.momentum ? h->at<float>(h->plan.off_mom) : nullptr;
}
float* m_lr(const shampoo_ctx* h) { return h->at<float>(h->plan.off_lr); }
float* m_xroot(const shampoo_ctx* h) { return h->at<float>(h->plan.off_xroot); }
float* m_xalt(const shampoo_ctx* h) { return h->at<float>(h->plan.off_xalt); }
float* m_s(const shampoo_ctx* h, int i) {
  return h->at<float>(i == 0 ? h->plan.off_s0 : i == 1 ? h->plan.off_s1 : h->plan.off_s2);
}
float* m_gpT(const shampoo_ctx* h) { return m_s(h, 2); }   // packed transpose lives in Newton scratch
// bf16 gradients: the packed block and its transpose as bf16 (statistics on the
// bf16 MFMA), in the same scratch
bool m_bf16_stats(const shampoo_ctx* h) { return h->cfg.grad_dtype == SHAMPOO_BF16; }
uint16_t* m_gpH(const shampoo_ctx* h) { return reinterpret_cast<uint16_t*>(m_s(h, 2)); }
uint16_t* m_gpTH(const shampoo_ctx* h) { return m_gpH(h) + h->plan.B * h->plan.br * h->plan.bc; }
float* m_tmpT(const shampoo_ctx* h) { return m_s(h, 1); }  // apply intermediate likewise
// fp16 split products: maximum words per factor of xroot, xalt, s0, s1, s2,
// s3 (i = 0..5), then per block of Gp, the momentum buffer and the apply
// intermediate (i = 6, 7, 8); NULL on the other paths
bool m_f16(const shampoo_ctx* h) { return h->cfg.fp32_gemm == SHAMPOO_GEMM_SPLIT_F16; }
uint64_t* m_mx(const shampoo_ctx* h, int i) {
  if (h->plan.off_mx < 0) return nullptr;
  const int64_t B = h->plan.B;
  return h->at<uint64_t>(h->plan.off_mx) + (i < 6 ? i * 2 * B : 12 * B + (i - 6) * B);
}

shp::FactorSet m_factors(const shampoo_ctx* h) {
  const Plan& plan = h->plan;
  shp::FactorSet fs{};
  fs.B = (int32_t)plan.B;
  fs.n_groups = 2;
  fs.side[0] = plan.br;
  fs.side[1] = plan.bc;
  fs.off[0] = 0;
  fs.off[1] = plan.fl;
  fs.nreal = h->at<int32_t>(plan.off_nreal);
  return fs;
}

shp::NewtonCtl m_ctl(const shampoo_ctx* h) {
  const Plan& plan = h->plan;
  const shampoo_config_t& cfg = h->cfg;
  shp::NewtonCtl c{};
  c.solver = cfg.root_method;
  c.status = h->at<int32_t>(plan.off_status);
  c.final_iter = h->at<int32_t>(plan.off_final);
  c.scale = h->at<float>(plan.off_scale);
  c.rprev = h->at<float>(plan.off_rprev);
  c.cfac = h->at<float>(plan.off_cfac);
  c.resid = h->at<float>(plan.off_resid);
  c.resid_stride = plan.resid_stride;
  c.ntiles[0] = plan.ntiles_l;
  c.ntiles[1] = plan.ntiles_r;
  c.active_count = h->at<int32_t>(plan.off_active);
  c.flops_acc = h->at<double>(plan.off_flops);
  c.tol = (float)cfg.newton_tol;
  c.floor = 0.f;
  c.cheb = plan.off_cheb >= 0 ? h->at<float>(plan.off_cheb) : nullptr;
  c.degree = cfg.cheb_degree;
  c.max_iters = cfg.newton_max_iters;
  c.scale_mode = cfg.newton_scale_mode;
  c.p = 4;
  c.lo = h->at<float>(plan.off_lo);
  c.coef = h->at<float>(plan.off_coef);
  return c;
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
  // the table travels in kernel arguments: nothing to wait for
  HIP_CHECK(shp::launch_upload(h->at<void>(h->plan.off_mats), m.data(), n * sizeof(shp::MatMeta), s));
  h->meta_host = m;
  h->meta_valid = true;
  return SHAMPOO_OK;
}

}  // namespace

int check_ptrs(const shampoo_ctx* h, const void* const* ptrs, int dtype, const char* what) {
  const int n = (int)h->empty_item.size();
  if (n > 0 && !ptrs) return fail(SHAMPOO_ERR_INVALID_ARG, std::string(what) + " is NULL");
  const uintptr_t align = dtype == SHAMPOO_BF16 ? 2 : 4;
  for (int i = 0; i < n; ++i) {
    const bool empty = h->empty_item[i] != 0;
    if (!ptrs[i] && !empty)
      return fail(SHAMPOO_ERR_INVALID_ARG, std::string(what) + "[" + std::to_string(i) + "] is NULL");
    if (reinterpret_cast<uintptr_t>(ptrs[i]) % align)
      return fail(SHAMPOO_ERR_MISALIGNED,
                  std::string(what) + "[" + std::to_string(i) + "] is not " + std::to_string(align) +
                      "-byte aligned");
  }
  return SHAMPOO_OK;
}

namespace {

double sym_flops(double n, double k) { return n * (n + 1.0) * k; }

int do_pack(shampoo_ctx* h, hipStream_t s) {
  const Plan& p = h->plan;
  double real = 0.0;
  for (const auto& b : h->blocks) real += (double)b.m * b.n;
  const double esz = h->cfg.grad_dtype == SHAMPOO_BF16 ? 2.0 : 4.0;
  const bool hb = m_bf16_stats(h);
  // the fp32 transpose feeds the fp32-MFMA statistics only (the split path
  // reads the packed block by rows and by columns)
  const bool want_t = !hb && h->cfg.fp32_gemm == SHAMPOO_GEMM_F32;
  const double fp32_copies = 1.0 + (want_t ? 1.0 : 0.0) + (p.momentum ? 2.0 : 0.0);
  const double bytes = real * esz + fp32_copies * 4.0 * (double)p.B * p.br * p.bc +
                       (hb ? 2.0 * 2.0 * (double)p.B * p.br * p.bc : 0.0);
  shp::MaxOut mo{};
  if (m_f16(h)) {
    mo.a = m_mx(h, 6);
    mo.b = p.momentum ? m_mx(h, 7) : nullptr;
    mo.ver = h->next_ver();
  }
  return timed(h, kPack, 0.0, bytes, s, [&] {
    return shp::launch_pack(h->at<shp::BlockMeta>(p.off_blocks), h->at<shp::MatMeta>(p.off_mats),
                            (int32_t)p.B, p.br, p.bc, h->cfg.grad_dtype == SHAMPOO_BF16, m_gp(h),
                            want_t ? m_gpT(h) : nullptr, m_mom(h), (float)h->cfg.momentum,
                            hb ? m_gpH(h) : nullptr, hb ? m_gpTH(h) : nullptr, s, mo);
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
  // fp32 MFMA: C = P^T Q, so L = beta2 L + g Gp Gp^T reads P = Q = GpT and
  // R = beta2 R + g Gp^T Gp reads P = Q = Gp. Split path: C = A A^T with
  // A = Gp read by rows for L and by columns for R (Gp stored [K = br][M = bc]).
  const bool split = h->cfg.fp32_gemm != SHAMPOO_GEMM_F32;
  float* opL = split ? m_gp(h) : m_gpT(h);
  g.p[0] = sym_problem(opL, opL, m_lr(h), (int64_t)p.bc * p.br, p.br, p.bc, (int)p.B);
  g.p[1] = sym_problem(m_gp(h), m_gp(h), m_lr(h) + p.fl, (int64_t)p.br * p.bc, p.bc, p.br, (int)p.B);
  g.p[1].p_cols = g.p[1].q_cols = split ? 1 : 0;
  for (int i = 0; i < 2; ++i) {
    g.p[i].alpha = h->stat_scale;
    g.p[i].beta = (float)h->cfg.beta2;
    g.p[i].D = g.p[i].C;  // EMA: reads the old statistic in place
    g.p[i].sD = g.p[i].sC;
    g.p[i].mP = g.p[i].mQ = m_mx(h, 6);  // fp16 split: the packed blocks' maxima
  }
  g.n_problems = 2;
  const bool hb = m_bf16_stats(h);
  if (hb) {
    // bf16 operands, k contiguous: L from the rows of Gp, R from the rows of Gp^T
    g.p[0].Xh = m_gpH(h);
    g.p[0].sXh = (int64_t)p.br * p.bc;
    g.p[1].Xh = m_gpTH(h);
    g.p[1].sXh = (int64_t)p.br * p.bc;
  }
  double flops = 0.0;
  for (const auto& b : h->blocks) flops += sym_flops(b.m, b.n) + sym_flops(b.n, b.m);
  const double bytes = (double)p.B * ((hb ? 2.0 : 4.0) * 2.0 * p.br * p.bc +
                                      4.0 * (2.0 * (double)p.br * p.br + 2.0 * (double)p.bc * p.bc));
  return timed(h, kStats, flops, bytes, s, [&] {
    return hb ? shp::launch_gemm_sym_bf16(g, p.bf16_tile, s)
              : shp::launch_gemm_sym(g, p.sym_tile, false, h->cfg.fp32_gemm, s);
  });
}

// t_stats: the step whose statistics the roots are taken of (for the
// Chebyshev interval's lower end beta2^t eps).
int do_refresh(shampoo_ctx* h, hipStream_t s, int64_t t_stats) {
  const Plan& p = h->plan;
  if (p.B == 0) {
    h->roots_valid = true;
    return SHAMPOO_OK;
  }
  RootJob j;
  j.fs = m_factors(h);
  j.c = m_ctl(h);
  j.A = m_lr(h);
  j.xroot = m_xroot(h);
  j.xalt = m_xalt(h);
  for (int i = 0; i < 3; ++i) j.s[i] = m_s(h, i);
  j.s[3] = p.off_s3 >= 0 ? h->at<float>(p.off_s3) : nullptr;
  j.tile[0] = j.tile[1] = p.sym_tile;
  j.gemm_mode = h->cfg.fp32_gemm;
  for (int i = 0; i < 6; ++i) j.mx[i] = m_mx(h, i);
  for (const auto& b : h->blocks)
    j.real_cube += (double)b.m * b.m * (b.m + 1.0) + (double)b.n * b.n * (b.n + 1.0);
  j.t_stats = t_stats;
  const int rc = run_roots(h, j, s);
  if (rc) return rc;
  h->roots_valid = true;
  return SHAMPOO_OK;
}

// tmp / tmp_words: where the intermediate X_L G (or its transpose on the
// fp32 MFMA path) and its per-block maximum words go; NULL: the workspace's
int do_apply(shampoo_ctx* h, hipStream_t s, float* out_packed, float* tmp = nullptr,
             uint64_t* tmp_words = nullptr) {
  const Plan& p = h->plan;
  if (p.B == 0) return SHAMPOO_OK;
  if (tmp == nullptr) tmp = m_tmpT(h);
  if (tmp_words == nullptr && m_f16(h)) tmp_words = m_mx(h, 8);
  // the preconditioned matrix: the packed gradient, or the momentum buffer
  const float* G = p.momentum ? m_mom(h) : m_gp(h);
  const bool split = h->cfg.fp32_gemm != SHAMPOO_GEMM_F32;
  shp::GemmLaunch g1{};
  shp::GemmProblem a{};
  if (split) {
    // Tmp[m][n] = sum_k X_L[m][k] G[k][n] (= X_L G, br x bc): A = X_L (rows,
    // symmetric), B = G^T read by columns from G (the packed transpose shares
    // memory with the root iterations, which overwrite it on refresh steps)
    a.P = m_xroot(h);
    a.sP = (int64_t)p.br * p.br;
    a.Q = G;
    a.sQ = (int64_t)p.br * p.bc;
    a.q_cols = 1;
    a.M = p.br;
    a.N = p.bc;
  } else {
    // TmpT[m][n] = sum_k G[k][m] X_L[k][n]   (= (X_L G)^T, bc x br)
    a.P = G;
    a.sP = (int64_t)p.br * p.bc;
    a.Q = m_xroot(h);
    a.sQ = (int64_t)p.br * p.br;
    a.M = p.bc;
    a.N = p.br;
  }
  a.C = tmp;
  a.sC = (int64_t)p.bc * p.br;
  a.K = p.br;
  a.batch = (int)p.B;
  a.alpha = 1.f;
  if (m_f16(h)) {  // maxima: left roots, the preconditioned blocks; raises Tmp's
    a.mP = m_mx(h, 0);
    a.mQ = m_mx(h, p.momentum ? 7 : 6);
    a.mC = tmp_words;
    a.ver = h->next_ver();
  }
  g1.p[0] = a;
  g1.n_problems = 1;
  // U = X_L G X_R (br x bc). fp32 MFMA: U[m][n] = sum_k TmpT[k][m] X_R[k][n];
  // split: U[m][n] = sum_k Tmp[m][k] X_R[n][k] (X_R symmetric)
  shp::GemmLaunch g2{};
  shp::GemmProblem b{};
  b.P = tmp;
  b.sP = (int64_t)p.bc * p.br;
  b.Q = m_xroot(h) + p.fl;
  b.sQ = (int64_t)p.bc * p.bc;
  b.C = nullptr;
  b.M = p.br;
  b.N = p.bc;
  b.K = p.bc;
  b.batch = (int)p.B;
  b.alpha = 1.f;
  if (m_f16(h)) {  // maxima: Tmp, right roots
    b.mP = tmp_words;
    b.mQ = m_mx(h, 0) + p.B;
  }
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
  const int mode = h->cfg.fp32_gemm;
  // split path: 256 x 256 tiles when both block sides allow them (half the
  // operand traffic of 128 x 128 tiles per flop)
  const int tile = split && p.br % 256 == 0 && p.bc % 256 == 0 ? 256 : p.tile;
  int rc = timed(h, kApply, f1, 0.0, s, [&] { return shp::launch_gemm_full(g1, tile, mode, s); });
  if (rc) return rc;
  return timed(h, kApply, f2, 0.0, s,
               [&] { return shp::launch_gemm_update(g2, u, tile, mode, s); });
}

}  // namespace
}  // namespace shp_rt

using namespace shp_rt;

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
  cfg->newton_scale_mode = 3;
  cfg->param_dtype = SHAMPOO_F32;
  cfg->grad_dtype = SHAMPOO_F32;
  cfg->momentum = 0.0;
  cfg->root_method = shp::kCoupledNewton;
  cfg->cheb_degree = 128;
  cfg->fp32_gemm = SHAMPOO_GEMM_SPLIT_F16;
  return SHAMPOO_OK;
}

int shampoo_workspace_size(const shampoo_config_t* cfg, const shampoo_matrix_desc_t* mats,
                           int32_t n_mats, size_t* bytes_out) {
  int rc = validate_config(cfg, false);
  if (rc) return rc;
  rc = validate_mats(mats, n_mats);
  if (rc) return rc;
  if (!bytes_out) return fail(SHAMPOO_ERR_INVALID_ARG, "bytes_out is NULL");
  *bytes_out = (size_t)make_plan(cfg, mats, n_mats).total;
  return SHAMPOO_OK;
}

int shampoo_init(const shampoo_config_t* cfg, const shampoo_matrix_desc_t* mats, int32_t n_mats,
                 void* workspace, size_t workspace_bytes, void* hip_stream, shampoo_t* out) {
  int rc = validate_config(cfg, false);
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
  h->off_flops = plan.off_flops;
  h->ws = static_cast<char*>(workspace);
  h->mats.assign(mats, mats + n_mats);
  for (int i = 0; i < n_mats; ++i) h->empty_item.push_back(mats[i].rows == 0 || mats[i].cols == 0);
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
    e = shp::launch_upload(h->at<void>(plan.off_blocks), h->blocks.data(),
                           plan.B * sizeof(shp::BlockMeta), s);
    if (e == hipSuccess)
      e = shp::launch_upload(h->at<void>(plan.off_nreal), nreal.data(), nreal.size() * 4, s);
    if (e == hipSuccess) e = hipMemsetAsync(h->at<void>(plan.off_status), 0, 2 * plan.B * 4, s);
    if (e == hipSuccess) e = hipMemsetAsync(h->at<void>(plan.off_final), 0, 2 * plan.B * 4, s);
    if (e == hipSuccess) e = hipMemsetAsync(h->at<void>(plan.off_scale), 0, 2 * plan.B * 4, s);
    if (e == hipSuccess) e = hipMemsetAsync(h->at<void>(plan.off_flops), 0, 8, s);
    if (e == hipSuccess && plan.momentum)
      e = hipMemsetAsync(h->at<void>(plan.off_mom), 0, plan.B * plan.br * plan.bc * 4, s);
    if (e == hipSuccess && plan.off_mx >= 0)  // no maximum word written yet
      e = hipMemsetAsync(h->at<void>(plan.off_mx), 0, (6 * 2 * plan.B + 3 * plan.B) * 8, s);
    if (e == hipSuccess)
      e = shp::launch_init_state(m_lr(h), plan.fl, plan.br, plan.fr, plan.bc, (int32_t)plan.B,
                                 (float)cfg->eps, s);
    // the address of the library's scratch on this device (set-up of
    // shampoo_precondition_noalloc; fetched once per device)
    void* scratch = nullptr;
    if (e == hipSuccess) e = shp::scratch_address(&scratch);
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
  if (h->tensor) {
    if ((rc = tensor_step(h, params, grads, refresh, t, s))) return rc;
    h->t = t;
    return SHAMPOO_OK;
  }
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
  if (h->tensor) return tensor_refresh(h, static_cast<hipStream_t>(hip_stream), h->t);
  return do_refresh(h, static_cast<hipStream_t>(hip_stream), h->t);
}

int shampoo_destroy(shampoo_t h) {
  if (!h) return fail(SHAMPOO_ERR_INVALID_ARG, "handle is NULL");
  for (auto& r : h->timed) {
    (void)hipEventDestroy(r.start);
    (void)hipEventDestroy(r.stop);
  }
  for (auto e : h->event_pool) (void)hipEventDestroy(e);
  delete h;
  return SHAMPOO_OK;
}

int shampoo_state_layout(shampoo_t h, shampoo_layout_t* out) {
  if (!h || !out) return fail(SHAMPOO_ERR_INVALID_ARG, "NULL argument");
  if (h->tensor) return tensor_layout(h, out);
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
  out->root_maxima = h->plan.off_mx;
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

int shampoo_restore(shampoo_t h, int64_t t, void* hip_stream) {
  if (!h || t < 0) return fail(SHAMPOO_ERR_INVALID_ARG, "NULL handle or negative step");
  if (h->tensor) {
    const int rc = tensor_rebase_words(h, static_cast<hipStream_t>(hip_stream));
    if (rc) return rc;
  } else if (h->plan.off_mx >= 0) {
    // words written by another handle carry its versions: take them as this
    // handle's current ones, so every later write wins over them
    const uint64_t ver = h->next_ver();
    const int64_t n = 6 * 2 * h->plan.B + 3 * h->plan.B;
    const hipError_t e =
        shp::launch_rebase_words(h->at<uint64_t>(h->plan.off_mx), n, ver, static_cast<hipStream_t>(hip_stream));
    if (e != hipSuccess) return hip_fail(e, "rebase of the maximum words");
  }
  h->t = t;
  h->roots_valid = t > 0;
  return SHAMPOO_OK;
}

int shampoo_pack(shampoo_t h, const void* const* grads, void* hip_stream) {
  if (!h) return fail(SHAMPOO_ERR_INVALID_ARG, "handle is NULL");
  int rc = check_ptrs(h, grads, h->cfg.grad_dtype, "grads");
  if (rc) return rc;
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  if (h->tensor) return tensor_pack(h, grads, s);
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
  if (h->tensor) return tensor_unpack(h, dst, s);
  std::vector<shp::MatMeta> m(p.n_mats);
  for (int i = 0; i < p.n_mats; ++i) {
    m[i].grad = nullptr;
    m[i].param = dst[i];
    m[i].ld = h->mats[i].ld;
  }
  HIP_CHECK(shp::launch_upload(h->at<void>(p.off_umats), m.data(), m.size() * sizeof(shp::MatMeta), s));
  HIP_CHECK(shp::launch_unpack(h->at<shp::BlockMeta>(p.off_blocks), h->at<shp::MatMeta>(p.off_umats),
                               (int32_t)p.B, p.br, p.bc, m_gp(h), s));
  return SHAMPOO_OK;
}

int shampoo_precondition(shampoo_t h, void* out, void* hip_stream) {
  if (!h) return fail(SHAMPOO_ERR_INVALID_ARG, "handle is NULL");
  shampoo_layout_t lay{};
  if (h->tensor) tensor_layout(h, &lay);
  const int64_t nb = h->tensor ? lay.n_blocks : h->plan.B;
  if (!out && nb) return fail(SHAMPOO_ERR_INVALID_ARG, "out is NULL");
  if (reinterpret_cast<uintptr_t>(out) % 16) return fail(SHAMPOO_ERR_MISALIGNED, "out not 16-byte aligned");
  if (!h->roots_valid) return fail(SHAMPOO_ERR_NO_ROOTS, "no roots yet");
  if (h->tensor)
    return tensor_precondition(h, static_cast<float*>(out), static_cast<hipStream_t>(hip_stream));
  return do_apply(h, static_cast<hipStream_t>(hip_stream), static_cast<float*>(out));
}

int shampoo_precondition_noalloc(shampoo_t h, void* out, void* hip_stream) {
  if (!h) return fail(SHAMPOO_ERR_INVALID_ARG, "handle is NULL");
  if (h->tensor)
    return fail(SHAMPOO_ERR_UNSUPPORTED, "shampoo_precondition_noalloc takes matrix handles only");
  const Plan& p = h->plan;
  if (!out && p.B) return fail(SHAMPOO_ERR_INVALID_ARG, "out is NULL");
  if (reinterpret_cast<uintptr_t>(out) % 16) return fail(SHAMPOO_ERR_MISALIGNED, "out not 16-byte aligned");
  if (!h->roots_valid) return fail(SHAMPOO_ERR_NO_ROOTS, "no roots yet");
  // the intermediate, then its maximum words (fp16 split), in the library's scratch
  const int64_t tmp_bytes = (p.B * (int64_t)p.br * p.bc * 4 + 255) / 256 * 256;
  const int64_t need = tmp_bytes + (m_f16(h) ? 8 * p.B : 0);
  if (need > shp::kScratchBytes)
    return fail(SHAMPOO_ERR_UNSUPPORTED,
                "shampoo_precondition_noalloc: the intermediate needs " + std::to_string(need) +
                    " bytes of scratch, more than the " + std::to_string(shp::kScratchBytes) +
                    " the library holds per GPU (use shampoo_precondition)");
  if (p.B == 0) return SHAMPOO_OK;
  void* base = nullptr;
  HIP_CHECK(shp::scratch_address(&base));
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  float* tmp = static_cast<float*>(base);
  uint64_t* words = nullptr;
  if (m_f16(h)) {
    // words left by an earlier call (of any handle) carry other versions:
    // clear them so this call's writes define them
    words = reinterpret_cast<uint64_t*>(static_cast<char*>(base) + tmp_bytes);
    HIP_CHECK(shp::launch_zero_words(words, p.B, s));
  }
  return do_apply(h, s, static_cast<float*>(out), tmp, words);
}

int shampoo_get_status(shampoo_t h, void* hip_stream, int32_t* n_diverged_out) {
  if (!h || !n_diverged_out) return fail(SHAMPOO_ERR_INVALID_ARG, "NULL argument");
  int64_t off = h->plan.off_status, count = 2 * h->plan.B;
  if (h->tensor) tensor_status_count(h, &off, &count);
  std::vector<int32_t> st(count);
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  if (count) {
    HIP_CHECK(hipMemcpyAsync(st.data(), h->at<void>(off), st.size() * 4, hipMemcpyDeviceToHost, s));
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
    HIP_CHECK(hipMemsetAsync(h->at<void>(h->off_flops), 0, 8,
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
  HIP_CHECK(hipMemcpy(&nf, h->at<void>(h->off_flops), sizeof(double), hipMemcpyDeviceToHost));
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
