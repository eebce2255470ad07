// Order-k tensor handles (podcast "Preconditioned Optimization Without the
// Full Matrix Cost", cue 26): one statistic per dimension, roots A^(-1/2k),
// the update as k mode products.
//
// Layout of one step on the stream, for B packed blocks of E elements:
//   pack      tensors -> Gp [B][E] (+ momentum)
//   stats     dimension i blocked at a multiple of 32: the unfolding made a
//             k-major operand (batched transpose of Gp viewed as
//             [b_0..b_i][b_(i+1)..], no copy for the last dimension) and the
//             MFMA SYRK with the EMA epilogue; dimension blocked at <= 8: a
//             fixed-order reduction over Gp.
//   refresh   the MFMA root solver over the large factors (p = 2k), fp64
//             Jacobi over the small ones
//   apply     k products along the leading dimension, each moving it last,
//             so after k of them the block is back in its own order:
//             MFMA (C = P^T X with P the block as [b_i][E / b_i]) or the FMA
//             kernel; the update W -= lr U in the last FMA product's epilogue
//             when the last dimension is small, else a scatter kernel.
#include <algorithm>
#include <cmath>
#include <cstring>
#include <new>

#include "runtime_common.h"

namespace shp_rt {

struct TensorState {
  int k = 0;
  int b[shp::kMaxOrder] = {1, 1, 1, 1};
  int32_t E = 1;
  int64_t B = 0;
  int n_tensors = 0;
  std::vector<shampoo_tensor_desc_t> descs;
  std::vector<shp::TBlockMeta> blocks;
  std::vector<shp::TensorMeta> meta_host;
  bool meta_valid = false;
  // dimensions by kind; group[i]: index of dimension i's factors in the
  // per-factor arrays (large dimensions first, in order, then the small ones)
  int nbig = 0, nsmall = 0;
  int big[shp::kMaxOrder], small[shp::kMaxOrder], group[shp::kMaxOrder];
  bool is_big[shp::kMaxOrder] = {false, false, false, false};
  int stat_tile[shp::kMaxOrder] = {32, 32, 32, 32};
  int apply_tile[shp::kMaxOrder] = {0, 0, 0, 0};  // 0: FMA mode product
  int64_t Kp[shp::kMaxOrder] = {0, 0, 0, 0};      // padded unfolding length (large dims)
  bool rotate[shp::kMaxOrder] = {false, false, false, false};
  // statistics read the block itself by rows (dimension 0 on the split paths)
  bool rows[shp::kMaxOrder] = {false, false, false, false};
  int ntiles[shp::kMaxOrder] = {0, 0, 0, 0};
  int resid_stride = 1, gram_chunks = 1, p = 4;
  bool momentum = false;
  int64_t fbig = 0, fall = 0;             // elements of the large / all factors
  int64_t foff[shp::kMaxOrder] = {0, 0, 0, 0};  // element offset of dimension i's factors
  int64_t rot_stride = 0;                 // elements per block of the transpose buffer
  double real_cube = 0.0;                 // sum of n^2 (n + 1) over the large factors (real n)
  double real_elems = 0.0;
  // algorithmic flops per dimension on real extents: its statistic and its mode product
  double stat_flops[shp::kMaxOrder] = {0, 0, 0, 0}, apply_flops[shp::kMaxOrder] = {0, 0, 0, 0};
  int64_t off_blocks, off_meta, off_umeta, off_nreal, off_status, off_final, off_scale, off_rprev,
      off_cfac, off_lo, off_coef, off_active, off_flops, off_cheb, off_resid, off_partial, off_gp,
      off_mom, off_ap0,
      off_ap1, off_stats, off_xroot, off_xalt, off_s[4], total;
  // fp16 split products: maximum words (uint64, see shp::max_word) per large
  // factor of xroot, xalt, s0..s3 (6 x nbig B, xroot's first: the roots') and
  // per block of Gp, the momentum buffer and the two apply buffers (4 x B);
  // -1 on the other product paths
  int64_t off_mx = -1;
  int64_t n_mx = 0;
};

void destroy_tensor_state(TensorState* t) {
  if (!t) return;
  delete t;
}

namespace {

bool small_side(int n) { return n >= 1 && n <= shp::kMaxSmallSide; }

// MFMA tile of the symmetric products of side n over `count` factors: the
// largest whose launch still gives every CU two workgroups of four waves (a
// 128 x 128 factor is one tile at 128, three at 64, ten at 32). The 32-tile
// runs one wave per workgroup and re-reads its operands far more often: for
// 201 factors of 128, the 64-tile statistics ran 1.35x faster than the
// 32-tile ones with three times as many workgroups.
int occupancy_tile(int n, int64_t count) {
  for (int t : {128, 64}) {
    if (n % t == 0 && count * shp::sym_tiles(n, t) >= 512) return t;
  }
  return 32;
}
bool big_side(int n) { return n >= 32 && n <= shp::kMaxSide && n % 32 == 0; }

int make_tensor_plan(const shampoo_config_t* cfg, int32_t order, const int32_t* bd,
                     const shampoo_tensor_desc_t* d, int32_t n, TensorState& ts) {
  int rc = validate_config(cfg, true);
  if (rc) return rc;
  if (order < 2 || order > shp::kMaxOrder)
    return fail(SHAMPOO_ERR_UNSUPPORTED, "order must be 2, 3 or 4");
  if (!bd) return fail(SHAMPOO_ERR_INVALID_ARG, "block_dims is NULL");
  if (n < 0) return fail(SHAMPOO_ERR_INVALID_ARG, "n_tensors must be >= 0");
  if (n > 0 && !d) return fail(SHAMPOO_ERR_INVALID_ARG, "tensor descriptors are NULL");
  ts.k = order;
  int64_t E = 1;
  for (int i = 0; i < order; ++i) {
    if (!small_side(bd[i]) && !big_side(bd[i]))
      return fail(SHAMPOO_ERR_UNSUPPORTED, "block_dims[" + std::to_string(i) +
                                               "] must be 1..8 or a multiple of 32 up to 4096");
    ts.b[i] = bd[i];
    E *= bd[i];
    if (E > ((int64_t)1 << 30)) return fail(SHAMPOO_ERR_UNSUPPORTED, "a block exceeds 2^30 elements");
  }
  ts.E = (int32_t)E;
  ts.p = 2 * order;
  if (cfg->root_method == shp::kNewtonDB && ts.p != 4)
    return fail(SHAMPOO_ERR_UNSUPPORTED, "Newton-DB computes 4th roots only (order 2)");
  for (int t = 0; t < n; ++t) {
    if (d[t].order != order)
      return fail(SHAMPOO_ERR_INVALID_ARG, "tensor " + std::to_string(t) + ": order differs");
    for (int i = 0; i < order; ++i) {
      if (d[t].dims[i] < 0 || d[t].dims[i] > INT32_MAX)
        return fail(SHAMPOO_ERR_INVALID_ARG, "tensor " + std::to_string(t) + ": bad extent");
      if (d[t].strides[i] < 1)
        return fail(SHAMPOO_ERR_INVALID_ARG, "tensor " + std::to_string(t) + ": strides must be >= 1");
    }
  }
  ts.descs.assign(d, d + n);
  ts.n_tensors = n;
  // block map: tensors in registration order, row-major blocks inside each
  ts.blocks.clear();
  for (int t = 0; t < n; ++t) {
    bool empty = false;
    int64_t cnt[shp::kMaxOrder] = {1, 1, 1, 1};
    for (int i = 0; i < order; ++i) {
      empty = empty || d[t].dims[i] == 0;
      cnt[i] = (d[t].dims[i] + ts.b[i] - 1) / ts.b[i];
    }
    if (empty) continue;
    int64_t idx[shp::kMaxOrder] = {0, 0, 0, 0};
    for (;;) {
      shp::TBlockMeta m{};
      m.tensor = t;
      for (int i = 0; i < order; ++i) {
        m.origin[i] = (int32_t)(idx[i] * ts.b[i]);
        m.extent[i] = (int32_t)std::min<int64_t>(ts.b[i], d[t].dims[i] - m.origin[i]);
      }
      ts.blocks.push_back(m);
      int i = order - 1;
      while (i >= 0 && ++idx[i] == cnt[i]) idx[i--] = 0;
      if (i < 0) break;
    }
  }
  ts.B = (int64_t)ts.blocks.size();
  if (ts.B > ((int64_t)1 << 24)) return fail(SHAMPOO_ERR_UNSUPPORTED, "too many blocks");
  // dimensions: large ones first in the per-factor arrays
  ts.nbig = ts.nsmall = 0;
  for (int i = 0; i < order; ++i) {
    ts.is_big[i] = big_side(ts.b[i]);
    if (ts.is_big[i]) ts.big[ts.nbig++] = i;
  }
  for (int i = 0; i < order; ++i)
    if (!ts.is_big[i]) ts.small[ts.nsmall++] = i;
  for (int g = 0; g < ts.nbig; ++g) ts.group[ts.big[g]] = g;
  for (int g = 0; g < ts.nsmall; ++g) ts.group[ts.small[g]] = ts.nbig + g;
  // factor storage: large factors (MFMA solver layout) then small ones
  int64_t fo = 0;
  for (int g = 0; g < ts.nbig; ++g) {
    const int i = ts.big[g];
    ts.foff[i] = fo;
    fo += ts.B * ts.b[i] * ts.b[i];
  }
  ts.fbig = fo;
  for (int g = 0; g < ts.nsmall; ++g) {
    const int i = ts.small[g];
    ts.foff[i] = fo;
    fo += ts.B * ts.b[i] * ts.b[i];
  }
  ts.fall = fo;
  ts.rot_stride = 0;
  ts.resid_stride = 1;
  int64_t before = 1;
  for (int i = 0; i < order; ++i) {
    const int64_t K = E / ts.b[i];
    before *= ts.b[i];
    const int64_t after = E / before;
    if (ts.is_big[i]) {
      ts.stat_tile[i] = occupancy_tile(ts.b[i], ts.B);
      ts.Kp[i] = (K + 15) / 16 * 16;

      // The unfolding of dimension 0 is the block itself, [b_0][K] with k
      // contiguous: the split paths read it by rows when K-tiles pair up (the
      // fp32 MFMA path wants it k-major). The last dimension's unfolding is
      // k-major already; the others are transposed first.
      ts.rows[i] = i == 0 && cfg->fp32_gemm != SHAMPOO_GEMM_F32 && K % 32 == 0;
      ts.rotate[i] = !ts.rows[i] && !(after == 1 && K == ts.Kp[i]);
      if (ts.rotate[i]) ts.rot_stride = std::max<int64_t>(ts.rot_stride, ts.Kp[i] * ts.b[i]);
      ts.apply_tile[i] = K % 32 == 0 ? pick_tile((int)std::min<int64_t>(K, 1 << 30), ts.b[i]) : 0;
      ts.ntiles[ts.group[i]] = shp::sym_tiles(ts.b[i], ts.stat_tile[i]);
      ts.resid_stride = std::max(ts.resid_stride, ts.ntiles[ts.group[i]]);
    }
  }
  // algorithmic counts on real extents
  ts.real_cube = ts.real_elems = 0.0;
  for (int i = 0; i < shp::kMaxOrder; ++i) ts.stat_flops[i] = ts.apply_flops[i] = 0.0;
  for (const auto& m : ts.blocks) {
    double vol = 1.0;
    for (int i = 0; i < order; ++i) vol *= m.extent[i];
    ts.real_elems += vol;
    for (int i = 0; i < order; ++i) {
      const double e = m.extent[i];
      ts.stat_flops[i] += e * (e + 1.0) * (vol / e);
      ts.apply_flops[i] += 2.0 * e * vol;
      if (ts.is_big[i]) ts.real_cube += e * e * (e + 1.0);
    }
  }
  ts.gram_chunks = (int)std::max<int64_t>(1, std::min<int64_t>(256, (2048 + ts.B - 1) / std::max<int64_t>(ts.B, 1)));
  ts.momentum = cfg->momentum > 0.0;
  const int64_t nf = (int64_t)order * ts.B;
  Carver c;
  ts.off_blocks = c.take(ts.B * (int64_t)sizeof(shp::TBlockMeta));
  ts.off_meta = c.take(n * (int64_t)sizeof(shp::TensorMeta));
  ts.off_umeta = c.take(n * (int64_t)sizeof(shp::TensorMeta));
  ts.off_nreal = c.take(nf * 4);
  ts.off_status = c.take(nf * 4);
  ts.off_final = c.take(nf * 4);
  ts.off_scale = c.take(nf * 4);
  ts.off_rprev = c.take(nf * 4);
  ts.off_cfac = c.take(nf * 4);
  ts.off_lo = c.take(nf * 4);
  ts.off_coef = c.take(nf * shp::kCoefRecord * 4);
  ts.off_active = c.take((int64_t)(cfg->newton_max_iters + 1) * shp::kMaxGroups * 4);
  ts.off_flops = c.take(8);
  ts.off_cheb = cfg->root_method == shp::kChebyshev && ts.nbig
                    ? c.take((int64_t)ts.nbig * ts.B * shp::cheb_floats(cfg->cheb_degree) * 4)
                    : -1;
  ts.off_resid = c.take((int64_t)ts.nbig * ts.B * ts.resid_stride * 4);
  ts.off_partial = ts.nsmall ? c.take(ts.B * ts.gram_chunks * 36 * 4) : -1;
  const int64_t be = ts.B * (int64_t)E * 4;
  ts.off_gp = c.take(be);
  ts.off_mom = ts.momentum ? c.take(be) : -1;
  ts.off_ap0 = c.take(ts.B * std::max<int64_t>(E, ts.rot_stride) * 4);
  ts.off_ap1 = c.take(be);

  ts.off_stats = c.take(ts.fall * 4);
  ts.off_xroot = c.take(ts.fall * 4);
  const bool scratch = ts.nbig > 0;
  ts.off_xalt = scratch ? c.take(ts.fbig * 4) : -1;
  for (int i = 0; i < 4; ++i)
    // the fourth: the coupled Newton at p > 4, and the Chebyshev giant steps
    ts.off_s[i] = scratch && (i < 3 || ts.p > 4 || cfg->root_method == shp::kChebyshev)
                      ? c.take(ts.fbig * 4)
                      : -1;
  if (cfg->fp32_gemm == SHAMPOO_GEMM_SPLIT_F16) {
    ts.n_mx = 6 * (int64_t)ts.nbig * ts.B + 4 * ts.B;
    ts.off_mx = c.take(ts.n_mx * 8);
  }
  ts.total = c.o;
  return SHAMPOO_OK;
}

TensorState& T(shampoo_ctx* h) { return *h->tensor; }
const TensorState& T(const shampoo_ctx* h) { return *h->tensor; }

shp::TensorGeom geom(const TensorState& ts) {
  shp::TensorGeom g{};
  g.order = ts.k;
  for (int i = 0; i < shp::kMaxOrder; ++i) {
    g.b[i] = i < ts.k ? ts.b[i] : 1;
    g.magic[i] = shp::division_magic((uint32_t)g.b[i]);
  }
  g.E = ts.E;
  return g;
}

float* fptr(const shampoo_ctx* h, int64_t off) { return off < 0 ? nullptr : h->at<float>(off); }

// Maximum words (fp16 split): i = 0..5 per large factor of xroot, xalt,
// s0..s3; i = 6..9 per block of Gp, the momentum buffer, ap0, ap1. NULL on the
// other product paths.
uint64_t* tmx(const shampoo_ctx* h, int i) {
  const TensorState& ts = *h->tensor;
  if (ts.off_mx < 0) return nullptr;
  const int64_t nfb = (int64_t)ts.nbig * ts.B;
  return h->at<uint64_t>(ts.off_mx) + (i < 6 ? i * nfb : 6 * nfb + (i - 6) * ts.B);
}

// The words of one of the per-block buffers (Gp, momentum, apply buffers).
uint64_t* tmx_of(const shampoo_ctx* h, const float* buf) {
  const TensorState& ts = *h->tensor;
  const int64_t offs[4] = {ts.off_gp, ts.off_mom, ts.off_ap0, ts.off_ap1};
  for (int i = 0; i < 4; ++i)
    if (offs[i] >= 0 && buf == h->at<float>(offs[i])) return tmx(h, 6 + i);
  return nullptr;
}

int upload_tensor_meta(shampoo_ctx* h, const void* const* grads, void* const* params,
                       hipStream_t s) {
  TensorState& ts = T(h);
  const int n = ts.n_tensors;
  std::vector<shp::TensorMeta> m(n);
  for (int i = 0; i < n; ++i) {
    m[i].grad = grads ? grads[i] : (ts.meta_valid ? ts.meta_host[i].grad : nullptr);
    m[i].param = params ? params[i] : (ts.meta_valid ? ts.meta_host[i].param : nullptr);
    for (int dd = 0; dd < shp::kMaxOrder; ++dd) m[i].stride[dd] = dd < ts.k ? ts.descs[i].strides[dd] : 1;
  }
  bool same = ts.meta_valid;
  for (int i = 0; same && i < n; ++i)
    same = m[i].grad == ts.meta_host[i].grad && m[i].param == ts.meta_host[i].param;
  if (same) return SHAMPOO_OK;
  // the table travels in kernel arguments: nothing to wait for
  HIP_CHECK(shp::launch_upload(h->at<void>(ts.off_meta), m.data(), n * sizeof(shp::TensorMeta), s));
  ts.meta_host = m;
  ts.meta_valid = true;
  return SHAMPOO_OK;
}

int do_tensor_pack(shampoo_ctx* h, hipStream_t s) {
  const TensorState& ts = T(h);
  const double esz = h->cfg.grad_dtype == SHAMPOO_BF16 ? 2.0 : 4.0;
  const double bytes = ts.real_elems * esz + (ts.momentum ? 3.0 : 1.0) * 4.0 * (double)ts.B * ts.E;
  shp::MaxOut mo{};
  if (ts.off_mx >= 0) {
    mo.a = tmx(h, 6);
    mo.b = ts.momentum ? tmx(h, 7) : nullptr;
    mo.ver = h->next_ver();
  }
  return timed(h, kPack, 0.0, bytes, s, [&] {
    return shp::launch_tensor_pack(h->at<shp::TBlockMeta>(ts.off_blocks),
                                   h->at<shp::TensorMeta>(ts.off_meta), geom(ts), (int32_t)ts.B,
                                   h->cfg.grad_dtype == SHAMPOO_BF16, fptr(h, ts.off_gp),
                                   fptr(h, ts.off_mom), (float)h->cfg.momentum, s, mo);
  });
}

bool split_gemm(const shampoo_ctx* h) { return h->cfg.fp32_gemm != SHAMPOO_GEMM_F32; }

int do_tensor_stats(shampoo_ctx* h, hipStream_t s) {
  const TensorState& ts = T(h);
  if (ts.B == 0) return SHAMPOO_OK;
  const float* gp = fptr(h, ts.off_gp);
  float* rot = fptr(h, ts.off_ap0);
  float* stats = fptr(h, ts.off_stats);
  int64_t before = 1;
  for (int i = 0; i < ts.k; ++i) {
    const int n = ts.b[i];
    const int64_t A = before;
    before *= n;
    const int64_t C = ts.E / before;
    float* H = stats + ts.foff[i];
    const double fl = ts.stat_flops[i];
    int rc;
    if (ts.is_big[i]) {
      const float* op = gp;
      int64_t op_stride = ts.E;
      if (ts.rotate[i]) {
        // [b_0..b_i][b_(i+1)..] -> [b_(i+1)..][b_0..b_i]: rows of n along the
        // unfolding's column index, zero rows up to Kp
        rc = timed(h, kStatsAux, 0.0, 8.0 * ts.B * ts.E, s, [&] {
          return shp::launch_transpose(gp, ts.E, rot, ts.Kp[i] * n, (int32_t)(A * n), (int32_t)C,
                                       (int32_t)ts.B, s);
        });
        if (rc) return rc;
        op = rot;
        op_stride = ts.Kp[i] * n;
      }
      shp::GemmLaunch g{};
      shp::GemmProblem& q = g.p[0];
      q.P = op;
      q.Q = op;
      q.C = H;
      q.D = H;  // EMA: reads the old statistic in place
      q.sP = q.sQ = op_stride;
      q.sC = q.sD = (int64_t)n * n;
      q.M = q.N = n;
      q.K = (int32_t)ts.Kp[i];
      q.batch = (int32_t)ts.B;
      q.alpha = h->stat_scale;
      q.beta = (float)h->cfg.beta2;
      g.n_problems = 1;
      // split paths: the k-major operand [Kp][n] read by columns, or for
      // dimension 0 the block itself [n][K] read by rows; K-tiles run in
      // pairs, so an unfolding padded to an odd multiple of 16 stays on the
      // fp32 MFMA. The transposed copy holds Gp's values (and zeros), so Gp's
      // maxima serve it.
      const int mode = split_gemm(h) && ts.Kp[i] % 32 == 0 ? h->cfg.fp32_gemm : shp::kGemmF32;
      q.p_cols = q.q_cols = mode != shp::kGemmF32 && !ts.rows[i] ? 1 : 0;
      q.mP = q.mQ = tmx(h, 6);
      rc = timed(h, kStats, fl, 0.0, s,
                 [&] { return shp::launch_gemm_sym(g, ts.stat_tile[i], false, mode, s); });
    } else if (i == ts.k - 2 && !ts.is_big[i + 1] && ts.b[i + 1] == n &&
               n <= shp::kMaxFusedSide) {
      // both small trailing dimensions in one pass over the blocks
      rc = timed(h, kStatsAux, fl + ts.stat_flops[i + 1], 4.0 * ts.B * ts.E, s, [&] {
        return shp::launch_small_gram2(gp, ts.E, (int32_t)(ts.E / ((int64_t)n * n)), n,
                                       (int32_t)ts.B, fptr(h, ts.off_partial), ts.gram_chunks, H,
                                       stats + ts.foff[i + 1], (float)h->cfg.beta2,
                                       h->stat_scale, s);
      });
      if (rc) return rc;
      break;  // the last dimension's statistic is formed too
    } else {
      rc = timed(h, kStatsAux, fl, 4.0 * ts.B * ts.E, s, [&] {
        return shp::launch_small_gram(gp, ts.E, (int32_t)A, n, (int32_t)C, (int32_t)ts.B,
                                      fptr(h, ts.off_partial), ts.gram_chunks, H,
                                      (float)h->cfg.beta2, h->stat_scale, s);
      });
    }
    if (rc) return rc;
  }
  return SHAMPOO_OK;
}

shp::FactorSet tensor_factors(const shampoo_ctx* h) {
  const TensorState& ts = T(h);
  shp::FactorSet fs{};
  fs.B = (int32_t)ts.B;
  fs.n_groups = ts.nbig;
  for (int g = 0; g < ts.nbig; ++g) {
    fs.side[g] = ts.b[ts.big[g]];
    fs.off[g] = ts.foff[ts.big[g]];
  }
  fs.nreal = h->at<int32_t>(ts.off_nreal);
  return fs;
}

shp::NewtonCtl tensor_ctl(const shampoo_ctx* h) {
  const TensorState& ts = T(h);
  const shampoo_config_t& cfg = h->cfg;
  shp::NewtonCtl c{};
  c.solver = cfg.root_method;
  c.status = h->at<int32_t>(ts.off_status);
  c.final_iter = h->at<int32_t>(ts.off_final);
  c.scale = h->at<float>(ts.off_scale);
  c.rprev = h->at<float>(ts.off_rprev);
  c.cfac = h->at<float>(ts.off_cfac);
  c.resid = h->at<float>(ts.off_resid);
  c.resid_stride = ts.resid_stride;
  for (int g = 0; g < ts.nbig; ++g) c.ntiles[g] = ts.ntiles[g];
  c.active_count = h->at<int32_t>(ts.off_active);
  c.flops_acc = h->at<double>(ts.off_flops);
  c.tol = (float)cfg.newton_tol;
  c.cheb = ts.off_cheb >= 0 ? h->at<float>(ts.off_cheb) : nullptr;
  c.degree = cfg.cheb_degree;
  c.max_iters = cfg.newton_max_iters;
  c.scale_mode = cfg.newton_scale_mode;
  c.p = ts.p;
  c.lo = h->at<float>(ts.off_lo);
  c.coef = h->at<float>(ts.off_coef);
  return c;
}

// U of every block from the current packed gradient (or momentum) and roots;
// out: packed destination, or nullptr to update the parameters.
int do_tensor_apply(shampoo_ctx* h, hipStream_t s, float* out) {
  const TensorState& ts = T(h);
  if (ts.B == 0) return SHAMPOO_OK;
  const float* cur = ts.momentum ? fptr(h, ts.off_mom) : fptr(h, ts.off_gp);
  const float* roots = fptr(h, ts.off_xroot);
  float* ap[2] = {fptr(h, ts.off_ap0), fptr(h, ts.off_ap1)};
  for (int i = 0; i < ts.k; ++i) {
    const int n = ts.b[i];
    const int64_t R = ts.E / n;
    float* dst = (i == ts.k - 1 && out) ? out : ap[i & 1];
    // the product's maxima are needed only when an MFMA mode product reads it next
    const bool words = i + 1 < ts.k && ts.is_big[i + 1] && ts.apply_tile[i + 1] > 0;
    const float* X = roots + ts.foff[i];
    const double fl = ts.apply_flops[i];
    const double esz = h->cfg.param_dtype == SHAMPOO_BF16 ? 2.0 : 4.0;
    int rc;
    if (i == ts.k - 2 && !out && !ts.is_big[i] && !ts.is_big[i + 1] && ts.b[i + 1] == n &&
        n <= shp::kMaxFusedSide) {
      // the last two products (two small dimensions of one side) and the
      // update in one pass
      const int64_t R2 = R / n;
      const double fl2 = fl + ts.apply_flops[i + 1];
      return timed(h, kApplyAux, fl2, 4.0 * ts.B * ts.E + 2.0 * esz * ts.real_elems, s, [&] {
        return shp::launch_mode_product2_update(
            cur, ts.E, X, roots + ts.foff[i + 1], (int64_t)n * n,
            h->at<shp::TBlockMeta>(ts.off_blocks), h->at<shp::TensorMeta>(ts.off_meta),
            geom(ts), (int32_t)R2, (int32_t)ts.B, (float)h->cfg.lr,
            h->cfg.param_dtype == SHAMPOO_BF16, s);
      });
    }
    if (i == ts.k - 1 && !out && !ts.is_big[i]) {
      // last product of the chain with the update in its epilogue
      rc = timed(h, kApplyAux, fl, 4.0 * ts.B * ts.E + 2.0 * esz * ts.real_elems, s, [&] {
        return shp::launch_mode_product_update(
            cur, ts.E, X, (int64_t)n * n, h->at<shp::TBlockMeta>(ts.off_blocks),
            h->at<shp::TensorMeta>(ts.off_meta), geom(ts), (int32_t)R, (int32_t)ts.B,
            (float)h->cfg.lr, h->cfg.param_dtype == SHAMPOO_BF16, s);
      });
      return rc;
    }
    if (ts.is_big[i] && ts.apply_tile[i] > 0) {
      // C[r][j] = sum_l cur[l][r] X[l][j]: the product along dimension i (X is
      // symmetric), which leaves dimension i last. On the split path cur is
      // the A operand read by columns (stored [K = n][M = R]).
      shp::GemmLaunch g{};
      shp::GemmProblem& q = g.p[0];
      q.P = cur;
      q.sP = ts.E;
      q.Q = X;
      q.sQ = (int64_t)n * n;
      q.C = dst;
      q.sC = ts.E;
      q.M = (int32_t)R;
      q.N = n;
      q.K = n;
      q.batch = (int32_t)ts.B;
      q.alpha = 1.f;
      // fp16 split: maxima of the current block, of dimension i's roots and
      // of the product (unless it is the caller's output)
      q.mP = tmx_of(h, cur);
      q.mQ = tmx(h, 0) != nullptr ? tmx(h, 0) + (int64_t)ts.group[i] * ts.B : nullptr;
      q.mC = words ? tmx_of(h, dst) : nullptr;
      if (q.mC != nullptr) q.ver = h->next_ver();
      g.n_problems = 1;
      const int mode = split_gemm(h) ? h->cfg.fp32_gemm : shp::kGemmF32;
      q.p_cols = mode != shp::kGemmF32 ? 1 : 0;
      rc = timed(h, kApply, fl, 0.0, s,
                 [&] { return shp::launch_gemm_full(g, ts.apply_tile[i], mode, s); });
    } else {
      shp::MaxOut mo{};
      mo.a = words ? tmx_of(h, dst) : nullptr;
      if (mo.a != nullptr) mo.ver = h->next_ver();
      rc = timed(h, kApplyAux, fl, 8.0 * ts.B * ts.E, s, [&] {
        return shp::launch_mode_product(cur, ts.E, X, (int64_t)n * n, dst, ts.E, n, (int32_t)R,
                                        (int32_t)ts.B, s, mo);
      });
    }
    if (rc) return rc;
    cur = dst;
  }
  if (out) return SHAMPOO_OK;
  const double esz = h->cfg.param_dtype == SHAMPOO_BF16 ? 2.0 : 4.0;
  return timed(h, kApplyAux, 0.0, 4.0 * ts.B * ts.E + 2.0 * esz * ts.real_elems, s, [&] {
    return shp::launch_tensor_scatter(h->at<shp::TBlockMeta>(ts.off_blocks),
                                      h->at<shp::TensorMeta>(ts.off_meta), geom(ts), (int32_t)ts.B,
                                      cur, (float)h->cfg.lr, h->cfg.param_dtype == SHAMPOO_BF16, 1,
                                      s);
  });
}

}  // namespace

int tensor_refresh(shampoo_ctx* h, hipStream_t s, int64_t t_stats) {
  const TensorState& ts = T(h);
  if (ts.B == 0) {
    h->roots_valid = true;
    return SHAMPOO_OK;
  }
  if (ts.nbig) {
    RootJob j;
    j.fs = tensor_factors(h);
    j.c = tensor_ctl(h);
    j.A = fptr(h, ts.off_stats);
    j.xroot = fptr(h, ts.off_xroot);
    j.xalt = fptr(h, ts.off_xalt);
    for (int i = 0; i < 4; ++i) j.s[i] = ts.off_s[i] >= 0 ? fptr(h, ts.off_s[i]) : nullptr;
    for (int g = 0; g < ts.nbig; ++g) j.tile[g] = ts.stat_tile[ts.big[g]];
    j.real_cube = ts.real_cube;
    j.t_stats = t_stats;
    j.gemm_mode = h->cfg.fp32_gemm;
    for (int i = 0; i < 6; ++i) j.mx[i] = tmx(h, i);
    const int rc = run_roots(h, j, s);
    if (rc) return rc;
  }
  const float floor = (float)(std::pow(h->cfg.beta2, (double)t_stats) * h->cfg.eps);
  for (int g = 0; g < ts.nsmall; ++g) {
    const int i = ts.small[g];
    const int64_t f0 = (int64_t)ts.group[i] * ts.B;
    const int rc = timed(h, kNewtonAux, 0.0, 0.0, s, [&] {
      return shp::launch_small_root(fptr(h, ts.off_stats) + ts.foff[i],
                                    fptr(h, ts.off_xroot) + ts.foff[i], ts.b[i], (int32_t)ts.B,
                                    h->at<int32_t>(ts.off_nreal) + f0, floor, ts.p,
                                    h->at<int32_t>(ts.off_status) + f0,
                                    h->at<int32_t>(ts.off_final) + f0,
                                    h->at<float>(ts.off_rprev) + f0, s);
    });
    if (rc) return rc;
  }
  h->roots_valid = true;
  return SHAMPOO_OK;
}

int tensor_step(shampoo_ctx* h, void* const* params, const void* const* grads, bool refresh,
                int64_t t, hipStream_t s) {
  int rc = upload_tensor_meta(h, grads, params, s);
  if (rc) return rc;
  if ((rc = do_tensor_pack(h, s))) return rc;
  if ((rc = do_tensor_stats(h, s))) return rc;
  if (refresh && (rc = tensor_refresh(h, s, t))) return rc;
  return do_tensor_apply(h, s, nullptr);
}

int tensor_pack(shampoo_ctx* h, const void* const* grads, hipStream_t s) {
  const int rc = upload_tensor_meta(h, grads, nullptr, s);
  if (rc) return rc;
  return do_tensor_pack(h, s);
}

int tensor_unpack(shampoo_ctx* h, void* const* dst, hipStream_t s) {
  const TensorState& ts = T(h);
  std::vector<shp::TensorMeta> m(ts.n_tensors);
  for (int i = 0; i < ts.n_tensors; ++i) {
    m[i].grad = nullptr;
    m[i].param = dst[i];
    for (int dd = 0; dd < shp::kMaxOrder; ++dd) m[i].stride[dd] = dd < ts.k ? ts.descs[i].strides[dd] : 1;
  }
  HIP_CHECK(shp::launch_upload(h->at<void>(ts.off_umeta), m.data(), m.size() * sizeof(shp::TensorMeta),
                               s));
  HIP_CHECK(shp::launch_tensor_scatter(h->at<shp::TBlockMeta>(ts.off_blocks),
                                       h->at<shp::TensorMeta>(ts.off_umeta), geom(ts),
                                       (int32_t)ts.B, fptr(h, ts.off_gp), 0.f, 0, 0, s));
  return SHAMPOO_OK;
}

int tensor_precondition(shampoo_ctx* h, float* out, hipStream_t s) {
  return do_tensor_apply(h, s, out);
}

int tensor_layout(const shampoo_ctx* h, shampoo_layout_t* out) {
  const TensorState& ts = T(h);
  out->n_blocks = ts.B;
  out->grad_packed = ts.off_gp;
  out->stats = ts.off_stats;
  out->roots = ts.off_xroot;
  out->newton_status = ts.off_status;
  out->newton_iters = ts.off_final;
  out->newton_scale = ts.off_scale;
  out->newton_residual = ts.off_rprev;
  out->momentum = ts.off_mom;
  out->workspace_bytes = ts.total;
  out->root_maxima = ts.off_mx;
  return SHAMPOO_OK;
}

int tensor_rebase_words(shampoo_ctx* h, hipStream_t s) {
  const TensorState& ts = T(h);
  if (ts.off_mx < 0) return SHAMPOO_OK;
  const hipError_t e = shp::launch_rebase_words(h->at<uint64_t>(ts.off_mx), ts.n_mx, h->next_ver(), s);
  return e == hipSuccess ? SHAMPOO_OK : hip_fail(e, "rebase of the maximum words");
}

int tensor_status_count(const shampoo_ctx* h, int64_t* off, int64_t* count) {
  const TensorState& ts = T(h);
  *off = ts.off_status;
  *count = (int64_t)ts.k * ts.B;
  return SHAMPOO_OK;
}

}  // namespace shp_rt

using namespace shp_rt;

extern "C" {

int shampoo_tensor_workspace_size(const shampoo_config_t* cfg, int32_t order,
                                  const int32_t* block_dims, const shampoo_tensor_desc_t* tensors,
                                  int32_t n_tensors, size_t* bytes_out) {
  if (!bytes_out) return fail(SHAMPOO_ERR_INVALID_ARG, "bytes_out is NULL");
  TensorState ts;
  const int rc = make_tensor_plan(cfg, order, block_dims, tensors, n_tensors, ts);
  if (rc) return rc;
  *bytes_out = (size_t)ts.total;
  return SHAMPOO_OK;
}

int shampoo_tensor_init(const shampoo_config_t* cfg, int32_t order, const int32_t* block_dims,
                        const shampoo_tensor_desc_t* tensors, int32_t n_tensors, void* workspace,
                        size_t workspace_bytes, void* hip_stream, shampoo_t* out) {
  if (!out) return fail(SHAMPOO_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  TensorState* ts = new (std::nothrow) TensorState();
  if (!ts) return fail(SHAMPOO_ERR_INVALID_ARG, "out of host memory");
  int rc = make_tensor_plan(cfg, order, block_dims, tensors, n_tensors, *ts);
  if (rc) {
    delete ts;
    return rc;
  }
  if (!workspace) {
    delete ts;
    return fail(SHAMPOO_ERR_INVALID_ARG, "workspace is NULL");
  }
  if (reinterpret_cast<uintptr_t>(workspace) % kAlign) {
    delete ts;
    return fail(SHAMPOO_ERR_MISALIGNED, "workspace is not 256-byte aligned");
  }
  if ((int64_t)workspace_bytes < ts->total) {
    const int64_t need = ts->total;
    delete ts;
    return fail(SHAMPOO_ERR_WORKSPACE_TOO_SMALL, "workspace has " + std::to_string(workspace_bytes) +
                                                     " bytes, needs " + std::to_string(need));
  }
  shampoo_ctx* h = new (std::nothrow) shampoo_ctx();
  if (!h) {
    delete ts;
    return fail(SHAMPOO_ERR_INVALID_ARG, "out of host memory");
  }
  h->tensor.reset(ts);
  h->cfg = *cfg;
  h->ws = static_cast<char*>(workspace);
  h->off_flops = ts->off_flops;
  h->stat_scale = (float)(cfg->stat_scale < 0.0 ? 1.0 - cfg->beta2 : cfg->stat_scale);
  for (int t = 0; t < n_tensors; ++t) {
    bool empty = false;
    for (int i = 0; i < order; ++i) empty = empty || tensors[t].dims[i] == 0;
    h->empty_item.push_back(empty);
  }
  std::vector<int32_t> nreal((size_t)order * ts->B);
  for (int i = 0; i < order; ++i)
    for (int64_t b = 0; b < ts->B; ++b) nreal[ts->group[i] * ts->B + b] = ts->blocks[b].extent[i];
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  hipError_t e = hipSuccess;
  const int64_t nf = (int64_t)order * ts->B;
  if (ts->B) {
    e = shp::launch_upload(h->at<void>(ts->off_blocks), ts->blocks.data(),
                           ts->B * sizeof(shp::TBlockMeta), s);
    if (e == hipSuccess)
      e = shp::launch_upload(h->at<void>(ts->off_nreal), nreal.data(), nreal.size() * 4, s);
    if (e == hipSuccess) e = hipMemsetAsync(h->at<void>(ts->off_status), 0, nf * 4, s);
    if (e == hipSuccess) e = hipMemsetAsync(h->at<void>(ts->off_final), 0, nf * 4, s);
    if (e == hipSuccess) e = hipMemsetAsync(h->at<void>(ts->off_scale), 0, nf * 4, s);
    if (e == hipSuccess) e = hipMemsetAsync(h->at<void>(ts->off_rprev), 0, nf * 4, s);
    if (e == hipSuccess && ts->momentum)
      e = hipMemsetAsync(h->at<void>(ts->off_mom), 0, ts->B * (int64_t)ts->E * 4, s);
    if (e == hipSuccess && ts->off_mx >= 0)  // no maximum word written yet
      e = hipMemsetAsync(h->at<void>(ts->off_mx), 0, ts->n_mx * 8, s);
    for (int i = 0; i < order && e == hipSuccess; ++i) {
      const int n = ts->b[i];
      e = shp::launch_init_state(h->at<float>(ts->off_stats) + ts->foff[i], ts->B * n * n, n, 0, 1,
                                 (int32_t)ts->B, (float)cfg->eps, s);
    }
  }
  if (e == hipSuccess) e = hipMemsetAsync(h->at<void>(ts->off_flops), 0, 8, s);
  if (e != hipSuccess) {
    const int code = hip_fail(e, "shampoo_tensor_init");
    delete h;
    return code;
  }
  *out = h;
  return SHAMPOO_OK;
}

int shampoo_tensor_info(shampoo_t h, shampoo_tensor_info_t* out) {
  if (!h || !out) return fail(SHAMPOO_ERR_INVALID_ARG, "NULL argument");
  if (!h->tensor) return fail(SHAMPOO_ERR_INVALID_ARG, "not a tensor handle");
  const TensorState& ts = *h->tensor;
  std::memset(out, 0, sizeof(*out));
  out->order = ts.k;
  out->n_blocks = ts.B;
  out->block_elems = ts.E;
  for (int i = 0; i < ts.k; ++i) {
    out->block_dims[i] = ts.b[i];
    out->stats[i] = ts.off_stats + ts.foff[i] * 4;
    out->roots[i] = ts.off_xroot + ts.foff[i] * 4;
    out->factor_group[i] = ts.group[i];
  }
  return SHAMPOO_OK;
}

}  // extern "C"
