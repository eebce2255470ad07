// Host runtime internals shared by the matrix path (runtime.cpp), the
// order-k tensor path (tensor_runtime.cpp) and the root solvers (roots.cpp).
// Not part of the public C ABI.
#pragma once

#include "../../include/shampoo.h"

#include <hip/hip_runtime.h>

#include <memory>
#include <string>
#include <vector>

#include "kernels.h"

namespace shp_rt {

int fail(int code, const std::string& msg);
int hip_fail(hipError_t e, const char* where);

#define HIP_CHECK(expr)                                       \
  do {                                                        \
    hipError_t e_ = (expr);                                   \
    if (e_ != hipSuccess) return shp_rt::hip_fail(e_, #expr); \
  } while (0)

constexpr int64_t kAlign = 256;
inline int64_t align_up(int64_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Largest of 128, 64, 32 that divides both a and b (callers keep them
// multiples of 32).
int pick_tile(int a, int b);

int validate_config(const shampoo_config_t* c, bool tensor);

// Sequential carving of a workspace into 256-byte-aligned pieces.
struct Carver {
  int64_t o = 0;
  int64_t take(int64_t bytes) {
    const int64_t at = o;
    o = align_up(o + (bytes > 1 ? bytes : 1));
    return at;
  }
};

// Layout of the caller's workspace for a matrix handle (byte offsets).
struct Plan {
  int64_t B = 0;
  int br = 0, bc = 0, n_mats = 0, tile = 32, max_iters = 1;
  // tile of the symmetric products (statistics of fp32 gradients, roots):
  // 256 on the fp16 split when both block sides allow it, else `tile`
  int sym_tile = 32;
  // tile of the statistics of bf16 gradients (bf16 MFMA): 256 when both block
  // sides are multiples of 256 of at least 512, else `tile`
  int bf16_tile = 32;
  int ntiles_l = 0, ntiles_r = 0, resid_stride = 0;
  int64_t fl = 0, fr = 0;  // elements of all left / right factors
  int64_t off_blocks, off_mats, off_umats, off_nreal, off_status, off_final, off_scale, off_rprev,
      off_cfac, off_lo, off_coef, off_active, off_flops, off_resid, off_gp, off_mom, off_lr,
      off_xroot, off_xalt, off_s0, off_s1, off_s2, off_s3, off_cheb, total;
  // fp16 split products: maximum words (uint64, see shp::max_word) per
  // factor of xroot, xalt, s0..s3 (6 x 2B, xroot's first: the roots') and
  // per block of Gp, the momentum buffer and the apply intermediate (3 x B);
  // -1 on the other product paths
  int64_t off_mx = -1;
  bool momentum = false;
};

enum {
  kPack = 0,
  kStats = 1,
  kNorms = 2,
  kNewtonGemm = 3,
  kNewtonAux = 4,
  kApply = 5,
  kStatsAux = 6,
  kApplyAux = 7
};

struct TimedLaunch {
  int cls;
  hipEvent_t start, stop;
  double flops, bytes;
};

struct TensorState;  // tensor_runtime.cpp
void destroy_tensor_state(TensorState* t);
struct TensorStateDeleter {
  void operator()(TensorState* t) const { destroy_tensor_state(t); }
};

}  // namespace shp_rt

struct shampoo_ctx {
  shampoo_config_t cfg;
  shp_rt::Plan plan;  // matrix handles
  std::unique_ptr<shp_rt::TensorState, shp_rt::TensorStateDeleter> tensor;  // tensor handles
  char* ws = nullptr;
  std::vector<shampoo_matrix_desc_t> mats;
  std::vector<uint8_t> empty_item;      // per registered matrix / tensor: no elements
  std::vector<shp::BlockMeta> blocks;
  std::vector<shp::MatMeta> meta_host;  // what the device table holds
  bool meta_valid = false;
  int64_t t = 0;
  bool roots_valid = false;
  // version of the last launch that wrote maximum words; grows by one per
  // such launch (shampoo_restore rebases restored words onto it)
  uint64_t ver_count = 0;
  float stat_scale = 0.f;
  // timing
  bool timing = false;
  std::vector<shp_rt::TimedLaunch> timed;
  std::vector<hipEvent_t> event_pool;
  int64_t off_flops = 0;  // device double: flops of the Newton products run

  template <class T>
  T* at(int64_t off) const { return reinterpret_cast<T*>(ws + off); }
  hipEvent_t get_event();
  uint64_t next_ver() { return ++ver_count; }
};

namespace shp_rt {

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

// One inverse-root computation over a set of factor groups (roots.cpp):
// statistics A, result in xroot, scratch xalt and s[0..3] (s[3] only for
// p > 4), all with the FactorSet's layout; tile[g] is the MFMA tile of group
// g's symmetric products.
struct RootJob {
  shp::FactorSet fs{};
  shp::NewtonCtl c{};
  float* A = nullptr;
  float* xroot = nullptr;
  float* xalt = nullptr;
  float* s[4] = {nullptr, nullptr, nullptr, nullptr};
  // how the products run (shp::GemmMode); kGemmSplitF16 needs the maximum
  // words per factor of xroot, xalt, s[0..3] in mx[0..5]
  int gemm_mode = shp::kGemmSplit;
  uint64_t* mx[6] = {nullptr, nullptr, nullptr, nullptr, nullptr, nullptr};
  int tile[shp::kMaxGroups] = {32, 32, 32, 32};
  double real_cube = 0.0;  // sum over factors of n^2 (n + 1), n the real extent
  int64_t t_stats = 0;     // step whose statistics are taken (Chebyshev floor)
};

int run_roots(shampoo_ctx* h, const RootJob& j, hipStream_t s);

// Pointer arrays of a step: one per registered matrix / tensor, non-NULL
// unless it has no elements, aligned to the element size.
int check_ptrs(const shampoo_ctx* h, const void* const* ptrs, int dtype, const char* what);

// Tensor handles (tensor_runtime.cpp)
int tensor_step(shampoo_ctx* h, void* const* params, const void* const* grads, bool refresh,
                int64_t t, hipStream_t s);
int tensor_refresh(shampoo_ctx* h, hipStream_t s, int64_t t_stats);
int tensor_pack(shampoo_ctx* h, const void* const* grads, hipStream_t s);
int tensor_unpack(shampoo_ctx* h, void* const* dst, hipStream_t s);
int tensor_precondition(shampoo_ctx* h, float* out, hipStream_t s);
int tensor_layout(const shampoo_ctx* h, shampoo_layout_t* out);
int tensor_status_count(const shampoo_ctx* h, int64_t* off, int64_t* count);
// shampoo_restore on a tensor handle: every maximum word takes the current version.
int tensor_rebase_words(shampoo_ctx* h, hipStream_t s);

}  // namespace shp_rt
