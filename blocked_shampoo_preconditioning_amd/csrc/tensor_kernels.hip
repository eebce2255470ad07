// HIP kernels of order-k tensor Shampoo (podcast "Preconditioned
// Optimization Without the Full Matrix Cost", cue 26) that are not dense
// contractions: gather / scatter of tensor blocks, the batched transpose that
// makes a dimension's unfolding a k-major operand of the MFMA SYRK, the
// statistics, roots and mode products of dimensions blocked at <= 8 (all
// memory-bound or tiny: no MFMA), and the FMA mode product for row counts the
// MFMA tiles do not divide.
#include <math.h>

#include "kernels.h"

namespace shp {
namespace {

__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// fp32 -> bfloat16, round to nearest, ties to even (NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// A block's geometry in registers: K is the order (compile-time, so every
// per-dimension array is indexed by constants and stays in registers).
template <int K>
struct BlockGeo {
  int b[K], ext[K];
  uint64_t magic[K];
  int64_t base;        // element offset of the block's origin
  int64_t stride[K];
  __device__ __forceinline__ void load(const TensorGeom& g, const TBlockMeta& bm,
                                       const TensorMeta& tm) {
    base = 0;
#pragma unroll
    for (int d = 0; d < K; ++d) {
      b[d] = g.b[d];
      magic[d] = g.magic[d];
      ext[d] = bm.extent[d];
      stride[d] = tm.stride[d];
      base += (int64_t)bm.origin[d] * tm.stride[d];
    }
  }
  // Offset of packed element e from the tensor's start, and whether it lies
  // inside the block's real extent. The index divisions are multiply-highs
  // with the host's magic numbers (a runtime integer division would dominate
  // this memory-bound kernel).
  __device__ __forceinline__ bool offset(int e, int64_t& off) const {
    off = base;
    bool in = true;
#pragma unroll
    for (int d = K - 1; d >= 0; --d) {
      int i = e;
      if (d > 0) {
        const int q = magic[d] == 0 ? e : (int)__umul64hi((uint64_t)(uint32_t)e, magic[d]);
        i = e - q * b[d];
        e = q;
      }
      in = in && i < ext[d];
      off += (int64_t)i * stride[d];
    }
    return in;
  }
  // Indices of packed element e (the last dimension fastest), the offset and
  // real-extent test of an index, and the next element in packed order: a
  // thread that takes consecutive elements decomposes only the first.
  __device__ __forceinline__ void indices(int e, int (&idx)[K]) const {
#pragma unroll
    for (int d = K - 1; d > 0; --d) {
      const int q = magic[d] == 0 ? e : (int)__umul64hi((uint64_t)(uint32_t)e, magic[d]);
      idx[d] = e - q * b[d];
      e = q;
    }
    idx[0] = e;
  }
  __device__ __forceinline__ bool at(const int (&idx)[K], int64_t& off) const {
    off = base;
    bool in = true;
#pragma unroll
    for (int d = 0; d < K; ++d) {
      in = in && idx[d] < ext[d];
      off += (int64_t)idx[d] * stride[d];
    }
    return in;
  }
  __device__ __forceinline__ void step(int (&idx)[K]) const {
#pragma unroll
    for (int d = K - 1; d >= 0; --d) {
      if (++idx[d] < b[d]) return;
      idx[d] = 0;
    }
  }
};

// floor(i / d) for 0 <= i < 2^22 and d >= 1, from inv = 1 / d: the float
// quotient is within one of the integer one, which the correction fixes.
__device__ __forceinline__ int div_small(int i, int d, float inv) {
  int q = (int)((float)i * inv);
  if (q * d > i)
    --q;
  else if ((q + 1) * d <= i)
    ++q;
  return q;
}

template <int K>
__global__ __launch_bounds__(256) void tensor_pack_kernel(const TBlockMeta* __restrict__ blocks,
                                                          const TensorMeta* __restrict__ tensors,
                                                          TensorGeom g, int bf16,
                                                          float* __restrict__ Gp,
                                                          float* __restrict__ Mom, float momentum,
                                                          MaxOut mo) {
  const int b = blockIdx.y;
  float mg = 0.f, mm = 0.f;  // largest |value| written to Gp and Mom
  const TBlockMeta bm = blocks[b];
  BlockGeo<K> geo;
  geo.load(g, bm, tensors[bm.tensor]);
  const void* grad = tensors[bm.tensor].grad;
  if ((g.E & 3) == 0) {
    // four consecutive elements a thread: one index decomposition, 16-byte
    // stores of the packed block (and momentum). Four grid-stride steps'
    // loads are issued before their stores: a load written after a store
    // stays behind it, and the wait for it would cover the store.
    const int stride = gridDim.x * 256 * 4;
    for (int e0 = (blockIdx.x * 256 + threadIdx.x) * 4; e0 < g.E; e0 += 4 * stride) {
      float v[4][4], mv[4][4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int e = e0 + u * stride;
        if (e >= g.E) break;
        int idx[K];
        geo.indices(e, idx);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          int64_t off;
          v[u][q] = 0.f;
          if (geo.at(idx, off))
            v[u][q] = bf16 ? bf16_to_f32(reinterpret_cast<const uint16_t*>(grad)[off])
                           : reinterpret_cast<const float*>(grad)[off];
          if (q < 3) geo.step(idx);
        }
        if (Mom != nullptr) {
          const float4 m = *reinterpret_cast<const float4*>(Mom + (size_t)b * g.E + e);
          mv[u][0] = m.x;
          mv[u][1] = m.y;
          mv[u][2] = m.z;
          mv[u][3] = m.w;
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int e = e0 + u * stride;
        if (e >= g.E) break;
        const size_t o = (size_t)b * g.E + e;
        *reinterpret_cast<float4*>(Gp + o) = make_float4(v[u][0], v[u][1], v[u][2], v[u][3]);
        mg = fmaxf(mg, fmaxf(fmaxf(fabsf(v[u][0]), fabsf(v[u][1])),
                             fmaxf(fabsf(v[u][2]), fabsf(v[u][3]))));
        if (Mom != nullptr) {
          float4 m;
          m.x = momentum * mv[u][0] + v[u][0];
          m.y = momentum * mv[u][1] + v[u][1];
          m.z = momentum * mv[u][2] + v[u][2];
          m.w = momentum * mv[u][3] + v[u][3];
          *reinterpret_cast<float4*>(Mom + o) = m;
          mm = fmaxf(mm, fmaxf(fmaxf(fabsf(m.x), fabsf(m.y)), fmaxf(fabsf(m.z), fabsf(m.w))));
        }
      }
    }
  } else {
    for (int e = blockIdx.x * 256 + threadIdx.x; e < g.E; e += gridDim.x * 256) {
      int64_t off;
      float v = 0.f;
      if (geo.offset(e, off))
        v = bf16 ? bf16_to_f32(reinterpret_cast<const uint16_t*>(grad)[off])
                 : reinterpret_cast<const float*>(grad)[off];
      const size_t o = (size_t)b * g.E + e;
      Gp[o] = v;
      mg = fmaxf(mg, fabsf(v));
      if (Mom != nullptr) {
        const float m = momentum * Mom[o] + v;
        Mom[o] = m;
        mm = fmaxf(mm, fabsf(m));
      }
    }
  }
  if (mo.a != nullptr || mo.b != nullptr)
    raise_max2_wg<256>(mo.a != nullptr ? mo.a + b : nullptr, mg,
                       mo.b != nullptr ? mo.b + b : nullptr, mm, mo.ver);
}

template <int K>
__global__ __launch_bounds__(256) void tensor_scatter_kernel(const TBlockMeta* __restrict__ blocks,
                                                             const TensorMeta* __restrict__ tensors,
                                                             TensorGeom g,
                                                             const float* __restrict__ Src, float lr,
                                                             int bf16, int update) {
  const int b = blockIdx.y;
  const TBlockMeta bm = blocks[b];
  BlockGeo<K> geo;
  geo.load(g, bm, tensors[bm.tensor]);
  void* param = tensors[bm.tensor].param;
  for (int e = blockIdx.x * 256 + threadIdx.x; e < g.E; e += gridDim.x * 256) {
    int64_t off;
    if (!geo.offset(e, off)) continue;
    const float u = Src[(size_t)b * g.E + e];
    if (!update) {
      reinterpret_cast<float*>(param)[off] = u;
    } else if (bf16) {
      uint16_t* w = reinterpret_cast<uint16_t*>(param) + off;
      *w = f32_to_bf16(bf16_to_f32(*w) - lr * u);
    } else {
      float* w = reinterpret_cast<float*>(param) + off;
      *w = *w - lr * u;
    }
  }
}

// Batched transpose through LDS. A tile is TH x TW of the input (TW <= 64,
// TH * (TW | 1) <= 4096), elements taken in linear order on both sides so that
// thin matrices (a handful of columns) still read and write whole lines.
__global__ __launch_bounds__(256) void transpose_kernel(const float* __restrict__ In,
                                                        int64_t in_stride, float* __restrict__ Out,
                                                        int64_t out_stride, int R, int C, int TH,
                                                        int TW) {
  __shared__ float tile[4096 + 64];
  const int b = blockIdx.y;
  const int tcn = (C + TW - 1) / TW;
  const int r0 = (blockIdx.x / tcn) * TH, c0 = (blockIdx.x % tcn) * TW;
  const int th = min(TH, R - r0), tw = min(TW, C - c0);
  const int pitch = tw | 1;  // odd pitch: column reads spread over the banks
  const float* in = In + (size_t)b * in_stride;
  float* out = Out + (size_t)b * out_stride;
  // tile-local indices by a float reciprocal and one correction (an integer
  // division per element would bound this memory-bound kernel)
  const float itw = 1.f / (float)tw, ith = 1.f / (float)th;
  for (int i = threadIdx.x; i < th * tw; i += 256) {
    const int r = div_small(i, tw, itw), c = i - r * tw;
    tile[r * pitch + c] = in[(size_t)(r0 + r) * C + c0 + c];
  }
  __syncthreads();
  for (int i = threadIdx.x; i < th * tw; i += 256) {
    const int c = div_small(i, th, ith), r = i - c * th;
    out[(size_t)(c0 + c) * R + r0 + r] = tile[r * pitch + c];
  }
}

__global__ __launch_bounds__(256) void fill_zero_kernel(float* __restrict__ Out, int64_t stride,
                                                        int64_t from) {
  float* out = Out + (size_t)blockIdx.y * stride;
  for (int64_t e = from + blockIdx.x * 256 + threadIdx.x; e < stride; e += gridDim.x * 256)
    out[e] = 0.f;
}

// Pair (l, l') with l <= l' of an n x n symmetric statistic, packed row by row.
constexpr int kMaxPairs = kMaxSmallSide * (kMaxSmallSide + 1) / 2;

template <int N>
__global__ __launch_bounds__(256) void small_gram_kernel(const float* __restrict__ In,
                                                         int64_t in_stride, int A, int C,
                                                         float* __restrict__ partial) {
  constexpr int NP = N * (N + 1) / 2;
  __shared__ float red[4][NP];
  const int b = blockIdx.y;
  const float* in = In + (size_t)b * in_stride;
  float acc[NP];
#pragma unroll
  for (int q = 0; q < NP; ++q) acc[q] = 0.f;
  const int64_t total = (int64_t)A * C;
  for (int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x; q < total;
       q += (int64_t)gridDim.x * 256) {
    const int64_t a = q / C, c = q - a * C;
    const float* src = in + (size_t)a * N * C + c;
    float v[N];
#pragma unroll
    for (int l = 0; l < N; ++l) v[l] = src[(size_t)l * C];
    int k = 0;
#pragma unroll
    for (int l = 0; l < N; ++l)
#pragma unroll
      for (int m = l; m < N; ++m) acc[k++] += v[l] * v[m];
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int q = 0; q < NP; ++q) {
    float x = acc[q];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
    if (lane == 0) red[wave][q] = x;
  }
  __syncthreads();
  for (int q = threadIdx.x; q < NP; q += 256)
    partial[((size_t)b * gridDim.x + blockIdx.x) * kMaxPairs + q] =
        red[0][q] + red[1][q] + red[2][q] + red[3][q];
}

// Both statistics of two small trailing dimensions of one side N in one pass:
// the block is [A][N][N] (slices S_a of N x N contiguous values). Dimension
// k - 2 sums S_a[l][c] S_a[m][c] over a and c, dimension k - 1 sums
// S_a[c][l] S_a[c][m]; their pairs go to q < NP and NP <= q < 2 NP of the
// chunk's partial row. Each workgroup stages its 256 slices through LDS, so
// the block is read in whole lines.
template <int N>
__global__ __launch_bounds__(256) void small_gram2_kernel(const float* __restrict__ In,
                                                          int64_t in_stride, int A,
                                                          float* __restrict__ partial) {
  constexpr int NN = N * N, NP = N * (N + 1) / 2;
  static_assert(2 * NP <= kMaxPairs, "pairs of both dimensions must fit one partial row");
  __shared__ __align__(16) float tile[256 * NN];
  __shared__ float red[4][2 * NP];
  const int b = blockIdx.y;
  const float* in = In + (size_t)b * in_stride;
  float acc[2 * NP];
#pragma unroll
  for (int q = 0; q < 2 * NP; ++q) acc[q] = 0.f;
  for (int64_t a0 = (int64_t)blockIdx.x * 256; a0 < A; a0 += (int64_t)gridDim.x * 256) {
    const int cnt = (int)min((int64_t)256, A - a0) * NN;
    __syncthreads();  // the previous slices have been read
    const float* src = in + a0 * NN;
    if ((in_stride & 3) == 0) {
      // 16-byte loads: 256 N N floats per step keep a0 N N a multiple of 4
      const int c4 = cnt >> 2;
      for (int e = threadIdx.x; e < c4; e += 256)
        reinterpret_cast<float4*>(tile)[e] = reinterpret_cast<const float4*>(src)[e];
      for (int e = 4 * c4 + threadIdx.x; e < cnt; e += 256) tile[e] = src[e];
    } else {
      for (int e = threadIdx.x; e < cnt; e += 256) tile[e] = src[e];
    }
    __syncthreads();
    if (a0 + threadIdx.x < A) {
      float v[N][N];
#pragma unroll
      for (int l = 0; l < N; ++l)
#pragma unroll
        for (int c = 0; c < N; ++c) v[l][c] = tile[threadIdx.x * NN + l * N + c];
      int k = 0;
#pragma unroll
      for (int l = 0; l < N; ++l)
#pragma unroll
        for (int m = l; m < N; ++m, ++k) {
          float x = 0.f, y = 0.f;
#pragma unroll
          for (int c = 0; c < N; ++c) {
            x += v[l][c] * v[m][c];
            y += v[c][l] * v[c][m];
          }
          acc[k] += x;
          acc[NP + k] += y;
        }
    }
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int q = 0; q < 2 * NP; ++q) {
    float x = acc[q];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
    if (lane == 0) red[wave][q] = x;
  }
  __syncthreads();
  for (int q = threadIdx.x; q < 2 * NP; q += 256)
    partial[((size_t)b * gridDim.x + blockIdx.x) * kMaxPairs + q] =
        red[0][q] + red[1][q] + red[2][q] + red[3][q];
}

// H <- beta2 H + gamma * (sum of the chunk partials). One wave per block and
// statistic: lanes take chunks lane, lane + 64, ... and a shuffle tree adds
// the lanes, in fp64 and a fixed order (a serial sum per pair had been one
// chain of dependent loads). blockIdx.y = 1 forms a second statistic H2 from
// the pairs that follow the first's in the partial row.
__global__ __launch_bounds__(64) void small_gram_ema_kernel(const float* __restrict__ partial,
                                                            int chunks, int n, float* __restrict__ H,
                                                            float* __restrict__ H2, float beta2,
                                                            float gamma) {
  const int b = blockIdx.x;
  const int np = n * (n + 1) / 2;
  const int q0 = blockIdx.y * np;
  float* h = (blockIdx.y == 0 ? H : H2) + (size_t)b * n * n;
  const int lane = threadIdx.x;
  for (int q = 0; q < np; ++q) {
    double s = 0.0;
    for (int c = lane; c < chunks; c += 64) s += partial[((size_t)b * chunks + c) * kMaxPairs + q0 + q];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
    if (lane == 0) {
      // pair q -> (l, m), l <= m
      int l = 0, rem = q;
      while (rem >= n - l) {
        rem -= n - l;
        ++l;
      }
      const int m = l + rem;
      const float v = beta2 * h[l * n + m] + gamma * (float)s;
      h[l * n + m] = v;
      h[m * n + l] = v;
    }
  }
}

// Out[r][j] = sum_l X[j][l] In[l][r] for J output columns j0 .. j0 + J - 1 per
// thread; X is uniform over the workgroup (scalar loads). When one workgroup
// covers all n columns, the [256][n] output tile is contiguous and is staged
// through LDS to leave as whole lines.
template <int J>
__global__ __launch_bounds__(256) void mode_product_kernel(const float* __restrict__ In,
                                                           int64_t in_stride,
                                                           const float* __restrict__ X,
                                                           int64_t x_stride, float* __restrict__ Out,
                                                           int64_t out_stride, int n, int R,
                                                           MaxOut mo) {
  __shared__ float stage[256 * J];
  const int b = blockIdx.z;
  const float* in = In + (size_t)b * in_stride;
  const float* x = X + (size_t)b * x_stride;
  float* out = Out + (size_t)b * out_stride;
  const int r0 = blockIdx.x * 256;
  const int r = r0 + threadIdx.x;
  const int j0 = blockIdx.y * J;
  float acc[J];
#pragma unroll
  for (int jj = 0; jj < J; ++jj) acc[jj] = 0.f;
  if (r < R) {
    for (int l = 0; l < n; ++l) {
      const float v = in[(size_t)l * R + r];
#pragma unroll
      for (int jj = 0; jj < J; ++jj)
        if (j0 + jj < n) acc[jj] += x[(j0 + jj) * n + l] * v;
    }
  }
  if (mo.a != nullptr) {  // the output's maximum (uniform branch)
    float mx = 0.f;
#pragma unroll
    for (int jj = 0; jj < J; ++jj)
      if (r < R && j0 + jj < n) mx = fmaxf(mx, fabsf(acc[jj]));
    raise_max2_wg<256>(mo.a + b, mx, nullptr, 0.f, mo.ver);
  }
  if (gridDim.y == 1 && n == J) {
#pragma unroll
    for (int jj = 0; jj < J; ++jj) stage[threadIdx.x * J + jj] = acc[jj];
    __syncthreads();
    const int rows = min(256, R - r0);
    float* dst = out + (size_t)r0 * J;
    for (int i = threadIdx.x; i < rows * J; i += 256) dst[i] = stage[i];
    return;
  }
  if (r < R) {
#pragma unroll
    for (int jj = 0; jj < J; ++jj)
      if (j0 + jj < n) out[(size_t)r * n + j0 + jj] = acc[jj];
  }
}

// The last product of the chain (leading dimension k-1, extent J = n <= 8)
// with the parameter update in its epilogue: output row r is the packed
// position r * J of the block in its own order, so one offset per thread and
// W[off + j * stride_(k-1)] -= lr * U[r][j] for j inside the real extent.
template <int J, int K>
__global__ __launch_bounds__(256) void mode_product_update_kernel(
    const float* __restrict__ In, int64_t in_stride, const float* __restrict__ X, int64_t x_stride,
    const TBlockMeta* __restrict__ blocks, const TensorMeta* __restrict__ tensors, TensorGeom g,
    int R, float lr, int bf16) {
  const int b = blockIdx.z;
  const float* in = In + (size_t)b * in_stride;
  const float* x = X + (size_t)b * x_stride;
  const int r = blockIdx.x * 256 + threadIdx.x;
  if (r >= R) return;
  const TBlockMeta bm = blocks[b];
  BlockGeo<K> geo;
  geo.load(g, bm, tensors[bm.tensor]);
  int64_t off;
  if (!geo.offset(r * J, off)) return;
  float acc[J];
#pragma unroll
  for (int jj = 0; jj < J; ++jj) acc[jj] = 0.f;
#pragma unroll
  for (int l = 0; l < J; ++l) {
    const float v = in[(size_t)l * R + r];
#pragma unroll
    for (int jj = 0; jj < J; ++jj) acc[jj] += x[jj * J + l] * v;
  }
  const int64_t st = geo.stride[K - 1];
  const int ext = geo.ext[K - 1];
  void* param = tensors[bm.tensor].param;
  // every parameter loaded before the first store (a load written after a
  // store stays behind it, and the wait for it would cover the store)
  float wv[J];
#pragma unroll
  for (int jj = 0; jj < J; ++jj) {
    wv[jj] = 0.f;
    if (jj < ext)
      wv[jj] = bf16 ? bf16_to_f32(reinterpret_cast<const uint16_t*>(param)[off + jj * st])
                    : reinterpret_cast<const float*>(param)[off + jj * st];
  }
#pragma unroll
  for (int jj = 0; jj < J; ++jj) {
    if (jj >= ext) break;
    const float v = wv[jj] - lr * acc[jj];
    if (bf16)
      reinterpret_cast<uint16_t*>(param)[off + jj * st] = f32_to_bf16(v);
    else
      reinterpret_cast<float*>(param)[off + jj * st] = v;
  }
}

// The last two products of the chain fused with the parameter update, for two
// small trailing dimensions of equal side N. In is the block rotated to
// [N][N][R] (dimensions k - 2 and k - 1 first, the others after them in
// order); for every r, T[l3][j2] = sum_l2 X2[j2][l2] In[l2][l3][r], then
// U[r][j2][j3] = sum_l3 X3[j3][l3] T[l3][j2] (the two mode products of the
// chain in their order, T kept in fp32 registers where the unfused chain
// stores it as fp32), and W -= lr U on the block's real extent. One pass over
// the block instead of two.
template <int N, int K>
__global__ __launch_bounds__(256) void mode_product2_update_kernel(
    const float* __restrict__ In, int64_t in_stride, const float* __restrict__ X2,
    const float* __restrict__ X3, int64_t x_stride, const TBlockMeta* __restrict__ blocks,
    const TensorMeta* __restrict__ tensors, TensorGeom g, int R, float lr, int bf16) {
  constexpr int NN = N * N;
  __shared__ float su[256 * NN];    // U of the workgroup's 256 r, [r][j2][j3]
  __shared__ int64_t soff[256];     // parameter offset of (r, 0, 0), -1 outside
  const int b = blockIdx.z;
  const float* in = In + (size_t)b * in_stride;
  const float* x2 = X2 + (size_t)b * x_stride;
  const float* x3 = X3 + (size_t)b * x_stride;
  const int r = blockIdx.x * 256 + threadIdx.x;
  const TBlockMeta bm = blocks[b];
  BlockGeo<K> geo;
  geo.load(g, bm, tensors[bm.tensor]);
  int64_t off = -1;
  const bool ok = r < R && geo.offset(r * NN, off);
  if (ok) {
    float t[N][N];  // [l3][j2]
#pragma unroll
    for (int l3 = 0; l3 < N; ++l3)
#pragma unroll
      for (int j2 = 0; j2 < N; ++j2) t[l3][j2] = 0.f;
#pragma unroll
    for (int l2 = 0; l2 < N; ++l2)
#pragma unroll
      for (int l3 = 0; l3 < N; ++l3) {
        const float v = in[(size_t)(l2 * N + l3) * R + r];
#pragma unroll
        for (int j2 = 0; j2 < N; ++j2) t[l3][j2] += x2[j2 * N + l2] * v;
      }
#pragma unroll
    for (int j2 = 0; j2 < N; ++j2)
#pragma unroll
      for (int j3 = 0; j3 < N; ++j3) {
        float u = 0.f;
#pragma unroll
        for (int l3 = 0; l3 < N; ++l3) u += x3[j3 * N + l3] * t[l3][j2];
        su[threadIdx.x * NN + j2 * N + j3] = u;
      }
  }
  soff[threadIdx.x] = ok ? off : -1;
  __syncthreads();
  // The update, element e of the workgroup's 256 N N values per thread step:
  // with the tensor's natural strides consecutive threads reach consecutive
  // parameters. All N N parameters of a thread are loaded before the first
  // store (a load written after a store stays behind it, and the wait for it
  // would cover the store).
  const int64_t st2 = geo.stride[K - 2], st3 = geo.stride[K - 1];
  const int ext2 = geo.ext[K - 2], ext3 = geo.ext[K - 1];
  void* param = tensors[bm.tensor].param;
  int64_t po[NN];
  float wv[NN];
#pragma unroll
  for (int k = 0; k < NN; ++k) {
    const int e = threadIdx.x + 256 * k;
    const int rl = e / NN, jj = e - rl * NN, j2 = jj / N, j3 = jj - j2 * N;
    const int64_t o0 = soff[rl];
    po[k] = (o0 < 0 || j2 >= ext2 || j3 >= ext3) ? -1 : o0 + j2 * st2 + j3 * st3;
    wv[k] = 0.f;
    if (po[k] >= 0)
      wv[k] = bf16 ? bf16_to_f32(reinterpret_cast<const uint16_t*>(param)[po[k]])
                   : reinterpret_cast<const float*>(param)[po[k]];
  }
#pragma unroll
  for (int k = 0; k < NN; ++k) {
    if (po[k] < 0) continue;
    const float v = wv[k] - lr * su[threadIdx.x + 256 * k];
    if (bf16)
      reinterpret_cast<uint16_t*>(param)[po[k]] = f32_to_bf16(v);
    else
      reinterpret_cast<float*>(param)[po[k]] = v;
  }
}

// One thread per factor: cyclic Jacobi in fp64 on the factor's real extent,
// matrix and eigenvectors in this thread's slice of LDS.
constexpr int kJacobiThreads = 64;
constexpr int kJacobiSweeps = 30;

__global__ __launch_bounds__(kJacobiThreads) void small_root_kernel(
    const float* __restrict__ H, float* __restrict__ X, int n, int count,
    const int32_t* __restrict__ nreal, float floor, int p, int32_t* __restrict__ status,
    int32_t* __restrict__ final_iter, float* __restrict__ resid) {
  constexpr int S = kMaxSmallSide;
  __shared__ double sa[kJacobiThreads][S * S];
  __shared__ double sv[kJacobiThreads][S * S];
  const int f = blockIdx.x * kJacobiThreads + threadIdx.x;
  if (f >= count) return;
  double* a = sa[threadIdx.x];
  double* v = sv[threadIdx.x];
  const float* h = H + (size_t)f * n * n;
  float* x = X + (size_t)f * n * n;
  const int m = nreal[f];
  bool finite = true;
  double diag2 = 0.0;
  for (int i = 0; i < m; ++i)
    for (int j = 0; j < m; ++j) {
      // the stored statistic is symmetric up to fp32 rounding; use its average
      const double y = 0.5 * ((double)h[i * n + j] + (double)h[j * n + i]);
      finite = finite && isfinite(y);
      a[i * S + j] = y;
      v[i * S + j] = i == j ? 1.0 : 0.0;
      if (i == j) diag2 += y * y;
    }
  int sweeps = 0;
  double off = 0.0;
  for (; finite && sweeps < kJacobiSweeps; ++sweeps) {
    off = 0.0;
    for (int i = 0; i < m; ++i)
      for (int j = i + 1; j < m; ++j) off += a[i * S + j] * a[i * S + j];
    if (off <= 1e-32 * diag2) break;
    for (int P = 0; P < m; ++P)
      for (int Q = P + 1; Q < m; ++Q) {
        const double apq = a[P * S + Q];
        if (apq == 0.0) continue;
        // rotation in the (P, Q) plane that zeroes a[P][Q]
        const double th = (a[Q * S + Q] - a[P * S + P]) / (2.0 * apq);
        const double t = (th >= 0.0 ? 1.0 : -1.0) / (fabs(th) + sqrt(th * th + 1.0));
        const double c = 1.0 / sqrt(t * t + 1.0), s = t * c;
        for (int r = 0; r < m; ++r) {  // columns P, Q
          const double arp = a[r * S + P], arq = a[r * S + Q];
          a[r * S + P] = c * arp - s * arq;
          a[r * S + Q] = s * arp + c * arq;
        }
        for (int r = 0; r < m; ++r) {  // rows P, Q
          const double apr = a[P * S + r], aqr = a[Q * S + r];
          a[P * S + r] = c * apr - s * aqr;
          a[Q * S + r] = s * apr + c * aqr;
        }
        for (int r = 0; r < m; ++r) {
          const double vrp = v[r * S + P], vrq = v[r * S + Q];
          v[r * S + P] = c * vrp - s * vrq;
          v[r * S + Q] = s * vrp + c * vrq;
        }
      }
  }
  double w[S];
  // the spectrum of the exact statistic is >= floor = beta2^t eps; rounding
  // below it (or an underflowed floor) is lifted to keep the root finite
  const double lo = fmax((double)floor, 1e-30);
  for (int i = 0; i < m; ++i) w[i] = pow(fmax(a[i * S + i], lo), -1.0 / p);
  for (int i = 0; i < n; ++i)
    for (int j = 0; j < n; ++j) {
      double y = 0.0;
      if (i < m && j < m && finite)
        for (int q = 0; q < m; ++q) y += v[i * S + q] * w[q] * v[j * S + q];
      x[i * n + j] = (float)y;
    }
  status[f] = finite ? 1 : 3;
  final_iter[f] = sweeps;
  resid[f] = diag2 > 0.0 ? (float)sqrt(off / diag2) : 0.f;
}

}  // namespace

hipError_t launch_tensor_pack(const TBlockMeta* blocks, const TensorMeta* tensors, TensorGeom g,
                              int32_t B, int32_t grad_bf16, float* Gp, float* Mom, float momentum,
                              hipStream_t s, MaxOut mo) {
  if (B == 0 || g.E == 0) return hipSuccess;
  // with maxima, 16 elements a thread (fewer workgroups raising each word)
  const int per = mo.a != nullptr || mo.b != nullptr ? 4096 : 1024;
  const int chunks = std::max(1, std::min(1024, (g.E + per - 1) / per));
  const dim3 grid(chunks, B);
  switch (g.order) {
    case 2:
      hipLaunchKernelGGL(tensor_pack_kernel<2>, grid, dim3(256), 0, s, blocks, tensors, g,
                         grad_bf16, Gp, Mom, momentum, mo);
      break;
    case 3:
      hipLaunchKernelGGL(tensor_pack_kernel<3>, grid, dim3(256), 0, s, blocks, tensors, g,
                         grad_bf16, Gp, Mom, momentum, mo);
      break;
    case 4:
      hipLaunchKernelGGL(tensor_pack_kernel<4>, grid, dim3(256), 0, s, blocks, tensors, g,
                         grad_bf16, Gp, Mom, momentum, mo);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_tensor_scatter(const TBlockMeta* blocks, const TensorMeta* tensors, TensorGeom g,
                                 int32_t B, const float* Src, float lr, int32_t param_bf16,
                                 int32_t update, hipStream_t s) {
  if (B == 0 || g.E == 0) return hipSuccess;
  const int chunks = std::max(1, std::min(1024, (g.E + 1023) / 1024));
  const dim3 grid(chunks, B);
  switch (g.order) {
    case 2:
      hipLaunchKernelGGL(tensor_scatter_kernel<2>, grid, dim3(256), 0, s, blocks, tensors, g, Src,
                         lr, param_bf16, update);
      break;
    case 3:
      hipLaunchKernelGGL(tensor_scatter_kernel<3>, grid, dim3(256), 0, s, blocks, tensors, g, Src,
                         lr, param_bf16, update);
      break;
    case 4:
      hipLaunchKernelGGL(tensor_scatter_kernel<4>, grid, dim3(256), 0, s, blocks, tensors, g, Src,
                         lr, param_bf16, update);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_transpose(const float* In, int64_t in_stride, float* Out, int64_t out_stride,
                            int32_t R, int32_t C, int32_t B, hipStream_t s) {
  if (B == 0 || R == 0 || C == 0) return hipSuccess;
  const int TW = std::min(C, 64);
  const int TH = std::min(R, 4096 / (TW | 1));  // TH rows of pitch <= (TW | 1) fit the tile
  const int tiles = ((R + TH - 1) / TH) * ((C + TW - 1) / TW);
  hipLaunchKernelGGL(transpose_kernel, dim3(tiles, B), dim3(256), 0, s, In, in_stride, Out,
                     out_stride, R, C, TH, TW);
  const int64_t used = (int64_t)R * C;
  if (out_stride > used) {
    const int chunks = (int)std::min<int64_t>(64, (out_stride - used + 255) / 256);
    hipLaunchKernelGGL(fill_zero_kernel, dim3(chunks, B), dim3(256), 0, s, Out, out_stride, used);
  }
  return hipGetLastError();
}

hipError_t launch_small_gram(const float* In, int64_t in_stride, int32_t A, int32_t n, int32_t C,
                             int32_t B, float* partial, int32_t chunks, float* H, float beta2,
                             float gamma, hipStream_t s) {
  if (B == 0) return hipSuccess;
  const dim3 grid(chunks, B);
  switch (n) {
#define SHP_GRAM(N)                                                                              \
  case N:                                                                                        \
    hipLaunchKernelGGL(small_gram_kernel<N>, grid, dim3(256), 0, s, In, in_stride, A, C, partial); \
    break;
    SHP_GRAM(1) SHP_GRAM(2) SHP_GRAM(3) SHP_GRAM(4) SHP_GRAM(5) SHP_GRAM(6) SHP_GRAM(7) SHP_GRAM(8)
#undef SHP_GRAM
    default:
      return hipErrorInvalidValue;
  }
  hipLaunchKernelGGL(small_gram_ema_kernel, dim3(B, 1), dim3(64), 0, s, partial, chunks, n, H,
                     nullptr, beta2, gamma);
  return hipGetLastError();
}

hipError_t launch_small_gram2(const float* In, int64_t in_stride, int32_t A, int32_t n,
                              int32_t B, float* partial, int32_t chunks, float* H2, float* H3,
                              float beta2, float gamma, hipStream_t s) {
  if (B == 0) return hipSuccess;
  const dim3 grid(chunks, B);
  switch (n) {
#define SHP_GRAM2(N)                                                                            \
  case N:                                                                                       \
    hipLaunchKernelGGL(small_gram2_kernel<N>, grid, dim3(256), 0, s, In, in_stride, A, partial); \
    break;
    SHP_GRAM2(1) SHP_GRAM2(2) SHP_GRAM2(3) SHP_GRAM2(4) SHP_GRAM2(5)
#undef SHP_GRAM2
    default:
      return hipErrorInvalidValue;
  }
  hipLaunchKernelGGL(small_gram_ema_kernel, dim3(B, 2), dim3(64), 0, s, partial, chunks, n, H2,
                     H3, beta2, gamma);
  return hipGetLastError();
}

hipError_t launch_mode_product(const float* In, int64_t in_stride, const float* X, int64_t x_stride,
                               float* Out, int64_t out_stride, int32_t n, int32_t R, int32_t B,
                               hipStream_t s, MaxOut mo) {
  if (B == 0 || R == 0) return hipSuccess;
  const int gx = (R + 255) / 256;
  switch (n <= kMaxSmallSide ? n : 0) {
#define SHP_MP(N)                                                                               \
  case N:                                                                                       \
    hipLaunchKernelGGL(mode_product_kernel<N>, dim3(gx, 1, B), dim3(256), 0, s, In, in_stride, X, \
                       x_stride, Out, out_stride, n, R, mo);                                    \
    break;
    SHP_MP(1) SHP_MP(2) SHP_MP(3) SHP_MP(4) SHP_MP(5) SHP_MP(6) SHP_MP(7) SHP_MP(8)
#undef SHP_MP
    default:
      hipLaunchKernelGGL(mode_product_kernel<8>, dim3(gx, (n + 7) / 8, B), dim3(256), 0, s, In,
                         in_stride, X, x_stride, Out, out_stride, n, R, mo);
  }
  return hipGetLastError();
}

hipError_t launch_mode_product_update(const float* In, int64_t in_stride, const float* X,
                                      int64_t x_stride, const TBlockMeta* blocks,
                                      const TensorMeta* tensors, TensorGeom g, int32_t R, int32_t B,
                                      float lr, int32_t param_bf16, hipStream_t s) {
  if (B == 0 || R == 0) return hipSuccess;
  const int n = g.b[g.order - 1];
  const dim3 grid((R + 255) / 256, 1, B);
  if (n < 1 || n > kMaxSmallSide || g.order < 2 || g.order > 4) return hipErrorInvalidValue;
#define SHP_MPU(N, K)                                                                          \
  if (n == N && g.order == K) {                                                                \
    hipLaunchKernelGGL((mode_product_update_kernel<N, K>), grid, dim3(256), 0, s, In, in_stride, \
                       X, x_stride, blocks, tensors, g, R, lr, param_bf16);                    \
    return hipGetLastError();                                                                  \
  }
#define SHP_MPU_K(N) SHP_MPU(N, 2) SHP_MPU(N, 3) SHP_MPU(N, 4)
  SHP_MPU_K(1) SHP_MPU_K(2) SHP_MPU_K(3) SHP_MPU_K(4) SHP_MPU_K(5) SHP_MPU_K(6) SHP_MPU_K(7)
  SHP_MPU_K(8)
#undef SHP_MPU_K
#undef SHP_MPU
  return hipErrorInvalidValue;
}

hipError_t launch_mode_product2_update(const float* In, int64_t in_stride, const float* X2,
                                       const float* X3, int64_t x_stride,
                                       const TBlockMeta* blocks, const TensorMeta* tensors,
                                       TensorGeom g, int32_t R, int32_t B, float lr,
                                       int32_t param_bf16, hipStream_t s) {
  if (B == 0 || R == 0) return hipSuccess;
  if (g.order < 2 || g.order > 4) return hipErrorInvalidValue;
  const int n = g.b[g.order - 1];
  if (g.b[g.order - 2] != n) return hipErrorInvalidValue;
  const dim3 grid((R + 255) / 256, 1, B);
#define SHP_MP2(N, K)                                                                          \
  if (n == N && g.order == K) {                                                                \
    hipLaunchKernelGGL((mode_product2_update_kernel<N, K>), grid, dim3(256), 0, s, In,          \
                       in_stride, X2, X3, x_stride, blocks, tensors, g, R, lr, param_bf16);    \
    return hipGetLastError();                                                                  \
  }
#define SHP_MP2_K(N) SHP_MP2(N, 2) SHP_MP2(N, 3) SHP_MP2(N, 4)
  SHP_MP2_K(1) SHP_MP2_K(2) SHP_MP2_K(3) SHP_MP2_K(4) SHP_MP2_K(5)
#undef SHP_MP2_K
#undef SHP_MP2
  return hipErrorInvalidValue;
}

hipError_t launch_small_root(const float* H, float* X, int32_t n, int32_t count,
                             const int32_t* nreal, float floor, int32_t p, int32_t* status,
                             int32_t* final_iter, float* resid, hipStream_t s) {
  if (count == 0) return hipSuccess;
  if (n < 1 || n > kMaxSmallSide) return hipErrorInvalidValue;
  hipLaunchKernelGGL(small_root_kernel, dim3((count + kJacobiThreads - 1) / kJacobiThreads),
                     dim3(kJacobiThreads), 0, s, H, X, n, count, nreal, floor, p, status,
                     final_iter, resid);
  return hipGetLastError();
}

}  // namespace shp
