/*
 * shampoo.h - C ABI of the blocked Shampoo optimizer step for AMD Instinct
 * MI355X (gfx950).
 *
 * The method (page "Shampoo optimizer", section "Key Components" and the
 * matrix-case loop under it; podcast "Preconditioned Optimization Without
 * the Full Matrix Cost", cues 20-22): every weight matrix W (m x n) keeps a
 * left statistic L (m x m) and a right statistic R (n x n), both started at
 * eps * I. Each step takes the gradient G and
 *     L <- beta2 L + stat_scale G G^T,   R <- beta2 R + stat_scale G^T G,
 *     W <- W - lr * L^(-1/4) G R^(-1/4).
 * The inverse fourth roots are recomputed only every root_every steps and
 * reused in between (podcast cue 28). Matrices are cut into blocks of
 * block_rows x block_cols that are preconditioned independently and stacked
 * into one batch (DASH page, abstract); tail blocks are zero-padded.
 *
 * Roots come from a norm-scaled coupled Newton iteration for the inverse
 * p-th root, p = 4 (Guo and Higham, SIAM J. Matrix Anal. Appl. 28(3), 2006):
 * M = A / s, X = s^(-1/4) I, then repeatedly T = (5 I - M) / 4, X <- X T,
 * M <- T^4 M, until ||M - I||_F / sqrt(n) <= newton_tol, the residual stops
 * decreasing, or newton_max_iters iterations have run. By default (scale
 * mode 3) the iteration also scales M every step to lift its small
 * eigenvalues faster, and an iteration whose next residual is bounded below
 * newton_tol forms only X. Newton-DB and Chebyshev roots are selectable
 * (root_method).
 *
 * Conventions of every entry point:
 *  - Return value: SHAMPOO_OK (0) or one of the SHAMPOO_ERR_* codes below.
 *    No C++ exception crosses this boundary. On error a message is kept per
 *    thread (shampoo_last_error) and no device work has been enqueued unless
 *    the code is SHAMPOO_ERR_HIP.
 *  - Pointers named "device" are device (HBM) addresses owned by the caller;
 *    the library never allocates or frees device memory. "host" pointers are
 *    read during the call only.
 *  - hip_stream is a hipStream_t (NULL = the default stream). All device
 *    work is enqueued on it asynchronously; calls return before it runs.
 *    Only shampoo_get_status and shampoo_get_timing wait for the GPU. Host
 *    tables (block map, pointer arrays) reach the device inside kernel
 *    arguments, so no other call waits, also when the parameter or
 *    gradient pointers change from one step to the next.
 *  - Matrices are row-major with a leading dimension ld (elements) >= cols.
 *  - A handle is not thread-safe; separate handles are independent.
 *  - Device faults surface as SHAMPOO_ERR_HIP at a later synchronising call.
 */
#ifndef SHAMPOO_MI355X_H
#define SHAMPOO_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ------------------------------------------------------------------ codes */
enum {
  SHAMPOO_OK = 0,
  SHAMPOO_ERR_INVALID_ARG = 1,        /* NULL handle/pointer, bad size or value    */
  SHAMPOO_ERR_UNSUPPORTED = 2,        /* dtype, block shape or mode not supported   */
  SHAMPOO_ERR_WORKSPACE_TOO_SMALL = 3,
  SHAMPOO_ERR_MISALIGNED = 4,         /* pointer not aligned as documented          */
  SHAMPOO_ERR_NO_ROOTS = 5,           /* step needs roots but none were computed    */
  SHAMPOO_ERR_HIP = 6                 /* a HIP runtime call failed (message kept)   */
};

/* Storage types of gradients and parameters. Statistics and roots are fp32. */
typedef enum { SHAMPOO_F32 = 0, SHAMPOO_BF16 = 1 } shampoo_dtype_t;

/* How the fp32 matrix products (statistics of fp32 gradients, root
 * iterations, preconditioning) run on the matrix cores. */
typedef enum {
  SHAMPOO_GEMM_F32 = 0,        /* fp32 MFMA (32x32x2)                           */
  SHAMPOO_GEMM_SPLIT_BF16 = 1, /* each fp32 operand split exactly into three
                                  bf16 terms x = h + m + l; the six products
                                  hh, hm, mh, hl, mm, lh on the bf16 MFMA
                                  (32x32x16), each exact in fp32, accumulated
                                  in fp32: the dropped terms are below 2^-24
                                  of |x y|, so the result has fp32 accuracy,
                                  at 6/16 of the fp32 MFMA time              */
  SHAMPOO_GEMM_SPLIT_F16 = 2   /* each fp32 operand scaled by a power of two
                                  (exact) that puts its largest |value| in
                                  [2^14, 2^15), then split into two fp16
                                  terms x = h + l + d, |d| <= 2^-22 |x| (or
                                  2^-39 of the largest |value| for tiny x);
                                  the three products hh, hl, lh on the fp16
                                  MFMA (32x32x16), exact in fp32, accumulated
                                  in fp32 and scaled back (exact): errors of
                                  order 2^-21 |x y| per term, fp32 level, at
                                  3/16 of the fp32 MFMA time. Every kernel
                                  that writes a product operand records the
                                  binary exponent of its largest |value| per
                                  block or factor (64-bit words with a
                                  version that grows with every launch that
                                  writes them); the roots' words are part of
                                  the state (layout.root_maxima) (default)   */
} shampoo_fp32_gemm_t;

/* Flags of shampoo_step. */
enum {
  SHAMPOO_FORCE_REFRESH = 1u,   /* recompute roots this step whatever the schedule */
  SHAMPOO_NO_AUTO_REFRESH = 2u  /* never recompute roots this step                 */
};

/* One registered matrix: rows x cols, row-major, leading dimension ld
 * (elements, cols <= ld <= 2^26; shampoo_init rejects a larger ld with
 * SHAMPOO_ERR_INVALID_ARG). Parameters and gradients of a matrix share this
 * shape and ld. Pointers must be aligned to their element size; 16-byte aligned
 * matrices with ld % 4 == 0 are read with vector loads. */
typedef struct {
  int64_t rows, cols, ld;
} shampoo_matrix_desc_t;

/* Hyper-parameters. shampoo_config_default fills every field. The real
 * values are given in double and rounded once to fp32, the precision every
 * kernel computes in. */
typedef struct {
  int32_t block_rows, block_cols; /* block shape; each a multiple of 32, <= 4096 */
  double beta2;                   /* weight of the old statistic                 */
  double stat_scale;              /* weight of the new outer product; a negative
                                     value means 1 - beta2 (formed in double)    */
  double eps;                     /* L and R start at eps * I (> 0)              */
  double lr;                      /* step size                                   */
  int32_t root_every;             /* refresh at t = 1, 1+k, 1+2k...; 0 = only on
                                     SHAMPOO_FORCE_REFRESH / refresh_roots       */
  int32_t newton_max_iters;       /* iteration cap, 1..64                        */
  double newton_tol;              /* stop when ||M - I||_F / sqrt(n) <= tol; a
                                     value <= 0 runs exactly newton_max_iters     */
  int32_t newton_scale_mode;      /* 0: s = ||A||_F (spectrum of A/s in (0,1]);
                                     1: s = min(||A||_F, ||A||_inf) * 2/5
                                        (spectrum in (0, 5/2]);
                                     2: s = lam/2 with lam = ||A v_16||, sixteen
                                        power-iteration products from
                                        v_0 = 1/sqrt(n) (lam <= lam_max, so the
                                        spectrum of A/s is in (0, ~2.2] unless v_0
                                        is almost orthogonal to the top
                                        eigenvector); lam = 0 falls back to 1;
                                     3: mode 2's s, then the coupled Newton
                                        iteration scales itself every step: from
                                        the second iteration on M is scaled by
                                        mu in [1, 0.9 (p + 1)] (X by mu^(1/p))
                                        chosen to balance the scalar map at a
                                        tracked estimate of the spectrum's bottom
                                        (started from Rayleigh quotients, never
                                        below the smallest eigenvalue), until the
                                        estimate passes 0.75; residual stall and
                                        divergence tests apply to unscaled
                                        iterates only. Same limit, fewer
                                        iterations on ill-conditioned factors.
                                        Newton-DB treats 3 as 2               */
  int32_t param_dtype;            /* shampoo_dtype_t of the parameters           */
  int32_t grad_dtype;             /* shampoo_dtype_t of the gradients; with bf16
                                     gradients the statistics run on the bf16
                                     MFMA (the products of bf16 values are exact
                                     in fp32; fp32 accumulation)                */
  double momentum;                /* alpha of ordinary momentum folded in before
                                     preconditioning (podcast cue 28):
                                     m = alpha m + G, W -= lr L^(-1/4) m R^(-1/4);
                                     statistics use the raw G. 0 = off (default) */
  int32_t root_method;            /* 0: coupled Newton for the inverse 4th root
                                        (default);
                                     1: Newton-DB: two Denman-Beavers square-root
                                        stages in inverse-free form, Y1 ~ A~^(1/2),
                                        then Z2 ~ Y1^(-1/2) = A~^(-1/4) (a reading
                                        of the DASH page's solver); newton_*
                                        settings apply to each stage and the
                                        spectral targets of the scale modes are 1;
                                     2: Chebyshev: X = s^(-1/4) p(A/s), p the
                                        degree-cheb_degree interpolant of x^(-1/4)
                                        on [beta2^t eps / s, 1] at the Chebyshev
                                        points, s an upper bound of the spectrum
                                        (min(lam/0.55, ||A||_F, ||A||_inf)),
                                        evaluated by baby steps (T_2, T_3) and
                                        giant steps in T_3 (T_3k = T_k o T_3):
                                        2 + ceil((cheb_degree - 2) / 3)
                                        products, no iteration, no early exit;
                                        one more scratch buffer of the roots'
                                        size in the workspace                  */
  int32_t cheb_degree;            /* 2..1024, default 128                        */
  int32_t fp32_gemm;              /* shampoo_fp32_gemm_t; default
                                     SHAMPOO_GEMM_SPLIT_F16. Statistics of bf16
                                     gradients always take the bf16 MFMA
                                     directly; a tensor dimension whose
                                     unfolding pads to an odd multiple of 16
                                     keeps its statistics on the fp32 MFMA    */
} shampoo_config_t;

/* Byte offsets of the state inside the caller's workspace (for inspection
 * and checkpointing). Square blocks of side b: stats holds B left
 * statistics [B][b][b] followed by B right statistics; roots likewise.
 * For rectangular blocks the left part has side block_rows and the right
 * part side block_cols. grad_packed is [B][block_rows][block_cols] fp32,
 * the last packed gradient. */
typedef struct {
  int64_t n_blocks;
  int64_t grad_packed;    /* fp32 [B][br][bc]                                   */
  int64_t stats;          /* fp32 [B][br][br] then [B][bc][bc]                  */
  int64_t roots;          /* fp32, same layout as stats                         */
  int64_t newton_status;  /* int32 [2B]: per factor, 0 none 1 converged 2 stalled
                             3 diverged 4 capped (left factors first); 5 only
                             while a refresh is in flight (converges after one
                             more X-only iteration)                               */
  int64_t newton_iters;   /* int32 [2B]: iterations behind the kept root         */
  int64_t newton_scale;   /* fp32 [2B]: the scale s of the last refresh           */
  int64_t newton_residual; /* fp32 [2B]: ||M - I||_F / sqrt(n) of the kept iterate  */
  int64_t momentum;       /* fp32 [B][br][bc] momentum, or -1 when it is off         */
  int64_t workspace_bytes;
  int64_t root_maxima;    /* fp32_gemm = SHAMPOO_GEMM_SPLIT_F16 only, else -1:
                             uint64 per root, the versioned binary exponent of
                             its largest |value|, which the preconditioning
                             products scale by: [2B] for matrix handles (left
                             factors first), [nb B] for tensor handles (the
                             nb dimensions blocked at a multiple of 32, in order;
                             smaller dimensions take no MFMA product). Part of
                             the state: a checkpoint keeps it with the roots,
                             and a restore writes both (shampoo_restore)       */
} shampoo_layout_t;

/* Accumulated kernel time per class while timing is enabled (milliseconds,
 * measured with HIP events on the stream the kernels run on) and the
 * algorithmic flop and byte counts of the launches timed. Classes: 0 pack,
 * 1 statistics (MFMA), 2 norms, 3 root products (MFMA), 4 root bookkeeping
 * (init, checks, final copy; small-side roots of tensors), 5 apply (MFMA
 * products and the fused parameter update), 6 memory-bound statistics
 * kernels of tensor handles (transposed unfoldings, small-side reductions),
 * 7 memory-bound apply kernels of tensor handles (FMA mode products, update
 * scatter). */
#define SHAMPOO_TIMING_CLASSES 8
typedef struct {
  double ms[SHAMPOO_TIMING_CLASSES];
  double flops[SHAMPOO_TIMING_CLASSES];
  double bytes[SHAMPOO_TIMING_CLASSES];
  int64_t launches[SHAMPOO_TIMING_CLASSES];
} shampoo_timing_t;

typedef struct shampoo_ctx* shampoo_t;

/* Fill *cfg with the defaults: square blocks of 1024, beta2 0.999,
 * stat_scale 1 - beta2, eps 1e-6, lr 1e-3, root_every 10, 25 Newton
 * iterations at most, tol 1e-6, scale mode 3, fp32 parameters and gradients,
 * no momentum, coupled Newton roots (Chebyshev degree 128 if selected). */
int shampoo_config_default(shampoo_config_t* cfg);

/* Bytes of device workspace needed for these matrices (host only, no HIP
 * call). mats: host array of n_mats descriptors. */
int shampoo_workspace_size(const shampoo_config_t* cfg, const shampoo_matrix_desc_t* mats,
                           int32_t n_mats, size_t* bytes_out);

/* Create a handle. workspace: device buffer of at least workspace_size
 * bytes, 256-byte aligned, owned by the caller and kept alive and unmoved
 * until shampoo_destroy. Enqueues on hip_stream the upload of the block map
 * and the start state L = R = eps I (page "Shampoo optimizer", matrix-case
 * loop: both statistics start at eps times the identity before the first
 * gradient); the step counter starts at 0 with no roots. *out receives the
 * handle. Returns without waiting for the enqueued work. */
int shampoo_init(const shampoo_config_t* cfg, const shampoo_matrix_desc_t* mats, int32_t n_mats,
                 void* workspace, size_t workspace_bytes, void* hip_stream, shampoo_t* out);

/* One optimizer step (page "Shampoo optimizer", matrix-case loop).
 * params: host array of n_mats device pointers, updated in place.
 * grads:  host array of n_mats device pointers, read only.
 * Packs the gradient blocks, updates L and R, recomputes the roots when the
 * schedule (or SHAMPOO_FORCE_REFRESH) asks, then applies
 * W -= lr * L^(-1/4) G R^(-1/4) on every block's real extent.
 * SHAMPOO_ERR_NO_ROOTS if roots are needed and SHAMPOO_NO_AUTO_REFRESH
 * forbids computing them. The step counter t is incremented on success. */
int shampoo_step(shampoo_t h, void* const* params, const void* const* grads, uint32_t flags,
                 void* hip_stream);

/* Recompute the roots L^(-1/4) and R^(-1/4) of every block from the
 * current L and R, as a step does on its refresh schedule (podcast
 * "Preconditioned Optimization Without the Full Matrix Cost", cue 28: the
 * roots are expensive and are recomputed only every few steps, reused in
 * between). The solver is root_method: by default the norm-scaled coupled
 * Newton iteration for the inverse 4th root (described at the top of this
 * file), a chain of symmetric matrix products on the matrix cores; a factor
 * whose iteration diverges gets status "diverged" and keeps finite roots
 * (shampoo_get_status counts them). Later steps use the new roots. */
int shampoo_refresh_roots(shampoo_t h, void* hip_stream);

/* Release the handle (host memory only; the workspace stays the caller's).
 * Waits for nothing: the caller must not free the workspace while work that
 * uses it is still queued. */
int shampoo_destroy(shampoo_t h);

/* ------------------------------------------------------ inspection hooks */
int shampoo_state_layout(shampoo_t h, shampoo_layout_t* out);
int shampoo_get_step(shampoo_t h, int64_t* t_out);
int shampoo_set_step(shampoo_t h, int64_t t);

/* Checkpoint restore, after the caller has written the state regions of
 * shampoo_state_layout (stats, roots, root_maxima when present, momentum
 * when on, the four Newton records) from a checkpoint taken at step t of a
 * handle with the same configuration and matrices: sets the step counter to
 * t and, for t > 0, takes the restored roots as current, so the next step
 * uses them unless the schedule refreshes them. With root_maxima present it
 * enqueues on hip_stream (after the caller's copies) one small kernel that
 * gives every maximum word this handle's current version, keeping its
 * exponent. The following steps then match the uninterrupted run bit for
 * bit. */
int shampoo_restore(shampoo_t h, int64_t t, void* hip_stream);

/* Pack alone: gather the gradient blocks into grad_packed (zero-padded). */
int shampoo_pack(shampoo_t h, const void* const* grads, void* hip_stream);

/* Unpack alone: write every block's real extent of grad_packed into dst
 * (host array of n_mats device pointers, fp32, the registered shapes/ld). */
int shampoo_unpack(shampoo_t h, void* const* dst, void* hip_stream);

/* Two-sided product alone: out (device, fp32 [B][br][bc]) receives
 * L^(-1/4) Gp R^(-1/4) of every block from the current packed gradient (the
 * momentum buffer when momentum is on) and roots; parameters are not
 * touched. */
int shampoo_precondition(shampoo_t h, void* out, void* hip_stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * result as shampoo_precondition, bit for bit, with the intermediate X_L Gp
 * (and its per-block maximum words on the fp16 split) kept in scratch memory
 * the library holds instead of in the workspace: a static device array of 64
 * MiB per GPU, alive until the process ends. Matrix handles only
 * (SHAMPOO_ERR_UNSUPPORTED for a tensor handle, and for a handle whose
 * intermediate, 4 * n_blocks * block_rows * block_cols bytes rounded up to
 * 256 plus 8 * n_blocks, exceeds 64 MiB). Calls no hipMalloc or other
 * allocating routine. Every call on one GPU shares that GPU's scratch:
 * calls that overlap on one GPU (other streams, other threads) race; calls
 * on one stream are ordered. */
int shampoo_precondition_noalloc(shampoo_t h, void* out, void* hip_stream);

/* Number of factors whose last Newton run diverged (non-finite or growing
 * residual). Synchronises hip_stream. */
int shampoo_get_status(shampoo_t h, void* hip_stream, int32_t* n_diverged_out);

/* Kernel timing with HIP events recorded on the stream of each launch (off
 * by default). Enabling clears the accumulators (the device flop counter is
 * cleared on hip_stream). shampoo_get_timing waits for the recorded events
 * and then reads the device flop counter of the Newton products. */
int shampoo_set_timing(shampoo_t h, int32_t enable, void* hip_stream);
int shampoo_get_timing(shampoo_t h, shampoo_timing_t* out);

const char* shampoo_status_string(int status);
const char* shampoo_last_error(void);

/* ------------------------------------------------------ order-k tensors
 * Podcast "Preconditioned Optimization Without the Full Matrix Cost", cue 26
 * (the order-k algorithm): a parameter tensor of order k keeps one statistic
 * per dimension i, H_i (n_i x n_i), started at eps * I and updated as
 *     H_i <- beta2 H_i + stat_scale G_(i) G_(i)^T
 * with G_(i) the mode-i unfolding of the gradient (rows: dimension i,
 * columns: all the others); the update is
 *     W <- W - lr * G x_1 H_1^(-1/2k) x_2 ... x_k H_k^(-1/2k),
 * x_i the product along dimension i (the products commute). k = 2 is the
 * matrix method above. Refresh schedule, momentum, dtypes and the root
 * settings of shampoo_config_t apply unchanged, with p = 2k; block_rows and
 * block_cols are not read.
 *
 * Blocks: dimension i is cut at block_dims[i]; a block is packed as a dense
 * row-major [block_dims[0]]...[block_dims[k-1]] fp32 array, zero past its
 * real extent. Every block_dims[i] is either 1..8 ("small": statistics and
 * mode products by memory-bound kernels, roots by an fp64 eigendecomposition)
 * or a multiple of 32 up to 4096 (statistics by the MFMA SYRK, roots by the
 * selected solver on the MFMA core, products by MFMA when the product of
 * the other block sizes is a multiple of 32). A packed block holds at most
 * 2^30 elements. root_method 1 (Newton-DB) needs k = 2.
 *
 * Handles made by shampoo_tensor_init take the same calls as matrix handles:
 * shampoo_step / refresh_roots / pack / unpack / precondition / get_status /
 * timing / state_layout / destroy, with one pointer per registered tensor
 * wherever the matrix calls take one per matrix. shampoo_precondition writes
 * [B][E] fp32 (E = product of block_dims). In shampoo_layout_t, stats and
 * roots point at the first statistic of the first dimension (see
 * shampoo_tensor_info for each dimension's place) and the per-factor arrays
 * hold k * B entries. */
#define SHAMPOO_MAX_ORDER 4

/* One registered tensor: extents and element strides (>= 1) of each of its
 * `order` dimensions; parameters and gradients share them. */
typedef struct {
  int32_t order;
  int64_t dims[SHAMPOO_MAX_ORDER];
  int64_t strides[SHAMPOO_MAX_ORDER];
} shampoo_tensor_desc_t;

/* Where each dimension's state lives (byte offsets into the workspace). */
typedef struct {
  int32_t order;
  int32_t block_dims[SHAMPOO_MAX_ORDER];
  int64_t n_blocks;
  int64_t block_elems;                    /* E                                   */
  int64_t stats[SHAMPOO_MAX_ORDER];       /* fp32 [B][n_i][n_i], n_i = block_dims[i] */
  int64_t roots[SHAMPOO_MAX_ORDER];       /* fp32 [B][n_i][n_i]                    */
  int32_t factor_group[SHAMPOO_MAX_ORDER]; /* dimension i's factors sit at entries
                                             [g B, (g + 1) B) of the per-factor
                                             arrays, g = factor_group[i]         */
} shampoo_tensor_info_t;

/* Bytes of device workspace for these tensors (host only, no HIP call).
 * block_dims: host array of `order` block sizes (2 <= order <= 4); tensors:
 * host array of n_tensors descriptors, each of that order. */
int shampoo_tensor_workspace_size(const shampoo_config_t* cfg, int32_t order,
                                  const int32_t* block_dims, const shampoo_tensor_desc_t* tensors,
                                  int32_t n_tensors, size_t* bytes_out);

/* Create a tensor handle; workspace, stream and start state as shampoo_init
 * (every H_i = eps I, t = 0, no roots). */
int shampoo_tensor_init(const shampoo_config_t* cfg, int32_t order, const int32_t* block_dims,
                        const shampoo_tensor_desc_t* tensors, int32_t n_tensors, void* workspace,
                        size_t workspace_bytes, void* hip_stream, shampoo_t* out);

/* Per-dimension layout of a tensor handle; SHAMPOO_ERR_INVALID_ARG for a
 * matrix handle. */
int shampoo_tensor_info(shampoo_t h, shampoo_tensor_info_t* out);

#ifdef __cplusplus
}
#endif
#endif /* SHAMPOO_MI355X_H */
