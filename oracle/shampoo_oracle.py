"""Oracle for the blocked Shampoo step: plain, slow, fp64, CPU only.

TEST INFRASTRUCTURE. Only the test suite, the package's smoke check and the
CPU-baseline leg of the benchmark may import this module. The product path
(the HIP library and its Python binding) never calls it, and this module
imports nothing from the product path. It shares no code with the kernels.

What it computes, and where the pages define it:

* Matrix Shampoo ("Shampoo optimizer" page, section "Key Components" and the
  simplified matrix-case loop under it; podcast "Preconditioned Optimization
  Without the Full Matrix Cost", cue 20): for a weight block W (m x n) with
  gradient G, keep a left statistic L (m x m) and a right statistic R (n x n),
  both started at eps * identity, accumulate G G^T into L and G^T G into R,
  and move W by -lr * L^(-1/4) G R^(-1/4).
* The statistics are an exponential moving average with weight beta2 on the
  old value and stat_scale (default 1 - beta2) on the new outer product, the
  form the SOAP record sweeps as beta_shampoo. beta2 = stat_scale = 1 gives
  the plain running sum of the "Shampoo optimizer" loop.
* The quarter power on each side (podcast cue 22) makes the two-sided product
  equal to the Kronecker preconditioner (L kron R)^(-1/4) applied to the
  row-major flattening of G. The oracle never uses that identity; the tests
  use it as an independent check.
* Roots are recomputed only every k steps and reused in between (podcast
  cue 28). Reading taken: the first step always computes roots, so refresh
  happens at steps t = 1, 1 + k, 1 + 2k, ...
* Optional momentum (podcast cue 28: ordinary momentum, alpha = 0.9, folded in
  before preconditioning). Reading taken: m_t = alpha m_{t-1} + G_t per block,
  statistics still accumulate the raw G_t, and the update is
  -lr L^(-1/4) m_t R^(-1/4).
* Gradients are cut into blocks that are stacked into a batch (DASH page,
  abstract). Reading taken: blocks of block_rows x block_cols in row-major
  block order inside a matrix, matrices in registration order; a tail block
  keeps its real (smaller) extent here, since zero padding decouples exactly.

Roots are the plain definition: the principal inverse p-th root of a
symmetric positive definite matrix from its symmetric eigendecomposition
(numpy.linalg.eigh, i.e. LAPACK). The GPU reaches the same matrix by an
iteration; the oracle also carries that iteration, written from its
published definition (coupled Newton for the inverse p-th root, Guo and
Higham, SIAM J. Matrix Anal. Appl. 28(3), 2006), for the fixed-iteration
workload and for tests of the iteration itself.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "BlockInfo",
    "block_table",
    "pack_blocks",
    "unpack_blocks",
    "update_statistics",
    "inverse_root_eigh",
    "newton_scale",
    "newton_map",
    "newton_balance",
    "spectrum_floor_estimate",
    "power_pair",
    "SCALED_PHASE_END",
    "final_step_bound",
    "inverse_root_coupled_newton",
    "db_scale",
    "sqrt_pair_db",
    "inverse_root_newton_db",
    "chebyshev_interval",
    "chebyshev_coefficients",
    "inverse_root_chebyshev",
    "precondition",
    "round_to_bf16",
    "is_refresh_step",
    "ShampooOracle",
]


# ---------------------------------------------------------------------------
# Block map (DASH page, abstract: preconditioner blocks stacked into a batch)
# ---------------------------------------------------------------------------
@dataclass(frozen=True)
class BlockInfo:
    """One block of one registered matrix.

    id:     position in the stacked batch.
    mat:    index of the matrix in registration order.
    bi, bj: block row / block column inside that matrix.
    r0, c0: first row / column of the block in the matrix.
    m, n:   real extent of the block (smaller than the block shape for tails).

    Pinned by: test_block_counts_of_the_workloads, test_pack_matches_elementwise_enumeration.
    """

    id: int
    mat: int
    bi: int
    bj: int
    r0: int
    c0: int
    m: int
    n: int


def block_table(shapes, block_rows, block_cols):
    """Enumerate the blocks of every matrix.

    Matrices keep registration order; inside a matrix, blocks go in row-major
    block order; a tail block keeps its real extent.

    Pinned by: test_block_counts_of_the_workloads (the workloads' block counts from their shapes),
        test_pack_matches_elementwise_enumeration (row-major order).
    """
    table = []
    for mat, (rows, cols) in enumerate(shapes):
        nbr = -(-rows // block_rows)
        nbc = -(-cols // block_cols)
        for bi in range(nbr):
            for bj in range(nbc):
                r0, c0 = bi * block_rows, bj * block_cols
                table.append(BlockInfo(len(table), mat, bi, bj, r0, c0,
                                       min(block_rows, rows - r0),
                                       min(block_cols, cols - c0)))
    return table


def pack_blocks(mats, table, block_rows, block_cols):
    """Stack every block into a [B, block_rows, block_cols] array.

    Values are copied unchanged (same dtype as the inputs); entries outside
    a tail block's real extent are +0.0.

    Pinned by: test_pack_matches_elementwise_enumeration (an independent per-element enumeration,
        zero tails), test_tail_blocks_equal_padded_blocks.
    """
    dtype = mats[0].dtype if mats else np.float32
    out = np.zeros((len(table), block_rows, block_cols), dtype=dtype)
    for b in table:
        out[b.id, :b.m, :b.n] = mats[b.mat][b.r0:b.r0 + b.m, b.c0:b.c0 + b.n]
    return out


def unpack_blocks(packed, table, shapes):
    """Inverse of pack_blocks: write each block's real extent back.

    Pinned by: test_pack_matches_elementwise_enumeration (the exact round trip).
    """
    mats = [np.zeros(s, dtype=packed.dtype) for s in shapes]
    for b in table:
        mats[b.mat][b.r0:b.r0 + b.m, b.c0:b.c0 + b.n] = packed[b.id, :b.m, :b.n]
    return mats


# ---------------------------------------------------------------------------
# Statistics ("Shampoo optimizer" page, matrix-case loop; podcast cue 20;
# EMA weight as in the SOAP record's beta_shampoo sweep)
# ---------------------------------------------------------------------------
def update_statistics(L, R, G, beta2, stat_scale):
    """L <- beta2 L + stat_scale G G^T ;  R <- beta2 R + stat_scale G^T G.

    Pinned by: test_statistics_closed_sum (the non-recursive sum), test_kronecker_bruteforce_tiny,
        test_first_step_svd_closed_form, test_two_by_two_example_all_ones.
    """
    G = np.asarray(G, dtype=np.float64)
    L_new = beta2 * L + stat_scale * (G @ G.T)
    R_new = beta2 * R + stat_scale * (G.T @ G)
    return L_new, R_new


# ---------------------------------------------------------------------------
# Inverse roots
# ---------------------------------------------------------------------------
def inverse_root_eigh(A, p=4):
    """Principal inverse p-th root of a symmetric positive definite matrix.

    A = Q diag(lam) Q^T  =>  A^(-1/p) = Q diag(lam^(-1/p)) Q^T.  A matrix
    that is not positive definite is an error, never silently clamped.

    Pinned by: test_inverse_root_2x2_analytic, test_invariants, test_scalar_one_by_one,
        test_diagonal_gradients_closed_form, test_kronecker_bruteforce_tiny.
    """
    A = np.asarray(A, dtype=np.float64)
    lam, Q = np.linalg.eigh(A)
    if not lam.min() > 0.0:
        raise np.linalg.LinAlgError(
            f"inverse root of a matrix that is not positive definite "
            f"(smallest eigenvalue {lam.min():.3e})")
    return (Q * lam ** (-1.0 / p)) @ Q.T


def _power_lambda(A, power_iters=8):
    """||A v_k|| after power_iters products from v_0 = 1 / sqrt(n) (0 if A v = 0).

    Pinned by: test_newton_scale_mode2_power_iteration (closed form on a diagonal matrix).
    """
    v = np.full(A.shape[0], 1.0 / math.sqrt(A.shape[0]))
    lam = 0.0
    for _ in range(power_iters):
        w = A @ v
        lam = float(np.sqrt(np.sum(w * w)))
        if lam == 0.0:
            break
        v = w / lam
    return lam


def newton_scale(A, p=4, mode=1, power_iters=8):
    """Norm used to scale A before the coupled Newton iteration.

    mode 0: s = ||A||_F, which puts the spectrum of A/s in (0, 1].
    mode 1: s = min(||A||_F, ||A||_inf) * 2 / (p + 1), which puts the
            spectrum of A/s in (0, (p + 1) / 2]; both norms bound the
            largest eigenvalue of a symmetric matrix.
    The DASH page (abstract) stresses that this scaling decides how fast
    Shampoo's root solver converges; the limit reached does not depend on it.
    mode 3: mode 2's s, and the iteration then scales itself every step
            (see newton_balance).
    mode 2: s = lam / 2, where lam is the power-iteration estimate of the
            largest eigenvalue: from v_0 = (1, ..., 1) / sqrt(n), repeat
            w = A v, lam = ||w||, v = w / lam, power_iters (8) times. For a
            symmetric A the ratios ||A^(j+1) v|| / ||A^j v|| never decrease, so
            lam >= lam_max * |c_1|^(1/8), c_1 the component of v_0 along the top
            eigenvector: the spectrum of A / s stays below 5 (the iteration's
            convergence region) unless |c_1| < 0.4^8 = 6.6e-4. If lam is 0,
            s falls back to min(||A||_F, ||A||_inf) * 2 / (p + 1).

    Pinned by: test_newton_scale_bounds_spectrum, test_newton_scale_mode2_power_iteration.
    """
    A = np.asarray(A, dtype=np.float64)
    fro = math.sqrt(float(np.sum(A * A)))
    if mode == 0:
        return fro
    inf = float(np.max(np.sum(np.abs(A), axis=1)))
    if mode == 1:
        return min(fro, inf) * 2.0 / (p + 1)
    if mode == 2:
        lam = _power_lambda(A, power_iters)
        return lam / 2.0 if lam > 0.0 else min(fro, inf) * 2.0 / (p + 1)
    if mode == 3:  # the start of mode 2; the iteration then scales itself
        return newton_scale(A, p, 2, power_iters)
    raise ValueError(f"unknown scale mode {mode}")


# ---------------------------------------------------------------------------
# Per-iteration scaling (scale mode 3)
#
# One coupled Newton iteration acts on every eigenvalue m of M through the
# scalar map f(m) = m ((p + 1 - m) / p)^p, which has its maximum 1 at m = 1
# and maps (0, p + 1) into (0, 1]. After the first iteration the spectrum
# lies in (0, 1], so M may be scaled by any mu in [1, 0.9 (p + 1)] (and X by
# mu^(1/p), keeping X^p A = M) without leaving the convergence region; a
# mu > 1 lifts the small eigenvalues, the slow ones, mu times faster, at the
# price of pulling the eigenvalues near 1 down to f(mu). With an estimate a
# of the bottom of the spectrum the best mu balances the two ends,
# f(mu a) = f(mu). The estimate starts from spectrum_floor_estimate (Rayleigh
# quotients, never below the smallest eigenvalue: the scaling can only err on
# the cautious side) and follows the scalar map. Scaling stops once the estimate passes
# SCALED_PHASE_END; the quadratic phase then runs unscaled. (A reading: the
# pages name no iteration; scaling the coupled iteration this way follows
# the scaled Newton methods for matrix roots in the numerical literature.)
# ---------------------------------------------------------------------------
SCALED_PHASE_END = 0.75
BALANCE_STEPS = 40


def power_pair(A, power_iters=8):
    """Top and bottom power iterations run side by side (one pass over A per
    step serves both): v_0 = (1, ..., 1) / sqrt(n) for the top, u_0 = (1, -1,
    1, ...) / sqrt(n) for the bottom; step j forms A v_j and A u_j, takes
    lam_j = ||A v_j||, v_(j+1) = A v_j / lam_j, the Rayleigh quotient
    q_j = u_j^T A u_j and u_(j+1) the normalised lam_j u_j - A u_j (a power
    step on lam_j I - A, whose top eigenvector is A's bottom one). Returns
    (lam_(P-1), q_(P-1)) for P = power_iters: lam is mode 2's estimate, q a
    Rayleigh quotient (never below the smallest eigenvalue).

    Pinned by: test_power_pair_top_matches_mode_2_and_bottom_converges.
    """
    A = np.asarray(A, dtype=np.float64)
    n = A.shape[0]
    v = np.full(n, 1.0 / math.sqrt(n))
    u = np.array([1.0 if i % 2 == 0 else -1.0 for i in range(n)]) / math.sqrt(n)
    lam, q = 0.0, math.inf
    for _ in range(power_iters):
        Av, Au = A @ v, A @ u
        lam = float(np.sqrt(np.sum(Av * Av)))
        q = float(u @ Au)
        if lam == 0.0:
            break
        v = Av / lam
        w = lam * u - Au
        nw = float(np.sqrt(np.sum(w * w)))
        if nw == 0.0:
            break
        u = w / nw
    return lam, q


def spectrum_floor_estimate(A, power_iters=8):
    """Estimate of the smallest eigenvalue of a symmetric A that is never
    below it: the smaller of the smallest diagonal entry and power_pair's
    Rayleigh quotient (both are Rayleigh quotients of A).

    Pinned by: test_spectrum_floor_estimate_bounds.
    """
    A = np.asarray(A, dtype=np.float64)
    return min(float(np.min(np.diag(A))), power_pair(A, power_iters)[1])


def newton_map(m, p, mu=1.0):
    """f(mu m) = mu m ((p + 1 - mu m) / p)^p.

    Pinned by: test_newton_map_shape (maximum 1 at the fixed point, the quadratic constant (p + 1) /
        (2 p)).
    """
    y = mu * m
    return y * ((p + 1 - y) / p) ** p


def newton_balance(a, p):
    """mu in [1, 0.9 (p + 1)] with f(mu a) = f(mu), by BALANCE_STEPS bisection
    steps (the lower end of the last bracket); 0.9 (p + 1) when f(mu a) < f(mu)
    holds even there.

    Pinned by: test_newton_balance_closed_form (closed-form balance point, an independent root
        finder, the cap).
    """
    lo, hi = 1.0, 0.9 * (p + 1)
    if newton_map(a, p, hi) < newton_map(1.0, p, hi):
        return hi
    for _ in range(BALANCE_STEPS):
        mid = 0.5 * (lo + hi)
        if newton_map(a, p, mid) < newton_map(1.0, p, mid):
            lo = mid
        else:
            hi = mid
    return lo


@dataclass
class NewtonInfo:
    iters: int
    residuals: list = field(default_factory=list)
    status: str = "capped"  # converged | stalled | diverged | capped
    mus: list = field(default_factory=list)  # scale of M at every iteration (1 unless mode 3)
    last_x_only: bool = False  # the last iteration formed only X (final_step_bound met tol)


FLOOR_GUARD = 1e-3  # a residual that grows from below this is at the rounding floor


# Residual below which rounding, not the iteration, sets ||M - I||_F / sqrt(n)
# (twice the unit roundoff of the precision computed in): a tolerance under it
# is not attainable, and the final-step bound is not trusted there.
ROUNDING_FLOOR = 2.0 * float(np.finfo(np.float64).eps)


def final_step_bound(r, n, p):
    """Bound on the residual after one more unscaled iteration from an
    iterate with residual r = ||M - I||_F / sqrt(n). Near the fixed point the
    scalar map sends 1 + e to 1 - C e^2 + O(e^3), C = (p + 1) / (2 p), and
    sum e^4 <= (sum e^2)^2, so the new residual is at most C sqrt(n) r^2 (to
    leading order). When this is already below tol the last iteration needs
    only X <- X T: M would be formed only to be checked. (A reading: the stop
    rule's tolerance is met by the bound instead of by a formed residual.)

    Pinned by: test_final_step_forms_only_x (the bound holds against the formed residual and the
        eigh root).
    """
    return (p + 1) / (2.0 * p) * math.sqrt(n) * r * r


def inverse_root_coupled_newton(A, p=4, max_iters=25, tol=0.0, scale_mode=1,
                                divergence_factor=1.2):
    """Coupled Newton iteration for A^(-1/p) (Guo and Higham 2006).

    Start from M = A / s and X = s^(-1/p) I. Each iteration forms
    T = ((p + 1) I - M) / p, then X <- X T and M <- T^p M; X tends to
    A^(-1/p) while M tends to I. The spectrum of M must start in (0, p + 1).

    Stopping: after each iteration the residual r = ||M - I||_F / sqrt(n) is
    compared with tol (stop, keep this X), with the previous residual (no
    decrease: stop, keep the previous X) and with divergence_factor times
    the previous residual (diverged: keep the previous X; only when the
    previous residual exceeds FLOOR_GUARD, since in exact arithmetic the
    residual shrinks every step and a growth from a small residual is the
    rounding floor). tol <= 0 runs exactly max_iters iterations and skips
    those tests; in both modes a non-finite residual stops the iteration and
    keeps the previous X.

    Pinned by: test_newton_converges_to_eigh, test_newton_orthogonal_similarity,
        test_newton_scalar_fixed_point_and_monotone, test_newton_guard_keeps_finite_iterate,
        test_scaled_newton_reaches_the_root, test_scaled_newton_diagonal_closed_form.
    """
    A = np.asarray(A, dtype=np.float64)
    n = A.shape[0]
    eye = np.eye(n)
    s = newton_scale(A, p, scale_mode)
    M = A / s
    X = s ** (-1.0 / p) * eye
    info = NewtonInfo(0)
    scaled = scale_mode == 3
    if scaled:
        # lower estimate of the spectrum of M after the first (unscaled)
        # iteration: f(a_0) for the smallest, f(b_0) for the largest eigenvalue
        # (b_0 = lam / s = 2, or (p + 1) / 2 when the fallback norm was used)
        lam = _power_lambda(A)
        b0 = 2.0 if lam > 0.0 else (p + 1) / 2.0
        a = min(newton_map(spectrum_floor_estimate(A) / s, p), newton_map(b0, p))
    mu = 1.0
    r_prev = math.inf
    for k in range(max_iters):
        Ms = mu * M
        T = ((p + 1) * eye - Ms) / p
        X_new = mu ** (1.0 / p) * X @ T
        M_new = np.linalg.matrix_power(T, p) @ Ms
        r = float(np.sqrt(np.sum((M_new - eye) ** 2)) / math.sqrt(n))
        info.residuals.append(r)
        info.mus.append(mu)
        if not math.isfinite(r):
            info.status = "diverged"
            break
        if tol > 0.0 and mu == 1.0:
            if r > divergence_factor * r_prev and r_prev > FLOOR_GUARD:
                info.status = "diverged"
                break
            if r >= r_prev:
                info.status = "stalled"
                break
        # a scaled iterate need not shrink the residual: accept it and start
        # the monotone checks afresh once the scaling has stopped
        X, M, r_prev = X_new, M_new, (r if mu == 1.0 else math.inf)
        info.iters = k + 1
        if tol > 0.0 and r <= tol:
            info.status = "converged"
            break
        mu_next = 1.0
        if scaled:
            mu_next = newton_balance(a, p) if a < SCALED_PHASE_END else 1.0
            a = newton_map(a, p, mu_next)
        if (tol > 0.0 and mu == 1.0 and mu_next == 1.0 and k + 1 < max_iters
                and max(final_step_bound(r, n, p), ROUNDING_FLOOR) <= tol):
            # the next iterate is certain to meet tol: form only its X
            X = X @ (((p + 1) * eye - M) / p)
            info.iters = k + 2
            info.residuals.append(final_step_bound(r, n, p))
            info.status = "converged"
            info.last_x_only = True
            break
        mu = mu_next
    return X, info


def db_scale(A, mode=2, power_iters=8):
    """Scale for the Denman-Beavers stages: the iteration converges for a
    spectrum inside (0, 2), so the spectral target is 1 instead of Newton's:
    mode 0 ||A||_F, mode 1 min(||A||_F, ||A||_inf), mode 2 the power estimate
    lam itself (norm bound when lam is 0).

    Pinned by: test_newton_db_root_matches_eigh.
    """
    A = np.asarray(A, dtype=np.float64)
    fro = math.sqrt(float(np.sum(A * A)))
    if mode == 0:
        return fro
    bound = min(fro, float(np.max(np.sum(np.abs(A), axis=1))))
    if mode == 1:
        return bound
    if mode in (2, 3):  # mode 3's per-iteration scaling belongs to the coupled Newton iteration
        lam = _power_lambda(A, power_iters)
        return lam if lam > 0.0 else bound
    raise ValueError(f"unknown scale mode {mode}")


def sqrt_pair_db(A, max_iters=25, tol=0.0, divergence_factor=1.2):
    """Denman-Beavers pair iteration for the square root, inverse-free form
    (Newton-Schulz): Y_0 = A, Z_0 = I, M_k = Z_k Y_k,
    Y_{k+1} = Y_k (3 I - M_k) / 2, Z_{k+1} = (3 I - M_k) Z_k / 2.
    Y tends to A^(1/2) and Z to A^(-1/2) when the spectrum of A lies in (0, 2).

    The residual r_k = ||M_k - I||_F / sqrt(n) belongs to the pair k. Stops
    at r_k <= tol (keep pair k), on r_k >= r_(k-1) (stalled, or diverged for a
    growth beyond divergence_factor from r_(k-1) > FLOOR_GUARD; keep pair
    k - 1), on a non-finite r_k (keep pair k - 1), or after max_iters updates.
    tol <= 0: exactly max_iters updates (only the non-finite guard).

    Pinned by: test_db_pair_gives_square_root_and_inverse, test_db_scalar_map,
        test_growth_at_the_floor_is_a_stall_not_divergence.
    """
    A = np.asarray(A, dtype=np.float64)
    n = A.shape[0]
    eye = np.eye(n)
    Y, Z = A.copy(), eye.copy()
    info = NewtonInfo(0)
    prev = (Y, Z)
    r_prev = math.inf
    for k in range(max_iters + 1):
        M = Z @ Y
        r = float(np.sqrt(np.sum((M - eye) ** 2)) / math.sqrt(n))
        info.residuals.append(r)
        if not math.isfinite(r):
            info.status = "diverged"
            Y, Z = prev
            break
        if tol > 0.0:
            if r <= tol:
                info.status = "converged"
                break
            if r > divergence_factor * r_prev and r_prev > FLOOR_GUARD:
                info.status = "diverged"
                Y, Z = prev
                break
            if r >= r_prev:
                info.status = "stalled"
                Y, Z = prev
                break
        if k == max_iters:
            break
        prev = (Y, Z)
        r_prev = r
        T = (3.0 * eye - M) / 2.0
        Y, Z = Y @ T, T @ Z
        info.iters = k + 1
    return Y, Z, info


def inverse_root_newton_db(A, max_iters=25, tol=0.0, scale_mode=2):
    """A^(-1/4) by two Denman-Beavers square-root stages (a reading of the
    DASH page's "Newton-DB" solver, whose formula the page does not give):
    with A~ = A / s, the first stage gives Y1 ~ A~^(1/2); the second, run on
    Y1, gives Z2 ~ Y1^(-1/2) = A~^(-1/4); the root is s^(-1/4) Z2.
    Returns (X, (info_stage1, info_stage2)).

    Pinned by: test_newton_db_root_matches_eigh, test_newton_db_orthogonal_similarity.
    """
    A = np.asarray(A, dtype=np.float64)
    s = db_scale(A, scale_mode)
    Y1, _, info1 = sqrt_pair_db(A / s, max_iters, tol)
    _, Z2, info2 = sqrt_pair_db(Y1, max_iters, tol)
    return s ** -0.25 * Z2, (info1, info2)


def chebyshev_interval(A, floor, power_iters=16):
    """Scale s and lower end r of the Chebyshev interval [r, 1] for A / s.

    s = min(lam / 0.55, min(||A||_F, ||A||_inf)) bounds the largest eigenvalue
    from above (lam is mode 2's power estimate, which is at least 0.55 lam_max
    unless v_0 is almost orthogonal to the top eigenvector; the norms bound it
    always). floor is a lower bound of the smallest eigenvalue: for a Shampoo
    statistic, beta2^t eps (the decayed eps I start plus a PSD sum). r =
    floor / s, kept below 0.999.

    Pinned by: test_chebyshev_converges_to_eigh_and_interval_is_valid.
    """
    A = np.asarray(A, dtype=np.float64)
    fro = math.sqrt(float(np.sum(A * A)))
    bound = min(fro, float(np.max(np.sum(np.abs(A), axis=1))))
    lam = 2.0 * newton_scale(A, 4, 2, power_iters)
    s = min(lam / 0.55, bound) if lam > 0.0 else bound
    r = min(floor / s, 0.999) if s > 0.0 else 0.999
    return s, r


def chebyshev_coefficients(r, degree):
    """Coefficients c_0..c_d of the Chebyshev interpolant of x^(-1/4) on
    [r, 1] at the d + 1 Chebyshev points (first kind): with
    theta_j = pi (j + 1/2) / (d + 1) and x_j = ((1 - r) cos theta_j + 1 + r) / 2,
    c_k = 2 / (d + 1) sum_j x_j^(-1/4) cos(k theta_j); the interpolant is
    c_0 / 2 + sum_{k>=1} c_k T_k(t), t = (2 x - 1 - r) / (1 - r).

    Pinned by: test_chebyshev_matches_numpy_interpolant_on_scalars,
        test_chebyshev_coefficients_reproduce_the_function_at_the_nodes.
    """
    N = degree + 1
    theta = math.pi * (np.arange(N) + 0.5) / N
    x = ((1.0 - r) * np.cos(theta) + 1.0 + r) / 2.0
    fx = x ** -0.25
    return np.array([2.0 / N * float(np.sum(fx * np.cos(k * theta))) for k in range(N)])


def inverse_root_chebyshev(A, floor, degree=128, power_iters=16, interval=None):
    """A^(-1/4) as s^(-1/4) p(A / s), p the degree-d Chebyshev interpolant of
    x^(-1/4) on [r, 1] (chebyshev_interval), evaluated by the Clenshaw
    recurrence in matrices: B_(d+1) = B_(d+2) = 0,
    B_k = c_k I + 2 T B_(k+1) - B_(k+2), p = c_0 / 2 I + T B_1 - B_2 with
    T = (2 A / s - (1 + r) I) / (1 - r). A reading of the DASH page's
    Chebyshev inverse-root solver (the page gives no formula). interval, if
    given, is the (s, r) to use instead of chebyshev_interval's.

    Pinned by: test_chebyshev_converges_to_eigh_and_interval_is_valid,
        test_chebyshev_orthogonal_similarity.
    """
    A = np.asarray(A, dtype=np.float64)
    n = A.shape[0]
    eye = np.eye(n)
    s, r = chebyshev_interval(A, floor, power_iters) if interval is None else interval
    c = chebyshev_coefficients(r, degree)
    T = (2.0 * A / s - (1.0 + r) * eye) / (1.0 - r)
    b1 = np.zeros((n, n))
    b2 = np.zeros((n, n))
    for k in range(degree, 0, -1):
        b1, b2 = c[k] * eye + 2.0 * T @ b1 - b2, b1
    P = 0.5 * c[0] * eye + T @ b1 - b2
    return s ** -0.25 * P, (s, r)


# ---------------------------------------------------------------------------
# Preconditioned update ("Shampoo optimizer" page, last line of the loop;
# podcast cue 20)
# ---------------------------------------------------------------------------
def precondition(XL, G, XR):
    """U = L^(-1/4) G R^(-1/4), given the two roots.

    Pinned by: test_precondition_is_left_then_right, test_kronecker_bruteforce_tiny,
        test_first_step_svd_closed_form.
    """
    return np.asarray(XL, np.float64) @ np.asarray(G, np.float64) @ np.asarray(XR, np.float64)


def round_to_bf16(x):
    """Round fp64 values to the nearest bfloat16 value, ties to even.

    bfloat16 keeps 8 significant bits: write x = f * 2^e with f in [0.5, 1),
    round f * 256 to an integer with ties to even, scale back. Finite normal
    range only (the parameters here are far from under- and overflow).

    Pinned by: test_round_to_bf16_matches_torch (torch's bfloat16 cast, ties included).
    """
    x = np.asarray(x, dtype=np.float64)
    f, e = np.frexp(x)
    return np.ldexp(np.rint(f * 256.0) / 256.0, e)


def is_refresh_step(t, root_every):
    """Roots are recomputed at t = 1, 1 + k, 1 + 2k, ... (k = root_every).

    Pinned by: test_refresh_schedule.
    """
    return root_every > 0 and (t - 1) % root_every == 0


# ---------------------------------------------------------------------------
# The whole step over a set of matrices
# ---------------------------------------------------------------------------
@dataclass
class _BlockState:
    L: np.ndarray
    R: np.ndarray
    XL: np.ndarray | None = None
    XR: np.ndarray | None = None
    mom: np.ndarray | None = None
    newton_L: NewtonInfo | None = None
    newton_R: NewtonInfo | None = None


class ShampooOracle:
    """Blocked Shampoo over a list of matrices, block by block, in fp64.

    shapes:       (rows, cols) of each matrix, in registration order.
    block_rows, block_cols: the block shape.
    beta2, stat_scale: EMA weights of the statistics (stat_scale None means
                  1 - beta2).
    eps:          L and R start at eps * I.
    lr:           step size.
    root_every:   k of the refresh schedule (0: only explicit refresh).
    blocks:       optional subset of block ids to track (blocks are
                  independent, so a sample can be run alone).
    root_method:  "eigh" (the definition), "newton" (coupled Newton),
                  "newton_db" (two Denman-Beavers stages), the iterations with
                  newton_iters / newton_tol / newton_scale_mode, or "chebyshev"
                  (degree cheb_degree on [beta2^t eps / s, 1]).
    param_bf16:   parameters are stored in bfloat16 after every update.
    momentum:     alpha of the momentum folded in before preconditioning
                  (0: none).

    Pinned by: test_kronecker_bruteforce_single_64x32, test_shared_singular_vectors_multistep,
        test_stale_roots_between_refreshes, test_update_sign_and_step_size,
        test_momentum_constant_gradient_closed_form, test_momentum_is_linear_sum_of_past_updates,
        test_bf16_params_are_rounded_after_each_step, test_two_by_two_example_diagonal_sum_form.
    """

    def __init__(self, shapes, block_rows, block_cols, beta2, eps, lr, root_every,
                 stat_scale=None, blocks=None, root_method="eigh", newton_iters=25,
                 newton_tol=0.0, newton_scale_mode=1, param_bf16=False, p=4, momentum=0.0,
                 cheb_degree=128):
        self.shapes = [tuple(s) for s in shapes]
        self.table = block_table(self.shapes, block_rows, block_cols)
        self.ids = list(range(len(self.table))) if blocks is None else sorted(set(blocks))
        self.beta2 = float(beta2)
        self.stat_scale = 1.0 - self.beta2 if stat_scale is None else float(stat_scale)
        self.eps = float(eps)
        self.lr = float(lr)
        self.root_every = int(root_every)
        self.root_method = root_method
        self.newton_iters = newton_iters
        self.newton_tol = newton_tol
        self.newton_scale_mode = newton_scale_mode
        self.param_bf16 = param_bf16
        self.p = p
        self.momentum = float(momentum)
        self.cheb_degree = int(cheb_degree)
        self.t = 0
        self.state = {}
        for i in self.ids:
            b = self.table[i]
            self.state[i] = _BlockState(self.eps * np.eye(b.m), self.eps * np.eye(b.n),
                                        mom=np.zeros((b.m, b.n)))

    def _root(self, A):
        if self.root_method == "eigh":
            return inverse_root_eigh(A, self.p), None
        if self.root_method == "newton":
            return inverse_root_coupled_newton(A, self.p, self.newton_iters, self.newton_tol,
                                               self.newton_scale_mode)
        if self.root_method == "newton_db":
            return inverse_root_newton_db(A, self.newton_iters, self.newton_tol,
                                          self.newton_scale_mode)
        if self.root_method == "chebyshev":
            floor = (self.beta2 ** self.t) * self.eps
            return inverse_root_chebyshev(A, floor, self.cheb_degree)
        raise ValueError(self.root_method)

    def refresh_roots(self):
        for i in self.ids:
            st = self.state[i]
            st.XL, st.newton_L = self._root(st.L)
            st.XR, st.newton_R = self._root(st.R)

    def step_blocks(self, block_grads, block_params=None, force_refresh=False, auto_refresh=True):
        """One step on the tracked blocks.

        block_grads:  {block id: gradient block (real extent)} for every
                      tracked block.
        block_params: optional {block id: parameter block}; when given, each
                      is moved by -lr * U (and rounded to bfloat16 when the
                      parameters are bfloat16).
        Returns ({block id: new parameter block} or None, {block id: U}).
        """
        self.t += 1
        G = {i: np.asarray(block_grads[i], dtype=np.float64) for i in self.ids}
        for i in self.ids:
            st = self.state[i]
            st.L, st.R = update_statistics(st.L, st.R, G[i], self.beta2, self.stat_scale)
        if force_refresh or (auto_refresh and is_refresh_step(self.t, self.root_every)):
            self.refresh_roots()
        updates = {}
        for i in self.ids:
            st = self.state[i]
            if st.XL is None:
                raise RuntimeError("step before any root refresh")
            D = G[i]
            if self.momentum != 0.0:
                st.mom = self.momentum * st.mom + G[i]
                D = st.mom
            updates[i] = precondition(st.XL, D, st.XR)
        if block_params is None:
            return None, updates
        new = {}
        for i in self.ids:
            W = np.asarray(block_params[i], dtype=np.float64) - self.lr * updates[i]
            new[i] = round_to_bf16(W) if self.param_bf16 else W
        return new, updates

    def step(self, grads, params, force_refresh=False, auto_refresh=True):
        """One step over full matrices (lists, any float dtype).

        Returns (new params as fp64 arrays, {block id: U}); only the tracked
        blocks of the parameters change.
        """
        sl = {i: (self.table[i].mat, slice(self.table[i].r0, self.table[i].r0 + self.table[i].m),
                  slice(self.table[i].c0, self.table[i].c0 + self.table[i].n)) for i in self.ids}
        gb = {i: grads[m][r, c] for i, (m, r, c) in sl.items()}
        new_params = [np.array(p, dtype=np.float64) for p in params]
        wb = {i: new_params[m][r, c] for i, (m, r, c) in sl.items()}
        new_blocks, updates = self.step_blocks(gb, wb, force_refresh, auto_refresh)
        for i, (m, r, c) in sl.items():
            new_params[m][r, c] = new_blocks[i]
        return new_params, updates
