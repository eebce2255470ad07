"""Pins of the fp64 oracle against facts the pages and the mathematics fix.

None of these compare the oracle with itself: each check uses a closed form,
an identity, an independent library routine (SVD, Kronecker eigendecomposition,
torch's bfloat16 cast) or brute force on tiny inputs. Every part of the
oracle is covered by at least one check that a dropped term, a wrong sign or
index, or a transposed operand would fail (see test_planted_mistakes).
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import (ShampooOracle, block_table, inverse_root_coupled_newton, inverse_root_eigh,
                    newton_balance, newton_map,
                    is_refresh_step, newton_scale, pack_blocks, precondition, round_to_bf16,
                    unpack_blocks, update_statistics)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rel(a, b):
    return float(np.linalg.norm(np.asarray(a) - np.asarray(b)) / np.linalg.norm(np.asarray(b)))


def run_oracle(G_steps, W0, beta2, eps, lr, root_every=1, stat_scale=None, **kw):
    m, n = np.asarray(G_steps[0]).shape
    o = ShampooOracle([(m, n)], m, n, beta2, eps, lr, root_every, stat_scale=stat_scale, **kw)
    W = [np.asarray(W0, dtype=np.float64)]
    Us = []
    for G in G_steps:
        W, U = o.step([np.asarray(G, dtype=np.float64)], W)
        Us.append(U[0])
    return o, W[0], Us


# ---------------------------------------------------------------------------
# The 2x2 example of the "Shampoo optimizer" page (no numbers printed there)
# ---------------------------------------------------------------------------
def test_two_by_two_example_all_ones():
    case = json.load(open(os.path.join(GOLDEN, "two_by_two.json")))["cases"][0]
    G = np.array(case["G"])
    W0 = np.array(case["W0"])
    b2, eps, lr = case["beta2"], case["eps"], case["lr"]
    _, W1, Us = run_oracle([G], W0, b2, eps, lr)
    U_cf = G / math.sqrt(b2 * eps + 4 * (1 - b2))
    assert rel(Us[0], U_cf) < 1e-12
    assert rel(W1, W0 - lr * U_cf) < 1e-14


def test_two_by_two_example_diagonal_sum_form():
    case = json.load(open(os.path.join(GOLDEN, "two_by_two.json")))["cases"][1]
    Gs = [np.array(g) for g in case["G_steps"]]
    eps = case["eps"]
    _, _, Us = run_oracle(Gs, np.zeros((2, 2)), case["beta2"], eps, case["lr"],
                          stat_scale=case["stat_scale"])
    acc = np.full(2, eps)
    for G, U in zip(Gs, Us):
        g = np.diag(G)
        acc = acc + g * g
        assert np.allclose(U, np.diag(g / np.sqrt(acc)), rtol=1e-13, atol=1e-15)


# ---------------------------------------------------------------------------
# Diagonal gradients: every root is elementwise (closed form)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("m,n", [(5, 5), (6, 3), (3, 7)])
def test_diagonal_gradients_closed_form(m, n):
    rng = np.random.default_rng(3)
    b2, eps, lr, k = 0.9, 1e-3, 0.1, 1
    d = min(m, n)
    Gs = []
    for _ in range(6):
        G = np.zeros((m, n))
        G[np.arange(d), np.arange(d)] = rng.standard_normal(d)
        Gs.append(G)
    _, _, Us = run_oracle(Gs, np.zeros((m, n)), b2, eps, lr, root_every=k)
    ell = np.full(d, eps)
    for G, U in zip(Gs, Us):
        g = np.diag(G)[:d] if m == n else G[np.arange(d), np.arange(d)]
        ell = b2 * ell + (1 - b2) * g * g
        expect = np.zeros((m, n))
        expect[np.arange(d), np.arange(d)] = g / np.sqrt(ell)
        assert np.allclose(U, expect, rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------------------
# Kronecker brute force (podcast cue 22): vec_r(U) = (L kron R)^(-1/4) vec_r(G)
# ---------------------------------------------------------------------------
def kron_update(L, R, G):
    K = np.kron(L, R)
    lam, Q = np.linalg.eigh(K)
    return ((Q * lam ** -0.25) @ Q.T @ G.reshape(-1)).reshape(G.shape)


@pytest.mark.parametrize("m,n", [(1, 1), (2, 3), (4, 5), (6, 6), (7, 2)])
def test_kronecker_bruteforce_tiny(m, n):
    rng = np.random.default_rng(m * 10 + n)
    b2, eps = 0.95, 1e-2
    Gs = [rng.standard_normal((m, n)) for _ in range(4)]
    o, _, Us = run_oracle(Gs, np.zeros((m, n)), b2, eps, 1e-3, root_every=1)
    L = eps * np.eye(m)
    R = eps * np.eye(n)
    for G, U in zip(Gs, Us):
        L = b2 * L + (1 - b2) * G @ G.T
        R = b2 * R + (1 - b2) * G.T @ G
        assert rel(U, kron_update(L, R, G)) < 1e-10


def test_kronecker_bruteforce_single_64x32():
    """The whole single-matrix workload (64x32, 10 steps, roots every step)."""
    rng = np.random.default_rng(1001)
    Gs = [rng.standard_normal((64, 32)) for _ in range(10)]
    b2, eps = 0.999, 1e-6
    _, _, Us = run_oracle(Gs, np.zeros((64, 32)), b2, eps, 1e-3, root_every=1)
    L, R = eps * np.eye(64), eps * np.eye(32)
    for t, (G, U) in enumerate(zip(Gs, Us)):
        L = b2 * L + (1 - b2) * G @ G.T
        R = b2 * R + (1 - b2) * G.T @ G
        if t in (0, 1, 9):
            assert rel(U, kron_update(L, R, G)) < 1e-9


# ---------------------------------------------------------------------------
# First step from the SVD (independent LAPACK routine)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("m,n", [(8, 8), (9, 4), (3, 10)])
def test_first_step_svd_closed_form(m, n):
    rng = np.random.default_rng(7)
    G = rng.standard_normal((m, n))
    b2, eps = 0.999, 1e-6
    _, _, Us = run_oracle([G], np.zeros((m, n)), b2, eps, 1e-3)
    P, s, Qt = np.linalg.svd(G, full_matrices=False)
    U_cf = (P * (s / np.sqrt(b2 * eps + (1 - b2) * s * s))) @ Qt
    assert rel(Us[0], U_cf) < 1e-11


def test_shared_singular_vectors_multistep():
    rng = np.random.default_rng(11)
    n = 6
    P, _ = np.linalg.qr(rng.standard_normal((n, n)))
    Q, _ = np.linalg.qr(rng.standard_normal((n, n)))
    b2, eps = 0.9, 1e-4
    sv = [np.abs(rng.standard_normal(n)) + 0.1 for _ in range(5)]
    Gs = [(P * s) @ Q.T for s in sv]
    _, _, Us = run_oracle(Gs, np.zeros((n, n)), b2, eps, 1e-3, root_every=1)
    ell = np.full(n, eps)
    for s, U in zip(sv, Us):
        ell = b2 * ell + (1 - b2) * s * s
        assert rel(U, (P * (s / np.sqrt(ell))) @ Q.T) < 1e-11


# ---------------------------------------------------------------------------
# Statistics: the recursion equals the closed sum
# ---------------------------------------------------------------------------
def test_statistics_closed_sum():
    rng = np.random.default_rng(5)
    m, n, T = 5, 3, 7
    b2, eps, gam = 0.8, 0.3, 0.45
    L, R = eps * np.eye(m), eps * np.eye(n)
    Gs = [rng.standard_normal((m, n)) for _ in range(T)]
    for G in Gs:
        L, R = update_statistics(L, R, G, b2, gam)
    L_cf = b2 ** T * eps * np.eye(m) + gam * sum(b2 ** (T - 1 - s) * Gs[s] @ Gs[s].T for s in range(T))
    R_cf = b2 ** T * eps * np.eye(n) + gam * sum(b2 ** (T - 1 - s) * Gs[s].T @ Gs[s] for s in range(T))
    assert rel(L, L_cf) < 1e-14 and rel(R, R_cf) < 1e-14


def test_scalar_one_by_one():
    b2, eps, lr = 0.99, 1e-5, 0.5
    gs = [0.3, -1.2, 2.0, 0.0, -0.7]
    _, _, Us = run_oracle([[[g]] for g in gs], [[0.0]], b2, eps, lr)
    for t, (g, U) in enumerate(zip(gs, Us), start=1):
        ell = b2 ** t * eps + (1 - b2) * sum(b2 ** (t - s) * gs[s - 1] ** 2 for s in range(1, t + 1))
        assert abs(U[0, 0] - g * ell ** -0.5) <= 1e-12 * max(1.0, abs(g * ell ** -0.5))


# ---------------------------------------------------------------------------
# Invariants: symmetric PSD statistics, X^4 A = I
# ---------------------------------------------------------------------------
def test_invariants():
    rng = np.random.default_rng(9)
    o = ShampooOracle([(12, 20), (20, 12)], 8, 8, 0.999, 1e-6, 1e-3, 2)
    W = [np.zeros((12, 20)), np.zeros((20, 12))]
    for _ in range(3):
        W, _ = o.step([rng.standard_normal((12, 20)), rng.standard_normal((20, 12))], W)
    for st in o.state.values():
        for A, X in ((st.L, st.XL), (st.R, st.XR)):
            assert np.array_equal(A, A.T)
            assert np.linalg.eigvalsh(A).min() > 0
            X4 = np.linalg.matrix_power(X, 4)
            assert np.linalg.norm(X4 @ A - np.eye(A.shape[0])) / math.sqrt(A.shape[0]) < 1e-10


def test_inverse_root_rejects_indefinite():
    with pytest.raises(np.linalg.LinAlgError):
        inverse_root_eigh(np.diag([1.0, -1e-3]))
    with pytest.raises(np.linalg.LinAlgError):
        inverse_root_eigh(np.zeros((3, 3)))


def test_inverse_root_2x2_analytic():
    a, b, c = 3.0, 1.25, 2.0
    A = np.array([[a, b], [b, c]])
    disc = math.sqrt(((a - c) / 2) ** 2 + b * b)
    lam = np.array([(a + c) / 2 - disc, (a + c) / 2 + disc])
    # eigenvector of the larger eigenvalue, by hand
    v = np.array([b, lam[1] - a])
    v /= np.linalg.norm(v)
    w = np.array([-v[1], v[0]])
    X_cf = lam[1] ** -0.25 * np.outer(v, v) + lam[0] ** -0.25 * np.outer(w, w)
    assert rel(inverse_root_eigh(A), X_cf) < 1e-14


# ---------------------------------------------------------------------------
# Refresh schedule (podcast cue 28: roots reused between refreshes)
# ---------------------------------------------------------------------------
def test_refresh_schedule():
    assert [t for t in range(1, 32) if is_refresh_step(t, 10)] == [1, 11, 21, 31]
    assert all(is_refresh_step(t, 1) for t in range(1, 5))
    assert not any(is_refresh_step(t, 0) for t in range(1, 5))


def test_stale_roots_between_refreshes():
    """With G_t = c_t G0 and roots frozen after step 1, U_t = (c_t / c_1) U_1;
    at the refresh step the SVD closed form with accumulated scales holds."""
    rng = np.random.default_rng(21)
    n = 5
    G0 = rng.standard_normal((n, n))
    cs = [1.0, 0.5, -2.0, 3.0, 0.25]
    b2, eps, k = 0.9, 1e-3, 3
    _, _, Us = run_oracle([c * G0 for c in cs], np.zeros((n, n)), b2, eps, 1e-3, root_every=k)
    for t in (1, 2):
        assert rel(Us[t], cs[t] * Us[0]) < 1e-13
    # step 4 (t index 3) refreshes: L_4 = b2^4 eps I + (1-b2) S P Sigma^2 P^T
    P, s, Qt = np.linalg.svd(G0)
    S = sum(b2 ** (3 - j) * cs[j] ** 2 for j in range(4))
    U_cf = (P * (cs[3] * s / np.sqrt(b2 ** 4 * eps + (1 - b2) * S * s * s))) @ Qt
    assert rel(Us[3], U_cf) < 1e-11
    # step 5 is stale again: scaled copy of step 4
    assert rel(Us[4], cs[4] / cs[3] * Us[3]) < 1e-13


def test_update_sign_and_step_size():
    rng = np.random.default_rng(4)
    G = rng.standard_normal((4, 3))
    W0 = rng.standard_normal((4, 3))
    _, W1a, Ua = run_oracle([G], W0, 0.9, 1e-3, 0.0)
    assert np.array_equal(W1a, W0)
    _, W1, U = run_oracle([G], W0, 0.9, 1e-3, 0.25)
    assert rel(W1, W0 - 0.25 * U[0]) < 1e-15
    # the update points along the gradient (preconditioner is positive definite)
    assert float(np.sum(U[0] * G)) > 0


# ---------------------------------------------------------------------------
# Block map: row-major blocks, zero-padded tails, exact round trip
# ---------------------------------------------------------------------------
def test_block_counts_of_the_workloads():
    gpt = [(768, 2304), (768, 768), (768, 3072), (3072, 768)] * 12
    dec = [(2048, 6144), (2048, 2048), (2048, 8192), (8192, 2048)] * 24
    assert len(block_table([(64, 32)], 64, 32)) == 1
    assert len(block_table(gpt, 256, 256)) == 1296
    t512 = block_table(gpt, 512, 512)
    assert len(t512) == 456
    assert sum(1 for b in t512 if (b.m, b.n) != (512, 512)) == 252
    assert len(block_table(dec, 1024, 1024)) == 1152


def test_pack_matches_elementwise_enumeration():
    rng = np.random.default_rng(2)
    shapes = [(7, 5), (3, 9), (8, 8)]
    mats = [rng.standard_normal(s).astype(np.float32) for s in shapes]
    br, bc = 4, 3
    table = block_table(shapes, br, bc)
    P = pack_blocks(mats, table, br, bc)
    # independent enumeration: walk every element of the packed array
    base = 0
    for mat, (rows, cols) in enumerate(shapes):
        nbr, nbc = -(-rows // br), -(-cols // bc)
        for idx in range(nbr * nbc * br * bc):
            blk, rem = divmod(idx, br * bc)
            r, c = divmod(rem, bc)
            bi, bj = divmod(blk, nbc)
            gr, gc = bi * br + r, bj * bc + c
            v = P[base + blk, r, c]
            if gr < rows and gc < cols:
                assert v == mats[mat][gr, gc]
            else:
                assert v == 0.0 and not np.signbit(v)
        base += nbr * nbc
    assert base == P.shape[0]
    back = unpack_blocks(P, table, shapes)
    for a, b in zip(mats, back):
        assert np.array_equal(a, b)


def test_tail_blocks_equal_padded_blocks():
    """Zero padding decouples exactly: the padded block's update restricted to
    the real extent equals the update of the real block."""
    rng = np.random.default_rng(8)
    m, n, bm, bn = 5, 3, 8, 4
    Gs = [rng.standard_normal((m, n)) for _ in range(3)]
    _, _, Us = run_oracle(Gs, np.zeros((m, n)), 0.9, 1e-2, 1e-3)
    Gp = [np.pad(G, ((0, bm - m), (0, bn - n))) for G in Gs]
    _, _, Up = run_oracle(Gp, np.zeros((bm, bn)), 0.9, 1e-2, 1e-3)
    for U, V in zip(Us, Up):
        assert rel(V[:m, :n], U) < 1e-12
        assert np.abs(V[m:, :]).max() == 0 and np.abs(V[:, n:]).max() == 0


# ---------------------------------------------------------------------------
# Coupled Newton iteration (the GPU's method) against the definition
# ---------------------------------------------------------------------------
def spd(n, cond, rng):
    Q, _ = np.linalg.qr(rng.standard_normal((n, n)))
    lam = np.geomspace(1.0, 1.0 / cond, n)
    return (Q * lam) @ Q.T, Q, lam


@pytest.mark.parametrize("mode", [0, 1])
def test_newton_converges_to_eigh(mode):
    rng = np.random.default_rng(13)
    A, _, _ = spd(24, 1e3, rng)
    A *= 7.5
    X, info = inverse_root_coupled_newton(A, 4, max_iters=60, tol=1e-13, scale_mode=mode)
    assert info.status in ("converged", "stalled")
    assert rel(X, inverse_root_eigh(A)) < 1e-11


def test_newton_orthogonal_similarity():
    """Newton commutes with an orthogonal change of basis: on Q diag(a) Q^T it
    returns Q diag(x) Q^T with x from the diagonal matrix (fixed 5 iterations,
    far from converged, so this checks the iteration itself)."""
    rng = np.random.default_rng(17)
    A, Q, lam = spd(6, 50.0, rng)
    Xa, _ = inverse_root_coupled_newton(A, 4, max_iters=5, tol=0.0, scale_mode=0)
    Xd, _ = inverse_root_coupled_newton(np.diag(lam), 4, max_iters=5, tol=0.0, scale_mode=0)
    assert np.allclose(Xd, np.diag(np.diag(Xd)), atol=0)
    assert rel(Xa, Q @ Xd @ Q.T) < 1e-12


def test_newton_scalar_fixed_point_and_monotone():
    """On a 1x1 matrix the iteration is the scalar map x -> x (5 - m)/4,
    m -> m ((5 - m)/4)^4, whose fixed point is a^(-1/4) and whose residual
    |m - 1| decreases every step for m in (0, 5)."""
    a = 3.7e-4
    # scale mode 1 maps a 1x1 matrix to m0 = 5/2, away from the fixed point
    X, info = inverse_root_coupled_newton(np.array([[a]]), 4, max_iters=30, tol=0.0, scale_mode=1)
    r = info.residuals
    assert r[0] == pytest.approx(abs(2.5 * (2.5 / 4) ** 4 - 1), rel=1e-14)
    assert all(r2 < r1 for r1, r2 in zip(r, r[1:]) if r1 > 1e-15)
    assert abs(X[0, 0] - a ** -0.25) < 1e-12 * a ** -0.25


def test_newton_scale_bounds_spectrum():
    rng = np.random.default_rng(19)
    A, _, lam = spd(10, 20.0, rng)
    A *= 3.0
    lam = lam * 3.0
    # ||A||_F^2 = sum of squared eigenvalues (symmetric A)
    assert abs(newton_scale(A, 4, 0) ** 2 - float(np.sum(lam ** 2))) < 1e-12 * float(np.sum(lam ** 2))
    s1 = newton_scale(A, 4, 1)
    assert lam.max() / s1 <= 2.5 + 1e-12
    D = np.diag([4.0, 1.0, 0.5])
    assert abs(newton_scale(D, 4, 1) - 4.0 * 2 / 5) < 1e-15  # inf-norm 4 < fro
    with pytest.raises(ValueError):
        newton_scale(D, 4, 7)


def test_newton_guard_keeps_finite_iterate():
    """An indefinite input makes the iteration blow up; with a tolerance the
    guard stops and keeps the last finite iterate."""
    A = np.diag([1.0, 0.5, -0.4])
    X, info = inverse_root_coupled_newton(A, 4, max_iters=60, tol=1e-12, scale_mode=0)
    assert np.all(np.isfinite(X))
    assert info.status in ("diverged", "stalled")


# ---------------------------------------------------------------------------
# bfloat16 rounding against torch's cast (round to nearest, ties to even)
# ---------------------------------------------------------------------------
def test_round_to_bf16_matches_torch():
    rng = np.random.default_rng(23)
    x = (rng.standard_normal(20000) * 0.05).astype(np.float32).astype(np.float64)
    # add exact ties: values halfway between two bf16 numbers
    ties = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(0.5 + 2 ** -9), 0.02 + 0.0])
    x = np.concatenate([x, ties.astype(np.float32).astype(np.float64)])
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(round_to_bf16(x), ref)
    assert round_to_bf16(np.array([1.0 + 2 ** -8]))[0] == 1.0           # tie to even
    assert round_to_bf16(np.array([1.0 + 3 * 2 ** -8]))[0] == 1.0 + 2 ** -6


def test_bf16_params_are_rounded_after_each_step():
    rng = np.random.default_rng(29)
    G = rng.standard_normal((4, 4))
    W0 = round_to_bf16(rng.standard_normal((4, 4)) * 0.02)
    _, W1, U = run_oracle([G], W0, 0.999, 1e-6, 1e-3, param_bf16=True)
    assert np.array_equal(W1, round_to_bf16(W0 - 1e-3 * U[0]))
    assert np.array_equal(round_to_bf16(W1), W1)


def test_precondition_is_left_then_right():
    XL = np.array([[2.0, 0.0], [0.0, 3.0]])
    XR = np.array([[5.0, 0.0, 0.0], [0.0, 7.0, 0.0], [0.0, 0.0, 11.0]])
    G = np.ones((2, 3))
    assert np.array_equal(precondition(XL, G, XR), np.outer([2.0, 3.0], [5.0, 7.0, 11.0]))


def test_newton_scale_mode2_power_iteration():
    """Mode 2 on a diagonal matrix: v_k is proportional to A^k 1, so the
    estimate after k products is ||A^k 1|| / ||A^(k-1) 1|| (closed form)."""
    a = np.array([3.0, 1.0, 0.5, 2.5, 0.1])
    A = np.diag(a)
    k = 8  # the default count of power products
    lam = math.sqrt(np.sum(a ** (2 * k))) / math.sqrt(np.sum(a ** (2 * (k - 1))))
    assert newton_scale(A, 4, 2) == pytest.approx(lam / 2, rel=1e-13)
    assert lam <= a.max()
    # zero matrix: falls back to the norm bound (0 here)
    assert newton_scale(np.zeros((3, 3)), 4, 2) == 0.0
    # random SPD: the estimate is within the bound of the proof and the scaled
    # spectrum lies inside the convergence region
    rng = np.random.default_rng(31)
    for _ in range(5):
        B, Q, lam_true = spd(40, 1e4, rng)
        c1 = abs(Q[:, 0] @ np.full(40, 1 / math.sqrt(40)))  # top eigenvector first in spd()
        s = newton_scale(B, 4, 2)
        assert 2 * s >= lam_true.max() * c1 ** (1 / 8) * (1 - 1e-12)
        assert 1.0 < lam_true.max() / s < 5.0
    X, info = inverse_root_coupled_newton(B, 4, max_iters=60, tol=1e-13, scale_mode=2)
    assert rel(X, inverse_root_eigh(B)) < 1e-10


# ---------------------------------------------------------------------------
# Momentum before preconditioning (podcast cue 28)
# ---------------------------------------------------------------------------
def test_momentum_constant_gradient_closed_form():
    """Constant gradient, roots frozen after step 1: the momentum after t steps
    is G (1 - a^t) / (1 - a), so U_t = (1 - a^t) / (1 - a) U_1."""
    rng = np.random.default_rng(41)
    G = rng.standard_normal((5, 3))
    a = 0.9
    _, _, Us = run_oracle([G] * 6, np.zeros((5, 3)), 0.99, 1e-3, 1e-2, root_every=100, momentum=a)
    for t, U in enumerate(Us, start=1):
        assert rel(U, (1 - a ** t) / (1 - a) * Us[0]) < 1e-13


def test_momentum_is_linear_sum_of_past_updates():
    """With frozen roots the preconditioner is linear: U_t = sum_s a^(t-s) P(G_s)
    where P is the plain (momentum-free) update with the same roots."""
    rng = np.random.default_rng(43)
    Gs = [rng.standard_normal((4, 6)) for _ in range(5)]
    a = 0.9
    _, _, Um = run_oracle(Gs, np.zeros((4, 6)), 0.95, 1e-2, 1e-3, root_every=100, momentum=a)
    # momentum-free run with the same statistics gives the same roots (k = 100)
    o, _, _ = run_oracle(Gs[:1], np.zeros((4, 6)), 0.95, 1e-2, 1e-3, root_every=100)
    XL, XR = o.state[0].XL, o.state[0].XR
    for t in range(5):
        ref = sum(a ** (t - s) * XL @ Gs[s] @ XR for s in range(t + 1))
        assert rel(Um[t], ref) < 1e-12
    # momentum 0 is the plain method
    _, _, U0 = run_oracle(Gs, np.zeros((4, 6)), 0.95, 1e-2, 1e-3, root_every=1, momentum=0.0)
    _, _, Up = run_oracle(Gs, np.zeros((4, 6)), 0.95, 1e-2, 1e-3, root_every=1)
    for u, v in zip(U0, Up):
        assert np.array_equal(u, v)


# ---------------------------------------------------------------------------
# Newton-DB: two Denman-Beavers square-root stages
# ---------------------------------------------------------------------------
from oracle import db_scale, inverse_root_newton_db, sqrt_pair_db  # noqa: E402


def test_db_pair_gives_square_root_and_inverse():
    rng = np.random.default_rng(51)
    A, Q, lam = spd(20, 50.0, rng)
    A *= 1.5  # spectrum in (0.03, 1.5], inside (0, 2)
    Y, Z, info = sqrt_pair_db(A, 40, 1e-13)
    assert info.status in ("converged", "stalled")
    sq = (Q * np.sqrt(1.5 * lam)) @ Q.T  # square root from the eigenpairs
    assert rel(Y, sq) < 1e-11 and rel(Z, np.linalg.inv(sq)) < 1e-11
    assert rel(Y @ Y, A) < 1e-11


def test_db_scalar_map():
    """1x1: y <- y (3 - zy) / 2, z <- (3 - zy) z / 2 from (a, 1); z y tends to 1
    and y to sqrt(a); one step by hand."""
    a = 0.3
    Y, Z, info = sqrt_pair_db(np.array([[a]]), 1, 0.0)
    t = (3 - a) / 2
    assert Y[0, 0] == pytest.approx(a * t, rel=1e-15) and Z[0, 0] == pytest.approx(t, rel=1e-15)
    Y, Z, _ = sqrt_pair_db(np.array([[a]]), 40, 1e-14)
    assert Y[0, 0] == pytest.approx(math.sqrt(a), rel=1e-13)
    assert Z[0, 0] == pytest.approx(1 / math.sqrt(a), rel=1e-13)


def test_newton_db_root_matches_eigh():
    rng = np.random.default_rng(53)
    for mode in (0, 1, 2):
        A, _, _ = spd(24, 300.0, rng)
        A *= 3e-3
        X, (i1, i2) = inverse_root_newton_db(A, 60, 1e-13, mode)
        assert rel(X, inverse_root_eigh(A)) < 1e-10
    assert db_scale(np.diag([4.0, 1.0]), 1) == pytest.approx(4.0)


def test_newton_db_orthogonal_similarity():
    rng = np.random.default_rng(57)
    A, Q, lam = spd(6, 20.0, rng)
    Xa, _ = inverse_root_newton_db(A, 4, 0.0, 0)
    Xd, _ = inverse_root_newton_db(np.diag(lam), 4, 0.0, 0)
    assert np.allclose(Xd, np.diag(np.diag(Xd)), atol=0)
    assert rel(Xa, Q @ Xd @ Q.T) < 1e-12


def test_growth_at_the_floor_is_a_stall_not_divergence():
    """A residual that grows from below the floor guard stops the iteration as
    'stalled' and keeps the previous iterate; from above it, 'diverged'."""
    # fp32-like floor emulated on a diagonal matrix: the iteration reaches the
    # fp64 floor (~1e-16) and stalls there, never reported as divergence
    A = np.diag(np.geomspace(1.0, 1e-3, 30))
    for tol in (1e-20, 1e-30):
        X, info = inverse_root_coupled_newton(A, 4, max_iters=60, tol=tol, scale_mode=2)
        assert info.status == "stalled", info
        assert rel(X, inverse_root_eigh(A)) < 1e-12
    _, _, i_db = sqrt_pair_db(A / db_scale(A, 2), 60, 1e-30)
    assert i_db.status == "stalled"


# ---------------------------------------------------------------------------
# Chebyshev inverse root (interpolant of x^(-1/4), Clenshaw in matrices)
# ---------------------------------------------------------------------------
from oracle import chebyshev_coefficients, chebyshev_interval, inverse_root_chebyshev  # noqa: E402


def test_chebyshev_matches_numpy_interpolant_on_scalars():
    """1x1 and diagonal matrices: the matrix Clenshaw result equals numpy's own
    Chebyshev interpolant of x^(-1/4) (an independent routine) evaluated at
    a / s, times s^(-1/4)."""
    a = np.array([3e-3, 0.02, 0.5, 1.0, 0.7])
    floor = 1e-3
    for deg in (8, 33):
        X, (s, r) = inverse_root_chebyshev(np.diag(a), floor, deg)
        p = np.polynomial.Chebyshev.interpolate(lambda t: t ** -0.25, deg, domain=[r, 1.0])
        assert np.allclose(np.diag(X), s ** -0.25 * p(a / s), rtol=1e-11, atol=0)
        assert np.count_nonzero(X - np.diag(np.diag(X))) == 0


def test_chebyshev_coefficients_reproduce_the_function_at_the_nodes():
    r, d = 0.05, 20
    c = chebyshev_coefficients(r, d)
    theta = math.pi * (np.arange(d + 1) + 0.5) / (d + 1)
    x = ((1 - r) * np.cos(theta) + 1 + r) / 2
    vals = 0.5 * c[0] + sum(c[k] * np.cos(k * theta) for k in range(1, d + 1))
    assert np.allclose(vals, x ** -0.25, rtol=1e-13)


def test_chebyshev_converges_to_eigh_and_interval_is_valid():
    rng = np.random.default_rng(61)
    A, Q, lam = spd(16, 30.0, rng)
    A = 2e-3 * A + 1e-5 * np.eye(16)
    floor = 1e-5
    s, r = chebyshev_interval(A, floor)
    lam = np.linalg.eigvalsh(A)
    assert lam.max() <= s * (1 + 1e-12) and lam.min() >= r * s * (1 - 1e-12)
    errs = [rel(inverse_root_chebyshev(A, floor, d)[0], inverse_root_eigh(A)) for d in (16, 48, 128)]
    assert errs[0] > errs[1] > errs[2] and errs[2] < 1e-8


def test_chebyshev_orthogonal_similarity():
    rng = np.random.default_rng(63)
    A, Q, lam = spd(6, 20.0, rng)
    # the interval is not rotation-invariant (power iteration from the
    # all-ones vector, inf-norm), the polynomial is: use one interval for both
    iv = chebyshev_interval(A, 0.01)
    Xa, _ = inverse_root_chebyshev(A, 0.01, 12, interval=iv)
    Xd, _ = inverse_root_chebyshev(np.diag(lam), 0.01, 12, interval=iv)
    assert np.count_nonzero(Xd - np.diag(np.diag(Xd))) == 0
    assert rel(Xa, Q @ Xd @ Q.T) < 1e-12


# ---------------------------------------------------------------------------
# Scale mode 3: the coupled Newton iteration that scales itself every step
# ---------------------------------------------------------------------------
def _rotated(n, cond, seed):
    rng = np.random.default_rng(seed)
    Q, _ = np.linalg.qr(rng.standard_normal((n, n)))
    lam = np.geomspace(1.0, 1.0 / cond, n)
    return (Q * lam) @ Q.T


def _column_scaled_stat(n, seed):
    rng = np.random.default_rng(seed)
    cs = np.exp(rng.uniform(np.log(1e-2), 0.0, n))
    G = rng.standard_normal((n, n)) * 1e-2 * cs[None, :]
    return 1e-3 * G.T @ G + 1e-7 * np.eye(n)


@pytest.mark.parametrize("p", [4, 6, 8])
@pytest.mark.parametrize("kind,cond", [("rot", 1e2), ("rot", 1e4), ("colscaled", None)])
def test_scaled_newton_reaches_the_root(p, kind, cond):
    A = _rotated(96, cond, 3) if kind == "rot" else _column_scaled_stat(96, 5)
    X, info = inverse_root_coupled_newton(A, p, 60, 1e-11, scale_mode=3)
    ref = inverse_root_eigh(A, p)
    assert info.status == "converged"
    assert np.linalg.norm(X - ref) / np.linalg.norm(ref) < 1e-8
    # the scales stay inside the safe range and the first iteration is unscaled
    assert info.mus[0] == 1.0 and all(1.0 <= m <= 0.9 * (p + 1) for m in info.mus)


@pytest.mark.parametrize("kind,cond", [("rot", 1e3), ("rot", 1e5), ("colscaled", None)])
def test_scaled_newton_needs_fewer_iterations(kind, cond):
    A = _rotated(96, cond, 7) if kind == "rot" else _column_scaled_stat(128, 9)
    _, i2 = inverse_root_coupled_newton(A, 4, 60, 1e-10, scale_mode=2)
    _, i3 = inverse_root_coupled_newton(A, 4, 60, 1e-10, scale_mode=3)
    assert i3.iters < i2.iters, (i3.iters, i2.iters)
    assert any(m > 1.0 for m in i3.mus)


def test_scaled_newton_diagonal_closed_form():
    lam = np.geomspace(3.0, 3e-4, 40)
    X, info = inverse_root_coupled_newton(np.diag(lam), 4, 60, 1e-12, scale_mode=3)
    assert np.abs(X - np.diag(lam ** -0.25)).max() / lam.min() ** -0.25 < 1e-9
    assert np.abs(X - np.diag(np.diag(X))).max() == 0.0  # stays diagonal


def test_spectrum_floor_estimate_bounds():
    from oracle import spectrum_floor_estimate
    for seed in range(4):
        A = _rotated(64, 10.0 ** (seed + 1), seed)
        lam = np.linalg.eigvalsh(A)
        e = spectrum_floor_estimate(A)
        assert lam[0] - 1e-12 <= e <= np.diag(A).min() + 1e-12
    D = np.diag(np.linspace(2.0, 0.5, 9))
    assert spectrum_floor_estimate(D) == 0.5


def test_power_pair_top_matches_mode_2_and_bottom_converges():
    from oracle import power_pair
    A = _rotated(48, 1e3, 13)
    lam, q = power_pair(A, 8)
    assert lam == pytest.approx(2.0 * newton_scale(A, 4, 2), rel=1e-15)  # the same top iteration
    assert q >= np.linalg.eigvalsh(A)[0]
    # an isolated bottom eigenvalue: the bottom Rayleigh quotient reaches it
    rng = np.random.default_rng(17)
    Q, _ = np.linalg.qr(rng.standard_normal((48, 48)))
    ev = np.concatenate([np.linspace(1.0, 0.2, 47), [1e-3]])
    _, qb = power_pair((Q * ev) @ Q.T, 200)
    assert 1e-3 <= qb <= 1e-3 * (1 + 1e-6)


@pytest.mark.parametrize("mode", [2, 3])
def test_final_step_forms_only_x(mode):
    """When the final-step bound already meets tol, the last iteration forms
    only X: the result still meets the bound against the true root (the
    root's relative error is about r / p), and it takes no more iterations
    than the residual test would."""
    for cond in (1e2, 1e4):
        A = _rotated(64, cond, 11)
        X, info = inverse_root_coupled_newton(A, 4, 40, 1e-9, scale_mode=mode)
        assert info.status == "converged" and info.last_x_only
        assert rel(X, inverse_root_eigh(A)) < 1e-9
        M = np.linalg.matrix_power(X, 4) @ A  # the residual of the kept X, formed here
        # (formed again here, so up to the rounding of X^4 A itself)
        assert np.linalg.norm(M - np.eye(64)) / 8.0 <= info.residuals[-1] * 1.01 + 1e-11


# ---------------------------------------------------------------------------
# The scalar map of one coupled Newton iteration and the balance of scale
# mode 3, pinned by their closed forms (not by the code's own formula)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("p", [4, 6, 8])
def test_newton_map_shape(p):
    """f(m) = m ((p + 1 - m)/p)^p is the eigenvalue map of one iteration. Its
    fixed point 1 is a maximum of value 1 (f'(1) = 0 only for the exponent
    p), f is 0 at both ends of (0, p + 1) and maps the interval into (0, 1],
    and near 1 it is quadratic: 1 - f(1 + e) = C e^2 + O(e^3) with
    C = (p + 1) / (2 p), the constant of the final-step bound."""
    assert newton_map(1.0, p) == 1.0
    assert newton_map(0.0, p) == 0.0 and abs(newton_map(p + 1.0, p)) == 0.0
    m = np.linspace(1e-6, p + 1 - 1e-6, 4001)
    fm = np.array([newton_map(x, p) for x in m])
    assert np.all(fm > 0.0) and np.all(fm <= 1.0)
    assert np.all(np.diff(fm[m < 1.0]) > 0.0) and np.all(np.diff(fm[m > 1.0]) < 0.0)
    for e in (1e-3, -1e-3):
        assert newton_map(1.0 + e, p) < 1.0
        C = (1.0 - newton_map(1.0 + e, p)) / (e * e)
        assert C == pytest.approx((p + 1) / (2.0 * p), rel=5e-3)
    # mu scales the argument: f(m; mu) = f(mu m)
    assert newton_map(0.3, p, 2.5) == newton_map(0.75, p)


def _balance_closed_form(a, p):
    """f(mu a) = f(mu) reduces to a^(1/p) (p + 1 - mu a) = p + 1 - mu, so
    mu = (p + 1)(1 - c) / (1 - c a) with c = a^(1/p); capped at 0.9 (p + 1)."""
    c = a ** (1.0 / p)
    return min((p + 1) * (1.0 - c) / (1.0 - c * a), 0.9 * (p + 1))


@pytest.mark.parametrize("p", [4, 6, 8])
def test_newton_balance_closed_form(p):
    """The bisection lands within its final bracket of the closed-form
    balance point, the balance holds there (f(mu a) = f(mu) up to the bracket
    width times the map's slope), and a bottom estimate too small to balance
    inside [1, 0.9 (p + 1)] returns the cap."""
    from scipy.optimize import brentq
    width = (0.9 * (p + 1) - 1.0) / 2.0 ** 40
    for a in (1e-3, 0.01, 0.05, 0.1, 0.3, 0.5, 0.74):
        mu = newton_balance(a, p)
        ref = _balance_closed_form(a, p)
        assert 1.0 <= mu <= 0.9 * (p + 1)
        assert abs(mu - ref) <= 2.0 * width + 1e-14 * ref, (a, mu, ref)
        if ref < 0.9 * (p + 1):
            # an independent root finder on the defining equation
            g = lambda x: x * a * (p + 1 - x * a) ** p - x * (p + 1 - x) ** p  # noqa: E731
            assert abs(mu - brentq(g, 1.0, 0.9 * (p + 1), xtol=1e-15, rtol=1e-15)) <= 2.0 * width
            # the two ends of the spectrum land together
            assert abs(newton_map(mu * a, p) - newton_map(mu, p)) < 1e-9
    # tiny bottom estimate: the balance point lies beyond the cap
    assert _balance_closed_form(1e-12, p) == 0.9 * (p + 1)
    assert newton_balance(1e-12, p) == 0.9 * (p + 1)
