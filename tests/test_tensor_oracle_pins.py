"""Pins of the order-k tensor oracle (podcast cue 26)."""
import math

import numpy as np
import pytest

from oracle import ShampooOracle, inverse_root_eigh
from oracle.tensor_oracle import (TensorShampooOracle, mode_product, mode_unfold,
                                  pack_tensor_blocks, precondition_tensor, tensor_block_table)


def rel(a, b):
    return float(np.linalg.norm(np.asarray(a) - np.asarray(b)) / np.linalg.norm(np.asarray(b)))


def run(shape, Gs, b2=0.95, eps=1e-2, k_root=1):
    o = TensorShampooOracle([shape], max(shape), b2, eps, 1e-3, k_root)
    return o, [o.step_blocks({0: G})[1][0] for G in Gs]


def test_unfold_and_mode_product_by_hand():
    G = np.arange(24.0).reshape(2, 3, 4)
    U1 = mode_unfold(G, 1)
    assert U1.shape == (3, 8) and U1[2, 5] == G[1, 2, 1]  # columns (a, c) row-major
    X = np.arange(9.0).reshape(3, 3)
    Y = mode_product(G, X, 1)
    for a in range(2):
        for j in range(3):
            for c in range(4):
                assert Y[a, j, c] == sum(X[j, l] * G[a, l, c] for l in range(3))


@pytest.mark.parametrize("momentum", [0.0, 0.9])
def test_order_two_is_the_matrix_method(momentum):
    """k = 2: power -1/4, left and right statistics, the same momentum."""
    rng = np.random.default_rng(71)
    Gs = [rng.standard_normal((5, 7)) for _ in range(4)]
    o = TensorShampooOracle([(5, 7)], 7, 0.9, 1e-3, 1e-3, 2, momentum=momentum)
    Ut = [o.step_blocks({0: G})[1][0] for G in Gs]
    m = ShampooOracle([(5, 7)], 5, 7, 0.9, 1e-3, 1e-3, 2, momentum=momentum)
    Um = [m.step([G], [np.zeros((5, 7))])[1][0] for G in Gs]
    for a, b in zip(Ut, Um):
        assert rel(a, b) < 1e-12


@pytest.mark.parametrize("shape", [(2, 3, 2), (3, 2, 2, 2)])
def test_kronecker_bruteforce(shape):
    """vec_r(U) = (H_1 kron ... kron H_k)^(-1/(2k)) vec_r(G)."""
    rng = np.random.default_rng(73)
    Gs = [rng.standard_normal(shape) for _ in range(3)]
    o, Us = run(shape, Gs)
    H = o.H[0]
    K = H[0]
    for h in H[1:]:
        K = np.kron(K, h)
    lam, Q = np.linalg.eigh(K)
    ref = ((Q * lam ** (-1.0 / (2 * len(shape)))) @ Q.T @ Gs[-1].reshape(-1)).reshape(shape)
    assert rel(Us[-1], ref) < 1e-10


def test_rank_one_closed_form():
    """G = a o b o c, one step: every statistic has its factor as an eigenvector
    with eigenvalue b2 eps + g |G|^2, so U = G / sqrt(b2 eps + g |G|^2)."""
    rng = np.random.default_rng(75)
    a, b, c = rng.standard_normal(4), rng.standard_normal(3), rng.standard_normal(5)
    G = np.einsum("i,j,k->ijk", a, b, c)
    b2, eps = 0.9, 1e-2
    _, Us = run(G.shape, [G], b2, eps)
    assert rel(Us[0], G / math.sqrt(b2 * eps + (1 - b2) * np.sum(G * G))) < 1e-12


def test_mode_order_does_not_matter():
    rng = np.random.default_rng(77)
    G = rng.standard_normal((3, 4, 2, 3))
    roots = [inverse_root_eigh(np.cov(rng.standard_normal((n, 3 * n))) + np.eye(n), 8)
             for n in G.shape]
    ref = precondition_tensor(G, roots)
    for order in ((3, 1, 0, 2), (2, 3, 1, 0)):
        assert rel(precondition_tensor(G, roots, order), ref) < 1e-13


def test_tensor_block_table():
    t = tensor_block_table([(5, 3, 8)], 4)
    assert len(t) == 2 * 1 * 2
    assert t[0].origin == (0, 0, 0) and t[0].extent == (4, 3, 4)
    assert t[3].origin == (4, 0, 4) and t[3].extent == (1, 3, 4)


def test_tensor_block_table_per_dimension_sizes():
    t = tensor_block_table([(70, 3, 3), (40, 2, 5)], (32, 4, 4))
    # tensor 0: 3 x 1 x 1 blocks, tensor 1: 2 x 1 x 2
    assert len(t) == 3 + 4
    assert t[2].origin == (64, 0, 0) and t[2].extent == (6, 3, 3)
    assert t[3].tensor == 1 and t[6].origin == (32, 0, 4) and t[6].extent == (8, 2, 1)


def test_pack_tensor_blocks_places_and_pads():
    rng = np.random.default_rng(79)
    T = rng.standard_normal((5, 3, 6))
    table = tensor_block_table([T.shape], (4, 4, 4))
    P = pack_tensor_blocks([T], table, (4, 4, 4))
    assert P.shape == (4, 4, 4, 4)
    assert np.array_equal(P[3, :1, :3, :2], T[4:, :, 4:])
    assert not P[3, 1:].any() and not P[3, :, 3:].any() and not P[3, :, :, 2:].any()
    assert np.array_equal(P[0, :4, :3, :4], T[:4, :, :4])


@pytest.mark.parametrize("k", [3, 4])
def test_newton_root_at_power_2k(k):
    """The coupled Newton root at p = 2k satisfies X^p H = I and is symmetric."""
    rng = np.random.default_rng(81 + k)
    shape = (6, 5, 4, 3)[:k]
    o = TensorShampooOracle([shape], 8, 0.9, 1e-2, 1e-3, 1, root_method="newton",
                            newton_tol=1e-12, newton_iters=60)
    o.step_blocks({0: rng.standard_normal(shape)})
    for H, X in zip(o.H[0], o.X[0]):
        n = H.shape[0]
        assert np.abs(X - X.T).max() < 1e-10
        assert np.abs(np.linalg.matrix_power(X, 2 * k) @ H - np.eye(n)).max() < 1e-8


def test_statistics_sum_over_every_other_dimension_by_hand():
    """H_1[a, b] = beta2 eps [a = b] + g sum_(j, l) G[a, j, l] G[b, j, l] after one step."""
    rng = np.random.default_rng(83)
    G = rng.standard_normal((2, 3, 4))
    b2, eps = 0.8, 0.1
    o, _ = run(G.shape, [G], b2, eps)
    for m, n in ((0, 2), (1, 3), (2, 4)):
        H = o.H[0][m]
        for a in range(n):
            for b in range(n):
                idx_a = [slice(None)] * 3
                idx_b = [slice(None)] * 3
                idx_a[m], idx_b[m] = a, b
                want = b2 * eps * (a == b) + (1 - b2) * np.sum(G[tuple(idx_a)] * G[tuple(idx_b)])
                assert abs(H[a, b] - want) < 1e-13


def test_full_tensor_step_moves_only_its_blocks():
    rng = np.random.default_rng(85)
    shapes = [(9, 3, 3), (4, 5, 2)]
    grads = [rng.standard_normal(s) for s in shapes]
    params = [rng.standard_normal(s) for s in shapes]
    o = TensorShampooOracle(shapes, (4, 4, 4), 0.9, 1e-2, 0.1, 1, blocks=[1])
    new, U = o.step(grads, params)
    b = o.table[1]
    assert np.array_equal(new[1], params[1])
    changed = np.zeros(shapes[0], bool)
    changed[b.slices()] = True
    assert np.array_equal(new[0][~changed], params[0][~changed])
    assert rel(new[0][b.slices()], params[0][b.slices()] - 0.1 * U[1]) < 1e-15


# ---- planted mistakes: each must make one of the pins above fail ----
import oracle.tensor_oracle as tor  # noqa: E402

_PINS = [test_unfold_and_mode_product_by_hand, test_rank_one_closed_form,
         test_statistics_sum_over_every_other_dimension_by_hand,
         lambda: test_kronecker_bruteforce((2, 3, 2)), lambda: test_kronecker_bruteforce((3, 2, 2, 2)),
         lambda: test_order_two_is_the_matrix_method(0.0),
         lambda: test_order_two_is_the_matrix_method(0.9), test_pack_tensor_blocks_places_and_pads,
         test_tensor_block_table_per_dimension_sizes]


def _transposed_operand(G, X, i):
    return np.moveaxis(np.tensordot(np.asarray(X).T, np.asarray(G, np.float64), axes=([1], [i])), 0, i)


_EIGH = tor.inverse_root_eigh


def _root_quarter_power(H, p=4):
    return _EIGH(H, 4)


def _modes_reversed(G, roots, order=None):
    U = np.asarray(G, np.float64)
    k = U.ndim
    for i in range(k):
        U = tor.mode_product(U, roots[k - 1 - i], i)
    return U


@pytest.mark.parametrize("name,value,module_attr", [
    ("transposed X in the mode product", _transposed_operand, "mode_product"),
    ("power -1/4 for every order", _root_quarter_power, "inverse_root_eigh"),
    ("roots applied along the wrong modes", _modes_reversed, "precondition_tensor"),
])
def test_planted_mistake_is_caught(monkeypatch, name, value, module_attr):
    monkeypatch.setattr(tor, module_attr, value)
    monkeypatch.setitem(globals(), module_attr, value)
    failed = 0
    for pin in _PINS:
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            failed += 1
    assert failed > 0, name
