"""Planted mistakes: each mutation of the oracle must make some pin fail.

A mutation is planted in the oracle module on the CPU only (monkeypatch);
the pins in test_oracle_pins are then run against the mutated oracle and at
least one of them has to fail.
"""
import numpy as np
import pytest

import oracle.shampoo_oracle as orc
from tests import test_oracle_pins as pins

_ORIG = {name: getattr(orc, name) for name in
         ("update_statistics", "precondition", "inverse_root_eigh", "pack_blocks", "block_table",
          "newton_map", "newton_balance")}


def _stats_L_uses_GtG(L, R, G, beta2, stat_scale):
    G = np.asarray(G, np.float64)
    if G.shape[0] != G.shape[1]:
        return _ORIG["update_statistics"](L, R, G, beta2, stat_scale)
    return beta2 * L + stat_scale * (G.T @ G), beta2 * R + stat_scale * (G @ G.T)


def _stats_no_decay_on_old(L, R, G, beta2, stat_scale):
    G = np.asarray(G, np.float64)
    return L + stat_scale * (G @ G.T), R + stat_scale * (G.T @ G)


def _stats_gamma_dropped(L, R, G, beta2, stat_scale):
    G = np.asarray(G, np.float64)
    return beta2 * L + G @ G.T, beta2 * R + G.T @ G


def _precondition_sides_swapped(XL, G, XR):
    # roots on the wrong sides: a shape error for rectangular blocks
    return np.asarray(XR) @ np.asarray(G, np.float64) @ np.asarray(XL)


def _precondition_transposed_gradient(XL, G, XR):
    G = np.asarray(G, np.float64)
    if G.shape[0] == G.shape[1]:
        return XL @ G.T @ XR
    return XL @ G @ XR


def _root_half_power(A, p=4):
    return _ORIG["inverse_root_eigh"](A, 2)


def _root_wrong_sign_power(A, p=4):
    A = np.asarray(A, np.float64)
    lam, Q = np.linalg.eigh(A)
    return (Q * lam ** (1.0 / p)) @ Q.T


def _pack_transposed_blocks(mats, table, br, bc):
    out = np.zeros((len(table), br, bc), dtype=mats[0].dtype)
    for b in table:
        blk = mats[b.mat][b.r0:b.r0 + b.m, b.c0:b.c0 + b.n]
        out[b.id, :b.m, :b.n] = blk[::-1, :] if b.m > 1 else blk
    return out


def _table_column_major(shapes, br, bc):
    t = _ORIG["block_table"](shapes, br, bc)
    out = []
    for mat in sorted({b.mat for b in t}):
        bs = sorted([b for b in t if b.mat == mat], key=lambda b: (b.bj, b.bi))
        out.extend(bs)
    return [orc.BlockInfo(i, b.mat, b.bi, b.bj, b.r0, b.c0, b.m, b.n) for i, b in enumerate(out)]


def _map_exponent_off_by_one(m, p, mu=1.0):
    # one power too few in the eigenvalue map of a Newton iteration
    y = mu * m
    return y * ((p + 1 - y) / p) ** (p - 1)


def _balance_branch_flipped(a, p):
    # the bisection keeps the wrong half of its bracket
    lo, hi = 1.0, 0.9 * (p + 1)
    if orc.newton_map(a, p, hi) < orc.newton_map(1.0, p, hi):
        return hi
    for _ in range(orc.BALANCE_STEPS):
        mid = 0.5 * (lo + hi)
        if orc.newton_map(a, p, mid) < orc.newton_map(1.0, p, mid):
            hi = mid
        else:
            lo = mid
    return lo


PIN_TESTS = [
    ("two_by_two_all_ones", pins.test_two_by_two_example_all_ones, ()),
    ("two_by_two_sum", pins.test_two_by_two_example_diagonal_sum_form, ()),
    ("diag_rect", pins.test_diagonal_gradients_closed_form, (6, 3)),
    ("kron_rect", pins.test_kronecker_bruteforce_tiny, (4, 5)),
    ("kron_square", pins.test_kronecker_bruteforce_tiny, (6, 6)),
    ("svd_rect", pins.test_first_step_svd_closed_form, (9, 4)),
    ("shared_sv", pins.test_shared_singular_vectors_multistep, ()),
    ("closed_sum", pins.test_statistics_closed_sum, ()),
    ("scalar", pins.test_scalar_one_by_one, ()),
    ("stale", pins.test_stale_roots_between_refreshes, ()),
    ("pack_enum", pins.test_pack_matches_elementwise_enumeration, ()),
    ("analytic_2x2", pins.test_inverse_root_2x2_analytic, ()),
    ("newton_map_shape", pins.test_newton_map_shape, (4,)),
    ("newton_balance", pins.test_newton_balance_closed_form, (4,)),
]

MUTATIONS = [
    ("update_statistics", _stats_L_uses_GtG),
    ("update_statistics", _stats_no_decay_on_old),
    ("update_statistics", _stats_gamma_dropped),
    ("precondition", _precondition_sides_swapped),
    ("precondition", _precondition_transposed_gradient),
    ("inverse_root_eigh", _root_half_power),
    ("inverse_root_eigh", _root_wrong_sign_power),
    ("pack_blocks", _pack_transposed_blocks),
    ("block_table", _table_column_major),
    ("newton_map", _map_exponent_off_by_one),
    ("newton_balance", _balance_branch_flipped),
]


@pytest.mark.parametrize("name,mutant", MUTATIONS, ids=[m[1].__name__ for m in MUTATIONS])
def test_some_pin_catches_mutation(monkeypatch, name, mutant):
    monkeypatch.setattr(orc, name, mutant)
    monkeypatch.setattr(pins, name, mutant, raising=False)
    caught = []
    for label, fn, args in PIN_TESTS:
        try:
            fn(*args)
        except (AssertionError, np.linalg.LinAlgError, ValueError, IndexError):
            caught.append(label)
    assert caught, f"no pin fails when {name} is replaced by {mutant.__name__}"
