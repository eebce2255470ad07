"""Oracle for order-k tensor Shampoo: plain, slow, fp64, CPU only.

TEST INFRASTRUCTURE: only the test suite, the package's smoke check and the
benchmark's CPU baseline import it; the product path never does.

What it computes (podcast "Preconditioned Optimization Without the Full
Matrix Cost", cue 26, the order-k algorithm): a parameter tensor of order k
keeps one statistic per dimension; the statistic of dimension i accumulates
the contraction of the gradient with itself over every other dimension
(G_(i) G_(i)^T with G_(i) the mode-i unfolding); the update applies each
statistic's -1/(2k) power to the gradient through a product along its own
mode, in any order (the mode products commute). For k = 2 this is the matrix
method with power -1/4.

Readings taken where the cue is silent: the statistics are the same EMA as
for matrices (weight beta2, stat_scale, start eps I), the refresh schedule
and the momentum of cue 28 are the matrices' ones; blocks are cut per
dimension at that dimension's block size (a dimension shorter than its block
size is one block), row-major block order inside a tensor, tensors in
registration order, tails keep their real extents.
"""
from __future__ import annotations

import itertools
from dataclasses import dataclass

import numpy as np

from .shampoo_oracle import (inverse_root_coupled_newton, inverse_root_eigh, is_refresh_step,
                             round_to_bf16)

__all__ = ["TensorBlock", "tensor_block_table", "mode_unfold", "mode_product",
           "precondition_tensor", "pack_tensor_blocks", "TensorShampooOracle"]


@dataclass(frozen=True)
class TensorBlock:
    id: int
    tensor: int
    origin: tuple  # first index of the block in every dimension
    extent: tuple  # real extent in every dimension

    def slices(self):
        return tuple(slice(o, o + e) for o, e in zip(self.origin, self.extent))


def _sizes(b, k):
    return (int(b),) * k if np.isscalar(b) else tuple(int(x) for x in b)


def tensor_block_table(shapes, b):
    """Blocks of every tensor: b is one block size for every dimension or one
    per dimension; dimension i is cut into chunks of b_i (the last one ragged).
    Row-major block order inside a tensor, tensors in registration order.

    Pinned by: test_tensor_block_table, test_tensor_block_table_per_dimension_sizes.
    """
    table = []
    for t, shape in enumerate(shapes):
        sizes = _sizes(b, len(shape))
        counts = [max(1, -(-d // s)) for d, s in zip(shape, sizes)]
        for idx in itertools.product(*[range(c) for c in counts]):
            origin = tuple(i * s for i, s in zip(idx, sizes))
            extent = tuple(min(s, d - o) for s, d, o in zip(sizes, shape, origin))
            if min(extent) > 0:
                table.append(TensorBlock(len(table), t, origin, extent))
    return table


def pack_tensor_blocks(tensors, table, b):
    """[n_blocks, b_1, ..., b_k]: each block at its origin, zeros past its real extent.

    Pinned by: test_pack_tensor_blocks_places_and_pads.
    """
    k = len(table[0].extent) if table else 0
    sizes = _sizes(b, k)
    out = np.zeros((len(table),) + sizes, dtype=np.asarray(tensors[0]).dtype if tensors else float)
    for blk in table:
        out[(blk.id,) + tuple(slice(0, e) for e in blk.extent)] = \
            np.asarray(tensors[blk.tensor])[blk.slices()]
    return out


def mode_unfold(G, i):
    """Mode-i unfolding: rows indexed by dimension i, columns by the others
    in their original (row-major) order.

    Pinned by: test_unfold_and_mode_product_by_hand,
        test_statistics_sum_over_every_other_dimension_by_hand.
    """
    G = np.asarray(G)
    return np.moveaxis(G, i, 0).reshape(G.shape[i], -1)


def mode_product(G, X, i):
    """G x_i X: Y[..., j, ...] = sum_l X[j, l] G[..., l, ...] along dimension i.

    Pinned by: test_unfold_and_mode_product_by_hand, test_mode_order_does_not_matter.
    """
    return np.moveaxis(np.tensordot(X, np.asarray(G, np.float64), axes=([1], [i])), 0, i)


def precondition_tensor(G, roots, order=None):
    """G x_1 X_1 x_2 X_2 ... x_k X_k (in the given order of dimensions).

    Pinned by: test_kronecker_bruteforce, test_rank_one_closed_form,
        test_mode_order_does_not_matter.
    """
    U = np.asarray(G, np.float64)
    for i in (range(U.ndim) if order is None else order):
        U = mode_product(U, roots[i], i)
    return U


class TensorShampooOracle:
    """Blocked order-k Shampoo over tensors of one order k, in fp64.

    shapes: tensor shapes (all of order k); b: block size (one, or one per
    dimension); root_method "eigh" (the definition) or "newton" (coupled
    Newton for the inverse 2k-th root, newton_iters / newton_tol /
    newton_scale_mode as for matrices). Other arguments as ShampooOracle.

    Pinned by: test_order_two_is_the_matrix_method, test_kronecker_bruteforce,
        test_newton_root_at_power_2k, test_full_tensor_step_moves_only_its_blocks.
    """

    def __init__(self, shapes, b, beta2, eps, lr, root_every, stat_scale=None, blocks=None,
                 root_method="eigh", newton_iters=25, newton_tol=0.0, newton_scale_mode=2,
                 param_bf16=False, momentum=0.0):
        self.shapes = [tuple(s) for s in shapes]
        self.k = len(self.shapes[0])
        if any(len(s) != self.k for s in self.shapes):
            raise ValueError("all tensors must have the same order")
        self.table = tensor_block_table(self.shapes, b)
        self.ids = list(range(len(self.table))) if blocks is None else sorted(set(blocks))
        self.beta2 = float(beta2)
        self.stat_scale = 1.0 - self.beta2 if stat_scale is None else float(stat_scale)
        self.eps, self.lr, self.root_every = float(eps), float(lr), int(root_every)
        self.root_method = root_method
        self.newton_iters, self.newton_tol = newton_iters, newton_tol
        self.newton_scale_mode = newton_scale_mode
        self.param_bf16 = param_bf16
        self.momentum = float(momentum)
        self.t = 0
        self.H = {i: [self.eps * np.eye(e) for e in self.table[i].extent] for i in self.ids}
        self.X = {i: None for i in self.ids}
        self.info = {i: None for i in self.ids}
        self.mom = {i: np.zeros(self.table[i].extent) for i in self.ids}

    @property
    def p(self):
        return 2 * self.k

    def _root(self, H):
        if self.root_method == "eigh":
            return inverse_root_eigh(H, self.p), None
        if self.root_method == "newton":
            return inverse_root_coupled_newton(H, self.p, self.newton_iters, self.newton_tol,
                                               self.newton_scale_mode)
        raise ValueError(self.root_method)

    def refresh_roots(self):
        for i in self.ids:
            pairs = [self._root(H) for H in self.H[i]]
            self.X[i] = [x for x, _ in pairs]
            self.info[i] = [inf for _, inf in pairs]

    def block(self, A, i):
        b = self.table[i]
        return np.asarray(A[b.tensor][b.slices()], dtype=np.float64)

    def step_blocks(self, block_grads, block_params=None, force_refresh=False, auto_refresh=True):
        """One step on the tracked blocks; returns ({id: new block} or None, {id: U})."""
        self.t += 1
        G = {i: np.asarray(block_grads[i], np.float64) for i in self.ids}
        for i in self.ids:
            for m in range(self.k):
                # the statistic of dimension m: the matrices' EMA (the left
                # statistic's rule) on the unfolding, H <- beta2 H + g G_(m) G_(m)^T
                Gm = mode_unfold(G[i], m)
                self.H[i][m] = self.beta2 * self.H[i][m] + self.stat_scale * (Gm @ Gm.T)
        if force_refresh or (auto_refresh and is_refresh_step(self.t, self.root_every)):
            self.refresh_roots()
        updates, new = {}, {}
        for i in self.ids:
            if self.X[i] is None:
                raise RuntimeError("step before any root refresh")
            D = G[i]
            if self.momentum != 0.0:
                self.mom[i] = self.momentum * self.mom[i] + G[i]
                D = self.mom[i]
            updates[i] = precondition_tensor(D, self.X[i])
            if block_params is not None:
                W = np.asarray(block_params[i], np.float64) - self.lr * updates[i]
                new[i] = round_to_bf16(W) if self.param_bf16 else W
        return (new if block_params is not None else None), updates

    def step(self, grads, params, force_refresh=False, auto_refresh=True):
        """One step over full tensors; returns (new params in fp64, {id: U})."""
        gb = {i: self.block(grads, i) for i in self.ids}
        new_params = [np.array(p, dtype=np.float64) for p in params]
        wb = {i: self.block(new_params, i) for i in self.ids}
        new_blocks, updates = self.step_blocks(gb, wb, force_refresh, auto_refresh)
        for i in self.ids:
            b = self.table[i]
            new_params[b.tensor][b.slices()] = new_blocks[i]
        return new_params, updates
