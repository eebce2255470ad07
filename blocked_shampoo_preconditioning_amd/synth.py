"""Seeded synthetic inputs: gradients and initial parameters.

This module holds input generation only and none of the method's arithmetic;
the same tensors feed the HIP library and the fp64 oracle. Values are drawn
with torch's generator on the chosen device, so a given (workload, seed,
step, device type) always gives the same tensors.

Distributions (per workload, see ``configs``):
  iid         G ~ N(0, grad_std^2) elementwise.
  row_scaled  G = N(0, grad_std^2) * s_row, s_row log-uniform on [1e-2, 1],
              drawn once per matrix row and kept for every step.
  col_scaled  the same with one scale per column.
  low_rank    G = A diag(c_t) B^T + N(0, noise_std^2); A (rows x rank) and
              B (cols x rank) have N(0, grad_std^2) entries and are fixed per
              matrix, c_t ~ N(0, 1)^rank is drawn per step.
  diag_fraction > 0: that fraction of all blocks (rounded, chosen once by a
              seeded permutation over all blocks of all matrices) carries a
              diagonal gradient: off-diagonal entries of the block are 0.
Initial parameters: N(0, init_std^2), stored in the workload's dtype.

Tensor workloads (TensorGradientSource): iid N(0, grad_std^2), or row_scaled
with one log-uniform [1e-2, 1] scale per index of the first dimension (the
output channel of a conv filter), fixed for every step.
"""
from __future__ import annotations

import math

import torch

from .configs import TensorWorkload, Workload

_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16}


def torch_dtype(w):
    return _DTYPES[w.dtype]


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) & 0x7FFF_FFFF_FFFF_FFFF)
    return g


def diagonal_blocks(w: Workload, seed=None):
    """Set of (matrix, block_row, block_col) whose gradient is diagonal."""
    if w.diag_fraction <= 0.0:
        return set()
    coords = []
    for i, (r, c) in enumerate(w.shapes):
        for bi in range(-(-r // w.block_rows)):
            for bj in range(-(-c // w.block_cols)):
                coords.append((i, bi, bj))
    k = int(round(w.diag_fraction * len(coords)))
    perm = torch.randperm(len(coords), generator=_gen("cpu", (w.seed if seed is None else seed) * 7 + 3))
    return {coords[j] for j in perm[:k].tolist()}


class GradientSource:
    """Deterministic per-step gradients of one workload."""

    def __init__(self, w: Workload, device="cpu", seed=None):
        self.w = w
        self.device = torch.device(device)
        self.seed = w.seed if seed is None else int(seed)
        dev_type = self.device.type
        g = _gen(dev_type, self.seed * 1_000_003 + 17)
        lo, hi = math.log(1e-2), 0.0
        self._scale = []
        self._factors = []
        for (r, c) in w.shapes:
            if w.grad == "row_scaled":
                u = torch.rand(r, 1, generator=g, device=self.device)
                self._scale.append(torch.exp(lo + (hi - lo) * u))
            elif w.grad == "col_scaled":
                u = torch.rand(1, c, generator=g, device=self.device)
                self._scale.append(torch.exp(lo + (hi - lo) * u))
            else:
                self._scale.append(None)
            if w.grad == "low_rank":
                A = torch.randn(r, w.rank, generator=g, device=self.device) * w.grad_std
                B = torch.randn(c, w.rank, generator=g, device=self.device) * w.grad_std
                self._factors.append((A, B))
            else:
                self._factors.append(None)
        self._diag = {}
        for (i, bi, bj) in diagonal_blocks(w, self.seed):
            self._diag.setdefault(i, []).append((bi, bj))

    def grads(self, step):
        """Gradients of step `step` (1-based), one tensor per matrix."""
        w = self.w
        g = _gen(self.device.type, self.seed * 1_000_003 + 101 * int(step) + 29)
        out = []
        for i, (r, c) in enumerate(w.shapes):
            if w.grad == "low_rank":
                A, B = self._factors[i]
                coef = torch.randn(w.rank, generator=g, device=self.device)
                G = (A * coef) @ B.T
                G += torch.randn(r, c, generator=g, device=self.device) * w.noise_std
            else:
                G = torch.randn(r, c, generator=g, device=self.device) * w.grad_std
                if self._scale[i] is not None:
                    G *= self._scale[i]
            for (bi, bj) in self._diag.get(i, ()):
                r0, c0 = bi * w.block_rows, bj * w.block_cols
                blk = G[r0:r0 + w.block_rows, c0:c0 + w.block_cols]
                d = torch.diagonal(blk).clone()
                blk.zero_()
                torch.diagonal(blk).copy_(d)
            out.append(G.to(torch_dtype(w)).contiguous())
        return out

    def init_params(self):
        w = self.w
        g = _gen(self.device.type, self.seed * 1_000_003 + 5)
        return [(torch.randn(r, c, generator=g, device=self.device) * w.init_std)
                .to(torch_dtype(w)).contiguous() for (r, c) in w.shapes]


class TensorGradientSource:
    """Deterministic per-step gradients of a tensor workload."""

    def __init__(self, w: TensorWorkload, device="cpu", seed=None):
        self.w = w
        self.device = torch.device(device)
        self.seed = w.seed if seed is None else int(seed)
        g = _gen(self.device.type, self.seed * 1_000_003 + 19)
        lo, hi = math.log(1e-2), 0.0
        self._scale = []
        for shape in w.shapes:
            if w.grad == "row_scaled":
                u = torch.rand((shape[0],) + (1,) * (len(shape) - 1), generator=g, device=self.device)
                self._scale.append(torch.exp(lo + (hi - lo) * u))
            else:
                self._scale.append(None)

    def grads(self, step):
        w = self.w
        g = _gen(self.device.type, self.seed * 1_000_003 + 101 * int(step) + 31)
        out = []
        for i, shape in enumerate(w.shapes):
            G = torch.randn(shape, generator=g, device=self.device) * w.grad_std
            if self._scale[i] is not None:
                G *= self._scale[i]
            out.append(G.to(torch_dtype(w)).contiguous())
        return out

    def init_params(self):
        w = self.w
        g = _gen(self.device.type, self.seed * 1_000_003 + 7)
        return [(torch.randn(s, generator=g, device=self.device) * w.init_std)
                .to(torch_dtype(w)).contiguous() for s in w.shapes]
