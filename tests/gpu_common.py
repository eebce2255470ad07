"""Shared driver of the GPU parity tests: runs the HIP library through the C
ABI (via the ctypes binding) and the fp64 oracle side by side on the same
seeded gradients, and compares sampled blocks."""
from __future__ import annotations

import dataclasses
import math
import sys

import numpy as np
import torch

from blocked_shampoo_preconditioning_amd import configs, synth
from blocked_shampoo_preconditioning_amd.shampoo import Shampoo
from oracle import ShampooOracle, block_table

STATS_TOL = 1e-5     # relative Frobenius error of L and R
UPDATE_TOL = 2e-3    # relative Frobenius error of the preconditioned update


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (nb if nb > 0 else 1.0))


def workload(name, **over):
    return dataclasses.replace(configs.get(name), **over)


def make_shampoo(w):
    return Shampoo(w.shapes, w.block_rows, w.block_cols, beta2=w.beta2, eps=w.eps, lr=w.lr,
                   root_every=w.root_every, newton_max_iters=w.newton_max_iters,
                   newton_tol=w.newton_tol, newton_scale_mode=w.newton_scale_mode, dtype=w.dtype,
                   momentum=w.momentum, root_method=w.root_method, cheb_degree=w.cheb_degree,
                   fp32_gemm=w.fp32_gemm)


def sample_blocks(w, k, seed=0):
    """Seeded sample of about k block ids: one block of every matrix shape,
    up to a third tail blocks, the rest at random."""
    table = block_table(w.shapes, w.block_rows, w.block_cols)
    rng = np.random.default_rng(seed)
    ids = set()
    by_shape = {}
    for b in table:
        by_shape.setdefault(w.shapes[b.mat], []).append(b.id)
    for lst in by_shape.values():
        ids.add(int(rng.choice(lst)))
    tails = [b.id for b in table if (b.m, b.n) != (w.block_rows, w.block_cols)]
    for i in rng.permutation(tails)[: k // 3]:
        ids.add(int(i))
    rest = [b.id for b in table if b.id not in ids]
    for i in rng.permutation(rest)[: max(0, k - len(ids))]:
        ids.add(int(i))
    return sorted(ids)


def spread_sample(w, k, seed=0, residues=8):
    """sample_blocks(w, k, seed) widened so that it holds the first and the
    last block and a block of every residue of the block id mod `residues`
    (the symmetric products deal factor f to XCD f mod 8, and factor ids
    are block ids for L and B + block id for R)."""
    B = len(block_table(w.shapes, w.block_rows, w.block_cols))
    ids = set(sample_blocks(w, k, seed)) | {0, B - 1}
    rng = np.random.default_rng(seed + 1000)
    for r in range(residues):
        if not any(i % residues == r for i in ids):
            ids.add(int(rng.choice(np.arange(r, B, residues))))
    return sorted(ids)


def block_of(t, b):
    """Host fp64 copy of block b (real extent) of a device matrix."""
    return t[b.r0:b.r0 + b.m, b.c0:b.c0 + b.n].float().cpu().numpy().astype(np.float64)


@dataclasses.dataclass
class Record:
    t: int
    stats_err: float
    update_err: float
    per_block: dict


def run_parity(w, steps, ids=None, root_method="eigh", check_update=True, on_step=None,
               compare=None):
    """Run `steps` steps of workload w on the GPU and in the oracle (tracked
    blocks `ids`, default all), comparing after every step t with
    compare(t) true (default: all). Returns (records, shampoo, oracle,
    params, oracle parameter blocks)."""
    dev = torch.device("cuda")
    table = block_table(w.shapes, w.block_rows, w.block_cols)
    ids = list(range(len(table))) if ids is None else list(ids)
    src = synth.GradientSource(w, device=dev)
    params = src.init_params()
    sh = make_shampoo(w)
    orc = ShampooOracle(w.shapes, w.block_rows, w.block_cols, w.beta2, w.eps, w.lr, w.root_every,
                        blocks=ids, root_method=root_method, newton_iters=w.newton_max_iters,
                        newton_tol=w.newton_tol, newton_scale_mode=w.newton_scale_mode,
                        param_bf16=(w.dtype == "bf16"), momentum=w.momentum,
                        cheb_degree=w.cheb_degree)
    W = {i: block_of(params[table[i].mat], table[i]) for i in ids}
    B, br, bc = sh.n_blocks, w.block_rows, w.block_cols
    U_out = torch.empty(B * br * bc, dtype=torch.float32, device=dev) if check_update else None
    records = []
    for t in range(1, steps + 1):
        if on_step is not None:
            on_step(t - 1, sh, orc, params, None, None, None)
        grads = src.grads(t)
        G = {i: block_of(grads[table[i].mat], table[i]) for i in ids}
        sh.step(params, grads)
        W, U = orc.step_blocks(G, W)
        if compare is not None and not compare(t):
            continue
        torch.cuda.synchronize()
        Lg, Rg = sh.stats()
        per = {}
        se = ue = 0.0
        Ugpu = {}
        if check_update:
            sh.precondition(U_out)
            Ug = U_out.view(B, br, bc)
        for i in ids:
            b = table[i]
            st = orc.state[i]
            eL = rel(Lg[i, :b.m, :b.m].cpu().numpy(), st.L)
            eR = rel(Rg[i, :b.n, :b.n].cpu().numpy(), st.R)
            if check_update:
                Ugpu[i] = Ug[i, :b.m, :b.n].cpu().numpy().astype(np.float64)
            eU = rel(Ugpu[i], U[i]) if check_update else float("nan")
            per[i] = (eL, eR, eU)
            se = max(se, eL, eR)
            if check_update:
                ue = max(ue, eU)
        records.append(Record(t, se, ue, per))
        if on_step is not None:
            on_step(t, sh, orc, params, grads, U, Ugpu)
        log(f"  {w.name} t={t}: stats {se:.2e} update {ue:.2e}")
    return records, sh, orc, params, W


def assert_params_match(w, params, W, tol=UPDATE_TOL):
    """The fused parameter write of every tracked block: the GPU's cumulative
    parameter change against the oracle's, relative Frobenius error <= tol
    per block (the update bar applied to the sum of the steps)."""
    table = block_table(w.shapes, w.block_rows, w.block_cols)
    W0 = synth.GradientSource(w, device="cuda").init_params()
    worst = 0.0
    for i, Wo in W.items():
        b = table[i]
        w0 = block_of(W0[b.mat], b)
        e = rel(block_of(params[b.mat], b) - w0, Wo - w0)
        worst = max(worst, e)
        assert e <= tol, (i, e)
    log(f"  parameter change vs oracle, worst block: {worst:.2e}")
    return worst


def cond_of(A):
    lam = np.linalg.eigvalsh(A)
    return float(lam.max() / lam.min()) if lam.min() > 0 else math.inf
