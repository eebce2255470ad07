"""GPU parity of order-k tensor Shampoo (podcast cue 26) through the C ABI
against the fp64 tensor oracle.

Bars as for matrices: statistics <= 1e-5 relative Frobenius error per
dimension and block, the preconditioned update <= 2e-3 per block, the
parameter change likewise, pack / unpack bit-exact. The cases cover every
kernel path: dimensions blocked at multiples of 32 (MFMA SYRK after a
transpose, without one for the last dimension, MFMA and FMA mode products),
dimensions blocked at <= 8 (reduction statistics, fp64 Jacobi roots, FMA
mode products), ragged tails in every dimension, strided tensors, orders
2, 3 and 4.
"""
import dataclasses

import numpy as np
import pytest
import torch

from blocked_shampoo_preconditioning_amd import configs, synth
from blocked_shampoo_preconditioning_amd import shampoo as S
from oracle.tensor_oracle import TensorShampooOracle, pack_tensor_blocks, tensor_block_table
from tests.gpu_common import STATS_TOL, UPDATE_TOL, log, rel

pytestmark = pytest.mark.gpu


def tw(name="case", **kw):
    base = dict(name=name, shapes=((64, 32, 3, 3),), block_dims=(64, 32, 3, 3), beta2=0.95,
                eps=1e-4, lr=1e-2, root_every=2, steps=4, grad="row_scaled", grad_std=1e-1,
                seed=11)
    base.update(kw)
    return configs.TensorWorkload(**base)


CASES = {
    # two large dimensions (SYRK in place and after a transpose, MFMA
    # products), two small ones (their products fused with the update); the
    # second tensor is one ragged block, the third ragged in the small
    # dimensions too
    "conv4_64x32": tw(shapes=((64, 32, 3, 3), (40, 20, 3, 3), (16, 8, 2, 3))),
    # large dimension whose unfolding length (12) needs padding and whose
    # product runs on the FMA kernel; ragged in every dimension
    "conv3_fma": tw(shapes=((96, 3, 3), (50, 7, 2)), block_dims=(32, 4, 3)),
    # small dimensions first; the last dimension needs no transpose
    "order4_last_large": tw(shapes=((3, 3, 64, 32), (2, 3, 50, 40)), block_dims=(3, 3, 64, 32)),
    # small dimension between two large ones
    "order3_mixed": tw(shapes=((64, 5, 64), (33, 4, 70)), block_dims=(32, 5, 32)),
    # order 2: the matrix method
    "order2": tw(shapes=((96, 64), (50, 70)), block_dims=(64, 32)),
}


def make(w, **over):
    kw = dict(beta2=w.beta2, eps=w.eps, lr=w.lr, root_every=w.root_every,
              newton_max_iters=w.newton_max_iters, newton_tol=w.newton_tol,
              newton_scale_mode=w.newton_scale_mode, dtype=w.dtype, momentum=w.momentum,
              root_method=w.root_method, cheb_degree=w.cheb_degree, fp32_gemm=w.fp32_gemm)
    kw.update(over)
    return S.TensorShampoo(w.shapes, w.block_dims, **kw)


def host(t):
    return t.float().cpu().numpy().astype(np.float64)


def run_tensor_parity(w, steps, ids=None, root_method="eigh", sh_over=None):
    """Steps on the GPU and in the oracle, compared after every step; returns
    the worst statistic and update errors and the final parameter error."""
    dev = torch.device("cuda")
    table = tensor_block_table(w.shapes, w.block_dims)
    ids = list(range(len(table))) if ids is None else list(ids)
    src = synth.TensorGradientSource(w, device=dev)
    params = src.init_params()
    P0 = [host(p) for p in params]
    sh = make(w, **(sh_over or {}))
    orc = TensorShampooOracle(w.shapes, w.block_dims, w.beta2, w.eps, w.lr, w.root_every,
                              blocks=ids, root_method=root_method,
                              newton_iters=w.newton_max_iters, newton_tol=w.newton_tol,
                              newton_scale_mode=w.newton_scale_mode,
                              param_bf16=(w.dtype == "bf16"), momentum=w.momentum)
    Wo = {i: orc.block(P0, i) for i in ids}
    B, E = sh.n_blocks, int(sh.info.block_elems)
    Uout = torch.empty(B * E, dtype=torch.float32, device=dev)
    worst_s = worst_u = 0.0
    for t in range(1, steps + 1):
        grads = src.grads(t)
        hg = [host(g) for g in grads]
        G = {i: orc.block(hg, i) for i in ids}
        sh.step(params, grads)
        Wo, U = orc.step_blocks(G, Wo)
        torch.cuda.synchronize()
        stats = sh.stats()
        sh.precondition(Uout)
        Ug = Uout.view(B, *w.block_dims)
        for i in ids:
            b = table[i]
            for d, e in enumerate(b.extent):
                worst_s = max(worst_s, rel(stats[d][i, :e, :e].cpu().numpy(), orc.H[i][d]))
            got = Ug[(i,) + tuple(slice(0, e) for e in b.extent)].cpu().numpy()
            worst_u = max(worst_u, rel(got, U[i]))
        log(f"  {w.name} t={t}: stats {worst_s:.2e} update {worst_u:.2e}")
    wp = 0.0
    for i in ids:
        b = table[i]
        got = host(params[b.tensor])[b.slices()] - P0[b.tensor][b.slices()]
        wp = max(wp, rel(got, Wo[i] - P0[b.tensor][b.slices()]))
    return worst_s, worst_u, wp, sh, orc


# blocks of an odd element count (3 x 5 x 3): the pack's one-element path
PACK_CASES = dict(CASES, odd_block=tw(shapes=((7, 5, 3), (3, 2, 3)), block_dims=(3, 5, 3)))


@pytest.mark.parametrize("case", sorted(PACK_CASES))
def test_tensor_pack_unpack_bitexact(case):
    w = PACK_CASES[case]
    log(f"tensor pack {case}")
    src = synth.TensorGradientSource(w, device="cuda")
    grads = src.grads(1)
    sh = make(w)
    sh.pack(grads)
    torch.cuda.synchronize()
    got = sh.grad_packed().cpu().numpy()
    table = tensor_block_table(w.shapes, w.block_dims)
    ref = pack_tensor_blocks([g.cpu().numpy() for g in grads], table, w.block_dims)
    assert got.shape == ref.shape
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    dst = [torch.full_like(g, float("nan")) for g in grads]
    sh.unpack(dst)
    for g, d in zip(grads, dst):
        assert torch.equal(g, d)
    sh.close()


def test_tensor_pack_strided():
    """A permuted (non-contiguous) view registered with its strides."""
    gen = torch.Generator(device="cuda").manual_seed(5)
    base = torch.randn(3, 70, 6, generator=gen, device="cuda")
    view = base.permute(1, 2, 0)  # (70, 6, 3), strides (6, 1, 420)
    sh = S.TensorShampoo([tuple(view.shape)], (32, 4, 3), strides=[view.stride()])
    S.shampoo_pack(sh.handle, [view.data_ptr()], sh._stream())
    torch.cuda.synchronize()
    table = tensor_block_table([tuple(view.shape)], (32, 4, 3))
    ref = pack_tensor_blocks([view.cpu().numpy()], table, (32, 4, 3))
    got = sh.grad_packed().cpu().numpy()
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    out = torch.zeros_like(base)
    S.shampoo_unpack(sh.handle, [out.data_ptr()], sh._stream())
    torch.cuda.synchronize()
    assert torch.equal(out, base)
    sh.close()


@pytest.mark.parametrize("case", sorted(CASES))
def test_tensor_step_parity(case):
    w = CASES[case]
    log(f"tensor step {case}")
    s, u, wp, sh, _ = run_tensor_parity(w, w.steps)
    assert s <= STATS_TOL and u <= UPDATE_TOL and wp <= UPDATE_TOL, (s, u, wp)
    for d, (st, it, sc) in enumerate(sh.newton_info()):
        assert set(st.cpu().tolist()) <= {1, 2}, (d, st)  # converged, or stalled at the fp32 floor
    assert sh.n_diverged() == 0
    sh.close()


@pytest.mark.parametrize("case", ["conv4_64x32", "order3_mixed"])
def test_tensor_momentum_and_bf16(case):
    w = dataclasses.replace(CASES[case], momentum=0.9)
    log(f"tensor momentum {case}")
    s, u, wp, sh, _ = run_tensor_parity(w, 3)
    assert s <= STATS_TOL and u <= UPDATE_TOL and wp <= UPDATE_TOL, (s, u, wp)
    sh.close()
    wb = dataclasses.replace(CASES[case], dtype="bf16", lr=1e-3, root_every=1)
    log(f"tensor bf16 {case}")
    s, u, _, sh, _ = run_tensor_parity(wb, 2)
    # bf16 gradients widen exactly; the parameters round once per step, so the
    # update (compared before rounding) keeps the fp32 bar
    assert s <= STATS_TOL and u <= UPDATE_TOL, (s, u)
    sh.close()


def test_tensor_scaled_newton():
    """Scale mode 3 at p = 8 (order 4) and p = 6 (order 3)."""
    for case in ("conv4_64x32", "order3_mixed"):
        w = dataclasses.replace(CASES[case], newton_scale_mode=3)
        log(f"tensor scaled newton {case}")
        s, u, wp, sh, _ = run_tensor_parity(w, 3)
        assert s <= STATS_TOL and u <= UPDATE_TOL and wp <= UPDATE_TOL, (s, u, wp)
        assert sh.n_diverged() == 0
        sh.close()


@pytest.mark.parametrize("case", ["conv4_64x32", "order2"])
def test_tensor_chebyshev(case):
    """Order 4 (p = 8) and order 2 (p = 4: the fourth scratch buffer exists
    for the Chebyshev giant steps only)."""
    w = dataclasses.replace(CASES[case], root_method="chebyshev")
    log(f"tensor chebyshev {case}")
    s, u, wp, sh, _ = run_tensor_parity(w, 3)
    assert s <= STATS_TOL and u <= UPDATE_TOL and wp <= UPDATE_TOL, (s, u, wp)
    sh.close()


@pytest.mark.parametrize("name", sorted(configs.TENSOR_WORKLOADS))
def test_tensor_workloads_sampled(name):
    """The conv workloads at full size, two refreshes, sampled blocks."""
    w = dataclasses.replace(configs.get_tensor(name), root_every=3)
    table = tensor_block_table(w.shapes, w.block_dims)
    rng = np.random.default_rng(9)
    ids = sorted({0, len(table) - 1} | set(rng.choice(len(table), 6, replace=False).tolist()))
    log(f"tensor workload {name} blocks {ids}")
    s, u, wp, sh, _ = run_tensor_parity(w, 4, ids=ids)
    assert s <= STATS_TOL and u <= UPDATE_TOL and wp <= UPDATE_TOL, (s, u, wp)
    assert sh.n_diverged() == 0
    sh.close()


def test_tensor_only_small_dimensions():
    """Every dimension blocked at <= 8: no MFMA factor at all (reductions,
    fp64 Jacobi roots, FMA mode products), ragged tails."""
    w = tw(name="small_only", shapes=((5, 3, 7), (8, 2, 4)), block_dims=(4, 3, 4), root_every=2,
           steps=3)
    s, u, wp, sh, _ = run_tensor_parity(w, 3)
    assert s <= STATS_TOL and u <= UPDATE_TOL and wp <= UPDATE_TOL, (s, u, wp)
    sh.close()


@pytest.mark.parametrize("shapes,block_dims", [
    (((5, 4, 4), (3, 2, 3)), (4, 4, 4)),   # order 3, last two dimensions 4 x 4, ragged
    (((5, 5), (3, 2)), (5, 5)),            # order 2: both dimensions small and equal
    (((40, 2, 2), (70, 1, 2)), (32, 2, 2)),  # a large dimension, then 2 x 2, ragged
])
def test_tensor_fused_small_pair(shapes, block_dims):
    """The two small trailing dimensions of one side: statistics from one pass
    and the last two mode products fused with the update (other sides and
    orders than the conv filters' 3 x 3), with momentum on one step path."""
    w = tw(name="small_pair", shapes=shapes, block_dims=block_dims, root_every=2, steps=3)
    s, u, wp, sh, _ = run_tensor_parity(w, 3)
    assert s <= STATS_TOL and u <= UPDATE_TOL and wp <= UPDATE_TOL, (s, u, wp)
    sh.close()
    w = dataclasses.replace(w, momentum=0.9)
    s, u, wp, sh, _ = run_tensor_parity(w, 3)
    assert s <= STATS_TOL and u <= UPDATE_TOL and wp <= UPDATE_TOL, (s, u, wp)
    sh.close()


def test_tensor_empty_and_zero_tensors():
    """A handle with no tensors steps as a no-op; a zero-extent tensor among
    others is skipped (its pointer may be NULL)."""
    sh = S.TensorShampoo([], (32, 3))
    sh.step([], [])
    sh.close()
    shapes = [(40, 3), (0, 3), (33, 2)]
    sh = S.TensorShampoo(shapes, (32, 3), root_every=1)
    gen = torch.Generator(device="cuda").manual_seed(7)
    params = [torch.zeros(s, device="cuda") for s in shapes]
    grads = [torch.randn(s, generator=gen, device="cuda") for s in shapes]
    S.shampoo_step(sh.handle, [params[0].data_ptr(), 0, params[2].data_ptr()],
                   [grads[0].data_ptr(), 0, grads[2].data_ptr()], 0, sh._stream())
    torch.cuda.synchronize()
    assert torch.isfinite(params[0]).all() and params[0].abs().sum() > 0
    assert torch.isfinite(params[2]).all() and params[2].abs().sum() > 0
    sh.close()


@pytest.mark.parametrize("gemm", ["f32", "split", "split16"])
def test_tensor_fp32_gemm_paths(gemm):
    """Every MFMA product of a tensor handle (statistics of dimensions whose
    unfolding pads to a multiple of 32, roots, mode products) on each product
    path."""
    w = dataclasses.replace(CASES["conv4_64x32"], fp32_gemm=gemm)
    log(f"tensor gemm path {gemm}")
    s, u, wp, sh, _ = run_tensor_parity(w, 3)
    assert s <= STATS_TOL and u <= UPDATE_TOL and wp <= UPDATE_TOL, (s, u, wp)
    assert sh.n_diverged() == 0
    sh.close()


@pytest.mark.parametrize("gemm", ["split", "split16"])
def test_tensor_restore_matches_uninterrupted(gemm):
    """Checkpoint and restore of a tensor handle through its documented state
    (statistics and roots of every dimension, momentum, the Newton records,
    the large dimensions' root maxima on the fp16 split) and shampoo_restore
    into another handle with a history of its own, between two refreshes: the
    following steps, a refresh among them, give bit-identical parameters to an
    uninterrupted run."""
    w = dataclasses.replace(CASES["conv4_64x32"], fp32_gemm=gemm, momentum=0.9, root_every=3)
    gen = torch.Generator(device="cuda").manual_seed(17)
    grads = [[torch.randn(s, generator=gen, device="cuda") * 0.1 for s in w.shapes] for _ in range(7)]
    ref = make(w, root_method="newton")
    p_ref = [torch.zeros(s, device="cuda") for s in w.shapes]
    for t in range(7):
        ref.step(p_ref, grads[t])
    a = make(w, root_method="newton")
    p = [torch.zeros(s, device="cuda") for s in w.shapes]
    for t in range(4):
        a.step(p, grads[t])
    torch.cuda.synchronize()
    saved = [x.clone() for x in a.state_regions()]
    t_saved = a.t
    a.close()
    b = make(w, root_method="newton")
    q = [torch.zeros(s, device="cuda") for s in w.shapes]
    for t in range(2):
        b.step(q, [g * 1e3 for g in grads[6 - t]])
    for dst, src in zip(b.state_regions(), saved):
        dst.copy_(src)
    S.shampoo_restore(b.handle, t_saved, torch.cuda.current_stream().cuda_stream)
    for t in range(4, 7):
        b.step(p, grads[t])
    torch.cuda.synchronize()
    for x, y in zip(p, p_ref):
        assert torch.equal(x, y), float((x - y).abs().max())
    assert b.n_diverged() == 0
    b.close()
    ref.close()
