"""GPU parity over the workloads' full step counts (100 steps for the GPT-small
sets, 50 for the 1B-class sets), on seeded samples of blocks: several root
refreshes, stale roots in between, EMA decay of the eps start. Compared at the
first ten steps and every fifth step after."""
import numpy as np
import pytest

from oracle import block_table
from tests.gpu_common import (STATS_TOL, UPDATE_TOL, block_of, cond_of, log, rel, run_parity,
                              sample_blocks, workload)
from blocked_shampoo_preconditioning_amd import synth

pytestmark = pytest.mark.gpu


def every(t):
    return t <= 10 or t % 5 == 0


def _check(w, recs, gate_from=1):
    for r in recs:
        assert r.stats_err <= STATS_TOL, r
        if r.t >= gate_from:
            assert r.update_err <= UPDATE_TOL, r


def test_gpt_small_b256_100_steps():
    w = workload("gpt_small_b256")
    recs, sh, orc, params, W = run_parity(w, w.steps, ids=sample_blocks(w, 8, seed=21),
                                          compare=every)
    _check(w, recs)
    sh.close()


def test_gpt_small_b512_lowrank_100_steps():
    """Updates gated once the statistics are representable in fp32 (from the
    refresh at t = 11 on; cond(L) is ~1e9 before it)."""
    w = workload("gpt_small_b512_lowrank")
    ids = sample_blocks(w, 6, seed=22)
    recs, sh, orc, params, W = run_parity(w, w.steps, ids=ids, compare=every)
    _check(w, recs, gate_from=11)
    log(f"  max cond(L) at t={w.steps}: {max(cond_of(orc.state[i].L) for i in ids):.2e}")
    sh.close()


def test_decoder_1b_f32_50_steps():
    w = workload("decoder_1b_b1024_f32")
    recs, sh, orc, params, W = run_parity(w, w.steps, ids=sample_blocks(w, 3, seed=23),
                                          compare=every)
    _check(w, recs)
    # cumulative parameter change after 50 steps
    table = block_table(w.shapes, w.block_rows, w.block_cols)
    W0 = synth.GradientSource(w, device="cuda").init_params()
    for i in W:
        b = table[i]
        d_gpu = block_of(params[b.mat], b) - block_of(W0[b.mat], b)
        assert rel(d_gpu, W[i] - block_of(W0[b.mat], b)) <= UPDATE_TOL
    sh.close()


def test_decoder_1b_bf16_50_steps():
    w = workload("decoder_1b_b1024_bf16")
    table = block_table(w.shapes, w.block_rows, w.block_cols)
    diag = synth.diagonal_blocks(w)
    diag_ids = sorted(b.id for b in table if (b.mat, b.bi, b.bj) in diag)
    ids = sorted(set(sample_blocks(w, 2, seed=24)) | set(diag_ids[:2]))
    recs, sh, orc, params, W = run_parity(w, w.steps, ids=ids, root_method="newton",
                                          compare=every)
    _check(w, recs)
    sh.close()
