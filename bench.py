#!/usr/bin/env python3
"""Benchmark of the blocked Shampoo step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

NAME is a matrix workload (default decoder_1b_b1024_f32) or one of the
order-k tensor workloads (resnet32_cifar_convs, resnet32_x8_convs_b128).

A step is the whole optimizer step on one batch of gradients: pack, EMA
statistics, the coupled-Newton roots when the refresh schedule asks (every
root_every steps, so K = 20 after W = 10 holds exactly two refreshes), and the
two-sided apply with the parameter update. Gradients are seeded synthetic
tensors resident in HBM before the timed region (by default one distinct
set per step, as the workload's distribution prescribes). Prints one JSON line with steps/s, blocks/s, per-kernel-class times
and TFLOP/s measured with HIP events on the stream the kernels run on, the
roofline fraction of the dominant kernel (the Newton products) against the
peak of the matrix-core path it runs on, and the fp64 oracle timed on the
host cores on a bounded sample of blocks.

The K timed steps run without instrumentation (steps/s comes from them); K
further steps (as many refreshes) then run with the library's per-launch
events for the per-class times and the roofline. The events cost little on the
large matrix sets but a quarter to a half of the step on the latency-bound
tensor sets, so the instrumented pass reports its own ms per step.

Peaks: fp32 products on the fp32 MFMA take its 157.3 TFLOP/s; fp32 products
split into three bf16 terms run six bf16 MFMA products per fp32 product, so
their ceiling in fp32 FLOP/s is the 2.5 PFLOP/s bf16 peak / 6 = 416.7
TFLOP/s; split into two fp16 terms they run three fp16 MFMA products, a
ceiling of 2.5 PFLOP/s / 3 = 833.3 TFLOP/s; statistics of bf16 gradients take
the bf16 peak itself.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "Shampoo optimizer steps/sec + batched GEMM TFLOP/s vs MFMA peak, 1 GPU"
PEAK_FP32_MFMA_TFLOPS = 157.3   # MI355X dense fp32 matrix peak
PEAK_BF16_MFMA_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak (the statistics of bf16 gradients)
PEAK_SPLIT_TFLOPS = PEAK_BF16_MFMA_TFLOPS / 6.0  # fp32 products as six bf16 products
PEAK_F16_MFMA_TFLOPS = 2500.0   # MI355X dense fp16 matrix peak
PEAK_SPLIT16_TFLOPS = PEAK_F16_MFMA_TFLOPS / 3.0  # fp32 products as three fp16 products
PEAK_HBM_GBS = 8000.0           # MI355X HBM3E
PATH_PEAKS = {"f32": PEAK_FP32_MFMA_TFLOPS, "bf16": PEAK_BF16_MFMA_TFLOPS,
              "split": PEAK_SPLIT_TFLOPS, "split16": PEAK_SPLIT16_TFLOPS}
GEMM_HOW = {"split16": "fp32 operands scaled and split into two fp16 terms, three fp16 MFMA "
                       "32x32x16 products",
            "split": "fp32 operands split into three bf16 terms, six bf16 MFMA 32x32x16 products",
            "f32": "fp32 MFMA 32x32x2"}
DEFAULT_WORKLOAD = "decoder_1b_b1024_f32"
# the arithmetic the fp32 products execute, for the JSON line's dtype
DTYPE_OF_PATH = {"split16": "f32 storage; products as fp16x2 split (3 fp16 MFMA, fp32 accumulate)",
                 "split": "f32 storage; products as bf16x3 split (6 bf16 MFMA, fp32 accumulate)",
                 "f32": "f32 (fp32 MFMA)"}


def dtype_label(w):
    d = DTYPE_OF_PATH[w.fp32_gemm]
    if w.dtype == "bf16":
        d += "; bf16 gradients and parameters, their statistics on the bf16 MFMA"
    return d


def newton_kernel_desc(w):
    """The Newton product kernel and tile the library's plan picks for the
    workload: factors of side <= 64 iterate in one launch; otherwise the
    symmetric products take 256x256 tiles on the fp16 split when both block
    sides are multiples of 256 and at least 512, else the largest of 128, 64,
    32 that divides both sides."""
    br, bc = w.block_rows, w.block_cols
    if max(br, bc) <= 64:
        return "newton_small_kernel (one workgroup per factor, every iteration in one launch)"
    if w.fp32_gemm == "split16" and br % 256 == 0 and bc % 256 == 0 and min(br, bc) >= 512:
        tile = 256
    else:
        g = math.gcd(br, bc)
        tile = 128 if g % 128 == 0 else 64 if g % 64 == 0 else 32
    return f"newton_sym_kernel ({tile}x{tile} tiles, symmetric outputs)"


def cpu_model():
    """The host CPU's model name, from /proc/cpuinfo."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def cpu_baseline(w, grad_sets, budget_s=15.0, max_blocks=32, seed=0, one_thread=False):
    """Time the oracle (as it stands) on a sample of blocks: one refresh step
    and one non-refresh step per block, extrapolated linearly to all blocks
    over one root cycle (blocks are independent). With one_thread, the same
    timing again with the BLAS limited to one thread, reported beside it."""
    import numpy as np

    single = None
    if one_thread:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            single = cpu_baseline(w, grad_sets, budget_s / 2, max_blocks, seed)

    from oracle import ShampooOracle, block_table
    try:
        from threadpoolctl import threadpool_info
        cores = max([int(p.get("num_threads", 1)) for p in threadpool_info()] or [1])
    except Exception:
        cores = len(os.sched_getaffinity(0))
    table = block_table(w.shapes, w.block_rows, w.block_cols)
    rng = np.random.default_rng(seed)
    by_shape = {}
    for b in table:
        by_shape.setdefault(w.shapes[b.mat], []).append(b.id)
    order = [int(rng.choice(v)) for v in by_shape.values()]
    rest = [int(i) for i in rng.permutation(len(table)) if int(i) not in order]
    order += rest
    g1, g2 = grad_sets[0], grad_sets[1 % len(grad_sets)]
    t_ref = t_non = 0.0
    used = 0
    start = time.perf_counter()
    for i in order[:max_blocks]:
        b = table[i]
        blk = lambda g: g[b.mat][b.r0:b.r0 + b.m, b.c0:b.c0 + b.n].float().cpu().numpy()
        G1, G2 = blk(g1), blk(g2)
        o = ShampooOracle(w.shapes, w.block_rows, w.block_cols, w.beta2, w.eps, w.lr,
                          w.root_every, blocks=[i], momentum=w.momentum)
        a = time.perf_counter()
        o.step_blocks({i: G1})          # t = 1: refresh step
        bt = time.perf_counter()
        o.step_blocks({i: G2})          # t = 2: stale roots
        c = time.perf_counter()
        t_ref += bt - a
        t_non += c - bt
        used += 1
        if time.perf_counter() - start > budget_s and used >= 4:
            break
    k = max(1, w.root_every)
    per_block_cycle = (t_ref + (k - 1) * t_non) / used
    steps_per_s = k / (per_block_cycle * len(table))
    return {
        "value": steps_per_s, "unit": "steps/s", "cores": cores, "kind": "oracle",
        "sample": (f"fp64 oracle (numpy/LAPACK, eigh roots) on {used} of {len(table)} blocks "
                   f"(every matrix shape): one refresh step ({t_ref / used * 1e3:.1f} ms/block) and "
                   f"one non-refresh step ({t_non / used * 1e3:.1f} ms/block), extrapolated "
                   f"linearly to all blocks over a {k}-step root cycle"),
        "blocks_per_s": steps_per_s * len(table),
        "cpu_seconds": t_ref + t_non,
        "cpu_model": cpu_model(),
        "one_thread": None if single is None else {
            k: single[k] for k in ("value", "blocks_per_s", "cores", "sample")},
    }


def cpu_baseline_tensor(w, grad_sets, budget_s=15.0, max_blocks=16, seed=0):
    """The tensor oracle (as it stands) on a sample of blocks, timed and
    extrapolated like cpu_baseline."""
    import numpy as np

    from oracle.tensor_oracle import TensorShampooOracle, tensor_block_table
    try:
        from threadpoolctl import threadpool_info
        cores = max([int(p.get("num_threads", 1)) for p in threadpool_info()] or [1])
    except Exception:
        cores = len(os.sched_getaffinity(0))
    table = tensor_block_table(w.shapes, w.block_dims)
    rng = np.random.default_rng(seed)
    order = [int(i) for i in rng.permutation(len(table))]
    g1, g2 = grad_sets[0], grad_sets[1 % len(grad_sets)]
    t_ref = t_non = 0.0
    used = 0
    start = time.perf_counter()
    for i in order[:max_blocks]:
        b = table[i]
        G1 = g1[b.tensor][b.slices()].float().cpu().numpy()
        G2 = g2[b.tensor][b.slices()].float().cpu().numpy()
        o = TensorShampooOracle(w.shapes, w.block_dims, w.beta2, w.eps, w.lr, w.root_every,
                                blocks=[i], momentum=w.momentum)
        a = time.perf_counter()
        o.step_blocks({i: G1})
        bt = time.perf_counter()
        o.step_blocks({i: G2})
        c = time.perf_counter()
        t_ref += bt - a
        t_non += c - bt
        used += 1
        if time.perf_counter() - start > budget_s and used >= 4:
            break
    k = max(1, w.root_every)
    per_block_cycle = (t_ref + (k - 1) * t_non) / used
    steps_per_s = k / (per_block_cycle * len(table))
    return {
        "value": steps_per_s, "unit": "steps/s", "cores": cores, "kind": "oracle",
        "sample": (f"fp64 tensor oracle (numpy/LAPACK, eigh roots) on {used} of {len(table)} "
                   f"blocks: one refresh step ({t_ref / used * 1e3:.1f} ms/block) and one "
                   f"non-refresh step ({t_non / used * 1e3:.1f} ms/block), extrapolated "
                   f"linearly to all blocks over a {k}-step root cycle"),
        "blocks_per_s": steps_per_s * len(table),
        "cpu_seconds": t_ref + t_non,
        "cpu_model": cpu_model(),
    }


def class_table(tm, paths):
    """Per timing class: time, launches, TFLOP/s and the fraction of the
    peak of its matrix-core path (paths: class -> "f32" | "bf16" | "split" | "split16")."""
    kernels = {}
    for name, d in tm.items():
        entry = {"ms": round(d["ms"], 3), "launches": d["launches"]}
        if d["flops"] > 0 and d["ms"] > 0:
            tf = d["flops"] / (d["ms"] * 1e-3) / 1e12
            entry["tflops"] = round(tf, 2)
            path = paths.get(name, "f32")
            entry["mfma_path"] = path
            entry["frac_mfma"] = round(tf / PATH_PEAKS[path], 4)
        if d["bytes"] > 0 and d["ms"] > 0:
            gbs = d["bytes"] / (d["ms"] * 1e-3) / 1e9
            entry["gbs"] = round(gbs, 1)
            entry["frac_hbm"] = round(gbs / PEAK_HBM_GBS, 4)
        kernels[name] = entry
    return kernels


def timed_steps(torch, sh, params, grad_sets, t0, steps, stream):
    """Runs `steps` optimizer steps (gradient sets t0, t0 + 1, ... in turn) between two HIP
    events on the library's stream; returns (event seconds, wall seconds)."""
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    e0.record(stream)
    for t in range(steps):
        sh.step(params, grad_sets[(t0 + t) % len(grad_sets)])
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / 1e3, time.perf_counter() - wall0


def run_tensor(args, w, torch, S, synth):
    """Order-k tensor workloads: the same step, timing and JSON line."""
    import dataclasses
    if args.momentum is not None:
        w = dataclasses.replace(w, momentum=args.momentum)
    if args.root_method is not None:
        w = dataclasses.replace(w, root_method=args.root_method)
    if args.scale_mode is not None:
        w = dataclasses.replace(w, newton_scale_mode=args.scale_mode)
    if args.fp32_gemm is not None:
        w = dataclasses.replace(w, fp32_gemm=args.fp32_gemm)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"tensor workload {w.name}: {len(w.shapes)} tensors, blocks {w.block_dims}")
    src = synth.TensorGradientSource(w, device=dev)
    params = src.init_params()
    total = args.steps + args.warmup
    n_sets = total if args.grad_sets <= 0 else max(1, min(args.grad_sets, total))
    grad_sets = []
    for t in range(1, n_sets + 1):
        grad_sets.append(src.grads(t))
        if t % 10 == 0 or t == n_sets:
            torch.cuda.synchronize()
            log(f"gradient sets generated: {t}/{n_sets}")
    sh = S.TensorShampoo(w.shapes, w.block_dims, beta2=w.beta2, eps=w.eps, lr=w.lr,
                         root_every=w.root_every, newton_max_iters=w.newton_max_iters,
                         newton_tol=w.newton_tol, newton_scale_mode=w.newton_scale_mode,
                         dtype=w.dtype, momentum=w.momentum, root_method=w.root_method,
                         cheb_degree=w.cheb_degree, fp32_gemm=w.fp32_gemm)
    B = sh.n_blocks
    log(f"{B} blocks of {int(sh.info.block_elems)} elements, workspace "
        f"{sh.workspace.numel() / 2**30:.2f} GiB")
    for t in range(args.warmup):
        sh.step(params, grad_sets[t % n_sets])
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    elapsed, _ = timed_steps(torch, sh, params, grad_sets, args.warmup, args.steps, stream)
    sh.set_timing(True)
    elapsed_i, _ = timed_steps(torch, sh, params, grad_sets, args.warmup + args.steps,
                               args.steps, stream)
    tm = sh.timing()
    sh.set_timing(False)
    n_div = sh.n_diverged()
    # statistics (of dimensions whose unfolding pads to a multiple of 32),
    # MFMA mode products and roots all take the configured path
    paths = {"stats": w.fp32_gemm, "apply": w.fp32_gemm, "newton_gemm": w.fp32_gemm}
    kernels = class_table(tm, paths)
    # dominant class by kernel time; its roofline against its matrix-core
    # path (statistics, root products, apply products) or HBM (the others)
    dom = max(tm, key=lambda k: tm[k]["ms"])
    d = tm[dom]
    if dom not in ("stats", "newton_gemm", "apply"):
        ach = d["bytes"] / (d["ms"] * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(ach / PEAK_HBM_GBS, 4)}
    else:
        ach = d["flops"] / (d["ms"] * 1e-3) / 1e12 if d["ms"] > 0 else 0.0
        peak = PATH_PEAKS[paths[dom]]
        roof = {"bound": "mfma", "achieved": round(ach, 2), "peak": round(peak, 1),
                "unit": "TFLOP/s", "frac": round(ach / peak, 4)}
    roof.update({"traffic": None, "kernel": f"class {dom}", "launches": d["launches"],
                 "avg_launch_ms": d["ms"] / max(1, d["launches"])})
    cpu = None if args.no_cpu_baseline else cpu_baseline_tensor(w, grad_sets)
    steps_per_s = args.steps / elapsed
    out = {
        "metric": METRIC, "value": round(steps_per_s, 4), "unit": "steps/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(elapsed / args.steps * 1e3, 3),
        "ms_per_step_instrumented": round(elapsed_i / args.steps * 1e3, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": dtype_label(w),
        "data": "synthetic (seeded gradients with conv-filter shapes)",
        "config": {"workload": w.name, "tensors": len(w.shapes), "blocks": B,
                   "block": list(w.block_dims), "root_every": w.root_every,
                   "root_method": w.root_method, "momentum": w.momentum,
                   "fp32_gemm": w.fp32_gemm, "grad_sets": n_sets},
        "blocks_per_s": round(steps_per_s * B, 1),
        "kernels": kernels, "n_diverged": n_div, "roofline": roof, "cpu_baseline": cpu,
    }
    sh.close()
    print(json.dumps(out), flush=True)


def measure_matrix(args, w, torch, S, params, grad_sets):
    """Warmup, the timed pass and the instrumented pass of one matrix
    workload on a fresh handle; returns what the JSON line reports."""
    n_sets = len(grad_sets)
    sh = S.Shampoo(w.shapes, w.block_rows, w.block_cols, beta2=w.beta2, eps=w.eps, lr=w.lr,
                   root_every=w.root_every, newton_max_iters=w.newton_max_iters,
                   newton_tol=w.newton_tol, newton_scale_mode=w.newton_scale_mode, dtype=w.dtype,
                   momentum=w.momentum, root_method=w.root_method, cheb_degree=w.cheb_degree,
                   fp32_gemm=w.fp32_gemm)
    B = sh.n_blocks
    log(f"{B} blocks, workspace {sh.workspace.numel() / 2**30:.1f} GiB, products {w.fp32_gemm}")
    for t in range(args.warmup):
        sh.step(params, grad_sets[t % n_sets])
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} steps done")

    stream = torch.cuda.current_stream()
    # the measured pass: no per-launch events
    elapsed, wall = timed_steps(torch, sh, params, grad_sets, args.warmup, args.steps, stream)
    # the instrumented pass over as many further steps (as many refreshes):
    # per-class times, the Newton statistics and the roofline
    sh.set_timing(True)
    elapsed_i, _ = timed_steps(torch, sh, params, grad_sets, args.warmup + args.steps,
                               args.steps, stream)
    tm = sh.timing()
    sh.set_timing(False)
    n_div = sh.n_diverged()
    st, it, _ = sh.newton_info()
    iters = it.cpu().tolist()
    status = st.cpu().tolist()
    resid = sh.newton_residual().cpu()
    B_ = len(iters) // 2
    newton_stats = {
        "status_counts": {name: status.count(code) for code, name in
                          ((1, "converged"), (2, "stalled"), (3, "diverged"), (4, "capped"))},
        "iters_left_mean": sum(iters[:B_]) / max(1, B_),
        "iters_right_mean": sum(iters[B_:]) / max(1, B_),
        "iters_min": min(iters) if iters else 0, "iters_max": max(iters) if iters else 0,
        "residual_median": float(resid.median()) if len(resid) else 0.0,
        "residual_max": float(resid.max()) if len(resid) else 0.0,
        "n_diverged": n_div,
    }
    log(f"timed {args.steps} steps: {elapsed * 1e3:.1f} ms (wall {wall * 1e3:.1f} ms); "
        f"instrumented: {elapsed_i * 1e3:.1f} ms")
    sh.close()
    del sh
    torch.cuda.empty_cache()
    # statistics of bf16 gradients take the bf16 MFMA; the other products
    # the configured fp32 path
    paths = {"stats": "bf16" if w.dtype == "bf16" else w.fp32_gemm,
             "newton_gemm": w.fp32_gemm, "apply": w.fp32_gemm}
    return {"B": B, "elapsed": elapsed, "elapsed_i": elapsed_i, "tm": tm, "newton": newton_stats,
            "kernels": class_table(tm, paths)}


def newton_traffic(workload, gemm):
    """HBM bytes per Newton-product launch from the committed rocprofv3
    counter summary of this workload and product path, if it was taken on the
    current kernel source (its SHA-256 is recorded with the counters); None
    otherwise."""
    import hashlib
    tag = "" if gemm == "split16" else "_" + gemm
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}{tag}.json")
    src = os.path.join(ROOT, "blocked_shampoo_preconditioning_amd", "csrc", "kernels.hip")
    try:
        rec = json.load(open(path))
        sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256") != sha:
        return None
    return round(rec["kernels"]["newton_sym_kernel"]["traffic_bytes_per_launch"])


def vendor_gemm(torch, w, reps=10):
    """Rate of torch.bmm (the vendor GEMM library) on [B, n, n] x [B, n, n], B the workload's
    block count and n its block side: a full product with none of the fused work (no
    symmetry, no split, no epilogue), timed like the step. Context for the hand-written
    products, not part of the step."""
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    n = w.block_rows
    B = sum(((r + n - 1) // n) * ((c + w.block_cols - 1) // w.block_cols) for r, c in w.shapes)
    out = {"vendor_gemm": "torch.bmm", "shape": [B, n, n, n]}
    for name, dt in (("fp16", torch.float16), ("bf16", torch.bfloat16), ("fp32", torch.float32)):
        g = torch.Generator(device=dev).manual_seed(0)
        a = torch.randn(B, n, n, device=dev, dtype=dt, generator=g)
        b = torch.randn(B, n, n, device=dev, dtype=dt, generator=g)
        c = torch.empty(B, n, n, device=dev, dtype=dt)
        for _ in range(3):
            torch.bmm(a, b, out=c)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            torch.bmm(a, b, out=c)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        out[name] = {"ms": round(ms, 3), "tflops": round(2.0 * B * n ** 3 / (ms * 1e-3) / 1e12, 1)}
        log(f"vendor {name}: {out[name]}")
        del a, b, c
        torch.cuda.empty_cache()
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--grad-sets", type=int, default=0,
                    help="distinct gradient sets held in HBM, used in turn (0: one per step)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--momentum", type=float, default=None,
                    help="momentum folded in before preconditioning (default: the workload's, 0)")
    ap.add_argument("--root-method", default=None, choices=("newton", "newton_db", "chebyshev"),
                    help="inverse-root solver (default: the workload's, coupled Newton)")
    ap.add_argument("--scale-mode", type=int, default=None, choices=(0, 1, 2, 3),
                    help="Newton scale mode (default: the workload's)")
    ap.add_argument("--cheb-degree", type=int, default=None,
                    help="Chebyshev degree (default: the workload's, 128)")
    ap.add_argument("--fp32-gemm", default=None, choices=("split16", "split", "f32"),
                    help="fp32 products: scaled and split into two fp16 terms on the fp16 MFMA "
                         "(default), split into three bf16 terms on the bf16 MFMA, or the "
                         "fp32 MFMA")
    ap.add_argument("--vendor-gemm", action="store_true",
                    help="instead of the step, time the vendor library's batched GEMM "
                         "(torch.bmm on hipBLASLt) at the workload's block shape in fp16, bf16 "
                         "and fp32: the practical ceiling of a plain product on this chip")
    ap.add_argument("--no-f32-pass", action="store_true",
                    help="skip the second timed pass with every fp32 product on the fp32 MFMA")
    ap.add_argument("--copy-probe", action="store_true",
                    help="end with one plain 1 GiB device copy (a known-size kernel that "
                         "calibrates the HBM traffic counters)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the blocked step shards by blocks with no communication but the parameter "
              "all-gather, which this build does not run.", file=sys.stderr)
        sys.exit(2)

    import torch

    from blocked_shampoo_preconditioning_amd import configs, synth
    from blocked_shampoo_preconditioning_amd import shampoo as S

    if not os.path.exists(S.LIB_PATH):
        from blocked_shampoo_preconditioning_amd import build
        build.build()
    S.load_library()
    if args.vendor_gemm:
        return vendor_gemm(torch, configs.get(args.workload))
    if args.workload in configs.TENSOR_WORKLOADS:
        return run_tensor(args, configs.get_tensor(args.workload), torch, S, synth)
    w = configs.get(args.workload)
    import dataclasses
    if args.momentum is not None:
        w = dataclasses.replace(w, momentum=args.momentum)
    if args.root_method is not None:
        w = dataclasses.replace(w, root_method=args.root_method)
    if args.cheb_degree is not None:
        w = dataclasses.replace(w, cheb_degree=args.cheb_degree)
    if args.scale_mode is not None:
        w = dataclasses.replace(w, newton_scale_mode=args.scale_mode)
    if args.fp32_gemm is not None:
        w = dataclasses.replace(w, fp32_gemm=args.fp32_gemm)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"workload {w.name}: {len(w.shapes)} matrices, blocks {w.block_rows}x{w.block_cols}")
    src = synth.GradientSource(w, device=dev)
    params = src.init_params()
    total = args.steps + args.warmup
    n_sets = total if args.grad_sets <= 0 else max(1, min(args.grad_sets, total))
    grad_sets = []
    for t in range(1, n_sets + 1):
        grad_sets.append(src.grads(t))
        if t % 10 == 0 or t == n_sets:
            torch.cuda.synchronize()
            log(f"gradient sets generated: {t}/{n_sets}")
    r = measure_matrix(args, w, torch, S, params, grad_sets)
    B, elapsed, elapsed_i, tm, kernels = r["B"], r["elapsed"], r["elapsed_i"], r["tm"], r["kernels"]
    steps_per_s = args.steps / elapsed
    nw = tm["newton_gemm"]
    achieved = nw["flops"] / (nw["ms"] * 1e-3) / 1e12 if nw["ms"] > 0 else 0.0
    traffic = newton_traffic(w.name, w.fp32_gemm)
    peak = PATH_PEAKS[w.fp32_gemm]
    how = GEMM_HOW[w.fp32_gemm]
    roofline = {
        "bound": "mfma", "achieved": round(achieved, 2), "peak": round(peak, 1),
        "unit": "TFLOP/s", "frac": round(achieved / peak, 4), "traffic": traffic,
        "kernel": f"{newton_kernel_desc(w)} ({how}; {w.root_method} root products)",
        "launches": nw["launches"],
        "flops_per_launch": nw["flops"] / max(1, nw["launches"]),
        "avg_launch_ms": nw["ms"] / max(1, nw["launches"]),
        # the same fp32 flops over the fp32 MFMA's peak: not a roofline fraction
        # (the split products do not run on the fp32 MFMA), a comparison of rates
        "fp32_equiv_vs_fp32_mfma_peak": round(achieved / PEAK_FP32_MFMA_TFLOPS, 4),
    }
    # the same workload with every fp32 product on the fp32 MFMA, timed the
    # same way in the same run (its roofline is the fp32 MFMA's own peak)
    f32_pass = None
    if w.fp32_gemm != "f32" and not args.no_f32_pass:
        wf = dataclasses.replace(w, fp32_gemm="f32")
        rf = measure_matrix(args, wf, torch, S, params, grad_sets)
        kf = rf["kernels"]
        f32_pass = {
            "value": round(args.steps / rf["elapsed"], 4), "unit": "steps/s",
            "ms_per_step": round(rf["elapsed"] / args.steps * 1e3, 3),
            "dtype": dtype_label(wf),
            "gemm": {k: {"tflops": kf[k].get("tflops"), "frac_mfma": kf[k].get("frac_mfma"),
                         "mfma_path": kf[k].get("mfma_path")}
                     for k in ("stats", "newton_gemm", "apply") if k in kf},
            "newton": {k: rf["newton"][k] for k in ("iters_left_mean", "iters_right_mean",
                                                    "n_diverged")},
        }
    cpu = None
    if not args.no_cpu_baseline:
        log("timing the oracle on the host")
        cpu = cpu_baseline(w, grad_sets, one_thread=w.name in ("single_64x32", "gpt_small_b256"))
    out = {
        "metric": METRIC, "value": round(steps_per_s, 4), "unit": "steps/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(elapsed / args.steps * 1e3, 3),
        "ms_per_step_instrumented": round(elapsed_i / args.steps * 1e3, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": dtype_label(w),
        "data": "synthetic (seeded gradients with transformer-layer shapes)",
        "config": {"workload": w.name, "matrices": len(w.shapes), "blocks": B,
                   "block": [w.block_rows, w.block_cols], "root_every": w.root_every,
                   "newton_max_iters": w.newton_max_iters, "newton_tol": w.newton_tol,
                   "newton_scale_mode": w.newton_scale_mode, "momentum": w.momentum,
                   "root_method": w.root_method, "fp32_gemm": w.fp32_gemm,
                   "cheb_degree": w.cheb_degree if w.root_method == "chebyshev" else None,
                   "grad_sets": n_sets},
        "blocks_per_s": round(steps_per_s * B, 1),
        "gemm_tflops": {k: kernels[k].get("tflops") for k in ("stats", "newton_gemm", "apply")},
        "kernels": kernels,
        "newton": r["newton"],
        "roofline": roofline,
        "fp32_mfma_pass": f32_pass,
        "cpu_baseline": cpu,
    }
    if args.copy_probe:
        n = 1 << 28  # 1 GiB of fp32
        src_t = torch.ones(n, dtype=torch.float32, device=dev)
        dst_t = torch.empty_like(src_t)
        torch.cuda.synchronize()
        dst_t.copy_(src_t)
        torch.cuda.synchronize()
        out["copy_probe_bytes"] = 4 * n
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
