"""The synthetic workloads the step is tested and measured on (five, plus one
GPU's eighth share of the 1B-class set).

Each workload is a set of weight matrices with transformer-layer shapes, a
block shape, the optimizer's hyper-parameters and the distribution of the
synthetic gradients. The pages measure on CIFAR ResNets, LM1B and 360M-660M
language models (podcast "Preconditioned Optimization Without the Full Matrix
Cost", cue 36; SOAP record); the optimizer step only ever sees gradient
tensors, so seeded synthetic gradients with the shapes of a GPT-small layer
set and of a 1B-class decoder layer set stand in for those models.

Where a workload leaves a hyper-parameter open, beta2 = 0.999, eps = 1e-6 and
lr = 1e-3 (the values given for the single-matrix case) are used. "N(0, x)"
means standard deviation x.
"""
from __future__ import annotations

from dataclasses import dataclass, field

GPT_SMALL_LAYER = ((768, 2304), (768, 768), (768, 3072), (3072, 768))
DECODER_1B_LAYER = ((2048, 6144), (2048, 2048), (2048, 8192), (8192, 2048))


@dataclass(frozen=True)
class Workload:
    name: str
    shapes: tuple                 # (rows, cols) per matrix, registration order
    block_rows: int
    block_cols: int
    beta2: float = 0.999
    eps: float = 1e-6
    lr: float = 1e-3
    root_every: int = 10
    steps: int = 10
    dtype: str = "f32"            # gradient and parameter storage: f32 | bf16
    grad: str = "iid"             # iid | row_scaled | col_scaled | low_rank
    grad_std: float = 1.0
    noise_std: float = 0.0        # low_rank: additive noise
    rank: int = 0                 # low_rank: rank of the factor product
    diag_fraction: float = 0.0    # fraction of blocks whose gradient is diagonal
    newton_max_iters: int = 25
    newton_tol: float = 1e-6      # <= 0: exactly newton_max_iters iterations
    newton_scale_mode: int = 3    # 3: the iteration scales itself (fewer iterations)
    momentum: float = 0.0         # ordinary momentum folded in before preconditioning
    root_method: str = "newton"   # newton (coupled) | newton_db (Denman-Beavers) | chebyshev
    cheb_degree: int = 128        # degree of the Chebyshev interpolant (chebyshev only)
    fp32_gemm: str = "split16"    # fp32 products: split16 (two scaled fp16 terms) | split (three bf16 terms) | f32 (fp32 MFMA)
    init_std: float = 0.02
    seed: int = 0
    notes: str = field(default="", compare=False)


def _layers(layer, n):
    return tuple(s for _ in range(n) for s in layer)


WORKLOADS = {
    "single_64x32": Workload(
        name="single_64x32", shapes=((64, 32),), block_rows=64, block_cols=32,
        root_every=1, steps=10, grad="iid", grad_std=1.0, seed=1001,
        notes="one 64x32 matrix, one block, roots every step"),
    "gpt_small_b256": Workload(
        name="gpt_small_b256", shapes=_layers(GPT_SMALL_LAYER, 12), block_rows=256,
        block_cols=256, root_every=10, steps=100, grad="row_scaled", grad_std=1e-2,
        seed=1002, notes="12 GPT-small layers, 1296 blocks of 256x256, no tails"),
    "gpt_small_b512_lowrank": Workload(
        name="gpt_small_b512_lowrank", shapes=_layers(GPT_SMALL_LAYER, 12), block_rows=512,
        block_cols=512, eps=1e-12, root_every=10, steps=100, grad="low_rank", rank=16,
        grad_std=0.05, noise_std=1e-3, seed=1003,
        notes="12 GPT-small layers, 456 blocks of 512x512 (252 tails), ill-conditioned"),
    "decoder_1b_b1024_f32": Workload(
        name="decoder_1b_b1024_f32", shapes=_layers(DECODER_1B_LAYER, 24), block_rows=1024,
        block_cols=1024, root_every=10, steps=50, grad="col_scaled", grad_std=1e-2,
        seed=1004, notes="24 1B-class decoder layers, 1152 blocks of 1024x1024, fp32"),
    "decoder_1b_b1024_f32_shard8": Workload(
        name="decoder_1b_b1024_f32_shard8", shapes=_layers(DECODER_1B_LAYER, 3), block_rows=1024,
        block_cols=1024, root_every=10, steps=50, grad="col_scaled", grad_std=1e-2,
        seed=1004, notes="one GPU's share of the 1B-class set split 8 ways by blocks: 3 of its "
                         "24 layers, 144 blocks of 1024x1024, fp32"),
    "decoder_1b_b1024_bf16": Workload(
        name="decoder_1b_b1024_bf16", shapes=_layers(DECODER_1B_LAYER, 24), block_rows=1024,
        block_cols=1024, root_every=10, steps=50, dtype="bf16", grad="col_scaled",
        grad_std=1e-2, diag_fraction=0.1, newton_max_iters=10, newton_tol=0.0,
        newton_scale_mode=2, seed=1005,
        notes="as decoder_1b_b1024_f32 with bf16 gradients and parameters, 10 fixed "
              "(unscaled) Newton iterations, 10% diagonal blocks"),
}

# ---------------------------------------------------------------------------
# Order-k tensors (podcast cue 26): conv filters [out, in, kh, kw]. The
# podcast's image test bed is CIFAR-10 on a 32-layer ResNet (cue 36); its
# convolution filters are 3 x 3 with 16, 32 and 64 channels in three stages
# of five residual blocks (two convolutions each) after a 3 -> 16 stem.
# ---------------------------------------------------------------------------
def resnet_cifar_convs(n_blocks_per_stage=5, width=1):
    """Conv filter shapes of a CIFAR ResNet (6n + 2 layers) at width x."""
    c = [16 * width, 32 * width, 64 * width]
    shapes = [(c[0], 3, 3, 3)]
    cin = c[0]
    for cout in c:
        for _ in range(n_blocks_per_stage):
            shapes.append((cout, cin, 3, 3))
            shapes.append((cout, cout, 3, 3))
            cin = cout
    return tuple(shapes)


@dataclass(frozen=True)
class TensorWorkload:
    name: str
    shapes: tuple                 # per tensor, all of one order k
    block_dims: tuple             # block size of every dimension
    beta2: float = 0.999
    eps: float = 1e-6
    lr: float = 1e-3
    root_every: int = 10
    steps: int = 10
    dtype: str = "f32"
    grad: str = "iid"             # iid | row_scaled (one scale per index of dimension 0)
    grad_std: float = 1.0
    newton_max_iters: int = 25
    newton_tol: float = 1e-6
    newton_scale_mode: int = 3
    momentum: float = 0.0
    root_method: str = "newton"
    cheb_degree: int = 128
    fp32_gemm: str = "split16"
    init_std: float = 0.02
    seed: int = 0
    notes: str = field(default="", compare=False)


TENSOR_WORKLOADS = {
    "resnet32_cifar_convs": TensorWorkload(
        name="resnet32_cifar_convs", shapes=resnet_cifar_convs(5, 1), block_dims=(64, 64, 3, 3),
        root_every=10, steps=20, grad="row_scaled", grad_std=1e-2, seed=2001,
        notes="the 31 conv filters of ResNet-32 for CIFAR-10, one block each (channels "
              "zero-padded to 64)"),
    "resnet32_x8_convs_b128": TensorWorkload(
        name="resnet32_x8_convs_b128", shapes=resnet_cifar_convs(5, 8),
        block_dims=(128, 128, 3, 3), root_every=10, steps=20, grad="row_scaled", grad_std=1e-2,
        seed=2002,
        notes="ResNet-32's conv filters at 8x channel width (128 / 256 / 512), blocks of "
              "128 x 128 x 3 x 3: 201 blocks"),
}


def get_tensor(name) -> TensorWorkload:
    return TENSOR_WORKLOADS[name]


# Short aliases in the order the workloads are listed.
ORDER = ("single_64x32", "gpt_small_b256", "gpt_small_b512_lowrank",
         "decoder_1b_b1024_f32", "decoder_1b_b1024_bf16")


def get(name) -> Workload:
    return WORKLOADS[name]


def n_blocks(w: Workload) -> int:
    return sum(-(-r // w.block_rows) * -(-c // w.block_cols) for r, c in w.shapes)
