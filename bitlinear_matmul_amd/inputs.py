"""Seeded synthetic inputs for every workload.

This module holds no step of the method: it only draws the fp32 tensors the
method is applied to (activations and fp32 master weights), with the shapes
and value distributions of the workloads, from ``numpy.random.default_rng``.
Both the HIP path's tests/benchmark and the CPU oracle take their inputs from
here; neither side's arithmetic lives here.

Shapes are given as the weight is stored: ``W[N][K]`` (out x in, K
contiguous), so ``y = x W^T`` maps ``x [M, K]`` to ``y [M, N]``.

Distributions follow the pages' workloads: fp32 masters ~ N(0, 0.02^2)
(absmean then gives ~31% zeros, the fraction the "a 1-bit llm, from scratch"
page reports for its trained model), activations ~ N(0, 1); the prefill
activations additionally carry 1% outlier channels scaled by 20.
"""
from dataclasses import dataclass

import numpy as np

SIGMA_W = np.float32(0.02)
EPS = 1e-5


def normal(rng, shape, sigma=None):
    """fp32 normals; multiplied by sigma in fp32 when given."""
    a = rng.standard_normal(shape, dtype=np.float32)
    if sigma is not None:
        a *= np.float32(sigma)
    return a


# ---------------------------------------------------------------------------
# Tiny single BitLinear: x [32,128], W [N=512, K=128], seed 0.
# ---------------------------------------------------------------------------
def tiny_layer():
    rng = np.random.default_rng(0)
    x = normal(rng, (32, 128))
    W = normal(rng, (512, 128), SIGMA_W)
    return x, W


# ---------------------------------------------------------------------------
# Decode stack, batch 1: 8 layers of {qkv 384->1152, o 384->384,
# up 384->1536, down 1536->384} plus a 384->4096 head.
# ---------------------------------------------------------------------------
DECODE_STACK_MATS = (  # (name, K, N)
    ("qkv", 384, 1152),
    ("o", 384, 384),
    ("up", 384, 1536),
    ("down", 1536, 384),
)
DECODE_STACK_LAYERS = 8
DECODE_STACK_HEAD = ("head", 384, 4096)


def decode_stack_shapes():
    """List of (layer, mat_index, name, K, N) in pass order; the head is
    layer 8, mat 0."""
    out = []
    for layer in range(DECODE_STACK_LAYERS):
        for mi, (name, K, N) in enumerate(DECODE_STACK_MATS):
            out.append((layer, mi, name, K, N))
    name, K, N = DECODE_STACK_HEAD
    out.append((DECODE_STACK_LAYERS, 0, name, K, N))
    return out


def decode_stack_matrix(layer, mat, K, N):
    """fp32 master W [N,K] and a fresh activation x [1,K] for one matrix."""
    rng = np.random.default_rng([2, layer, mat])
    W = normal(rng, (N, K), SIGMA_W)
    x = normal(rng, (1, K))
    return x, W


# ---------------------------------------------------------------------------
# Prefill GEMM, 2B-class: M = 4096 tokens; j = 0: K=2560 -> N=6912,
# j = 1: K=6912 -> N=2560.  1% of the K channels (chosen without
# replacement) are scaled by 20.
# ---------------------------------------------------------------------------
PREFILL_M = 4096
PREFILL_SHAPES = ((2560, 6912), (6912, 2560))  # (K, N)


def prefill_inputs(j, M=PREFILL_M):
    K, N = PREFILL_SHAPES[j]
    rng = np.random.default_rng([3, j])
    x = normal(rng, (PREFILL_M, K))
    n_out = int(round(0.01 * K))
    ch = rng.choice(K, size=n_out, replace=False)
    x[:, ch] *= np.float32(20.0)
    W = normal(rng, (N, K), SIGMA_W)
    return x[:M], W, np.sort(ch)


# ---------------------------------------------------------------------------
# Batched decode sweep: M in {1,4,16,64} x (K,N) in the three 2B-class
# shapes.  x is drawn at M=64 and sliced, so smaller M are prefixes.
# ---------------------------------------------------------------------------
SWEEP_MS = (1, 4, 16, 64)
SWEEP_SHAPES = ((2560, 6912), (6912, 2560), (2560, 2560))  # (K, N)


def sweep_inputs(shape_idx, M):
    K, N = SWEEP_SHAPES[shape_idx]
    rng = np.random.default_rng([4, shape_idx])
    W = normal(rng, (N, K), SIGMA_W)
    x = normal(rng, (max(SWEEP_MS), K))
    return x[:M].copy(), W


# ---------------------------------------------------------------------------
# Full stack with requantization: 30 layers of {up 2560->6912,
# down 6912->2560}; x0 [2048, 2560]; RMSNorm gain = ones.
# ---------------------------------------------------------------------------
STACK_LAYERS = 30
STACK_M = 2048
STACK_SHAPES = ((2560, 6912), (6912, 2560))  # (K, N) for up, down


def stack_master(layer, which):
    K, N = STACK_SHAPES[which]
    rng = np.random.default_rng([5, layer, which])
    return normal(rng, (N, K), SIGMA_W)


def stack_x0(M=STACK_M):
    rng = np.random.default_rng([5, 99])
    return normal(rng, (STACK_M, STACK_SHAPES[0][0]))[:M].copy()


@dataclass(frozen=True)
class Workload:
    name: str
    description: str


WORKLOADS = {
    "tiny": Workload("tiny", "single BitLinear x[32,128] W[512,128], 1 trit/byte"),
    "decode_stack": Workload("decode_stack",
                             "batch-1 decode pass: 8 x {384->1152, 384->384, 384->1536, "
                             "1536->384} + 384->4096 head, 5 trits/byte"),
    "prefill": Workload("prefill", "M=4096 int8 x ternary GEMM, 2560->6912 and 6912->2560"),
    "sweep": Workload("sweep", "decode GEMV M in {1,4,16,64} x 2B-class shapes, 5 trits/byte"),
    "stack": Workload("stack", "30 x {2560->6912, 6912->2560} requant + RMSNorm/quant + GEMM, "
                               "M=2048"),
}
