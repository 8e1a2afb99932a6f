"""Seeded synthetic inputs and workload shapes for BitLinear W1.58A8.

This module only draws random numbers and names shapes.  It holds none of the
layer's arithmetic (no quantisation, packing or products), so both the CPU
oracle's tests and the GPU library's tests and benchmark can take their
inputs from it without sharing any of the method's code.

Recipe (the pages' 2B-class BitNet b1.58 workload, with random data standing
in for trained weights and real token activations):
  * one ``torch.Generator('cpu')`` per problem, seeded explicitly;
  * draw order: weights first, then activations;
  * weights  W ~ N(0, 0.02^2), fp32, shape [N, K] (nn.Linear layout);
  * activations X ~ N(0, 1), shape [M, K]; for the decode / batched / prefill
    workloads 1% of the K channels (``randperm(K)[:round(0.01 K)]``, the same
    channels for every token) are scaled by 20 to mimic outlier channels, and
    X is then rounded to bf16;
  * QAT backward: the output gradient dY ~ N(0, 0.001^2), fp32 [M, N], drawn
    after W and X from the same generator.
"""
from dataclasses import dataclass, field
from typing import List, Tuple

import torch

W_STD = 0.02
OUTLIER_FRAC = 0.01
OUTLIER_GAIN = 20.0


def generator(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def weight(g: torch.Generator, N: int, K: int) -> torch.Tensor:
    """fp32 master weight [N, K] ~ N(0, 0.02^2)."""
    return torch.randn(N, K, generator=g, dtype=torch.float32) * W_STD


def activations(g: torch.Generator, M: int, K: int, dtype=torch.bfloat16,
                outliers: bool = True) -> torch.Tensor:
    """Token activations [M, K] ~ N(0, 1), optional x20 outlier channels."""
    X = torch.randn(M, K, generator=g, dtype=torch.float32)
    if outliers and K > 0:
        n_out = int(round(OUTLIER_FRAC * K))
        idx = torch.randperm(K, generator=g)[:n_out]
        X[:, idx] *= OUTLIER_GAIN
    return X.to(dtype)


def bitlinear_problem(seed: int, M: int, K: int, N: int, dtype=torch.bfloat16,
                      outliers: bool = True):
    """(W fp32 [N, K], X [M, K]) for one BitLinear, drawn in that order."""
    g = generator(seed)
    W = weight(g, N, K)
    X = activations(g, M, K, dtype=dtype, outliers=outliers)
    return W, X


def ffn_problem(seed: int, M: int, K: int, F: int, N: int, dtype=torch.bfloat16,
                outliers: bool = True):
    """(Wg [F, K], Wu [F, K], Wd [N, F], X [M, K]) for one ReLU^2 FFN block."""
    g = generator(seed)
    Wg = weight(g, F, K)
    Wu = weight(g, F, K)
    Wd = weight(g, N, F)
    X = activations(g, M, K, dtype=dtype, outliers=outliers)
    return Wg, Wu, Wd, X


GRAD_STD = 1e-3


def grad_output(g: torch.Generator, M: int, N: int) -> torch.Tensor:
    """fp32 output gradient dY [M, N] ~ N(0, 0.001^2)."""
    return torch.randn(M, N, generator=g, dtype=torch.float32) * GRAD_STD


def qat_problem(seed: int, M: int, K: int, N: int, dtype=torch.bfloat16, outliers: bool = True):
    """(W fp32 [N, K], X [M, K], dY fp32 [M, N]) for one BitLinear's training
    step, drawn in that order."""
    g = generator(seed)
    W = weight(g, N, K)
    X = activations(g, M, K, dtype=dtype, outliers=outliers)
    dY = grad_output(g, M, N)
    return W, X, dY


def bf16_bits(X: torch.Tensor):
    """bf16 tensor -> numpy uint16 bit patterns (for the CPU oracle)."""
    return X.contiguous().view(torch.int16).numpy().view("uint16")


# --------------------------------------------------------------------------
# Workload shapes (2B-class BitNet b1.58 linear layers: hidden 2560,
# k/v 640, FFN 6912, 30 layers).

@dataclass(frozen=True)
class Shape:
    K: int
    N: int
    name: str = ""


TINY = dict(M=4, K=256, N=256, seed=0, dtype=torch.float32, outliers=False)

DECODE_SHAPES: List[Shape] = [
    Shape(2560, 2560, "q/o 2560->2560"),
    Shape(2560, 640, "k/v 2560->640"),
    Shape(2560, 6912, "gate/up 2560->6912"),
    Shape(6912, 2560, "down 6912->2560"),
]

BATCHED_M = (8, 32, 64)
BATCHED_SHAPES: List[Shape] = [
    Shape(2560, 6912, "gate/up 2560->6912"),
    Shape(6912, 2560, "down 6912->2560"),
]

PREFILL = dict(M=2048, K=2560, F=6912, N=2560, seed=0)

# QAT backward: one 2048-token batch through the FFN's BitLinears.
QAT_M = 2048
QAT_SHAPES: List[Shape] = [
    Shape(2560, 6912, "gate/up 2560->6912"),
    Shape(6912, 2560, "down 6912->2560"),
]

HIDDEN = 2560
KV = 640
FFN = 6912
LAYERS = 30
# (name, K, N) of the seven BitLinears of one layer, in projection order.
LAYER_PROJS: List[Tuple[str, int, int]] = [
    ("q", HIDDEN, HIDDEN),
    ("k", HIDDEN, KV),
    ("v", HIDDEN, KV),
    ("o", HIDDEN, HIDDEN),
    ("gate", HIDDEN, FFN),
    ("up", HIDDEN, FFN),
    ("down", FFN, HIDDEN),
]


def stack_seed(layer: int, proj: int) -> int:
    return 7 * layer + proj


STACK_NAMES = ("Wq", "Wk", "Wv", "Wo", "Wg", "Wu", "Wd")
HEAD_DIM = 128


def stack_layer_weights(seed: int, layer: int, H: int, KV: int, F: int, device="cpu"):
    """fp32 master weights of one layer of the linear stack, in projection
    order q, k, v, o, gate, up, down ([N, K] each), one generator per
    projection seeded with seed + stack_seed(layer, p).  With device="cuda"
    the generator and the draw are on the GPU (bench-sized stacks)."""
    dims = [(H, H), (KV, H), (KV, H), (H, H), (F, H), (F, H), (H, F)]
    out = {}
    for p, (name, (N, K)) in enumerate(zip(STACK_NAMES, dims)):
        g = torch.Generator(device=device)
        g.manual_seed(int(seed + stack_seed(layer, p)))
        out[name] = torch.randn(N, K, generator=g, dtype=torch.float32, device=device) * W_STD
    return out


def stack_norm_gain(seed: int, layer: int, F: int, gain: bool = True):
    """subln gain [F] of one layer: ones (random init), or with gain=True
    U(0.5, 1.5) so that the gain is exercised."""
    if not gain:
        return torch.ones(F, dtype=torch.float32)
    g = generator(seed + 1_000_003 + layer)
    return 0.5 + torch.rand(F, generator=g, dtype=torch.float32)


def stack_token(seed: int, H: int) -> torch.Tensor:
    """fp32 residual-stream input [H] for one decode token (outliers on)."""
    return activations(generator(seed + 2_000_003), 1, H, dtype=torch.float32)[0]
