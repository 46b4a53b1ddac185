"""Seeded synthetic inputs and the transformer-shaped matrix groups the Muon
step is measured on.

This module holds no arithmetic of the method.  It only draws random numbers,
encodes them as fp32 or bf16 bit patterns (round to nearest even), and lists
shapes.  Both the HIP-path tests and the oracle tests take their inputs from
here, so both sides see identical bits.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


# ------------------------------------------------------------- encodings


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest, ties to even.
    Inputs here are finite Gaussians, so NaN handling is not needed."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    r = (b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


# ---------------------------------------------------------------- drawing


def gaussian(shape, seed: int, sigma: float = 1.0) -> np.ndarray:
    """i.i.d. N(0, sigma^2) as float32, numpy PCG64 seeded with `seed`."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return (rng.standard_normal(shape, dtype=np.float32) * np.float32(sigma)).astype(np.float32)


def grad_seed(config_id: int, matrix: int, micro: int = 0, step: int = 0) -> int:
    """Seed of one micro-batch gradient: 1000*config + 10*matrix + micro,
    shifted by 100000*step for later optimizer steps."""
    return 1000 * config_id + 10 * matrix + micro + 100000 * step


def make_grad(shape, seed: int, sigma: float, dtype: str) -> np.ndarray:
    """One gradient in storage form: float32 array ('fp32') or uint16 bf16
    bits ('bf16')."""
    g = gaussian(shape, seed, sigma)
    if dtype == "fp32":
        return g
    if dtype == "bf16":
        return f32_to_bf16_bits(g)
    raise ValueError(dtype)


def warm_momentum(shape, seed: int, sigma: float) -> np.ndarray:
    """A non-zero fp32 momentum state (so the blend is not a pure rescale)."""
    return gaussian(shape, seed + 500, sigma)


# ------------------------------------------------------------- workloads


@dataclass
class Workload:
    name: str
    config_id: int
    shapes: list                 # [(rows, cols)] in group order
    heads: list                  # per matrix: 0/1 = unsplit, h = row blocks
    grad_dtype: str              # storage dtype of the step's gradient input
    micro_dtype: str             # storage dtype of each micro-batch gradient
    sigma: float
    gas: int                     # micro-batches accumulated per step
    steps: int                   # optimizer steps in the workload
    num_partitions: int
    align: int = 16
    methods: tuple = ("standard",)
    precision: str = "bf16"
    note: str = ""
    layer_kinds: list = field(default_factory=list)

    @property
    def numel(self) -> int:
        return sum(r * c for r, c in self.shapes)


def tiny() -> Workload:
    """Two fp32 matrices 17x13 and 9x17 that straddle two partitions."""
    return Workload(
        name="tiny", config_id=0, shapes=[(17, 13), (9, 17)], heads=[0, 0],
        grad_dtype="fp32", micro_dtype="fp32", sigma=1.0, gas=3, steps=3,
        num_partitions=2, methods=("standard", "gram"), precision="fp32",
        layer_kinds=["w0", "w1"])


def h1024(layers: int = 12) -> Workload:
    """12-layer transformer, hidden 1024: q,k,v,o 1024x1024, MLP 1024x4096
    and 4096x1024."""
    shapes, kinds = [], []
    for _ in range(layers):
        for k in ("q", "k", "v", "o"):
            shapes.append((1024, 1024)); kinds.append(k)
        shapes.append((1024, 4096)); kinds.append("mlp_wide")
        shapes.append((4096, 1024)); kinds.append("mlp_tall")
    return Workload(
        name="h1024_12layer", config_id=1, shapes=shapes, heads=[0] * len(shapes),
        grad_dtype="bf16", micro_dtype="bf16", sigma=0.02, gas=1, steps=1,
        num_partitions=1, layer_kinds=kinds)


def per_head(layers: int = 32) -> Workload:
    """32 layers of q and k 4096x4096 split into 32 heads of 128 rows, plus
    o 4096x4096 unsplit; Gram form."""
    shapes, heads, kinds = [], [], []
    for _ in range(layers):
        for k, h in (("q", 32), ("k", 32), ("o", 0)):
            shapes.append((4096, 4096)); heads.append(h); kinds.append(k)
    return Workload(
        name="per_head_32layer", config_id=2, shapes=shapes, heads=heads,
        grad_dtype="bf16", micro_dtype="bf16", sigma=0.02, gas=1, steps=1,
        num_partitions=1, methods=("gram", "standard"), layer_kinds=kinds)


def llama7b(layers: int = 32) -> Workload:
    """Llama-7B-shaped group: per layer 4x 4096x4096, 2x 4096x11008,
    1x 11008x4096; bf16 micro-batch grads accumulated (gas=4) into fp32, one
    step, 8 notional partitions.  sigma is not stated for this workload;
    N(0, 0.02^2) like the other bf16 groups."""
    shapes, kinds = [], []
    for _ in range(layers):
        for k in ("q", "k", "v", "o"):
            shapes.append((4096, 4096)); kinds.append(k)
        shapes.append((4096, 11008)); kinds.append("gate")
        shapes.append((4096, 11008)); kinds.append("up")
        shapes.append((11008, 4096)); kinds.append("down")
    return Workload(
        name="llama7b_32layer", config_id=3, shapes=shapes, heads=[0] * len(shapes),
        grad_dtype="fp32", micro_dtype="bf16", sigma=0.02, gas=4, steps=1,
        num_partitions=8, methods=("standard", "gram"), layer_kinds=kinds)


def share70b(layers: int = 8) -> Workload:
    """70B-shaped single-GPU share: 8 layers of q,o 8192x8192, k,v 8192x1024,
    gate,up 8192x28672, down 28672x8192."""
    shapes, kinds = [], []
    for _ in range(layers):
        shapes += [(8192, 8192), (8192, 1024), (8192, 1024), (8192, 8192),
                   (8192, 28672), (8192, 28672), (28672, 8192)]
        kinds += ["q", "k", "v", "o", "gate", "up", "down"]
    return Workload(
        name="share70b_8layer", config_id=4, shapes=shapes, heads=[0] * len(shapes),
        grad_dtype="bf16", micro_dtype="bf16", sigma=0.01, gas=1, steps=1,
        num_partitions=1, methods=("standard", "gram"), layer_kinds=kinds)


def custom(spec: str) -> Workload:
    """A synthetic group from a spec "custom:RxC*N[/H],RxC*N,..." (N copies of
    a rows x cols matrix, optionally split into H heads); bf16 N(0, 0.02^2)
    grads, one step, one partition."""
    shapes, heads = [], []
    for part in spec.split(":", 1)[1].split(","):
        h = 0
        if "/" in part:
            part, hs = part.split("/")
            h = int(hs)
        dims, _, cnt = part.partition("*")
        r, c = (int(v) for v in dims.split("x"))
        for _ in range(int(cnt or 1)):
            shapes.append((r, c)); heads.append(h)
    return Workload(name=spec, config_id=9, shapes=shapes, heads=heads, grad_dtype="bf16", micro_dtype="bf16",
                    sigma=0.02, gas=1, steps=1, num_partitions=1, methods=("standard", "gram"))


ALL = {w().name: w for w in (tiny, h1024, per_head, llama7b, share70b)}
