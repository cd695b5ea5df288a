"""Workload shapes: the linear layers of the models the pages measure.

Shapes are (rows, cols) = (d_out, d_in) of each projection of one decoder
layer.  The pages report end-to-end decode speed on Llama-3.1-8B,
Llama-3.3-70B, Qwen3-14B and Qwen3-32B ("Experiments", Table 3 paragraph);
the per-layer shapes below are those models' published architectures.
"""

from __future__ import annotations

from dataclasses import dataclass

# Llama-3.1-8B: hidden 4096, 32 query heads / 8 kv heads of 128, MLP 14336.
LLAMA8B_LAYER = (
    ("q", 4096, 4096),
    ("k", 1024, 4096),
    ("v", 1024, 4096),
    ("o", 4096, 4096),
    ("gate", 14336, 4096),
    ("up", 14336, 4096),
    ("down", 4096, 14336),
)

# Llama-3.3-70B: hidden 8192, 64 query heads / 8 kv heads of 128, MLP 28672.
LLAMA70B_SHAPES = (
    ("70b.q", 8192, 8192),
    ("70b.k", 1024, 8192),
    ("70b.gate", 28672, 8192),
    ("70b.down", 8192, 28672),
)

# Qwen3-32B: hidden 5120, 64 query heads of 128 (8192 wide), MLP 25600.
QWEN32B_SHAPES = (
    ("qwen32b.q", 8192, 5120),
    ("qwen32b.o", 5120, 8192),
    ("qwen32b.gate", 25600, 5120),
    ("qwen32b.down", 5120, 25600),
)

PATTERNS_50 = ((2, 4), (4, 8), (8, 16), (16, 32))

# N:M densities other than 50% (M | 32): the same format with 32N/M kept
# columns per mask word.
OTHER_DENSITIES = ((1, 4), (3, 4), (1, 8), (3, 8))


@dataclass(frozen=True)
class Matrix:
    name: str
    rows: int
    cols: int
    n: int
    m: int
    dtype: str  # "f16" or "bf16"
    seed: int
    outliers: bool  # whether x carries outlier channels


def decode_layer(config: int, layer: int = 0, n: int = 2, m: int = 4, dtype: str = "f16"):
    """The seven projections of one Llama-3.1-8B decoder layer."""
    from .synth import layer_seed
    return [Matrix(name, r, c, n, m, dtype, layer_seed(config, layer, i), True)
            for i, (name, r, c) in enumerate(LLAMA8B_LAYER)]


def config_matrices(config: int):
    """Every (matrix, batches) pair of a workload, 1-based config number.

    1: one 2:4 fp16 4096x4096 matrix, seed 0, no outlier channels, batch 1.
    2: one Llama-3.1-8B layer (q, k, v, o, gate, up, down), 2:4 fp16, batch 1, 4.
    3: the same shapes under 4:8, 8:16 and 16:32, bf16, batch 1, 2, 8.
    4: Llama-3.3-70B and Qwen3-32B layer shapes, 2:4 fp16, batch 1, 8.
    5: 32 stacked Llama-3.1-8B layers, 2:4 fp16, batch 1, 2, 4, 8.
    """
    from .synth import layer_seed
    if config == 1:
        return [(Matrix("single", 4096, 4096, 2, 4, "f16", 0, False), (1,))]
    if config == 2:
        return [(mt, (1, 4)) for mt in decode_layer(2)]
    if config == 3:
        out = []
        for (n, m) in PATTERNS_50[1:]:
            for i, (name, r, c) in enumerate(LLAMA8B_LAYER):
                seed = layer_seed(3, m, i)
                out.append((Matrix(f"{name}.{n}:{m}", r, c, n, m, "bf16", seed, True), (1, 2, 8)))
        return out
    if config == 4:
        shapes = LLAMA70B_SHAPES + QWEN32B_SHAPES
        return [(Matrix(name, r, c, 2, 4, "f16", layer_seed(4, 0, i), True), (1, 8))
                for i, (name, r, c) in enumerate(shapes)]
    if config == 5:
        out = []
        for layer in range(32):
            for mt in decode_layer(5, layer):
                out.append((mt, (1, 2, 4, 8)))
        return out
    raise ValueError(f"no workload {config}")


def density_matrices():
    """The 8B gate (14336x4096) and down (4096x14336) shapes at the densities
    other than 50%, fp16, batch 1 and 8 (seeds from workload 6)."""
    from .synth import layer_seed
    out = []
    for j, (n, m) in enumerate(OTHER_DENSITIES):
        for i, (name, r, c) in enumerate(LLAMA8B_LAYER):
            if name in ("gate", "down"):
                out.append((Matrix(f"{name}.{n}:{m}", r, c, n, m, "f16", layer_seed(6, j, i), True),
                            (1, 8)))
    return out


def sparse_bytes(rows: int, cols: int, n: int, m: int, batch: int, out_bytes: int) -> int:
    """Algorithmic HBM bytes of one sparse call: packed values, mask words,
    x and y, each read or written once."""
    return rows * cols * n // m * 2 + rows * cols // 8 + batch * cols * 2 + batch * rows * out_bytes


def dense_bytes(rows: int, cols: int, batch: int, out_bytes: int) -> int:
    """Algorithmic HBM bytes of one dense 16-bit GEMV call."""
    return rows * cols * 2 + batch * cols * 2 + batch * rows * out_bytes
