"""Seeded synthetic inputs for the WTConv layer.

This module only draws random numbers: it holds none of the layer's arithmetic.
Both the GPU library's tests/benchmark and the CPU oracle's tests take their
inputs from here.

The pages evaluate "the WTConvNeXt configuration across decomposition levels and
a broad range of tensor shapes" without listing the shapes (abstract of "Fast and
Memory-Efficient Wavelet Convolutions via I/O-Aware Reformulation").  The named
workloads below stand in for them: WTConvNeXt stage shapes, a level sweep and a
large-map stress case, all with k = 5 (the kernel size the pages' comparison
against the 7x7 depthwise conv uses, technical summary, Results).

Recipe (every workload): numpy ``default_rng(seed)``, float32 standard normals,
drawn in this order: x, dy, base weight, bias, then for each level its weight
and its scale jitter.  Values:
    x, dy            N(0, 1)
    w_base, w_lvl    N(0, 0.05^2)
    bias             N(0, 0.01^2)
    s_base           exactly 1
    s_lvl            0.1 + N(0, 0.01^2)
For fp16 workloads x and dy are rounded to fp16 (round to nearest even); the
parameters stay float32.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    n: int
    c: int
    h: int
    w: int
    k: int
    levels: int
    dtype: str  # "f32" or "f16" activation storage
    seed: int

    @property
    def elems(self) -> int:
        return self.n * self.c * self.h * self.w

    @property
    def ebytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    def with_levels(self, levels: int, dtype: str | None = None) -> "Workload":
        return Workload(self.name, self.n, self.c, self.h, self.w, self.k, levels,
                        dtype or self.dtype, self.seed)


WORKLOADS = {
    "tiny": Workload("tiny", 2, 8, 16, 16, 5, 2, "f32", 0),
    "stage1": Workload("stage1", 64, 96, 56, 56, 5, 3, "f32", 1),
    "stage2": Workload("stage2", 64, 192, 28, 28, 5, 2, "f16", 2),
    "sweep": Workload("sweep", 32, 128, 128, 128, 5, 3, "f32", 3),  # levels 1..5, f32 and f16
    "large": Workload("large", 16, 256, 256, 256, 5, 4, "f16", 4),
}


def sweep_workloads():
    """The level sweep: 32x128x128x128, k=5, L=1..5, fp32 and fp16 storage."""
    base = WORKLOADS["sweep"]
    return [base.with_levels(l, dt) for dt in ("f32", "f16") for l in range(1, 6)]


@dataclass
class Inputs:
    x: np.ndarray       # (N, C, H, W) float32 (fp16-representable values for f16)
    dy: np.ndarray      # (N, C, H, W)
    w_base: np.ndarray  # (C, k, k) float32
    bias: np.ndarray    # (C,)
    s_base: np.ndarray  # (C,)
    w_lvl: np.ndarray   # (L, 4C, k, k), band b of channel c at 4c+b
    s_lvl: np.ndarray   # (L, 4C)


def make_inputs(n, c, h, w, k, levels, dtype="f32", seed=0, activations=True) -> Inputs:
    """Draw one seeded input set (see the module docstring for the recipe)."""
    rng = np.random.default_rng(seed)
    if activations:
        x = rng.standard_normal((n, c, h, w), dtype=np.float32)
        dy = rng.standard_normal((n, c, h, w), dtype=np.float32)
        if dtype == "f16":
            x = x.astype(np.float16).astype(np.float32)
            dy = dy.astype(np.float16).astype(np.float32)
    else:
        x = dy = None
    w_base = (0.05 * rng.standard_normal((c, k, k), dtype=np.float32)).astype(np.float32)
    bias = (0.01 * rng.standard_normal((c,), dtype=np.float32)).astype(np.float32)
    s_base = np.ones((c,), dtype=np.float32)
    w_lvl = np.empty((levels, 4 * c, k, k), dtype=np.float32)
    s_lvl = np.empty((levels, 4 * c), dtype=np.float32)
    for l in range(levels):
        w_lvl[l] = 0.05 * rng.standard_normal((4 * c, k, k), dtype=np.float32)
        s_lvl[l] = 0.1 + 0.01 * rng.standard_normal((4 * c,), dtype=np.float32)
    return Inputs(x, dy, w_base, bias, s_base, w_lvl, s_lvl)


def workload_inputs(wl: Workload, activations=True) -> Inputs:
    return make_inputs(wl.n, wl.c, wl.h, wl.w, wl.k, wl.levels, wl.dtype, wl.seed, activations)
