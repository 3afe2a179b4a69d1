"""Seeded synthetic inputs for block-scaled FP8 / MXFP4 GEMM.

This module only draws random FP32 matrices; it holds none of the method's
arithmetic (no scaling, rounding or encoding).  Both the CPU oracle's tests and
the HIP path's tests and benchmark take their inputs from here, so the two
sides see identical data.

Every matrix is drawn in float64 from ``numpy.random.Generator(PCG64(seed))``
and rounded to float32 (round-to-nearest-even, numpy's ``astype``).  The right
operand B is drawn directly in its stored layout, N rows of K contiguous
elements (a K x N column-major matrix).

The five workloads follow the shapes and value distributions of the pages:
a small square case, a 4096-cube square case (the size the FP8 GEMM article on
CDNA4 compares precisions at, section 5.4, and the size of the MXFP4 host
example in the Rubin FP4 GEMM article, section 4.4), a Transformer
feed-forward shape (the motivation in section 1.1 of the CDNA4 article), a
weight-gradient shape with E5M2 gradients (section 2.2 of the same article
assigns E5M2 to gradients), and an MXFP4 square case.  Two more are
decode-shaped (16 tokens against an 8192 x 8192 weight, FP8 and MXFP4): their
GEMM streams the weight once and is bound by HBM bandwidth, not by the matrix
cores.  They are synthetic stand-ins; no dataset or trained weights are
involved.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

__all__ = ["Workload", "WORKLOADS", "by_name", "normal", "laplace",
           "with_outliers", "operands"]


@dataclass(frozen=True)
class Workload:
    index: int            # 1-based, fixes the seeds 1000*index + {1, 2, 3}
    name: str
    M: int
    N: int
    K: int
    a_fmt: str            # "e4m3" | "e5m2" | "mxfp4"
    b_fmt: str
    out: str              # "f32" | "bf16"
    a_dist: tuple         # ("normal", std) | ("laplace", scale) | ("normal_outliers", std, frac, factor)
    b_dist: tuple
    note: str = ""

    @property
    def seed_a(self) -> int:
        return 1000 * self.index + 1

    @property
    def seed_b(self) -> int:
        return 1000 * self.index + 2

    @property
    def seed_mask(self) -> int:
        return 1000 * self.index + 3

    @property
    def flops(self) -> float:
        return 2.0 * self.M * self.N * self.K


WORKLOADS = [
    Workload(1, "tiny_e4m3_256", 256, 256, 256, "e4m3", "e4m3", "f32",
             ("normal", 1.0), ("normal", 1.0),
             "A 256x256 and B 256x256 ~N(0,1); 128x32 tiles; FP32 output"),
    Workload(2, "square_e4m3_4096", 4096, 4096, 4096, "e4m3", "e4m3", "bf16",
             ("normal", 1.0), ("normal", 1.0),
             "M=N=K=4096 ~N(0,1); 128x32 tiles; bf16 output"),
    Workload(3, "ffn_e4m3_16384x14336x4096", 16384, 14336, 4096, "e4m3", "e4m3", "bf16",
             ("normal_outliers", 1.0, 0.001, 100.0), ("normal", 0.02),
             "activations ~N(0,1) with 0.1% of entries x100; weights ~N(0,0.02); bf16 output"),
    Workload(4, "dw_e5m2xe4m3_4096x4096x16384", 4096, 4096, 16384, "e5m2", "e4m3", "f32",
             ("laplace", 1e-3), ("normal", 1.0),
             "G^T in E5M2 ~Laplace(0,1e-3); X in E4M3 ~N(0,1); FP32 output"),
    Workload(5, "mxfp4_8192", 8192, 8192, 8192, "mxfp4", "mxfp4", "bf16",
             ("normal", 1.0), ("normal", 1.0),
             "A, B ~N(0,1); E2M1 in 32-wide K blocks with E8M0 scales; bf16 output"),
    Workload(6, "skinny_e4m3_16x8192x8192", 16, 8192, 8192, "e4m3", "e4m3", "bf16",
             ("normal", 1.0), ("normal", 0.02),
             "16 tokens ~N(0,1) against weights ~N(0,0.02); 128x32 tiles; bf16 output; HBM-bound"),
    Workload(7, "skinny_mxfp4_16x8192x8192", 16, 8192, 8192, "mxfp4", "mxfp4", "bf16",
             ("normal", 1.0), ("normal", 0.02),
             "16 tokens ~N(0,1) against weights ~N(0,0.02); E2M1 with E8M0 scales; bf16 output; HBM-bound"),
]


def by_name(name: str) -> Workload:
    for w in WORKLOADS:
        if w.name == name or str(w.index) == str(name):
            return w
    raise KeyError(name)


def normal(seed: int, rows: int, cols: int, std: float = 1.0) -> np.ndarray:
    """rows x cols float32, N(0, std^2), drawn in float64 then rounded."""
    g = np.random.Generator(np.random.PCG64(seed))
    x = g.standard_normal((rows, cols))
    if std != 1.0:
        x *= std
    return x.astype(np.float32)


def laplace(seed: int, rows: int, cols: int, scale: float) -> np.ndarray:
    """rows x cols float32, Laplace(0, scale), no clamping."""
    g = np.random.Generator(np.random.PCG64(seed))
    return g.laplace(0.0, scale, size=(rows, cols)).astype(np.float32)


def with_outliers(x: np.ndarray, seed: int, frac: float, factor: float) -> np.ndarray:
    """Multiply round(frac * x.size) distinct, uniformly chosen entries by factor (in place)."""
    g = np.random.Generator(np.random.PCG64(seed))
    n = int(round(frac * x.size))
    idx = g.choice(x.size, size=n, replace=False)
    flat = x.reshape(-1)
    flat[idx] = (flat[idx].astype(np.float64) * factor).astype(np.float32)
    return x


def _draw(dist: tuple, seed: int, seed_mask: int, rows: int, cols: int) -> np.ndarray:
    kind = dist[0]
    if kind == "normal":
        return normal(seed, rows, cols, dist[1])
    if kind == "laplace":
        return laplace(seed, rows, cols, dist[1])
    if kind == "normal_outliers":
        x = normal(seed, rows, cols, dist[1])
        return with_outliers(x, seed_mask, dist[2], dist[3])
    raise ValueError(kind)


def operands(w: Workload, M: Optional[int] = None, N: Optional[int] = None,
             K: Optional[int] = None):
    """Return (A [M x K], B [N x K]) float32 for workload w.

    M, N, K default to the workload's own sizes; smaller values draw the same
    distributions at a reduced shape (used for fast CPU checks)."""
    M = w.M if M is None else M
    N = w.N if N is None else N
    K = w.K if K is None else K
    a = _draw(w.a_dist, w.seed_a, w.seed_mask, M, K)
    b = _draw(w.b_dist, w.seed_b, w.seed_mask + 1000000, N, K)
    return a, b
