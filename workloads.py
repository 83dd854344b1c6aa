"""Seeded synthetic inputs for C = alpha*A@B + beta*C, shared by the tests, the
benchmark and the oracle checks.

This module holds random draws and casts only -- none of the method's
arithmetic (no rounding to f16, no products).  The pages measure no dataset:
their workloads are dense iid random matrices (the lab draws U[0,1) and normal
matrices with a fixed seed), so these generators are the workload.

Recipe: ``numpy.random.default_rng(seed)``, draw A, then B, then C, each in
float64 at its full (M,K), (K,N), (M,N) shape, cast to float32.  Distributions
are ``uniform(-1, 1)``, ``standard_normal``, or ``centered`` (U[0,1) - 0.5, the
inputs of the lab's precision study).  With padded leading dimensions
the matrix is drawn at its logical shape and placed into a larger zero buffer.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    mode: str                 # "f32" or "f16r"
    M: int
    N: int
    K: int
    alpha: float
    beta: float
    dist: str                 # "uniform" (U[-1,1]) or "normal" (N(0,1))
    seed: int = 0
    lda: int | None = None    # leading dims; None = dense (row length)
    ldb: int | None = None
    ldc: int | None = None
    extra_betas: tuple = field(default_factory=tuple)

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K


# The five workloads (names say what they are).  The two runs of the f32 4096^3
# workload share A, B, C and differ only in beta.
WORKLOADS = {
    "f32_256_a1.5_b0.5": Workload("f32_256_a1.5_b0.5", "f32", 256, 256, 256, 1.5, 0.5, "uniform"),
    "f32_4096_a1_b0": Workload("f32_4096_a1_b0", "f32", 4096, 4096, 4096, 1.0, 0.0, "uniform"),
    "f32_4096_a1_b1": Workload("f32_4096_a1_b1", "f32", 4096, 4096, 4096, 1.0, 1.0, "uniform"),
    "f16r_4096_a1_b0.5": Workload("f16r_4096_a1_b0.5", "f16r", 4096, 4096, 4096, 1.0, 0.5,
                                  "uniform"),
    "f32_4000x4097x4093_a2_b-1": Workload("f32_4000x4097x4093_a2_b-1", "f32", 4000, 4097, 4093,
                                          2.0, -1.0, "normal"),
    "f16r_8192_a0.75_b-0.25": Workload("f16r_8192_a0.75_b-0.25", "f16r", 8192, 8192, 8192,
                                       0.75, -0.25, "normal"),
}


def _draw(rng, dist, shape):
    if dist == "uniform":
        return rng.uniform(-1.0, 1.0, size=shape)
    if dist == "centered":          # the lab's precision inputs: U[0,1) - 0.5
        return rng.random(size=shape) - 0.5
    if dist == "normal":
        return rng.standard_normal(size=shape)
    if dist == "ones":
        return np.ones(shape)
    raise ValueError(f"unknown distribution {dist!r}")


def _place(x64, ld):
    rows, cols = x64.shape
    if ld is None or ld == cols:
        return x64.astype(np.float32)
    if ld < cols:
        raise ValueError("leading dimension smaller than the row length")
    buf = np.zeros((rows, ld), dtype=np.float32)
    buf[:, :cols] = x64.astype(np.float32)
    return buf[:, :cols]


def make_inputs(M, N, K, dist="uniform", seed=0, lda=None, ldb=None, ldc=None):
    """(A, B, C) float32 row-major views with the given leading dimensions."""
    rng = np.random.default_rng(seed)
    A = _place(_draw(rng, dist, (M, K)), lda)
    B = _place(_draw(rng, dist, (K, N)), ldb)
    C = _place(_draw(rng, dist, (M, N)), ldc)
    return A, B, C


def workload_inputs(w: Workload):
    return make_inputs(w.M, w.N, w.K, w.dist, w.seed, w.lda, w.ldb, w.ldc)


def small_integers(M, N, K, lo=-8, hi=8, seed=0, lda=None, ldb=None, ldc=None):
    """Integer-valued float32 matrices with entries in [lo, hi]."""
    rng = np.random.default_rng(seed)
    A = _place(rng.integers(lo, hi + 1, size=(M, K)).astype(np.float64), lda)
    B = _place(rng.integers(lo, hi + 1, size=(K, N)).astype(np.float64), ldb)
    C = _place(rng.integers(lo, hi + 1, size=(M, N)).astype(np.float64), ldc)
    return A, B, C


def sample_indices(M, N, n, seed=1):
    """n (row, col) sample positions: the four corners, the last row and column
    (the ragged edge), and uniformly random positions."""
    rng = np.random.default_rng(seed)
    fixed_r = [0, 0, M - 1, M - 1]
    fixed_c = [0, N - 1, 0, N - 1]
    edge = min(64, max(n // 8, 1))
    er = list(rng.integers(0, M, size=edge)) + [M - 1] * edge
    ec = [N - 1] * edge + list(rng.integers(0, N, size=edge))
    k = max(n - len(fixed_r) - len(er), 0)
    rr = list(rng.integers(0, M, size=k))
    cc = list(rng.integers(0, N, size=k))
    rows = np.array(fixed_r + er + rr, dtype=np.int64)
    cols = np.array(fixed_c + ec + cc, dtype=np.int64)
    return rows, cols
