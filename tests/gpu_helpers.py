"""Helpers of the GPU parity tests: move seeded numpy inputs to the device with
their leading dimensions, run one call through the C ABI, fetch the result."""
from __future__ import annotations

import contextlib
import sys

import numpy as np
import torch

import gemm_tiled_amd as g

DEV = torch.device("cuda:0")


def say(msg):
    """Name the case before it reaches the GPU (flushed, so it survives a crash)."""
    print(msg, flush=True)
    sys.stdout.flush()


def ld_of(x):
    x = np.asarray(x)
    if x.shape[0] <= 1 or x.size == 0:
        return max(x.shape[1], 1)
    return x.strides[0] // 4


def to_device(x):
    """A device copy of a (possibly padded) row-major float32 view, same leading dimension."""
    x = np.asarray(x, dtype=np.float32)
    rows, cols = x.shape
    ld = ld_of(x)
    full = np.zeros((max(rows, 1), ld), dtype=np.float32)
    full[:rows, :cols] = x
    t = torch.from_numpy(full).to(DEV)
    return t[:rows, :cols]


def run(mode, A, B, C, alpha, beta, stream=None):
    """C_out = alpha*A@B + beta*C on the GPU through the C ABI; numpy result."""
    tA, tB, tC = to_device(A), to_device(B), to_device(C)
    g.gemm(mode, tA, tB, tC, alpha, beta, stream=stream)
    torch.cuda.synchronize()
    return tC.cpu().numpy()


@contextlib.contextmanager
def pinned(mode, spec):
    g.set_config(mode, spec)
    try:
        yield
    finally:
        g.set_config(mode, None)
