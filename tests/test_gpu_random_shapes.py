"""Seeded random shapes through the library's own choice of configuration (no
pins), both modes, every element of C against the oracle's bound.

The shapes are drawn once from a fixed seed: each of M, N and K log-uniform
in 1..16 one time in five and in 17..1500 otherwise (so few rows, few
columns, ragged tiles, short and ragged K all occur), leading dimensions the
matrix width plus 0, 1, 3 or 4 (16-byte, 8-byte and 4-byte aligned rows),
each operand stored transposed one time in four, alpha and
beta from a small set that includes beta = 0 (C must then not be read: it
holds NaN).  The product M N K is kept under 2^27 so the float64 oracle
finishes each case in well under a second.  Every case names its shape before
it reaches the GPU.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from workloads import make_inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():   # collected on CPU-only hosts, never run there
    pytest.skip("no GPU", allow_module_level=True)

import gemm_tiled_amd as g  # noqa: E402
from tests.gpu_helpers import say, to_device  # noqa: E402


def _cases(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        # a dimension is small (1..16) one time in five, else 17..1500
        M, N, K = (int(np.exp(rng.uniform(0.0, np.log(17.0)))) if rng.random() < 0.2
                   else int(np.exp(rng.uniform(np.log(17.0), np.log(1500.0)))) for _ in range(3))
        if M * N * K >= 1 << 27:
            continue
        ta, tb = bool(rng.random() < 0.25), bool(rng.random() < 0.25)
        pads = [int(rng.choice([0, 1, 3, 4])) for _ in range(3)]
        alpha = float(rng.choice([1.0, -0.5, 1.75]))
        beta = float(rng.choice([0.0, 1.0, -0.25]))
        out.append((M, N, K, ta, tb, pads, alpha, beta))
    return out


CASES = [(mode, i, c) for mode, seed in (("f32", 101), ("f16r", 102))
         for i, c in enumerate(_cases(150, seed))]


@pytest.mark.parametrize("mode,i,case", CASES, ids=[f"{m}-{i}" for m, i, _ in CASES])
def test_random_shape_against_the_oracle(mode, i, case):
    M, N, K, ta, tb, pads, alpha, beta = case
    # the operands as the call sees them (op(A) M x K, op(B) K x N), stored
    # transposed where asked, each with its padded leading dimension
    A, B, C = make_inputs(M, N, K, "normal", seed=1000 + i)
    if beta == 0.0:
        C = np.full((M, N), np.nan, dtype=np.float32)
    sa = np.ascontiguousarray(A.T) if ta else A
    sb = np.ascontiguousarray(B.T) if tb else B

    def padded(x, pad):
        full = np.zeros((x.shape[0], x.shape[1] + pad), dtype=np.float32)
        full[:, :x.shape[1]] = x
        return full[:, :x.shape[1]]

    tA, tB, tC = to_device(padded(sa, pads[0])), to_device(padded(sb, pads[1])), \
        to_device(padded(C, pads[2]))
    plan = g.get_plan(mode, M, N, K, lda=tA.stride(0), ldb=tB.stride(0), ldc=tC.stride(0),
                      beta=beta, transa=ta, transb=tb)
    say(f"[random] {mode} #{i} {M}x{N}x{K} ta={ta} tb={tb} pads={pads} alpha={alpha} "
        f"beta={beta} {plan}")
    g.gemm(mode, tA, tB, tC, alpha, beta, transa=ta, transb=tb)
    torch.cuda.synchronize()
    got = tC.cpu().numpy()
    Cref = np.zeros((M, N), dtype=np.float32) if beta == 0.0 else C
    st = oracle.check(mode, A, B, Cref, alpha, beta, got)
    assert st["n_fail"] == 0, (case, plan, st)
