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
from workloads import make_inputs, sample_indices

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


def _large_cases(n, seed):
    """Larger shapes, where the rings, their stream-K and masked forms, the
    f32-panel ring and the packed path run: each dimension uniform in
    200..3000, a multiple of 4 half the time (16-byte rows with the matrix
    width as leading dimension), otherwise padded by 0..3."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        dims = []
        for _ in range(3):
            d = int(rng.integers(200, 3001))
            dims.append(d - d % 4 if rng.random() < 0.5 else d)
        pads = [int(rng.choice([0, 0, 1, 3])) for _ in range(3)]
        beta = float(rng.choice([0.0, 1.0, -0.25]))
        out.append((*dims, pads, beta))
    return out


LARGE = [(mode, i, c) for mode, seed in (("f32", 201), ("f16r", 202))
         for i, c in enumerate(_large_cases(30, seed))]


@pytest.mark.parametrize("mode,i,case", LARGE, ids=[f"{m}-{i}" for m, i, _ in LARGE])
def test_random_large_shape_sampled(mode, i, case):
    """The last row and column in full, plus sampled elements, against the
    oracle (the full product is too long for the float64 oracle here)."""
    M, N, K, pads, beta = case
    A, B, C = make_inputs(M, N, K, "normal", seed=2000 + i,
                          lda=K + pads[0], ldb=N + pads[1], ldc=N + pads[2])
    Cin = np.full_like(C, np.nan) if beta == 0.0 else C
    plan = g.get_plan(mode, M, N, K, lda=K + pads[0], ldb=N + pads[1], ldc=N + pads[2], beta=beta)
    say(f"[random large] {mode} #{i} {M}x{N}x{K} pads={pads} beta={beta} {plan}")
    tA, tB, tC = to_device(A), to_device(B), to_device(Cin)
    g.gemm(mode, tA, tB, tC, 0.75, beta)
    torch.cuda.synchronize()
    got = tC.cpu().numpy()
    Cref = np.zeros_like(C) if beta == 0.0 else C
    r = np.concatenate([np.full(N, M - 1), np.arange(M), sample_indices(M, N, 2048, seed=i)[0]])
    c = np.concatenate([np.arange(N), np.full(M, N - 1), sample_indices(M, N, 2048, seed=i)[1]])
    ref, W = oracle.entries(mode, A, B, Cref, 0.75, beta, r, c)
    err = np.abs(got[r, c].astype(np.float64) - ref)
    bad = ~(err <= oracle.TOL[mode] * W)
    assert not bad.any(), (case, plan, int(bad.sum()), r[bad][:5], c[bad][:5])
