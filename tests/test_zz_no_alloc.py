"""gemm355_gemm_noalloc: the variant of gemm_f32_ex / gemm_f16r_f32acc_ex whose
scratch is the library's fixed per-GPU array.  Through the C ABI, its result
must equal the allocating entry point's bit for bit (same configuration, same
kernels: only the scratch differs) and lie inside the oracle's bound, on two
calls in a row, the second smaller (the array keeps the first call's
contents, its counters included).  A call too large for the array is refused
with nothing launched; and a call captured into a graph on a fresh stream (no
eager call first) replays correctly, since nothing needs allocating.
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
from tests.gpu_helpers import pinned, say, to_device  # noqa: E402


def _pair(mode, M, N, K, seed, alpha, beta, transa=False, transb=False):
    A, B, C = make_inputs(M, N, K, "normal", seed=seed)
    Aop, Bop = A, B
    if transa:
        A = np.ascontiguousarray(A.T)
    if transb:
        B = np.ascontiguousarray(B.T)
    tA, tB = to_device(A), to_device(B)
    c_ref, c_na = to_device(C), to_device(C)
    say(f"[noalloc] {mode} {M}x{N}x{K} ta={transa} tb={transb} "
        f"{g.get_plan(mode, M, N, K, beta=beta, transa=transa, transb=transb)}")
    g.gemm(mode, tA, tB, c_ref, alpha, beta, transa=transa, transb=transb)
    g.gemm_noalloc(mode, tA, tB, c_na, alpha, beta, transa=transa, transb=transb)
    torch.cuda.synchronize()
    ref, got = c_ref.cpu().numpy(), c_na.cpu().numpy()
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), \
        f"{int((got != ref).sum())} elements differ from the allocating entry point"
    st = oracle.check(mode, Aop, Bop, C, alpha, beta, got)
    assert st["n_fail"] == 0, st


# Each pair: a call that needs scratch, then a smaller one.
@pytest.mark.parametrize("mode,first,second", [
    # f16r packed operands (+ stream-K partials and counters at 2048^3)
    ("f16r", (2048, 2048, 2048), (1000, 700, 300)),
    # f16r rounding on load, K split (partials + counters), then fewer tiles
    ("f16r", (256, 4096, 4096), (40, 1000, 2048)),
    # f32 ring with K split over idle CUs (partials + counters), then split-K tiles
    ("f32", (256, 4096, 4096), (100, 520, 2000)),
    # f32 few rows with K split (partials + counters), then fewer rows
    ("f32", (16, 4096, 4096), (9, 3000, 4096)),
])
def test_noalloc_matches_the_allocating_entry_point(mode, first, second):
    _pair(mode, *first, seed=1, alpha=1.25, beta=-0.5)
    _pair(mode, *second, seed=2, alpha=0.75, beta=0.5)


@pytest.mark.parametrize("mode", ["f32", "f16r"])
def test_noalloc_layouts_and_special_cases(mode):
    _pair(mode, 300, 260, 500, seed=3, alpha=1.0, beta=0.25, transa=True)
    _pair(mode, 64, 900, 1500, seed=4, alpha=1.0, beta=0.0, transb=True)
    # K = 0: C = beta * C; M = 0: nothing
    A = torch.zeros((5, 0), device="cuda")
    B = torch.zeros((0, 7), device="cuda")
    C = torch.ones((5, 7), device="cuda")
    g.gemm_noalloc(mode, A, B, C, 1.0, 2.0)
    torch.cuda.synchronize()
    assert torch.equal(C, torch.full((5, 7), 2.0, device="cuda"))


def test_noalloc_refuses_a_call_larger_than_its_array():
    """f16r 8192^3 packs 256 MiB of operands: more than the 160 MiB array.
    The call returns GEMM355_ERR_SCRATCH (-107) and C stays as it was."""
    n = 8192
    tA = torch.ones((n, n), device="cuda")
    tB = torch.ones((n, n), device="cuda")
    tC = torch.full((n, n), 3.0, device="cuda")
    say("[noalloc] refusal at f16r 8192^3")
    with pytest.raises(g.Gemm355Error) as err:
        g.gemm_noalloc("f16r", tA, tB, tC, 1.0, 1.0)
    assert err.value.status == -107, err.value
    torch.cuda.synchronize()
    assert bool((tC == 3.0).all())


@pytest.mark.parametrize("mode,M,N,K,cfg", [
    ("f16r", 1280, 384, 3072, None),          # packed operands
    ("f32", 16, 384, 4096, None),             # few rows: partials + counters
    ("f32", 2048, 2048, 1024, "BM=256 BN=256 BK=16 ST=4 WM=4 WN=2"),   # stream-K ring
])
def test_noalloc_captured_on_a_fresh_stream(mode, M, N, K, cfg):
    """No eager call first: capture into a graph works at once, and every
    replay (eager work and synchronisations in between) equals the eager
    result of the allocating entry point bit for bit."""
    A, B, C = make_inputs(M, N, K, "uniform", seed=5)
    tA, tB, tC = to_device(A), to_device(B), to_device(C)
    C0 = tC.clone()
    s = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    ctx = pinned(mode, cfg) if cfg else pinned(mode, None)
    with ctx:
        eager = C0.clone()
        g.gemm(mode, tA, tB, eager, 1.25, 0.5)
        torch.cuda.synchronize()
        say(f"[noalloc] capture {mode} {M}x{N}x{K}")
        with torch.cuda.graph(graph, stream=s):
            g.gemm_noalloc(mode, tA, tB, tC, 1.25, 0.5)
    for _ in range(3):
        tC.copy_(C0)
        other = C0.clone()
        g.gemm(mode, tA, tB, other, 0.5, 1.0)     # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(tC, eager)
    st = oracle.check(mode, A, B, C, 1.25, 0.5, tC.cpu().numpy())
    assert st["n_fail"] == 0, st
