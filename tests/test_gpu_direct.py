"""GPU parity tests of the f16r configurations that round the operands to
binary16 as they stage them (KS=3: no packing pass, K split over workgroups
with the last workgroup of a tile adding the slices in order).

Same bound as the other parity tests: |C_gpu - C_ref| <= 4e-5 * W elementwise
against the float64 oracle of the rounded operands; exact results on small
integers; bitwise repeatability (the slice order is fixed).
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from workloads import make_inputs, small_integers

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():   # collected on CPU-only hosts, never run there
    pytest.skip("no GPU", allow_module_level=True)

import gemm_tiled_amd as g  # noqa: E402
from tests.gpu_helpers import pinned, run, say, to_device  # noqa: E402

DIRECT = ["BM=64 BN=64 BK=64 KS=3", "BM=32 BN=64 BK=64 KS=3", "BM=128 BN=128 BK=64 KS=3",
          "BM=64 BN=256 BK=64 KS=3",
          # f32 panels through a ring of direct-to-LDS copies, rounded as read
          "BM=16 BN=128 BK=32 ST=4 WM=1 WN=2 KS=3",
          "BM=32 BN=64 BK=32 ST=4 WM=2 WN=1 KS=3", "BM=32 BN=128 BK=32 ST=4 WM=2 WN=2 KS=3",
          "BM=64 BN=64 BK=32 ST=4 WM=4 WN=1 KS=3", "BM=64 BN=128 BK=32 ST=3 WM=2 WN=2 KS=3",
          "BM=128 BN=128 BK=32 ST=3 WM=4 WN=2 KS=3", "BM=128 BN=256 BK=32 ST=3 WM=2 WN=4 KS=3",
          "BM=256 BN=128 BK=32 ST=3 WM=4 WN=2 KS=3"]
RINGS = [c for c in DIRECT if "ST=" in c]


def assert_parity(A, B, C, alpha, beta, got):
    st = oracle.check("f16r", A, B, C, alpha, beta, got)
    assert st["n_fail"] == 0, st


@pytest.mark.parametrize("cfg", DIRECT)
@pytest.mark.parametrize("M,N,K,lds", [
    (64, 4096, 4096, {}),                           # many slices
    (256, 4096, 4096, {}),                          # fewer slices, whole tiles
    (17, 1000, 4093, {}),                           # ragged everywhere, last slice short
    (300, 520, 2100, {"lda": 2103, "ldb": 523, "ldc": 521}),   # odd lds: 4-byte rows
    (1000, 300, 777, {}),                           # many tile rows, one or two slices
    (33, 256, 64, {}),                              # one panel
])
def test_direct_against_the_oracle(cfg, M, N, K, lds):
    A, B, C = make_inputs(M, N, K, "normal", seed=21, **lds)
    with pinned("f16r", cfg):
        say(f"[direct] {cfg} {M}x{N}x{K} {lds}")
        got = run("f16r", A, B, C, 1.25, -0.5)
        again = run("f16r", A, B, C, 1.25, -0.5)
    assert_parity(A, B, C, 1.25, -0.5, got)
    assert np.array_equal(got.view(np.uint32), again.view(np.uint32))   # fixed slice order


@pytest.mark.parametrize("cfg", RINGS)
@pytest.mark.parametrize("M,N,K,lds", [
    (17, 1000, 4096, {}),                           # ragged M and N (N % 4 == 0), many slices
    (300, 520, 2112, {"lda": 2116, "ldb": 524, "ldc": 521}),   # padded 16-byte rows, odd ldc
    (1000, 300, 800, {}),                           # many tile rows, one or two slices
    (64, 4096, 4096, {}),                           # whole tiles
    (33, 256, 32, {}),                              # one panel
    (130, 2052, 1024, {"ldc": 2056}),               # a column group past N in a ragged tile
])
def test_direct_ring_shapes(cfg, M, N, K, lds):
    """The shapes the f32-panel ring takes itself (16-byte rows, N % 4 == 0,
    K % 32 == 0), ragged in M and N."""
    A, B, C = make_inputs(M, N, K, "normal", seed=25, **lds)
    with pinned("f16r", cfg):
        say(f"[direct ring] {cfg} {M}x{N}x{K} {lds}")
        got = run("f16r", A, B, C, -0.75, 1.5)
        again = run("f16r", A, B, C, -0.75, 1.5)
    assert_parity(A, B, C, -0.75, 1.5, got)
    assert np.array_equal(got.view(np.uint32), again.view(np.uint32))


@pytest.mark.parametrize("cfg", RINGS)
@pytest.mark.parametrize("ldc_pad", [0, 2])
def test_ring32_epilogue_paths(cfg, ldc_pad):
    """The 32-deep ring's epilogue, bit-exact on small integers: a lane's four
    columns as one access when C's rows allow it (ldc % 4 == 0), element by
    element otherwise (ldc = N + 2); f32 C with beta != 0 and with beta = 0
    (NaN in C, never read), binary16 C as the f32 result rounded once."""
    M, N, K = 150, 1000, 1024
    A, B, C = small_integers(M, N, K, seed=26, ldc=N + ldc_pad)
    exact = A.astype(np.float64) @ B.astype(np.float64)
    Cn = np.full((M, N + ldc_pad), np.nan, dtype=np.float32)[:, :N]
    with pinned("f16r", cfg):
        say(f"[ring32 epilogue] {cfg} {M}x{N}x{K} ldc={N + ldc_pad}")
        got = run("f16r", A, B, C, -2.0, 0.5)
        assert np.array_equal(got, (-2.0 * exact + 0.5 * C.astype(np.float64)).astype(np.float32))
        got = run("f16r", A, B, Cn, 1.0, 0.0)
        assert np.array_equal(got, exact.astype(np.float32))
        tA, tB = to_device(A), to_device(B)
        t16 = torch.zeros((M, N + ldc_pad), dtype=torch.float16, device="cuda")[:, :N]
        t16.copy_(torch.from_numpy(C.astype(np.float16)))
        t32 = to_device(C.astype(np.float16).astype(np.float32))
        g.gemm_f16r_f16out(tA, tB, t16, 0.75, -0.25)
        g.gemm("f16r", tA, tB, t32, 0.75, -0.25)
        torch.cuda.synchronize()
    want = t32.cpu().numpy().astype(np.float16)
    assert np.array_equal(t16.cpu().numpy().view(np.uint16), want.view(np.uint16))


@pytest.mark.parametrize("cfg", DIRECT)
@pytest.mark.parametrize("M", [1, 40, 200])
def test_direct_small_integers_exact_and_beta_zero(cfg, M):
    N, K = 2048, 4096
    A, B, C = small_integers(M, N, K, seed=22)
    exact = A.astype(np.float64) @ B.astype(np.float64)
    with pinned("f16r", cfg):
        say(f"[direct exact] {cfg} {M}x{N}x{K}")
        got = run("f16r", A, B, C, -2.0, 0.5)
        assert np.array_equal(got, (-2.0 * exact + 0.5 * C.astype(np.float64)).astype(np.float32))
        Cn = np.full((M, N), np.nan, dtype=np.float32)
        got = run("f16r", A, B, Cn, 1.0, 0.0)
        assert np.array_equal(got, exact.astype(np.float32))


@pytest.mark.parametrize("cfg", DIRECT[:2] + RINGS[:1])
@pytest.mark.parametrize("ta,tb,M,N", [(True, False, 96, 1028), (False, True, 96, 1027),
                                       (True, True, 70, 1027), (True, False, 33, 61),
                                       (False, True, 128, 512)])
def test_direct_layouts(cfg, ta, tb, M, N):
    K = 2052
    A, B, C = make_inputs(M, N, K, "uniform", seed=23)
    tA = to_device(np.ascontiguousarray(A.T) if ta else A)
    tB = to_device(np.ascontiguousarray(B.T) if tb else B)
    tC = to_device(C)
    with pinned("f16r", cfg):
        say(f"[direct layout] {cfg} ta={ta} tb={tb} {M}x{N}x{K}")
        g.gemm("f16r", tA, tB, tC, 0.5, 2.0, transa=ta, transb=tb)
        torch.cuda.synchronize()
    assert_parity(A, B, C, 0.5, 2.0, tC.cpu().numpy())


@pytest.mark.parametrize("cfg", DIRECT)
@pytest.mark.parametrize("M,N,K", [(48, 2048, 4096), (257, 129, 67)])
def test_direct_f16_output(cfg, M, N, K):
    """binary16 C: the f32-output result of the same call, rounded once."""
    A, B, C = make_inputs(M, N, K, "normal", seed=24)
    C16 = C.astype(np.float16)
    tA, tB = to_device(A), to_device(B)
    t16 = torch.from_numpy(C16.copy()).to("cuda")
    t32 = to_device(C16.astype(np.float32))
    with pinned("f16r", cfg):
        say(f"[direct f16-out] {cfg} {M}x{N}x{K}")
        g.gemm_f16r_f16out(tA, tB, t16, 0.75, -0.25)
        g.gemm("f16r", tA, tB, t32, 0.75, -0.25)
        torch.cuda.synchronize()
    want = t32.cpu().numpy().astype(np.float16)
    got = t16.cpu().numpy()
    assert np.array_equal(got.view(np.uint16), want.view(np.uint16))


def test_direct_counters_reset_between_shapes():
    """Calls of different tile counts in a row share the arrival counters: each
    launch must leave every counter it used at zero."""
    cfg = DIRECT[0]
    with pinned("f16r", cfg):
        for (M, N, K) in [(64, 4096, 4096), (200, 1024, 3000), (64, 4096, 4096), (20, 300, 8000)]:
            A, B, C = make_inputs(M, N, K, "normal", seed=M + N)
            say(f"[direct counters] {cfg} {M}x{N}x{K}")
            got = run("f16r", A, B, C, 1.0, 1.0)
            assert_parity(A, B, C, 1.0, 1.0, got)
