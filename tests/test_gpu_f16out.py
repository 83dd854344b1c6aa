"""GPU tests of the f16-output variant of the f16r mode (gemm_f16r_f16out):
operands rounded to binary16, products accumulated in f32, C stored as
binary16 and the f32 epilogue value rounded once to nearest even.

Pins: the result is bit for bit numpy's float16 rounding of the f32-output
call of the same configuration on the same inputs (the two compute the same f32
value); it is inside the oracle's bound widened by half a binary16 ulp; small
integers whose results are exact in binary16 come back exactly.
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

DEV = torch.device("cuda:0")


def run16(A, B, C16, alpha, beta):
    tC = torch.from_numpy(C16.copy()).to(DEV)
    g.gemm_f16r_f16out(to_device(A), to_device(B), tC, alpha, beta)
    torch.cuda.synchronize()
    return tC.cpu().numpy()


def inside_bound(A, B, C16, alpha, beta, got16, rows=None):
    """|C16 - Cref| <= 4e-5 W + 2^-11 (|Cref| + 4e-5 W) + 2^-25: the f16r bound
    plus the final rounding to binary16 (half an ulp, relative 2^-11, or 2^-25
    among subnormals)."""
    C = C16.astype(np.float32)
    r0, r1 = rows or (0, C.shape[0])
    ref, W = oracle.gemm("f16r", A[r0:r1], B, C[r0:r1], alpha, beta)
    err = np.abs(got16[r0:r1].astype(np.float64) - ref)
    tol = oracle.TOL["f16r"] * W
    return np.all(err <= tol + 2.0 ** -11 * (np.abs(ref) + tol) + 2.0 ** -25)


@pytest.mark.parametrize("M,N,K", [(300, 200, 150), (512, 512, 256), (1000, 999, 1001)])
def test_f16out_is_the_rounded_f32_result(M, N, K):
    A, B, C = make_inputs(M, N, K, "normal", seed=31)
    C16 = C.astype(np.float16)
    for alpha, beta in ((1.0, 0.0), (0.75, -0.25)):
        cfg = g.get_config("f16r", M, N, K, beta=beta).split(" source=")[0]
        with pinned("f16r", cfg):
            say(f"[f16-out] {M}x{N}x{K} {cfg} alpha={alpha} beta={beta}")
            got16 = run16(A, B, C16, alpha, beta)
            got32 = run("f16r", A, B, C16.astype(np.float32), alpha, beta)
        assert np.array_equal(got16.view(np.uint16), got32.astype(np.float16).view(np.uint16))
        assert inside_bound(A, B, C16, alpha, beta, got16)


@pytest.mark.parametrize("M,N,K", [(257, 129, 67),     # ragged: masked epilogues
                                   (512, 512, 256)])   # whole tiles: the staged epilogue
def test_f16out_every_config(M, N, K):
    A, B, C = make_inputs(M, N, K, "uniform", seed=32)
    C16 = C.astype(np.float16)
    for cfg in g.list_configs("f16r"):
        with pinned("f16r", cfg):
            say(f"[f16-out] every config {cfg} {M}x{N}x{K}")
            got16 = run16(A, B, C16, 1.5, 0.5)
            got32 = run("f16r", A, B, C16.astype(np.float32), 1.5, 0.5)
        assert inside_bound(A, B, C16, 1.5, 0.5, got16), cfg
        assert np.array_equal(got16.view(np.uint16), got32.astype(np.float16).view(np.uint16)), cfg


def test_f16out_small_integers_exact():
    # entries in [-2, 2], K = 100: |result| <= 2 * 400 + 2 * 2 < 2048, exact in binary16
    M, N, K = 700, 600, 100
    A, B, C = small_integers(M, N, K, lo=-2, hi=2, seed=33)
    exact = 2.0 * (A.astype(np.float64) @ B.astype(np.float64)) - 1.0 * C.astype(np.float64)
    say(f"[f16-out exact] {M}x{N}x{K}")
    got16 = run16(A, B, C.astype(np.float16), 2.0, -1.0)
    assert np.array_equal(got16.astype(np.float64), exact)


def test_f16out_beta_only_and_few_rows():
    A, B, C = make_inputs(16, 4096, 4096, "normal", seed=34)
    C16 = C.astype(np.float16)
    say("[f16-out] alpha = 0")
    got16 = run16(A, B, C16, 0.0, -0.5)
    assert np.array_equal(got16.view(np.uint16),
                          (np.float32(-0.5) * C16.astype(np.float32)).astype(np.float16).view(np.uint16))
    for cfg in ("BM=32 BN=128 BK=32 KS=1", "BM=16 BN=64 BK=64 KS=2"):
        say(f"[f16-out] 16 rows, {cfg}")
        with pinned("f16r", cfg):
            got16 = run16(A, B, C16, 1.0, 0.25)
        assert inside_bound(A, B, C16, 1.0, 0.25, got16)
    assert "KS=2" in g.get_config("f16r", 16, 4096, 4096, beta=0.25)


@pytest.mark.parametrize("ta,tb", [(True, False), (False, True), (True, True)],
                         ids=["TN", "NT", "TT"])
@pytest.mark.parametrize("M,cfg", [
    (16, None),                                           # the library's choice (B^T: panel ring)
    (40, "BM=32 BN=128 BK=32 ST=4 WM=2 WN=2 KS=3"),       # f32-panel ring, ragged rows
    (200, "BM=128 BN=256 BK=32 ST=3 WM=2 WN=4 KS=3"),
])
def test_f16out_layouts_on_the_panel_ring(ta, tb, M, cfg):
    """The binary16 epilogues of the f32-panel ring in the transposed layouts
    (the block-layout epilogue with B stored N x K, the column-dealt one
    otherwise): bit for bit the rounding of the f32-output call, inside the
    widened bound."""
    N, K = 1000, 2048
    A, B, C = make_inputs(M, N, K, "normal", seed=35)
    C16 = C.astype(np.float16)
    tA = to_device(np.ascontiguousarray(A.T) if ta else A)
    tB = to_device(np.ascontiguousarray(B.T) if tb else B)
    spec = cfg or g.get_config("f16r", M, N, K, beta=0.5, transa=ta, transb=tb).split(" source=")[0]
    assert "KS=3" in spec or not tb, spec
    with pinned("f16r", spec):
        say(f"[f16-out layout] ta={ta} tb={tb} {M}x{N}x{K} {spec}")
        t16 = torch.from_numpy(C16.copy()).to(DEV)
        g.gemm_f16r_f16out(tA, tB, t16, 1.25, 0.5, transa=ta, transb=tb)
        t32 = to_device(C16.astype(np.float32))
        g.gemm("f16r", tA, tB, t32, 1.25, 0.5, transa=ta, transb=tb)
        torch.cuda.synchronize()
    got16, got32 = t16.cpu().numpy(), t32.cpu().numpy()
    assert np.array_equal(got16.view(np.uint16), got32.astype(np.float16).view(np.uint16))
    assert inside_bound(A, B, C16, 1.25, 0.5, got16)
