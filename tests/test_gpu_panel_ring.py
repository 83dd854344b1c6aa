"""GPU parity tests of the f32-panel ring in the f32 mode (KS=3, BK=32: f32
panels through direct-to-LDS copies, multiplied as read on the f32 matrix
instruction, K split over workgroups with the last workgroup of a tile adding
the slices in order).

Same bound as the other f32 parity tests against the float64 oracle; exact
results on small integers; bitwise repeatability (the slice order is fixed);
the shapes the ring does not take (K % 32 != 0, unaligned rows, N % 4 != 0
for B stored K x N, M % 4 != 0 for A stored K x M) handed to the split-K
tiles.  The transposed layouts of the ring are tested in
test_gpu_layouts.py.
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

RINGS = ["BM=16 BN=128 BK=32 ST=4 WM=1 WN=2 KS=3",
         "BM=32 BN=64 BK=32 ST=4 WM=2 WN=1 KS=3", "BM=32 BN=128 BK=32 ST=4 WM=2 WN=2 KS=3",
         "BM=64 BN=64 BK=32 ST=4 WM=4 WN=1 KS=3", "BM=64 BN=128 BK=32 ST=3 WM=2 WN=2 KS=3",
         "BM=128 BN=128 BK=32 ST=3 WM=4 WN=2 KS=3"]


def assert_parity(A, B, C, alpha, beta, got):
    st = oracle.check("f32", A, B, C, alpha, beta, got)
    assert st["n_fail"] == 0, st


@pytest.mark.parametrize("cfg", RINGS)
@pytest.mark.parametrize("M,N,K,lds", [
    (17, 1000, 4096, {}),                           # ragged M and N (N % 4 == 0), many slices
    (300, 520, 2112, {"lda": 2116, "ldb": 524, "ldc": 521}),   # padded 16-byte rows, odd ldc
    (1000, 300, 800, {}),                           # many tile rows, one or two slices
    (64, 4096, 4096, {}),                           # whole tiles
    (33, 256, 32, {}),                              # one panel
    (130, 2052, 1024, {"ldc": 2056}),               # a column group past N in a ragged tile
])
def test_panel_ring_against_the_oracle(cfg, M, N, K, lds):
    A, B, C = make_inputs(M, N, K, "normal", seed=31, **lds)
    with pinned("f32", cfg):
        say(f"[panel ring f32] {cfg} {M}x{N}x{K} {lds}")
        got = run("f32", A, B, C, -0.75, 1.5)
        again = run("f32", A, B, C, -0.75, 1.5)
    assert_parity(A, B, C, -0.75, 1.5, got)
    assert np.array_equal(got.view(np.uint32), again.view(np.uint32))


@pytest.mark.parametrize("cfg", RINGS)
@pytest.mark.parametrize("M,ldc_pad", [(1, 0), (40, 2), (200, 0)])
def test_panel_ring_small_integers_exact(cfg, M, ldc_pad):
    """Exact on small integers, with the epilogue's vector path (ldc % 4 == 0)
    and its element-by-element one (ldc = N + 2); beta = 0 never reads C (NaN
    there)."""
    N, K = 2048, 4096
    A, B, C = small_integers(M, N, K, seed=32, ldc=N + ldc_pad)
    exact = A.astype(np.float64) @ B.astype(np.float64)
    Cn = np.full((M, N + ldc_pad), np.nan, dtype=np.float32)[:, :N]
    with pinned("f32", cfg):
        say(f"[panel ring f32 exact] {cfg} {M}x{N}x{K} ldc={N + ldc_pad}")
        got = run("f32", A, B, C, -2.0, 0.5)
        assert np.array_equal(got, (-2.0 * exact + 0.5 * C.astype(np.float64)).astype(np.float32))
        got = run("f32", A, B, Cn, 1.0, 0.0)
        assert np.array_equal(got, exact.astype(np.float32))


@pytest.mark.parametrize("M,N,K,lds,trans", [
    (64, 1024, 4080, {}, (False, False)),           # K % 32 != 0
    (64, 1022, 2048, {}, (False, False)),           # N % 4 != 0
    (64, 1024, 2048, {"lda": 2049}, (False, False)),   # rows not 16-byte aligned
    (62, 1024, 2048, {}, (True, False)),            # A stored K x M with M % 4 != 0
    (64, 1024, 2048, {"ldb": 2049}, (False, True)),    # B stored N x K, rows not 16-byte aligned
])
def test_panel_ring_hands_other_shapes_to_split_k(M, N, K, lds, trans):
    ta, tb = trans
    A, B, C = make_inputs(M, N, K, "uniform", seed=33, **({} if tb else lds))

    def stored(x, t, ld):
        if not t:
            return to_device(x)
        buf = np.zeros((x.shape[1], ld or x.shape[0]), dtype=np.float32)
        buf[:, :x.shape[0]] = x.T
        return torch.from_numpy(buf).to("cuda")[:, :x.shape[0]]
    tA = stored(A, ta, lds.get("lda") if ta else None)
    tB = stored(B, tb, lds.get("ldb") if tb else None)
    tC = to_device(C)
    with pinned("f32", RINGS[0]):
        say(f"[panel ring f32 hand-off] {M}x{N}x{K} {lds} ta={ta} tb={tb}")
        g.gemm("f32", tA, tB, tC, 0.5, 2.0, transa=ta, transb=tb)
        torch.cuda.synchronize()
    assert_parity(A, B, C, 0.5, 2.0, tC.cpu().numpy())


def test_panel_ring_counters_reset_between_shapes():
    """Calls of different tile counts in a row share the arrival counters: each
    launch must leave every counter it used at zero."""
    with pinned("f32", RINGS[3]):
        for (M, N, K) in [(64, 4096, 4096), (200, 1024, 3008), (64, 4096, 4096), (20, 300, 8000)]:
            A, B, C = make_inputs(M, N, K, "normal", seed=M + N)
            say(f"[panel ring f32 counters] {M}x{N}x{K}")
            got = run("f32", A, B, C, 1.0, 1.0)
            assert_parity(A, B, C, 1.0, 1.0, got)
