"""Shapes at the edges of the kernels' own limits, through the C ABI, against
the oracle element by element (every operand's extent stays below 2 GiB):

- leading dimensions too large for the f32 ring's 32-bit copy offsets (lda at
  least 2^20, ldb at least 2^24): a pinned ring configuration runs the call in
  the register-staged kernel of the same tile, and the library's own choice
  is right too;
- a very deep K (2^20) for few rows and columns: split-K slices, the f16r
  configurations that round on load;
- a long ragged K (2^18) under a ragged 300 x 200 output: the masked ring on
  the block of whole tiles plus strips (f32);
- a tall output (2^17 rows, 64 columns, K = 64).
"""
from __future__ import annotations

import pytest

import oracle
from workloads import make_inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():   # collected on CPU-only hosts, never run there
    pytest.skip("no GPU", allow_module_level=True)

import gemm_tiled_amd as g  # noqa: E402
from tests.gpu_helpers import pinned, run, say  # noqa: E402

RING = {"f32": "BM=256 BN=256 BK=16 ST=3 WM=2 WN=4 GM=8",
        "f16r": "BM=256 BN=256 BK=32 ST=5 WM=4 WN=2 GM=8"}


def _check(mode, M, N, K, lds, pin=None, dist="uniform", seed=0):
    A, B, C = make_inputs(M, N, K, dist, seed=seed, **lds)
    for x, ld in ((A, lds.get("lda")), (B, lds.get("ldb")), (C, lds.get("ldc"))):
        assert x.shape[0] * (ld or x.shape[1]) * 4 < 2 ** 31
    plan = g.get_plan(mode, M, N, K, beta=0.5, **lds) if not pin else f"pinned {pin}"
    say(f"[limits] {mode} {M}x{N}x{K} {lds} {plan}")
    if pin:
        with pinned(mode, pin):
            got = run(mode, A, B, C, 1.25, 0.5)
    else:
        got = run(mode, A, B, C, 1.25, 0.5)
    st = oracle.check(mode, A, B, C, 1.25, 0.5, got)
    assert st["n_fail"] == 0, st


@pytest.mark.parametrize("mode", ["f32", "f16r"])
@pytest.mark.parametrize("pin", [False, True])
def test_lda_beyond_the_ring_copy_offsets(mode, pin):
    _check(mode, 256, 512, 256, {"lda": (1 << 20) + 4}, pin=RING[mode] if pin else None, seed=1)


@pytest.mark.parametrize("mode", ["f32", "f16r"])
@pytest.mark.parametrize("pin", [False, True])
def test_ldb_beyond_the_ring_copy_offsets(mode, pin):
    _check(mode, 256, 512, 16, {"ldb": (1 << 24) + 4}, pin=RING[mode] if pin else None, seed=2)


@pytest.mark.parametrize("mode", ["f32", "f16r"])
def test_very_deep_k(mode):
    _check(mode, 64, 64, 1 << 20, {}, dist="normal", seed=3)


@pytest.mark.parametrize("mode", ["f32", "f16r"])
def test_long_ragged_k_under_a_ragged_output(mode):
    _check(mode, 300, 200, (1 << 18) + 5, {}, dist="normal", seed=4)


@pytest.mark.parametrize("mode", ["f32", "f16r"])
def test_tall_output(mode):
    _check(mode, 1 << 17, 64, 64, {}, seed=5)
