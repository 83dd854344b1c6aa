"""Whole-output checks at the full workload sizes, through the C ABI.

1. The workloads with their own data and the library's own configuration:
   every element of C against the oracle's bound (the oracle streams over all
   rows, computing each reference element in float64).
2. Small-integer inputs (entries in [-8, 8]) at 4096^3 f32 and 8192^3 f16r, once
   per tile configuration the tuner can pick there (every compiled
   configuration that does not split K), each pinned: every partial sum is an
   integer below 2^24 (|sum| <= 64 K), so the result is exact in f32 in any
   summation order and the integers are exact in binary16; every element
   must equal the oracle's float64 result bit for bit.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from workloads import WORKLOADS, small_integers, workload_inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():   # collected on CPU-only hosts, never run there
    pytest.skip("no GPU", allow_module_level=True)

import gemm_tiled_amd as g  # noqa: E402
from tests.gpu_helpers import pinned, say, to_device  # noqa: E402


@pytest.mark.parametrize("name", ["f32_4096_a1_b0", "f32_4096_a1_b1", "f16r_4096_a1_b0.5",
                                  "f32_4000x4097x4093_a2_b-1", "f16r_8192_a0.75_b-0.25"])
def test_workload_every_element(name):
    w = WORKLOADS[name]
    A, B, C = workload_inputs(w)
    say(f"[full] {w.name} {g.get_config(w.mode, w.M, w.N, w.K, beta=w.beta)}")
    tA, tB, tC = to_device(A), to_device(B), to_device(C)
    g.gemm(w.mode, tA, tB, tC, w.alpha, w.beta)
    torch.cuda.synchronize()
    got = tC.cpu().numpy()
    del tA, tB, tC
    st = oracle.check(w.mode, A, B, C, w.alpha, w.beta, got)
    say(f"[full] {w.name}: max err/W {st['max_ratio']:.3e}")
    assert st["n_fail"] == 0, st
    assert st["max_ratio"] < 0.1 * oracle.TOL[w.mode], st   # about 100x inside the bound


def _tile_configs(mode):
    return [c for c in g.list_configs(mode) if "KS=" not in c]


_EXACT = {}


def _exact(mode, n, alpha, beta):
    """Small-integer inputs and the oracle's result (exact), computed once."""
    key = (mode, n, alpha, beta)
    if key not in _EXACT:
        A, B, C = small_integers(n, n, n, seed=90 + n % 7)
        say(f"[full exact] oracle {mode} {n}^3")
        ref, _ = oracle.gemm(mode, A, B, C, alpha, beta)
        exp = ref.astype(np.float32)
        assert np.array_equal(exp.astype(np.float64), ref)   # representable: exact in f32
        _EXACT.clear()   # one size at a time (8192^2 float64 is 512 MiB)
        _EXACT[key] = (A, B, C, exp)
    return _EXACT[key]


def _exact_tile(mode, n, alpha, beta, idx):
    cfgs = _tile_configs(mode)
    if idx >= len(cfgs):
        pytest.skip(f"{mode} has {len(cfgs)} tile configurations")
    cfg = cfgs[idx]
    A, B, C, exp = _exact(mode, n, alpha, beta)
    say(f"[full exact] {mode} {n}^3 {cfg}")
    tA, tB, tC = to_device(A), to_device(B), to_device(C)
    with pinned(mode, cfg):
        g.gemm(mode, tA, tB, tC, alpha, beta)
        torch.cuda.synchronize()
    got = tC.cpu().numpy()
    del tA, tB, tC
    bad = got != exp
    assert not bad.any(), f"{cfg}: {int(bad.sum())} elements differ, first at {np.argwhere(bad)[:3]}"


@pytest.mark.parametrize("idx", range(13))
def test_every_f32_tile_exact_at_4096(idx):
    _exact_tile("f32", 4096, 1.0, 1.0, idx)


@pytest.mark.parametrize("idx", range(19))
def test_every_f16r_tile_exact_at_8192(idx):
    _exact_tile("f16r", 8192, 0.75, -0.25, idx)
