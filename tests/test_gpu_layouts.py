"""GPU parity of the operand layouts: C = alpha*op(A)@op(B) + beta*C with
op(A) = A^T (A stored K x M) and/or op(B) = B^T (B stored N x K), through the
_ex entry points of the C ABI, against the CPU oracle given op(A) and op(B)
as plain row-major matrices.  Bound and checks as in test_gpu_parity.py:
every compiled configuration on small aligned, ragged and odd-leading-dimension
shapes (whole output), the 4096^3 workloads on row bands and sampled elements,
and small integers bit-exact.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from workloads import make_inputs, sample_indices, small_integers

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():   # collected on CPU-only hosts, never run there
    pytest.skip("no GPU", allow_module_level=True)

import gemm_tiled_amd as g  # noqa: E402
from tests.gpu_helpers import pinned, say, to_device  # noqa: E402

MODES = ["f32", "f16r"]
LAYOUTS = [(True, False), (False, True), (True, True)]


def _name(ta, tb):
    return ("T" if ta else "N") + ("T" if tb else "N")


def stored(op, t, ld=None):
    """The array a transposed operand is stored in: op^T, row-major, with an
    optional padded leading dimension."""
    if not t:
        return op
    rows, cols = op.shape[1], op.shape[0]
    ld = ld or max(cols, 1)
    buf = np.zeros((rows, ld), dtype=np.float32)
    buf[:, :cols] = op.T
    return buf[:, :cols]


def run_ex(mode, A_op, B_op, C, alpha, beta, ta, tb, lda=None, ldb=None):
    tA = to_device(stored(A_op, ta, lda))
    tB = to_device(stored(B_op, tb, ldb))
    tC = to_device(C)
    g.gemm(mode, tA, tB, tC, alpha, beta, transa=ta, transb=tb)
    torch.cuda.synchronize()
    return tC.cpu().numpy()


def check(mode, A, B, C, alpha, beta, got, rows=None):
    st = oracle.check(mode, np.ascontiguousarray(A), np.ascontiguousarray(B), C, alpha, beta,
                      got, rows=rows)
    assert st["n_fail"] == 0, st


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("ta,tb", LAYOUTS, ids=[_name(*x) for x in LAYOUTS])
def test_every_config_each_layout(mode, ta, tb):
    shapes = [
        (512, 512, 256, {}),
        (300, 200, 150, {}),
        (129, 77, 45, {"lda": 131, "ldb": 47}),   # odd leading dimensions: 4-byte rows
    ]
    for cfg in g.list_configs(mode):
        for (M, N, K, lds) in shapes:
            A, B, C = make_inputs(M, N, K, "uniform", seed=21)
            say(f"[layout] {mode} {_name(ta, tb)} {cfg} {M}x{N}x{K} {lds}")
            with pinned(mode, cfg):
                got = run_ex(mode, A, B, C, 1.5, 0.5, ta, tb, lds.get("lda"), lds.get("ldb"))
            check(mode, A, B, C, 1.5, 0.5, got)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("ta,tb", LAYOUTS, ids=[_name(*x) for x in LAYOUTS])
def test_layout_4096(mode, ta, tb):
    n = 4096
    A, B, C = make_inputs(n, n, n, "uniform", seed=3)
    say(f"[layout] {mode} {_name(ta, tb)} {n}^3 {g.get_config(mode, n, n, n, beta=1.0, transa=ta, transb=tb)}")
    got = run_ex(mode, A, B, C, 1.0, 1.0, ta, tb)
    assert np.isfinite(got).all()
    check(mode, A, B, C, 1.0, 1.0, got, rows=(0, 48))
    check(mode, A, B, C, 1.0, 1.0, got, rows=(n - 48, n))
    r, c = sample_indices(n, n, 2048, seed=1)
    ref, W = oracle.entries(mode, np.ascontiguousarray(A), np.ascontiguousarray(B), C, 1.0, 1.0,
                            r, c)
    err = np.abs(got[r, c].astype(np.float64) - ref)
    assert np.all(err <= oracle.TOL[mode] * W)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("ta,tb", LAYOUTS, ids=[_name(*x) for x in LAYOUTS])
def test_layout_small_integers_exact(mode, ta, tb):
    M, N, K = 1000, 999, 1001
    A, B, C = small_integers(M, N, K, seed=8)
    exact = A.astype(np.float64) @ B.astype(np.float64)
    for alpha, beta in ((1.0, 1.0), (-2.0, 0.5)):
        say(f"[layout exact] {mode} {_name(ta, tb)} {M}x{N}x{K} alpha={alpha} beta={beta}")
        got = run_ex(mode, A, B, C, alpha, beta, ta, tb, lda=M + 3 if ta else None,
                     ldb=K + 1 if tb else None)
        exp = (alpha * exact + beta * C.astype(np.float64)).astype(np.float32)
        assert np.array_equal(got, exp), f"{int((got != exp).sum())} elements differ"


@pytest.mark.parametrize("mode", MODES)
def test_layout_tuner_keys_the_layout(mode):
    M, N, K = 768, 640, 512
    A, B, C = make_inputs(M, N, K, "normal", seed=9)
    tA, tB, tC = to_device(stored(A, True)), to_device(B), to_device(C)
    before = tC.clone()
    say(f"[layout tune] {mode} TN {M}x{N}x{K}")
    g.tune(mode, tA, tB, tC, beta=0.5, transa=True)
    torch.cuda.synchronize()
    assert torch.equal(tC, before)
    assert g.get_config(mode, M, N, K, beta=0.5, transa=True).endswith("source=tuned")
    got = run_ex(mode, A, B, C, 1.0, 0.5, True, False)
    check(mode, A, B, C, 1.0, 0.5, got)
