"""GPU parity tests: the HIP path through the C ABI against the CPU oracle.

Bound (both modes): |C_gpu - C_ref| <= tol * W elementwise, with
W = |alpha|*(|r(A)||r(B)|)_ij + |beta||C_ij| and tol = 1e-5 (f32), 4e-5 (f16r).
Small shapes are checked element by element over the whole output; the full
workload sizes are checked on bands of whole rows at both edges plus sampled
elements the oracle computes one by one, and through properties that hold at
any size (exact small-integer results, identity, alpha = 0, determinism).
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from workloads import WORKLOADS, make_inputs, sample_indices, small_integers, workload_inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():   # collected on CPU-only hosts, never run there
    pytest.skip("no GPU", allow_module_level=True)

import gemm_tiled_amd as g  # noqa: E402
from tests.gpu_helpers import pinned, run, say, to_device  # noqa: E402

TOL = oracle.TOL
MODES = ["f32", "f16r"]


def assert_parity(mode, A, B, C, alpha, beta, got, rows=None):
    st = oracle.check(mode, A, B, C, alpha, beta, got, rows=rows)
    assert st["n_fail"] == 0, st
    return st


def assert_sampled(mode, A, B, C, alpha, beta, got, n=4096, seed=1):
    M, N = got.shape
    r, c = sample_indices(M, N, n, seed)
    ref, W = oracle.entries(mode, A, B, C, alpha, beta, r, c)
    err = np.abs(got[r, c].astype(np.float64) - ref)
    bad = ~(err <= TOL[mode] * W)
    assert not bad.any(), (int(bad.sum()), r[bad][:5], c[bad][:5])
    return float(np.max(err / np.where(W > 0, W, 1.0)))


# ---------------------------------------------------------------------------
# Every compiled tile configuration, aligned and ragged (the tuner may pick any
# of them, so each must be right on its own).
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("mode", MODES)
def test_every_config_aligned_and_ragged(mode):
    shapes = [
        (512, 512, 256, {}),                                    # whole tiles
        (512, 512, 256, {"ldc": 514}),                          # whole tiles, C rows 8-byte aligned
        (300, 200, 150, {}),                                    # ragged in M, N, K
        (257, 129, 67, {"lda": 68, "ldb": 132, "ldc": 131}),    # ragged, padded lds
        (129, 77, 45, {"lda": 47, "ldb": 79, "ldc": 77}),       # odd lds: 4-byte rows
    ]
    for cfg in g.list_configs(mode):
        for (M, N, K, lds) in shapes:
            A, B, C = make_inputs(M, N, K, "uniform", seed=11, **lds)
            say(f"[parity] {mode} {cfg} {M}x{N}x{K} {lds}")
            with pinned(mode, cfg):
                got = run(mode, A, B, C, 1.5, 0.5)
            assert_parity(mode, A, B, C, 1.5, 0.5, got)


# ---------------------------------------------------------------------------
# The five workloads, at their full sizes, with the library's own choice of
# configuration (heuristic) and after tuning.
# ---------------------------------------------------------------------------

def test_workload_f32_256():
    w = WORKLOADS["f32_256_a1.5_b0.5"]
    A, B, C = workload_inputs(w)
    say(f"[parity] {w.name}")
    got = run(w.mode, A, B, C, w.alpha, w.beta)
    assert_parity(w.mode, A, B, C, w.alpha, w.beta, got)


@pytest.mark.parametrize("name", ["f32_4096_a1_b0", "f32_4096_a1_b1", "f16r_4096_a1_b0.5",
                                  "f32_4000x4097x4093_a2_b-1"])
def test_workload_full_size(name):
    w = WORKLOADS[name]
    A, B, C = workload_inputs(w)
    say(f"[parity] {w.name} {g.get_config(w.mode, w.M, w.N, w.K, beta=w.beta)}")
    got = run(w.mode, A, B, C, w.alpha, w.beta)
    assert np.isfinite(got).all()
    assert_parity(w.mode, A, B, C, w.alpha, w.beta, got, rows=(0, 96))
    assert_parity(w.mode, A, B, C, w.alpha, w.beta, got, rows=(w.M - 96, w.M))
    assert_sampled(w.mode, A, B, C, w.alpha, w.beta, got)


def test_workload_f16r_8192():
    w = WORKLOADS["f16r_8192_a0.75_b-0.25"]
    A, B, C = workload_inputs(w)
    say(f"[parity] {w.name} {g.get_config(w.mode, w.M, w.N, w.K, beta=w.beta)}")
    got = run(w.mode, A, B, C, w.alpha, w.beta)
    assert np.isfinite(got).all()
    assert_parity(w.mode, A, B, C, w.alpha, w.beta, got, rows=(0, 32))
    assert_parity(w.mode, A, B, C, w.alpha, w.beta, got, rows=(w.M - 32, w.M))
    assert_sampled(w.mode, A, B, C, w.alpha, w.beta, got, n=4096)


# ---------------------------------------------------------------------------
# The split-K configuration (KS=1) for few rows of C: K is cut into slices
# whose partial tiles a second pass adds in order, then alpha and beta.  With
# K = 4096 (or the ragged 4093) and a handful of tiles, every case below runs
# several slices.  In the f16r mode it rounds the operands as it loads them.
# ---------------------------------------------------------------------------

SPLITK = "BM=32 BN=128 BK=32 KS=1"


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("M,N,K,lds", [
    (1, 4096, 4096, {}),
    (7, 1000, 4093, {}),
    (64, 4096, 4096, {}),
    (33, 515, 2049, {"lda": 2051, "ldb": 517, "ldc": 516}),   # odd lds, ragged everything
])
def test_splitk_against_the_oracle(mode, M, N, K, lds):
    A, B, C = make_inputs(M, N, K, "normal", seed=12, **lds)
    with pinned(mode, SPLITK):
        say(f"[split-K] {mode} {M}x{N}x{K} {lds}")
        got = run(mode, A, B, C, 1.25, -0.5)
        again = run(mode, A, B, C, 1.25, -0.5)
    assert_parity(mode, A, B, C, 1.25, -0.5, got)
    assert np.array_equal(got.view(np.uint32), again.view(np.uint32))   # fixed slice order


@pytest.mark.parametrize("mode", MODES)
def test_splitk_small_integers_exact_and_beta_zero(mode):
    M, N, K = 5, 4096, 4096
    A, B, C = small_integers(M, N, K, seed=13)
    exact = A.astype(np.float64) @ B.astype(np.float64)
    with pinned(mode, SPLITK):
        say(f"[split-K exact] {mode} {M}x{N}x{K}")
        got = run(mode, A, B, C, -2.0, 0.5)
        assert np.array_equal(got, (-2.0 * exact + 0.5 * C.astype(np.float64)).astype(np.float32))
        Cn = np.full((M, N), np.nan, dtype=np.float32)
        got = run(mode, A, B, Cn, 1.0, 0.0)
        assert np.array_equal(got, exact.astype(np.float32))


ROWS = "BM=16 BN=64 BK=64 KS=2"


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("M,N,K,lds", [
    (1, 4096, 4096, {}),
    (16, 4096, 4096, {}),
    (17, 1000, 4093, {}),                     # 32-row group, ragged K and N
    (64, 4096, 4096, {}),
    (65, 516, 777, {"lda": 779, "ldc": 517}),   # two 64-row groups, odd lda/ldc
    (5, 4100, 300, {"ldb": 4104}),            # one slice: the epilogue in the kernel
    (3, 514, 1024, {}),                       # N % 4 != 0: falls back to split-K
])
def test_rows_against_the_oracle(mode, M, N, K, lds):
    A, B, C = make_inputs(M, N, K, "normal", seed=15, **lds)
    with pinned(mode, ROWS):
        say(f"[rows] {mode} {M}x{N}x{K} {lds}")
        got = run(mode, A, B, C, 1.25, -0.5)
        again = run(mode, A, B, C, 1.25, -0.5)
    assert_parity(mode, A, B, C, 1.25, -0.5, got)
    assert np.array_equal(got.view(np.uint32), again.view(np.uint32))   # fixed slice order


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("M", [1, 2, 9, 32, 48])
def test_rows_small_integers_exact_and_beta_zero(mode, M):
    N, K = 2048, 4096
    A, B, C = small_integers(M, N, K, seed=16)
    exact = A.astype(np.float64) @ B.astype(np.float64)
    with pinned(mode, ROWS):
        say(f"[rows exact] {mode} {M}x{N}x{K}")
        got = run(mode, A, B, C, -2.0, 0.5)
        assert np.array_equal(got, (-2.0 * exact + 0.5 * C.astype(np.float64)).astype(np.float32))
        Cn = np.full((M, N), np.nan, dtype=np.float32)
        got = run(mode, A, B, Cn, 1.0, 0.0)
        assert np.array_equal(got, exact.astype(np.float32))


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("ta,tb,N", [(True, False, 1028), (False, True, 1028), (True, True, 1028),
                                     (False, True, 1027), (True, True, 61)])
def test_rows_layouts(mode, ta, tb, N):
    M, K = 24, 2052
    A, B, C = make_inputs(M, N, K, "uniform", seed=17)
    tA = to_device(np.ascontiguousarray(A.T) if ta else A)
    tB = to_device(np.ascontiguousarray(B.T) if tb else B)
    tC = to_device(C)
    with pinned(mode, ROWS):
        say(f"[rows layout] {mode} ta={ta} tb={tb} {M}x{N}x{K}")  # B^T: any N
        g.gemm(mode, tA, tB, tC, 0.5, 2.0, transa=ta, transb=tb)
        torch.cuda.synchronize()
    assert_parity(mode, A, B, C, 0.5, 2.0, tC.cpu().numpy())


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("M", [1, 2])
@pytest.mark.parametrize("ta,tb,N", [(False, False, 1028), (True, False, 1028), (False, True, 1027),
                                     (True, True, 1027)])
def test_rows_vector_form(mode, M, ta, tb, N):
    """One or two rows with K a multiple of 64 take the vector-FMA form."""
    K = 2048
    A, B, C = make_inputs(M, N, K, "normal", seed=19)
    tA = to_device(np.ascontiguousarray(A.T) if ta else A)
    tB = to_device(np.ascontiguousarray(B.T) if tb else B)
    tC = to_device(C)
    with pinned(mode, ROWS):
        say(f"[rows vector] {mode} M={M} ta={ta} tb={tb} {M}x{N}x{K}")
        g.gemm(mode, tA, tB, tC, -0.75, 0.5, transa=ta, transb=tb)
        torch.cuda.synchronize()
    assert_parity(mode, A, B, C, -0.75, 0.5, tC.cpu().numpy())


# The few-columns form of the same configuration: C with at most 16 columns
# and more rows runs as C^T = op(B)^T op(A)^T on the few-rows kernel, which
# then streams A, and stores C transposed.
@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("M,N,K,lds", [
    (4096, 1, 4096, {}),                            # one column (C^T: the vector form)
    (4096, 16, 4096, {}),
    (1000, 7, 1000, {}),                            # ragged M, odd N, K tail
    (4100, 12, 1024, {"lda": 1028, "ldc": 13}),     # padded lda, ldc past N
    (17, 16, 100, {}),                              # just past the few-rows sizes
    (300, 3, 64, {"ldb": 5}),                       # odd ldb: B read element by element
])
def test_columns_against_the_oracle(mode, M, N, K, lds):
    A, B, C = make_inputs(M, N, K, "normal", seed=20, **lds)
    with pinned(mode, ROWS):
        plan = g.get_plan(mode, M, N, K, beta=-0.5, **lds)
        assert plan.startswith("form=columns"), plan
        say(f"[columns] {mode} {M}x{N}x{K} {lds}")
        got = run(mode, A, B, C, 1.25, -0.5)
        again = run(mode, A, B, C, 1.25, -0.5)
    assert_parity(mode, A, B, C, 1.25, -0.5, got)
    assert np.array_equal(got.view(np.uint32), again.view(np.uint32))   # fixed slice order


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("N", [1, 2, 9, 16])
def test_columns_small_integers_exact_and_beta_zero(mode, N):
    M, K = 2048, 4096
    A, B, C = small_integers(M, N, K, seed=21)
    exact = A.astype(np.float64) @ B.astype(np.float64)
    with pinned(mode, ROWS):
        say(f"[columns exact] {mode} {M}x{N}x{K}")
        got = run(mode, A, B, C, -2.0, 0.5)
        assert np.array_equal(got, (-2.0 * exact + 0.5 * C.astype(np.float64)).astype(np.float32))
        Cn = np.full((M, N), np.nan, dtype=np.float32)
        got = run(mode, A, B, Cn, 1.0, 0.0)
        assert np.array_equal(got, exact.astype(np.float32))


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("ta,tb", [(True, False), (False, True), (True, True)])
@pytest.mark.parametrize("N", [1, 13])
def test_columns_layouts(mode, ta, tb, N):
    M, K = 2052, 1028
    A, B, C = make_inputs(M, N, K, "uniform", seed=22)
    tA = to_device(np.ascontiguousarray(A.T) if ta else A)
    tB = to_device(np.ascontiguousarray(B.T) if tb else B)
    tC = to_device(C)
    with pinned(mode, ROWS):
        say(f"[columns layout] {mode} ta={ta} tb={tb} {M}x{N}x{K}")
        g.gemm(mode, tA, tB, tC, 0.5, 2.0, transa=ta, transb=tb)
        torch.cuda.synchronize()
    assert_parity(mode, A, B, C, 0.5, 2.0, tC.cpu().numpy())


def test_columns_f16_output():
    M, N, K = 2048, 12, 4096
    A, B, C = make_inputs(M, N, K, "normal", seed=23)
    C16 = C.astype(np.float16)
    tA, tB = to_device(A), to_device(B)
    t16 = torch.from_numpy(C16.copy()).to("cuda")
    t32 = to_device(C16.astype(np.float32))
    with pinned("f16r", ROWS):
        say(f"[columns f16-out] {M}x{N}x{K}")
        g.gemm_f16r_f16out(tA, tB, t16, 0.75, -0.25)
        g.gemm("f16r", tA, tB, t32, 0.75, -0.25)
        torch.cuda.synchronize()
    want = t32.cpu().numpy().astype(np.float16)
    got = t16.cpu().numpy()
    assert np.array_equal(got.view(np.uint16), want.view(np.uint16))


# The few-columns form of the f32-panel ring's 16-row tile: C with at most 16
# columns and more rows, A stored M x K, runs as C^T = op(B)^T op(A)^T on the
# ring (op(A)^T read as B^T, whole rows per copy) with C stored transposed.
PR16 = "BM=16 BN=128 BK=32 ST=4 WM=1 WN=2 KS=3"


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("M,N,K,lds,tb", [
    (4096, 16, 4096, {}, False),
    (4096, 4, 4096, {}, False),
    (1000, 8, 1024, {}, False),                             # ragged M (a partial 128-column tile)
    (4100, 12, 1024, {"lda": 1028, "ldc": 13}, False),      # padded lda, odd ldc: element stores
    (300, 3, 64, {}, True),                                 # B stored N x K: any N
    (2052, 13, 2048, {"ldc": 16}, True),
])
def test_panel_ring_columns_against_the_oracle(mode, M, N, K, lds, tb):
    A, B, C = make_inputs(M, N, K, "normal", seed=24, **lds)
    tA = to_device(A)
    tB = to_device(np.ascontiguousarray(B.T) if tb else B)
    tC0 = to_device(C)
    with pinned(mode, PR16):
        plan = g.get_plan(mode, M, N, K, beta=-0.5, transb=tb, **lds)
        assert plan.split()[0] in ("form=panel-ring-columns", "form=round-on-load-columns"), plan
        say(f"[panel-ring columns] {mode} tb={tb} {M}x{N}x{K} {lds}")
        outs = []
        for _ in range(2):
            tC = tC0.clone()
            g.gemm(mode, tA, tB, tC, 1.25, -0.5, transb=tb)
            torch.cuda.synchronize()
            outs.append(tC.cpu().numpy())
    assert_parity(mode, A, B, C, 1.25, -0.5, outs[0])
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("N", [4, 16])
def test_panel_ring_columns_small_integers_exact_and_beta_zero(mode, N):
    M, K = 2048, 4096
    A, B, C = small_integers(M, N, K, seed=25)
    exact = A.astype(np.float64) @ B.astype(np.float64)
    with pinned(mode, PR16):
        assert g.get_plan(mode, M, N, K, beta=0.5).split()[0].endswith("-columns")
        say(f"[panel-ring columns exact] {mode} {M}x{N}x{K}")
        got = run(mode, A, B, C, -2.0, 0.5)
        assert np.array_equal(got, (-2.0 * exact + 0.5 * C.astype(np.float64)).astype(np.float32))
        Cn = np.full((M, N), np.nan, dtype=np.float32)
        got = run(mode, A, B, Cn, 1.0, 0.0)
        assert np.array_equal(got, exact.astype(np.float32))


def test_panel_ring_columns_f16_output():
    M, N, K = 2048, 12, 4096
    A, B, C = make_inputs(M, N, K, "normal", seed=26)
    C16 = C.astype(np.float16)
    tA, tB = to_device(A), to_device(B)
    t16 = torch.from_numpy(C16.copy()).to("cuda")
    t32 = to_device(C16.astype(np.float32))
    with pinned("f16r", PR16):
        say(f"[panel-ring columns f16-out] {M}x{N}x{K}")
        g.gemm_f16r_f16out(tA, tB, t16, 0.75, -0.25)
        g.gemm("f16r", tA, tB, t32, 0.75, -0.25)
        torch.cuda.synchronize()
    want = t32.cpu().numpy().astype(np.float16)
    got = t16.cpu().numpy()
    assert np.array_equal(got.view(np.uint16), want.view(np.uint16))


def test_rows_f16_output():
    M, N, K = 12, 2048, 4096
    A, B, C = make_inputs(M, N, K, "normal", seed=18)
    C16 = C.astype(np.float16)
    tA, tB = to_device(A), to_device(B)
    t16 = torch.from_numpy(C16.copy()).to("cuda")
    t32 = to_device(C16.astype(np.float32))
    with pinned("f16r", ROWS):
        say(f"[rows f16-out] {M}x{N}x{K}")
        g.gemm_f16r_f16out(tA, tB, t16, 0.75, -0.25)
        g.gemm("f16r", tA, tB, t32, 0.75, -0.25)
        torch.cuda.synchronize()
    want = t32.cpu().numpy().astype(np.float16)
    got = t16.cpu().numpy()
    assert np.array_equal(got.view(np.uint16), want.view(np.uint16))


def test_splitk_is_the_default_for_few_rows():
    for mode in MODES:
        assert "KS=2" in g.get_config(mode, 1, 4096, 4096)
        assert "KS=2" in g.get_config(mode, 16, 4096, 4096)
        assert "KS=" not in g.get_config(mode, 4096, 4096, 4096)
    # f32: the f32-panel ring up to 256 rows where it takes the shape, else
    # the split-K tiles up to 128 rows
    assert g.get_config("f32", 17, 4096, 4096).startswith("BM=32 BN=128 BK=32 ST=4")
    assert g.get_config("f32", 64, 4096, 4096).startswith("BM=64 BN=64 BK=32 ST=4")
    assert g.get_config("f32", 256, 4096, 4096).startswith("BM=64 BN=128 BK=32 ST=3")
    assert all("KS=3" in g.get_config("f32", m, 4096, 4096) for m in (17, 64, 256))
    assert "KS=" not in g.get_config("f32", 257, 4096, 4096)
    assert "KS=1" in g.get_config("f32", 64, 4096, 4080)
    # f16r: the configurations that round on load -- the f32-panel ring up to
    # 512 rows where it takes the shape (K % 32 == 0; up to 1024 rows for a
    # small N x K), else the register-staged one up to 384 rows
    assert g.get_config("f16r", 17, 4096, 4096).startswith("BM=32 BN=64 BK=32")
    assert g.get_config("f16r", 64, 4096, 4096).startswith("BM=32 BN=64 BK=32")
    assert g.get_config("f16r", 128, 4096, 4096).startswith("BM=64 BN=64 BK=32")
    assert g.get_config("f16r", 256, 4096, 4096).startswith("BM=128 BN=128 BK=32")
    assert g.get_config("f16r", 512, 4096, 4096).startswith("BM=128 BN=256 BK=32")
    assert g.get_config("f16r", 512, 2048, 2048).startswith("BM=128 BN=128 BK=32")
    assert g.get_config("f16r", 1024, 1024, 1024).startswith("BM=64 BN=64 BK=32")
    assert all("KS=3" in g.get_config("f16r", m, 4096, 4096) for m in (17, 64, 384, 512))
    assert "KS=" not in g.get_config("f16r", 513, 4096, 4096)
    assert g.get_config("f16r", 64, 4096, 4080).startswith("BM=64 BN=64 BK=64")
    assert g.get_config("f16r", 384, 4096, 4080).startswith("BM=128 BN=128 BK=64")
    assert "KS=" not in g.get_config("f16r", 385, 4096, 4080)


# ---------------------------------------------------------------------------
# Exact results: small integers make every partial sum exact in f32 in any
# order, so the GPU must match the exact product bit for bit (both modes: the
# integers are exact in f16 too).  The exact product comes from a float64
# matrix product, exact here because every partial sum is below 2^53.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("mode,M,N,K,lds", [
    ("f32", 256, 256, 256, {}),
    ("f16r", 256, 256, 256, {}),
    ("f32", 4096, 4096, 4096, {}),
    ("f16r", 4096, 4096, 4096, {}),
    ("f32", 4000, 4097, 4093, {}),
    ("f16r", 4000, 4097, 4093, {}),
    ("f32", 1000, 999, 1001, {"lda": 1004, "ldb": 1001, "ldc": 1003}),
])
def test_small_integers_exact(mode, M, N, K, lds):
    A, B, C = small_integers(M, N, K, seed=5, **lds)
    exact_p = A.astype(np.float64) @ B.astype(np.float64)
    for alpha, beta in ((1.0, 1.0), (2.0, -1.0), (-1.0, 0.5), (0.5, 0.0)):
        say(f"[exact] {mode} {M}x{N}x{K} {lds} alpha={alpha} beta={beta}")
        got = run(mode, A, B, C, alpha, beta)
        exp = (alpha * exact_p + beta * C.astype(np.float64)).astype(np.float32)
        assert np.array_equal(got, exp), f"{int((got != exp).sum())} elements differ"


# ---------------------------------------------------------------------------
# Closed forms.
# ---------------------------------------------------------------------------

def _rounding_probe_matrix(rows, cols, seed):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal(size=(rows, cols)).astype(np.float32)
    specials = np.array([1 + 2 ** -11, 1 + 3 * 2 ** -11, -(1 + 2 ** -11), 2 ** -24, 2 ** -25,
                         1.5 * 2 ** -24, 2.5 * 2 ** -24, 2 ** -14 - 2 ** -25, 65504.0, 65519.0,
                         -65519.0, 0.1, -0.3, 1e-6, 3.0e-5, 6.0e-8], dtype=np.float32)
    X.ravel()[: specials.size] = specials
    # plus a band of values right at f16 ties across many binades
    tie = (np.float32(1.0) + np.float32(2 ** -11)) * (2.0 ** rng.integers(-14, 15, size=cols))
    X[-1, :] = tie.astype(np.float32) * rng.choice([-1, 1], size=cols)
    return X


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("n,N", [(64, 96), (300, 517)])
def test_identity_returns_the_rounded_operand(mode, n, N):
    """A = I: C = r(B) exactly at alpha=1, beta=0; B = I likewise gives r(A).
    In f16r mode r is round-to-nearest-even to binary16, checked bit for bit
    against numpy's conversion, including ties and subnormals."""
    B = _rounding_probe_matrix(n, N, seed=1)
    I = np.eye(n, dtype=np.float32)
    say(f"[identity] {mode} A=I {n}x{N}")
    got = run(mode, I, B, np.zeros((n, N), np.float32), 1.0, 0.0)
    exp = B.astype(np.float16).astype(np.float32) if mode == "f16r" else B
    # a signed zero may come back as +0 (adding zero products); compare with -0 folded to +0
    assert np.array_equal((got + np.float32(0)).view(np.uint32),
                          (exp + np.float32(0)).view(np.uint32))
    A = _rounding_probe_matrix(N, n, seed=2)
    say(f"[identity] {mode} B=I {N}x{n}")
    got = run(mode, A, I, np.zeros((N, n), np.float32), 1.0, 0.0)
    exp = A.astype(np.float16).astype(np.float32) if mode == "f16r" else A
    assert np.array_equal((got + np.float32(0)).view(np.uint32),
                          (exp + np.float32(0)).view(np.uint32))


@pytest.mark.parametrize("mode", MODES)
def test_alpha_zero_and_k_zero_scale_c_exactly(mode):
    A, B, C = make_inputs(333, 444, 55, "normal", seed=3)
    say(f"[closed form] {mode} alpha=0")
    got = run(mode, A, B, C, 0.0, -0.75)
    assert np.array_equal(got, (np.float32(-0.75) * C).astype(np.float32))
    # K = 0: the product term is empty; A and B are not read (NULL is valid)
    tC = to_device(C)
    say(f"[closed form] {mode} K=0")
    fn = g.lib().gemm_f32 if mode == "f32" else g.lib().gemm_f16r_f32acc
    st = fn(333, 444, 0, 1.0, None, 1, None, 444, 2.0, tC.data_ptr(), tC.stride(0), None)
    torch.cuda.synchronize()
    assert st == 0
    assert np.array_equal(tC.cpu().numpy(), (np.float32(2.0) * C).astype(np.float32))


@pytest.mark.parametrize("mode", MODES)
def test_beta_zero_does_not_read_c(mode):
    A, B, _ = make_inputs(300, 260, 70, "uniform", seed=4)
    C = np.full((300, 260), np.nan, dtype=np.float32)
    C[::3, ::5] = np.inf
    say(f"[closed form] {mode} beta=0 with NaN/inf in C")
    got = run(mode, A, B, C, 1.25, 0.0)
    assert np.isfinite(got).all()
    assert_parity(mode, A, B, C, 1.25, 0.0, got)
    # alpha = 0 and beta = 0: zeros, C not read
    got = run(mode, A, B, C, 0.0, 0.0)
    assert np.array_equal(got, np.zeros_like(got))


@pytest.mark.parametrize("mode", MODES)
def test_all_ones_a_gives_column_sums(mode):
    rng = np.random.default_rng(6)
    M, N, K = 200, 333, 1000
    B = rng.integers(-100, 101, size=(K, N)).astype(np.float32)
    A = np.ones((M, K), dtype=np.float32)
    say(f"[closed form] {mode} all-ones A")
    got = run(mode, A, B, np.zeros((M, N), np.float32), 1.0, 0.0)
    colsum = B.astype(np.int64).sum(axis=0).astype(np.float32)
    assert np.array_equal(got, np.broadcast_to(colsum, (M, N)))


# ---------------------------------------------------------------------------
# Edge cases and brute force on tiny shapes.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("mode", MODES)
def test_tiny_shapes_against_the_oracle(mode):
    dims = [1, 2, 3, 5, 7, 8, 31, 33]
    for M in dims:
        for N in dims:
            for K in (1, 2, 3, 7, 17):
                A, B, C = make_inputs(M, N, K, "normal", seed=M * 1000 + N * 10 + K)
                say(f"[tiny] {mode} {M}x{N}x{K}")
                got = run(mode, A, B, C, 0.75, -0.25)
                assert_parity(mode, A, B, C, 0.75, -0.25, got)


@pytest.mark.parametrize("mode", MODES)
def test_empty_output_leaves_c_alone(mode):
    fn = g.lib().gemm_f32 if mode == "f32" else g.lib().gemm_f16r_f32acc
    tC = torch.full((4, 4), 7.0, device="cuda:0")
    say(f"[edge] {mode} M=0 / N=0")
    assert fn(0, 4, 4, 1.0, None, 4, None, 4, 0.0, tC.data_ptr(), 4, None) == 0
    assert fn(4, 0, 4, 1.0, None, 4, None, 1, 0.0, tC.data_ptr(), 4, None) == 0
    torch.cuda.synchronize()
    assert bool((tC == 7.0).all())


@pytest.mark.parametrize("mode", MODES)
def test_bitwise_deterministic(mode):
    A, B, C = make_inputs(1024, 768, 1000, "normal", seed=8)
    say(f"[determinism] {mode}")
    first = run(mode, A, B, C, 1.0, 1.0)
    for _ in range(3):
        again = run(mode, A, B, C, 1.0, 1.0)
        assert np.array_equal(first.view(np.uint32), again.view(np.uint32))


@pytest.mark.parametrize("mode", MODES)
def test_non_default_stream(mode):
    A, B, C = make_inputs(640, 384, 512, "uniform", seed=9)
    s = torch.cuda.Stream()
    tA, tB, tC = to_device(A), to_device(B), to_device(C)
    torch.cuda.synchronize()
    say(f"[stream] {mode}")
    with torch.cuda.stream(s):
        g.gemm(mode, tA, tB, tC, 1.0, 0.5)
    s.synchronize()
    assert_parity(mode, A, B, C, 1.0, 0.5, tC.cpu().numpy())


@pytest.mark.parametrize("mode,M,K", [("f32", 640, 512), ("f16r", 640, 512), ("f16r", 1280, 3072),
                                      ("f16r", 16, 4096), ("f32", 16, 4096), ("f16r", 64, 4096),
                                      ("f32", 64, 4096)])
def test_graph_capture_replays(mode, M, K):
    """The calls enqueue kernels only (no allocation once the stream's workspace
    exists, no memset), so they can be captured into a HIP graph; every replay,
    with eager work and synchronisations in between, matches the eager call bit
    for bit.  M = 16 takes the few-rows path (partials + counters), M = 64 the
    f32-panel ring split over K (partials + counters), f16r 1280 rows the
    packed path (packed operands in scratch)."""
    N = 384
    A, B, C = make_inputs(M, N, K, "uniform", seed=14)
    tA, tB, tC = to_device(A), to_device(B), to_device(C)
    C0 = tC.clone()
    s = torch.cuda.Stream()
    say(f"[graph] {mode} {M}x{N}x{K} {g.get_config(mode, M, N, K, beta=0.5)}")
    with torch.cuda.stream(s):
        g.gemm(mode, tA, tB, tC, 1.25, 0.5)          # eager; creates the stream's workspace
    s.synchronize()
    eager = tC.clone()
    graph = torch.cuda.CUDAGraph()
    tC.copy_(C0)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=s):
        g.gemm(mode, tA, tB, tC, 1.25, 0.5)
    for _ in range(3):
        tC.copy_(C0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(tC, eager)
    assert_parity(mode, A, B, C, 1.25, 0.5, tC.cpu().numpy())


@pytest.mark.parametrize("mode", MODES)
def test_tuner_leaves_c_alone_and_its_choice_is_correct(mode):
    M, N, K = 1536, 1280, 1024
    A, B, C = make_inputs(M, N, K, "uniform", seed=10)
    tA, tB, tC = to_device(A), to_device(B), to_device(C)
    g.cache_clear()
    try:
        say(f"[tune] {mode} {M}x{N}x{K}")
        g.tune(mode, tA, tB, tC, beta=0.5)
        assert np.array_equal(tC.cpu().numpy(), C)
        cfg = g.get_config(mode, M, N, K, beta=0.5)
        assert cfg.endswith("source=tuned"), cfg
        g.gemm(mode, tA, tB, tC, 1.0, 0.5)
        torch.cuda.synchronize()
        assert_parity(mode, A, B, C, 1.0, 0.5, tC.cpu().numpy())
    finally:
        g.cache_clear()


# ---------------------------------------------------------------------------
# The f32 ring splits K over workgroups when its tiles leave CUs idle; the
# last workgroup of a tile adds the slices in slice order.
# ---------------------------------------------------------------------------
RINGS = [c for c in g.list_configs("f32") if "BK=16" in c and int(c.split("ST=")[1].split()[0]) >= 3]


@pytest.mark.parametrize("cfg", RINGS)
@pytest.mark.parametrize("M,N,K", [(256, 4096, 4096), (512, 1024, 8192), (2048, 2048, 1024),
                                   (256, 512, 1040)])
def test_ring_split_against_the_oracle(cfg, M, N, K):
    A, B, C = make_inputs(M, N, K, "normal", seed=31)
    with pinned("f32", cfg):
        say(f"[ring split] {cfg} {M}x{N}x{K}")
        got = run("f32", A, B, C, 1.25, -0.5)
        again = run("f32", A, B, C, 1.25, -0.5)
    assert_parity("f32", A, B, C, 1.25, -0.5, got)
    assert np.array_equal(got.view(np.uint32), again.view(np.uint32))   # fixed slice order


@pytest.mark.parametrize("cfg", RINGS[:1] + RINGS[-1:])
def test_ring_split_small_integers_exact_and_beta_zero(cfg):
    M, N, K = 256, 2048, 4096
    A, B, C = small_integers(M, N, K, seed=32)
    exact = A.astype(np.float64) @ B.astype(np.float64)
    with pinned("f32", cfg):
        say(f"[ring split exact] {cfg} {M}x{N}x{K}")
        got = run("f32", A, B, C, -2.0, 0.5)
        assert np.array_equal(got, (-2.0 * exact + 0.5 * C.astype(np.float64)).astype(np.float32))
        Cn = np.full((M, N), np.nan, dtype=np.float32)
        got = run("f32", A, B, Cn, 1.0, 0.0)
        assert np.array_equal(got, exact.astype(np.float32))


def test_ring_split_graph_capture_replays():
    M, N, K = 256, 512, 4096
    A, B, C = make_inputs(M, N, K, "uniform", seed=33)
    tA, tB, tC = to_device(A), to_device(B), to_device(C)
    C0 = tC.clone()
    s = torch.cuda.Stream()
    with pinned("f32", RINGS[0]):
        say(f"[graph ring split] {RINGS[0]} {M}x{N}x{K}")
        with torch.cuda.stream(s):
            g.gemm("f32", tA, tB, tC, 1.25, 0.5)     # eager; creates the workspace and counters
        s.synchronize()
        eager = tC.clone()
        graph = torch.cuda.CUDAGraph()
        tC.copy_(C0)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=s):
            g.gemm("f32", tA, tB, tC, 1.25, 0.5)
        for _ in range(3):
            tC.copy_(C0)
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            assert torch.equal(tC, eager)
    assert_parity("f32", A, B, C, 1.25, 0.5, tC.cpu().numpy())


# ---------------------------------------------------------------------------
# The f16r half-depth ring takes the stream-K form when whole rounds of
# tiles leave CUs idle (not with 128 x 128 wave tiles; only while the tiles
# left after the whole rounds fill at most a quarter of the slots): 1024 x
# 4096^2 and 1000 x 3000 x 2000 on 256^2 tiles (no whole round), 4352 x 4224
# x 4096 on every ring (one or two whole rounds, then 33 or 98 tiles in runs).
# ---------------------------------------------------------------------------
F16_RINGS = [c for c in g.list_configs("f16r")
             if "BK=32" in c and "KS=" not in c and "BM=256 BN=256 BK=32 ST=5 WM=2 WN=2" not in c]


@pytest.mark.parametrize("cfg", F16_RINGS)
@pytest.mark.parametrize("M,N,K,full", [(1024, 4096, 4096, True), (1000, 3000, 2000, True),
                                        (3072, 3072, 3072, False), (4352, 4224, 4096, False)])
def test_f16_ring_stream_k_against_the_oracle(cfg, M, N, K, full):
    A, B, C = make_inputs(M, N, K, "normal", seed=41)
    with pinned("f16r", cfg):
        say(f"[f16 ring stream-K] {cfg} {M}x{N}x{K}")
        got = run("f16r", A, B, C, 0.75, -0.25)
        again = run("f16r", A, B, C, 0.75, -0.25)
    if full:
        assert_parity("f16r", A, B, C, 0.75, -0.25, got)
    else:
        assert_sampled("f16r", A, B, C, 0.75, -0.25, got)
    assert np.array_equal(got.view(np.uint32), again.view(np.uint32))   # parts added in k order


@pytest.mark.parametrize("cfg", F16_RINGS[:1] + F16_RINGS[-1:])
def test_f16_ring_stream_k_small_integers_and_f16_output(cfg):
    M, N, K = 512, 2048, 4096
    A, B, C = small_integers(M, N, K, seed=42)
    exact = A.astype(np.float64) @ B.astype(np.float64)
    with pinned("f16r", cfg):
        say(f"[f16 ring stream-K exact] {cfg} {M}x{N}x{K}")
        got = run("f16r", A, B, C, -2.0, 0.5)
        assert np.array_equal(got, (-2.0 * exact + 0.5 * C.astype(np.float64)).astype(np.float32))
        A2, B2, C2 = make_inputs(M, N, K, "normal", seed=43)
        C16 = C2.astype(np.float16)
        tA, tB = to_device(A2), to_device(B2)
        t16 = torch.from_numpy(C16.copy()).to("cuda")
        t32 = to_device(C16.astype(np.float32))
        g.gemm_f16r_f16out(tA, tB, t16, 0.75, -0.25)
        g.gemm("f16r", tA, tB, t32, 0.75, -0.25)
        torch.cuda.synchronize()
    want = t32.cpu().numpy().astype(np.float16)
    assert np.array_equal(t16.cpu().numpy().view(np.uint16), want.view(np.uint16))


# ---------------------------------------------------------------------------
# A ragged call of an f32 ring configuration: the ring takes the block of
# whole tiles over K rounded down to 16, the register-staged tile the k tail
# and the right and bottom strips.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("cfg", RINGS)
@pytest.mark.parametrize("M,N,K,full,lds", [
    (1000, 1030, 1000, True, {"lda": 1000, "ldb": 1032, "ldc": 1030}),
    (2100, 2090, 2070, True, {"lda": 2072, "ldb": 2092, "ldc": 2090}),
    (4097, 4097, 4097, False, {"lda": 4100, "ldb": 4100, "ldc": 4100}),
])
def test_ring_ragged_decomposition(cfg, M, N, K, full, lds):
    """16-byte aligned rows (lda, ldb % 4 == 0), so the ring takes the block of
    whole tiles and the strips go to the other configurations."""
    A, B, C = make_inputs(M, N, K, "normal", seed=51, **lds)
    with pinned("f32", cfg):
        say(f"[ring ragged] {cfg} {M}x{N}x{K}")
        got = run("f32", A, B, C, 1.25, -0.5)
        again = run("f32", A, B, C, 1.25, -0.5)
    if full:
        assert_parity("f32", A, B, C, 1.25, -0.5, got)
    else:
        assert_sampled("f32", A, B, C, 1.25, -0.5, got)
        # whole rows (every column, the right strip's too) at the edges of
        # the parts: the first rows, both sides of row 3840 and of 4096
        for band in [(0, 2), (254, 258), (3838, 3842), (4094, 4097)]:
            st = oracle.check("f32", A, B, C, 1.25, -0.5, got, rows=band)
            assert st["n_fail"] == 0, (band, st)
    assert np.array_equal(got.view(np.uint32), again.view(np.uint32))


@pytest.mark.parametrize("cfg", RINGS[:1] + RINGS[-1:])
def test_ring_ragged_small_integers_exact_and_beta_zero(cfg):
    M, N, K = 1000, 1032, 1000     # N % 4 == 0: B's rows 16-byte aligned
    A, B, C = small_integers(M, N, K, seed=52)
    exact = A.astype(np.float64) @ B.astype(np.float64)
    with pinned("f32", cfg):
        say(f"[ring ragged exact] {cfg} {M}x{N}x{K}")
        got = run("f32", A, B, C, -2.0, 0.5)
        assert np.array_equal(got, (-2.0 * exact + 0.5 * C.astype(np.float64)).astype(np.float32))
        Cn = np.full((M, N), np.nan, dtype=np.float32)
        got = run("f32", A, B, Cn, 1.0, 0.0)
        assert np.array_equal(got, exact.astype(np.float32))


# ---------------------------------------------------------------------------
# The masked form of the f32 ring: any shape and any leading dimensions, the
# copies zero-filling A and B past M, N and K (4-byte copies, so rows need no
# 16-byte alignment), stream-K when whole rounds of tiles leave CUs idle.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("cfg", RINGS)
@pytest.mark.parametrize("M,N,K,lds", [
    (1000, 1030, 1000, {}),                                  # ragged, 8-byte rows
    (300, 517, 333, {"lda": 335, "ldb": 519, "ldc": 521}),   # odd lds: 4-byte rows
    (1, 1, 1, {}),                                           # one element
    (33, 300, 7, {}),                                        # K shorter than a panel
    (256, 256, 4093, {}),                                    # one tile, long ragged K
    (513, 2049, 1100, {"lda": 1101}),                        # stream-K over ragged tiles
    (1000, 1025, 1001, {"lda": 1001}),                       # one column past whole tiles
])
def test_ring_masked_against_the_oracle(cfg, M, N, K, lds):
    A, B, C = make_inputs(M, N, K, "normal", seed=61, **lds)
    with pinned("f32", cfg):
        say(f"[ring masked] {cfg} {M}x{N}x{K} {lds}")
        got = run("f32", A, B, C, 1.25, -0.5)
        again = run("f32", A, B, C, 1.25, -0.5)
    assert_parity("f32", A, B, C, 1.25, -0.5, got)
    assert np.array_equal(got.view(np.uint32), again.view(np.uint32))


@pytest.mark.parametrize("cfg", RINGS[:1] + RINGS[-1:])
def test_ring_masked_zero_fills_past_the_edges(cfg):
    """NaN in the padding of A's rows (k >= K) and of B's rows (columns >= N),
    and in the rows of B after K: a masked copy that read any of them would
    put NaN into C, since NaN times the zero of the other operand is NaN."""
    M, N, K, lda, ldb = 300, 517, 333, 337, 523
    A, B, C = small_integers(M, N, K, seed=62)
    fa = np.full((M, lda), np.nan, dtype=np.float32)
    fa[:, :K] = A
    fb = np.full((K + 40, ldb), np.nan, dtype=np.float32)
    fb[:K, :N] = B
    tA = torch.from_numpy(fa).to("cuda")[:, :K]
    tB = torch.from_numpy(fb).to("cuda")[:K, :N]
    tC = to_device(C)
    exact = A.astype(np.float64) @ B.astype(np.float64)
    with pinned("f32", cfg):
        say(f"[ring masked nan] {cfg} {M}x{N}x{K}")
        g.gemm("f32", tA, tB, tC, 1.0, -1.0)
        torch.cuda.synchronize()
    got = tC.cpu().numpy()
    assert np.array_equal(got, (exact - C.astype(np.float64)).astype(np.float32))


# The masked f32 ring with 16-byte copies: 16-byte aligned rows (leading
# dimensions multiples of 4) and N, K multiples of 4, so each lane's chunk of
# four floats lies wholly inside or outside the matrix.  Every case checks that
# the pinned ring runs the whole call masked with aligned rows (the plan).
WIDE_CASES = [
    (1000, 1000, 1000, {}),                                     # ragged M, N; K tail of 8
    (1001, 1028, 1004, {}),                                     # odd M; K tail of 12
    (700, 1020, 100, {"lda": 104, "ldb": 1024, "ldc": 1021}),   # padded lds, odd ldc
    (4000, 4000, 4000, {}),                                     # stream-K over ragged tiles
]


@pytest.mark.parametrize("cfg", RINGS)
@pytest.mark.parametrize("M,N,K,lds", WIDE_CASES)
def test_ring_wide_masked_copies_against_the_oracle(cfg, M, N, K, lds):
    A, B, C = make_inputs(M, N, K, "normal", seed=64, **lds)
    with pinned("f32", cfg):
        plan = g.get_plan("f32", M, N, K, beta=-0.5, **lds)
        assert plan == f"form=ring-masked block={M}x{N}x{K}", plan
        say(f"[ring wide masked] {cfg} {M}x{N}x{K} {lds}")
        got = run("f32", A, B, C, 1.25, -0.5)
        again = run("f32", A, B, C, 1.25, -0.5)
    if M * N <= 2 ** 21:
        assert_parity("f32", A, B, C, 1.25, -0.5, got)
    else:
        assert_sampled("f32", A, B, C, 1.25, -0.5, got)
    assert np.array_equal(got.view(np.uint32), again.view(np.uint32))


@pytest.mark.parametrize("cfg", RINGS[:1] + RINGS[-1:])
def test_ring_wide_masked_zero_fills_past_the_edges(cfg):
    """NaN in the padding of A's rows (k >= K), of B's rows (columns >= N) and
    in the rows of B after K, with 16-byte copies: a chunk that read any of
    them would put NaN into C.  Small integers, so the result is exact."""
    M, N, K, lda, ldb = 1000, 1012, 332, 336, 1016
    A, B, C = small_integers(M, N, K, seed=65)
    fa = np.full((M, lda), np.nan, dtype=np.float32)
    fa[:, :K] = A
    fb = np.full((K + 40, ldb), np.nan, dtype=np.float32)
    fb[:K, :N] = B
    tA = torch.from_numpy(fa).to("cuda")[:, :K]
    tB = torch.from_numpy(fb).to("cuda")[:K, :N]
    tC = to_device(C)
    exact = A.astype(np.float64) @ B.astype(np.float64)
    with pinned("f32", cfg):
        plan = g.get_plan("f32", M, N, K, lda=lda, ldb=ldb, beta=-1.0)
        assert plan == f"form=ring-masked block={M}x{N}x{K}", plan
        say(f"[ring wide masked nan] {cfg} {M}x{N}x{K}")
        g.gemm("f32", tA, tB, tC, 1.0, -1.0)
        torch.cuda.synchronize()
    got = tC.cpu().numpy()
    assert np.array_equal(got, (exact - C.astype(np.float64)).astype(np.float32))


@pytest.mark.parametrize("cfg", RINGS[:1] + RINGS[-1:])
def test_ring_wide_masked_small_integers_exact_and_beta_zero(cfg):
    M, N, K = 4000, 4092, 1004
    A, B, C = small_integers(M, N, K, seed=66)
    exact = A.astype(np.float64) @ B.astype(np.float64)
    with pinned("f32", cfg):
        assert g.get_plan("f32", M, N, K, beta=0.5) == f"form=ring-masked block={M}x{N}x{K}"
        say(f"[ring wide masked exact] {cfg} {M}x{N}x{K}")
        got = run("f32", A, B, C, -2.0, 0.5)
        assert np.array_equal(got, (-2.0 * exact + 0.5 * C.astype(np.float64)).astype(np.float32))
        Cn = np.full((M, N), np.nan, dtype=np.float32)
        got = run("f32", A, B, Cn, 1.0, 0.0)
        assert np.array_equal(got, exact.astype(np.float32))


@pytest.mark.parametrize("cfg", RINGS[:1] + RINGS[-1:])
def test_ring_masked_small_integers_exact_and_beta_zero(cfg):
    M, N, K = 4000, 4097, 1001    # rows of B and C start 16-byte aligned every fourth row
    A, B, C = small_integers(M, N, K, seed=63)
    exact = A.astype(np.float64) @ B.astype(np.float64)
    with pinned("f32", cfg):
        say(f"[ring masked exact] {cfg} {M}x{N}x{K}")
        got = run("f32", A, B, C, -2.0, 0.5)
        assert np.array_equal(got, (-2.0 * exact + 0.5 * C.astype(np.float64)).astype(np.float32))
        Cn = np.full((M, N), np.nan, dtype=np.float32)
        got = run("f32", A, B, Cn, 1.0, 0.0)
        assert np.array_equal(got, exact.astype(np.float32))
