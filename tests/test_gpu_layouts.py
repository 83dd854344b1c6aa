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


# ---------------------------------------------------------------------------
# The f32 ring of direct-to-LDS copies in the transposed layouts: a transposed
# operand's panels are copied along its stored rows (k-rows of A^T; rows of
# B^T, along which k runs), in every ring configuration and form -- whole tiles
# in whole rounds or dealt to the CUs in runs (stream-K), the 16-byte masked
# copies (16-byte aligned rows, each operand's contiguous extent a multiple of
# 4) and the 4-byte ones.  The plan must name the ring for the whole call.
# ---------------------------------------------------------------------------
RINGS = [c for c in g.list_configs("f32") if "BK=16" in c and int(c.split("ST=")[1].split()[0]) >= 3]
RING_CASES = [
    (1024, 1024, 1024, 0, "ring"),          # whole tiles; few tiles: runs of panels
    (4096, 4096, 64, 0, "ring"),            # whole tiles in whole rounds
    (1000, 1004, 1008, 0, "ring-masked"),   # 16-byte masked copies
    (300, 517, 333, 3, "ring-masked"),      # odd leading dimensions: 4-byte copies
    (513, 2049, 1100, 1, "ring-masked"),    # runs over ragged tiles
    (1, 1, 1, 0, "ring-masked"),            # one element
    (33, 300, 7, 0, "ring-masked"),         # K shorter than a panel
]


def _lds(M, N, K, ta, tb, pad):
    return ((M if ta else K) + pad if pad else None), ((K if tb else N) + pad if pad else None)


@pytest.mark.parametrize("cfg", RINGS)
@pytest.mark.parametrize("ta,tb", LAYOUTS, ids=[_name(*x) for x in LAYOUTS])
@pytest.mark.parametrize("M,N,K,pad,form", RING_CASES)
def test_ring_layouts_against_the_oracle(cfg, ta, tb, M, N, K, pad, form):
    A, B, C = make_inputs(M, N, K, "normal", seed=71)
    lda, ldb = _lds(M, N, K, ta, tb, pad)
    with pinned("f32", cfg):
        plan = g.get_plan("f32", M, N, K, lda=lda, ldb=ldb, beta=-0.5, transa=ta, transb=tb)
        assert plan.startswith(f"form={form} block={M}x{N}x{K}"), plan
        say(f"[ring layout] {_name(ta, tb)} {cfg} {M}x{N}x{K} lda={lda} ldb={ldb}")
        got = run_ex("f32", A, B, C, 1.25, -0.5, ta, tb, lda, ldb)
        again = run_ex("f32", A, B, C, 1.25, -0.5, ta, tb, lda, ldb)
    assert np.array_equal(got.view(np.uint32), again.view(np.uint32))
    if M * N <= 2 ** 21:
        check("f32", A, B, C, 1.25, -0.5, got)
    else:
        check("f32", A, B, C, 1.25, -0.5, got, rows=(0, 48))
        check("f32", A, B, C, 1.25, -0.5, got, rows=(M - 48, M))
        r, c = sample_indices(M, N, 2048, seed=2)
        ref, W = oracle.entries("f32", np.ascontiguousarray(A), np.ascontiguousarray(B), C, 1.25,
                                -0.5, r, c)
        assert np.all(np.abs(got[r, c].astype(np.float64) - ref) <= oracle.TOL["f32"] * W)


def _nan_padded(op, t, ld, extra=40):
    """op stored as itself or transposed, in a NaN-filled buffer with a padded
    leading dimension and extra NaN rows after it; the view of the stored
    array."""
    st = op.T if t else op
    buf = np.full((st.shape[0] + extra, ld), np.nan, dtype=np.float32)
    buf[:st.shape[0], :st.shape[1]] = st
    return torch.from_numpy(buf).to("cuda")[:st.shape[0], :st.shape[1]]


@pytest.mark.parametrize("cfg", RINGS[:1] + RINGS[-1:])
@pytest.mark.parametrize("ta,tb", LAYOUTS, ids=[_name(*x) for x in LAYOUTS])
@pytest.mark.parametrize("M,N,K,pad", [(1000, 1012, 332, 4), (301, 517, 333, 3)])
def test_ring_layouts_zero_fill_past_the_edges(cfg, ta, tb, M, N, K, pad):
    """NaN in the padding of every stored row and in the rows after each
    stored array: a masked copy (16-byte ones for the first shape, 4-byte ones
    for the second) that read any of them would put NaN into C.  Small
    integers, so the result is exact."""
    A, B, C = small_integers(M, N, K, seed=72)
    lda, ldb = _lds(M, N, K, ta, tb, pad)
    tA, tB, tC = _nan_padded(A, ta, lda), _nan_padded(B, tb, ldb), to_device(C)
    exact = A.astype(np.float64) @ B.astype(np.float64)
    with pinned("f32", cfg):
        plan = g.get_plan("f32", M, N, K, lda=lda, ldb=ldb, beta=-1.0, transa=ta, transb=tb)
        assert plan.startswith(f"form=ring-masked block={M}x{N}x{K}"), plan
        say(f"[ring layout nan] {_name(ta, tb)} {cfg} {M}x{N}x{K}")
        g.gemm("f32", tA, tB, tC, 1.0, -1.0, transa=ta, transb=tb)
        torch.cuda.synchronize()
    got = tC.cpu().numpy()
    assert np.array_equal(got, (exact - C.astype(np.float64)).astype(np.float32))


@pytest.mark.parametrize("cfg", RINGS[:1] + RINGS[-1:])
@pytest.mark.parametrize("ta,tb", LAYOUTS, ids=[_name(*x) for x in LAYOUTS])
@pytest.mark.parametrize("M,N,K", [(2048, 1024, 1024), (4000, 4092, 1004)])
def test_ring_layouts_small_integers_exact_and_beta_zero(cfg, ta, tb, M, N, K):
    A, B, C = small_integers(M, N, K, seed=73)
    exact = A.astype(np.float64) @ B.astype(np.float64)
    with pinned("f32", cfg):
        say(f"[ring layout exact] {_name(ta, tb)} {cfg} {M}x{N}x{K}")
        got = run_ex("f32", A, B, C, -2.0, 0.5, ta, tb)
        assert np.array_equal(got, (-2.0 * exact + 0.5 * C.astype(np.float64)).astype(np.float32))
        Cn = np.full((M, N), np.nan, dtype=np.float32)
        got = run_ex("f32", A, B, Cn, 1.0, 0.0, ta, tb)
        assert np.array_equal(got, exact.astype(np.float32))


# ---------------------------------------------------------------------------
# The f32-panel ring (KS=3, BK=32: f32 panels through direct-to-LDS copies,
# rounded to binary16 as read in f16r, K split over workgroups) in the
# transposed layouts: A^T staged as k-rows, B^T as swizzled rows read in the
# block layout of the 16-column blocks, both modes, every configuration.
# ---------------------------------------------------------------------------
PANEL_RINGS = {m: [c for c in g.list_configs(m) if "KS=3" in c and "BK=32" in c] for m in MODES}
PANEL_CASES = [
    (20, 1000, 4096, 0),     # ragged M and N, many slices
    (300, 520, 2112, 4),     # padded 16-byte rows
    (64, 4096, 4096, 0),     # whole tiles
    (36, 256, 32, 0),        # one panel
    (128, 1001, 1024, 0),    # N % 4 != 0: B^T taken, B as stored handed to other tiles
]


@pytest.mark.parametrize("mode,cfg", [(m, c) for m in MODES for c in PANEL_RINGS[m]])
@pytest.mark.parametrize("ta,tb", LAYOUTS, ids=[_name(*x) for x in LAYOUTS])
@pytest.mark.parametrize("M,N,K,pad", PANEL_CASES)
def test_panel_ring_layouts_against_the_oracle(mode, cfg, ta, tb, M, N, K, pad):
    A, B, C = make_inputs(M, N, K, "normal", seed=74)
    lda, ldb = _lds(M, N, K, ta, tb, pad)
    with pinned(mode, cfg):
        say(f"[panel ring layout] {mode} {_name(ta, tb)} {cfg} {M}x{N}x{K} lda={lda} ldb={ldb}")
        got = run_ex(mode, A, B, C, -0.75, 1.5, ta, tb, lda, ldb)
        again = run_ex(mode, A, B, C, -0.75, 1.5, ta, tb, lda, ldb)
    assert np.array_equal(got.view(np.uint32), again.view(np.uint32))
    check(mode, A, B, C, -0.75, 1.5, got)


@pytest.mark.parametrize("mode,cfg", [(m, c) for m in MODES for c in PANEL_RINGS[m][:1] + PANEL_RINGS[m][-1:]])
@pytest.mark.parametrize("ta,tb", LAYOUTS, ids=[_name(*x) for x in LAYOUTS])
def test_panel_ring_layouts_small_integers_exact_and_beta_zero(mode, cfg, ta, tb):
    M, N, K = 40, 2048, 4096
    A, B, C = small_integers(M, N, K, seed=75)
    exact = A.astype(np.float64) @ B.astype(np.float64)
    with pinned(mode, cfg):
        say(f"[panel ring layout exact] {mode} {_name(ta, tb)} {cfg} {M}x{N}x{K}")
        got = run_ex(mode, A, B, C, -2.0, 0.5, ta, tb)
        assert np.array_equal(got, (-2.0 * exact + 0.5 * C.astype(np.float64)).astype(np.float32))
        Cn = np.full((M, N), np.nan, dtype=np.float32)
        got = run_ex(mode, A, B, Cn, 1.0, 0.0, ta, tb)
        assert np.array_equal(got, exact.astype(np.float32))


@pytest.mark.parametrize("mode,cfg", [(m, c) for m in MODES for c in PANEL_RINGS[m][:1] + PANEL_RINGS[m][-1:]])
@pytest.mark.parametrize("ta,tb", [(False, False)] + LAYOUTS, ids=["NN"] + [_name(*x) for x in LAYOUTS])
def test_panel_ring_layouts_never_read_past_the_matrix(mode, cfg, ta, tb):
    """NaN in the padding of every stored row (16-byte aligned leading
    dimensions) and in 40 rows after each stored array; M and N ragged
    against the tiles.  The panel ring clamps every copy to the matrix, so a
    read of any NaN would show in C.  Small integers: the result is exact."""
    M, N, K = 44, 1000, 2048
    A, B, C = small_integers(M, N, K, seed=76)
    lda, ldb = _lds(M, N, K, ta, tb, 4)
    tA, tB, tC = _nan_padded(A, ta, lda), _nan_padded(B, tb, ldb), to_device(C)
    exact = A.astype(np.float64) @ B.astype(np.float64)
    with pinned(mode, cfg):
        plan = g.get_plan(mode, M, N, K, lda=lda, ldb=ldb, beta=-1.0, transa=ta, transb=tb)
        assert plan.split()[0] in ("form=panel-ring", "form=round-on-load"), plan
        say(f"[panel ring layout nan] {mode} {_name(ta, tb)} {cfg} {M}x{N}x{K}")
        g.gemm(mode, tA, tB, tC, 1.0, -1.0, transa=ta, transb=tb)
        torch.cuda.synchronize()
    got = tC.cpu().numpy()
    assert np.array_equal(got, (exact - C.astype(np.float64)).astype(np.float32))
