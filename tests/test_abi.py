"""CPU tests of the C ABI: the library loads, exports what include/gemm355.h
declares, and the host-side logic (argument checks, special cases decided
before any launch, configuration grammar, tuning cache) behaves as documented.
No call here reaches the GPU."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

import gemm_tiled_amd as g

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gemm355.h")

# a plausible, 256-byte aligned device address; never dereferenced because
# every call below returns before any launch
FAKE = ctypes.c_void_p(1 << 40)


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = "\n".join(ln for ln in text.splitlines() if not ln.lstrip().startswith("#"))
    return sorted(set(re.findall(r"\b([A-Za-z_][A-Za-z0-9_]*)\s*\(", text)) -
                  {"if", "defined", "sizeof"})


def test_header_declares_the_two_gemm_calls():
    names = _declared_functions()
    assert "gemm_f32" in names and "gemm_f16r_f32acc" in names


def test_library_exports_every_declared_symbol():
    handle = ctypes.CDLL(g.library_path())
    for name in _declared_functions():
        assert hasattr(handle, name), f"{name} not exported"
    assert set(_declared_functions()) == set(g.EXPORTS), "binding and header disagree"


def test_version_and_strerror():
    assert re.match(r"^\d+\.\d+\.\d+$", g.version())
    assert g.strerror(0) == "success"
    assert "lda" in g.strerror(-6)
    assert g.strerror(-101).startswith("tile configuration")


def _call(fn, M, N, K, A=FAKE, lda=None, B=FAKE, ldb=None, C=FAKE, ldc=None, alpha=1.0, beta=0.0):
    lda = max(K, 1) if lda is None else lda
    ldb = max(N, 1) if ldb is None else ldb
    ldc = max(N, 1) if ldc is None else ldc
    return fn(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, None)


@pytest.mark.parametrize("name", ["gemm_f32", "gemm_f16r_f32acc"])
def test_argument_checks_follow_xerbla_numbering(name):
    fn = getattr(g.lib(), name)
    assert _call(fn, -1, 4, 4) == -1
    assert _call(fn, 4, -1, 4) == -2
    assert _call(fn, 4, 4, -1) == -3
    assert _call(fn, 1 << 31, 4, 4) == -1
    assert _call(fn, 4, 4, 4, A=None) == -5
    assert _call(fn, 4, 4, 8, lda=7) == -6
    assert _call(fn, 4, 4, 4, B=None) == -7
    assert _call(fn, 4, 8, 4, ldb=7) == -8
    assert _call(fn, 4, 4, 4, C=None) == -10
    assert _call(fn, 4, 8, 4, ldc=7) == -11
    # the first invalid argument wins
    assert _call(fn, -1, -1, -1, A=None, lda=0) == -1
    # leading dimensions must be >= 1 even for empty rows
    assert _call(fn, 4, 0, 4, ldb=0) == -8
    assert _call(fn, 4, 4, 0, lda=0) == -6


def _call_ex(fn, ta, tb, M, N, K, A=FAKE, lda=None, B=FAKE, ldb=None, C=FAKE, ldc=None):
    lda = max(M if ta else K, 1) if lda is None else lda
    ldb = max(K if tb else N, 1) if ldb is None else ldb
    ldc = max(N, 1) if ldc is None else ldc
    return fn(ta, tb, M, N, K, 1.0, A, lda, B, ldb, 0.0, C, ldc, None)


@pytest.mark.parametrize("name", ["gemm_f32_ex", "gemm_f16r_f32acc_ex"])
def test_layout_argument_checks_follow_sgemm_numbering(name):
    """op(A) = A^T is stored K x M (lda >= M), op(B) = B^T N x K (ldb >= K);
    codes are BLAS sgemm's argument numbers."""
    fn = getattr(g.lib(), name)
    assert _call_ex(fn, 2, 0, 4, 4, 4) == -1
    assert _call_ex(fn, 0, -1, 4, 4, 4) == -2
    assert _call_ex(fn, 0, 0, -1, 4, 4) == -3
    assert _call_ex(fn, 1, 0, 4, -1, 4) == -4
    assert _call_ex(fn, 0, 1, 4, 4, -1) == -5
    assert _call_ex(fn, 1, 1, 4, 4, 4, A=None) == -7
    assert _call_ex(fn, 0, 0, 4, 4, 8, lda=7) == -8
    # transposed A: the row of the stored array has M elements
    assert _call_ex(fn, 1, 0, 8, 4, 4, lda=7) == -8
    assert _call_ex(fn, 1, 1, 4, 4, 4, B=None) == -9
    assert _call_ex(fn, 0, 1, 4, 4, 8, ldb=7) == -10
    assert _call_ex(fn, 0, 0, 4, 8, 4, ldb=7) == -10
    assert _call_ex(fn, 0, 0, 4, 4, 4, C=None) == -12
    assert _call_ex(fn, 1, 1, 4, 8, 4, ldc=7) == -13
    # M == 0: nothing to do, whatever the layout
    assert _call_ex(fn, 1, 1, 0, 5, 7, A=None, B=None, C=None) == 0


def test_f16out_argument_checks():
    fn = g.lib().gemm_f16r_f16out
    assert _call_ex(fn, 3, 0, 4, 4, 4) == -1
    assert _call_ex(fn, 0, 0, 4, 4, 8, lda=7) == -8
    assert _call_ex(fn, 0, 0, 4, 4, 4, C=None) == -12
    assert _call_ex(fn, 0, 0, 4, 8, 4, ldc=7) == -13
    assert _call_ex(fn, 0, 0, 0, 8, 4, A=None, B=None, C=None) == 0


def test_layout_configs_are_keyed_apart(tmp_path):
    """The tuning cache keys the operand layout: a tuned transposed shape does
    not leak into the plain layout of the same shape, and the cache file names
    the layout after the mode ("f32:TN")."""
    path = tmp_path / "tune.txt"
    cfg = g.list_configs("f32")[-1]
    path.write_text(f"f32:TN 2048 2048 2048 1 1 1 {cfg}\nf32:XY 64 64 64 1 1 1 {cfg}\n")
    g.cache_clear()
    try:
        assert g.cache_load(str(path)) == 1
        assert g.get_config("f32", 2048, 2048, 2048, transa=True) == cfg + " source=tuned"
        assert g.get_config("f32", 2048, 2048, 2048).endswith("source=heuristic")
        assert g.get_config("f32", 2048, 2048, 2048, transb=True).endswith("source=heuristic")
        out = tmp_path / "saved.txt"
        assert g.cache_save(str(out)) == 1
        assert out.read_text().strip() == f"f32:TN 2048 2048 2048 1 1 1 {cfg}"
    finally:
        g.cache_clear()
    # the plain-layout codes of get_config are unchanged by the _ex numbering
    buf = ctypes.create_string_buffer(64)
    assert g.lib().gemm355_get_config(0, 4, 4, 8, 7, 4, 4, 0.0, buf, 64) == -6
    assert g.lib().gemm355_get_config_ex(0, 1, 0, 8, 4, 4, 7, 4, 4, 0.0, buf, 64) == -8
    assert g.lib().gemm355_get_config_ex(0, 0, 3, 8, 4, 4, 4, 4, 4, 0.0, buf, 64) == -2
    # transposed A with K > M: lda >= M suffices (host-only check, no launch)
    assert g.lib().gemm355_get_config_ex(0, 1, 0, 8, 4, 16, 8, 4, 4, 0.0, buf, 64) == 0
    assert g.lib().gemm355_get_config_ex(1, 1, 1, 8, 4, 16, 8, 16, 4, 0.0, buf, 64) == 0


@pytest.mark.parametrize("name", ["gemm_f32", "gemm_f16r_f32acc"])
def test_empty_output_returns_without_launch(name):
    fn = getattr(g.lib(), name)
    # M == 0 or N == 0: nothing to do, even with NULL pointers
    assert _call(fn, 0, 5, 7, A=None, B=None, C=None) == 0
    assert _call(fn, 5, 0, 7, A=None, B=None, C=None) == 0
    assert _call(fn, 0, 0, 0, A=None, B=None, C=None) == 0


def test_null_operands_allowed_when_not_read():
    # alpha == 0 or K == 0 means A and B are not read, so NULL is valid; the
    # call then scales C on the GPU, which is only checked for its argument
    # acceptance here through gemm355_get_config (host only)
    assert g.lib().gemm355_get_config(0, 4, 4, 0, 1, 4, 4, 0.0, ctypes.create_string_buffer(64),
                                      64) == 0


def test_config_grammar():
    assert g.parse_config("f32", "BM=128 BN=128 BK=16") .startswith("BM=128 BN=128 BK=16")
    # the page's pin grammar, case-insensitive keys
    assert g.parse_config("f32", "TILE_M=256 TILE_N=256 TILE_K=16") \
        .startswith("BM=256 BN=256 BK=16")
    assert g.parse_config("f16r", "tile_m=256 tile_n=256 tile_k=64") \
        .startswith("BM=256 BN=256 BK=64")
    for bad in ["", "BM=", "BM=abc", "BM=128x", "XX=1", "BM=100", "BM=128 BN=128 BK=4",
                "=5", "BM=-1", "BM=128 BN"]:
        with pytest.raises(g.Gemm355Error):
            g.parse_config("f32", bad)
    with pytest.raises(g.Gemm355Error):
        g.parse_config(7, "BM=128")


def test_list_configs_are_unique_and_reparse():
    for mode in ("f32", "f16r"):
        cs = g.list_configs(mode)
        assert len(cs) >= 4 and len(set(cs)) == len(cs)
        for c in cs:
            assert g.parse_config(mode, c) == c


def test_pin_overrides_heuristic_and_clears():
    base = g.get_config("f32", 4096, 4096, 4096)
    assert base.endswith("source=heuristic")
    g.set_config("f32", "BM=64 BN=64 BK=16")
    try:
        got = g.get_config("f32", 4096, 4096, 4096)
        assert got.startswith("BM=64 BN=64 BK=16") and got.endswith("source=pin")
        # the other mode is unaffected
        assert g.get_config("f16r", 4096, 4096, 4096).endswith("source=heuristic")
        with pytest.raises(g.Gemm355Error):
            g.set_config("f32", "BM=3")
        # a rejected pin leaves the previous one in place
        assert g.get_config("f32", 4096, 4096, 4096).endswith("source=pin")
    finally:
        g.set_config("f32", None)
    assert g.get_config("f32", 4096, 4096, 4096) == base


def test_heuristic_covers_every_shape_class():
    for (M, N, K) in [(1, 1, 1), (256, 256, 256), (4000, 4097, 4093), (8192, 8192, 8192),
                      (1, 8192, 8192), (8192, 1, 3)]:
        for mode in ("f32", "f16r"):
            cfg = g.get_config(mode, M, N, K)
            assert g.parse_config(mode, cfg.split(" source=")[0])


def test_tuning_cache_roundtrip_and_corrupt_lines(tmp_path):
    path = tmp_path / "tune.txt"
    cfg = g.list_configs("f32")[-1]
    path.write_text(
        f"f32 4096 4096 4096 1 1 1 {cfg}\n"
        "garbage line\n"
        "f32 1 2\n"
        "f16r 64 64 64 1 1 0 BM=3 BN=3\n"           # names no compiled instance
        "xx 64 64 64 1 1 0 BM=64 BN=64 BK=64\n")    # unknown mode
    g.cache_clear()
    try:
        assert g.cache_load(str(path)) == 1
        got = g.get_config("f32", 4096, 4096, 4096, beta=0.0)
        assert got == cfg + " source=tuned"
        # beta != 0 is another key
        assert g.get_config("f32", 4096, 4096, 4096, beta=1.0).endswith("source=heuristic")
        out = tmp_path / "saved.txt"
        assert g.cache_save(str(out)) == 1
        assert out.read_text().strip() == f"f32 4096 4096 4096 1 1 1 {cfg}"
    finally:
        g.cache_clear()
    assert g.get_config("f32", 4096, 4096, 4096).endswith("source=heuristic")
    assert g.cache_load(str(tmp_path / "missing.txt")) == 0


def test_roof_and_copy_reject_bad_buffers_before_launch():
    L = g.lib()
    flops = ctypes.c_double(0)
    assert L.gemm355_roof_mfma(5, 0, 10, 1, FAKE, ctypes.byref(flops), None) == -103
    assert L.gemm355_roof_mfma(0, 0, 0, 1, FAKE, ctypes.byref(flops), None) == -104
    assert L.gemm355_roof_mfma(1, 2, 10, 1, FAKE, ctypes.byref(flops), None) == -104
    assert L.gemm355_roof_fma(0, 1, FAKE, ctypes.byref(flops), None) == -104
    assert L.gemm355_roof_fma(10, 0, FAKE, ctypes.byref(flops), None) == -104
    assert L.gemm355_roof_hbm(FAKE, 17, 1, FAKE, None) == -104
    assert L.gemm355_roof_hbm(ctypes.c_void_p((1 << 40) + 4), 32, 1, FAKE, None) == -104
    assert L.gemm355_copy_f32(None, FAKE, 4, None) == -104
    assert L.gemm355_copy_f32(FAKE, FAKE, 0, None) == 0


def test_tune_rejects_bad_arguments_before_any_allocation():
    L = g.lib()
    assert L.gemm355_tune(9, 4, 4, 4, FAKE, 4, FAKE, 4, 0.0, 4, None) == -103
    assert L.gemm355_tune(0, -1, 4, 4, FAKE, 4, FAKE, 4, 0.0, 4, None) == -1
    assert L.gemm355_tune(0, 4, 4, 4, FAKE, 4, FAKE, 4, 0.0, 3, None) == -11
    assert L.gemm355_tune(0, 0, 4, 4, FAKE, 4, FAKE, 4, 0.0, 4, None) == 0


def test_python_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(g, "_lib", None)
    monkeypatch.setattr(g, "_HERE", str(tmp_path))
    with pytest.raises(ImportError):
        g.lib()


def test_plan_names_the_path_and_the_ring_block():
    """Host-only: gemm355_get_plan_ex.  A ring configuration runs whole tiles
    unmasked; with 16-byte rows a call one element past whole tiles gives the
    ring the block of whole tiles and the strips to other configurations; with
    rows that are not 16-byte aligned the masked ring runs the call, here
    without the last partial tile column (one column of C)."""
    ring = "BM=256 BN=256 BK=16 ST=3 WM=2 WN=4 GM=8"
    g.set_config("f32", ring)
    try:
        assert g.get_plan("f32", 4096, 4096, 4096) == "form=ring block=4096x4096x4096"
        assert g.get_plan("f32", 4100, 4100, 4100) == "form=ring block=4096x4096x4096"
        plan = g.get_plan("f32", 4000, 4097, 4093)
        assert plan == "form=ring-masked block=4000x4096x4093 rows=4-byte", plan
        assert g.get_plan("f32", 300, 517, 333, lda=335, ldb=519, ldc=521) == \
            "form=ring-masked block=300x517x333 rows=4-byte"
        # transposed operands: the ring too, copying each panel along the
        # stored rows, and whole (the block and strips take the plain layout
        # only); leading dimensions past its copies' 32-bit offsets (256
        # stored rows of B^T, 16 of A^T) run the register-staged kernel
        assert g.get_plan("f32", 4096, 4096, 4096, transa=True) == "form=ring block=4096x4096x4096"
        assert g.get_plan("f32", 4100, 4100, 4100, transb=True) == \
            "form=ring-masked block=4100x4100x4100"
        assert g.get_plan("f32", 300, 517, 333, lda=301, ldb=335, transa=True, transb=True) == \
            "form=ring-masked block=300x517x333 rows=4-byte"
        assert g.get_plan("f32", 256, 512, 16, ldb=(1 << 20) + 4, transb=True) == \
            "form=tiles block=256x512x16"
        assert g.get_plan("f32", 256, 512, 16, lda=(1 << 20) + 4, transa=True) == \
            "form=ring block=256x512x16"
        assert g.get_plan("f32", 256, 512, 16, lda=(1 << 24) + 4, transa=True) == \
            "form=tiles block=256x512x16"
    finally:
        g.set_config("f32", None)
    assert g.get_plan("f32", 8, 4096, 4096) == "form=rows block=8x4096x4096"
    # a few columns: the few-rows configuration on the transposed problem, or
    # (f32, A stored M x K, N % 4 == 0 or B stored N x K) the 16-row tile of the
    # f32-panel ring on it
    assert g.get_plan("f32", 4096, 2, 4096) == "form=columns block=4096x2x4096 rows=4-byte"
    assert g.get_plan("f32", 4096, 8, 4096) == "form=panel-ring-columns block=4096x8x4096"
    assert g.get_plan("f32", 4096, 8, 4096, transa=True) == "form=columns block=4096x8x4096"
    assert g.get_plan("f16r", 4096, 1, 4096) == "form=columns block=4096x1x4096 rows=4-byte"
    # 16-byte rows with N and K multiples of 4: the masked ring whole (16-byte copies)
    assert g.get_plan("f32", 4000, 4000, 4000) == "form=ring-masked block=4000x4000x4000"
    assert g.get_plan("f16r", 8192, 8192, 8192).startswith("form=packed block=8192x8192x8192")
    with pytest.raises(g.Gemm355Error):
        g.get_plan("f32", -1, 4, 4)


# The heuristic's choices where the configurations were timed against each
# other on an MI355X (host only: no kernel runs).  Each row: mode, shape, the
# configuration the measurements favour (prefix), and what was measured.
HEURISTIC_PICKS = [
    # f32 scored shapes: the 256^2 ring (the tuner's winner within 2%)
    ("f32", (4096, 4096, 4096), "BM=256 BN=256 BK=16 ST=3 WM=2 WN=4"),
    # f32 few rows: the few-rows configuration up to 16 rows, then the
    # f32-panel ring (32 rows: 32 x 128, 20 us against 22 us split-K tiles;
    # 128 rows: 64 x 64, 42 against 54 us; 256 rows: 64 x 128, 73 against 79)
    ("f32", (16, 4096, 4096), "BM=16 BN=64 BK=64"),
    # few columns (M = K = 4096): f32 the same configuration on the
    # transposed problem for one or two columns (18.7 us), from 4 to 16 the
    # f32-panel ring's 16-row tile on it (18.3-18.5 us against 19.8-20.1;
    # 81 us on the 128 x 256 ring), then the f32-panel ring on 64 x 64 tiles
    # (26 us at 64 columns); f16r the transposed form for one or two columns
    # (18.5 us), the f32-panel ring on 32 x 64 tiles from 4 (16 us against 21)
    ("f32", (4096, 2, 4096), "BM=16 BN=64 BK=64"),
    ("f32", (4096, 16, 4096), "BM=16 BN=128 BK=32 ST=4 WM=1 WN=2 GM=8 KS=3"),
    ("f32", (4096, 64, 4096), "BM=64 BN=64 BK=32 ST=4 WM=4 WN=1 GM=8 KS=3"),
    ("f16r", (4096, 1, 4096), "BM=16 BN=64 BK=64"),
    ("f16r", (4096, 16, 4096), "BM=32 BN=64 BK=32 ST=4 WM=2 WN=1 GM=8 KS=3"),
    ("f16r", (4096, 64, 4096), "BM=32 BN=64 BK=32 ST=4 WM=2 WN=1 GM=8 KS=3"),
    ("f32", (32, 4096, 4096), "BM=32 BN=128 BK=32 ST=4"),
    ("f32", (128, 4096, 4096), "BM=64 BN=64 BK=32 ST=4"),
    ("f32", (256, 4096, 4096), "BM=64 BN=128 BK=32 ST=3"),
    # f32 mid sizes (every configuration timed pinned): the f32-panel ring
    # at 1024^3 (26 us against 29 on the best tile that does not split K),
    # the 128 x 256 ring at 2000^3 (154 us; the register-staged 128 x 64
    # tile chosen before, 185), the masked 256^2 ring at 3000^3 (463 us;
    # 128 x 256 on a block plus strips, chosen before, 511)
    ("f32", (1024, 1024, 1024), "BM=64 BN=128 BK=32 ST=3 WM=2 WN=2 GM=8 KS=3"),
    ("f32", (2000, 2000, 2000), "BM=128 BN=256 BK=16 ST=4 WM=2 WN=4"),
    ("f32", (3000, 3000, 3000), "BM=256 BN=256 BK=16 ST=3 WM=2 WN=4"),
    # f16r scored shape: the 256^2 half-depth ring
    ("f16r", (8192, 8192, 8192), "BM=256 BN=256 BK=32 ST=5 WM=4 WN=2"),
    # f16r few rows: the f32-panel ring rounding on load (64 rows: 32 x 64,
    # 17.5 us against 24 us before it; 512 rows: 128 x 256, 38 against 54)
    ("f16r", (64, 4096, 4096), "BM=32 BN=64 BK=32 ST=4"),
    ("f16r", (512, 4096, 4096), "BM=128 BN=256 BK=32 ST=3"),
    # f16r, few packed tiles for a deep K or a shallow K that the packing pass
    # dominates: the f32-panel ring (A/B of the library before and after the
    # rule: 1024 x 2048 x 4096 41 us against 56, 1024^2 x 8192 48 against 75,
    # 2048^2 x 512 12.8 against 18.8, 1448^2 x 4096 43 against 46); 1792^2 x
    # 4096 stays packed (46 us against 54 on the ring)
    ("f16r", (1024, 2048, 4096), "BM=128 BN=256 BK=32 ST=3 WM=2 WN=4 GM=8 KS=3"),
    ("f16r", (2048, 2048, 512), "BM=128 BN=128 BK=32 ST=3 WM=4 WN=2 GM=8 KS=3"),
    ("f16r", (1448, 1448, 4096), "BM=128 BN=256 BK=32 ST=3 WM=2 WN=4 GM=8 KS=3"),
    ("f16r", (1792, 1792, 4096), "BM=128 BN=128 BK=32 ST=5"),
    # f16r, K = 513-2048 on a grid of 128^2 tiles that fits one round in
    # 1024-deep slices: the 128^2 f32-panel ring (1792^2 x 1024 19.7 us
    # against 23.8 packed, 1280^2 x 2048 23.1 against 27.7); a whole K of
    # 2048 a tile stays packed (1792^2 x 2048 28 us against 32 on the ring)
    ("f16r", (1792, 1792, 1024), "BM=128 BN=128 BK=32 ST=3 WM=4 WN=2 GM=8 KS=3"),
    ("f16r", (1280, 1280, 2048), "BM=128 BN=128 BK=32 ST=3 WM=4 WN=2 GM=8 KS=3"),
    ("f16r", (1792, 1792, 2048), "BM=128 BN=128 BK=32 ST=5"),
    # K <= 1024 past one round of 128^2 tiles: the 256 x 128 ring, its long
    # side along the longer of M and N, while that grid fits one round
    # (2560^2 x 1024 29.0 us against 30.9 packed, 2048 x 4096 x 1024 29.9
    # against 32.1); 3072^2 x 1024 (288 tiles) stays packed (37 us against 50)
    ("f16r", (2560, 2560, 1024), "BM=256 BN=128 BK=32 ST=3 WM=4 WN=2 GM=8 KS=3"),
    ("f16r", (2048, 4096, 1024), "BM=128 BN=256 BK=32 ST=3 WM=2 WN=4 GM=8 KS=3"),
    ("f16r", (3072, 3072, 1024), "BM=128 BN=128 BK=32 ST=5"),
    # the f32-panel ring's 128 x 256 tile gives way to 128^2 from 6 slices
    # (512 x 1024 x 8192: 16 slices 49.9 us, 128^2 in 8 33.5), not at 5
    # (384 x 4096^2: 35.8 us against 39.8 on 128^2)
    ("f16r", (512, 1024, 8192), "BM=128 BN=128 BK=32 ST=3 WM=4 WN=2 GM=8 KS=3"),
    ("f16r", (384, 4096, 4096), "BM=128 BN=256 BK=32 ST=3 WM=2 WN=4 GM=8 KS=3"),
    # f16r mid sizes on the packed path (every half-depth ring timed pinned;
    # the pick within 2.3% of the fastest): 128^2 60 us at 1024 x 4096^2,
    # 100 at 2048^2 x 8192 and 194 at 4352^3 (256 x 128 70, 119 and 205),
    # with eight waves on a grid of one round (up to 512 tiles: 1792^3 29.7
    # us against 30.8 with four, 2048^3 33.2 against 34.6), four on a larger
    # one (4352^3 193 against 195);
    # 256 x 128 52 us at 2560^3, 76 at 1536 x 4096^2, 219 at 4608^3, 200 at
    # 4097^3 and 458 at 6144^3 (128^2: 55, 81, 232, 208, 465; 256^2: 68, 100,
    # 242, 220, 448); the 256^2 ring 89 us at 3072^3 (144 tiles; 256 x 128 in
    # runs 95)
    ("f16r", (1024, 4096, 4096), "BM=128 BN=128 BK=32 ST=5 WM=4 WN=2"),
    ("f16r", (2048, 2048, 8192), "BM=128 BN=128 BK=32 ST=5 WM=4 WN=2"),
    ("f16r", (1792, 1792, 1792), "BM=128 BN=128 BK=32 ST=5 WM=4 WN=2"),
    ("f16r", (2048, 2048, 2048), "BM=128 BN=128 BK=32 ST=5 WM=4 WN=2"),
    ("f16r", (4352, 4352, 4352), "BM=128 BN=128 BK=32 ST=5 WM=2 WN=2"),
    ("f16r", (2560, 2560, 2560), "BM=256 BN=128 BK=32 ST=4 WM=4 WN=2"),
    ("f16r", (1536, 4096, 4096), "BM=256 BN=128 BK=32 ST=4 WM=4 WN=2"),
    ("f16r", (4608, 4608, 4608), "BM=256 BN=128 BK=32 ST=4 WM=4 WN=2"),
    ("f16r", (4097, 4097, 4097), "BM=256 BN=128 BK=32 ST=4 WM=4 WN=2"),
    ("f16r", (6144, 6144, 6144), "BM=256 BN=128 BK=32 ST=4 WM=4 WN=2"),
    ("f16r", (3072, 3072, 3072), "BM=256 BN=256 BK=32 ST=5 WM=4 WN=2"),
]


@pytest.mark.parametrize("mode,shape,want", HEURISTIC_PICKS)
def test_heuristic_picks_the_measured_best(mode, shape, want):
    g.cache_clear()
    got = g.get_config(mode, *shape, beta=0.0)
    assert got.endswith("source=heuristic") and got.startswith(want), (mode, shape, got)


# Few rows with B stored N x K (op(B) = B^T) at K = N = 4096: the f32-panel
# ring on 16 x 128 tiles (f16r 15.9-16.2 us against 19.3-21.9 on the few-rows
# configuration at 1 to 16 rows, f32 18.2-18.5 against 19.3-20.6); with A
# also stored transposed and M % 4 != 0 the ring does not take the call and
# the few-rows configuration stays (f16r TT 1 row 18.9 us).
@pytest.mark.parametrize("mode", ["f32", "f16r"])
@pytest.mark.parametrize("M,ta,want", [
    (1, False, "BM=16 BN=128 BK=32 ST=4 WM=1 WN=2 GM=8 KS=3"),
    (16, False, "BM=16 BN=128 BK=32 ST=4 WM=1 WN=2 GM=8 KS=3"),
    (8, True, "BM=16 BN=128 BK=32 ST=4 WM=1 WN=2 GM=8 KS=3"),
    (2, True, "BM=16 BN=64 BK=64 ST=1"),
])
def test_heuristic_few_rows_with_b_transposed(mode, M, ta, want):
    g.cache_clear()
    got = g.get_config(mode, M, 4096, 4096, beta=0.0, transa=ta, transb=True)
    assert got.endswith("source=heuristic") and got.startswith(want), (mode, M, ta, got)
    # the plain layout keeps the few-rows configuration
    assert g.get_config(mode, M, 4096, 4096, beta=0.0).startswith("BM=16 BN=64 BK=64")
