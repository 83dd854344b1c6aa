"""CPU tests of the oracle against its pins (no GPU needed)."""
from __future__ import annotations

import os

import numpy as np
import pytest
import torch

import oracle
from tests import oracle_pins as pins
from workloads import make_inputs, small_integers

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

MODES = ["f32", "f16r"]


def _oracle_ref(mode, A, B, C, alpha, beta):
    return oracle.gemm(mode, A, B, C, alpha, beta)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_meets_pin(pin, mode):
    pin(_oracle_ref, mode)


# ---------------------------------------------------------------------------
# Planted mistakes: each must be caught by at least one pin.  The mutants are
# small numpy re-implementations of the reference with one mistake each; the
# unmutated one must pass every pin, which shows the harness itself is sound.
# ---------------------------------------------------------------------------

def _rtz_f16(x):
    """Round toward zero to f16 (a plausible wrong rounding mode)."""
    x = np.asarray(x, dtype=np.float32)
    with np.errstate(over="ignore"):
        h = x.astype(np.float16).astype(np.float64)
    too_big = np.abs(h) > np.abs(x.astype(np.float64))
    # step one f16 ulp toward zero where RNE rounded away from zero
    h2 = np.where(too_big, np.nextafter(h.astype(np.float16), np.float16(0)).astype(np.float64), h)
    return h2


def _mutant(kind):
    def ref(mode, A, B, C, alpha, beta):
        A = np.asarray(A, dtype=np.float32)
        B = np.asarray(B, dtype=np.float32)
        C = np.asarray(C, dtype=np.float32)
        if mode == "f16r" and kind == "no_rounding":
            rA, rB = A.astype(np.float64), B.astype(np.float64)
        elif mode == "f16r" and kind == "rtz_rounding":
            rA, rB = _rtz_f16(A), _rtz_f16(B)
        else:
            rA, rB = pins.np_operand(mode, A), pins.np_operand(mode, B)
        if kind == "drop_last_k" and rA.shape[1] > 1:
            rA = rA[:, :-1]
            rB = rB[:-1, :]
        if kind == "reversed_columns":
            rB = rB[:, ::-1]
        if kind == "f32_accumulate":
            P = np.zeros((rA.shape[0], rB.shape[1]), dtype=np.float32)
            for k in range(rA.shape[1]):
                P += np.outer(rA[:, k], rB[k, :]).astype(np.float32)
            P = P.astype(np.float64)
        else:
            P = rA @ rB
        Mg = np.abs(rA) @ np.abs(rB)
        c = C.astype(np.float64)
        if kind == "literal_beta_times_c":
            with np.errstate(invalid="ignore"):
                Cref = alpha * P + beta * c
                W = abs(alpha) * Mg + abs(beta) * np.abs(c)
        else:
            bsign = -1.0 if kind == "beta_sign" else 1.0
            Cref = alpha * P + (bsign * beta * c if beta != 0 else 0.0)
            W = abs(alpha) * Mg + (abs(beta) * np.abs(c) if beta != 0 else 0.0)
        if kind == "alpha_scales_c":
            Cref = alpha * (P + (beta * c if beta != 0 else 0.0))
        return np.ascontiguousarray(Cref, dtype=np.float64), np.ascontiguousarray(W + 0.0)
    ref.__name__ = f"mutant_{kind}"
    return ref


def _caught(ref, modes):
    for mode in modes:
        for pin in pins.ALL_PINS:
            try:
                pin(ref, mode)
            except AssertionError:
                return True
    return False


def test_unmutated_numpy_reference_passes_all_pins():
    ref = _mutant("none")
    for mode in MODES:
        for pin in pins.ALL_PINS:
            pin(ref, mode)


@pytest.mark.parametrize("kind,modes", [
    ("drop_last_k", MODES),
    ("reversed_columns", MODES),
    ("beta_sign", MODES),
    ("alpha_scales_c", MODES),
    ("f32_accumulate", ["f32"]),
    ("literal_beta_times_c", MODES),
    ("no_rounding", ["f16r"]),
    ("rtz_rounding", ["f16r"]),
])
def test_pins_catch_planted_mistake(kind, modes):
    assert _caught(_mutant(kind), modes), f"no pin caught mutant {kind}"


# ---------------------------------------------------------------------------
# The operand rounding of the f16r mode.
# ---------------------------------------------------------------------------

def _golden_f16_cases():
    rows = []
    with open(os.path.join(GOLDEN, "f16_rne_cases.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            a, b = line.split()[:2]
            rows.append((int(a, 16), int(b, 16), line))
    return rows


@pytest.mark.parametrize("f32_bits,f16_bits,line", _golden_f16_cases(),
                         ids=lambda v: v if isinstance(v, str) else None)
def test_rn_f16_golden_case(f32_bits, f16_bits, line):
    x = np.array([f32_bits], dtype=np.uint32).view(np.float32)
    assert int(oracle.rn_f16_bits(x)[0]) == f16_bits, line


def _torch_f16_bits(f):
    t = torch.from_numpy(f)
    return t.to(torch.float16).view(torch.int16).numpy().view(np.uint16)


def test_rn_f16_exhaustive_over_the_f16_range():
    """Every positive f32 whose exponent lies where binary16 results are not
    trivially 0 or infinity (|x| in [2^-26, 2^17)), against the CPU's own
    float16 conversion (torch on x86, IEEE round to nearest even)."""
    lo = 101 << 23          # 2^-26
    hi = 144 << 23          # 2^17
    step = 1 << 25
    for base in range(lo, hi, step):
        u = np.arange(base, min(base + step, hi), dtype=np.uint32)
        f = u.view(np.float32)
        got = oracle.rn_f16_bits(f)
        exp = _torch_f16_bits(f)
        bad = np.flatnonzero(got != exp)
        assert bad.size == 0, f"first mismatch at f32 bits {u[bad[0]]:#010x}"


def test_rn_f16_strided_over_all_bit_patterns():
    """All sign/exponent combinations (both signs), strided mantissas, NaNs."""
    u = np.arange(0, 1 << 32, 4099, dtype=np.uint64).astype(np.uint32)
    f = u.view(np.float32)
    got = oracle.rn_f16_bits(f)
    exp = _torch_f16_bits(f)
    nan = np.isnan(f)
    assert np.array_equal(got[~nan], exp[~nan])
    h = got[nan]
    assert np.all(((h & 0x7c00) == 0x7c00) & ((h & 0x3ff) != 0))


def test_f16_bits_to_double_is_exact():
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    finite = (bits & 0x7c00) != 0x7c00
    got = oracle.f16_bits_to_float64(bits[finite][::7])
    exp = bits[finite][::7].view(np.float16).astype(np.float64)
    assert np.array_equal(got, exp)


# ---------------------------------------------------------------------------
# The sampled-entry and streaming-check entry points.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("mode", MODES)
def test_entries_match_full_reference_bitwise(mode):
    A, B, C = make_inputs(61, 67, 71, "normal", seed=2, lda=75, ldb=70, ldc=69)
    Cref, W = oracle.gemm(mode, A, B, C, 0.75, -0.25)
    rng = np.random.default_rng(0)
    rows = rng.integers(0, 61, size=300)
    cols = rng.integers(0, 67, size=300)
    ref, w = oracle.entries(mode, A, B, C, 0.75, -0.25, rows, cols)
    assert np.array_equal(ref, Cref[rows, cols]) and np.array_equal(w, W[rows, cols])


@pytest.mark.parametrize("mode", MODES)
def test_check_accepts_rounded_reference_and_flags_planted_errors(mode):
    A, B, C = make_inputs(48, 40, 64, "uniform", seed=9)
    Cref, W = oracle.gemm(mode, A, B, C, 1.5, 0.5)
    got = Cref.astype(np.float32)
    st = oracle.check(mode, A, B, C, 1.5, 0.5, got)
    assert st["n_fail"] == 0 and st["max_ratio"] < 1e-6
    tol = oracle.TOL[mode]
    bad = got.copy()
    bad[3, 5] = np.float32(Cref[3, 5] + 3 * tol * W[3, 5])
    bad[47, 39] = np.nan
    st = oracle.check(mode, A, B, C, 1.5, 0.5, bad)
    assert st["n_fail"] == 2 and np.isinf(st["max_ratio"])
    band = oracle.check(mode, A, B, C, 1.5, 0.5, bad, rows=(0, 3))
    assert band["n_fail"] == 0


def test_check_error_summaries_hand_example():
    """The lab's two error summaries on a case worked by hand: A = I, B =
    diag(3, 4), C = 0, alpha 1, beta 0, so the reference is diag(3, 4); one
    element off by 1 gives max|err| / max|ref| = 1/4 and
    ||err||_F / ||ref||_F = 1 / sqrt(9 + 16) = 1/5."""
    A = np.eye(2, dtype=np.float32)
    B = np.array([[3.0, 0.0], [0.0, 4.0]], dtype=np.float32)
    C = np.zeros((2, 2), dtype=np.float32)
    got = np.array([[3.0, 1.0], [0.0, 4.0]], dtype=np.float32)
    for mode in MODES:
        st = oracle.check(mode, A, B, C, 1.0, 0.0, got, tol=1.0)
        assert st["err_max_norm"] == 0.25, st
        assert st["err_fro"] == 0.2, st


@pytest.mark.parametrize("mode", MODES)
def test_check_error_summaries_match_numpy_norms(mode):
    """err_max_norm and err_fro against numpy's norms of planted errors, on
    small-integer inputs whose exact product numpy's float64 matmul gives
    (every partial sum is an integer below 2^53), so the reference side is
    independent of the oracle."""
    A, B, C = small_integers(37, 29, 53, seed=21)
    alpha, beta = 2.0, -0.5
    ref = alpha * (A.astype(np.float64) @ B.astype(np.float64)) + beta * C.astype(np.float64)
    rng = np.random.default_rng(22)
    d = np.zeros_like(ref)
    pos = rng.integers(0, ref.size, size=40)
    d.flat[pos] = rng.uniform(-3.0, 3.0, size=40)
    got = (ref + d).astype(np.float32)
    d = got.astype(np.float64) - ref            # the error actually planted, after rounding
    st = oracle.check(mode, A, B, C, alpha, beta, got, tol=1.0)
    want_max = np.abs(d).max() / np.abs(ref).max()
    want_fro = np.linalg.norm(d) / np.linalg.norm(ref)
    assert st["err_max_norm"] == pytest.approx(want_max, rel=1e-12)
    assert st["err_fro"] == pytest.approx(want_fro, rel=1e-12)
    # a reference without error reads zero in both
    st0 = oracle.check(mode, A, B, C, alpha, beta, ref.astype(np.float32), tol=1.0)
    assert st0["err_max_norm"] == 0.0 and st0["err_fro"] == 0.0


def test_check_requires_exact_zero_where_w_is_zero():
    A = np.zeros((4, 4), dtype=np.float32)
    B = np.zeros((4, 4), dtype=np.float32)
    C = np.zeros((4, 4), dtype=np.float32)
    got = np.zeros((4, 4), dtype=np.float32)
    assert oracle.check("f32", A, B, C, 1.0, 1.0, got)["n_fail"] == 0
    got[1, 1] = 1e-30
    assert oracle.check("f32", A, B, C, 1.0, 1.0, got)["n_fail"] == 1


def test_degenerate_shapes():
    A = np.zeros((0, 5), dtype=np.float32)
    B = np.zeros((5, 3), dtype=np.float32)
    C = np.zeros((0, 3), dtype=np.float32)
    Cref, W = oracle.gemm("f32", A, B, C, 1.0, 1.0)
    assert Cref.shape == (0, 3)
    # K = 0: the product term is empty, C = beta * C
    A = np.zeros((3, 0), dtype=np.float32)
    B = np.zeros((0, 4), dtype=np.float32)
    C = np.arange(12, dtype=np.float32).reshape(3, 4)
    Cref, _ = oracle.gemm("f16r", A, B, C, 2.0, -0.5)
    assert np.array_equal(Cref, -0.5 * C.astype(np.float64))
