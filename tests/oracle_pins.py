"""Pins for the CPU oracle: checks against things other than the oracle itself.

Each pin takes a reference function ``ref(mode, A, B, C, alpha, beta) ->
(Cref, W)`` and raises AssertionError when it disagrees with what the pages
and the mathematics fix.  ``tests/test_oracle.py`` runs every pin on the real
oracle (all must pass) and on planted mistakes (each mistake must be caught by
at least one pin).

Sources of truth used here, none of which is the oracle:
  * exact rational arithmetic (``fractions.Fraction``) on tiny shapes;
  * numpy float64 matrix products;
  * closed forms: alpha = 0, identity A or B, all-ones A;
  * exact integer arithmetic (numpy int64);
  * numpy's float32 -> float16 conversion (IEEE round to nearest even) for
    the operand rounding of the f16r mode.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

from workloads import make_inputs, small_integers

EPS = 2.0 ** -52


def np_round_f16(x):
    """Operand rounding of the f16r mode, by numpy (independent of the oracle)."""
    with np.errstate(over="ignore"):
        return np.asarray(x, dtype=np.float32).astype(np.float16).astype(np.float64)


def np_operand(mode, x):
    return np_round_f16(x) if mode == "f16r" else np.asarray(x, dtype=np.float64)


def pin_bruteforce_fraction(ref, mode, shapes=((1, 1, 1), (2, 3, 5), (3, 2, 1), (5, 7, 3),
                                              (7, 5, 8), (8, 8, 8), (1, 8, 7), (3, 5, 2)),
                            seed=0):
    """Exact rational result on tiny shapes; the oracle must agree within
    K * 2^-52 relative to W (its double sums) plus one double rounding."""
    rng = np.random.default_rng(seed)
    for (M, N, K) in shapes:
        A = (rng.uniform(-4, 4, size=(M, K)) * rng.choice([-1, 1], size=(M, K))).astype(np.float32)
        B = rng.standard_normal(size=(K, N)).astype(np.float32) * np.float32(3.0)
        C = rng.uniform(-2, 2, size=(M, N)).astype(np.float32)
        alpha = float(np.float32(rng.uniform(-2, 2)))
        beta = float(np.float32(rng.uniform(-2, 2)))
        rA = np_operand(mode, A)
        rB = np_operand(mode, B)
        Cref, W = ref(mode, A, B, C, alpha, beta)
        for i in range(M):
            for j in range(N):
                s = sum((Fraction(float(rA[i, k])) * Fraction(float(rB[k, j])) for k in range(K)),
                        Fraction(0))
                exact = Fraction(alpha) * s + Fraction(beta) * Fraction(float(C[i, j]))
                w = abs(alpha) * sum(abs(float(rA[i, k])) * abs(float(rB[k, j])) for k in range(K)) \
                    + abs(beta) * abs(float(C[i, j]))
                err = abs(Fraction(float(Cref[i, j])) - exact)
                bound = Fraction((K + 4) * EPS * w)
                assert err <= bound, (mode, (M, N, K), i, j, float(err), float(bound))
                assert abs(W[i, j] - w) <= (K + 4) * EPS * w, (mode, (M, N, K), i, j)


def pin_numpy_matmul(ref, mode, M=256, N=256, K=256, alpha=1.5, beta=0.5, seed=0,
                     dist="uniform"):
    """numpy float64 matmul of the (rounded) operands; agreement to 1e-12 of W."""
    A, B, C = make_inputs(M, N, K, dist, seed)
    rA, rB = np_operand(mode, A), np_operand(mode, B)
    exp = alpha * (rA @ rB) + beta * C.astype(np.float64)
    wexp = abs(alpha) * (np.abs(rA) @ np.abs(rB)) + abs(beta) * np.abs(C.astype(np.float64))
    Cref, W = ref(mode, A, B, C, alpha, beta)
    assert np.all(np.abs(Cref - exp) <= 1e-12 * wexp), float(np.max(np.abs(Cref - exp) / wexp))
    assert np.all(np.abs(W - wexp) <= 1e-12 * wexp)


def pin_alpha_zero(ref, mode, M=33, N=17, K=9, beta=-0.75, seed=3):
    """alpha = 0: C = beta * C exactly (a single product of two f32 values)."""
    A, B, C = make_inputs(M, N, K, "normal", seed)
    Cref, W = ref(mode, A, B, C, 0.0, beta)
    assert np.array_equal(Cref, beta * C.astype(np.float64))
    assert np.array_equal(W, abs(beta) * np.abs(C.astype(np.float64)))


def pin_beta_zero_ignores_c(ref, mode, M=9, N=11, K=13, seed=4):
    """beta = 0: C is not read, so NaN or infinity in C does not reach the result."""
    A, B, _ = make_inputs(M, N, K, "uniform", seed)
    C = np.full((M, N), np.nan, dtype=np.float32)
    C[::2, ::3] = np.inf
    Cref, W = ref(mode, A, B, C, 1.25, 0.0)
    exp = 1.25 * (np_operand(mode, A) @ np_operand(mode, B))
    assert np.all(np.isfinite(Cref)) and np.all(np.isfinite(W))
    assert np.all(np.abs(Cref - exp) <= 1e-12 * np.abs(exp).max())


def pin_identity(ref, mode, n=24, N=40, seed=5):
    """A = I: C = alpha * r(B) + beta * C exactly; B = I: C = alpha * r(A) + beta * C.
    In the f16r mode with alpha = 1, beta = 0 the result is numpy's float16 of
    the other operand, bit for bit, which fixes the operand rounding."""
    rng = np.random.default_rng(seed)
    # values that exercise the rounding: ties, subnormals, near the largest finite
    specials = np.array([1 + 2 ** -11, 1 + 3 * 2 ** -11, -(1 + 2 ** -11), 2 ** -24, 2 ** -25,
                         1.5 * 2 ** -24, 2 ** -14 - 2 ** -25, 65504.0, 65519.0, -65519.0,
                         0.1, -0.3, 1e-6, 3.14159265], dtype=np.float32)
    B = rng.standard_normal(size=(n, N)).astype(np.float32)
    B.ravel()[: specials.size] = specials
    A = np.eye(n, dtype=np.float32)
    C = rng.uniform(-1, 1, size=(n, N)).astype(np.float32)
    for alpha, beta in ((1.0, 0.0), (2.0, 0.5), (-0.5, -1.0)):
        Cref, _ = ref(mode, A, B, C, alpha, beta)
        exp = alpha * np_operand(mode, B) + (beta * C.astype(np.float64) if beta else 0.0)
        assert np.array_equal(Cref, exp), (mode, alpha, beta)
    # right identity: rounding of A
    A2 = rng.standard_normal(size=(N, n)).astype(np.float32)
    A2.ravel()[: specials.size] = specials
    C2 = np.zeros((N, n), dtype=np.float32)
    Cref, _ = ref(mode, A2, np.eye(n, dtype=np.float32), C2, 1.0, 0.0)
    assert np.array_equal(Cref, np_operand(mode, A2)), mode


def pin_all_ones(ref, mode, M=7, N=23, K=31, seed=6):
    """A = all ones: every row of A@B is the vector of B's column sums (exact
    for integer B)."""
    rng = np.random.default_rng(seed)
    B = rng.integers(-50, 51, size=(K, N)).astype(np.float32)
    A = np.ones((M, K), dtype=np.float32)
    C = np.zeros((M, N), dtype=np.float32)
    Cref, _ = ref(mode, A, B, C, 1.0, 0.0)
    colsum = B.astype(np.int64).sum(axis=0).astype(np.float64)
    assert np.array_equal(Cref, np.broadcast_to(colsum, (M, N)))


def pin_small_integers(ref, mode, M=37, N=29, K=53, seed=7):
    """Entries in [-8, 8]: the exact integer result, bit for bit."""
    A, B, C = small_integers(M, N, K, seed=seed)
    for alpha, beta in ((1.0, 1.0), (2.0, -1.0), (-1.0, 0.5), (0.5, 0.0)):
        Cref, _ = ref(mode, A, B, C, alpha, beta)
        prod = A.astype(np.int64) @ B.astype(np.int64)
        exp = alpha * prod.astype(np.float64) + beta * C.astype(np.float64)
        assert np.array_equal(Cref, exp), (mode, alpha, beta)


def pin_leading_dims(ref, mode, M=19, N=21, K=23, seed=8):
    """Padded leading dimensions read the same logical matrices."""
    A, B, C = make_inputs(M, N, K, "uniform", seed, lda=K + 3, ldb=N + 5, ldc=N + 1)
    Ad, Bd, Cd = (np.ascontiguousarray(x) for x in (A, B, C))
    r1 = ref(mode, A, B, C, 0.5, 2.0)
    r2 = ref(mode, Ad, Bd, Cd, 0.5, 2.0)
    assert np.array_equal(r1[0], r2[0]) and np.array_equal(r1[1], r2[1])


ALL_PINS = [pin_bruteforce_fraction, pin_numpy_matmul, pin_alpha_zero, pin_beta_zero_ignores_c,
            pin_identity, pin_all_ones, pin_small_integers, pin_leading_dims]
