"""Pins of the CPU oracle against facts that do not come from the oracle.

Each pin is a plain function that raises AssertionError when the oracle
given to it is wrong.  ``test_oracle.py`` runs them on the real oracle and on
builds with planted mistakes (a dropped term, a transposed operand, a sign
error, an ignored leading dimension), each of which must trip at least one.

What pins what:
  * exact rational arithmetic on tiny inputs (brute force with Fraction);
  * closed forms: B = I gives alpha A + beta C0, A = I gives alpha B + beta C0,
    all-ones operands give alpha K + beta C0;
  * exact integers: entries in [-4, 4] make every sum an integer, compared
    with numpy's int64 product;
  * linearity in alpha and beta;
  * transpose identity (A B)^T = B^T A^T;
  * leading dimensions: NaN-padded rows give the packed result;
  * the read conventions for beta == 0, alpha == 0 and K == 0;
  * the fused epilogue (bias + ReLU): a hand-worked example, the bias axis
    (alpha = beta = 0 leaves the bias in every row), the exact identity
    relu(v) - relu(-v) = v under negation of alpha, beta and the bias, the
    bound, NaN/inf handling, and entries against the full result.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

import oracle
from fp32_gemm_06_amd import inputs

U = 2.0 ** -53


def _varied(g, shape):
    """fp32 values with a spread of exponents and both signs."""
    m = g.uniform(0.5, 1.0, size=shape)
    e = g.integers(-6, 7, size=shape)
    s = np.where(g.random(size=shape) < 0.5, -1.0, 1.0)
    return (s * m * np.exp2(e)).astype(np.float32)


def _exact(A, B, C0, alpha, beta, M, N, K):
    """Exact rational alpha * A B + beta * C0 with the read conventions."""
    out = [[Fraction(0)] * N for _ in range(M)]
    fa, fb = Fraction(float(np.float32(alpha))), Fraction(float(np.float32(beta)))
    for i in range(M):
        for j in range(N):
            s = Fraction(0)
            if alpha != 0 and K > 0:
                for k in range(K):
                    s += Fraction(float(A[i, k])) * Fraction(float(B[k, j]))
            v = fa * s
            if beta != 0:
                v += fb * Fraction(float(C0[i, j]))
            out[i][j] = v
    return out


def pin_bruteforce(lib):
    g = inputs.rng(7)
    shapes = [(1, 1, 1), (2, 3, 4), (3, 2, 5), (4, 4, 1), (5, 3, 7), (1, 6, 3), (3, 5, 8)]
    for (M, N, K) in shapes:
        for (alpha, beta) in [(1.0, 0.0), (0.75, -1.5), (-2.0, 0.5)]:
            A, B, C0 = _varied(g, (M, K)), _varied(g, (K, N)), _varied(g, (M, N))
            got = oracle.sgemm(A, B, C0, alpha, beta, lib=lib)
            ex = _exact(A, B, C0, alpha, beta, M, N, K)
            bnd = oracle.bound(A, B, C0, alpha, beta, lib=lib)
            for i in range(M):
                for j in range(N):
                    # bound itself pinned: |alpha| sum|a||b| + |beta||c0| exactly
                    eb = abs(Fraction(float(np.float32(alpha)))) * sum(
                        (abs(Fraction(float(A[i, k]))) * abs(Fraction(float(B[k, j])))
                         for k in range(K)), Fraction(0))
                    if beta != 0:
                        eb += abs(Fraction(float(np.float32(beta)))) * abs(Fraction(float(C0[i, j])))
                    assert abs(Fraction(bnd[i, j]) - eb) <= Fraction((K + 2) * U) * eb, \
                        ("bound", M, N, K, i, j)
                    err = abs(Fraction(got[i, j]) - ex[i][j])
                    assert err <= Fraction((K + 3) * U) * eb + Fraction(2.0 ** -1074), \
                        ("value", M, N, K, alpha, beta, i, j, float(err))


def pin_identity(lib):
    g = inputs.rng(11)
    for (M, n) in [(7, 9), (16, 16), (33, 5)]:
        A, C0 = inputs.uniform(g, (M, n)), inputs.uniform(g, (M, n))
        for (alpha, beta) in [(1.0, 0.0), (1.0, 0.5), (-0.5, 2.0)]:
            got = oracle.sgemm(A, inputs.identity(n), C0, alpha, beta, lib=lib)
            want = np.float64(alpha) * A.astype(np.float64)
            if beta != 0:
                want = want + np.float64(beta) * C0.astype(np.float64)
            assert np.array_equal(got, want), ("B = I", M, n, alpha, beta)
        # A = I: C = alpha B + beta C0
        B = inputs.uniform(g, (M, n))
        C1 = inputs.uniform(g, (M, n))
        got = oracle.sgemm(inputs.identity(M), B, C1, 0.5, 1.0, lib=lib)
        want = 0.5 * B.astype(np.float64) + C1.astype(np.float64)
        assert np.array_equal(got, want), ("A = I", M, n)


def pin_ones(lib):
    g = inputs.rng(13)
    for (M, N, K) in [(3, 5, 1), (4, 7, 128), (2, 3, 4092)]:
        C0 = inputs.uniform(g, (M, N))
        for (alpha, beta) in [(1.0, 0.0), (2.0, 0.5), (0.5, 1.0)]:
            got = oracle.sgemm(inputs.ones(M, K), inputs.ones(K, N), C0, alpha, beta, lib=lib)
            want = np.full((M, N), np.float64(alpha) * K)
            if beta != 0:
                want = want + np.float64(beta) * C0.astype(np.float64)
            assert np.array_equal(got, want), ("ones", M, N, K, alpha, beta)


def pin_integers(lib):
    for seed, (M, N, K) in enumerate([(9, 13, 17), (31, 7, 64), (5, 40, 33), (64, 64, 64)]):
        A, B, C0 = inputs.random_case(100 + seed, M, N, K, kind="int")
        prod = A.astype(np.int64) @ B.astype(np.int64)   # exact integer product
        got = oracle.sgemm(A, B, C0, 1.0, 0.5, lib=lib)
        want = prod.astype(np.float64) + 0.5 * C0.astype(np.float64)
        assert np.array_equal(got, want), ("int", M, N, K)


def pin_linearity(lib):
    A, B, C0 = inputs.random_case(21, 19, 23, 29, kind="normal")
    base = oracle.sgemm(A, B, None, 1.0, 0.0, lib=lib)
    bnd1 = oracle.bound(A, B, C0, 1.0, 1.0, lib=lib)
    for (alpha, beta) in [(0.5, 1.0), (-3.0, 0.25), (2.0, -1.0)]:
        got = oracle.sgemm(A, B, C0, alpha, beta, lib=lib)
        want = alpha * base + beta * C0.astype(np.float64)
        scale = max(abs(alpha), abs(beta)) * bnd1
        assert np.all(np.abs(got - want) <= 8 * U * scale), ("linearity", alpha, beta)


def pin_transpose(lib):
    A, B, C0 = inputs.random_case(31, 12, 17, 9, kind="uniform")
    got = oracle.sgemm(A, B, C0, 1.5, -0.5, lib=lib)
    At, Bt, C0t = (np.ascontiguousarray(x.T) for x in (A, B, C0))
    gotT = oracle.sgemm(Bt, At, C0t, 1.5, -0.5, lib=lib)
    # the same products summed in the same k order: bit-identical
    assert np.array_equal(got, gotT.T), "transpose identity"


def pin_leading_dims(lib):
    M, N, K = 6, 10, 7
    A, B, C0 = inputs.random_case(41, M, N, K, kind="uniform")
    Ap, Bp, Cp = inputs.random_case(41, M, N, K, kind="uniform", lda=K + 5, ldb=N + 3, ldc=N + 6)
    assert np.array_equal(A, Ap) and np.array_equal(B, Bp) and np.array_equal(C0, Cp)
    want = oracle.sgemm(A, B, C0, 1.0, 0.5, lib=lib)
    got = oracle.sgemm(Ap, Bp, Cp, 1.0, 0.5, lib=lib)
    assert np.array_equal(got, want), "leading dimensions"
    rows = np.array([0, 5, 3, 5], dtype=np.int32)
    cols = np.array([0, 9, 4, 0], dtype=np.int32)
    ent = oracle.sgemm_entries(rows, cols, Ap, Bp, Cp, 1.0, 0.5, lib=lib)
    assert np.array_equal(ent, want[rows, cols]), "entries"
    bfull = oracle.bound(A, B, C0, 1.0, 0.5, lib=lib)
    bent = oracle.bound_entries(rows, cols, Ap, Bp, Cp, 1.0, 0.5, lib=lib)
    assert np.array_equal(bent, bfull[rows, cols]), "bound entries"


def pin_read_conventions(lib):
    M, N, K = 4, 5, 6
    A, B, C0 = inputs.random_case(51, M, N, K, kind="uniform")
    nanC = np.full((M, N), np.nan, dtype=np.float32)
    got = oracle.sgemm(A, B, nanC, 1.0, 0.0, lib=lib)
    assert np.all(np.isfinite(got)), "beta == 0 must not read C0"
    nanA = np.full((M, K), np.nan, dtype=np.float32)
    got = oracle.sgemm(nanA, B, C0, 0.0, 2.0, lib=lib)
    assert np.array_equal(got, 2.0 * C0.astype(np.float64)), "alpha == 0 must not read A"
    got = oracle.sgemm(np.zeros((M, 0), np.float32), np.zeros((0, N), np.float32), C0, 1.0, -1.0,
                       K=0, lib=lib)
    assert np.array_equal(got, -C0.astype(np.float64)), "K == 0 gives beta C0"


# ---- fused epilogue: act(alpha A B + beta C0 + bias[j]) -------------------

def pin_epilogue_worked_example(lib):
    """By hand: A = [1 2 3], B columns (1, 0, -1) and (0, 1, -1), so
    A B = [1 - 3, 2 - 3] = [-2, -1]."""
    A = np.array([[1, 2, 3]], np.float32)
    B = np.array([[1, 0], [0, 1], [-1, -1]], np.float32)
    bias = np.array([1, 5], np.float32)
    # [-2 + 1, -1 + 5] = [-1, 4]; ReLU clears the negative one
    assert np.array_equal(oracle.sgemm_fused(A, B, None, 1.0, 0.0, bias, 0, lib=lib), [[-1, 4]])
    assert np.array_equal(oracle.sgemm_fused(A, B, None, 1.0, 0.0, bias, 1, lib=lib), [[0, 4]])
    # with C0 = [3, -10], beta = 1/2: [-2 + 1.5 + 1, -1 - 5 + 5] = [0.5, -1]
    C0 = np.array([[3, -10]], np.float32)
    assert np.array_equal(oracle.sgemm_fused(A, B, C0, 1.0, 0.5, bias, 1, lib=lib), [[0.5, 0]])
    assert np.array_equal(oracle.sgemm_fused(A, B, C0, 1.0, 0.5, None, 1, lib=lib), [[0, 0]])
    # tolerance scale: |A||B| = [1 + 3, 2 + 3], plus |bias|
    assert np.array_equal(oracle.bound_fused(A, B, None, 1.0, 0.0, -bias, lib=lib), [[5, 10]])


def pin_epilogue_bias_axis(lib):
    """alpha = beta = 0 leaves act(bias[j]) in every row: one bias value per
    column of C, the same for all rows."""
    M, N, K = 3, 5, 4
    bias = np.array([-2.5, 1.0, 0.0, 7.0, -0.25], np.float32)
    A, B, _ = inputs.random_case(61, M, N, K, kind="int")
    for act, want in ((0, bias.astype(np.float64)), (1, np.array([0, 1, 0, 7, 0], np.float64))):
        got = oracle.sgemm_fused(A, B, None, 0.0, 0.0, bias, act, lib=lib)
        assert np.array_equal(got, np.tile(want, (M, 1))), ("bias axis", act)


def pin_epilogue_relu_identity(lib):
    """relu(v) - relu(-v) = v exactly, and negating alpha, beta and the bias
    negates v: the ReLU results at (alpha, beta, bias) and (-alpha, -beta,
    -bias) must differ by the identity-activation result.  Integer data keep
    every value exact; the identity result minus the plain product is the
    bias, row by row; ReLU results are never negative."""
    M, N, K = 6, 7, 9
    A, B, C0 = inputs.random_case(62, M, N, K, kind="int")
    bias = inputs.rng(63).integers(-30, 31, size=N).astype(np.float32)
    for alpha, beta in ((1.0, 0.5), (-2.0, 1.0), (3.0, 0.0)):
        lin = oracle.sgemm_fused(A, B, C0, alpha, beta, bias, 0, lib=lib)
        pos = oracle.sgemm_fused(A, B, C0, alpha, beta, bias, 1, lib=lib)
        neg = oracle.sgemm_fused(A, B, C0, -alpha, -beta, -bias, 1, lib=lib)
        assert np.array_equal(pos - neg, lin), ("relu identity", alpha, beta)
        assert np.all(pos >= 0), "relu result negative"
        plain = oracle.sgemm(A, B, C0, alpha, beta, lib=lib)
        assert np.array_equal(lin - plain, np.tile(bias.astype(np.float64), (M, 1))), "bias add"
        bnd = oracle.bound_fused(A, B, C0, alpha, beta, bias, lib=lib)
        assert np.array_equal(bnd - oracle.bound(A, B, C0, alpha, beta, lib=lib),
                              np.tile(np.abs(bias).astype(np.float64), (M, 1))), "bound"


def pin_epilogue_special_values(lib):
    """NaN passes through the ReLU (it is not below zero); -inf becomes 0."""
    A = np.zeros((2, 1), np.float32)
    B = np.zeros((1, 2), np.float32)
    C0 = np.array([[np.nan, -np.inf], [np.inf, -0.0]], np.float32)
    got = oracle.sgemm_fused(A, B, C0, 1.0, 1.0, None, 1, lib=lib)
    assert np.isnan(got[0, 0]) and got[0, 1] == 0.0 and got[1, 0] == np.inf and got[1, 1] == 0.0


def pin_epilogue_entries(lib):
    M, N, K = 9, 11, 5
    A, B, C0 = inputs.random_case(64, M, N, K, kind="uniform")
    bias = inputs.uniform(inputs.rng(65), (N,))
    rows = np.array([0, 3, 8, 8, 5], np.int32)
    cols = np.array([10, 0, 4, 10, 7], np.int32)
    for act in (0, 1):
        full = oracle.sgemm_fused(A, B, C0, 1.5, -0.5, bias, act, lib=lib)
        ent = oracle.sgemm_fused_entries(rows, cols, A, B, C0, 1.5, -0.5, bias, act, lib=lib)
        assert np.array_equal(ent, full[rows, cols]), ("entries", act)
    bfull = oracle.bound_fused(A, B, C0, 1.5, -0.5, bias, lib=lib)
    bent = oracle.bound_fused_entries(rows, cols, A, B, C0, 1.5, -0.5, bias, lib=lib)
    assert np.array_equal(bent, bfull[rows, cols]), "bound entries"


ALL_PINS = [pin_bruteforce, pin_identity, pin_ones, pin_integers, pin_linearity,
            pin_transpose, pin_leading_dims, pin_read_conventions,
            pin_epilogue_worked_example, pin_epilogue_bias_axis, pin_epilogue_relu_identity,
            pin_epilogue_special_values, pin_epilogue_entries]
