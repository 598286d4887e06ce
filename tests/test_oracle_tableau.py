"""Pins of the oracle's Runge-Kutta and Rosenbrock coefficients.

The pages (arXiv 2609.02876, Sec. 2.1 and Sec. 3.1) name the Tsit5 pair -- a
fifth-order explicit pair with s = 7 stages whose last stage is reused (FSAL)
-- and the Rosenbrock23 method, but print neither table.  The oracle takes the
values from the primary sources; these tests pin them to what the mathematics
fixes: Butcher's order conditions (enumerated here over rooted trees, with no
code from the oracle), the FSAL structure, the null-space structure of the
error weights, and the Rosenbrock23 stability function.
"""
import itertools
from functools import lru_cache

import numpy as np
import pytest


# --- rooted trees and elementary weights (Butcher) ---------------------------
@lru_cache(None)
def trees(order):
    """All rooted trees with `order` vertices, as sorted tuples of child trees."""
    if order == 1:
        return ((),)
    out = set()

    def forests(rem, min_key):
        if rem == 0:
            yield ()
            return
        for m in range(1, rem + 1):
            for t in trees(m):
                key = (m, t)
                if min_key is not None and key < min_key:
                    continue
                for rest in forests(rem - m, key):
                    yield ((m, t),) + rest

    for f in forests(order - 1, None):
        out.add(tuple(sorted(t for _, t in f)))
    return tuple(sorted(out))


def tree_order(t):
    return 1 + sum(tree_order(s) for s in t)


def density(t):
    g = tree_order(t)
    for s in t:
        g *= density(s)
    return g


def stage_weights(A, t):
    v = np.ones(A.shape[0])
    for s in t:
        v = v * (A @ stage_weights(A, s))
    return v


def residuals(A, b, max_order):
    res = []
    for p in range(1, max_order + 1):
        for t in trees(p):
            res.append(b @ stage_weights(A, t) - 1.0 / density(t))
    return np.array(res)


def test_tree_counts():
    # Number of rooted trees of order 1..7 is 1, 1, 2, 4, 9, 20, 48 (OEIS
    # A000081): 85 conditions up to order 7, 37 up to order 6.
    assert [len(trees(p)) for p in range(1, 8)] == [1, 1, 2, 4, 9, 20, 48]


def test_tsit5_row_sums_and_fsal(orc):
    c, A, b, bt = orc.tsit5_table()
    assert np.max(np.abs(A.sum(axis=1) - c)) < 1e-15
    assert np.all(np.triu(A) == 0.0)  # explicit
    assert b[6] == 0.0 and c[6] == 1.0  # the 7th stage sits at y_new (FSAL)
    assert np.array_equal(A[6], b)
    assert c[5] == 1.0


def test_tsit5_fifth_order(orc):
    c, A, b, bt = orc.tsit5_table()
    r = residuals(A, b, 5)
    assert r.size == 17
    assert np.max(np.abs(r)) < 5e-14


def test_tsit5_embedded_fourth_order(orc):
    c, A, b, bt = orc.tsit5_table()
    bhat = b - bt
    assert np.max(np.abs(residuals(A, bhat, 4))) < 5e-14
    # ... and genuinely not fifth order, so e = y_new - yhat_new is O(h^5)
    assert np.max(np.abs(residuals(A, bhat, 5)[8:])) > 1e-4


def test_tsit5_error_weights_span_the_null_space(orc):
    # b - bhat annihilates every order <= 4 condition; that null space is 1-D,
    # so the error weights are fixed up to one scale (bt_7 = 1/66 is the
    # primary source's normalisation: parity unpinned by the pages).
    c, A, b, bt = orc.tsit5_table()
    M = np.array([stage_weights(A, t) for p in range(1, 5) for t in trees(p)])
    s = np.linalg.svd(M, compute_uv=False)
    assert s[-1] < 1e-14 * s[0] and s[-2] > 1e-3
    assert np.max(np.abs(M @ bt)) < 1e-15 * 1e2
    assert bt[6] == pytest.approx(1.0 / 66.0, rel=1e-15)


def test_order_conditions_catch_a_wrong_coefficient(orc):
    # Planted mistakes (in a copy of the table, on the CPU): any single
    # coefficient off in its 8th significant digit, or with its sign flipped,
    # must break a fifth-order condition or a row sum.
    c, A, b, bt = orc.tsit5_table()
    for i, j in itertools.product(range(1, 7), range(6)):
        if j >= i:
            continue
        for bad in (A[i, j] * (1 + 1e-8), -A[i, j]):
            A2 = A.copy()
            A2[i, j] = bad
            b2 = A2[6].copy()
            row = np.max(np.abs(A2.sum(axis=1) - c))
            cond = np.max(np.abs(residuals(A2, b2, 5)))
            assert max(row, cond) > 1e-12, (i, j)


def test_ros23_l_stability_root(orc):
    # One Rosenbrock23 step on y' = lambda y gives
    #   R(z) = 1 + z w (2 - w + z w / 2),  w = 1 / (1 - d z),
    # whose limit at z -> -inf is 1 - 2/d + 1/(2 d^2); L-stability makes it 0,
    # i.e. d is the smaller root 1 - sqrt(2)/2 = 1/(2 + sqrt 2).
    d, e32 = orc.ros23_consts()
    assert abs(1 - 2 / d + 1 / (2 * d * d)) < 1e-14
    assert d == pytest.approx(1 - np.sqrt(2) / 2, rel=1e-15)
    assert e32 == pytest.approx(6 + np.sqrt(2), rel=1e-15)


def test_ros23_stability_function(orc):
    d, _ = orc.ros23_consts()
    for z in (-1e-3, -0.1, -1.0, -7.0, -1e3, -1e8, 0.05):
        w = 1.0 / (1.0 - d * z)
        R = 1.0 + z * w * (2.0 - w + 0.5 * z * w)
        ynew, _ = orc.step("decay", "rosenbrock23", [-z], [1.0], 1.0)  # h=1, theta=-z
        assert ynew[0] == pytest.approx(R, rel=1e-13, abs=1e-15)
    big, _ = orc.step("decay", "rosenbrock23", [1e12], [1.0], 1.0)
    assert abs(big[0]) < 1e-11  # L-stable: R(-inf) = 0
    # order 2: R(z) - exp(z) = O(z^3)
    for z in (-1e-2, -5e-3):
        ynew, _ = orc.step("decay", "rosenbrock23", [-z], [1.0], 1.0)
        assert abs(ynew[0] - np.exp(z)) < 0.2 * abs(z) ** 3


def _tsit5_R(orc, z):
    c, A, b, bt = orc.tsit5_table()
    return 1.0 + z * b @ np.linalg.solve(np.eye(7) - z * A, np.ones(7))


def test_tsit5_stability_function_from_table(orc):
    # The replay of y' = -theta y is y_{n+1} = R(-theta h) y_n exactly (up to
    # rounding), with R the stability polynomial of the table.
    for z in (-0.01, -0.3, -1.0, -2.5):
        ynew, _ = orc.step("decay", "tsit5", [-z], [1.0], 1.0)
        assert ynew[0] == pytest.approx(_tsit5_R(orc, z), rel=2e-15)
        # fifth order: R(z) - exp(z) = O(z^6)
    for z in (-0.05, -0.1):
        assert abs(_tsit5_R(orc, z) - np.exp(z)) < 1e-2 * abs(z) ** 6


@pytest.mark.parametrize("q", [10, 6, 14])
def test_controller_power_matches_exact_power(orc, q):
    # The controller factor 0.9 * msq^(-1/q), clamped to [0.2, 10], is the
    # integral controller err^(-1/(order+1)) on the mean square msq = err^2.
    # The oracle evaluates the power by a polynomial rule; pin it to the exact
    # power inside its range, and check that the clamped range only cuts where
    # the clamped factor saturates anyway.
    lo, hi = {10: (1e-12, 1e8), 6: (1e-8, 1e5), 14: (1e-15, 1e10)}[q]
    x = np.logspace(np.log10(lo), np.log10(hi), 4001)
    x = np.concatenate([x, x * (1 + 1e-9), np.nextafter(x, 0)])
    x = x[(x >= lo) & (x <= hi)]
    got = orc.ctrl_root(x, q)
    exact = x ** (-1.0 / q)
    assert np.max(np.abs(got / exact - 1)) < 1e-7
    got32 = orc.ctrl_root(x.astype(np.float32), q, dtype="f32")
    exact32 = x.astype(np.float32).astype(np.float64) ** (-1.0 / q)
    assert np.max(np.abs(got32 / exact32 - 1)) < 2e-6
    assert 0.9 * lo ** (-1.0 / q) >= 10 and 0.9 * hi ** (-1.0 / q) <= 0.2
    out = orc.ctrl_root(np.array([lo * 1e-3, hi * 1e3]), q)
    assert out[0] == orc.ctrl_root(np.array([lo]), q)[0]
    assert out[1] == orc.ctrl_root(np.array([hi]), q)[0]


# --- Verner 7(6) --------------------------------------------------------------
# The pages name the pair (the library paper's method list; the application
# paper's precession arm runs on it) and print no coefficients; the oracle
# holds Verner's published ten-stage table.  Pinned here by all 85 conditions
# of order 7 on b, all 37 of order 6 on bhat (and bhat genuinely of order 6),
# the structure of the table, and its stability polynomial.
def test_vern7_structure(orc):
    c, A, b, bh = orc.vern7_table()
    assert np.max(np.abs(A.sum(axis=1) - c)) < 2e-14
    assert np.all(np.triu(A) == 0.0)  # explicit
    assert c[8] == 1.0 and c[9] == 1.0
    assert b[1] == b[2] == b[9] == 0.0  # seventh order uses stages 1, 4-9
    assert bh[1] == bh[2] == bh[7] == bh[8] == 0.0  # sixth order: 1, 4-7, 10
    assert A[9, 7] == A[9, 8] == 0.0  # stage 10 needs only stages 1-7
    assert not np.allclose(A[9], b)  # not FSAL: stage 10 is not the new state


def test_vern7_seventh_order(orc):
    c, A, b, bh = orc.vern7_table()
    r = residuals(A, b, 7)
    assert r.size == 85
    assert np.max(np.abs(r)) < 1e-14


def test_vern7_embedded_sixth_order(orc):
    c, A, b, bh = orc.vern7_table()
    r6 = residuals(A, bh, 6)
    assert r6.size == 37
    assert np.max(np.abs(r6)) < 1e-14
    # ... and not seventh order, so the estimate b - bhat is O(h^7)
    assert np.max(np.abs(residuals(A, bh, 7)[37:])) > 1e-5


def test_vern7_order_conditions_catch_a_wrong_coefficient(orc):
    # Planted mistakes in a copy of the table: each nonzero coefficient of A,
    # b or bhat off in its 8th significant digit, or sign-flipped, breaks an
    # order condition or a row sum.
    c, A, b, bh = orc.vern7_table()
    for i, j in itertools.product(range(10), range(10)):
        if A[i, j] == 0.0:
            continue
        for bad in (A[i, j] * (1 + 1e-8), -A[i, j]):
            A2 = A.copy()
            A2[i, j] = bad
            row = np.max(np.abs(A2.sum(axis=1) - c))
            cond = max(np.max(np.abs(residuals(A2, b, 7))), np.max(np.abs(residuals(A2, bh, 6))))
            assert max(row, cond) > 1e-12, (i, j)
    for w, order in ((b, 7), (bh, 6)):
        for j in np.flatnonzero(w):
            for bad in (w[j] * (1 + 1e-8), -w[j]):
                w2 = w.copy()
                w2[j] = bad
                assert np.max(np.abs(residuals(A, w2, order))) > 1e-12, j


def test_vern7_stability_function_from_table(orc):
    # the replay of y' = -theta y multiplies by the table's stability
    # polynomial; seventh order: R(z) - exp(z) = O(z^8)
    c, A, b, bh = orc.vern7_table()

    def R(z):
        return 1.0 + z * b @ np.linalg.solve(np.eye(10) - z * A, np.ones(10))

    for z in (-0.01, -0.3, -1.0, -2.5):
        ynew, _ = orc.step("decay", "vern7", [-z], [1.0], 1.0)
        assert ynew[0] == pytest.approx(R(z), rel=2e-15)
    for z in (-0.05, -0.1):
        assert abs(R(z) - np.exp(z)) < 1e-3 * abs(z) ** 8
    # the polynomial's coefficients b^T A^(j-1) 1 are 1/j! for j <= 7, and
    # the eighth is not (order exactly 7 on the linear test equation)
    v = np.ones(10)
    for j in range(1, 8):
        assert b @ v == pytest.approx(1.0 / np.prod(np.arange(1, j + 1)), rel=1e-12)
        v = A @ v
    assert abs((b @ v) * 40320.0 - 1.0) > 1e-3


# --- Rodas5P ------------------------------------------------------------------
# Named on the pages (the general stiff default, timed against Kvaerno5),
# coefficients not printed; the oracle holds Steinebach's table.  Pinned by
# its linear stability function (computed here from the table alone): order
# 5 on y' = lambda y, L-stability R(-inf) = 0, |R| <= 1 on the closed left
# half-plane; the nonlinear orders are pinned in test_oracle_systems.py.
def _rodas_R(orc, z, embedded=False):
    g, A, C = orc.rodas5p_table()
    z = complex(z)
    u = []
    Y = 1.0
    for i in range(8):
        if i == 0:
            Y = 1.0
        elif i <= 5:
            Y = 1.0 + sum(A[i, j] * u[j] for j in range(i))
        else:
            Y = Y + u[i - 1]
        rhs = z * Y + sum(C[i, j] * u[j] for j in range(i))
        u.append(rhs / (1.0 / g - z))  # h = 1
    return Y if embedded else Y + u[7]


def test_rodas5p_linear_order_and_l_stability(orc):
    import math

    for z in (-1e-3, -2e-3):
        # order 5: R(z) - exp(z) = O(z^6); embedded order 4: O(z^5)
        assert abs(_rodas_R(orc, z) - np.exp(z)) < 1e-2 * abs(z) ** 6 * 40
        assert abs(_rodas_R(orc, z, True) - np.exp(z)) < abs(z) ** 5
    # R(-inf) = 0 (stiff accuracy): |R(z)| falls like 1/|z|
    assert abs(_rodas_R(orc, -1e12)) < 1e-10 and abs(_rodas_R(orc, -1e6)) < 1e-4
    for x in [-10.0 ** k for k in range(-3, 7)] + [0.0]:
        for yi in (0.0, 0.5, 2.0, 10.0, 100.0, 1e4):
            if x == 0.0 and yi == 0.0:
                continue
            assert abs(_rodas_R(orc, complex(x, yi))) <= 1.0 + 1e-12
    # the replay of y' = -theta y multiplies by R(-theta h), bit-level close
    for z in (-0.01, -0.5, -3.0, -300.0):
        ynew, _ = orc.step("decay", "rodas5p", [-z], [1.0], 1.0)
        assert ynew[0] == pytest.approx(_rodas_R(orc, z).real, rel=1e-13, abs=1e-16)
    assert math.isclose(orc.rodas5p_table()[0], 0.21193756319429014, rel_tol=1e-16)


def test_rodas5p_table_perturbation_breaks_order(orc):
    # Planted mistakes (on the CPU, in a copy of the table): a C or a entry off
    # in its 8th significant digit changes R(z) - exp(z) at order <= 5 or the
    # limit R(-inf) for some entry, so the linear checks above would catch
    # many mistakes; the nonlinear local-order test catches the rest.
    g, A, C = orc.rodas5p_table()
    assert np.count_nonzero(A) == 15 and np.count_nonzero(C) == 28
