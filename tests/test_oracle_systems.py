"""Pins of the oracle's solve, replay and gradient against closed forms,
invariants and independent derivatives (CPU only).

Sources of each pin:
* the decay system y' = -theta y: exact discrete solution y0 * prod R(-theta h_n)
  and its exact theta-derivative on the frozen mesh (arXiv 2609.02876,
  Sec. 3.1: the gradient is that of the replay chain with h fixed), plus the
  continuous solution y0 exp(-theta t) within the tolerance;
* conserved quantities of Lotka-Volterra, the halo orbit and Robertson;
* special initial states that reduce a system to the decay system;
* complex-step and central finite differences on the frozen mesh (the pages'
  own check perturbs inputs inside the same recorded replay, Sec. 3.1);
* field derivatives: the oracle Jacobians vs complex-step of the fields.
"""
import numpy as np
import pytest

import dao_inputs as di

TSIT = "tsit5"
ROS = "rosenbrock23"
VERN = "vern7"
RODAS = "rodas5p"


def R_poly(orc, z):
    c, A, b, bt = orc.tsit5_table()
    z = np.atleast_1d(z)
    return np.array([1.0 + zz * b @ np.linalg.solve(np.eye(7) - zz * A, np.ones(7)) for zz in z])


def dR_poly(orc, z, eps=1e-30):
    c, A, b, bt = orc.tsit5_table()
    out = []
    for zz in np.atleast_1d(z):
        zc = complex(zz, eps)
        r = 1.0 + zc * b @ np.linalg.solve(np.eye(7) - zc * A, np.ones(7))
        out.append(r.imag / eps)
    return np.array(out)


def solve_w(orc, w, **kw):
    kw.setdefault("s_cap", 8192)
    kw.setdefault("dtype", w.dtype)
    return orc.solve(w.system, w.method, w.theta, w.y0, w.t0, w.t1, w.rtol, w.atol, **kw)


# ---------------------------------------------------------------- decay
def test_decay_discrete_closed_form(orc):
    w = di.make("decay", 64)
    r = solve_w(orc, w)
    assert np.all(r["status"] == 0)
    lam = dLdy = np.ones((1, w.n))
    dth, dy0, yS = orc.grad(w.system, w.method, w.theta, w.y0, r["count"], r["h"], dLdy)
    for k in range(w.n):
        S = r["count"][k]
        h = r["h"][k, :S]
        z = -w.theta[0, k] * h
        Rz = R_poly(orc, z)
        exact = w.y0[0, k] * np.prod(Rz)
        dexact = exact * np.sum(-h * dR_poly(orc, z) / Rz)
        assert yS[0, k] == pytest.approx(exact, rel=1e-13)
        assert r["y1"][0, k] == yS[0, k]  # the replay reproduces the solve bit for bit
        assert dth[0, k] == pytest.approx(dexact, rel=1e-12)
        assert dy0[0, k] == pytest.approx(np.prod(Rz), rel=1e-13)
        # continuous solution to within the tolerance scale
        cont = w.y0[0, k] * np.exp(-w.theta[0, k] * w.t1)
        assert abs(r["y1"][0, k] - cont) <= 50 * (w.rtol * abs(cont) + w.atol)
        assert abs(dth[0, k] - (-w.t1 * cont)) <= 1e-5 * abs(w.t1 * cont)


def test_decay_discrete_closed_form_vern7(orc):
    # The same closed forms with Verner 7's stability polynomial.
    c, A, b, bh = orc.vern7_table()

    def R(z):
        return 1.0 + z * b @ np.linalg.solve(np.eye(10) - z * A, np.ones(10))

    def dR(z, eps=1e-30):
        zc = complex(z, eps)
        return (1.0 + zc * b @ np.linalg.solve(np.eye(10) - zc * A, np.ones(10))).imag / eps

    w = di.make("decay", 32)
    w.method = VERN
    r = solve_w(orc, w)
    assert np.all(r["status"] == 0)
    dth, dy0, yS = orc.grad(w.system, w.method, w.theta, w.y0, r["count"], r["h"],
                            np.ones((1, w.n)))
    for k in range(w.n):
        h = r["h"][k, :r["count"][k]]
        z = -w.theta[0, k] * h
        Rz = np.array([R(zz) for zz in z])
        exact = w.y0[0, k] * np.prod(Rz)
        dexact = exact * np.sum(-h * np.array([dR(zz) for zz in z]) / Rz)
        assert yS[0, k] == pytest.approx(exact, rel=1e-13)
        assert r["y1"][0, k] == yS[0, k]
        assert dth[0, k] == pytest.approx(dexact, rel=1e-12)
        cont = w.y0[0, k] * np.exp(-w.theta[0, k] * w.t1)
        assert abs(r["y1"][0, k] - cont) <= 50 * (w.rtol * abs(cont) + w.atol)


def test_record_mesh_invariants(orc):
    w = di.make("lorenz63", 32)
    r = solve_w(orc, w)
    for k in range(w.n):
        S = r["count"][k]
        t, h = r["t"][k, :S], r["h"][k, :S]
        assert t[0] == w.t0
        assert np.all(h > 0)
        assert np.all(t[1:] == t[:-1] + h[:-1])  # t_{n+1} = t_n + h_n exactly
        assert t[-1] + h[-1] == pytest.approx(w.t1, rel=1e-15)  # clipped last step
        assert np.all(r["h"][k, S:] == 0.0)  # unused rows stay zero


def test_zero_padding_rows_are_identity(orc):
    # Section 3.1: a step of size zero leaves the state unchanged.
    w = di.make("lotka_volterra", 16)
    r = solve_w(orc, w)
    y_a = orc.replay(w.system, w.method, w.theta, w.y0, r["count"], r["h"])
    y_b = orc.replay(w.system, w.method, w.theta, w.y0, r["count"] + 5, r["h"])
    assert np.array_equal(y_a, y_b)
    wr = di.make("robertson", 4)
    rr = solve_w(orc, wr)
    ya = orc.replay(wr.system, wr.method, wr.theta, wr.y0, rr["count"], rr["h"])
    yb = orc.replay(wr.system, wr.method, wr.theta, wr.y0, rr["count"] + 3, rr["h"])
    assert np.array_equal(ya, yb)


# ---------------------------------------------------------------- Lotka-Volterra
def test_lv_invariant(orc):
    w = di.make("lotka_volterra", 128)
    r = solve_w(orc, w)
    a, b, g, d = w.theta

    def V(y):
        return d * y[0] - g * np.log(y[0]) + b * y[1] - a * np.log(y[1])

    drift = np.abs(V(r["y1"]) - V(w.y0)) / np.abs(V(w.y0))
    assert np.max(drift) < 2e-5  # rtol 1e-6 over ten time units
    assert np.median(drift) < 2e-6


def test_lv_prey_only_reduces_to_decay(orc):
    w = di.make("lotka_volterra", 16)
    y0 = w.y0.copy()
    y0[1] = 0.0  # no predators: y2 stays exactly 0 and y1 grows like y' = a y
    r = orc.solve(w.system, w.method, w.theta, y0, 0.0, 3.0, 1e-8, 1e-10, s_cap=4096)
    assert np.all(r["y1"][1] == 0.0)
    for k in range(w.n):
        S = r["count"][k]
        z = w.theta[0, k] * r["h"][k, :S]
        assert r["y1"][0, k] == pytest.approx(y0[0, k] * np.prod(R_poly(orc, z)), rel=1e-13)


# ---------------------------------------------------------------- Lorenz
def test_lorenz_z_axis_closed_form(orc):
    w = di.make("lorenz63", 8)
    y0 = np.zeros_like(w.y0)
    y0[2] = w.y0[2]
    r = orc.solve(w.system, w.method, w.theta, y0, w.t0, w.t1, w.rtol, w.atol, s_cap=4096)
    assert np.all(r["y1"][:2] == 0.0)
    lam = np.array([[0.3], [-0.7], [1.1]]) * np.ones((3, w.n))
    dth, dy0, yS = orc.grad(w.system, w.method, w.theta, y0, r["count"], r["h"], lam)
    assert np.all(dth[0] == 0.0) and np.all(dth[1] == 0.0)  # sigma, rho do not enter
    for k in range(w.n):
        S = r["count"][k]
        h = r["h"][k, :S]
        z = -w.theta[2, k] * h
        Rz = R_poly(orc, z)
        y3 = y0[2, k] * np.prod(Rz)
        assert yS[2, k] == pytest.approx(y3, rel=1e-13)
        assert dth[2, k] == pytest.approx(lam[2, k] * y3 * np.sum(-h * dR_poly(orc, z) / Rz),
                                          rel=1e-12)


# ---------------------------------------------------------------- Robertson
def test_robertson_mass_conservation(orc):
    w = di.make("robertson", 32)
    r = solve_w(orc, w, s_cap=4096)
    assert np.all(r["status"] == 0)
    assert np.max(np.abs(r["y1"].sum(axis=0) - 1.0)) < 1e-13
    assert np.all(r["y1"] > -1e-12)


def test_robertson_mass_cotangent(orc):
    # 1^T f = 0 and 1^T J = 0, so sum(y) is invariant along the replay: with
    # dL/dy = (1,1,1) the rate gradient vanishes and dL/dy0 = (1,1,1).
    w = di.make("robertson", 8)
    r = solve_w(orc, w, s_cap=4096)
    ones = np.ones((3, w.n))
    dth, dy0, _ = orc.grad(w.system, w.method, w.theta, w.y0, r["count"], r["h"], ones)
    lam = np.zeros((3, w.n))
    lam[0] = 1.0
    dth_ref, _, _ = orc.grad(w.system, w.method, w.theta, w.y0, r["count"], r["h"], lam)
    scale = np.abs(dth_ref * w.theta).max(axis=0)
    assert np.all(np.abs(dth * w.theta).max(axis=0) < 1e-10 * scale)
    assert np.max(np.abs(dy0 - 1.0)) < 1e-12


# ---------------------------------------------------------------- HIRES
def test_hires_linear_invariant(orc):
    # y7' + y8' = 0 identically, and the Jacobian's rows 7 and 8 sum to zero,
    # so every Rosenbrock stage keeps k7 + k8 = 0 and y7 + y8 is carried
    # through the solve up to rounding.
    w = di.make("hires", 16)
    r = solve_w(orc, w, s_cap=4096)
    assert np.all(r["status"] == 0)
    drift = np.abs((r["y1"][6] + r["y1"][7]) - (w.y0[6] + w.y0[7]))
    assert drift.max() < 1e-15
    assert np.all(r["y1"] > -1e-12)


def test_hires_invariant_cotangent(orc):
    # With dL/dy1 = e7 + e8 the loss is the invariant itself: no rate
    # constant moves it (gradient zero to rounding) and dL/dy0 = e7 + e8.
    w = di.make("hires", 4)
    r = solve_w(orc, w, s_cap=4096)
    lam = np.zeros((8, w.n))
    lam[6:8] = 1.0
    dth, dy0, _ = orc.grad(w.system, w.method, w.theta, w.y0, r["count"], r["h"], lam)
    lam1 = np.zeros((8, w.n))
    lam1[6] = 1.0
    dth_ref, _, _ = orc.grad(w.system, w.method, w.theta, w.y0, r["count"], r["h"], lam1)
    scale = np.abs(dth_ref * w.theta).max(axis=0)
    assert np.all(np.abs(dth * w.theta).max(axis=0) < 1e-10 * scale)
    assert np.max(np.abs(dy0 - lam)) < 1e-12


def test_hires_matches_an_independent_implicit_solver(orc):
    # The oracle's Rosenbrock23 solve at a tight tolerance against SciPy's
    # Radau IIA (an independent fifth-order implicit method and code) at a
    # tighter one: agreement to the tolerance scale pins the stiff solve with
    # pivoting on an eight-dimensional system.
    from scipy.integrate import solve_ivp

    k = di.HIRES_RATES

    def field(t, y):
        a = k[9] * y[5] * y[7]
        return [-k[0] * y[0] + k[1] * y[1] + k[2] * y[2] + k[3], k[0] * y[0] - k[4] * y[1],
                -k[5] * y[2] + k[1] * y[3] + k[6] * y[4], k[2] * y[1] + k[0] * y[2] - k[7] * y[3],
                -k[8] * y[4] + k[1] * (y[5] + y[6]),
                k[10] * (y[3] + y[6]) + k[0] * y[4] - k[1] * y[5] - a, a - k[11] * y[6],
                k[11] * y[6] - a]

    w = di.make("hires", 3)
    w.rtol, w.atol = 1e-8, 1e-12
    r = solve_w(orc, w, s_cap=65536)
    assert np.all(r["status"] == 0)
    for j in range(w.n):
        s = solve_ivp(field, (w.t0, w.t1), w.y0[:, j], method="Radau", rtol=1e-12, atol=1e-16)
        ref = s.y[:, -1]
        assert np.allclose(r["y1"][:, j], ref, rtol=2e-6, atol=1e-12), (j, r["y1"][:, j], ref)


def test_ros23_error_estimate_tracks_local_error(orc):
    # The Rosenbrock23 estimate is the difference to the embedded third-order
    # solution, so est / (y_new - exact) -> 1 as h -> 0 on a smooth problem;
    # a wrong e32 breaks the limit.  Exact one-step values come from a very
    # fine Tsit5 replay.
    th = np.array([1.0, 0.7, 0.9, 1.2])  # Lotka-Volterra, non-stiff
    y = np.array([1.3, 0.8])
    ratios = []
    for h in (0.02, 0.01, 0.005):
        ynew, est = orc.step("lotka_volterra", ROS, th, y, h)
        nfine = 400
        exact = orc.replay("lotka_volterra", TSIT, th[:, None], y[:, None], np.array([nfine]),
                           np.full((1, nfine), h / nfine))[:, 0]
        true = ynew - exact
        ratios.append(np.linalg.norm(est) / np.linalg.norm(true))
    assert abs(ratios[-1] - 1.0) < 0.05
    assert abs(ratios[-1] - 1.0) < abs(ratios[0] - 1.0) + 1e-3


def test_vern7_error_estimate_order(orc):
    # e = h sum (b - bhat) k is O(h^7): halving h divides it by ~128.
    th = np.array([1.0, 0.7, 0.9, 1.2])
    y = np.array([1.3, 0.8])
    e = [np.linalg.norm(orc.step("lotka_volterra", VERN, th, y, h)[1]) for h in (0.08, 0.04, 0.02)]
    slopes = np.log2(np.array(e[:-1]) / np.array(e[1:]))
    assert np.all(np.abs(slopes - 7.0) < 0.3), slopes


@pytest.mark.parametrize("system", ["loghalo", "lorenz63"])
def test_rodas5p_local_orders(orc, system):
    # One Rodas5P step from a state against a tight reference (Verner 7 with
    # many substeps): the local error of y_new falls like h^6 (order 5) and
    # that of the embedded solution y_new - estimate like h^5 (order 4).  The
    # halo's field is not polynomial, so every elementary differential enters.
    w = di.make(system, 1)
    th = w.theta[:, 0]
    y = w.y0[:, 0] + (np.array([0.3, -0.2, 0.1, 0.05, 0.2, -0.1]) if system == "loghalo" else 0.0)
    # (the step sizes keep the error above rounding, where the slope is clean)
    hs = (0.08, 0.04, 0.02, 0.01) if system == "loghalo" else (0.02, 0.01, 0.005, 0.0025)
    e_main, e_emb = [], []
    for h in hs:
        ynew, est = orc.step(system, RODAS, th, y, h)
        nsub = 400
        ref = orc.replay(system, VERN, th[:, None], y[:, None], np.array([nsub]),
                         np.full((1, nsub), h / nsub))[:, 0]
        e_main.append(np.linalg.norm(ynew - ref))
        e_emb.append(np.linalg.norm(ynew - est - ref))
    s_main = np.log2(np.array(e_main[:-1]) / np.array(e_main[1:]))
    s_emb = np.log2(np.array(e_emb[:-1]) / np.array(e_emb[1:]))
    assert np.all(np.abs(s_main - 6.0) < 0.35) and abs(s_main[-1] - 6.0) < 0.1, s_main
    assert np.all(np.abs(s_emb - 5.0) < 0.3) and abs(s_emb[-1] - 5.0) < 0.1, s_emb


def test_rodas5p_decay_closed_form_and_robertson_invariants(orc):
    from test_oracle_tableau import _rodas_R

    w = di.make("decay", 24)
    w.method = RODAS
    r = solve_w(orc, w)
    assert np.all(r["status"] == 0)
    dth, dy0, yS = orc.grad(w.system, w.method, w.theta, w.y0, r["count"], r["h"],
                            np.ones((1, w.n)))
    for k in range(w.n):
        h = r["h"][k, :r["count"][k]]
        Rz = np.array([_rodas_R(orc, -w.theta[0, k] * hh).real for hh in h])
        assert yS[0, k] == pytest.approx(w.y0[0, k] * np.prod(Rz), rel=1e-12)
        assert dy0[0, k] == pytest.approx(np.prod(Rz), rel=1e-12)
        cont = w.y0[0, k] * np.exp(-w.theta[0, k] * w.t1)
        assert abs(r["y1"][0, k] - cont) <= 50 * (w.rtol * abs(cont) + w.atol)
    # Robertson: mass conserved by every stage solve; the cotangent (1,1,1)
    # gives zero rate gradient and dL/dy0 = (1,1,1)
    w = di.make("robertson_rodas5p", 16)
    r = solve_w(orc, w, s_cap=4096)
    assert np.all(r["status"] == 0)
    assert np.max(np.abs(r["y1"].sum(axis=0) - 1.0)) < 1e-13
    dth, dy0, _ = orc.grad(w.system, w.method, w.theta, w.y0, r["count"], r["h"],
                           np.ones((3, w.n)))
    assert np.max(np.abs(dth * w.theta)) < 1e-10
    assert np.max(np.abs(dy0 - 1.0)) < 1e-11


def test_tsit5_error_estimate_order(orc):
    # e = h sum (b - bhat) k is O(h^5): halving h divides it by ~32.
    th = np.array([1.0, 0.7, 0.9, 1.2])
    y = np.array([1.3, 0.8])
    e = [np.linalg.norm(orc.step("lotka_volterra", TSIT, th, y, h)[1]) for h in (0.04, 0.02, 0.01)]
    slopes = np.log2(np.array(e[:-1]) / np.array(e[1:]))
    assert np.all(np.abs(slopes - 5.0) < 0.3)


@pytest.mark.parametrize("method,order,system", [(TSIT, 5, "lotka_volterra"),
                                                  (ROS, 2, "lotka_volterra"),
                                                  (TSIT, 5, "loghalo"),
                                                  (VERN, 7, "lotka_volterra")])
def test_fixed_step_convergence_order(orc, method, order, system):
    # Global error of the fixed-step replay against a 20000-step reference.
    # Tsit5 approaches its asymptotic slope 5 from above at these step sizes.
    w = di.make(system, 1)
    T = 5.0
    nref = 20000
    ref = orc.replay(system, TSIT, w.theta, w.y0, np.array([nref]), np.full((1, nref), T / nref))
    errs = []
    ns = {TSIT: (32, 64, 128, 256), ROS: (64, 128, 256, 512), VERN: (16, 24, 32, 48, 64)}[method]
    for n in ns:
        y = orc.replay(system, method, w.theta, w.y0, np.array([n]), np.full((1, n), T / n))
        errs.append(np.linalg.norm(y - ref))
    slopes = np.log2(np.array(errs[:-1]) / np.array(errs[1:])) / np.log2(
        np.array(ns[1:]) / np.array(ns[:-1]))
    if method == VERN:
        # Verner's pair keeps its principal error coefficients small, so at
        # the step sizes where the error is above rounding (1e-5 .. 1e-12) the
        # slope is that of the next term, about 8; it is at least 7 and not 9.
        assert np.all((slopes > order - 0.5) & (slopes < order + 1.6)), slopes
    elif method == TSIT:
        assert np.all((slopes > 4.6) & (slopes < 6.2)), slopes
        assert abs(slopes[-1] - order) < 0.6, slopes
    else:
        assert np.all(np.abs(slopes - order) < 0.05), slopes


def test_tsit5_linear_order_coefficients(orc):
    # On y' = lambda y the step multiplies by R(z) = 1 + sum_j z^j b^T A^(j-1) 1;
    # fifth order means the first five coefficients are 1/j!.
    import math

    c, A, b, bt = orc.tsit5_table()
    coef = [b @ np.linalg.matrix_power(A, j - 1) @ np.ones(7) for j in range(1, 7)]
    for j in range(1, 6):
        assert coef[j - 1] == pytest.approx(1.0 / math.factorial(j), rel=1e-13)
    assert abs(coef[5] - 1.0 / 720.0) > 1e-5


# ---------------------------------------------------------------- orbits
def test_halo_conserved_quantities(orc):
    w = di.make("loghalo", 32)
    r = solve_w(orc, w, s_cap=8192)
    assert np.all(r["status"] == 0)
    v0, rc, q = w.theta

    def energy(y):
        D = rc ** 2 + y[0] ** 2 + y[1] ** 2 + y[2] ** 2 / q ** 2
        return 0.5 * (y[3] ** 2 + y[4] ** 2 + y[5] ** 2) + 0.5 * v0 ** 2 * np.log(D)

    def lz(y):
        return y[0] * y[4] - y[1] * y[3]

    E0, E1 = energy(w.y0), energy(r["y1"])
    assert np.max(np.abs(E1 - E0) / np.abs(E0)) < 1e-5
    assert np.max(np.abs(lz(r["y1"]) - lz(w.y0))) < 1e-5 * np.max(np.abs(lz(w.y0)))


def test_halo_planar_orbit_has_no_q_gradient(orc):
    w = di.make("loghalo", 8)
    y0 = w.y0.copy()
    y0[2] = 0.0
    y0[5] = 0.0
    r = orc.solve(w.system, w.method, w.theta, y0, 0.0, 10.0, 1e-8, 1e-10, s_cap=8192)
    assert np.all(r["y1"][2] == 0.0) and np.all(r["y1"][5] == 0.0)
    lam = np.random.default_rng(3).normal(size=(6, w.n))
    dth, _, _ = orc.grad(w.system, w.method, w.theta, y0, r["count"], r["h"], lam)
    assert np.all(dth[2] == 0.0)
    assert np.all(dth[0] != 0.0) and np.all(dth[1] != 0.0)


def test_halo_circular_orbit(orc):
    th = np.array([[1.0], [0.2], [0.9]])
    r0 = 1.3
    vc = th[0, 0] * r0 / np.sqrt(th[1, 0] ** 2 + r0 ** 2)
    y0 = np.array([[r0], [0.0], [0.0], [0.0], [vc], [0.0]])
    r = orc.solve("loghalo", TSIT, th, y0, 0.0, 40.0, 1e-8, 1e-10, s_cap=8192)
    rad = np.hypot(r["y1"][0, 0], r["y1"][1, 0])
    assert abs(rad - r0) < 1e-6


# ---------------------------------------------------------------- MLP
def test_mlp_constant_field(orc):
    # With W1 = W2 = 0 the field is the constant c = W3 tanh(b2) + b3, so
    # y(t) = y0 + c t and every weight gradient has a closed form.
    rng = np.random.default_rng(7)
    th = np.zeros(4740)
    b1 = rng.normal(size=64)
    b2 = rng.normal(size=64)
    W3 = rng.normal(size=(4, 64)) * 0.2
    b3 = rng.normal(size=4)
    th[256:320] = b1
    th[4416:4480] = b2
    th[4480:4736] = W3.ravel()
    th[4736:4740] = b3
    n = 5
    y0 = rng.normal(size=(4, n))
    r = orc.solve("mlp", TSIT, th, y0, 0.0, 1.0, 1e-5, 1e-7, s_cap=256)
    c = W3 @ np.tanh(b2) + b3
    assert np.allclose(r["y1"], y0 + c[:, None], rtol=1e-13, atol=1e-13)
    lam = rng.normal(size=(4, n))
    dth, dy0, _ = orc.grad("mlp", TSIT, th, y0, r["count"], r["h"], lam)
    L = lam.sum(axis=1)  # sum over trajectories, t1 = 1
    u = W3.T @ L * (1 - np.tanh(b2) ** 2)
    assert np.allclose(dth[4736:4740], L, rtol=1e-12)
    assert np.allclose(dth[4480:4736].reshape(4, 64), np.outer(L, np.tanh(b2)), rtol=1e-12,
                       atol=1e-14)
    assert np.allclose(dth[4416:4480], u, rtol=1e-12, atol=1e-14)
    assert np.allclose(dth[320:4416].reshape(64, 64), np.outer(u, np.tanh(b1)), rtol=1e-12,
                       atol=1e-14)
    assert np.allclose(dy0, lam, rtol=1e-13)


# ---------------------------------------------------------------- derivative pins
CASES = [("decay", TSIT), ("lotka_volterra", TSIT), ("lorenz63", TSIT), ("loghalo", TSIT),
         ("robertson", ROS), ("mlp", TSIT), ("lotka_volterra", ROS), ("lorenz63", ROS),
         ("hires", ROS), ("decay", VERN), ("lotka_volterra", VERN), ("lorenz63", VERN),
         ("loghalo", VERN), ("robertson", RODAS), ("lotka_volterra", RODAS), ("hires", RODAS)]


def _case(orc, system, method, n):
    w = di.make(system, n)
    if w.method != method:
        w.method = method
        if system == "lorenz63":
            w.t1 = 0.5
    r = solve_w(orc, w, s_cap=8192, dtype="f64")
    assert np.all(r["status"] == 0)
    theta = w.theta.astype(np.float64)
    y0 = w.y0.astype(np.float64)
    return w, r, theta, y0


@pytest.mark.parametrize("system,method", CASES)
def test_adjoint_matches_complex_step(orc, system, method):
    # <lambda, J v> from the complex step (forward direction) must equal
    # <J^T lambda, v> from the tape (reverse sweep): a dot-product test.
    w, r, theta, y0 = _case(orc, system, method, 3)
    rng = np.random.default_rng(11)
    lam = rng.normal(size=y0.shape)
    dth, dy0, yS = orc.grad(system, method, theta, y0, r["count"], r["h"], lam)
    for trial in range(2):
        vth = rng.normal(size=theta.shape) * np.abs(theta)
        vy = rng.normal(size=y0.shape)
        _, dyS = orc.replay_cs(system, method, theta, y0, vth, vy, r["count"], r["h"])
        lhs = np.sum(lam * dyS, axis=0)
        if system == "mlp":
            rhs = np.sum(dy0 * vy, axis=0)
            assert np.sum(lhs) == pytest.approx(np.sum(rhs) + np.sum(dth * vth), rel=1e-11)
        else:
            rhs = np.sum(dth * vth, axis=0) + np.sum(dy0 * vy, axis=0)
            assert np.allclose(lhs, rhs, rtol=1e-11, atol=1e-13 * np.abs(lhs).max())


@pytest.mark.parametrize("system,method", [c for c in CASES if c[0] != "mlp"])
def test_adjoint_matches_central_differences(orc, system, method):
    # The pages' own check: perturb the inputs inside the same recorded replay.
    w, r, theta, y0 = _case(orc, system, method, 2)
    rng = np.random.default_rng(5)
    lam = rng.normal(size=y0.shape)
    dth, dy0, yS = orc.grad(system, method, theta, y0, r["count"], r["h"], lam)
    for i in range(theta.shape[0]):
        e = 1e-6 * np.abs(theta[i])
        tp, tm = theta.copy(), theta.copy()
        tp[i] += e
        tm[i] -= e
        fp = np.sum(lam * orc.replay(system, method, tp, y0, r["count"], r["h"]), axis=0)
        fm = np.sum(lam * orc.replay(system, method, tm, y0, r["count"], r["h"]), axis=0)
        fd = (fp - fm) / (2 * e)
        assert np.allclose(fd, dth[i], rtol=2e-5, atol=1e-7 * np.abs(dth).max()), (i, fd, dth[i])


def test_gradient_is_per_trajectory(orc):
    # Brute force on tiny ensembles: each trajectory's gradient is its own.
    w = di.make("lorenz63", 6)
    r = solve_w(orc, w, s_cap=4096)
    lam = di.cotangent(w, r["y1"])
    dth, dy0, _ = orc.grad(w.system, w.method, w.theta, w.y0, r["count"], r["h"], lam)
    for k in range(w.n):
        s = slice(k, k + 1)
        dk, yk, _ = orc.grad(w.system, w.method, w.theta[:, s], w.y0[:, s], r["count"][s],
                             r["h"][s], lam[:, s])
        assert np.array_equal(dk[:, 0], dth[:, k]) and np.array_equal(yk[:, 0], dy0[:, k])


@pytest.mark.parametrize("system", ["lotka_volterra", "lorenz63", "robertson", "loghalo", "hires"])
def test_jacobians_match_complex_step_of_fields(orc, system):
    w = di.make(system, 4)
    for k in range(4):
        th = w.theta[:, k]
        y = w.y0[:, k] + (0.1 if system in ("robertson", "hires") else 0.0)
        J = orc.jac(system, th, y)
        d = len(y)
        for j in range(d):
            e = np.zeros(d)
            e[j] = 1e-7 * max(1.0, abs(y[j]))
            fd = (orc.rhs(system, th, y + e) - orc.rhs(system, th, y - e)) / (2 * e[j])
            assert np.allclose(J[:, j], fd, rtol=1e-6, atol=1e-6 * np.abs(J).max())


# ---------------------------------------------------------------- failures
def test_status_codes(orc):
    w = di.make("lorenz63", 4)
    r = orc.solve(w.system, w.method, w.theta, w.y0, w.t0, w.t1, w.rtol, w.atol, max_steps=10)
    assert np.all(r["status"] == 1) and np.all(np.isnan(r["y1"]))
    r = orc.solve(w.system, w.method, w.theta, w.y0, w.t0, w.t1, w.rtol, w.atol, s_cap=5)
    assert np.all(r["status"] == 4) and np.all(r["count"] == 5)
    th = w.theta.copy()
    th[0, 1] = np.nan
    r = orc.solve(w.system, w.method, th, w.y0, w.t0, w.t1, w.rtol, w.atol)
    assert r["status"][1] == 2 and np.all(r["status"][[0, 2, 3]] == 0)
    r = orc.solve(w.system, w.method, w.theta, w.y0, 1.0, 1.0, w.rtol, w.atol)
    assert np.all(r["count"] == 0) and np.array_equal(r["y1"], w.y0)
    with pytest.raises(ValueError):
        orc.solve(w.system, w.method, w.theta, w.y0, 1.0, 0.5, w.rtol, w.atol)
    with pytest.raises(ValueError):
        orc.solve(w.system, w.method, w.theta, w.y0, 0.0, 1.0, 0.0, w.atol)
