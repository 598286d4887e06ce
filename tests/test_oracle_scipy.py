"""The oracle's solve loop against SciPy's independent implementation of the
same control (CPU).

gradsolve (arXiv 2609.02876) Sec. 2.1 defines the accept test as the RMS of
e / (atol + rtol max(|y|, |y_new|)) and cites the standard proportional
controller without printing it; Sec. 2.3 names the starting step without a
formula.  The oracle reads both as Hairer, Norsett & Wanner do (Solving ODEs
I, Sec. II.4), with its controller factor truncated to 16 mantissa bits.
SciPy implements the same rules on its own:

* `select_initial_step` is the Hairer-Norsett-Wanner starting step in the
  same RMS norm.  The oracle's first attempted step must equal it truncated
  to 16 bits (0 <= 1 - ours / SciPy's < 2^-16, up to rounding);
* SciPy's explicit Runge-Kutta driver (`RungeKutta`, the engine of RK45)
  takes a tableau as data and applies that error norm, the safety factor
  0.9, the factor limits [0.2, 10], the cap at 1 after a rejection and the
  clip of the last step.  Given the oracle's Tsit5 and Verner 7(6) tableaux
  (pinned by their order conditions elsewhere) it must reproduce the
  oracle's solve: the same number of accepted steps, the same first steps
  to the truncation's drift (below 1e-3), and a final state within the
  tolerance's scale.  A wrong safety factor, exponent, norm or scale moves
  step sizes by per cents; the last test shows that an exponent off by one
  order already breaks the agreement.
"""
import inspect

import numpy as np
import pytest

import dao_inputs as di

scipy_rk = pytest.importorskip("scipy.integrate._ivp.rk")
scipy_common = pytest.importorskip("scipy.integrate._ivp.common")
from scipy.integrate import solve_ivp  # noqa: E402

# order of the higher solution: the starting step's exponent is 1/order in
# the oracle and 1/(est + 1) in SciPy, est = order - 1 the estimator's order
ORDER = {"tsit5": 5, "rosenbrock23": 2, "vern7": 7, "rodas5p": 5}


def scipy_h0(fun, t0, y0, t1, f0, est_order, rtol, atol):
    sel = scipy_common.select_initial_step
    if "t_bound" in inspect.signature(sel).parameters:
        return sel(fun, t0, y0, t1, np.inf, f0, 1, est_order, rtol, atol)
    return sel(fun, t0, y0, f0, 1, est_order, rtol, atol)


@pytest.mark.parametrize("name", ["decay", "lotka_volterra", "lorenz63", "robertson", "loghalo",
                                  "hires", "lorenz63_vern7", "robertson_rodas5p",
                                  "hires_rodas5p"])
def test_starting_step_is_scipys_truncated(orc, name):
    w = di.make(name, 16)
    for k in range(w.n):
        th, y0 = w.theta[:, k], w.y0[:, k]
        fun = lambda t, y: orc.rhs(w.system, th, y)  # noqa: E731
        hs = scipy_h0(fun, w.t0, y0, w.t1, fun(w.t0, y0), ORDER[w.method] - 1, w.rtol, w.atol)
        assert hs < w.t1 - w.t0  # no clip of the span on either side
        ho = orc.trace(w.system, w.method, th, y0, w.t0, w.t1, w.rtol, w.atol)["h"][0]
        rel = 1.0 - ho / hs
        assert -1e-12 <= rel < 2.0 ** -16 + 1e-12, (k, ho, hs)


def rk_class(orc, method, est_shift=0):
    """SciPy RungeKutta subclass with the oracle's tableau; est_shift moves
    the estimator order (a planted mistake, for the last test)."""
    if method == "tsit5":
        c_, A_, b_, bt_ = orc.tsit5_table()
        tab = dict(C=c_[:6].copy(), A=A_[:6, :6].copy(), B=b_[:6].copy(), E=bt_.copy(),
                   P=np.zeros((7, 1)), order=5, error_estimator_order=4 + est_shift, n_stages=6)
    else:
        c_, A_, b_, bh_ = orc.vern7_table()
        tab = dict(C=c_.copy(), A=A_.copy(), B=b_.copy(), E=np.concatenate([b_ - bh_, [0.0]]),
                   P=np.zeros((11, 1)), order=7, error_estimator_order=6 + est_shift,
                   n_stages=10)
    return type("OracleTableau", (scipy_rk.RungeKutta,), tab)


def compare(orc, name, n, est_shift=0):
    w = di.make(name, n)
    ref = orc.solve(w.system, w.method, w.theta, w.y0, w.t0, w.t1, w.rtol, w.atol, s_cap=16384)
    cls = rk_class(orc, w.method, est_shift)
    dcount, hdrift, ydev = [], [], []
    for k in range(w.n):
        th = w.theta[:, k]
        sol = solve_ivp(lambda t, y: orc.rhs(w.system, th, y), (w.t0, w.t1), w.y0[:, k],
                        method=cls, rtol=w.rtol, atol=w.atol)
        assert sol.status == 0
        hs = np.diff(sol.t)
        dcount.append(int(ref["count"][k]) - len(hs))
        m = min(20, len(hs), int(ref["count"][k]))
        hdrift.append(float(np.max(np.abs(hs[:m] - ref["h"][k, :m]) / hs[:m])))
        y1, yo = sol.y[:, -1], ref["y1"][:, k]
        ydev.append(float(np.max(np.abs(yo - y1) / (w.rtol * np.maximum(np.abs(yo), np.abs(y1))
                                                    + w.atol))))
    return np.array(dcount), np.array(hdrift), np.array(ydev)


# workload: (sample, bound on |y1 - y1_scipy| in units of rtol |y| + atol).
# The meshes drift apart by the truncation (ours is at most 2^-16 shorter per
# step), so the final states differ by about the global error: small for
# the decay and the predator-prey cycle, larger over the orbits' ten periods.
EXPLICIT = {"decay": (16, 1.0), "lotka_volterra": (16, 1.0), "lorenz63": (16, 10.0),
            "loghalo": (8, 100.0), "lorenz63_vern7": (16, 10.0), "loghalo_vern7": (8, 100.0)}


@pytest.mark.parametrize("name", list(EXPLICIT))
def test_explicit_solve_matches_scipys_driver(orc, name):
    n, ybound = EXPLICIT[name]
    dcount, hdrift, ydev = compare(orc, name, n)
    assert np.all(dcount == 0), dcount
    assert hdrift.max() < 1e-3, hdrift.max()
    assert ydev.max() < ybound, ydev.max()


def test_a_wrong_exponent_breaks_the_agreement(orc):
    # SciPy with the estimator's order off by one (controller exponent 1/4
    # instead of 1/5): the first steps part by far more than the truncation's
    # drift and the step counts change.
    dcount, hdrift, _ = compare(orc, "lorenz63", 8, est_shift=-1)
    assert hdrift.max() > 1e-2
    assert np.any(dcount != 0)
