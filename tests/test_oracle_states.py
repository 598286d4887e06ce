"""Pins of the oracle's states at requested times (CPU only).

The state between steps is a shortened step from the start of the accepted
step that holds the time (application paper arXiv 2609.28458, Sec. 2.3 and
Appendix A; the library paper's replay engines integrate one extra step to
each requested time).  Pins:
* decay: y0 * prod_{i<J} R(-theta h_i) * R(-theta (tau - t_J)) exactly, and
  the continuous y0 exp(-theta tau) within the tolerance scale;
* times on step boundaries reproduce the replay's states bit for bit, t1 the
  final state, t0 the initial state;
* invariants at interior times (Robertson's mass, the Lotka-Volterra V);
* interior states against a tight reference solve that ends at that time;
* times outside [t0, t1] or out of order give NaN.
"""
import numpy as np
import pytest

import dao_inputs as di

from test_oracle_systems import R_poly


def _solve(orc, w, s_cap=8192, **kw):
    r = orc.solve(w.system, w.method, w.theta, w.y0, w.t0, w.t1, w.rtol, w.atol, s_cap=s_cap,
                  **kw)
    assert np.all(r["status"] == 0)
    return r


def test_decay_states_closed_form(orc):
    w = di.make("decay", 16)
    r = _solve(orc, w)
    tq = np.linspace(w.t0, w.t1, 23)
    yq = orc.states_at(w.system, w.method, w.theta, w.y0, w.t0, w.t1, r["count"], r["h"], tq)
    for k in range(w.n):
        h = r["h"][k, :r["count"][k]]
        t = np.concatenate([[w.t0], w.t0 + np.cumsum(h)])
        for q, tau in enumerate(tq):
            J = min(np.searchsorted(t, tau, side="right") - 1, len(h) - 1)
            exact = w.y0[0, k] * np.prod(R_poly(orc, -w.theta[0, k] * h[:J])) * \
                R_poly(orc, -w.theta[0, k] * (tau - t[J]))[0]
            assert yq[q, 0, k] == pytest.approx(exact, rel=1e-13)
            cont = w.y0[0, k] * np.exp(-w.theta[0, k] * tau)
            assert abs(yq[q, 0, k] - cont) <= 50 * (w.rtol * abs(cont) + w.atol)


@pytest.mark.parametrize("system", ["lorenz63", "lotka_volterra", "robertson", "loghalo", "hires"])
def test_boundaries_reproduce_the_replay(orc, system):
    w = di.make(system, 4)
    if system == "loghalo":
        w.t1 = 5.0
    r = _solve(orc, w)
    for k in range(w.n):
        S = r["count"][k]
        h = r["h"][k:k + 1, :S]
        t = [w.t0]
        for j in range(S - 1):
            t.append(t[-1] + h[0, j])  # the solve's own time update
        js = sorted({0, 1, S // 3, S // 2, S - 1})
        tq = np.array([t[j] for j in js] + [w.t1])
        sub = di.subset(w, [k])
        yq = orc.states_at(system, w.method, sub.theta, sub.y0, w.t0, w.t1, r["count"][k:k + 1], h,
                           tq)
        for q, j in enumerate(js):
            cnt = np.array([j], np.int32)
            y_j = orc.replay(system, w.method, sub.theta, sub.y0, cnt, h)
            assert np.array_equal(yq[q], y_j)
        assert np.array_equal(yq[-1, :, 0], r["y1"][:, k])


def test_initial_and_final_times(orc):
    w = di.make("lorenz63", 8)
    r = _solve(orc, w)
    yq = orc.states_at(w.system, w.method, w.theta, w.y0, w.t0, w.t1, r["count"], r["h"],
                       np.array([w.t0, w.t1]))
    assert np.array_equal(yq[0], w.y0) and np.array_equal(yq[1], r["y1"])


def test_invariants_at_interior_times(orc):
    w = di.make("robertson", 6)
    r = _solve(orc, w, s_cap=4096)
    tq = np.array([1e-3, 0.37, 12.5, 4.4e3, 9.9e4])
    yq = orc.states_at(w.system, w.method, w.theta, w.y0, w.t0, w.t1, r["count"], r["h"], tq)
    assert np.max(np.abs(yq.sum(axis=1) - 1.0)) < 1e-13
    w = di.make("lotka_volterra", 6)
    r = _solve(orc, w)
    a, b, g, d = w.theta

    def V(y):
        return d * y[0] - g * np.log(y[0]) + b * y[1] - a * np.log(y[1])

    tq = np.linspace(0.1, 9.9, 9)
    yq = orc.states_at(w.system, w.method, w.theta, w.y0, w.t0, w.t1, r["count"], r["h"], tq)
    v0 = V(w.y0)
    for q in range(len(tq)):
        assert np.max(np.abs(V(yq[q]) - v0) / np.abs(v0)) < 1e-5


def test_interior_states_match_a_tight_solve(orc):
    w = di.make("lorenz63", 4)
    w.t1 = 0.5
    r = _solve(orc, w)
    tq = np.array([0.05, 0.123, 0.26, 0.4999])
    yq = orc.states_at(w.system, w.method, w.theta, w.y0, w.t0, w.t1, r["count"], r["h"], tq)
    for q, tau in enumerate(tq):
        ref = orc.solve(w.system, w.method, w.theta, w.y0, w.t0, tau, 1e-13, 1e-13,
                        s_cap=20000)["y1"]
        err = np.abs(yq[q] - ref) / (w.rtol * np.abs(ref) + w.atol)
        assert err.max() < 100, (tau, err.max())


def test_bad_times_give_nan(orc):
    w = di.make("lorenz63", 3)
    r = _solve(orc, w)
    tq = np.array([-0.1, 0.5, 0.25, 1.0, 2.5, np.nan])
    yq = orc.states_at(w.system, w.method, w.theta, w.y0, w.t0, w.t1, r["count"], r["h"], tq)
    bad = [0, 2, 4, 5]  # before t0, below its predecessor, after t1, NaN
    assert np.all(np.isnan(yq[bad]))
    assert np.all(np.isfinite(yq[[1, 3]]))
