"""Pins of the oracle's gradient of a loss on the states at requested times
(CPU only).

The states at requested times are a shortened step of the method from the
start of the accepted step that holds each time (application paper arXiv
2609.28458 Sec. 2.3 and Appendix A; the library paper's replay engines take
one extra step to each requested time).  The gradient of
L = sum_q <c_q, y(tau_q)> + <c_1, y(t1)> on the recorded mesh is pinned by:
* the decay system: the exact derivative of y0 prod R(-theta h_i) R(-theta (tau - t_J));
* tau = t1 alone: the plain gradient (the final state is the shortened last step);
* tau on a step boundary: the plain gradient of the replay cut at that step;
* central differences of the states (the pages' own check) on every system;
* linearity in the cotangents.
"""
import numpy as np
import pytest

import dao_inputs as di

from test_oracle_systems import R_poly, dR_poly

TSIT = "tsit5"
ROS = "rosenbrock23"


def _solve(orc, w, s_cap=8192):
    r = orc.solve(w.system, w.method, w.theta, w.y0, w.t0, w.t1, w.rtol, w.atol, s_cap=s_cap)
    assert np.all(r["status"] == 0)
    return r


def _case(name, n):
    w = di.make(name, n)
    if name == "loghalo":
        w.t1 = 5.0
    if name == "hires":
        w.t1 = 20.0
    return w


def test_decay_closed_form(orc):
    w = di.make("decay", 5)
    r = _solve(orc, w)
    tq = np.array([0.0, 0.37, 1.1, 1.9, w.t1])
    rng = np.random.default_rng(3)
    cq = rng.normal(size=(len(tq), 1, w.n))
    dth, dy0 = orc.grad_at("decay", TSIT, w.theta, w.y0, w.t0, w.t1, r["count"], r["h"], tq, cq)
    for k in range(w.n):
        th, S = w.theta[0, k], r["count"][k]
        h = r["h"][k, :S]
        t = np.concatenate([[w.t0], w.t0 + np.cumsum(h[:-1])])  # the solve's own time update
        g_th = g_y0 = 0.0
        for q, tau in enumerate(tq):
            J = min(np.searchsorted(t, tau, side="right") - 1, S - 1)
            hh = np.concatenate([h[:J], [tau - t[J]]])
            z = -th * hh
            P = np.prod(R_poly(orc, z))
            dP = P * np.sum(-hh * dR_poly(orc, z) / R_poly(orc, z))
            g_y0 += cq[q, 0, k] * P
            g_th += cq[q, 0, k] * w.y0[0, k] * dP
        assert dy0[0, k] == pytest.approx(g_y0, rel=1e-12)
        assert dth[0, k] == pytest.approx(g_th, rel=1e-11)


@pytest.mark.parametrize("name", ["lorenz63", "robertson", "hires"])
def test_final_time_alone_is_the_plain_gradient(orc, name):
    w = _case(name, 3)
    r = _solve(orc, w)
    lam = np.random.default_rng(4).normal(size=w.y0.shape)
    g_th, g_y0, _ = orc.grad(w.system, w.method, w.theta, w.y0, r["count"], r["h"], lam)
    a_th, a_y0 = orc.grad_at(w.system, w.method, w.theta, w.y0, w.t0, w.t1, r["count"], r["h"],
                             np.array([w.t1]), lam[None])
    assert np.allclose(a_th, g_th, rtol=1e-12, atol=1e-14 * np.abs(g_th).max())
    assert np.allclose(a_y0, g_y0, rtol=1e-12, atol=1e-14 * np.abs(g_y0).max())
    # split between the final state and a requested time at t1: the same sum
    b_th, b_y0 = orc.grad_at(w.system, w.method, w.theta, w.y0, w.t0, w.t1, r["count"], r["h"],
                             np.array([w.t1]), 0.5 * lam[None], dLdy1=0.5 * lam)
    assert np.allclose(b_th, g_th, rtol=1e-12, atol=1e-14 * np.abs(g_th).max())


def test_step_boundary_is_the_cut_replay(orc):
    w = _case("lorenz63", 2)
    r = _solve(orc, w)
    lam = np.random.default_rng(5).normal(size=w.y0.shape)
    for k in range(w.n):
        S = r["count"][k]
        h = r["h"][k:k + 1, :S]
        J = S // 2
        tau = w.t0
        for i in range(J):
            tau = tau + h[0, i]
        sub = di.subset(w, [k])
        a_th, a_y0 = orc.grad_at(w.system, w.method, sub.theta, sub.y0, w.t0, w.t1,
                                 r["count"][k:k + 1], h, np.array([tau]), lam[None, :, k:k + 1])
        g_th, g_y0, _ = orc.grad(w.system, w.method, sub.theta, sub.y0, np.array([J], np.int32),
                                 h, lam[:, k:k + 1])
        assert np.allclose(a_th, g_th, rtol=1e-12) and np.allclose(a_y0, g_y0, rtol=1e-12)


@pytest.mark.parametrize("name", ["lotka_volterra", "lorenz63", "loghalo", "robertson", "hires"])
def test_central_differences(orc, name):
    w = _case(name, 2)
    r = _solve(orc, w)
    tq = np.linspace(w.t0, w.t1, 7)[1:] - 0.013 * (w.t1 - w.t0)
    tq = np.concatenate([tq, [w.t1]])
    rng = np.random.default_rng(6)
    cq = rng.normal(size=(len(tq),) + w.y0.shape)
    c1 = rng.normal(size=w.y0.shape)
    dth, dy0 = orc.grad_at(w.system, w.method, w.theta, w.y0, w.t0, w.t1, r["count"], r["h"], tq,
                           cq, dLdy1=c1)

    def loss(theta, y0):
        yq = orc.states_at(w.system, w.method, theta, y0, w.t0, w.t1, r["count"], r["h"], tq)
        y1 = orc.replay(w.system, w.method, theta, y0, r["count"], r["h"])
        return np.sum(cq * yq, axis=(0, 1)) + np.sum(c1 * y1, axis=0)

    for i in range(w.theta.shape[0]):
        e = 1e-6 * np.abs(w.theta[i])
        tp, tm = w.theta.copy(), w.theta.copy()
        tp[i] += e
        tm[i] -= e
        fd = (loss(tp, w.y0) - loss(tm, w.y0)) / (2 * e)
        assert np.allclose(fd, dth[i], rtol=2e-5, atol=2e-7 * np.abs(dth * w.theta).max()
                           / np.abs(w.theta[i]).max()), (i, fd, dth[i])
    for c in range(w.y0.shape[0]):
        e = 1e-6 * max(1.0, np.abs(w.y0[c]).max())
        yp, ym = w.y0.copy(), w.y0.copy()
        yp[c] += e
        ym[c] -= e
        fd = (loss(w.theta, yp) - loss(w.theta, ym)) / (2 * e)
        assert np.allclose(fd, dy0[c], rtol=2e-5, atol=1e-7 * np.abs(dy0).max()), (c, fd, dy0[c])


def test_linear_in_the_cotangents(orc):
    w = _case("loghalo", 2)
    r = _solve(orc, w)
    tq = np.array([0.5, 1.5, 2.5, 4.0])
    rng = np.random.default_rng(7)
    cq = rng.normal(size=(len(tq),) + w.y0.shape)
    dth, dy0 = orc.grad_at(w.system, w.method, w.theta, w.y0, w.t0, w.t1, r["count"], r["h"], tq,
                           cq)
    sth, sy0 = np.zeros_like(dth), np.zeros_like(dy0)
    for q in range(len(tq)):
        one = np.zeros_like(cq)
        one[q] = cq[q]
        a, b = orc.grad_at(w.system, w.method, w.theta, w.y0, w.t0, w.t1, r["count"], r["h"], tq,
                           one)
        sth += a
        sy0 += b
    assert np.allclose(dth, sth, rtol=1e-12, atol=1e-15) and np.allclose(dy0, sy0, rtol=1e-12)


def test_bad_times_give_nan(orc):
    w = _case("lorenz63", 2)
    r = _solve(orc, w)
    for tq in (np.array([0.5, 0.2]), np.array([w.t1 + 0.1]), np.array([np.nan])):
        cq = np.ones((len(tq),) + w.y0.shape)
        dth, dy0 = orc.grad_at(w.system, w.method, w.theta, w.y0, w.t0, w.t1, r["count"],
                               r["h"], tq, cq)
        assert np.all(np.isnan(dth)) and np.all(np.isnan(dy0))
