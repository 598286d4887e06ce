"""Pins of the oracle's forward-mode sensitivities S = dy(t1)/dtheta and
dy(t1)/dy0 on a frozen mesh (CPU only).

The application paper (arXiv 2609.28458, Sec. 2.3 and Sec. 3) integrates the
sensitivity equations beside the orbit with the step size controlled on the
orbit alone; with the steps fixed that is the derivative of the discrete
solution, i.e. the Jacobian of the replay chain (gradsolve, arXiv 2609.02876,
Sec. 3.1).  Pins:
* decay: the exact derivatives of y0 * prod R(-theta h_n);
* the transpose identity lam^T S = the tape's reverse-mode gradient (two
  independent derivative codes: dual numbers forward, a tape backward);
* complex-step directional derivatives S v;
* special states: the Lorenz z axis, planar halo orbits, Robertson's mass,
  HIRES's y7 + y8.
"""
import numpy as np
import pytest

import dao_inputs as di

from test_oracle_systems import R_poly, dR_poly

TSIT = "tsit5"
ROS = "rosenbrock23"


def _solve(orc, w, y0=None, s_cap=8192, **kw):
    y0 = w.y0 if y0 is None else y0
    r = orc.solve(w.system, w.method, w.theta, y0, w.t0, kw.get("t1", w.t1), w.rtol, w.atol,
                  s_cap=s_cap)
    assert np.all(r["status"] == 0)
    return r


def test_decay_sensitivities_closed_form(orc):
    w = di.make("decay", 32)
    r = _solve(orc, w)
    S, Sy, yS = orc.sens(w.system, w.method, w.theta, w.y0, r["count"], r["h"])
    for k in range(w.n):
        h = r["h"][k, :r["count"][k]]
        z = -w.theta[0, k] * h
        Rz = R_poly(orc, z)
        prod = np.prod(Rz)
        assert yS[0, k] == r["y1"][0, k]
        assert S[0, 0, k] == pytest.approx(w.y0[0, k] * prod * np.sum(-h * dR_poly(orc, z) / Rz),
                                           rel=1e-12)
        assert Sy[0, 0, k] == pytest.approx(prod, rel=1e-13)


CASES = [("decay", TSIT), ("lotka_volterra", TSIT), ("lorenz63", TSIT), ("loghalo", TSIT),
         ("robertson", ROS), ("lorenz63", ROS), ("hires", ROS)]


def _case(orc, system, method, n):
    w = di.make(system, n)
    if w.method != method:
        w.method = method
        if system == "lorenz63":
            w.t1 = 0.5
    return w, _solve(orc, w)


@pytest.mark.parametrize("system,method", CASES)
def test_forward_transposes_to_the_tape_gradient(orc, system, method):
    w, r = _case(orc, system, method, 6)
    S, Sy, yS = orc.sens(system, method, w.theta, w.y0, r["count"], r["h"])
    assert np.array_equal(yS, r["y1"])
    lam = np.random.default_rng(7).normal(size=w.y0.shape)
    dth, dy0, _ = orc.grad(system, method, w.theta, w.y0, r["count"], r["h"], lam)
    g_fwd = np.einsum("cjk,ck->jk", S, lam)
    gy_fwd = np.einsum("cjk,ck->jk", Sy, lam)
    assert np.allclose(g_fwd, dth, rtol=1e-11, atol=1e-13 * np.abs(dth).max())
    assert np.allclose(gy_fwd, dy0, rtol=1e-11, atol=1e-13 * np.abs(dy0).max())


@pytest.mark.parametrize("system,method", CASES)
def test_forward_matches_complex_step(orc, system, method):
    w, r = _case(orc, system, method, 4)
    S, Sy, _ = orc.sens(system, method, w.theta, w.y0, r["count"], r["h"])
    rng = np.random.default_rng(5)
    vth = rng.normal(size=w.theta.shape) * np.abs(w.theta)
    vy = rng.normal(size=w.y0.shape)
    _, dyS = orc.replay_cs(system, method, w.theta, w.y0, vth, vy, r["count"], r["h"])
    pred = np.einsum("cjk,jk->ck", S, vth) + np.einsum("cjk,jk->ck", Sy, vy)
    assert np.allclose(pred, dyS, rtol=1e-11, atol=1e-13 * np.abs(dyS).max())


def test_sensitivities_without_initial_state_columns(orc):
    w, r = _case(orc, "lorenz63", TSIT, 5)
    S1, Sy, _ = orc.sens(w.system, w.method, w.theta, w.y0, r["count"], r["h"])
    S2, none, _ = orc.sens(w.system, w.method, w.theta, w.y0, r["count"], r["h"], with_y0=False)
    assert none is None
    assert np.array_equal(S1, S2)


def test_lorenz_z_axis_sensitivities(orc):
    w = di.make("lorenz63", 6)
    y0 = np.zeros_like(w.y0)
    y0[2] = w.y0[2]
    r = _solve(orc, w, y0=y0, s_cap=4096)
    S, Sy, _ = orc.sens(w.system, w.method, w.theta, y0, r["count"], r["h"])
    assert np.all(S[:2] == 0.0)            # x and y stay zero for every theta
    assert np.all(S[2, :2] == 0.0)         # sigma and rho do not enter z
    for k in range(w.n):
        h = r["h"][k, :r["count"][k]]
        z = -w.theta[2, k] * h
        Rz = R_poly(orc, z)
        y3 = y0[2, k] * np.prod(Rz)
        assert S[2, 2, k] == pytest.approx(y3 * np.sum(-h * dR_poly(orc, z) / Rz), rel=1e-12)
        assert Sy[2, 2, k] == pytest.approx(np.prod(Rz), rel=1e-13)


def test_halo_planar_orbit_has_no_q_sensitivity(orc):
    w = di.make("loghalo", 6)
    y0 = w.y0.copy()
    y0[2] = 0.0
    y0[5] = 0.0
    r = orc.solve(w.system, w.method, w.theta, y0, 0.0, 10.0, 1e-8, 1e-10, s_cap=8192)
    S, Sy, _ = orc.sens(w.system, w.method, w.theta, y0, r["count"], r["h"])
    assert np.all(S[:, 2] == 0.0)          # q enters only through z
    assert np.all(S[2] == 0.0) and np.all(S[5] == 0.0)
    assert np.all(S[0, 0] != 0.0)


def test_robertson_mass_sensitivities(orc):
    # sum(y) = sum(y0) along the replay for every theta: its theta-derivative
    # vanishes and its y0-derivative is one in every direction.
    w = di.make("robertson", 6)
    r = _solve(orc, w, s_cap=4096)
    S, Sy, _ = orc.sens(w.system, w.method, w.theta, w.y0, r["count"], r["h"])
    scale = np.abs(S * w.theta[None]).max(axis=(0, 1))
    assert np.all(np.abs((S * w.theta[None]).sum(axis=0)).max(axis=0) < 1e-10 * scale)
    assert np.max(np.abs(Sy.sum(axis=0) - 1.0)) < 1e-12


def test_hires_invariant_sensitivities(orc):
    # y7 + y8 is conserved, so its sensitivity to every rate constant is zero
    # and its sensitivity to y0 is the indicator of components 7 and 8.
    w = di.make("hires", 3)
    r = _solve(orc, w)
    S_th, S_y0, _ = orc.sens(w.system, w.method, w.theta, w.y0, r["count"], r["h"], with_y0=True)
    inv_th = S_th[6] + S_th[7]
    assert np.all(np.abs(inv_th * w.theta).max(axis=0) < 1e-12)
    inv_y0 = S_y0[6] + S_y0[7]
    ind = np.zeros(8)
    ind[6:8] = 1.0
    assert np.allclose(inv_y0, ind[:, None], rtol=0, atol=1e-12)


def test_planted_mistake_is_caught(orc):
    # A wrong derivative (one column of S scaled) must fail the transpose pin.
    w, r = _case(orc, "lotka_volterra", TSIT, 3)
    S, Sy, _ = orc.sens(w.system, w.method, w.theta, w.y0, r["count"], r["h"])
    S = S.copy()
    S[:, 1] *= 1.0 + 1e-6
    lam = np.random.default_rng(1).normal(size=w.y0.shape)
    dth, _, _ = orc.grad(w.system, w.method, w.theta, w.y0, r["count"], r["h"], lam)
    assert not np.allclose(np.einsum("cjk,ck->jk", S, lam), dth, rtol=1e-11, atol=0)
