"""Every right-hand side of the oracle against an independent NumPy restatement
(CPU).

Each field is written here again from its definition, at random points and
random parameters, and compared with the oracle's binary64 field and
Jacobian.  A dropped term, a wrong sign, a swapped rate constant or a
transposed weight matrix in the oracle fails one of these.

* Lotka-Volterra, Robertson: the equations as the benchmark ensembles state
  them (theta = (a, b, g, d): y1' = a y1 - b y1 y2, y2' = d y1 y2 - g y2;
  y1' = -k1 y1 + k3 y2 y3, y2' = k1 y1 - k2 y2^2 - k3 y2 y3, y3' = k2 y2^2).
* Lorenz-63: x' = sigma (y - x), y' = x (rho - z) - y, z' = x y - beta z.
* Flattened logarithmic halo (arXiv 2609.28458 Sec. 3): the acceleration is
  minus the gradient of Phi = 1/2 v0^2 ln(Rc^2 + x^2 + y^2 + z^2 / q^2),
  taken here by complex-step differentiation of Phi itself, so no derivative
  of the potential is written by hand on this side.
* HIRES (Hairer & Wanner, Solving ODEs II, Sec. IV.10): the eight equations
  with the nominal rate constants written as numbers, so the mapping of the
  twelve parameters onto the terms is pinned too.
* Neural field: y' = W3 tanh(W2 tanh(W1 y + b1) + b2) + b3 with random
  nonzero weights and biases in the packing [W1 (64x4, row-major) b1 W2
  (64x64) b2 W3 (4x64) b3].
* Every Jacobian against complex-step derivatives of the NumPy field.
"""
import numpy as np
import pytest

RNG = np.random.default_rng(20261203)


def f_decay(th, y):
    return np.array([-th[0] * y[0]])


def f_lv(th, y):
    a, b, g, d = th
    return np.array([a * y[0] - b * y[0] * y[1], d * y[0] * y[1] - g * y[1]])


def f_lorenz(th, y):
    s, r, b = th
    x, yy, z = y
    return np.array([s * (yy - x), x * (r - z) - yy, x * yy - b * z])


def f_rober(th, y):
    k1, k2, k3 = th
    y1, y2, y3 = y
    return np.array([-k1 * y1 + k3 * y2 * y3, k1 * y1 - k2 * y2 ** 2 - k3 * y2 * y3, k2 * y2 ** 2])


def phi_halo(th, x):
    v0, rc, q = th
    return 0.5 * v0 ** 2 * np.log(rc ** 2 + x[0] ** 2 + x[1] ** 2 + x[2] ** 2 / q ** 2)


def f_halo(th, y):
    """(x, v)' = (v, -grad Phi): the gradient by complex steps of Phi."""
    acc = np.zeros(3)
    xr = np.asarray(y[:3], dtype=np.float64)
    for j in range(3):
        e = np.zeros(3)
        e[j] = 1e-30
        acc[j] = -np.imag(phi_halo(th, xr + 1j * e)) / 1e-30
    return np.concatenate([np.asarray(y[3:]), acc])


def grad_phi_halo_analytic(th, x):
    # for the Jacobian test (a complex step over y needs a field without a
    # complex step inside); pinned to the complex-step gradient of Phi below
    v0, rc, q = th
    D = rc ** 2 + x[0] ** 2 + x[1] ** 2 + x[2] ** 2 / q ** 2
    return v0 ** 2 / D * np.array([x[0], x[1], x[2] / q ** 2])


def f_halo_analytic(th, y):
    return np.concatenate([y[3:], -grad_phi_halo_analytic(th, y[:3])])


HIRES_NOMINAL = np.array([1.71, 0.43, 8.32, 0.0007, 8.75, 10.03, 0.035, 1.12, 1.745, 280.0, 0.69,
                          1.81])


def f_hires_numbers(y):
    """HIRES as printed in the source, constants written as numbers."""
    y1, y2, y3, y4, y5, y6, y7, y8 = y
    return np.array([
        -1.71 * y1 + 0.43 * y2 + 8.32 * y3 + 0.0007,
        1.71 * y1 - 8.75 * y2,
        -10.03 * y3 + 0.43 * y4 + 0.035 * y5,
        8.32 * y2 + 1.71 * y3 - 1.12 * y4,
        -1.745 * y5 + 0.43 * y6 + 0.43 * y7,
        -280.0 * y6 * y8 + 0.69 * y4 + 1.71 * y5 - 0.43 * y6 + 0.69 * y7,
        280.0 * y6 * y8 - 1.81 * y7,
        -280.0 * y6 * y8 + 1.81 * y7,
    ])


def f_hires(th, y):
    """The same with the constants as parameters (k1 .. k12 in order of first
    appearance: 1.71 0.43 8.32 0.0007 8.75 10.03 0.035 1.12 1.745 280 0.69 1.81)."""
    k1, k2, k3, k4, k5, k6, k7, k8, k9, k10, k11, k12 = th
    y1, y2, y3, y4, y5, y6, y7, y8 = y
    return np.array([
        -k1 * y1 + k2 * y2 + k3 * y3 + k4,
        k1 * y1 - k5 * y2,
        -k6 * y3 + k2 * y4 + k7 * y5,
        k3 * y2 + k1 * y3 - k8 * y4,
        -k9 * y5 + k2 * y6 + k2 * y7,
        -k10 * y6 * y8 + k11 * y4 + k1 * y5 - k2 * y6 + k11 * y7,
        k10 * y6 * y8 - k12 * y7,
        -k10 * y6 * y8 + k12 * y7,
    ])


def unpack_mlp(th):
    W1 = th[0:256].reshape(64, 4)
    b1 = th[256:320]
    W2 = th[320:4416].reshape(64, 64)
    b2 = th[4416:4480]
    W3 = th[4480:4736].reshape(4, 64)
    b3 = th[4736:4740]
    return W1, b1, W2, b2, W3, b3


def f_mlp(th, y):
    W1, b1, W2, b2, W3, b3 = unpack_mlp(th)
    return W3 @ np.tanh(W2 @ np.tanh(W1 @ y + b1) + b2) + b3


def draw(system):
    if system == "decay":
        return RNG.uniform(0.5, 2, 1), RNG.normal(size=1)
    if system == "lotka_volterra":
        return RNG.uniform(0.5, 1.5, 4), RNG.uniform(0.1, 3, 2)
    if system == "lorenz63":
        return RNG.uniform([9, 20, 2], [11, 30, 3]), RNG.normal(0, 10, 3)
    if system == "robertson":
        return np.array([0.04, 3e7, 1e4]) * np.exp(0.1 * RNG.normal(size=3)), RNG.uniform(0, 1, 3)
    if system == "loghalo":
        return RNG.uniform([0.9, 0.1, 0.8], [1.1, 0.3, 1.0]), RNG.normal(0, 1, 6)
    if system == "hires":
        return HIRES_NOMINAL * RNG.uniform(0.5, 1.5, 12), RNG.uniform(0, 1, 8)
    if system == "mlp":
        return RNG.normal(0, 0.3, 4740), RNG.normal(size=4)
    raise KeyError(system)


FIELDS = {"decay": f_decay, "lotka_volterra": f_lv, "lorenz63": f_lorenz, "robertson": f_rober,
          "loghalo": f_halo, "hires": f_hires, "mlp": f_mlp}


@pytest.mark.parametrize("system", list(FIELDS))
def test_field_matches_restatement(orc, system):
    for _ in range(50):
        th, y = draw(system)
        got = orc.rhs(system, th, y)
        want = FIELDS[system](th, y)
        scale = np.abs(want).max() + 1e-300
        assert np.allclose(got, want, rtol=1e-13, atol=1e-14 * scale), (system, got, want)


def test_hires_at_nominal_rates_matches_the_printed_field(orc):
    for _ in range(50):
        y = RNG.uniform(0, 1, 8)
        got = orc.rhs("hires", HIRES_NOMINAL, y)
        want = f_hires_numbers(y)
        assert np.allclose(got, want, rtol=1e-13, atol=1e-15 * np.abs(want).max())


def test_halo_restatements_agree():
    """The complex-step gradient of Phi equals the analytic one used for the
    Jacobian test below."""
    for _ in range(20):
        th, y = draw("loghalo")
        assert np.allclose(f_halo(th, y), f_halo_analytic(th, y), rtol=1e-14, atol=1e-15)


def test_mlp_every_layer_matters(orc):
    """Each packed block changes the oracle's field the way the restatement
    says: perturbing one entry of W1, b1, W2, b2, W3 or b3 moves both the
    same way (a transposed W2 or misplaced block would not)."""
    th, y = draw("mlp")
    base = orc.rhs("mlp", th, y)
    for idx in (0 * 4 + 3, 17 * 4 + 1, 256 + 40, 320 + 5 * 64 + 60, 320 + 60 * 64 + 5, 4416 + 9,
                4480 + 2 * 64 + 33, 4736 + 1):
        t2 = th.copy()
        t2[idx] += 0.25
        d_or = orc.rhs("mlp", t2, y) - base
        d_np = f_mlp(t2, y) - f_mlp(th, y)
        assert np.allclose(d_or, d_np, rtol=1e-11, atol=1e-13), idx
        assert np.abs(d_np).max() > 1e-6


JAC_FIELDS = {"decay": f_decay, "lotka_volterra": f_lv, "lorenz63": f_lorenz,
              "robertson": f_rober, "loghalo": f_halo_analytic, "hires": f_hires}


@pytest.mark.parametrize("system", list(JAC_FIELDS))
def test_jacobian_matches_complex_step_of_restatement(orc, system):
    f = JAC_FIELDS[system]
    for _ in range(20):
        th, y = draw(system)
        J = orc.jac(system, th, y)
        d = len(y)
        Jcs = np.zeros((d, d))
        for j in range(d):
            e = np.zeros(d, complex)
            e[j] = 1e-30j
            Jcs[:, j] = np.imag(f(th, y + e)) / 1e-30
        assert np.allclose(J, Jcs, rtol=1e-12, atol=1e-13 * np.abs(Jcs).max()), system
