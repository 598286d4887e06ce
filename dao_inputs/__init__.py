"""Seeded synthetic ensembles shared by the tests, the benchmark and the oracle.

This module draws random inputs only: it holds none of the method's
arithmetic, imports neither the GPU library nor the oracle, and is the one
piece both sides read.  Generator: NumPy ``Generator(PCG64(seed))``; draw
order is parameter by parameter (n values each), then the initial state
component by component, then the targets.  Arrays are SoA: parameters
``[p][n]``, states ``[d][n]``.

Workloads (arXiv 2609.02876 names the systems; sizes and distributions are
the five benchmark ensembles):

* ``lotka_volterra``  theta=(a,b,g,d) ~ U[0.5,1.5], y0 ~ U[0.5,2]^2, t in [0,10]
* ``lorenz63``        sigma~U[9,11], rho~U[20,30], beta~U[2,3], y0 ~ N(0,1)^3+(1,1,20), t in [0,2]
* ``mlp``             4-64-64-4 tanh MLP, Glorot-uniform weights, zero biases, y0 ~ N(0,1)^4, t in [0,1]
* ``robertson``       k = (0.04, 3e7, 1e4) * exp(0.1 N(0,1)), y0 = (1,0,0), t in [0,1e5]
* ``loghalo``         v0~U[0.9,1.1], Rc~U[0.1,0.3], q~U[0.8,1.0]; x0~N(0,1)^3, v0~N(0,0.5)^3, t in [0,50]
* ``decay``           theta ~ U[0.5,2], y0 ~ U[0.5,2], t in [0,2]  (linear test system)
* ``lorenz63_spread`` the Lorenz ensemble with its difficulty spread (the divergence stress
                      test): rho log-uniform on [20, 1000], so that step counts range over
                      about an order of magnitude; sigma, beta, y0 and targets as ``lorenz63``
* ``<ensemble>_vern7``, ``<ensemble>_rodas5p``  an ensemble (same draws) integrated with
                      the Verner 7(6) pair or Rodas5P (METHOD_VARIANTS)
* ``hires``           HIRES, 8 species; the twelve rate constants at their nominal values for
                      every trajectory (the ensemble carries no free rate constant); the two
                      nonzero components of the standard initial state (1, 0, ..., 0, 0.0057)
                      each scaled by U[0.5,1.5]; t in [0, 321.8122]; targets U[0,0.01]^8

"N(0, s)" is read as standard deviation s.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


@dataclass
class Workload:
    name: str
    system: str
    method: str
    dtype: str
    n: int
    t0: float
    t1: float
    rtol: float
    atol: float
    theta: np.ndarray
    y0: np.ndarray
    target: np.ndarray
    loss: str  # "half_sq" (L = sum 1/2 |y - target|^2), "mse" (mean over n*d), "half_sq_pos"
    extra: dict = field(default_factory=dict)

    @property
    def d(self):
        return self.y0.shape[0]


SEED_BASE = 1000
DEFAULT_N = {"decay": 4096, "lotka_volterra": 256, "lorenz63": 65536, "mlp": 16384,
             "robertson": 262144, "loghalo": 1048576, "hires": 131072, "lorenz63_spread": 65536}
HIRES_RATES = (1.71, 0.43, 8.32, 0.0007, 8.75, 10.03, 0.035, 1.12, 1.745, 280.0, 0.69, 1.81)
HIRES_T1 = 321.8122
CONFIG_ORDER = ["lotka_volterra", "lorenz63", "mlp", "robertson", "loghalo"]



def _rng(name):
    seed = SEED_BASE + ({"decay": 0, "hires": len(CONFIG_ORDER) + 1,
                         "lorenz63_spread": len(CONFIG_ORDER) + 2}
                        | {k: i + 1 for i, k in enumerate(CONFIG_ORDER)})[name]
    return np.random.Generator(np.random.PCG64(seed))


def glorot(rng, fan_out, fan_in):
    lim = np.sqrt(6.0 / (fan_in + fan_out))
    return rng.uniform(-lim, lim, size=(fan_out, fan_in))


# the same ensembles (same draws) integrated with another method: name ->
# (ensemble, method)
METHOD_VARIANTS = {"lorenz63_vern7": ("lorenz63", "vern7"), "loghalo_vern7": ("loghalo", "vern7"),
                   "decay_vern7": ("decay", "vern7"),
                   "lotka_volterra_vern7": ("lotka_volterra", "vern7"),
                   "robertson_rodas5p": ("robertson", "rodas5p"),
                   "decay_rodas5p": ("decay", "rodas5p"),
                   "lotka_volterra_rodas5p": ("lotka_volterra", "rodas5p"),
                   "hires_rodas5p": ("hires", "rodas5p")}


def make(name: str, n: int | None = None) -> Workload:
    if name in METHOD_VARIANTS:
        ens, method = METHOD_VARIANTS[name]
        base = make(ens, n)
        return Workload(name, base.system, method, base.dtype, base.n, base.t0, base.t1,
                        base.rtol, base.atol, base.theta, base.y0, base.target, base.loss,
                        dict(base.extra))
    n = DEFAULT_N[name] if n is None else int(n)
    rng = _rng(name)
    if name == "decay":
        theta = rng.uniform(0.5, 2.0, size=(1, n))
        y0 = rng.uniform(0.5, 2.0, size=(1, n))
        target = rng.uniform(0.0, 1.0, size=(1, n))
        return Workload(name, name, "tsit5", "f64", n, 0.0, 2.0, 1e-8, 1e-10, theta, y0, target,
                        "half_sq")
    if name == "lotka_volterra":
        theta = rng.uniform(0.5, 1.5, size=(4, n))
        y0 = rng.uniform(0.5, 2.0, size=(2, n))
        target = rng.uniform(0.5, 2.0, size=(2, n))
        return Workload(name, name, "tsit5", "f64", n, 0.0, 10.0, 1e-6, 1e-8, theta, y0, target,
                        "half_sq")
    if name == "lorenz63":
        sigma = rng.uniform(9.0, 11.0, size=n)
        rho = rng.uniform(20.0, 30.0, size=n)
        beta = rng.uniform(2.0, 3.0, size=n)
        theta = np.stack([sigma, rho, beta])
        y0 = rng.normal(0.0, 1.0, size=(3, n)) + np.array([1.0, 1.0, 20.0])[:, None]
        target = rng.normal(0.0, 5.0, size=(3, n))
        return Workload(name, name, "tsit5", "f64", n, 0.0, 2.0, 1e-8, 1e-10, theta, y0, target,
                        "half_sq")
    if name == "lorenz63_spread":
        sigma = rng.uniform(9.0, 11.0, size=n)
        rho = 20.0 * np.power(50.0, rng.uniform(0.0, 1.0, size=n))
        beta = rng.uniform(2.0, 3.0, size=n)
        theta = np.stack([sigma, rho, beta])
        y0 = rng.normal(0.0, 1.0, size=(3, n)) + np.array([1.0, 1.0, 20.0])[:, None]
        target = rng.normal(0.0, 5.0, size=(3, n))
        return Workload(name, "lorenz63", "tsit5", "f64", n, 0.0, 2.0, 1e-8, 1e-10, theta, y0,
                        target, "half_sq")
    if name == "mlp":
        W1 = glorot(rng, 64, 4)
        W2 = glorot(rng, 64, 64)
        W3 = glorot(rng, 4, 64)
        theta = np.concatenate([W1.ravel(), np.zeros(64), W2.ravel(), np.zeros(64), W3.ravel(),
                                np.zeros(4)]).astype(np.float32)
        y0 = rng.normal(0.0, 1.0, size=(4, n)).astype(np.float32)
        target = rng.normal(0.0, 1.0, size=(4, n)).astype(np.float32)
        return Workload(name, name, "tsit5", "f32", n, 0.0, 1.0, 1e-5, 1e-7, theta, y0, target,
                        "mse")
    if name == "robertson":
        k = np.array([0.04, 3e7, 1e4])[:, None] * np.exp(0.1 * rng.normal(0.0, 1.0, size=(3, n)))
        y0 = np.zeros((3, n))
        y0[0] = 1.0
        target = np.repeat(robertson_target()[:, None], n, axis=1)
        return Workload(name, name, "rosenbrock23", "f64", n, 0.0, 1e5, 1e-6, 1e-10, k, y0,
                        target, "half_sq")
    if name == "loghalo":
        v0 = rng.uniform(0.9, 1.1, size=n)
        rc = rng.uniform(0.1, 0.3, size=n)
        q = rng.uniform(0.8, 1.0, size=n)
        theta = np.stack([v0, rc, q])
        x0 = rng.normal(0.0, 1.0, size=(3, n))
        v = rng.normal(0.0, 0.5, size=(3, n))
        y0 = np.concatenate([x0, v])
        target = np.concatenate([rng.normal(0.0, 1.0, size=(3, n)), np.zeros((3, n))])
        return Workload(name, name, "tsit5", "f64", n, 0.0, 50.0, 1e-8, 1e-10, theta, y0, target,
                        "half_sq_pos")
    if name == "hires":
        theta = np.repeat(np.array(HIRES_RATES)[:, None], n, axis=1)
        y0 = np.zeros((8, n))
        y0[0] = rng.uniform(0.5, 1.5, size=n)
        y0[7] = 0.0057 * rng.uniform(0.5, 1.5, size=n)
        target = rng.uniform(0.0, 0.01, size=(8, n))
        return Workload(name, name, "rosenbrock23", "f64", n, 0.0, HIRES_T1, 1e-6, 1e-10, theta,
                        y0, target, "half_sq")
    raise KeyError(name)


def robertson_target() -> np.ndarray:
    """State at t=1e5 of Robertson at the nominal rates (stored golden file)."""
    import json
    import os

    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "..", "tests", "golden",
                        "robertson_target.json")
    with open(path) as f:
        return np.array(json.load(f)["y"], dtype=np.float64)


def cotangent(w: Workload, y1: np.ndarray) -> np.ndarray:
    """dL/dy1 for the workload's loss, evaluated at y1 (numpy, float64)."""
    y1 = np.asarray(y1, dtype=np.float64)
    tgt = np.asarray(w.target, dtype=np.float64)
    if w.loss == "half_sq":
        return y1 - tgt
    if w.loss == "half_sq_pos":
        g = y1 - tgt
        g[3:] = 0.0
        return g
    if w.loss == "mse":
        return 2.0 * (y1 - tgt) / (w.n * w.d)
    raise KeyError(w.loss)


def subset(w: Workload, idx) -> Workload:
    """The same workload restricted to the trajectories ``idx`` (shared weights kept)."""
    idx = np.asarray(idx)
    shared = w.system == "mlp"
    return Workload(w.name, w.system, w.method, w.dtype, len(idx), w.t0, w.t1, w.rtol, w.atol,
                    w.theta if shared else np.ascontiguousarray(w.theta[:, idx]),
                    np.ascontiguousarray(w.y0[:, idx]), np.ascontiguousarray(w.target[:, idx]),
                    w.loss, dict(w.extra))
