"""CPU oracle for the ensemble ODE record / replay / discrete-adjoint path.

TEST INFRASTRUCTURE ONLY.  Imported by ``tests/``, by ``__graft_entry__.smoke``
and by the CPU-baseline leg of ``bench.py``; the GPU library never imports,
links or calls anything here, and this package imports nothing from it.

The arithmetic lives in ``oracle.cpp`` (binary64 C++, ``-ffp-contract=off``):

* adaptive Tsit5 / Rosenbrock23 solve with a record of accepted steps
  (arXiv 2609.02876, Sec. 2.1 and Sec. 3.1, Fig. 2);
* the fixed-step replay of a recorded mesh (Sec. 3.1, Eq. 4);
* the reverse-mode derivative of that replay, computed with a scalar tape
  (Sec. 3.1: exact gradient of the chain with the mesh held fixed);
* a complex-step replay for directional derivatives;
* the forward-mode sensitivities of the replayed final state (dual numbers
  carrying one derivative per parameter and initial-state component);
* states at requested times on a recorded mesh (a shortened step from the
  start of the step that holds each time).

Array layouts match the library boundary: parameters ``[p][n]`` (shared MLP
weights ``[4740]``), states ``[d][n]``, record rows ``[n][s_cap]``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "liboracle.so")
_SRC = os.path.join(_HERE, "oracle.cpp")

SYSTEMS = {"decay": 0, "lotka_volterra": 1, "lorenz63": 2, "mlp": 3, "robertson": 4, "loghalo": 5,
           "hires": 6}
METHODS = {"tsit5": 0, "rosenbrock23": 1, "vern7": 2, "rodas5p": 3}
STATUS = {0: "ok", 1: "max_steps", 2: "nonfinite", 3: "dt_underflow", 4: "capacity"}

_lib = None


def build(force: bool = True) -> str:
    """Compile liboracle.so with g++ (binary64, no FP contraction)."""
    if force or not os.path.exists(_SO):
        cmd = ["g++", "-std=c++17", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
               "-shared", "-pthread", _SRC, "-o", _SO + ".tmp"]
        subprocess.run(cmd, check=True)
        os.replace(_SO + ".tmp", _SO)
    return _SO


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
            build(force=True)
        L = ctypes.CDLL(_SO)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        D = ctypes.c_double
        I = ctypes.c_int
        L.oracle_dims.argtypes = [I, P, P, P]
        L.oracle_tsit5_table.argtypes = [P, P, P]
        L.oracle_ros23_consts.argtypes = [P, P]
        L.oracle_vern7_table.argtypes = [P, P, P, P]
        L.oracle_rodas5p_table.argtypes = [P, P, P]
        for name in ("oracle_solve_f64", "oracle_solve_f32", "oracle_solve_plain_f64",
                     "oracle_solve_plain_f32"):
            getattr(L, name).argtypes = [I, I, I64, P, P, D, D, D, D, D, I64, I64, P, P, P, P, P, P, I]
        for name in ("oracle_trace_f32", "oracle_trace_f64"):
            getattr(L, name).argtypes = [I, I, P, P, D, D, D, D, I64, I64, P, P, P, P, P]
            getattr(L, name).restype = I64
        L.oracle_replay_f64.argtypes = [I, I, I64, P, P, P, P, I64, P, I]
        L.oracle_replay_cs.argtypes = [I, I, I64, P, P, P, P, D, P, P, I64, P, P]
        L.oracle_grad_f64.argtypes = [I, I, I64, P, P, P, P, I64, P, P, P, P, I]
        L.oracle_sens_f64.argtypes = [I, I, I64, P, P, P, P, I64, P, P, P, I]
        L.oracle_states_at_f64.argtypes = [I, I, I64, P, P, D, D, P, P, I64, I64, P, P, I]
        L.oracle_grad_at_f64.argtypes = [I, I, I64, P, P, D, D, P, P, I64, I64, P, P, P, P, P,
                                         I]
        L.oracle_step_f64.argtypes = [I, I, P, P, D, P, P]
        L.oracle_rhs_f64.argtypes = [I, P, P, P]
        L.oracle_jac_f64.argtypes = [I, P, P, P]
        L.oracle_count_solve.argtypes = [I, I, P, P, D, D, D, D, I64, P]
        L.oracle_count_replay_step.argtypes = [I, I, P, P, D]
        L.oracle_count_replay_step.restype = I64
        L.oracle_count_grad_step.argtypes = [I, I, P, P, D, P]
        L.oracle_ctrl_root_f64.argtypes = [D, I]
        L.oracle_ctrl_root_f64.restype = D
        L.oracle_ctrl_root_f32.argtypes = [ctypes.c_float, I]
        L.oracle_ctrl_root_f32.restype = ctypes.c_float
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def dims(system: str):
    d, p, s = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    rc = lib().oracle_dims(SYSTEMS[system], ctypes.byref(d), ctypes.byref(p), ctypes.byref(s))
    assert rc == 0
    return d.value, p.value, bool(s.value)


def tsit5_table():
    c = np.zeros(7)
    A = np.zeros((7, 7))
    bt = np.zeros(7)
    lib().oracle_tsit5_table(_p(c), _p(A), _p(bt))
    return c, A, A[6].copy(), bt


def vern7_table():
    """(c, A, b, bhat) of the Verner 7(6) pair as the oracle holds them."""
    c, b, bh = np.zeros(10), np.zeros(10), np.zeros(10)
    A = np.zeros((10, 10))
    lib().oracle_vern7_table(_p(c), _p(A), _p(b), _p(bh))
    return c, A, b, bh


def rodas5p_table():
    """(gamma, a [8][8] (rows 1-5 of the stage sums; rows 6-7 are Y6 + u6,
    Y7 + u7), C [8][8]) of Rodas5P as the oracle holds them."""
    g = ctypes.c_double()
    A, C = np.zeros((8, 8)), np.zeros((8, 8))
    lib().oracle_rodas5p_table(ctypes.byref(g), _p(A), _p(C))
    return g.value, A, C


def ros23_consts():
    d, e = ctypes.c_double(), ctypes.c_double()
    lib().oracle_ros23_consts(ctypes.byref(d), ctypes.byref(e))
    return d.value, e.value


def solve(system, method, theta, y0, t0, t1, rtol, atol, dt0=0.0, max_steps=100000, s_cap=4096,
          dtype="f64", nthreads=1, record=True, plain=False):
    """Adaptive solve with record.  Returns a dict of numpy arrays.  plain=True
    runs the PLAIN instantiation: the error test e_c / sc_c by IEEE division,
    the controller power by the library pow, the LU by division by the pivot
    (the contract arithmetic's readings undone; rounding-level differences)."""
    d, p, shared = dims(system)
    np_t = np.float64 if dtype == "f64" else np.float32
    theta = np.ascontiguousarray(theta, dtype=np_t)
    y0 = np.ascontiguousarray(y0, dtype=np_t)
    n = y0.shape[-1] if y0.ndim == 2 else 0
    assert y0.shape == (d, n)
    assert theta.shape == ((p,) if shared else (p, n))
    y1 = np.zeros((d, n), np_t)
    count = np.zeros(n, np.int32)
    nrej = np.zeros(n, np.int32)
    status = np.zeros(n, np.int32)
    t_rec = np.zeros((n, s_cap), np_t) if record else None
    h_rec = np.zeros((n, s_cap), np_t) if record else None
    fn = getattr(lib(), f"oracle_solve{'_plain' if plain else ''}_{dtype}")
    rc = fn(SYSTEMS[system], METHODS[method], n, _p(theta), _p(y0), float(t0), float(t1),
            float(rtol), float(atol), float(dt0), int(max_steps), int(s_cap), _p(y1), _p(count),
            _p(nrej), _p(status), _p(t_rec), _p(h_rec), int(nthreads))
    if rc != 0:
        raise ValueError("oracle_solve: invalid argument")
    return dict(y1=y1, count=count, nrej=nrej, status=status, t=t_rec, h=h_rec)


def trace(system, method, theta, y0, t0, t1, rtol, atol, s_cap=4096, dtype="f64", cap=100000):
    """Per-attempt trace of ONE trajectory's solve (theta [p] or the shared
    weights, y0 [d]): dict of arrays h, msq, fac (0.9 msq^(-1/q) before
    truncation and clamping), floor (the mean square of the error
    combination's term sizes over sc, the scale of its rounding), acc."""
    np_t = np.float64 if dtype == "f64" else np.float32
    theta = np.ascontiguousarray(theta, dtype=np_t)
    y0 = np.ascontiguousarray(y0, dtype=np_t)
    out = {k: np.zeros(cap) for k in ("h", "msq", "fac", "floor")}
    acc = np.zeros(cap, np.int32)
    fn = lib().oracle_trace_f32 if dtype == "f32" else lib().oracle_trace_f64
    m = fn(SYSTEMS[system], METHODS[method], _p(theta), _p(y0), float(t0), float(t1),
           float(rtol), float(atol), int(s_cap), int(cap), _p(out["h"]), _p(out["msq"]),
           _p(out["fac"]), _p(out["floor"]), _p(acc))
    if m < 0:
        raise ValueError("oracle_trace: invalid argument")
    res = {k: v[:m] for k, v in out.items()}
    res["acc"] = acc[:m].astype(bool)
    return res


def replay(system, method, theta, y0, count, h, nthreads=1):
    d, p, shared = dims(system)
    theta = np.ascontiguousarray(theta, dtype=np.float64)
    y0 = np.ascontiguousarray(y0, dtype=np.float64)
    h = np.ascontiguousarray(h, dtype=np.float64)
    count = np.ascontiguousarray(count, dtype=np.int32)
    n = y0.shape[1]
    yS = np.zeros((d, n))
    rc = lib().oracle_replay_f64(SYSTEMS[system], METHODS[method], n, _p(theta), _p(y0), _p(count),
                                 _p(h), h.shape[1], _p(yS), int(nthreads))
    assert rc == 0
    return yS


def replay_cs(system, method, theta, y0, dtheta, dy0, count, h, eps=1e-30):
    """Complex-step directional derivative of the replayed final state."""
    d, p, shared = dims(system)
    theta = np.ascontiguousarray(theta, dtype=np.float64)
    y0 = np.ascontiguousarray(y0, dtype=np.float64)
    dtheta = np.ascontiguousarray(dtheta, dtype=np.float64)
    dy0 = np.ascontiguousarray(dy0, dtype=np.float64)
    h = np.ascontiguousarray(h, dtype=np.float64)
    count = np.ascontiguousarray(count, dtype=np.int32)
    n = y0.shape[1]
    yS = np.zeros((d, n))
    dyS = np.zeros((d, n))
    rc = lib().oracle_replay_cs(SYSTEMS[system], METHODS[method], n, _p(theta), _p(y0), _p(dtheta),
                                _p(dy0), float(eps), _p(count), _p(h), h.shape[1], _p(yS), _p(dyS))
    assert rc == 0
    return yS, dyS


def grad(system, method, theta, y0, count, h, dLdy, nthreads=1):
    """Reverse-mode gradient of L on the mesh (count, h).  Returns (dtheta, dy0, yS)."""
    d, p, shared = dims(system)
    theta = np.ascontiguousarray(theta, dtype=np.float64)
    y0 = np.ascontiguousarray(y0, dtype=np.float64)
    h = np.ascontiguousarray(h, dtype=np.float64)
    count = np.ascontiguousarray(count, dtype=np.int32)
    dLdy = np.ascontiguousarray(dLdy, dtype=np.float64)
    n = y0.shape[1]
    dtheta = np.zeros((p,) if shared else (p, n))
    dy0 = np.zeros((d, n))
    yS = np.zeros((d, n))
    rc = lib().oracle_grad_f64(SYSTEMS[system], METHODS[method], n, _p(theta), _p(y0), _p(count),
                               _p(h), h.shape[1], _p(dLdy), _p(dtheta), _p(dy0), _p(yS),
                               int(nthreads))
    assert rc == 0
    return dtheta, dy0, yS


def sens(system, method, theta, y0, count, h, with_y0=True, nthreads=1):
    """Forward-mode sensitivities of the replayed final state on the mesh
    (count, h): S_theta [d][p][n] = dy_S/dtheta and S_y0 [d][d][n] = dy_S/dy0
    (None unless with_y0).  Returns (S_theta, S_y0, yS)."""
    d, p, shared = dims(system)
    assert not shared
    theta = np.ascontiguousarray(theta, dtype=np.float64)
    y0 = np.ascontiguousarray(y0, dtype=np.float64)
    h = np.ascontiguousarray(h, dtype=np.float64)
    count = np.ascontiguousarray(count, dtype=np.int32)
    n = y0.shape[1]
    S_th = np.zeros((d, p, n))
    S_y0 = np.zeros((d, d, n)) if with_y0 else None
    yS = np.zeros((d, n))
    rc = lib().oracle_sens_f64(SYSTEMS[system], METHODS[method], n, _p(theta), _p(y0), _p(count),
                               _p(h), h.shape[1], _p(S_th), _p(S_y0), _p(yS), int(nthreads))
    assert rc == 0
    return S_th, S_y0, yS


def grad_at(system, method, theta, y0, t0, t1, count, h, tq, dLdyq, dLdy1=None, nthreads=1):
    """Gradient of L = sum_q <dLdyq[q], y(tq[q])> + <dLdy1, y(t1)> on the mesh
    (count, h), the states at tq taken as states_at takes them.  dLdyq
    [m][d][n]; dLdy1 [d][n] or None.  Returns (dtheta [p][n], dy0 [d][n])."""
    d, p, shared = dims(system)
    assert not shared
    theta = np.ascontiguousarray(theta, dtype=np.float64)
    y0 = np.ascontiguousarray(y0, dtype=np.float64)
    h = np.ascontiguousarray(h, dtype=np.float64)
    count = np.ascontiguousarray(count, dtype=np.int32)
    tq = np.ascontiguousarray(tq, dtype=np.float64)
    dLdyq = np.ascontiguousarray(dLdyq, dtype=np.float64)
    dLdy1 = None if dLdy1 is None else np.ascontiguousarray(dLdy1, dtype=np.float64)
    n = y0.shape[1]
    dtheta = np.zeros((p, n))
    dy0 = np.zeros((d, n))
    rc = lib().oracle_grad_at_f64(SYSTEMS[system], METHODS[method], n, _p(theta), _p(y0),
                                  float(t0), float(t1), _p(count), _p(h), h.shape[1], len(tq),
                                  _p(tq), _p(dLdyq), _p(dLdy1), _p(dtheta), _p(dy0),
                                  int(nthreads))
    assert rc == 0
    return dtheta, dy0


def states_at(system, method, theta, y0, t0, t1, count, h, tq, nthreads=1):
    """States at the requested times tq (ascending, in [t0, t1]) on the mesh
    (count, h): [m][d][n]."""
    d, p, shared = dims(system)
    theta = np.ascontiguousarray(theta, dtype=np.float64)
    y0 = np.ascontiguousarray(y0, dtype=np.float64)
    h = np.ascontiguousarray(h, dtype=np.float64)
    count = np.ascontiguousarray(count, dtype=np.int32)
    tq = np.ascontiguousarray(tq, dtype=np.float64)
    n, m = y0.shape[1], tq.shape[0]
    yq = np.zeros((m, d, n))
    rc = lib().oracle_states_at_f64(SYSTEMS[system], METHODS[method], n, _p(theta), _p(y0),
                                    float(t0), float(t1), _p(count), _p(h), h.shape[1], m, _p(tq),
                                    _p(yq), int(nthreads))
    assert rc == 0
    return yq


def step(system, method, theta, y, h):
    """One attempted step from y (no acceptance decision): (y_new, error estimate)."""
    d, p, _ = dims(system)
    theta = np.ascontiguousarray(theta, dtype=np.float64)
    y = np.ascontiguousarray(y, dtype=np.float64)
    ynew = np.zeros(d)
    err = np.zeros(d)
    rc = lib().oracle_step_f64(SYSTEMS[system], METHODS[method], _p(theta), _p(y), float(h),
                               _p(ynew), _p(err))
    assert rc == 0
    return ynew, err


def count_solve(system, method, theta, y0, t0, t1, rtol, atol, s_cap=100000):
    """Operation tally of one trajectory's solve: dict(total, init, attempts, accepted)."""
    theta = np.ascontiguousarray(theta, dtype=np.float64)
    y0 = np.ascontiguousarray(y0, dtype=np.float64)
    out = np.zeros(4, np.int64)
    rc = lib().oracle_count_solve(SYSTEMS[system], METHODS[method], _p(theta), _p(y0), float(t0),
                                  float(t1), float(rtol), float(atol), int(s_cap), _p(out))
    assert rc == 0, rc
    return dict(total=int(out[0]), init=int(out[1]), attempts=int(out[2]), accepted=int(out[3]))


def count_replay_step(system, method, theta, y, h):
    """Operation tally of one replay step from y with step h."""
    theta = np.ascontiguousarray(theta, dtype=np.float64)
    y = np.ascontiguousarray(y, dtype=np.float64)
    return int(lib().oracle_count_replay_step(SYSTEMS[system], METHODS[method], _p(theta), _p(y),
                                              float(h)))


def count_grad_step(system, method, theta, y, h):
    """Tally of one gradient step's parts: (replay step flops, reverse-mode
    flops of that step on the tape: 2 per local partial of a variable plus the
    partials' own quotients and tanh derivatives)."""
    theta = np.ascontiguousarray(theta, dtype=np.float64)
    y = np.ascontiguousarray(y, dtype=np.float64)
    out = np.zeros(2, np.int64)
    rc = lib().oracle_count_grad_step(SYSTEMS[system], METHODS[method], _p(theta), _p(y),
                                      float(h), _p(out))
    assert rc == 0
    return int(out[0]), int(out[1])


def ctrl_root(x, q, dtype="f64"):
    """The solve's controller power x^(-1/q) (q = 10 or 6), as the oracle evaluates it."""
    fn = lib().oracle_ctrl_root_f64 if dtype == "f64" else lib().oracle_ctrl_root_f32
    return np.array([fn(float(v), int(q)) for v in np.atleast_1d(x)])


def rhs(system, theta, y):
    d, p, _ = dims(system)
    theta = np.ascontiguousarray(theta, dtype=np.float64)
    y = np.ascontiguousarray(y, dtype=np.float64)
    dy = np.zeros(d)
    assert lib().oracle_rhs_f64(SYSTEMS[system], _p(theta), _p(y), _p(dy)) == 0
    return dy


def jac(system, theta, y):
    d, p, _ = dims(system)
    theta = np.ascontiguousarray(theta, dtype=np.float64)
    y = np.ascontiguousarray(y, dtype=np.float64)
    J = np.zeros((d, d))
    assert lib().oracle_jac_f64(SYSTEMS[system], _p(theta), _p(y), _p(J)) == 0
    return J
