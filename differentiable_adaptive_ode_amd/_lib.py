"""ctypes binding of libdao.so (the C ABI in include/dao.h), same names.

Argument marshalling only: every step of the solve and the gradient runs in
the library's HIP kernels.  There is no fallback: if libdao.so is missing or
fails to load, importing this module raises.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
SO_PATH = os.path.join(_HERE, "libdao.so")

DAO_OK, DAO_EINVAL, DAO_EDEVICE, DAO_EWORKSPACE, DAO_EUNSUPPORTED = range(5)
STATUS_NAMES = {0: "DAO_OK", 1: "DAO_EINVAL", 2: "DAO_EDEVICE", 3: "DAO_EWORKSPACE",
                4: "DAO_EUNSUPPORTED"}
SYSTEMS = {"decay": 0, "lotka_volterra": 1, "lorenz63": 2, "mlp": 3, "robertson": 4,
           "loghalo": 5, "hires": 6}
METHODS = {"tsit5": 0, "rosenbrock23": 1, "vern7": 2, "rodas5p": 3}
DTYPES = {"f64": 0, "f32": 1}
TRAJ_STATUS = {0: "ok", 1: "max_steps", 2: "nonfinite", 3: "dt_underflow", 4: "capacity"}


class dao_tol(ctypes.Structure):
    _fields_ = [("rtol", ctypes.c_double), ("atol", ctypes.c_double), ("dt0", ctypes.c_double),
                ("max_steps", ctypes.c_int64), ("phases", ctypes.c_int32)]


class dao_record(ctypes.Structure):
    _fields_ = [("s_cap", ctypes.c_int64), ("t", ctypes.c_void_p), ("h", ctypes.c_void_p),
                ("count", ctypes.c_void_p), ("nrej", ctypes.c_void_p),
                ("status", ctypes.c_void_p), ("y", ctypes.c_void_p)]


class DaoError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"{STATUS_NAMES.get(code, code)}: {msg}")
        self.code = code


def _load():
    if not os.path.exists(SO_PATH):
        raise ImportError(
            f"{SO_PATH} is not built; run differentiable_adaptive_ode_amd.build.build() "
            "(hipcc --offload-arch=gfx950)")
    L = ctypes.CDLL(SO_PATH)
    P, I, I64, D, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double, ctypes.c_size_t
    L.dao_system_dims.argtypes = [I, P, P, P]
    L.dao_system_dims.restype = I
    L.dao_solve_workspace_size.argtypes = [I, I, I, I64]
    L.dao_solve_workspace_size.restype = SZ
    L.dao_solve.argtypes = [I, I, I, I64, P, P, D, D, ctypes.POINTER(dao_tol), P,
                            ctypes.POINTER(dao_record), P, SZ, P]
    L.dao_solve.restype = I
    L.dao_grad_workspace_size.argtypes = [I, I, I, I64, I64]
    L.dao_grad_workspace_size.restype = SZ
    L.dao_grad_workspace_min.argtypes = [I, I, I, I64, I64]
    L.dao_grad_workspace_min.restype = SZ
    L.dao_grad.argtypes = [I, I, I, I64, P, P, ctypes.POINTER(dao_record), I64, P, P, P, P, SZ, P]
    L.dao_grad.restype = I
    L.dao_grad_order.argtypes = [I, I, I, I64, ctypes.POINTER(dao_record), I64, P, SZ, P]
    L.dao_grad_order.restype = I
    L.dao_grad_ordered.argtypes = [I, I, I, I64, P, P, ctypes.POINTER(dao_record), I64, P, P, P,
                                   P, SZ, P]
    L.dao_grad_ordered.restype = I
    L.dao_grad_noalloc.argtypes = [I, I, I, I64, P, P, ctypes.POINTER(dao_record), I64, P, P, P,
                                   P]
    L.dao_grad_noalloc.restype = I
    L.dao_solve_sens.argtypes = [I, I, I, I64, P, P, D, D, ctypes.POINTER(dao_tol), P,
                                 ctypes.POINTER(dao_record), P, P, SZ, P]
    L.dao_solve_sens.restype = I
    L.dao_sens_workspace_size.argtypes = [I, I, I, I64, I64]
    L.dao_sens_workspace_size.restype = SZ
    L.dao_sens.argtypes = [I, I, I, I64, P, P, ctypes.POINTER(dao_record), I64, P, P, P, SZ, P]
    L.dao_sens.restype = I
    L.dao_states_workspace_size.argtypes = [I, I, I, I64, I64]
    L.dao_states_workspace_size.restype = SZ
    L.dao_states_at.argtypes = [I, I, I, I64, P, P, D, D, ctypes.POINTER(dao_record), I64, I64,
                                P, P, P, SZ, P]
    L.dao_states_at.restype = I
    L.dao_grad_at_workspace_size.argtypes = [I, I, I, I64, I64, I64]
    L.dao_grad_at_workspace_size.restype = SZ
    L.dao_grad_at.argtypes = [I, I, I, I64, P, P, D, D, ctypes.POINTER(dao_record), I64, I64, P,
                              P, P, P, P, P, SZ, P]
    L.dao_grad_at.restype = I
    L.dao_record_stats.argtypes = [I64, ctypes.POINTER(dao_record), P, P]
    L.dao_record_stats.restype = I
    L.dao_sqerr_cotangent.argtypes = [I, I64, I, I, P, P, D, P, P]
    L.dao_sqerr_cotangent.restype = I
    L.dao_last_error.argtypes = []
    L.dao_last_error.restype = ctypes.c_char_p
    L.dao_version.argtypes = []
    L.dao_version.restype = ctypes.c_char_p
    return L


lib = _load()


def check(code: int):
    if code != DAO_OK:
        raise DaoError(code, lib.dao_last_error().decode())


def dao_system_dims(system: int):
    d, p, s = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    check(lib.dao_system_dims(system, ctypes.byref(d), ctypes.byref(p), ctypes.byref(s)))
    return d.value, p.value, bool(s.value)


def dao_solve_workspace_size(system, method, dtype, n):
    return lib.dao_solve_workspace_size(system, method, dtype, n)


def dao_solve(system, method, dtype, n, theta, y0, t0, t1, tol, y1, rec, workspace, ws_bytes,
              stream):
    return lib.dao_solve(system, method, dtype, n, theta, y0, t0, t1,
                         ctypes.byref(tol) if tol is not None else None, y1,
                         ctypes.byref(rec) if rec is not None else None, workspace, ws_bytes,
                         stream)


def dao_solve_sens(system, method, dtype, n, theta, y0, t0, t1, tol, y1, rec, S_theta, workspace,
                   ws_bytes, stream):
    return lib.dao_solve_sens(system, method, dtype, n, theta, y0, t0, t1,
                              ctypes.byref(tol) if tol is not None else None, y1,
                              ctypes.byref(rec) if rec is not None else None, S_theta, workspace,
                              ws_bytes, stream)


def dao_sens_workspace_size(system, method, dtype, n, s_max):
    return lib.dao_sens_workspace_size(system, method, dtype, n, s_max)


def dao_sens(system, method, dtype, n, theta, y0, rec, s_max, S_theta, S_y0, workspace, ws_bytes,
             stream):
    return lib.dao_sens(system, method, dtype, n, theta, y0,
                        ctypes.byref(rec) if rec is not None else None, s_max, S_theta, S_y0,
                        workspace, ws_bytes, stream)


def dao_states_workspace_size(system, method, dtype, n, s_max):
    return lib.dao_states_workspace_size(system, method, dtype, n, s_max)


def dao_states_at(system, method, dtype, n, theta, y0, t0, t1, rec, s_max, m, tq, yq, workspace,
                  ws_bytes, stream):
    return lib.dao_states_at(system, method, dtype, n, theta, y0, t0, t1,
                             ctypes.byref(rec) if rec is not None else None, s_max, m, tq, yq,
                             workspace, ws_bytes, stream)


def dao_grad_at_workspace_size(system, method, dtype, n, s_max, m):
    return lib.dao_grad_at_workspace_size(system, method, dtype, n, s_max, m)


def dao_grad_at(system, method, dtype, n, theta, y0, t0, t1, rec, s_max, m, tq, dLdyq, dLdy1,
                dLdtheta, dLdy0, workspace, ws_bytes, stream):
    return lib.dao_grad_at(system, method, dtype, n, theta, y0, t0, t1,
                           ctypes.byref(rec) if rec is not None else None, s_max, m, tq, dLdyq,
                           dLdy1, dLdtheta, dLdy0, workspace, ws_bytes, stream)


def dao_grad_workspace_size(system, method, dtype, n, s_max):
    return lib.dao_grad_workspace_size(system, method, dtype, n, s_max)


def dao_grad_workspace_min(system, method, dtype, n, s_max):
    return lib.dao_grad_workspace_min(system, method, dtype, n, s_max)


def dao_grad(system, method, dtype, n, theta, y0, rec, s_max, dLdy1, dLdtheta, dLdy0, workspace,
             ws_bytes, stream):
    return lib.dao_grad(system, method, dtype, n, theta, y0,
                        ctypes.byref(rec) if rec is not None else None, s_max, dLdy1, dLdtheta,
                        dLdy0, workspace, ws_bytes, stream)


def dao_grad_order(system, method, dtype, n, rec, s_max, workspace, ws_bytes, stream):
    return lib.dao_grad_order(system, method, dtype, n,
                              ctypes.byref(rec) if rec is not None else None, s_max, workspace,
                              ws_bytes, stream)


def dao_grad_ordered(system, method, dtype, n, theta, y0, rec, s_max, dLdy1, dLdtheta, dLdy0,
                     workspace, ws_bytes, stream):
    return lib.dao_grad_ordered(system, method, dtype, n, theta, y0,
                                ctypes.byref(rec) if rec is not None else None, s_max, dLdy1,
                                dLdtheta, dLdy0, workspace, ws_bytes, stream)


def dao_record_stats(n, rec, out, stream):
    return lib.dao_record_stats(n, ctypes.byref(rec) if rec is not None else None, out, stream)


def dao_grad_noalloc(system, method, dtype, n, theta, y0, rec, s_max, dLdy1, dLdtheta, dLdy0,
                     stream):
    return lib.dao_grad_noalloc(system, method, dtype, n, theta, y0,
                                ctypes.byref(rec) if rec is not None else None, s_max, dLdy1,
                                dLdtheta, dLdy0, stream)


def dao_sqerr_cotangent(dtype, n, d, d_used, y1, target, scale, out, stream):
    return lib.dao_sqerr_cotangent(dtype, n, d, d_used, y1, target, scale, out, stream)


def dao_last_error() -> str:
    return lib.dao_last_error().decode()


def dao_version() -> str:
    return lib.dao_version().decode()
