"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every function include/dao.h declares, and rejects invalid arguments before
enqueuing any work."""
import ctypes
import os
import re

import pytest

ROOT = os.path.abspath(os.path.join(os.path.dirname(__file__), ".."))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "dao.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(dao_[a-z_0-9]+)\s*\(", src, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def L():
    from differentiable_adaptive_ode_amd import _lib

    return _lib


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("dao_solve", "dao_grad", "dao_grad_order", "dao_grad_ordered", "dao_solve_sens",
              "dao_sens", "dao_sens_workspace_size", "dao_states_at", "dao_states_workspace_size",
              "dao_solve_workspace_size", "dao_grad_workspace_size", "dao_grad_at",
              "dao_grad_at_workspace_size",
              "dao_grad_workspace_min", "dao_system_dims", "dao_sqerr_cotangent",
              "dao_record_stats", "dao_last_error", "dao_version"):
        assert n in names, n


def test_library_exports_every_declared_symbol(L):
    lib = ctypes.CDLL(L.SO_PATH)
    for n in declared_functions():
        assert hasattr(lib, n), n


def test_system_dims(L):
    assert L.dao_system_dims(L.SYSTEMS["lorenz63"]) == (3, 3, False)
    assert L.dao_system_dims(L.SYSTEMS["mlp"]) == (4, 4740, True)
    assert L.dao_system_dims(L.SYSTEMS["loghalo"]) == (6, 3, False)
    assert L.dao_system_dims(L.SYSTEMS["hires"]) == (8, 12, False)
    with pytest.raises(L.DaoError):
        L.dao_system_dims(17)


def _solve(L, **over):
    args = dict(system=2, method=0, dtype=0, n=10, theta=1, y0=1, t0=0.0, t1=1.0,
                tol=L.dao_tol(1e-6, 1e-8, 0.0, 1000), y1=1,
                rec=L.dao_record(16, 1, 1, 1, 1, 1), ws=1, wsb=256, stream=None)
    args.update(over)
    return L.dao_solve(args["system"], args["method"], args["dtype"], args["n"], args["theta"],
                       args["y0"], args["t0"], args["t1"], args["tol"], args["y1"], args["rec"],
                       args["ws"], args["wsb"], args["stream"])


@pytest.mark.parametrize("over,code", [
    (dict(t1=-1.0), 1), (dict(t0=float("nan")), 1), (dict(n=-3), 1),
    (dict(system=9), 1), (dict(method=5), 1), (dict(dtype=7), 1),
    (dict(theta=None), 1), (dict(y0=None), 1), (dict(y1=None), 1), (dict(rec=None), 1),
    (dict(ws=None), 3), (dict(wsb=8), 3), (dict(system=5, method=1), 4), (dict(system=3), 4),
])
def test_solve_argument_errors(L, over, code):
    if "tol" not in over:
        pass
    assert _solve(L, **over) == code
    assert L.dao_last_error() != ""


@pytest.mark.parametrize("field,val", [("rtol", 0.0), ("atol", -1.0), ("max_steps", 0),
                                       ("dt0", float("inf")), ("phases", 3), ("phases", -1)])
def test_solve_tolerance_errors(L, field, val):
    tol = L.dao_tol(1e-6, 1e-8, 0.0, 1000)
    setattr(tol, field, val)
    assert _solve(L, tol=tol) == 1


def test_empty_ensemble_is_a_no_op(L):
    assert _solve(L, n=0, theta=None, y0=None, y1=None) == 0


def test_grad_argument_errors(L):
    rec = L.dao_record(16, None, 1, 1, None, 1)
    ok = dict(system=2, method=0, dtype=0, n=4, theta=1, y0=1, rec=rec, s_max=8, g=1, dth=1,
              dy0=1, ws=1, wsb=1 << 30, st=None)

    def call(**o):
        a = dict(ok)
        a.update(o)
        return L.dao_grad(a["system"], a["method"], a["dtype"], a["n"], a["theta"], a["y0"],
                          a["rec"], a["s_max"], a["g"], a["dth"], a["dy0"], a["ws"], a["wsb"],
                          a["st"])

    assert call(s_max=17) == 1          # s_max > s_cap
    assert call(s_max=-1) == 1
    assert call(rec=None) == 1
    assert call(g=None) == 1
    assert call(theta=None) == 1
    assert call(system=5, method=1) == 4
    assert call(n=0) == 0


def test_grad_order_and_ordered_argument_errors(L):
    rec = L.dao_record(16, None, 1, 1, None, 1)
    # the order step reads only the record's counts: no theta, y0 or cotangent
    assert L.dao_grad_order(2, 0, 0, 4, None, 8, 1, 1 << 30, None) == 1   # rec NULL
    assert L.dao_grad_order(2, 0, 0, 4, rec, 17, 1, 1 << 30, None) == 1   # s_max > s_cap
    assert L.dao_grad_order(2, 0, 0, 4, rec, 8, None, 1 << 30, None) == 3  # no workspace
    assert L.dao_grad_order(5, 1, 0, 4, rec, 8, 1, 1 << 30, None) == 4    # not provided
    assert L.dao_grad_order(2, 0, 0, 0, rec, 8, None, 0, None) == 0       # empty ensemble
    assert "dao_grad_order" in L.dao_last_error() or L.dao_last_error() == ""

    def ordered(**o):
        a = dict(theta=1, y0=1, g=1, ws=1, wsb=1 << 30, s_max=8)
        a.update(o)
        return L.dao_grad_ordered(2, 0, 0, 4, a["theta"], a["y0"], rec, a["s_max"], a["g"], 1, 1,
                                  a["ws"], a["wsb"], None)

    assert ordered(g=None) == 1
    assert "dao_grad_ordered" in L.dao_last_error()
    assert ordered(theta=None) == 1
    assert ordered(y0=None) == 1
    assert ordered(s_max=-1) == 1
    assert ordered(wsb=16) == 3


def test_sensitivity_argument_errors(L):
    tol = L.dao_tol(1e-6, 1e-8, 0.0, 1000)
    rec = L.dao_record(16, 1, 1, 1, 1, 1)

    def solve_sens(**o):
        a = dict(system=2, method=0, dtype=0, n=10, S=1, ws=1, wsb=256)
        a.update(o)
        return L.dao_solve_sens(a["system"], a["method"], a["dtype"], a["n"], 1, 1, 0.0, 1.0, tol,
                                1, rec, a["S"], a["ws"], a["wsb"], None)

    assert solve_sens(S=None) == 1
    assert "dao_solve_sens" in L.dao_last_error()
    assert solve_sens(system=3, dtype=1) == 4       # neural field: shared weights
    assert solve_sens(ws=None) == 3
    assert solve_sens(n=0) == 0                     # empty ensemble: nothing to do

    def sens(**o):
        a = dict(system=2, method=0, n=4, s_max=8, St=1, Sy=None, ws=1, wsb=1 << 20, theta=1)
        a.update(o)
        return L.dao_sens(a["system"], a["method"], 0, a["n"], a["theta"], 1, rec, a["s_max"],
                          a["St"], a["Sy"], a["ws"], a["wsb"], None)

    assert sens(St=None, Sy=None) == 1
    assert sens(s_max=17) == 1
    assert sens(theta=None) == 1
    assert sens(ws=None) == 3
    assert sens(system=3) == 4                      # the neural field: reverse mode only
    assert sens(n=0) == 0
    assert L.dao_sens_workspace_size(2, 0, 0, 100, 50) > 0
    assert L.dao_sens_workspace_size(3, 0, 1, 100, 50) == 0   # not provided


def test_states_at_argument_errors(L):
    rec = L.dao_record(16, None, 1, 1, None, 1)

    def call(**o):
        a = dict(system=2, method=0, n=4, t0=0.0, t1=1.0, s_max=8, m=3, tq=1, yq=1, ws=1,
                 wsb=1 << 20, theta=1)
        a.update(o)
        return L.dao_states_at(a["system"], a["method"], 0, a["n"], a["theta"], 1, a["t0"], a["t1"],
                               rec, a["s_max"], a["m"], a["tq"], a["yq"], a["ws"], a["wsb"], None)

    assert call(tq=None) == 1
    assert "dao_states_at" in L.dao_last_error()
    assert call(yq=None) == 1
    assert call(m=-1) == 1
    assert call(t1=-1.0) == 1
    assert call(t0=float("inf")) == 1
    assert call(s_max=17) == 1
    assert call(ws=None) == 3
    assert call(system=3, method=0) == 4       # the neural field: not provided
    assert call(m=0, tq=None, yq=None) == 0    # nothing requested
    assert call(n=0) == 0


def test_cotangent_argument_errors(L):
    assert L.dao_sqerr_cotangent(0, 4, 3, 4, 1, 1, 1.0, 1, None) == 1
    assert L.dao_sqerr_cotangent(0, 4, 0, 0, 1, 1, 1.0, 1, None) == 1
    assert L.dao_sqerr_cotangent(0, 4, 3, 3, None, 1, 1.0, 1, None) == 1
    assert L.dao_sqerr_cotangent(0, 0, 3, 3, None, None, 1.0, None, None) == 0


def test_record_stats_argument_errors(L):
    rec = L.dao_record(16, None, 1, 1, None, 1)
    assert L.dao_record_stats(-1, rec, 1, None) == 1
    assert "n = -1" in L.dao_last_error()
    assert L.dao_record_stats(4, rec, None, None) == 1
    assert "out" in L.dao_last_error()
    assert L.dao_record_stats(4, None, 1, None) == 1
    assert L.dao_record_stats(4, L.dao_record(16, None, 1, None, None, 1), 1, None) == 1
    assert L.dao_record_stats(4, L.dao_record(16, None, 1, 1, None, None), 1, None) == 1
    assert L.dao_record_stats(0, None, None, None) == 1


def test_solve_workspace_holds_two_phases(L):
    """The size dao_solve_workspace_size reports covers two phases for every
    per-trajectory system (any solve may be asked for them), and only the
    queue for the neural field; n = 0 gives the one-phase minimum."""
    ids = (L.SYSTEMS["lorenz63"], 0, 0)
    base = L.dao_solve_workspace_size(*ids, 0)
    assert L.dao_solve_workspace_size(*ids, 1000) >= base + 1000 * (2 * 3 + 2 + 9) * 8
    assert L.dao_solve_workspace_size(L.SYSTEMS["mlp"], 0, 1, 1000) == \
        L.dao_solve_workspace_size(L.SYSTEMS["mlp"], 0, 1, 0)


def test_grad_noalloc_rejects_before_touching_the_device(L):
    """More scratch than the static array holds is refused on the host, with
    the sizes in the message; argument errors come first, as in dao_grad."""
    rec = L.dao_record(1 << 20, None, 1, 1, None, 1)
    ids = (L.SYSTEMS["lorenz63"], 0, 0)
    assert L.dao_grad_noalloc(*ids, 64, 1, 1, rec, 1 << 20, 1, None, None, None) == \
        L.DAO_EWORKSPACE
    msg = L.dao_last_error()
    assert "dao_grad_noalloc" in msg and "static" in msg
    assert L.dao_grad_noalloc(*ids, 64, 1, 1, rec, -1, 1, None, None, None) == L.DAO_EINVAL
    assert L.dao_grad_noalloc(*ids, 64, None, 1, rec, 8, 1, None, None, None) == L.DAO_EINVAL
    assert L.dao_grad_noalloc(9, 0, 0, 64, 1, 1, rec, 8, 1, None, None, None) == L.DAO_EINVAL


def test_gradient_workspace_sizes_are_consistent(L):
    # For every supported (system, method, dtype): the minimum workspace fits
    # in the recommended one, both grow with n and s_max, and the neural
    # field's holds one row of 4,740 partial sums per chunk of 16-trajectory
    # groups (a chunk per group up to 2,048 groups, then 2,048 chunks).
    sizes = (0, 1, 65, 1000, 40_000, 1 << 20)
    for sysname, sid in L.SYSTEMS.items():
        for mname, mid in L.METHODS.items():
            for did in L.DTYPES.values():
                prev_min = prev_size = 0
                for n in sizes:
                    size = L.dao_grad_workspace_size(sid, mid, did, n, 64)
                    if size == 0:
                        break  # combination not provided
                    smin = L.dao_grad_workspace_min(sid, mid, did, n, 64)
                    assert 0 < smin <= size, (sysname, mname, did, n)
                    assert smin >= prev_min and size >= prev_size, (sysname, mname, did, n)
                    assert L.dao_grad_workspace_min(sid, mid, did, n, 256) >= smin
                    prev_min, prev_size = smin, size
    mlp = L.SYSTEMS["mlp"]
    for n in (1, 16 * 2048, 16 * 2048 + 1, 1 << 20):
        groups = (n + 15) // 16
        chunks = min(groups, 2048)
        rows = L.dao_grad_workspace_min(mlp, 0, 1, n, 64) - L.dao_grad_workspace_min(mlp, 0, 1, 0, 64)
        assert rows >= (chunks - 1) * 4740 * 4, n
