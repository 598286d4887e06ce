"""Torch-facing helpers over the C ABI: device buffers come from PyTorch's
caching allocator and the stream is torch's current stream; all compute is in
libdao's kernels.

    rec, y1 = solve("lorenz63", "tsit5", theta, y0, 0.0, 2.0, rtol=1e-8, atol=1e-10)
    g = cotangent(y1, target)                  # dL/dy1 of 1/2 |y1 - target|^2
    dtheta, dy0 = grad(rec, g)                 # discrete adjoint on the recorded mesh
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

from . import _lib

_TORCH_DTYPE = {"f64": torch.float64, "f32": torch.float32}


def _dtype_name(t: torch.Tensor) -> str:
    if t.dtype == torch.float64:
        return "f64"
    if t.dtype == torch.float32:
        return "f32"
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t):
    return None if t is None else t.data_ptr()


def _tstream(stream=None):
    return torch.cuda.current_stream() if stream is None else stream


def _stream(stream=None):
    return _tstream(stream).cuda_stream


def _expect(device, *specs, placed: bool = True):
    """Each (name, tensor, dtype, shape) of specs (None tensors skipped) must
    have that dtype and shape and be a contiguous device tensor on `device`
    (if given).  The kernels take plain pointers and trust the sizes they are
    told, so every array is checked before its pointer is passed: a cotangent
    of the wrong type would be read as the record's type, a short one read
    past its end.  Types and shapes of all arrays are checked first, then
    where they live (skipped with placed=False)."""
    for name, t, dtype, shape in specs:
        if t is None:
            continue
        if t.dtype != dtype:
            raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
        if tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    for name, t, _, _ in specs:
        if t is None or not placed:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device (cuda) tensor")
        if device is not None and t.device != device:
            raise ValueError(f"{name} is on {t.device}, expected {device}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")


def _check_dev(*ts):
    for t in ts:
        if t is not None:
            if not t.is_cuda:
                raise ValueError("all arrays must be device (cuda) tensors")
            if not t.is_contiguous():
                raise ValueError("all arrays must be contiguous")


@dataclass
class Record:
    """Step record of one ensemble solve (caller-owned device tensors).

    h, t: [n, s_cap] accepted step sizes / start times (rows past count unused)
    count, nrej, status: [n] int32
    The solve's inputs are kept so that grad() can replay the mesh.
    """

    system: str
    method: str
    dtype: str
    theta: torch.Tensor
    y0: torch.Tensor
    t0: float
    t1: float
    h: torch.Tensor
    t: torch.Tensor | None
    count: torch.Tensor
    nrej: torch.Tensor
    status: torch.Tensor
    y: torch.Tensor | None = None  # [n, s_cap, d] recorded states, or None

    @property
    def n(self):
        return self.count.shape[0]

    @property
    def s_cap(self):
        return self.h.shape[1]

    def check(self, placed: bool = True):
        """The record's arrays agree with each other and with its system (the
        kernels index them by n, s_cap and d alone); placed=False leaves out
        where they live."""
        if self.system not in _lib.SYSTEMS or self.method not in _lib.METHODS:
            raise ValueError(f"unknown system or method: {self.system}, {self.method}")
        if self.dtype not in _TORCH_DTYPE:
            raise ValueError(f"unknown dtype {self.dtype}")
        td = _TORCH_DTYPE[self.dtype]
        d, p, shared = _lib.dao_system_dims(_lib.SYSTEMS[self.system])
        if self.count.dim() != 1 or self.h.dim() != 2:
            raise ValueError("count must be [n] and h [n, s_cap]")
        n, s_cap = self.count.shape[0], self.h.shape[1]
        _expect(self.count.device, ("h", self.h, td, (n, s_cap)), ("t", self.t, td, (n, s_cap)),
                ("count", self.count, torch.int32, (n,)), ("nrej", self.nrej, torch.int32, (n,)),
                ("status", self.status, torch.int32, (n,)), ("y0", self.y0, td, (d, n)),
                ("theta", self.theta, td, (p,) if shared else (p, n)),
                ("y", self.y, td, (n, s_cap, d)), placed=placed)

    def stats(self, out=None, stream=None) -> torch.Tensor:
        """Device int64[4] = (max count, total accepted steps, failed
        trajectories, total rejected attempts), written in stream order by
        dao_record_stats; nothing is synchronised."""
        self.check(placed=False)
        _expect(self.count.device, ("out", out, torch.int64, (4,)), placed=False)
        self.check()
        _expect(self.count.device, ("out", out, torch.int64, (4,)))
        o = torch.empty(4, dtype=torch.int64, device=self.count.device) if out is None else out
        _lib.check(_lib.dao_record_stats(self.n, self.c_struct(), _ptr(o), _stream(stream)))
        return o

    def stats_host(self, stream=None) -> dict:
        """stats() read back to the host: this call synchronises the stream."""
        s = _tstream(stream)
        v = self.stats(stream=stream)
        s.synchronize()
        m, tot, bad, rej = (int(x) for x in v.cpu().tolist())
        return dict(s_max=m, steps=tot, failed=bad, rejected=rej)

    def c_struct(self, states: bool = True):
        return _lib.dao_record(self.s_cap, _ptr(self.t), _ptr(self.h), _ptr(self.count),
                               _ptr(self.nrej), _ptr(self.status),
                               _ptr(self.y) if states else None)


class Workspace:
    """Grow-only device scratch for calls on ONE stream (calls that share a
    workspace must not overlap in time).  The buffer is allocated on the
    stream the call launches on, so when it grows the caching allocator hands
    the old block only to later work on that same stream."""

    def __init__(self, device=None):
        self.buf = None
        self.device = device

    def get(self, nbytes: int, device, stream=None) -> torch.Tensor:
        nbytes = max(int(nbytes), 256)
        if self.buf is None or self.buf.numel() < nbytes or self.buf.device != device:
            self.buf = None
            with torch.cuda.stream(_tstream(stream)):
                self.buf = torch.empty(nbytes, dtype=torch.uint8, device=device)
        return self.buf


_default_ws: dict = {}


def _ws(device, ws=None, stream=None):
    """The caller's workspace, or the default one of the stream the call
    launches on (one per device and stream)."""
    if ws is not None:
        return ws
    key = (str(device), _stream(stream))
    if key not in _default_ws:
        _default_ws[key] = Workspace()
    return _default_ws[key]


def alloc_record(n: int, s_cap: int, dtype: str, device, with_t: bool = True,
                 states_dim: int = 0) -> dict:
    """Record buffers; states_dim > 0 also allocates the recorded states [n, s_cap, d]."""
    td = _TORCH_DTYPE[dtype]
    return dict(h=torch.empty((n, s_cap), dtype=td, device=device),
                t=torch.empty((n, s_cap), dtype=td, device=device) if with_t else None,
                count=torch.empty(n, dtype=torch.int32, device=device),
                nrej=torch.empty(n, dtype=torch.int32, device=device),
                status=torch.empty(n, dtype=torch.int32, device=device),
                y=(torch.empty((n, s_cap, states_dim), dtype=td, device=device)
                   if states_dim > 0 else None))


def _check_record_buffers(b: dict, n: int, d: int, dtype, device):
    """Record buffers passed in by the caller (see alloc_record)."""
    s_cap = b["h"].shape[1] if b["h"].dim() == 2 else -1
    _expect(device, ("rec_buffers['h']", b["h"], dtype, (n, s_cap)),
            ("rec_buffers['t']", b.get("t"), dtype, (n, s_cap)),
            *((f"rec_buffers['{k}']", b[k], torch.int32, (n,)) for k in ("count", "nrej", "status")),
            ("rec_buffers['y']", b.get("y"), dtype, (n, s_cap, d)))


def solve(system: str, method: str, theta: torch.Tensor, y0: torch.Tensor, t0: float, t1: float,
          rtol: float, atol: float, dt0: float = 0.0, max_steps: int = 100000, s_cap: int = 4096,
          record_t: bool = True, record_states: bool = False, out=None, rec_buffers=None,
          workspace=None, stream=None, out_sens=None, phases: int = 0, _sens=False):
    """Adaptive solve with record.  Returns (Record, y1).

    record_states: also keep the state at the start of every accepted step, so
    that grad() at the solve's theta skips the replay's forward pass.
    phases: 0 automatic, 1 or 2 forces one or two phases (same results).
    Failed trajectories do not raise: see Record.stats().
    """
    _check_dev(theta, y0)
    dtype = _dtype_name(y0)
    if theta.dtype != y0.dtype:
        raise TypeError("theta and y0 must share a dtype")
    d, p, shared = _lib.dao_system_dims(_lib.SYSTEMS[system])
    n = y0.shape[1] if y0.dim() == 2 else 0
    if y0.shape != (d, n):
        raise ValueError(f"y0 must be [{d}, n]")
    if tuple(theta.shape) != ((p,) if shared else (p, n)):
        raise ValueError("theta has the wrong shape")
    dev = y0.device
    _expect(dev, ("theta", theta, y0.dtype, theta.shape), ("out", out, y0.dtype, (d, n)),
            ("out_sens", out_sens if _sens else None, y0.dtype, (d, p, n)))
    y1 = torch.empty_like(y0) if out is None else out
    if rec_buffers is not None:
        _check_record_buffers(rec_buffers, n, d, y0.dtype, dev)
    bufs = rec_buffers if rec_buffers is not None else alloc_record(
        n, s_cap, dtype, dev, record_t, d if record_states else 0)
    rec = Record(system, method, dtype, theta, y0, float(t0), float(t1), bufs["h"], bufs.get("t"),
                 bufs["count"], bufs["nrej"], bufs["status"], bufs.get("y"))
    ws = _ws(dev, workspace, stream)
    sysid, mid, did = _lib.SYSTEMS[system], _lib.METHODS[method], _lib.DTYPES[dtype]
    nb = _lib.dao_solve_workspace_size(sysid, mid, did, n)
    buf = ws.get(nb, dev, stream)
    tol = _lib.dao_tol(float(rtol), float(atol), float(dt0), int(max_steps), int(phases))
    crec = rec.c_struct()
    if _sens:
        S = torch.empty((d, p, n), dtype=y0.dtype, device=dev) if out_sens is None else out_sens
        _lib.check(_lib.dao_solve_sens(sysid, mid, did, n, _ptr(theta), _ptr(y0), float(t0),
                                       float(t1), tol, _ptr(y1), crec, _ptr(S), _ptr(buf),
                                       buf.numel(), _stream(stream)))
        return rec, y1, S
    _lib.check(_lib.dao_solve(sysid, mid, did, n, _ptr(theta), _ptr(y0), float(t0), float(t1),
                              tol, _ptr(y1), crec, _ptr(buf), buf.numel(), _stream(stream)))
    return rec, y1


def solve_sens(system: str, method: str, theta: torch.Tensor, y0: torch.Tensor, t0: float,
               t1: float, rtol: float, atol: float, out_sens=None, **kw):
    """solve() that also integrates the forward sensitivities S = dy1/dtheta
    beside the state (steps chosen on the state alone).  Returns
    (Record, y1, S) with S[d][p][n]; Tsit5, per-trajectory theta only."""
    return solve(system, method, theta, y0, t0, t1, rtol, atol, out_sens=out_sens, _sens=True, **kw)


def sens(rec: Record, theta: torch.Tensor | None = None, with_theta: bool = True,
         with_y0: bool = False, s_max: int | None = None, workspace=None, stream=None):
    """Forward sensitivities of y1 through the replay of rec's mesh:
    (S_theta [d][p][n] or None, S_y0 [d][d][n] or None)."""
    rec.check(placed=False)
    th = rec.theta if theta is None else theta
    _expect(rec.count.device, ("theta", th, rec.y0.dtype, rec.theta.shape))
    rec.check()
    n = rec.n
    d, p, _ = _lib.dao_system_dims(_lib.SYSTEMS[rec.system])
    s_max = rec.s_cap if s_max is None else min(int(s_max), rec.s_cap)
    ids = _lib.SYSTEMS[rec.system], _lib.METHODS[rec.method], _lib.DTYPES[rec.dtype]
    dev = rec.count.device
    S_th = torch.empty((d, p, n), dtype=rec.y0.dtype, device=dev) if with_theta else None
    S_y0 = torch.empty((d, d, n), dtype=rec.y0.dtype, device=dev) if with_y0 else None
    nb = _lib.dao_sens_workspace_size(*ids, n, s_max)
    buf = _ws(dev, workspace, stream).get(nb, dev, stream)
    _lib.check(_lib.dao_sens(*ids, n, _ptr(th), _ptr(rec.y0), rec.c_struct(states=False), s_max,
                             _ptr(S_th), _ptr(S_y0), _ptr(buf), buf.numel(), _stream(stream)))
    return S_th, S_y0


def _grad_setup(rec: Record, s_max, workspace, device, stream):
    rec.check()
    n = rec.n
    s_max = rec.s_cap if s_max is None else min(int(s_max), rec.s_cap)
    ids = _lib.SYSTEMS[rec.system], _lib.METHODS[rec.method], _lib.DTYPES[rec.dtype]
    nb = _lib.dao_grad_workspace_size(*ids, n, s_max)
    buf = _ws(device, workspace, stream).get(nb, device, stream)
    return ids, n, s_max, buf


def _check_grad_arrays(rec: Record, th, dLdy1, out_theta, out_y0):
    """theta and the outputs like the solve's theta and y0; dLdy1 [d][n]."""
    rec.check(placed=False)
    td, shape = rec.y0.dtype, tuple(rec.y0.shape)
    _expect(rec.count.device, ("theta", th, td, rec.theta.shape), ("dLdy1", dLdy1, td, shape),
            ("out_theta", out_theta, td, rec.theta.shape), ("out_y0", out_y0, td, shape))


def grad_order(rec: Record, s_max: int | None = None, workspace=None, stream=None) -> int:
    """Sort rec's trajectories by step count into the workspace, for later
    grad(..., ordered=True) calls on the same record and workspace.  Returns
    the s_max it used (pass the same value to those calls)."""
    ids, n, s_max, buf = _grad_setup(rec, s_max, workspace, rec.count.device, stream)
    _lib.check(_lib.dao_grad_order(*ids, n, rec.c_struct(), s_max, _ptr(buf), buf.numel(),
                                   _stream(stream)))
    return s_max


def grad(rec: Record, dLdy1: torch.Tensor, theta: torch.Tensor | None = None, s_max: int | None = None,
         out_theta=None, out_y0=None, workspace=None, stream=None, ordered: bool = False):
    """dL/dtheta and dL/dy0 by the discrete adjoint on rec's mesh.

    theta:   parameters to differentiate at (default: the solve's theta).  At a
             theta other than the solve's, recorded states are not used.
    s_max:   an upper bound on rec.count (default: the record's capacity, which
             needs no read-back but a larger workspace; Record.stats() gives
             the exact one in stream order).
    ordered: the workspace already holds this record's order (grad_order with
             the same workspace and s_max); skips the sort.
    """
    th = rec.theta if theta is None else theta
    dev = rec.count.device
    if dLdy1 is None:
        raise ValueError("dLdy1 is required")
    _check_grad_arrays(rec, th, dLdy1, out_theta, out_y0)
    ids, n, s_max, buf = _grad_setup(rec, s_max, workspace, dev, stream)
    dth = torch.empty_like(th) if out_theta is None else out_theta
    dy0 = torch.empty_like(rec.y0) if out_y0 is None else out_y0
    crec = rec.c_struct(states=theta is None)
    fn = _lib.dao_grad_ordered if ordered else _lib.dao_grad
    _lib.check(fn(*ids, n, _ptr(th), _ptr(rec.y0), crec, s_max, _ptr(dLdy1), _ptr(dth), _ptr(dy0),
                  _ptr(buf), buf.numel(), _stream(stream)))
    return dth, dy0


def states_at(rec: Record, tq: torch.Tensor, theta: torch.Tensor | None = None,
              s_max: int | None = None, out=None, workspace=None, stream=None):
    """States at the requested times tq (device [m], ascending in [t0, t1]) on
    rec's mesh, by a shortened step from the start of the step that holds
    each time: [m][d][n]."""
    rec.check(placed=False)
    th = rec.theta if theta is None else theta
    n, m = rec.n, int(tq.numel())
    d, _, _ = _lib.dao_system_dims(_lib.SYSTEMS[rec.system])
    dev = rec.count.device
    if tq.dim() != 1:
        raise ValueError("tq must be one-dimensional")
    if tq.dtype != rec.y0.dtype:
        raise TypeError("tq must have the record's dtype")
    _expect(dev, ("theta", th, rec.y0.dtype, rec.theta.shape),
            ("out", out, rec.y0.dtype, (m, d, n)))
    _check_dev(tq)
    rec.check()
    s_max = rec.s_cap if s_max is None else min(int(s_max), rec.s_cap)
    ids = _lib.SYSTEMS[rec.system], _lib.METHODS[rec.method], _lib.DTYPES[rec.dtype]
    dev = rec.count.device
    yq = torch.empty((m, d, n), dtype=rec.y0.dtype, device=dev) if out is None else out
    nb = _lib.dao_states_workspace_size(*ids, n, s_max)
    buf = _ws(dev, workspace, stream).get(nb, dev, stream)
    tqc = tq.contiguous()  # kept alive until the call has enqueued its reads
    _lib.check(_lib.dao_states_at(*ids, n, _ptr(th), _ptr(rec.y0), rec.t0, rec.t1,
                                  rec.c_struct(states=False), s_max, m, _ptr(tqc),
                                  _ptr(yq), _ptr(buf), buf.numel(), _stream(stream)))
    if tqc is not tq:
        tqc.record_stream(_tstream(stream))
    return yq


def grad_at(rec: Record, tq: torch.Tensor, dLdyq: torch.Tensor, dLdy1: torch.Tensor | None = None,
            theta: torch.Tensor | None = None, s_max: int | None = None, out_theta=None,
            out_y0=None, workspace=None, stream=None):
    """dL/dtheta and dL/dy0 for L = sum_q <dLdyq[q], y(tq[q])> + <dLdy1, y(t1)>
    on rec's mesh, the states at tq taken as states_at() takes them.
    tq: device [m], ascending in [t0, t1]; dLdyq: [m][d][n]; dLdy1: [d][n] or None."""
    rec.check(placed=False)
    th = rec.theta if theta is None else theta
    if tq.dim() != 1:
        raise ValueError("tq must be one-dimensional")
    if tq.dtype != rec.y0.dtype or dLdyq.dtype != rec.y0.dtype:
        raise TypeError("tq and dLdyq must have the record's dtype")
    n, m = rec.n, int(tq.numel())
    d, _, _ = _lib.dao_system_dims(_lib.SYSTEMS[rec.system])
    if tuple(dLdyq.shape) != (m, d, n):
        raise ValueError(f"dLdyq must have shape {(m, d, n)}")
    _check_grad_arrays(rec, th, dLdy1, out_theta, out_y0)
    _check_dev(tq, dLdyq)
    rec.check()
    s_max = rec.s_cap if s_max is None else min(int(s_max), rec.s_cap)
    ids = _lib.SYSTEMS[rec.system], _lib.METHODS[rec.method], _lib.DTYPES[rec.dtype]
    dev = rec.count.device
    nb = _lib.dao_grad_at_workspace_size(*ids, n, s_max, m)
    buf = _ws(dev, workspace, stream).get(max(nb, 1), dev, stream)
    dth = torch.empty_like(th) if out_theta is None else out_theta
    dy0 = torch.empty_like(rec.y0) if out_y0 is None else out_y0
    # contiguous copies, kept alive (and tied to the launch stream) until the
    # kernels that read them have run
    tqc, cqc = tq.contiguous(), dLdyq.contiguous()
    g1 = None if dLdy1 is None else dLdy1.contiguous()
    _lib.check(_lib.dao_grad_at(*ids, n, _ptr(th), _ptr(rec.y0), rec.t0, rec.t1,
                                rec.c_struct(states=False), s_max, m, _ptr(tqc),
                                _ptr(cqc), _ptr(g1), _ptr(dth), _ptr(dy0),
                                _ptr(buf), buf.numel(), _stream(stream)))
    for c, orig in ((tqc, tq), (cqc, dLdyq), (g1, dLdy1)):
        if c is not None and c is not orig:
            c.record_stream(_tstream(stream))
    return dth, dy0


def cotangent(y1: torch.Tensor, target: torch.Tensor, scale: float = 1.0, d_used: int | None = None,
              out=None, stream=None):
    """dL/dy1 = scale * (y1 - target) on the first d_used components, 0 elsewhere."""
    _check_dev(y1)
    if y1.dim() != 2:
        raise ValueError("y1 must be [d, n]")
    d, n = y1.shape
    d_used = d if d_used is None else int(d_used)
    if not 0 <= d_used <= d:
        raise ValueError(f"d_used must lie in [0, {d}]")
    _expect(y1.device, ("target", target, y1.dtype, (d, n)), ("out", out, y1.dtype, (d, n)))
    o = torch.empty_like(y1) if out is None else out
    _lib.check(_lib.dao_sqerr_cotangent(_lib.DTYPES[_dtype_name(y1)], n, d, d_used, _ptr(y1),
                                        _ptr(target), float(scale), _ptr(o), _stream(stream)))
    return o
