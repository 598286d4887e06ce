"""GPU parity: the HIP kernels (through the C ABI) against the CPU oracle on
identical seeded inputs.

Bars (per trajectory, relative 2-norm, R14 reading):
* forward: accepted-step counts equal, final states within 1e-9 (fp64);
* gradient: with both sides on the oracle's recorded mesh, dL/dtheta and
  dL/dy0 within 1e-9 (fp64).  Robertson rate gradients are compared as
  log-sensitivities theta * dL/dtheta (the rates span 0.04 ... 3e7).
"""
import numpy as np
import pytest
import torch

import dao_inputs as di
import oracle
from mesh_certificate import certify

pytestmark = pytest.mark.gpu

TOL = 1e-9


@pytest.fixture(scope="module")
def dao():
    import differentiable_adaptive_ode_amd as m

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return m


DEV = "cuda:0"


def rel_err(a, b, axis=0):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = np.maximum(np.linalg.norm(b, axis=axis), 1e-300)
    return np.linalg.norm(a - b, axis=axis) / den


def gpu_solve(dao, w, s_cap, **kw):
    th = torch.tensor(w.theta, device=DEV)
    y0 = torch.tensor(w.y0, device=DEV)
    rec, y1 = dao.solve(w.system, w.method, th, y0, w.t0, w.t1, w.rtol, w.atol, s_cap=s_cap, **kw)
    torch.cuda.synchronize()
    return rec, y1


def oracle_solve(w, s_cap, **kw):
    return oracle.solve(w.system, w.method, w.theta, w.y0, w.t0, w.t1, w.rtol, w.atol,
                        s_cap=s_cap, dtype=w.dtype, nthreads=8, **kw)


def import_mesh(dao, w, ref, s_cap):
    """A device record holding the oracle's mesh (what the gradient replays)."""
    from differentiable_adaptive_ode_amd.api import Record

    n = w.n
    h = torch.zeros((n, s_cap), dtype=torch.float64, device=DEV)
    h[:, :ref["h"].shape[1]] = torch.tensor(ref["h"], device=DEV)
    return Record(w.system, w.method, w.dtype, torch.tensor(w.theta, device=DEV),
                  torch.tensor(w.y0, device=DEV), w.t0, w.t1, h, None,
                  torch.tensor(ref["count"], device=DEV), torch.tensor(ref["nrej"], device=DEV),
                  torch.tensor(ref["status"], device=DEV))


CASES = [("decay", 300, 256), ("lotka_volterra", 300, 256), ("lorenz63", 300, 1024),
         ("loghalo", 200, 4096), ("robertson", 200, 2048), ("hires", 200, 4096),
         ("lorenz63_spread", 300, 2048),
         ("decay_vern7", 300, 256), ("lotka_volterra_vern7", 300, 256),
         ("lorenz63_vern7", 300, 1024), ("loghalo_vern7", 200, 4096),
         ("decay_rodas5p", 300, 256), ("robertson_rodas5p", 200, 1024),
         ("lotka_volterra_rodas5p", 200, 256), ("hires_rodas5p", 130, 2048)]
# systems whose rate constants span orders of magnitude: their gradients are
# compared as log-sensitivities theta * dL/dtheta
LOG_RATES = ("robertson", "hires", "robertson_rodas5p", "hires_rodas5p")


@pytest.mark.parametrize("name,n,s_cap", CASES)
def test_forward_parity(dao, name, n, s_cap):
    w = di.make(name, n)
    print(f"[forward parity] {name} n={n}", flush=True)
    ref = oracle_solve(w, s_cap)
    rec, y1 = gpu_solve(dao, w, s_cap)
    cnt = rec.count.cpu().numpy()
    assert np.array_equal(rec.status.cpu().numpy(), ref["status"])
    assert np.array_equal(cnt, ref["count"]), np.flatnonzero(cnt != ref["count"])[:10]
    assert np.array_equal(rec.nrej.cpu().numpy(), ref["nrej"])
    err = rel_err(y1.cpu().numpy(), ref["y1"])
    assert err.max() <= TOL, err.max()
    h = rec.h.cpu().numpy()
    t = rec.t.cpu().numpy()
    mask = np.arange(s_cap)[None, :] < cnt[:, None]
    assert np.array_equal(h[mask], ref["h"][mask])  # same arithmetic, same mesh bits
    assert np.array_equal(t[mask], ref["t"][mask])


@pytest.mark.parametrize("name,n,s_cap", CASES)
def test_gradient_parity_on_oracle_mesh(dao, name, n, s_cap):
    w = di.make(name, n)
    print(f"[gradient parity] {name} n={n}", flush=True)
    ref = oracle_solve(w, s_cap)
    lam = di.cotangent(w, ref["y1"])
    dth_o, dy0_o, _ = oracle.grad(w.system, w.method, w.theta, w.y0, ref["count"], ref["h"], lam,
                                  nthreads=8)
    rec = import_mesh(dao, w, ref, s_cap)
    dth, dy0 = dao.grad(rec, torch.tensor(lam, device=DEV))
    torch.cuda.synchronize()
    dth = dth.cpu().numpy()
    if name in LOG_RATES:
        e = rel_err(dth * w.theta, dth_o * w.theta)
    else:
        e = rel_err(dth, dth_o)
    assert e.max() <= TOL, e.max()
    e0 = rel_err(dy0.cpu().numpy(), dy0_o)
    assert e0.max() <= TOL, e0.max()


@pytest.mark.parametrize("name,n,s_cap", CASES[:3])
def test_gradient_on_own_mesh_at_moved_theta(dao, name, n, s_cap):
    # Reusing a record while theta moves (Sec. 3.1): the derivative is taken at
    # the new theta on the old mesh.
    w = di.make(name, n)
    rec, y1 = gpu_solve(dao, w, s_cap)
    ref = oracle_solve(w, s_cap)
    th2 = w.theta * 1.001
    lam = np.random.default_rng(2).normal(size=w.y0.shape)
    dth_o, dy0_o, _ = oracle.grad(w.system, w.method, th2, w.y0, ref["count"], ref["h"], lam)
    dth, dy0 = dao.grad(rec, torch.tensor(lam, device=DEV), theta=torch.tensor(th2, device=DEV))
    torch.cuda.synchronize()
    assert rel_err(dth.cpu().numpy(), dth_o).max() <= TOL
    assert rel_err(dy0.cpu().numpy(), dy0_o).max() <= TOL


def test_lorenz_full_size_sampled(dao):
    # The benchmark's ensemble (65,536 Lorenz trajectories) in the benchmark's
    # launch configuration; a seeded sample is checked against the oracle.
    w = di.make("lorenz63")
    print(f"[full size] lorenz63 n={w.n}", flush=True)
    s_cap = 1024
    rec, y1 = gpu_solve(dao, w, s_cap)
    lam_all = torch.tensor(di.cotangent(w, y1.cpu().numpy()), device=DEV)
    dth, dy0 = dao.grad(rec, lam_all)
    torch.cuda.synchronize()
    cnt = rec.count.cpu().numpy()
    rng = np.random.default_rng(0)
    idx = np.unique(np.concatenate([rng.choice(w.n, 96, replace=False), [0, w.n - 1],
                                    [np.argmax(cnt), np.argmin(cnt)]]))
    ws = di.subset(w, idx)
    ref = oracle_solve(ws, s_cap)
    assert np.array_equal(cnt[idx], ref["count"])
    assert rel_err(y1.cpu().numpy()[:, idx], ref["y1"]).max() <= TOL
    lam = lam_all.cpu().numpy()[:, idx]
    dth_o, dy0_o, _ = oracle.grad(ws.system, ws.method, ws.theta, ws.y0, ref["count"], ref["h"],
                                  lam, nthreads=8)
    assert rel_err(dth.cpu().numpy()[:, idx], dth_o).max() <= TOL
    assert rel_err(dy0.cpu().numpy()[:, idx], dy0_o).max() <= TOL
    assert np.all(rec.status.cpu().numpy() == 0)


# ------------------------------------------------------------------ edge cases
def test_empty_ensemble(dao):
    th = torch.empty((3, 0), dtype=torch.float64, device=DEV)
    y0 = torch.empty((3, 0), dtype=torch.float64, device=DEV)
    rec, y1 = dao.solve("lorenz63", "tsit5", th, y0, 0.0, 1.0, 1e-6, 1e-8, s_cap=8)
    dth, dy0 = dao.grad(rec, torch.empty_like(y0), s_max=0)
    torch.cuda.synchronize()
    assert y1.shape == (3, 0) and dth.shape == (3, 0)


def test_single_trajectory_and_zero_span(dao):
    w = di.make("lorenz63", 1)
    rec, y1 = gpu_solve(dao, w, 1024)
    ref = oracle_solve(w, 1024)
    assert rec.count.item() == ref["count"][0]
    w0 = di.make("lorenz63", 70)
    w0.t1 = w0.t0
    rec, y1 = gpu_solve(dao, w0, 8)
    assert np.all(rec.count.cpu().numpy() == 0)
    assert np.array_equal(y1.cpu().numpy(), w0.y0)
    lam = np.random.default_rng(1).normal(size=w0.y0.shape)
    dth, dy0 = dao.grad(rec, torch.tensor(lam, device=DEV))
    torch.cuda.synchronize()
    assert np.array_equal(dy0.cpu().numpy(), lam) and np.all(dth.cpu().numpy() == 0)


def test_failure_statuses(dao):
    w = di.make("lorenz63", 130)
    rec, y1 = gpu_solve(dao, w, 1024, max_steps=10)
    assert np.all(rec.status.cpu().numpy() == 1) and torch.isnan(y1).all()
    rec, y1 = gpu_solve(dao, w, 5)
    ref = oracle_solve(w, 5)
    assert np.array_equal(rec.status.cpu().numpy(), ref["status"])
    assert np.all(rec.count.cpu().numpy() == 5)
    th = w.theta.copy()
    th[1, 7] = np.nan
    w2 = di.Workload(**{**w.__dict__, "theta": th})
    rec, y1 = gpu_solve(dao, w2, 1024)
    st = rec.status.cpu().numpy()
    assert st[7] == 2 and np.all(np.delete(st, 7) == 0)
    # gradient of a failed trajectory is NaN; the rest are unaffected
    lam = torch.ones_like(y1)
    dth, dy0 = dao.grad(rec, lam)
    torch.cuda.synchronize()
    assert torch.isnan(dth[:, 7]).all() and torch.isfinite(dth[:, :7]).all()


def test_s_max_bound_gives_nan_not_overrun(dao):
    w = di.make("lorenz63", 100)
    rec, y1 = gpu_solve(dao, w, 1024)
    cnt = rec.count.cpu().numpy()
    s_max = int(np.median(cnt))
    dth, dy0 = dao.grad(rec, torch.ones_like(y1), s_max=s_max)
    torch.cuda.synchronize()
    bad = cnt > s_max
    assert torch.isnan(dy0[:, torch.tensor(bad, device=DEV)]).all()
    assert torch.isfinite(dy0[:, torch.tensor(~bad, device=DEV)]).all()


def test_invalid_arguments_enqueue_nothing(dao):
    from differentiable_adaptive_ode_amd import DaoError

    w = di.make("lorenz63", 10)
    th = torch.tensor(w.theta, device=DEV)
    y0 = torch.tensor(w.y0, device=DEV)
    with pytest.raises(DaoError):
        dao.solve("lorenz63", "tsit5", th, y0, 1.0, 0.0, 1e-6, 1e-8)
    with pytest.raises(DaoError):
        dao.solve("lorenz63", "tsit5", th, y0, 0.0, 1.0, -1.0, 1e-8)
    with pytest.raises(DaoError):
        dao.solve("loghalo", "rosenbrock23", torch.zeros((3, 10), dtype=torch.float64, device=DEV),
                  torch.zeros((6, 10), dtype=torch.float64, device=DEV), 0.0, 1.0, 1e-6, 1e-8)


# ------------------------------------------------------- neural right-hand side
# Shared 4-64-64-4 tanh MLP weights, fp32, matrix-core kernels.  Bars (fp32):
# final states within 1e-4 of the fp64 oracle; on the oracle's mesh the
# shared-weight gradient (as one vector) and dL/dy0 (per trajectory) within
# 1e-3.  On this workload the binary32 error estimate is at the rounding level
# (the fp64 estimate of the same steps is ~1e-10 of the tolerance), so the
# controller factor, and with it the accepted-step count, is set by rounding
# noise: the fp32 and fp64 oracles themselves disagree on most trajectories.
# The mesh is therefore checked by what rounding cannot move: the first step
# equals the binary32 oracle's bit for bit, counts agree within one, and the
# recorded mesh, replayed by the fp64 oracle, reproduces the final state.
TOL32_Y, TOL32_G = 1e-4, 1e-3


def mlp_case(n):
    w = di.make("mlp", n)
    return w


@pytest.mark.parametrize("n", [200, 16 * 7 + 5])
def test_mlp_forward_parity(dao, n):
    w = mlp_case(n)
    print(f"[forward parity] mlp n={n}", flush=True)
    th64, y064 = w.theta.astype(np.float64), w.y0.astype(np.float64)
    ref64 = oracle.solve(w.system, w.method, th64, y064, w.t0, w.t1, w.rtol, w.atol, s_cap=256,
                         dtype="f64", nthreads=8)
    ref32 = oracle.solve(w.system, w.method, w.theta, w.y0, w.t0, w.t1, w.rtol, w.atol, s_cap=256,
                         dtype="f32", nthreads=8)
    rec, y1 = gpu_solve(dao, w, 256)
    st = rec.status.cpu().numpy()
    assert np.all(st == 0)
    y1 = y1.cpu().numpy()
    e = rel_err(y1, ref64["y1"])
    assert e.max() <= TOL32_Y, e.max()
    cnt = rec.count.cpu().numpy()
    h = rec.h.cpu().numpy()
    assert np.array_equal(h[:, 0], ref32["h"][:, 0])  # starting step, bit for bit
    assert np.all(np.abs(cnt - ref32["count"]) <= 1)
    # wherever the mesh parts from the binary32 oracle's, the oracle's own
    # decision there is within rounding of a boundary (borderline certificate)
    _certify_all(w, w.theta, w.y0, cnt, h, ref32, 10, 256)
    mask = np.arange(256)[None, :] < cnt[:, None]
    assert np.all(h[mask] > 0)
    h64 = np.zeros(h.shape)
    h64[mask] = h[mask]  # rows past a count hold unspecified values
    assert np.allclose(h64.sum(axis=1), w.t1 - w.t0, rtol=1e-6)
    # the recorded mesh is the one integrated: its fp64 replay gives y1
    y_rep = oracle.replay(w.system, w.method, th64, y064, cnt, h64)
    assert rel_err(y1, y_rep).max() <= TOL32_Y


def _certify_all(w, theta, y0, cnt, h, ref32, q, s_cap):
    """Every trajectory whose accepted mesh differs from the binary32 oracle's
    carries a borderline certificate (tests/mesh_certificate.py)."""
    shared = w.system == "mlp"
    failures = []
    for k in range(w.n):
        hk = h[k, :cnt[k]]
        if np.array_equal(hk, ref32["h"][k, :ref32["count"][k]]):
            continue
        th = theta if shared else theta[:, k]
        tr = oracle.trace(w.system, w.method, th, y0[:, k], w.t0, w.t1, w.rtol, w.atol,
                          s_cap=s_cap, dtype="f32")
        ok, info = certify(tr, hk, q)
        if not ok:
            failures.append((k, info))
    assert not failures, failures[:3]


@pytest.mark.parametrize("n", [200, 16 * 7 + 5])
def test_mlp_gradient_parity_on_oracle_mesh(dao, n):
    from differentiable_adaptive_ode_amd.api import Record

    w = mlp_case(n)
    print(f"[gradient parity] mlp n={n}", flush=True)
    th64, y064 = w.theta.astype(np.float64), w.y0.astype(np.float64)
    ref = oracle.solve(w.system, w.method, th64, y064, w.t0, w.t1, w.rtol, w.atol, s_cap=256,
                       dtype="f64", nthreads=8)
    lam = di.cotangent(w, ref["y1"])
    dth_o, dy0_o, _ = oracle.grad(w.system, w.method, th64, y064, ref["count"], ref["h"], lam,
                                  nthreads=8)
    rec = Record(w.system, w.method, w.dtype, torch.tensor(w.theta, device=DEV),
                 torch.tensor(w.y0, device=DEV), w.t0, w.t1,
                 torch.tensor(ref["h"].astype(np.float32), device=DEV), None,
                 torch.tensor(ref["count"], device=DEV), torch.tensor(ref["nrej"], device=DEV),
                 torch.tensor(ref["status"], device=DEV))
    dth, dy0 = dao.grad(rec, torch.tensor(lam.astype(np.float32), device=DEV))
    torch.cuda.synchronize()
    dth = dth.cpu().numpy().astype(np.float64)
    eg = np.linalg.norm(dth - dth_o) / np.linalg.norm(dth_o)
    assert eg <= TOL32_G, eg
    # every block of the packed weights, on its own
    for lo, hi in [(0, 256), (256, 320), (320, 4416), (4416, 4480), (4480, 4736), (4736, 4740)]:
        eb = np.linalg.norm(dth[lo:hi] - dth_o[lo:hi]) / np.linalg.norm(dth_o[lo:hi])
        assert eb <= TOL32_G, (lo, hi, eb)
    e0 = rel_err(dy0.cpu().numpy(), dy0_o)
    assert e0.max() <= TOL32_G, e0.max()


def test_mlp_full_size_sampled_and_additive(dao):
    # The benchmark-size ensemble (16,384 trajectories): sampled final states
    # and dL/dy0 against the oracle, and the shared-weight gradient is additive
    # over a split of the ensemble (each part on its own record).
    w = mlp_case(16384)
    print(f"[full size] mlp n={w.n}", flush=True)
    rec, y1 = gpu_solve(dao, w, 256)
    assert np.all(rec.status.cpu().numpy() == 0)
    y1n = y1.cpu().numpy()
    lam = torch.tensor(di.cotangent(w, y1n).astype(np.float32), device=DEV)
    dth, dy0 = dao.grad(rec, lam)
    torch.cuda.synchronize()
    rng = np.random.default_rng(0)
    idx = np.unique(np.concatenate([rng.choice(w.n, 48, replace=False), [0, w.n - 1]]))
    ws = di.subset(w, idx)
    ref = oracle.solve(ws.system, ws.method, ws.theta.astype(np.float64), ws.y0.astype(np.float64),
                       ws.t0, ws.t1, ws.rtol, ws.atol, s_cap=256, dtype="f64", nthreads=8)
    assert rel_err(y1n[:, idx], ref["y1"]).max() <= TOL32_Y
    # dL/dy0 of the sample against the oracle's tape gradient on the GPU's own
    # mesh (rows past a count are unspecified: masked)
    cnt = rec.count.cpu().numpy()[idx]
    h = rec.h.cpu().numpy()[idx]
    h = np.where(np.arange(h.shape[1])[None, :] < cnt[:, None], h, 0.0).astype(np.float64)
    _, dy0_o, _ = oracle.grad(ws.system, ws.method, ws.theta.astype(np.float64),
                              ws.y0.astype(np.float64), cnt, h,
                              lam.cpu().numpy()[:, idx].astype(np.float64), nthreads=8)
    assert rel_err(dy0.cpu().numpy()[:, idx], dy0_o).max() <= TOL32_G
    parts = []
    for sl in (slice(0, 6000), slice(6000, w.n)):
        sub = di.subset(w, np.arange(w.n)[sl])
        r2, _ = gpu_solve(dao, sub, 256)
        d2, _ = dao.grad(r2, lam[:, sl].contiguous())
        parts.append(d2)
    torch.cuda.synchronize()
    tot = (parts[0] + parts[1]).cpu().numpy()
    full = dth.cpu().numpy()
    assert np.linalg.norm(tot - full) / np.linalg.norm(full) <= 1e-4


def test_mlp_strided_chunks_cover_every_group(dao):
    # 40,000 trajectories are 2,500 groups in 2,048 partial-sum rows: rows
    # 0..451 hold two groups each (g and g + 2048).  Every trajectory's
    # dL/dy0 is written and equals, bit for bit, its value from the gradient
    # of a part of the ensemble (the records are the same per trajectory),
    # and the shared-weight gradient is the sum of the parts' (a group left
    # out or taken twice moves it by about 1/2500).
    w = mlp_case(40000)
    print(f"[strided chunks] mlp n={w.n}", flush=True)
    rec, y1 = gpu_solve(dao, w, 64)
    assert np.all(rec.status.cpu().numpy() == 0)
    lam = torch.tensor(di.cotangent(w, y1.cpu().numpy()).astype(np.float32), device=DEV)
    dy0 = torch.full_like(rec.y0, float("nan"))
    dth, _ = dao.grad(rec, lam, out_y0=dy0)
    parts_th, parts_y0 = [], []
    for sl in (slice(0, 17000), slice(17000, w.n)):
        sub = di.subset(w, np.arange(w.n)[sl])
        r2, _ = gpu_solve(dao, sub, 64)
        assert torch.equal(r2.count, rec.count[sl])
        d2, e2 = dao.grad(r2, lam[:, sl].contiguous())
        parts_th.append(d2)
        parts_y0.append(e2)
    torch.cuda.synchronize()
    assert torch.isfinite(dy0).all()
    assert torch.equal(torch.cat(parts_y0, dim=1), dy0)
    tot = (parts_th[0].double() + parts_th[1].double()).cpu().numpy()
    full = dth.double().cpu().numpy()
    e = np.linalg.norm(tot - full) / np.linalg.norm(full)
    print(f"  additivity {e:.2e}", flush=True)
    assert e <= 2e-5, e


def test_mlp_full_size_on_oracle_mesh(dao):
    # All 16,384 trajectories of the benchmark ensemble on the oracle's mesh
    # (its binary64 solve, the step sizes rounded to binary32 and handed to
    # both sides), through the benchmark's launch path: the sort, then the
    # gradient kernel over 1,024 wavefronts and the two-pass reduction of the
    # partial weight gradients (one row per group of 16 trajectories at this
    # size, summed in 16 runs of 64 rows).  Every packed block of the shared
    # weight gradient, and dL/dy0 per trajectory, within the binary32 bar of
    # the oracle's tape gradient.  Then the GPU's own full-size mesh against
    # the binary32 oracle: every diverging trajectory carries a borderline
    # certificate.
    from differentiable_adaptive_ode_amd.api import Record

    w = mlp_case(16384)
    print(f"[full size, oracle mesh] mlp n={w.n}", flush=True)
    th64, y064 = w.theta.astype(np.float64), w.y0.astype(np.float64)
    ref = oracle.solve(w.system, w.method, th64, y064, w.t0, w.t1, w.rtol, w.atol, s_cap=64,
                       dtype="f64", nthreads=16)
    assert np.all(ref["status"] == 0)
    h32 = ref["h"].astype(np.float32)
    lam32 = di.cotangent(w, ref["y1"]).astype(np.float32)
    dth_o, dy0_o, _ = oracle.grad(w.system, w.method, th64, y064, ref["count"],
                                  h32.astype(np.float64), lam32.astype(np.float64), nthreads=16)
    rec = Record(w.system, w.method, w.dtype, torch.tensor(w.theta, device=DEV),
                 torch.tensor(w.y0, device=DEV), w.t0, w.t1, torch.tensor(h32, device=DEV), None,
                 torch.tensor(ref["count"], device=DEV), torch.tensor(ref["nrej"], device=DEV),
                 torch.tensor(ref["status"], device=DEV))
    s_max = rec.stats_host()["s_max"]
    ws = dao.Workspace()
    dao.grad_order(rec, s_max=s_max, workspace=ws)
    dth, dy0 = dao.grad(rec, torch.tensor(lam32, device=DEV), s_max=s_max, workspace=ws,
                        ordered=True)
    torch.cuda.synchronize()
    dth = dth.cpu().numpy().astype(np.float64)
    for lo, hi in [(0, 256), (256, 320), (320, 4416), (4416, 4480), (4480, 4736), (4736, 4740)]:
        eb = np.linalg.norm(dth[lo:hi] - dth_o[lo:hi]) / np.linalg.norm(dth_o[lo:hi])
        assert eb <= TOL32_G, (lo, hi, eb)
    e0 = rel_err(dy0.cpu().numpy(), dy0_o)
    assert e0.max() <= TOL32_G, e0.max()
    # the GPU's own mesh of the full ensemble against the binary32 oracle
    rec2, _ = gpu_solve(dao, w, 64)
    cnt = rec2.count.cpu().numpy()
    ref32 = oracle.solve(w.system, w.method, w.theta, w.y0, w.t0, w.t1, w.rtol, w.atol, s_cap=64,
                         dtype="f32", nthreads=16)
    assert np.all(np.abs(cnt - ref32["count"]) <= 1)
    _certify_all(w, w.theta, w.y0, cnt, rec2.h.cpu().numpy(), ref32, 10, 64)


def test_mlp_empty_and_single(dao):
    th = torch.tensor(di.make("mlp", 1).theta, device=DEV)
    y0 = torch.empty((4, 0), dtype=torch.float32, device=DEV)
    rec, y1 = dao.solve("mlp", "tsit5", th, y0, 0.0, 1.0, 1e-5, 1e-7, s_cap=8)
    dth, dy0 = dao.grad(rec, torch.empty_like(y0), s_max=0)
    torch.cuda.synchronize()
    assert y1.shape == (4, 0)
    w = mlp_case(1)
    rec, y1 = gpu_solve(dao, w, 256)
    ref = oracle.solve(w.system, w.method, w.theta.astype(np.float64), w.y0.astype(np.float64),
                       w.t0, w.t1, w.rtol, w.atol, s_cap=256, dtype="f64")
    assert rel_err(y1.cpu().numpy(), ref["y1"]).max() <= TOL32_Y


@pytest.mark.parametrize("name,s_cap,record_t", [("robertson", 1024, True), ("loghalo", 8192, False),
                                                 ("hires", 4096, True),
                                                 ("lorenz63_spread", 2048, False)])
def test_full_size_sampled(dao, name, s_cap, record_t):
    # The benchmark ensembles at full size (262,144 stiff Robertson
    # trajectories; 1,048,576 orbits; 131,072 HIRES trajectories; the 65,536
    # Lorenz trajectories with the difficulty spread) in the
    # benchmark's launch configuration;
    # a seeded sample, plus the longest and shortest records, against the
    # oracle: equal accepted-step counts, final states and gradients within
    # the fp64 bar.
    w = di.make(name)
    print(f"[full size] {name} n={w.n}", flush=True)
    rec, y1 = gpu_solve(dao, w, s_cap, record_t=record_t)
    st = rec.status.cpu().numpy()
    assert np.all(st == 0), np.bincount(st)
    cnt = rec.count.cpu().numpy()
    y1n = y1.cpu().numpy()
    lam_all = torch.tensor(di.cotangent(w, y1n), device=DEV)
    dth, dy0 = dao.grad(rec, lam_all, s_max=int(cnt.max()))
    torch.cuda.synchronize()
    rng = np.random.default_rng(1)
    idx = np.unique(np.concatenate([rng.choice(w.n, 96, replace=False), [0, w.n - 1],
                                    [np.argmax(cnt), np.argmin(cnt)]]))
    ws = di.subset(w, idx)
    ref = oracle_solve(ws, s_cap)
    assert np.array_equal(cnt[idx], ref["count"])
    assert rel_err(y1n[:, idx], ref["y1"]).max() <= TOL
    lam = lam_all.cpu().numpy()[:, idx]
    dth_o, dy0_o, _ = oracle.grad(ws.system, ws.method, ws.theta, ws.y0, ref["count"], ref["h"],
                                  lam, nthreads=8)
    g = dth.cpu().numpy()[:, idx]
    if name in LOG_RATES:
        e = rel_err(g * ws.theta, dth_o * ws.theta)
    else:
        e = rel_err(g, dth_o)
    assert e.max() <= TOL, e.max()
    assert rel_err(dy0.cpu().numpy()[:, idx], dy0_o).max() <= TOL


@pytest.mark.parametrize("name,n,s_cap", [("lotka_volterra", 300, 256), ("lorenz63", 300, 1024),
                                          ("robertson", 200, 2048), ("loghalo", 130, 4096)])
def test_recorded_states(dao, name, n, s_cap):
    # The solve can keep the state at the start of every accepted step; the
    # gradient then skips the replay's forward pass.  Those states are the
    # replay's states bit for bit, so both gradients agree exactly; at a moved
    # theta the states are not used.
    w = di.make(name, n)
    print(f"[recorded states] {name} n={n}", flush=True)
    rec0, y1a = gpu_solve(dao, w, s_cap)
    rec1, y1b = gpu_solve(dao, w, s_cap, record_states=True)
    assert torch.equal(rec0.count, rec1.count) and torch.equal(y1a, y1b)
    cnt = rec1.count.cpu().numpy()
    ys = rec1.y.cpu().numpy()
    assert np.array_equal(ys[:, 0, :], w.y0.T)
    lam = torch.tensor(di.cotangent(w, y1a.cpu().numpy()), device=DEV)
    ga = dao.grad(rec0, lam)
    gb = dao.grad(rec1, lam)
    torch.cuda.synchronize()
    assert torch.equal(ga[0], gb[0]) and torch.equal(ga[1], gb[1])
    th2 = w.theta * 1.002
    gm = dao.grad(rec1, lam, theta=torch.tensor(th2, device=DEV))
    torch.cuda.synchronize()
    ref = oracle_solve(w, s_cap)
    dth_o, dy0_o, _ = oracle.grad(w.system, w.method, th2, w.y0, ref["count"], ref["h"],
                                  lam.cpu().numpy(), nthreads=8)
    if name == "robertson":
        e = rel_err(gm[0].cpu().numpy() * th2, dth_o * th2)
    else:
        e = rel_err(gm[0].cpu().numpy(), dth_o)
    assert e.max() <= TOL
    assert rel_err(gm[1].cpu().numpy(), dy0_o).max() <= TOL


@pytest.mark.parametrize("name,n,s_cap", [("lorenz63", 300, 1024), ("robertson", 200, 2048)])
def test_one_order_many_gradients(dao, name, n, s_cap):
    # dao_grad_order sorts a record's trajectories once; dao_grad_ordered then
    # serves several gradients at moved theta (Sec. 3.1 reuses one record
    # while theta moves).  Each equals dao_grad bit for bit and the oracle.
    from differentiable_adaptive_ode_amd import api

    w = di.make(name, n)
    print(f"[order once] {name} n={n}", flush=True)
    rec, y1 = gpu_solve(dao, w, s_cap)
    ref = oracle_solve(w, s_cap)
    ws = api.Workspace()
    s_max = dao.grad_order(rec, workspace=ws)
    lam = torch.tensor(np.random.default_rng(5).normal(size=w.y0.shape), device=DEV)
    for f in (1.0, 1.001, 0.999):
        th = torch.tensor(w.theta * f, device=DEV)
        go = dao.grad(rec, lam, theta=th, s_max=s_max, workspace=ws, ordered=True)
        gd = dao.grad(rec, lam, theta=th, s_max=s_max)  # its own workspace, sorted again
        torch.cuda.synchronize()
        assert torch.equal(go[0], gd[0]) and torch.equal(go[1], gd[1])
        dth_o, dy0_o, _ = oracle.grad(w.system, w.method, w.theta * f, w.y0, ref["count"],
                                      ref["h"], lam.cpu().numpy(), nthreads=8)
        scale = w.theta * f if name == "robertson" else 1.0
        assert rel_err(go[0].cpu().numpy() * scale, dth_o * scale).max() <= TOL
        assert rel_err(go[1].cpu().numpy(), dy0_o).max() <= TOL


@pytest.mark.parametrize("name,n,s_cap", [("lorenz63", 1000, 1024), ("mlp", 500, 64),
                                          ("mlp", 40000, 64)])
def test_gradient_with_the_minimum_workspace(dao, name, n, s_cap):
    # A workspace of dao_grad_workspace_min bytes holds the scratch of one
    # workgroup only: the gradient then runs its groups one workgroup at a
    # time.  The results are the same bit for bit, the neural field's
    # shared-weight sum included: its partial sums are taken per chunk of
    # groups, a split fixed by n (at n = 40000, 2500 groups in 2048 chunks,
    # some chunks hold two groups), not per wavefront.
    from differentiable_adaptive_ode_amd import _lib

    w = di.make(name, n)
    print(f"[min workspace] {name} n={n}", flush=True)
    th = torch.tensor(w.theta, device=DEV)
    y0 = torch.tensor(w.y0, device=DEV)
    rec, y1 = dao.solve(w.system, w.method, th, y0, w.t0, w.t1, w.rtol, w.atol, s_cap=s_cap)
    lam = torch.tensor(di.cotangent(w, y1.cpu().numpy()).astype(w.y0.dtype), device=DEV)
    s_max = int(rec.count.max().item())
    g_full = dao.grad(rec, lam, s_max=s_max)
    ids = _lib.SYSTEMS[w.system], _lib.METHODS[w.method], _lib.DTYPES[w.dtype]
    nmin = _lib.dao_grad_workspace_min(*ids, n, s_max)
    assert 0 < nmin < _lib.dao_grad_workspace_size(*ids, n, s_max)
    buf = torch.empty(nmin, dtype=torch.uint8, device=DEV)
    dth = torch.empty_like(g_full[0])
    dy0 = torch.empty_like(g_full[1])
    stream = torch.cuda.current_stream().cuda_stream
    _lib.check(_lib.dao_grad(*ids, n, th.data_ptr(), y0.data_ptr(), rec.c_struct(), s_max,
                             lam.data_ptr(), dth.data_ptr(), dy0.data_ptr(), buf.data_ptr(),
                             nmin, stream))
    torch.cuda.synchronize()
    assert torch.equal(dy0, g_full[1])
    assert torch.isfinite(dth).all()
    assert torch.equal(dth, g_full[0])
    # and the same call again (other wavefronts claim other chunks)
    assert torch.equal(dao.grad(rec, lam, s_max=s_max)[0], g_full[0])
    # one byte less is refused before anything runs
    with pytest.raises(_lib.DaoError, match="workspace"):
        _lib.check(_lib.dao_grad(*ids, n, th.data_ptr(), y0.data_ptr(), rec.c_struct(), s_max,
                                 lam.data_ptr(), dth.data_ptr(), dy0.data_ptr(), buf.data_ptr(),
                                 nmin - 1, stream))


@pytest.mark.parametrize("name,n,s_cap,record_t,states,max_steps",
                         [("decay", 300, 256, True, False, 100000),
                          ("lotka_volterra", 64 * 9 + 13, 256, True, False, 100000),
                          ("lorenz63", 1000, 1024, False, False, 100000),
                          ("lorenz63", 300, 1024, True, True, 100000),
                          ("loghalo", 400, 4096, True, False, 100000),
                          ("robertson", 300, 1024, True, False, 100000),
                          ("lorenz63", 200, 64, True, False, 100000),
                          ("lorenz63", 200, 1024, True, False, 150),
                          ("lorenz63", 200, 1024, True, False, 40)])
def test_two_phase_solve_equals_one_phase(dao, name, n, s_cap, record_t, states, max_steps):
    # Large ensembles are solved in two phases (64 probe attempts per
    # trajectory, then the unfinished ones longest-predicted first);
    # the solve's phases argument forces either.  Every trajectory takes the same
    # attempts: record, counts, statuses and final states equal bit for bit,
    # also when the record fills (s_cap 64), when the attempt cap ends
    # trajectories in phase 2 (150) or in phase 1 (40), and with recorded
    # states.
    w = di.make(name, n)
    print(f"[two-phase solve] {name} n={n} s_cap={s_cap} max_steps={max_steps}", flush=True)
    th = torch.tensor(w.theta, device=DEV)
    y0 = torch.tensor(w.y0, device=DEV)
    out = {}
    for mode in ("1", "2"):
        rec, y1 = dao.solve(w.system, w.method, th, y0, w.t0, w.t1, w.rtol, w.atol, s_cap=s_cap,
                            record_t=record_t, record_states=states, max_steps=max_steps,
                            phases=int(mode))
        torch.cuda.synchronize()
        out[mode] = (rec, y1)
    (r1, y1a), (r2, y1b) = out["1"], out["2"]
    assert torch.equal(r1.count, r2.count) and torch.equal(r1.status, r2.status)
    assert torch.equal(r1.nrej, r2.nrej)
    assert torch.equal(torch.nan_to_num(y1a, nan=7.0), torch.nan_to_num(y1b, nan=7.0))
    cnt = r1.count.cpu().numpy()
    mask = torch.tensor(np.arange(s_cap)[None, :] < cnt[:, None], device=DEV)
    assert torch.equal(r1.h[mask], r2.h[mask])
    if record_t:
        assert torch.equal(r1.t[mask], r2.t[mask])
    if states:
        assert torch.equal(r1.y[mask], r2.y[mask])
    st = r1.status.cpu().numpy()
    if (name, s_cap) == ("lorenz63", 64) or max_steps < 100000:
        assert np.any(st != 0)  # the failure paths are exercised
    else:
        assert np.all(st == 0)


@pytest.mark.parametrize("name,n,s_cap", [("lorenz63", 500, 1024), ("robertson", 300, 1024),
                                          ("loghalo", 300, 4096), ("lotka_volterra", 64 * 5 + 9, 256)])
def test_two_phase_solve_with_sensitivities_equals_one_phase(dao, name, n, s_cap):
    # The solve with forward sensitivities suspends and resumes S with the
    # state: both ways give the same S, record and final states bit for bit.
    w = di.make(name, n)
    print(f"[two-phase sens] {name} n={n}", flush=True)
    th = torch.tensor(w.theta, device=DEV)
    y0 = torch.tensor(w.y0, device=DEV)
    out = {}
    for mode in ("1", "2"):
        out[mode] = dao.solve_sens(w.system, w.method, th, y0, w.t0, w.t1, w.rtol, w.atol,
                                   s_cap=s_cap, phases=int(mode))
        torch.cuda.synchronize()
    (r1, y1a, Sa), (r2, y1b, Sb) = out["1"], out["2"]
    assert torch.equal(r1.count, r2.count) and torch.equal(r1.status, r2.status)
    assert torch.equal(y1a, y1b) and torch.equal(Sa, Sb)
    assert np.all(r1.status.cpu().numpy() == 0)
    cnt = r1.count.cpu().numpy()
    mask = torch.tensor(np.arange(s_cap)[None, :] < cnt[:, None], device=DEV)
    assert torch.equal(r1.h[mask], r2.h[mask]) and torch.equal(r1.t[mask], r2.t[mask])


def test_hires_with_tsit5(dao):
    # The explicit pair on the stiff eight-species field over a short span:
    # the mesh bit for bit, y1 and the gradient on the oracle's mesh (1e-9).
    w = di.make("hires", 130)
    w.method, w.t1 = "tsit5", 5.0
    print(f"[hires tsit5] n={w.n}", flush=True)
    ref = oracle_solve(w, 1024)
    rec, y1 = gpu_solve(dao, w, 1024)
    assert np.array_equal(rec.status.cpu().numpy(), ref["status"])
    assert np.array_equal(rec.count.cpu().numpy(), ref["count"])
    assert rel_err(y1.cpu().numpy(), ref["y1"]).max() <= TOL
    lam = di.cotangent(w, ref["y1"])
    dth_o, dy0_o, _ = oracle.grad(w.system, w.method, w.theta, w.y0, ref["count"], ref["h"], lam,
                                  nthreads=8)
    dth, dy0 = dao.grad(import_mesh(dao, w, ref, 1024), torch.tensor(lam, device=DEV))
    torch.cuda.synchronize()
    assert rel_err(dth.cpu().numpy() * w.theta, dth_o * w.theta).max() <= TOL
    assert rel_err(dy0.cpu().numpy(), dy0_o).max() <= TOL


def test_hires_single_precision(dao):
    # Rosenbrock23 in binary32 on HIRES against the oracle's binary32
    # instantiation (the same arithmetic): accepted-step counts within one,
    # and where they agree y1 within 1e-5; the gradient on the GPU's own mesh
    # within 1e-3 of the binary64 oracle on that mesh.  (y1 itself differs
    # from a binary64 replay of the mesh by up to ~1e-4 after a hundred
    # binary32 stiff steps; that is the precision, not the kernel.)
    w = di.make("hires", 130)
    w.rtol, w.atol = 1e-4, 1e-6
    th = torch.tensor(w.theta, dtype=torch.float32, device=DEV)
    y0 = torch.tensor(w.y0, dtype=torch.float32, device=DEV)
    rec, y1 = dao.solve(w.system, w.method, th, y0, w.t0, w.t1, w.rtol, w.atol, s_cap=1024)
    torch.cuda.synchronize()
    assert np.all(rec.status.cpu().numpy() == 0)
    ref32 = oracle.solve(w.system, w.method, w.theta.astype(np.float32), w.y0.astype(np.float32),
                         w.t0, w.t1, w.rtol, w.atol, s_cap=1024, dtype="f32", nthreads=8)
    cnt = rec.count.cpu().numpy()
    assert np.all(np.abs(cnt - ref32["count"]) <= 1)
    _certify_all(w, w.theta.astype(np.float32), w.y0.astype(np.float32), cnt,
                 rec.h.cpu().numpy(), ref32, 6, 1024)
    h = rec.h.cpu().numpy()  # rows past a count are unspecified: masked before the cast
    h = np.where(np.arange(h.shape[1])[None, :] < cnt[:, None], h, 0.0).astype(np.float64)
    th64 = th.cpu().numpy().astype(np.float64)
    y064 = y0.cpu().numpy().astype(np.float64)
    same = cnt == ref32["count"]
    assert same.mean() > 0.9
    assert rel_err(y1.cpu().numpy()[:, same], ref32["y1"][:, same]).max() <= 1e-5
    yS = oracle.replay(w.system, w.method, th64, y064, cnt, h)
    assert rel_err(y1.cpu().numpy(), yS).max() <= 1e-3
    lam = di.cotangent(w, yS)
    dth_o, dy0_o, _ = oracle.grad(w.system, w.method, th64, y064, cnt, h, lam, nthreads=8)
    dth, dy0 = dao.grad(rec, torch.tensor(lam, dtype=torch.float32, device=DEV))
    torch.cuda.synchronize()
    assert rel_err(dth.cpu().numpy() * th64, dth_o * th64).max() <= 1e-3
    assert rel_err(dy0.cpu().numpy(), dy0_o).max() <= 1e-3
