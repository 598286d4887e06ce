"""GPU tests of the Verner 7(6) pair beyond the shared parity lists: the
gradient at a moved theta on the GPU's own mesh, the full-size Lorenz and
orbit ensembles in the benchmark's launch configuration (sampled against the
oracle), the
two-phase solve of the orbit ensemble equal to one phase bit for bit, and the
refusal of the forward sensitivities it does not provide."""
import numpy as np
import pytest
import torch

import dao_inputs as di
import oracle

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL = 1e-9


@pytest.fixture(scope="module")
def dao():
    import differentiable_adaptive_ode_amd as m

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return m


def rel_err(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return np.linalg.norm(a - b, axis=0) / np.maximum(np.linalg.norm(b, axis=0), 1e-300)


def _solve(dao, w, s_cap, **kw):
    th = torch.tensor(w.theta, device=DEV)
    y0 = torch.tensor(w.y0, device=DEV)
    rec, y1 = dao.solve(w.system, w.method, th, y0, w.t0, w.t1, w.rtol, w.atol, s_cap=s_cap, **kw)
    torch.cuda.synchronize()
    return rec, y1


@pytest.mark.parametrize("name,n,s_cap", [("lorenz63_vern7", 300, 1024),
                                          ("loghalo_vern7", 130, 4096)])
def test_vern7_gradient_at_moved_theta(dao, name, n, s_cap):
    w = di.make(name, n)
    print(f"[vern7 moved theta] {name} n={n}", flush=True)
    rec, y1 = _solve(dao, w, s_cap)
    ref = oracle.solve(w.system, w.method, w.theta, w.y0, w.t0, w.t1, w.rtol, w.atol,
                       s_cap=s_cap, nthreads=8)
    assert np.array_equal(rec.count.cpu().numpy(), ref["count"])
    th2 = w.theta * 1.001
    lam = np.random.default_rng(3).normal(size=w.y0.shape)
    dth_o, dy0_o, _ = oracle.grad(w.system, w.method, th2, w.y0, ref["count"], ref["h"], lam,
                                  nthreads=8)
    dth, dy0 = dao.grad(rec, torch.tensor(lam, device=DEV), theta=torch.tensor(th2, device=DEV))
    torch.cuda.synchronize()
    assert rel_err(dth.cpu().numpy(), dth_o).max() <= TOL
    assert rel_err(dy0.cpu().numpy(), dy0_o).max() <= TOL


@pytest.mark.parametrize("name,s_cap", [("lorenz63_vern7", 1024), ("loghalo_vern7", 8192)])
def test_vern7_full_size_sampled(dao, name, s_cap):
    # the benchmark's ensemble at its own size and record capacity (the
    # orbits' 2^20 trajectories take the two-phase solve)
    w = di.make(name)
    print(f"[vern7 full size] {name} n={w.n}", flush=True)
    rec, y1 = _solve(dao, w, s_cap, record_t=False)
    assert rec.stats_host()["failed"] == 0
    cnt = rec.count.cpu().numpy()
    lam_all = torch.tensor(di.cotangent(w, y1.cpu().numpy()), device=DEV)
    s_max = int(cnt.max())
    dth, dy0 = dao.grad(rec, lam_all, s_max=s_max)
    torch.cuda.synchronize()
    rng = np.random.default_rng(7)
    idx = np.unique(np.concatenate([rng.choice(w.n, 96, replace=False), [0, w.n - 1],
                                    [np.argmax(cnt), np.argmin(cnt)]]))
    ws = di.subset(w, idx)
    ref = oracle.solve(ws.system, ws.method, ws.theta, ws.y0, ws.t0, ws.t1, ws.rtol, ws.atol,
                       s_cap=s_cap, nthreads=8)
    assert np.array_equal(cnt[idx], ref["count"])
    assert rel_err(y1.cpu().numpy()[:, idx], ref["y1"]).max() <= TOL
    h = rec.h.cpu().numpy()[idx]
    mask = np.arange(s_cap)[None, :] < cnt[idx][:, None]
    assert np.array_equal(h[mask], ref["h"][mask])
    dth_o, dy0_o, _ = oracle.grad(ws.system, ws.method, ws.theta, ws.y0, ref["count"], ref["h"],
                                  lam_all.cpu().numpy()[:, idx], nthreads=8)
    assert rel_err(dth.cpu().numpy()[:, idx], dth_o).max() <= TOL
    assert rel_err(dy0.cpu().numpy()[:, idx], dy0_o).max() <= TOL


def test_vern7_two_phase_equals_one_phase(dao):
    w = di.make("loghalo_vern7", 400)
    print("[vern7 two-phase] loghalo n=400", flush=True)
    out = [_solve(dao, w, 4096, phases=p) for p in (1, 2)]
    (r1, y1a), (r2, y1b) = out
    assert torch.equal(r1.count, r2.count) and torch.equal(r1.nrej, r2.nrej)
    assert torch.equal(y1a, y1b)
    cnt = r1.count.cpu().numpy()
    mask = torch.tensor(np.arange(4096)[None, :] < cnt[:, None], device=DEV)
    assert torch.equal(r1.h[mask], r2.h[mask])


def test_vern7_refuses_forward_sensitivities_and_other_dtypes(dao):
    from differentiable_adaptive_ode_amd import DaoError

    w = di.make("lorenz63_vern7", 70)
    th = torch.tensor(w.theta, device=DEV)
    y0 = torch.tensor(w.y0, device=DEV)
    with pytest.raises(DaoError, match="not provided"):
        dao.solve_sens(w.system, "vern7", th, y0, w.t0, w.t1, w.rtol, w.atol, s_cap=1024)
    rec, _ = dao.solve(w.system, "vern7", th, y0, w.t0, w.t1, w.rtol, w.atol, s_cap=1024)
    with pytest.raises(DaoError, match="not provided"):
        dao.sens(rec)
    with pytest.raises(DaoError, match="not provided"):
        dao.solve(w.system, "vern7", th.float(), y0.float(), w.t0, w.t1, w.rtol, w.atol,
                  s_cap=1024)
    wr = di.make("robertson", 8)
    with pytest.raises(DaoError, match="not provided"):
        dao.solve("robertson", "vern7", torch.tensor(wr.theta, device=DEV),
                  torch.tensor(wr.y0, device=DEV), 0.0, 1.0, 1e-6, 1e-10, s_cap=64)
