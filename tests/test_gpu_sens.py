"""GPU parity of the forward sensitivities S = dy(t1)/dtheta, dy(t1)/dy0
(through the C ABI) against the oracle's dual-number forward mode.

* dao_solve_sens (Tsit5 and Rosenbrock23): the record and y1 equal
  dao_solve's bit for bit (the steps are chosen on the state alone, arXiv
  2609.28458 Sec. 2.3); S_theta within 1e-9 of the oracle on that mesh (per
  trajectory, relative 2-norm of the d x p matrix; Robertson as theta * S).
* dao_sens (forward mode through the replay of the record): bit for bit the
  in-solve S_theta; S_y0 and a moved theta against the oracle.
* lam^T S_theta against the library's own reverse-mode gradient.
"""
import numpy as np
import pytest
import torch

import dao_inputs as di
import oracle

pytestmark = pytest.mark.gpu

TOL = 1e-9
DEV = "cuda:0"


@pytest.fixture(scope="module")
def dao():
    import differentiable_adaptive_ode_amd as m

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return m


def rel_err_mat(a, b):
    """Per trajectory ||a - b|| / ||b|| over all but the last axis."""
    a = np.asarray(a, dtype=np.float64).reshape(-1, a.shape[-1])
    b = np.asarray(b, dtype=np.float64).reshape(-1, b.shape[-1])
    return np.linalg.norm(a - b, axis=0) / np.maximum(np.linalg.norm(b, axis=0), 1e-300)


def solve_both(dao, w, s_cap):
    th = torch.tensor(w.theta, device=DEV)
    y0 = torch.tensor(w.y0, device=DEV)
    r0, y1a = dao.solve(w.system, w.method, th, y0, w.t0, w.t1, w.rtol, w.atol, s_cap=s_cap)
    r1, y1b, S = dao.solve_sens(w.system, w.method, th, y0, w.t0, w.t1, w.rtol, w.atol,
                                s_cap=s_cap)
    torch.cuda.synchronize()
    return r0, y1a, r1, y1b, S


CASES = [("decay", 300, 256, None), ("lotka_volterra", 300, 256, None),
         ("lorenz63", 300, 1024, None), ("loghalo", 200, 4096, None),
         ("robertson", 200, 2048, None), ("lotka_volterra", 200, 1024, "rosenbrock23"),
         ("lorenz63", 200, 2048, "rosenbrock23"), ("hires", 130, 4096, None)]


def case(name, n, method):
    w = di.make(name, n)
    if method is not None and method != w.method:
        w.method = method
        if name == "lorenz63":
            w.t1 = 0.5
    return w


@pytest.mark.parametrize("name,n,s_cap,method", CASES)
def test_solve_sens_parity(dao, name, n, s_cap, method):
    w = case(name, n, method)
    print(f"[solve_sens] {name} {w.method} n={n}", flush=True)
    r0, y1a, r1, y1b, S = solve_both(dao, w, s_cap)
    cnt = r1.count.cpu().numpy()
    assert torch.equal(r0.count, r1.count) and torch.equal(r0.nrej, r1.nrej)
    assert torch.equal(r0.status, r1.status) and torch.equal(y1a, y1b)
    mask = torch.arange(s_cap, device=DEV)[None, :] < r1.count[:, None]
    assert torch.equal(r0.h[mask], r1.h[mask])
    h = np.where(mask.cpu().numpy(), r1.h.cpu().numpy(), 0.0)
    S_o, Sy_o, yS = oracle.sens(w.system, w.method, w.theta, w.y0, cnt, h, nthreads=8)
    assert rel_err_mat(yS, y1b.cpu().numpy()).max() <= 1e-13  # the oracle's replay of that mesh
    # Robertson's rates span 0.04 ... 3e7 (HIRES's 7e-4 ... 280): compare
    # log-sensitivities theta dy/dtheta
    sc = w.theta[None] if name in ("robertson", "hires") else 1.0
    e = rel_err_mat(S.cpu().numpy() * sc, S_o * sc)
    assert e.max() <= TOL, e.max()
    # forward mode through the replay: the same numbers, bit for bit
    St, Sy = dao.sens(r1, with_y0=True)
    torch.cuda.synchronize()
    assert torch.equal(St, S)
    ey = rel_err_mat(Sy.cpu().numpy(), Sy_o)
    assert ey.max() <= TOL, ey.max()
    # transpose identity with the library's own reverse-mode gradient
    lam = torch.tensor(np.random.default_rng(9).normal(size=w.y0.shape), device=DEV)
    gth, gy0 = dao.grad(r1, lam)
    torch.cuda.synchronize()
    fwd = torch.einsum("cjk,ck->jk", S, lam).cpu().numpy()
    fwd_y = torch.einsum("cjk,ck->jk", Sy, lam).cpu().numpy()
    sc = w.theta if name in ("robertson", "hires") else 1.0
    e_t = rel_err_mat(fwd * sc, gth.cpu().numpy() * sc)
    e_y = rel_err_mat(fwd_y, gy0.cpu().numpy())
    assert e_t.max() <= TOL and e_y.max() <= TOL, (e_t.max(), e_y.max())


@pytest.mark.parametrize("name,n,s_cap,method", CASES[1:3] + CASES[5:6])
def test_sens_at_moved_theta_and_subsets(dao, name, n, s_cap, method):
    w = case(name, n, method)
    print(f"[sens moved theta] {name} n={n}", flush=True)
    th = torch.tensor(w.theta, device=DEV)
    y0 = torch.tensor(w.y0, device=DEV)
    rec, _ = dao.solve(w.system, w.method, th, y0, w.t0, w.t1, w.rtol, w.atol, s_cap=s_cap)
    cnt = rec.count.cpu().numpy()
    mask = np.arange(s_cap)[None, :] < cnt[:, None]
    h = np.where(mask, rec.h.cpu().numpy(), 0.0)
    th2 = w.theta * 1.003
    St, Sy = dao.sens(rec, theta=torch.tensor(th2, device=DEV), with_y0=True)
    only_y0 = dao.sens(rec, theta=torch.tensor(th2, device=DEV), with_theta=False, with_y0=True)
    torch.cuda.synchronize()
    assert only_y0[0] is None and torch.equal(only_y0[1], Sy)
    S_o, Sy_o, _ = oracle.sens(w.system, w.method, th2, w.y0, cnt, h, nthreads=8)
    assert rel_err_mat(St.cpu().numpy(), S_o).max() <= TOL
    assert rel_err_mat(Sy.cpu().numpy(), Sy_o).max() <= TOL


def test_sens_single_precision(dao):
    # binary32 on the GPU's own binary32 mesh, against the binary64 oracle on
    # that mesh (the gradient's single-precision bar, 1e-3).
    w = di.make("lorenz63", 200)
    w.t1 = 0.5
    th = torch.tensor(w.theta, dtype=torch.float32, device=DEV)
    y0 = torch.tensor(w.y0, dtype=torch.float32, device=DEV)
    rec, y1, S = dao.solve_sens(w.system, w.method, th, y0, w.t0, w.t1, 1e-5, 1e-7, s_cap=1024)
    torch.cuda.synchronize()
    assert np.all(rec.status.cpu().numpy() == 0)
    cnt = rec.count.cpu().numpy()
    mask = np.arange(1024)[None, :] < cnt[:, None]
    h = np.where(mask, rec.h.cpu().numpy(), 0.0).astype(np.float64)  # rows past count unspecified
    S_o, _, _ = oracle.sens(w.system, w.method, th.cpu().numpy().astype(np.float64),
                            y0.cpu().numpy().astype(np.float64), cnt, h, with_y0=False,
                            nthreads=8)
    assert rel_err_mat(S.cpu().numpy(), S_o).max() <= 1e-3


def test_loghalo_full_size_sampled(dao):
    # The orbit ensemble at its full size (1,048,576 trajectories) with the
    # in-kernel sensitivities, in the benchmark's launch configuration; a
    # seeded sample is checked against the oracle.
    w = di.make("loghalo")
    print(f"[solve_sens full size] loghalo n={w.n}", flush=True)
    th = torch.tensor(w.theta, device=DEV)
    y0 = torch.tensor(w.y0, device=DEV)
    rec, y1, S = dao.solve_sens(w.system, w.method, th, y0, w.t0, w.t1, w.rtol, w.atol,
                                s_cap=8192, record_t=False)
    torch.cuda.synchronize()
    assert np.all(rec.status.cpu().numpy() == 0)
    cnt = rec.count.cpu().numpy()
    rng = np.random.default_rng(4)
    idx = np.unique(np.concatenate([rng.choice(w.n, 48, replace=False), [0, w.n - 1],
                                    [np.argmax(cnt), np.argmin(cnt)]]))
    ws = di.subset(w, idx)
    h = rec.h[torch.tensor(idx, device=DEV)].cpu().numpy()
    h = np.where(np.arange(8192)[None, :] < cnt[idx][:, None], h, 0.0)
    S_o, _, yS = oracle.sens(ws.system, ws.method, ws.theta, ws.y0, cnt[idx], h, with_y0=False,
                             nthreads=8)
    assert rel_err_mat(yS, y1.cpu().numpy()[:, idx]).max() <= 1e-13
    assert rel_err_mat(S.cpu().numpy()[:, :, idx], S_o).max() <= TOL


def test_sens_unsupported_and_empty(dao):
    from differentiable_adaptive_ode_amd import DaoError

    w = di.make("mlp", 16)
    th = torch.tensor(w.theta, device=DEV)
    y0 = torch.tensor(w.y0, device=DEV)
    with pytest.raises(DaoError, match="not provided"):  # shared weights: reverse mode only
        dao.solve_sens(w.system, w.method, th, y0, 0.0, 1.0, 1e-5, 1e-7, s_cap=64)
    e = torch.empty((3, 0), dtype=torch.float64, device=DEV)
    tz = torch.empty((3, 0), dtype=torch.float64, device=DEV)
    rec, y1, S = dao.solve_sens("lorenz63", "tsit5", tz, e, 0.0, 1.0, 1e-6, 1e-8, s_cap=8)
    St, Sy = dao.sens(rec, with_y0=True, s_max=0)
    torch.cuda.synchronize()
    assert S.shape == (3, 3, 0) and St.shape == (3, 3, 0) and Sy.shape == (3, 3, 0)
