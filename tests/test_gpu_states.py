"""GPU parity of the states at requested times (through the C ABI) against
the oracle: a shortened step from the start of the accepted step that holds
each time (application paper arXiv 2609.28458, Sec. 2.3 and Appendix A).
Same arithmetic on both sides, so the bar is 1e-9 (observed: equality);
times on step boundaries and t1 reproduce the replay and y1 bit for bit."""
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


def rel_err(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return np.linalg.norm(a - b, axis=-2) / np.maximum(np.linalg.norm(b, axis=-2), 1e-300)


CASES = [("decay", 300, 256), ("lotka_volterra", 300, 256), ("lorenz63", 300, 1024),
         ("loghalo", 200, 4096), ("robertson", 200, 2048), ("hires", 200, 4096),
         ("decay_vern7", 300, 256), ("lotka_volterra_vern7", 300, 256),
         ("lorenz63_vern7", 300, 1024), ("loghalo_vern7", 200, 4096),
         ("decay_rodas5p", 300, 256), ("robertson_rodas5p", 200, 1024),
         ("lotka_volterra_rodas5p", 200, 256), ("hires_rodas5p", 130, 2048)]


@pytest.mark.parametrize("name,n,s_cap", CASES)
def test_states_at_parity(dao, name, n, s_cap):
    w = di.make(name, n)
    print(f"[states_at] {name} n={n}", flush=True)
    th = torch.tensor(w.theta, device=DEV)
    y0 = torch.tensor(w.y0, device=DEV)
    rec, y1 = dao.solve(w.system, w.method, th, y0, w.t0, w.t1, w.rtol, w.atol, s_cap=s_cap)
    rng = np.random.default_rng(3)
    span = w.t1 - w.t0
    tq = np.sort(np.concatenate([[w.t0, w.t1], w.t0 + span * rng.random(37)]))
    if name in ("robertson", "robertson_rodas5p"):  # stiff transient early on: log-spaced times too
        tq = np.sort(np.concatenate([tq, np.logspace(-5, 4.9, 12)]))
    tq_d = torch.tensor(tq, device=DEV)
    yq = dao.states_at(rec, tq_d)
    torch.cuda.synchronize()
    cnt = rec.count.cpu().numpy()
    h = np.where(np.arange(s_cap)[None, :] < cnt[:, None], rec.h.cpu().numpy(), 0.0)
    ref = oracle.states_at(w.system, w.method, w.theta, w.y0, w.t0, w.t1, cnt, h, tq, nthreads=8)
    yq = yq.cpu().numpy()
    assert np.all(np.isfinite(yq))
    e = rel_err(yq, ref)
    assert e.max() <= TOL, e.max()
    assert np.array_equal(yq[0], w.y0) and np.array_equal(yq[-1], y1.cpu().numpy())


def test_states_at_boundaries_and_bad_times(dao):
    w = di.make("lorenz63", 130)
    th = torch.tensor(w.theta, device=DEV)
    y0 = torch.tensor(w.y0, device=DEV)
    rec, y1 = dao.solve(w.system, w.method, th, y0, w.t0, w.t1, w.rtol, w.atol, s_cap=1024,
                        record_states=True)
    # the solve's recorded states are the replay's states at the step starts:
    # requested at a trajectory's own step start, the state comes back bit for bit
    t = rec.t.cpu().numpy()
    ys = rec.y.cpu().numpy()
    k = 17
    j = int(rec.count[k].item()) // 2
    tq = torch.tensor([t[k, j]], device=DEV)
    yq = dao.states_at(rec, tq)
    torch.cuda.synchronize()
    assert np.array_equal(yq.cpu().numpy()[0, :, k], ys[k, j])
    # times outside [t0, t1], not a number, or below a predecessor: NaN
    tq = torch.tensor([-0.5, 0.4, 0.2, 1.5, 3.0, float("nan")], dtype=torch.float64, device=DEV)
    yq = dao.states_at(rec, tq).cpu().numpy()
    assert np.all(np.isnan(yq[[0, 2, 4, 5]]))
    assert np.all(np.isfinite(yq[[1, 3]]))
    # at a moved theta, on the same mesh
    th2 = w.theta * 0.999
    tq = np.linspace(w.t0, w.t1, 9)
    yq = dao.states_at(rec, torch.tensor(tq, device=DEV), theta=torch.tensor(th2, device=DEV))
    cnt = rec.count.cpu().numpy()
    h = np.where(np.arange(1024)[None, :] < cnt[:, None], rec.h.cpu().numpy(), 0.0)
    ref = oracle.states_at(w.system, w.method, th2, w.y0, w.t0, w.t1, cnt, h, tq, nthreads=8)
    assert rel_err(yq.cpu().numpy(), ref).max() <= TOL


def test_states_at_empty_and_unsupported(dao):
    from differentiable_adaptive_ode_amd import DaoError

    w = di.make("lorenz63", 5)
    th = torch.tensor(w.theta, device=DEV)
    y0 = torch.tensor(w.y0, device=DEV)
    rec, y1 = dao.solve(w.system, w.method, th, y0, w.t0, w.t1, w.rtol, w.atol, s_cap=1024)
    yq = dao.states_at(rec, torch.empty(0, dtype=torch.float64, device=DEV))
    assert yq.shape == (0, 3, 5)
    wm = di.make("mlp", 16)
    thm = torch.tensor(wm.theta, device=DEV)
    y0m = torch.tensor(wm.y0, device=DEV)
    recm, _ = dao.solve(wm.system, wm.method, thm, y0m, 0.0, 1.0, 1e-5, 1e-7, s_cap=64)
    with pytest.raises(DaoError, match="not provided"):
        dao.states_at(recm, torch.tensor([0.5], dtype=torch.float32, device=DEV))
