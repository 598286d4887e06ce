"""HIRES's linear solves on the GPU skip the structural zeros of W while no
lane of a wavefront has exchanged rows, and run the dense elimination from
the first step at which one does.  Here every third trajectory has its rate
k3 raised by 30 % (theta[2]), which makes |W[3][1]| exceed |W[1][1]| once
the step is long enough: those lanes exchange rows at some attempts, and
their wavefronts (shared with ordinary trajectories) take the dense path
there.  The solve must still equal the oracle's dense LU with partial
pivoting bit for bit (counts, rejections, every recorded h) and the
gradient on the oracle's mesh must stay within the fp64 bar (1e-9, rates as
log-sensitivities).  A CPU check confirms that the inputs do exchange rows
(SciPy's LU with partial pivoting of W at sampled steps)."""
import numpy as np
import pytest
import torch

import dao_inputs as di
import oracle

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL = 1e-9
GAMMA = {"hires": 0.29289321881345248, "hires_rodas5p": 0.21193756319429014}


@pytest.fixture(scope="module")
def dao():
    import differentiable_adaptive_ode_amd as m

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return m


def rel_err(a, b):
    den = np.maximum(np.linalg.norm(b, axis=0), 1e-300)
    return np.linalg.norm(a - b, axis=0) / den


def exchanging_case(name, n):
    w = di.make(name, n)
    th = w.theta.copy()
    sel = np.arange(n) % 3 == 0
    th[2, sel] *= 1.3
    return w, th, sel


def rows_exchange_somewhere(w, th, sel, ref):
    from scipy.linalg import lu_factor

    g = GAMMA[w.name]
    for k in np.flatnonzero(sel)[:6]:
        c = int(ref["count"][k])
        for j in range(0, c, max(1, c // 12)):
            cnt = np.zeros(w.n, np.int32)
            cnt[k] = j
            yj = oracle.replay(w.system, w.method, th, w.y0, cnt, ref["h"])[:, k]
            J = oracle.jac(w.system, th[:, k], yj)
            hj = ref["h"][k, j]
            W = np.eye(8) - hj * g * J if w.method == "rosenbrock23" else np.eye(8) / (g * hj) - J
            if np.any(lu_factor(W)[1] != np.arange(8)):
                return True
    return False


@pytest.mark.parametrize("name", ["hires", "hires_rodas5p"])
def test_sparse_and_dense_paths_equal_the_dense_oracle(dao, name):
    from differentiable_adaptive_ode_amd.api import Record

    n, s_cap = 96, 4096
    w, th, sel = exchanging_case(name, n)
    print(f"[sparse LU] {name} n={n}", flush=True)
    ref = oracle.solve(w.system, w.method, th, w.y0, w.t0, w.t1, w.rtol, w.atol, s_cap=s_cap,
                       dtype="f64", nthreads=8)
    assert np.all(ref["status"] == 0)
    assert rows_exchange_somewhere(w, th, sel, ref)
    tht = torch.tensor(th, device=DEV)
    y0 = torch.tensor(w.y0, device=DEV)
    rec, y1 = dao.solve(w.system, w.method, tht, y0, w.t0, w.t1, w.rtol, w.atol, s_cap=s_cap)
    torch.cuda.synchronize()
    cnt = rec.count.cpu().numpy()
    assert np.array_equal(rec.status.cpu().numpy(), ref["status"])
    assert np.array_equal(cnt, ref["count"]), np.flatnonzero(cnt != ref["count"])[:10]
    assert np.array_equal(rec.nrej.cpu().numpy(), ref["nrej"])
    mask = np.arange(s_cap)[None, :] < cnt[:, None]
    assert np.array_equal(rec.h.cpu().numpy()[mask], ref["h"][mask])
    assert rel_err(y1.cpu().numpy(), ref["y1"]).max() <= TOL
    # the gradient on the oracle's mesh
    lam = di.cotangent(w, ref["y1"])
    dth_o, dy0_o, _ = oracle.grad(w.system, w.method, th, w.y0, ref["count"], ref["h"], lam,
                                  nthreads=8)
    h = torch.zeros((n, s_cap), dtype=torch.float64, device=DEV)
    h[:, :ref["h"].shape[1]] = torch.tensor(ref["h"], device=DEV)
    mrec = Record(w.system, w.method, w.dtype, tht, y0, w.t0, w.t1, h, None,
                  torch.tensor(ref["count"], device=DEV), torch.tensor(ref["nrej"], device=DEV),
                  torch.tensor(ref["status"], device=DEV))
    dth, dy0 = dao.grad(mrec, torch.tensor(lam, device=DEV))
    torch.cuda.synchronize()
    assert rel_err(dth.cpu().numpy() * th, dth_o * th).max() <= TOL
    assert rel_err(dy0.cpu().numpy(), dy0_o).max() <= TOL
