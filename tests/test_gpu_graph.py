"""The solve + cotangent + order + gradient step captured as one HIP graph
(torch.cuda.CUDAGraph on the stream the library launches on) and replayed:
every replay, with eager work and synchronisations between them, must give
the eager step's outputs bit for bit.  The library records no memset; its
counters are reset by a fill kernel, which a graph replays like any other."""
import numpy as np
import pytest
import torch

import dao_inputs as di

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def dao():
    import differentiable_adaptive_ode_amd as m

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return m


@pytest.mark.parametrize("name,n,s_cap", [("lorenz63", 700, 1024), ("robertson", 300, 1024),
                                          ("mlp", 1000, 64)])
def test_graph_replays_equal_the_eager_step(dao, name, n, s_cap):
    from differentiable_adaptive_ode_amd import api

    w = di.make(name, n)
    print(f"[graph] {name} n={n}", flush=True)
    th = torch.tensor(w.theta, device=DEV)
    y0 = torch.tensor(w.y0, device=DEV)
    tgt = torch.tensor(w.target, device=DEV)
    bufs = api.alloc_record(w.n, s_cap, w.dtype, torch.device(DEV), with_t=False)
    y1, lam = torch.empty_like(y0), torch.empty_like(y0)
    dth, dy0 = torch.empty_like(th), torch.empty_like(y0)
    wsp = api.Workspace()

    def step(s_max):
        rec, _ = dao.solve(w.system, w.method, th, y0, w.t0, w.t1, w.rtol, w.atol, s_cap=s_cap,
                           out=y1, rec_buffers=bufs, workspace=wsp)
        dao.cotangent(y1, tgt, 1.0, out=lam)
        dao.grad_order(rec, s_max=s_max, workspace=wsp)
        dao.grad(rec, lam, s_max=s_max, out_theta=dth, out_y0=dy0, workspace=wsp, ordered=True)
        return rec

    rec = step(s_cap)
    torch.cuda.synchronize()
    s_max = int(rec.count.max().item())
    step(s_max)
    torch.cuda.synchronize()
    def recorded_h():
        # rows past a trajectory's count are unspecified: compare the recorded steps only
        cols = torch.arange(bufs["h"].shape[1], device=DEV)[None, :]
        return torch.where(cols < bufs["count"][:, None], bufs["h"], torch.zeros_like(bufs["h"]))

    ref = [t.clone() for t in (y1, dth, dy0, bufs["count"])] + [recorded_h()]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(s_max)
    torch.cuda.synchronize()
    other = di.make("lotka_volterra", 64)
    for r in range(3):
        for t in (y1, dth, dy0):
            t.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip((y1, dth, dy0, bufs["count"], recorded_h()), ref):
            assert torch.equal(a, b), f"replay {r} differs"
        # eager work of the program's own between the replays (its own workspace)
        dao.solve(other.system, other.method, torch.tensor(other.theta, device=DEV),
                  torch.tensor(other.y0, device=DEV), other.t0, other.t1, other.rtol, other.atol,
                  s_cap=256)
        torch.cuda.synchronize()
