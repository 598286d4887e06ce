"""GPU tests of the boundary's bookkeeping: the stream-ordered record summary,
the call-level failure signal of the shared-weight gradient, and calls on
several streams at once (each with its own default workspace)."""
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


def _solve(dao, w, s_cap, **kw):
    th = torch.tensor(w.theta, device=DEV)
    y0 = torch.tensor(w.y0, device=DEV)
    return dao.solve(w.system, w.method, th, y0, w.t0, w.t1, w.rtol, w.atol, s_cap=s_cap, **kw)


def test_record_stats_match_the_record(dao):
    # a record with every kind of trajectory: finished, out of capacity, and
    # non-finite (a NaN rate)
    w = di.make("lorenz63", 64 * 4 + 17)
    th = w.theta.copy()
    th[0, 5] = np.nan
    w = di.Workload(**{**w.__dict__, "theta": th})
    print("[record stats] lorenz63 n=273", flush=True)
    for s_cap in (1024, 150):
        rec, _ = _solve(dao, w, s_cap)
        got = rec.stats()
        torch.cuda.synchronize()
        cnt = rec.count.cpu().numpy().astype(np.int64)
        st = rec.status.cpu().numpy()
        nrej = rec.nrej.cpu().numpy().astype(np.int64)
        want = [cnt.max(), cnt.sum(), int((st != 0).sum()), nrej.sum()]
        assert got.cpu().tolist() == [int(v) for v in want]
        assert rec.stats_host() == dict(s_max=int(cnt.max()), steps=int(cnt.sum()),
                                        failed=int((st != 0).sum()), rejected=int(nrej.sum()))
        assert int(got[2]) >= 1


def test_record_stats_of_an_empty_record(dao):
    rec, _ = _solve(dao, di.make("lorenz63", 0), 64)
    got = rec.stats()
    torch.cuda.synchronize()
    assert got.cpu().tolist() == [0, 0, 0, 0]


def test_record_stats_replace_a_host_read_of_s_max(dao):
    # The summary sizes the gradient exactly; the default (the capacity) gives
    # the same gradient with a larger workspace.
    w = di.make("lorenz63", 300)
    rec, y1 = _solve(dao, w, 1024)
    s_max = rec.stats_host()["s_max"]
    lam = torch.ones_like(y1)
    a = dao.grad(rec, lam, s_max=s_max)
    b = dao.grad(rec, lam)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_shared_weight_gradient_is_nan_when_a_trajectory_failed(dao):
    # The neural field's gradient sums over the ensemble: a failed trajectory,
    # or one with more steps than s_max, has no gradient, so the sum is NaN
    # rather than silently partial.  A clean ensemble gives finite values.
    w = di.make("mlp", 16 * 9 + 3)
    print("[mlp failure signal] n=147", flush=True)
    rec, y1 = _solve(dao, w, 64)
    lam = torch.ones_like(y1)
    dth, dy0 = dao.grad(rec, lam)
    torch.cuda.synchronize()
    assert torch.isfinite(dth).all() and torch.isfinite(dy0).all()
    stats = rec.stats_host()
    assert stats["failed"] == 0
    # count above s_max for the longest trajectories
    cnt = rec.count.cpu().numpy()
    if cnt.max() > cnt.min():
        dth2, dy02 = dao.grad(rec, lam, s_max=int(cnt.max()) - 1)
        torch.cuda.synchronize()
        assert torch.isnan(dth2).all()
        long = torch.tensor(cnt > cnt.max() - 1, device=DEV)
        assert torch.isnan(dy02[:, long]).all() and torch.isfinite(dy02[:, ~long]).all()
    # a non-finite initial state fails one trajectory in the solve
    y0 = w.y0.copy()
    y0[2, 40] = np.nan
    w2 = di.Workload(**{**w.__dict__, "y0": y0})
    rec2, y12 = _solve(dao, w2, 64)
    dth3, dy03 = dao.grad(rec2, torch.ones_like(y12))
    torch.cuda.synchronize()
    st = rec2.status.cpu().numpy()
    assert st[40] != 0 and np.all(np.delete(st, 40) == 0)
    assert rec2.stats_host()["failed"] == 1
    assert torch.isnan(dth3).all()
    assert torch.isnan(dy03[:, 40]).all()


def test_calls_on_two_streams_use_their_own_workspaces(dao):
    # Solve and gradient of two different ensembles enqueued on two streams
    # without synchronising between them: each stream gets its own default
    # workspace, so the results equal those of the same calls made one after
    # the other on the default stream, bit for bit.
    wa, wb = di.make("lorenz63", 2000), di.make("loghalo", 600)
    print("[two streams] lorenz63 2000 + loghalo 600", flush=True)

    def run(w, s_cap, stream):
        with torch.cuda.stream(stream):
            rec, y1 = _solve(dao, w, s_cap, stream=stream)
            lam = torch.ones_like(y1)
            dth, dy0 = dao.grad(rec, lam, stream=stream)
        return y1, dth, dy0

    ref_a = run(wa, 1024, torch.cuda.current_stream())
    ref_b = run(wb, 4096, torch.cuda.current_stream())
    torch.cuda.synchronize()
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    for _ in range(2):
        got_a = run(wa, 1024, sa)
        got_b = run(wb, 4096, sb)
        torch.cuda.synchronize()
        for x, y in zip(got_a + got_b, ref_a + ref_b):
            assert torch.equal(x, y)
