"""dao_grad_noalloc (the gradient with the library's static scratch instead of
a workspace) against dao_grad, through the C ABI: bit for bit, the neural
field's shared-weight sum included; two calls in a row per system, the second
on a smaller ensemble (the array keeps the first call's contents)."""
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


def _case(dao, name, n, s_cap):
    w = di.make(name, n)
    th = torch.tensor(w.theta, device=DEV)
    y0 = torch.tensor(w.y0, device=DEV)
    rec, y1 = dao.solve(w.system, w.method, th, y0, w.t0, w.t1, w.rtol, w.atol, s_cap=s_cap,
                        record_t=False)
    gen = torch.Generator(device=DEV).manual_seed(n)
    lam = torch.randn(y1.shape, dtype=y1.dtype, device=DEV, generator=gen)
    return w, th, y0, rec, lam


def _noalloc(dao, rec, th, y0, lam, s_max):
    from differentiable_adaptive_ode_amd import _lib

    ids = _lib.SYSTEMS[rec.system], _lib.METHODS[rec.method], _lib.DTYPES[rec.dtype]
    dth = torch.full_like(th, 7.0)
    dy0 = torch.full_like(y0, 7.0)
    _lib.check(_lib.dao_grad_noalloc(*ids, rec.n, th.data_ptr(), y0.data_ptr(),
                                     rec.c_struct(states=False), s_max, lam.data_ptr(),
                                     dth.data_ptr(), dy0.data_ptr(),
                                     torch.cuda.current_stream().cuda_stream))
    return dth, dy0


@pytest.mark.parametrize("name,sizes,s_cap", [("lorenz63", (3000, 700), 1024),
                                              ("loghalo", (1500, 250), 8192),
                                              ("robertson", (2000, 333), 1024),
                                              ("mlp", (1000, 16 * 3 + 5), 64)])
def test_noalloc_gradient_equals_dao_grad(dao, name, sizes, s_cap):
    for n in sizes:
        print(f"[grad noalloc] {name} n={n}", flush=True)
        w, th, y0, rec, lam = _case(dao, name, n, s_cap)
        s_max = rec.stats_host()["s_max"]
        ref_th, ref_y0 = dao.grad(rec, lam, s_max=s_max)
        dth, dy0 = _noalloc(dao, rec, th, y0, lam, s_max)
        torch.cuda.synchronize()
        assert torch.equal(dy0, ref_y0)
        assert torch.isfinite(dth).all()
        assert torch.equal(dth, ref_th)


def test_noalloc_rejects_more_than_its_scratch(dao):
    from differentiable_adaptive_ode_amd import _lib

    w, th, y0, rec, lam = _case(dao, "lorenz63", 64, 1024)
    ids = _lib.SYSTEMS["lorenz63"], 0, 0
    big = _lib.dao_record(1 << 20, None, rec.h.data_ptr(), rec.count.data_ptr(), None,
                          rec.status.data_ptr())
    code = _lib.dao_grad_noalloc(*ids, 64, th.data_ptr(), y0.data_ptr(), big, 1 << 20,
                                 lam.data_ptr(), None, None, None)
    assert code == _lib.DAO_EWORKSPACE
    assert "static" in _lib.dao_last_error()
