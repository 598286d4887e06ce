"""The Python binding's argument checks (no GPU needed).

The C ABI takes plain pointers and the sizes it is told, so the binding
checks each array's dtype, shape, device and layout before it passes a
pointer.  These checks come before any library call: CPU tensors of the
wrong dtype or shape raise TypeError / ValueError here, and right-sized CPU
tensors are still refused as host memory."""
import pytest
import torch

dao = pytest.importorskip("differentiable_adaptive_ode_amd")


def record(system="lorenz63", dtype=torch.float64, n=8, s_cap=4):
    d, p, shared = dao._lib.dao_system_dims(dao._lib.SYSTEMS[system])
    theta = torch.zeros((p,) if shared else (p, n), dtype=dtype)
    y0 = torch.zeros((d, n), dtype=dtype)
    i32 = lambda: torch.zeros(n, dtype=torch.int32)  # noqa: E731
    return dao.Record(system, "tsit5", "f64" if dtype == torch.float64 else "f32", theta, y0,
                      0.0, 1.0, torch.zeros((n, s_cap), dtype=dtype), None, i32(), i32(), i32())


def test_a_cotangent_of_another_dtype_is_refused():
    # float64 cotangent on a float32 (neural field) record: it would be read
    # as float32
    rec = record("mlp", torch.float32)
    with pytest.raises(TypeError, match="dLdy1"):
        dao.grad(rec, torch.zeros((4, 8), dtype=torch.float64))
    rec = record()
    with pytest.raises(TypeError, match="dLdy1"):
        dao.grad(rec, torch.zeros((3, 8), dtype=torch.float32))


@pytest.mark.parametrize("shape", [(3, 7), (8, 3), (24,), (3, 8, 1)])
def test_a_cotangent_of_another_shape_is_refused(shape):
    with pytest.raises(ValueError, match="dLdy1"):
        dao.grad(record(), torch.zeros(shape, dtype=torch.float64))


def test_theta_and_outputs_are_checked():
    rec = record()
    g = torch.zeros((3, 8), dtype=torch.float64)
    with pytest.raises(ValueError, match="theta"):
        dao.grad(rec, g, theta=torch.zeros((3, 7), dtype=torch.float64))
    with pytest.raises(TypeError, match="theta"):
        dao.grad(rec, g, theta=torch.zeros((3, 8), dtype=torch.float32))
    with pytest.raises(ValueError, match="out_theta"):
        dao.grad(rec, g, out_theta=torch.zeros((3, 9), dtype=torch.float64))
    with pytest.raises(ValueError, match="out_y0"):
        dao.grad(rec, g, out_y0=torch.zeros((8, 3), dtype=torch.float64))
    with pytest.raises(ValueError, match="theta"):
        dao.sens(rec, theta=torch.zeros(3, dtype=torch.float64))


def test_grad_at_and_states_at_arrays_are_checked():
    rec = record()
    tq = torch.zeros(5, dtype=torch.float64)
    with pytest.raises(ValueError, match="dLdyq"):
        dao.grad_at(rec, tq, torch.zeros((5, 3, 7), dtype=torch.float64))
    with pytest.raises(TypeError, match="dLdy1"):
        dao.grad_at(rec, tq, torch.zeros((5, 3, 8), dtype=torch.float64),
                    torch.zeros((3, 8), dtype=torch.float32))
    with pytest.raises(ValueError, match="one-dimensional"):
        dao.states_at(rec, torch.zeros((5, 1), dtype=torch.float64))
    with pytest.raises(ValueError, match="theta"):
        dao.states_at(rec, tq, theta=torch.zeros((3, 3), dtype=torch.float64))


def test_solve_outputs_and_record_buffers_are_checked():
    th = torch.zeros((3, 8), dtype=torch.float64)
    y0 = torch.zeros((3, 8), dtype=torch.float64)
    # the inputs themselves must be on the device
    with pytest.raises(ValueError, match="device"):
        dao.solve("lorenz63", "tsit5", th, y0, 0.0, 1.0, 1e-6, 1e-8)
    rec = record()
    with pytest.raises(ValueError, match="out"):
        rec.stats(out=torch.zeros(3, dtype=torch.int64))


def test_right_sized_host_arrays_are_still_refused():
    rec = record()
    with pytest.raises(ValueError, match="device"):
        dao.grad(rec, torch.zeros((3, 8), dtype=torch.float64))


def test_cotangent_target_is_checked():
    y1 = torch.zeros((3, 8), dtype=torch.float64)
    with pytest.raises(ValueError, match="device"):
        dao.cotangent(y1, torch.zeros((3, 8), dtype=torch.float64))


def test_an_inconsistent_record_is_refused():
    # the kernels index a record's arrays by n, s_cap and d alone
    rec = record()
    g = torch.zeros((3, 8), dtype=torch.float64)
    bad = [("count", torch.zeros(7, dtype=torch.int32), ValueError),  # n = 7: h, y0 disagree
           ("status", torch.zeros(8, dtype=torch.int64), TypeError),
           ("h", torch.zeros((8, 4), dtype=torch.float32), TypeError),
           ("t", torch.zeros((8, 5), dtype=torch.float64), ValueError),
           ("y0", torch.zeros((3, 9), dtype=torch.float64), ValueError),
           ("y", torch.zeros((8, 4, 2), dtype=torch.float64), ValueError)]
    for field, value, exc in bad:
        r = record()
        setattr(r, field, value)
        name = "h" if field == "count" else field
        with pytest.raises(exc, match=name):
            dao.grad(r, g)
        with pytest.raises(exc, match=name):
            dao.states_at(r, torch.zeros(2, dtype=torch.float64))
    with pytest.raises(ValueError, match="unknown"):
        r = record()
        r.method = "rk4"
        dao.grad(r, g)
    # consistent, but on the host: refused as such
    with pytest.raises(ValueError, match="device"):
        rec.check()
    rec.check(placed=False)
