"""The oracle's contract arithmetic against its PLAIN instantiation (CPU).

The solve's error test and controller follow fixed arithmetic readings (the
error weights s / sc_c formed before the last stage, the controller power by
a fixed polynomial rule, reciprocal pivots in the LU).  The gradsolve paper
(arXiv 2609.02876) defines the test as the RMS of e / (atol + rtol max(|y|,
|y_new|)) (Sec. 2.1) and the stiff step by a linear solve (Sec. 3.2); it fixes
no rounding.  The PLAIN instantiation writes those definitions out directly
(e_c / sc_c by IEEE division, the mean of squares as a sum over d, the library
pow, division by the pivot).  If the readings only change rounding, both give
the same solutions to well within the tolerance on every trajectory, and the
same accepted-step counts on nearly all of them: a different operation order
moves the 16-bit-truncated controller factor across a truncation boundary now
and then, which changes later step sizes but not the accuracy.

Samples of the five benchmark ensembles (and HIRES and the difficulty-spread
Lorenz ensemble), each drawn from the ensemble's own seeded stream.
"""
import os

import numpy as np
import pytest

import dao_inputs as di

NTHREADS = min(os.cpu_count() or 1, 8)

# workload: (sample size, record capacity)
SAMPLES = {
    "lotka_volterra": (256, 256),
    "lorenz63": (4096, 1024),
    "mlp": (1024, 64),
    "robertson": (4096, 1024),
    "loghalo": (1024, 8192),
    "hires": (512, 4096),
    "lorenz63_spread": (1024, 2048),
    "lorenz63_vern7": (2048, 1024),
    "loghalo_vern7": (512, 8192),
    "robertson_rodas5p": (2048, 1024),
    "hires_rodas5p": (256, 2048),
}


@pytest.mark.parametrize("name", list(SAMPLES))
def test_plain_and_contract_arithmetic_agree(orc, name):
    n, s_cap = SAMPLES[name]
    w = di.make(name, n)
    kw = dict(s_cap=s_cap, dtype=w.dtype, nthreads=NTHREADS)
    a = orc.solve(w.system, w.method, w.theta, w.y0, w.t0, w.t1, w.rtol, w.atol, **kw)
    b = orc.solve(w.system, w.method, w.theta, w.y0, w.t0, w.t1, w.rtol, w.atol, plain=True, **kw)
    assert np.all(a["status"] == 0) and np.all(b["status"] == 0)
    ya, yb = a["y1"].astype(np.float64), b["y1"].astype(np.float64)
    tol = 10.0 * (w.rtol * np.maximum(np.abs(ya), np.abs(yb)) + w.atol)
    assert np.all(np.abs(ya - yb) <= tol), float((np.abs(ya - yb) / tol).max())
    assert np.mean(a["count"] == b["count"]) >= 0.99
    # counts that differ differ by a step or two, not by a change of regime
    assert np.abs(a["count"].astype(np.int64) - b["count"]).max() <= 2


def test_plain_differs_from_contract_only_in_rounding(orc):
    """The two instantiations are not the same code: on the orbit ensemble some
    meshes differ (a truncated factor flips), and where the meshes agree the
    final states agree bit for bit (the readings touch only the error test
    and the controller, never the step itself)."""
    w = di.make("loghalo", 256)
    kw = dict(s_cap=8192, nthreads=NTHREADS)
    a = orc.solve(w.system, w.method, w.theta, w.y0, w.t0, w.t1, w.rtol, w.atol, **kw)
    b = orc.solve(w.system, w.method, w.theta, w.y0, w.t0, w.t1, w.rtol, w.atol, plain=True, **kw)
    same = np.array([np.array_equal(a["h"][k, :a["count"][k]], b["h"][k, :b["count"][k]])
                     for k in range(w.n)])
    assert 0 < same.sum() < w.n
    assert np.array_equal(a["y1"][:, same], b["y1"][:, same])


def test_plain_robertson_lu_divides_by_the_pivot(orc):
    """The Rosenbrock step's LU differs between the two (reciprocal pivots
    against division): at a fixed step the stage values differ in the last
    bits only, so the accepted meshes of a Robertson sample mostly differ while
    the final states agree to far below the tolerance."""
    w = di.make("robertson", 512)
    kw = dict(s_cap=1024, nthreads=NTHREADS)
    a = orc.solve(w.system, w.method, w.theta, w.y0, w.t0, w.t1, w.rtol, w.atol, **kw)
    b = orc.solve(w.system, w.method, w.theta, w.y0, w.t0, w.t1, w.rtol, w.atol, plain=True, **kw)
    rel = np.abs(a["y1"] - b["y1"]) / (w.rtol * np.abs(a["y1"]) + w.atol)
    assert rel.max() < 1e-2
    assert not np.array_equal(a["y1"], b["y1"])
