"""The benchmark's algorithmic work per unit, pinned to the oracle's operation
tally (a counting scalar type run through the same solve and replay code):
per-trajectory start-up, per attempted step, per replay step."""
import numpy as np
import pytest

import bench
import dao_inputs as di


@pytest.mark.parametrize("name", list(bench.WORKLOADS))
def test_solve_and_replay_tallies(orc, name):
    cfg = bench.WORKLOADS[name]
    w = di.make(name, 16)
    tot = pred = 0.0
    for k in range(w.n):
        th = (w.theta if w.system == "mlp" else w.theta[:, k]).astype(np.float64)
        y0 = w.y0[:, k].astype(np.float64)
        c = orc.count_solve(w.system, w.method, th, y0, w.t0, w.t1, w.rtol, w.atol)
        assert c["init"] == cfg["init"]
        tot += c["total"]
        pred += cfg["init"] + c["attempts"] * cfg["att"] + c["accepted"] * (1 + cfg.get("acc_extra", 0))
        assert orc.count_replay_step(w.system, w.method, th, y0, 1e-3) == cfg["replay"]
    # the model leaves out only the clip of the last step (one flop per trajectory)
    assert abs(pred - tot) / tot < 1e-3, (pred, tot)


def test_lorenz_gradient_step_by_hand():
    # replay 192 + recomputed stages 153 + k-bar seeds 24 + six VJPs 6 x 19
    # + lambda updates 18 + stage-cotangent updates 15 x 7
    assert bench.WORKLOADS["lorenz63"]["grad"] == 192 + 153 + 24 + 6 * 19 + 18 + 105 == 606


@pytest.mark.parametrize("name", list(bench.WORKLOADS))
def test_gradient_step_is_bounded_by_the_tape_tally(orc, name):
    # The benchmark's gradient step (forward replay + recomputed stages + the
    # hand-derived reverse sweep) never exceeds what the oracle tallies for
    # the same step done by reverse mode on its tape: the replay twice plus
    # one multiply-add per local partial derivative (and the partials' own
    # quotients and tanh derivatives).  So the gradient's roofline numerator
    # is bounded by an oracle tally, not by a hand formula alone.
    cfg = bench.WORKLOADS[name]
    w = di.make(name, 4)
    for k in range(w.n):
        th = (w.theta if w.system == "mlp" else w.theta[:, k]).astype(np.float64)
        rep, rev = orc.count_grad_step(w.system, w.method, th, w.y0[:, k].astype(np.float64), 1e-3)
        assert rep == cfg["replay"]
        assert cfg["replay"] < cfg["grad"] <= 2 * rep + rev, (cfg["grad"], 2 * rep + rev)
